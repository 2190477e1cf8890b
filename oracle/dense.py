"""Whole-matrix forms of the oracle's products, for checking every row of a
full-size output.

TEST INFRASTRUCTURE ONLY: imported by tests.  The product path never
imports it.

Each function computes the same definition as its counterpart in oracle.c,
with the same operands and the same rounding points; only the dot products
run as float64 matrix products (numpy, OpenBLAS) instead of written-out
loops, so a full-size output (billions of multiply-adds per output) takes
seconds instead of hours.  Sums are float64 in the library's order, so a
result can differ from oracle.c's by the order of float64 additions: that
moves a bf16 rounding by one unit only when a sum lands within about 1e-16
(relative) of a rounding boundary.  tests/test_oracle_dense.py pins these
functions against oracle.c, against closed forms and against torch.

Sources, cited by page title and section:
  [P2] "Marin 開始公開訓練 535B 參數 MoE 模型" (lamjinlab.com, zh-HK), section 二
  [P1] "从玩具到前沿:训练一个真正的大模型,到底难在哪里" (devpress.csdn.net),
       section 四 and appendix A.3
Readings the pages leave open (SwiGLU experts, bf16 rounding points,
output-major weights) are the same as oracle.c's.

Arrays are numpy; bf16 values travel as uint16 bit patterns.
"""
import numpy as np

_CHUNK = 2048          # rows per matrix product (bounds the float64 temporaries)


def to_f64(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    return (np.ascontiguousarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 of each float64 (ties to even), one rounding, as uint16.

    Normal range: the double's 52-bit fraction is rounded to bf16's 7 bits
    by integer arithmetic on its bit pattern (a carry into the exponent is
    the next binade, and past the largest finite bf16 it reaches infinity);
    the result has 8 significant bits, so float32 holds it exactly and its
    top 16 bits are the bf16.  Below 2^-126 bf16 is subnormal with spacing
    2^-133: those round with np.rint (ties to even) on that grid."""
    v = np.ascontiguousarray(v, np.float64)
    u = v.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    normal = r.view(np.float64)
    tiny = np.abs(v) < 2.0 ** -126
    if tiny.any():
        normal = np.where(tiny, np.rint(v * 2.0 ** 133) * 2.0 ** -133, normal)
    with np.errstate(over="ignore"):
        f = normal.astype(np.float32)
    out = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def _rows(n):
    for s in range(0, n, _CHUNK):
        yield s, min(n, s + _CHUNK)


def _silu(a):
    return a / (1.0 + np.exp(-a))


def latent(x: np.ndarray, w_ld_t: np.ndarray) -> np.ndarray:
    """z = bf16(x . W_ld), W_ld stored as W_ld^T [L, D] ([P2] section 二:
    activations go to the latent width before the exchange).  Same as
    orc_latent_rows over every row."""
    w = to_f64(w_ld_t)
    z = np.empty((x.shape[0], w.shape[0]), np.uint16)
    for s, e in _rows(x.shape[0]):
        z[s:e] = bf16_from_f64(to_f64(x[s:e]) @ w.T)
    return z


def ffn_rows(u: np.ndarray, wg_t: np.ndarray, wu_t: np.ndarray, wd_t: np.ndarray) -> np.ndarray:
    """One local expert on rows u [n, L] ([P1] section 四 / appendix A.3: the
    receiver runs its experts on their bank rows; SwiGLU reading):
    a = u.W_g, b = u.W_u (float64), h = bf16(silu(a) b), y = bf16(h . W_d).
    wg_t, wu_t [F, L]; wd_t [L, F].  Same as orc_ffn_row per row."""
    wg, wu, wd = to_f64(wg_t), to_f64(wu_t), to_f64(wd_t)
    y = np.empty((u.shape[0], wd.shape[0]), np.uint16)
    for s, e in _rows(u.shape[0]):
        uu = to_f64(u[s:e])
        a = uu @ wg.T
        b = uu @ wu.T
        h = to_f64(bf16_from_f64(_silu(a) * b))
        y[s:e] = bf16_from_f64(h @ wd.T)
    return y


def expert_ffn(d, bank: np.ndarray, bank_offsets, bank_src, bfill, w_gate, w_up, w_down,
               n_ret_rows: int) -> np.ndarray:
    """Every kept bank row through its local expert, written to the return
    buffer at bank_src; every other return row zero (orc_expert_ffn).
    bank [bank rows, L]; w_gate, w_up [E_l, F, L]; w_down [E_l, L, F].
    Fixed mode: group g = (w, j) starts at g * cap_recv; ragged: bank_offsets."""
    El = d.n_experts // d.n_ranks
    ret = np.zeros((n_ret_rows, d.latent), np.uint16)
    for j in range(El):
        pos = []
        for w in range(d.n_waves):
            g = w * El + j
            start = int(bank_offsets[g]) if bank_offsets is not None else g * d.cap_recv
            pos.append(np.arange(start, start + int(bfill[g])))
        pos = np.concatenate(pos).astype(np.int64)
        if len(pos) == 0:
            continue
        ret[bank_src[pos]] = ffn_rows(bank[pos], w_gate[j], w_up[j], w_down[j])
    return ret


def shared_h(x: np.ndarray, ws_gate: np.ndarray, ws_up: np.ndarray) -> np.ndarray:
    """h_s = bf16(silu(x.W_sg,s) * (x.W_su,s)) of every shared expert ([P2]
    section 二: the shared experts see every token), as [n, S*Fs] uint16."""
    S, Fs, _ = ws_gate.shape
    h = np.empty((x.shape[0], S * Fs), np.uint16)
    for sh in range(S):
        wg, wu = to_f64(ws_gate[sh]), to_f64(ws_up[sh])
        for s, e in _rows(x.shape[0]):
            xx = to_f64(x[s:e])
            h[s:e, sh * Fs:(sh + 1) * Fs] = bf16_from_f64(_silu(xx @ wg.T) * (xx @ wu.T))
    return h


def returned_rows(d, ret_offsets, topk: np.ndarray, slot: np.ndarray, tokens: np.ndarray):
    """Row of the returned buffer read by each (token, choice) of `tokens`,
    -1 where the choice was dropped or (ragged) its slot is past its segment
    ([P2] section 四: a dropped assignment loses its routed contribution).
    Waves by token; returned rows in the pools' (destination, wave, slot)
    order."""
    El = d.n_experts // d.n_ranks
    W = d.n_waves
    Tw = -(-d.T // W)
    tk = topk[tokens].astype(np.int64)
    sl = slot[tokens].astype(np.int64)
    seg = (tk // El) * W + (tokens // Tw)[:, None]
    if d.cap_send:
        row = seg * d.cap_send + sl
        return np.where(sl >= 0, row, -1)
    offs = np.asarray(ret_offsets, np.int64)
    inside = (sl >= 0) & (sl < offs[seg + 1] - offs[seg])
    return np.where(inside, offs[seg] + sl, -1)


def combine_tokens(d, returned: np.ndarray, ret_offsets, topk, slot, gates, x, w_lu_t, ws_gate,
                   ws_up, ws_down, tokens=None):
    """ylat and out of the given tokens (orc_combine_tokens, waves by token,
    no dedup):
      ylat[t] = bf16( sum_j [kept] g[t,j] returned[row(t,j)] )   (j ascending)
      out[t]  = bf16( ylat[t].W_lu + sum_s h_s(x[t]).W_sd,s )    (one sum)
    w_lu_t [D, L]; ws_gate, ws_up [S, Fs, D]; ws_down [S, D, Fs]."""
    assert d.wave_mode == 0 and not d.dedup
    tokens = np.arange(d.T) if tokens is None else np.asarray(tokens, np.int64)
    rows = returned_rows(d, ret_offsets, topk, slot, tokens)
    g = gates[tokens].astype(np.float64)
    L = d.latent
    acc = np.zeros((len(tokens), L))
    for j in range(d.top_k):
        m = rows[:, j] >= 0
        if m.any():
            acc[m] += g[m, j][:, None] * to_f64(returned[rows[m, j]])
    ylat = bf16_from_f64(acc)
    wlu = to_f64(w_lu_t)
    S = ws_gate.shape[0] if ws_gate is not None else 0
    out = np.empty((len(tokens), wlu.shape[0]), np.uint16)
    wsd = [to_f64(ws_down[s]) for s in range(S)]
    for s0, e0 in _rows(len(tokens)):
        o = to_f64(ylat[s0:e0]) @ wlu.T
        if S:
            h = to_f64(shared_h(x[tokens[s0:e0]], ws_gate, ws_up))
            Fs = ws_gate.shape[1]
            for s in range(S):
                o += h[:, s * Fs:(s + 1) * Fs] @ wsd[s].T
        out[s0:e0] = bf16_from_f64(o)
    return ylat, out


# ----------------------------------------------------------------------------
# Backward of the branch: whole rows of the weight gradients.  Each weight
# gradient is a sum over tokens (or bank rows) of an outer product; a row of
# it needs only one column of one factor, so the oracle can give a whole row
# (for the tolerance scale of a sampled row, and to check every entry of it)
# at full size.  Same definitions and rounding points as orc_*_backward.
# ----------------------------------------------------------------------------

def _silu_grad(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def outer_rows(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """bf16(p^T . q) for p [n, r] and q [n, c] (float64 operands): rows of a
    weight gradient that sums p[t, i] q[t, :] over t."""
    return bf16_from_f64(p.T @ q)


def expert_wgrad_rows(u: np.ndarray, dy: np.ndarray, wg_t, wu_t, wd_t, f_idx):
    """One local expert's weight gradients at intermediate units f_idx
    (orc_expert_ffn_backward): u [n, L] its bank rows, dy [n, L] their output
    gradients.  Returns dw_gate[f_idx, :], dw_up[f_idx, :] and
    dw_down[:, f_idx]^T, each [len(f_idx), L]:
      d_h = bf16(dy . W_d[:, f]), a, b = u.W_g[f], u.W_u[f],
      d_a = bf16(d_h b silu'(a)), d_b = bf16(d_h silu(a)), h = bf16(silu(a) b),
      dw_gate[f] = bf16(sum_r d_a u), dw_up[f] = bf16(sum_r d_b u),
      dw_down[:, f] = bf16(sum_r dy h[f])."""
    f_idx = np.asarray(f_idx, np.int64)
    wg, wu, wd = to_f64(wg_t[f_idx]), to_f64(wu_t[f_idx]), to_f64(wd_t[:, f_idx])
    L = u.shape[1]
    gg, gu, gd = (np.zeros((len(f_idx), L)) for _ in range(3))
    for s, e in _rows(u.shape[0]):          # float64 sums over the rows, chunk by chunk
        U, DY = to_f64(u[s:e]), to_f64(dy[s:e])
        a = U @ wg.T
        b = U @ wu.T
        dh = to_f64(bf16_from_f64(DY @ wd))
        gg += to_f64(bf16_from_f64(dh * b * _silu_grad(a))).T @ U
        gu += to_f64(bf16_from_f64(dh * _silu(a))).T @ U
        gd += to_f64(bf16_from_f64(_silu(a) * b)).T @ DY
    return bf16_from_f64(gg), bf16_from_f64(gu), bf16_from_f64(gd)


def shared_down_wgrad_cols(x, ws_gate, ws_up, d_out, sh: int, f_idx):
    """dws_down[sh][:, f_idx]^T ([len(f_idx), D]) = bf16(sum_t h_s[t, f] d_out[t])
    with h_s = bf16(silu(x.W_sg,s) (x.W_su,s)) (orc_combine_backward)."""
    f_idx = np.asarray(f_idx, np.int64)
    X = to_f64(x)
    a = X @ to_f64(ws_gate[sh][f_idx]).T
    b = X @ to_f64(ws_up[sh][f_idx]).T
    return outer_rows(to_f64(bf16_from_f64(_silu(a) * b)), to_f64(d_out))


def pack_dz(d, d_pools, topk, slot, pool_offsets=None) -> np.ndarray:
    """dz[t] = bf16(sum over kept (t, j) of d_pools[row(t, j)])
    (orc_pack_backward; j ascending; ragged: segments at pool_offsets, a slot
    past its segment adds nothing)."""
    rows = returned_rows(d, pool_offsets, topk, slot, np.arange(d.T))
    acc = np.zeros((d.T, d.latent))
    for j in range(d.top_k):
        m = rows[:, j] >= 0
        acc[m] += to_f64(d_pools[rows[m, j]])
    return bf16_from_f64(acc)
