"""Pins of the oracle's backward of the branch.

The oracle's gradients (chain rule written out by hand, bf16 rounding points
of its own) are checked against numbers that do not come from it:

- the router's logit gradient against central finite differences of a numpy
  softmax, and against torch autograd;
- the whole branch -- 8 ranks, exact exchanges in both directions, fixed
  capacities or ragged (dropless) -- against torch autograd (float64, no
  rounding) of a plain per-token forward that uses the keep decisions of the
  brute-force definition: every input and weight gradient, summed over
  shards where the weight is shared.

The two sides differ only by the oracle's bf16 rounding points, so the
comparison is per tensor within a few bf16 units; a dropped term, a wrong
sign, a transposed weight or a swapped gate / up gradient is far outside.
"""
import numpy as np
import pytest
import torch

from conftest import f64, u16
from test_oracle_e2e import brute_force, simulate
from synth import configs

F = torch.nn.functional
ERRS = []


def _close(got, ref, what, rel=1.5e-2, mx=5e-2):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    scale = np.abs(ref).max()
    assert scale > 0, what
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    ERRS.append((what, err))
    assert err < rel, f"{what}: relative error {err:.3g}"
    assert np.abs(got - ref).max() <= mx * scale, f"{what}: max error"


def _bf(v):
    return f64(u16(torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)))


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

def _gates_np(l, topk, renorm):
    l = l - l.max(axis=1, keepdims=True)
    if renorm:
        sel = np.take_along_axis(l, topk, 1)
        return np.exp(sel) / np.exp(sel).sum(1, keepdims=True)
    p = np.exp(l) / np.exp(l).sum(1, keepdims=True)
    return np.take_along_axis(p, topk, 1)


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("biased", [False, True])
def test_route_backward_finite_differences(orc, renorm, biased):
    rng = np.random.default_rng(40 + renorm + 2 * biased)
    T, E, k = 5, 12, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32) if biased else None
    topk, _ = orc.route_ex(lg, k, bias=bias, renorm=renorm)
    dg = rng.standard_normal((T, k)).astype(np.float32)
    got = orc.route_backward(lg, topk, dg, bias=bias, renorm=renorm)
    lb = (lg + bias if biased else lg).astype(np.float32).astype(np.float64)
    ref = np.zeros((T, E))
    h = 1e-6
    for t in range(T):
        for e in range(E):
            a, b = lb.copy(), lb.copy()
            a[t, e] += h
            b[t, e] -= h
            ref[t, e] = ((_gates_np(a, topk, renorm) - _gates_np(b, topk, renorm)) * dg).sum() / (2 * h)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-7)
    # torch autograd on the same definition
    lt = torch.tensor(lb, requires_grad=True)
    idx = torch.from_numpy(topk.astype(np.int64))
    g = (torch.softmax(lt.gather(1, idx), 1) if renorm else
         torch.softmax(lt, 1).gather(1, idx))
    (g * torch.from_numpy(dg.astype(np.float64))).sum().backward()
    np.testing.assert_allclose(got, lt.grad.numpy(), rtol=1e-5, atol=1e-7)
    if renorm:   # only the chosen logits move the renormalised gates
        mask = np.zeros((T, E), bool)
        np.put_along_axis(mask, topk, True, 1)
        assert (got[~mask] == 0).all()
    else:        # softmax is shift invariant: each row of the gradient sums to 0
        np.testing.assert_allclose(got.sum(1), 0, atol=1e-6)


# ----------------------------------------------------------------------------
# whole branch, 8 ranks
# ----------------------------------------------------------------------------

def oracle_backward(orc, cfg, d, W_, S, BK, OUT, d_out):
    """Backward of every shard and rank with exact exchanges, from the oracle
    (fixed capacities, or ragged: segments at each side's offsets)."""
    R, W, Cs = cfg.n_ranks, cfg.n_waves, d.cap_send

    def send_seg(s, dst, w):      # rows of shard s's pools (dst, w)
        if Cs:
            return slice((dst * W + w) * Cs, (dst * W + w + 1) * Cs)
        o = S[s]["pool_offsets"]
        return slice(int(o[dst * W + w]), int(o[dst * W + w + 1]))

    # rank r's receive layout: segments (source s, wave w) of shard s's demand
    lens = [[int(S[s]["demand"][r * W + w]) for s in range(R) for w in range(W)]
            for r in range(R)]
    RO = [np.concatenate([[0], np.cumsum(l)]).astype(np.int64) for l in lens]

    def recv_seg(r, s, w):        # rows of rank r's receive buffer (s, w)
        if Cs:
            return slice((s * W + w) * Cs, (s * W + w + 1) * Cs)
        return slice(int(RO[r][s * W + w]), int(RO[r][s * W + w + 1]))

    po = lambda s: None if Cs else S[s]["pool_offsets"]
    CB = []
    for s in range(R):
        CB.append(orc.combine_backward(d, S[s]["returned"], S[s]["topk"], S[s]["slot"],
                                       S[s]["gates"], W_["x"][s], OUT[s][0], W_["wlu"],
                                       W_["wsg"], W_["wsu"], W_["wsd"], d_out[s],
                                       ret_offsets=po(s)))
    # return exchange, reversed: rank r's rows (s, w, i) are shard s's rows (r, w, i)
    EB = []
    for r in range(R):
        d_ret = np.concatenate([CB[s][0][send_seg(s, r, w)] for s in range(R) for w in range(W)])
        EB.append(orc.expert_ffn_backward(d, BK[r]["bank"], BK[r]["bank_src"], BK[r]["bfill"],
                                          *W_["ex"][r], d_ret,
                                          bank_offsets=BK[r]["bank_offsets"]))
    PB, DL = [], []
    for s in range(R):
        d_pools = np.concatenate([EB[r][0][recv_seg(r, s, w)] for r in range(R) for w in range(W)])
        PB.append(orc.pack_backward(d, d_pools, S[s]["topk"], S[s]["slot"], W_["x"][s],
                                    CB[s][2], W_["wld"], W_["wsg"], W_["wsu"], pool_offsets=po(s)))
        DL.append(orc.route_backward(W_["logits"][s], S[s]["topk"], CB[s][1]))
    return CB, EB, PB, DL


def torch_backward(cfg, W_, S, keep, d_out):
    """float64 autograd of the per-token forward with the given keep mask."""
    R, El = cfg.n_ranks, cfg.experts_per_rank
    leaf = lambda a: torch.tensor(f64(a), requires_grad=True)
    X = [leaf(x) for x in W_["x"]]
    LG = [torch.tensor(np.asarray(l, np.float64), requires_grad=True) for l in W_["logits"]]
    wld, wlu = leaf(W_["wld"]), leaf(W_["wlu"])
    wsg, wsu, wsd = leaf(W_["wsg"]), leaf(W_["wsu"]), leaf(W_["wsd"])
    ex = [[leaf(w) for w in W_["ex"][r]] for r in range(R)]
    loss = 0
    for s in range(R):
        x = X[s]
        z = x @ wld.T
        topk = torch.from_numpy(S[s]["topk"].astype(np.int64))
        g = torch.softmax(LG[s], 1).gather(1, topk)
        kp = torch.from_numpy(keep[s])
        ylat = torch.zeros(cfg.T, cfg.latent, dtype=torch.float64)
        for e in range(cfg.n_experts):
            t, j = torch.nonzero((topk == e) & kp, as_tuple=True)
            if len(t) == 0:
                continue
            wg, wu, wd = (w[e % El] for w in ex[e // El])
            u = z[t]
            y = (F.silu(u @ wg.T) * (u @ wu.T)) @ wd.T
            ylat = ylat.index_add(0, t, g[t, j][:, None] * y)
        out = ylat @ wlu.T
        for sh in range(cfg.n_shared):
            out = out + (F.silu(x @ wsg[sh].T) * (x @ wsu[sh].T)) @ wsd[sh].T
        loss = loss + (out * torch.from_numpy(f64(d_out[s]))).sum()
    loss.backward()
    return X, LG, wld, wlu, wsg, wsu, wsd, ex


@pytest.mark.parametrize("case", ["1.10/1.15", "tight", "chunks", "t16", "t16_k1_w1_s0",
                                  "ragged", "t16_ragged_w1"])
def test_branch_backward_matches_autograd(orc, case):
    from dataclasses import replace
    from fractions import Fraction
    cfg = configs.TINY
    if case == "ragged":              # dropless: pools and bank sized from exact counts
        cfg = replace(cfg, cf_send=None, cf_recv=None)
    elif case == "t16_ragged_w1":
        cfg = replace(cfg, T=16, n_waves=1, cf_send=None, cf_recv=None)
    elif case == "t16":               # 16 tokens per shard: the quick case
        cfg = replace(cfg, T=16)
    elif case == "t16_k1_w1_s0":      # top-1, one wave, no shared experts
        cfg = replace(cfg, T=16, top_k=1, n_waves=1, n_shared=0)
    elif case == "tight":
        cfg = replace(cfg, cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2))
    elif case == "chunks":
        cfg = replace(cfg, waves="chunks")
    d, W_, S, BK, OUT = simulate(orc, cfg)
    keep = [k for _, _, k in brute_force(cfg, d, W_, S)]
    rng = np.random.default_rng(50)
    d_out = [u16(torch.from_numpy(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32))
                 .to(torch.bfloat16)) for _ in range(cfg.n_ranks)]
    CB, EB, PB, DL = oracle_backward(orc, cfg, d, W_, S, BK, OUT, d_out)
    X, LG, wld, wlu, wsg, wsu, wsd, ex = torch_backward(cfg, W_, S, keep, d_out)
    for s in range(cfg.n_ranks):
        _close(f64(PB[s][1]), X[s].grad.numpy(), f"dx shard {s}")
        _close(DL[s], LG[s].grad.numpy(), f"d_logits shard {s}")
    R = cfg.n_ranks
    _close(sum(f64(PB[s][2]) for s in range(R)), wld.grad.numpy(), "dw_lat_down")
    _close(sum(f64(CB[s][3]) for s in range(R)), wlu.grad.numpy(), "dw_lat_up")
    if cfg.n_shared:
        _close(sum(f64(PB[s][3]) for s in range(R)), wsg.grad.numpy(), "dws_gate")
        _close(sum(f64(PB[s][4]) for s in range(R)), wsu.grad.numpy(), "dws_up")
        _close(sum(f64(CB[s][4]) for s in range(R)), wsd.grad.numpy(), "dws_down")
    else:
        assert all(PB[s][3].size == PB[s][4].size == CB[s][4].size == 0 for s in range(R))
    for r in range(R):
        for i, name in ((1, "dw_gate"), (2, "dw_up"), (3, "dw_down")):
            ref = ex[r][i - 1].grad.numpy()
            got = f64(EB[r][i])
            for j in range(cfg.experts_per_rank):
                if np.abs(ref[j]).max() == 0:      # an expert no kept row reached
                    assert (got[j] == 0).all()
                else:
                    _close(got[j], ref[j], f"{name} rank {r} expert {j}")


def test_backward_structure(orc):
    """Zero rows and zero gates exactly where nothing was kept."""
    from dataclasses import replace
    from fractions import Fraction
    cfg = replace(configs.TINY, cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2))
    d, W_, S, BK, OUT = simulate(orc, cfg)
    rng = np.random.default_rng(51)
    d_out = [u16(torch.from_numpy(rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32))
                 .to(torch.bfloat16)) for _ in range(cfg.n_ranks)]
    CB, EB, PB, DL = oracle_backward(orc, cfg, d, W_, S, BK, OUT, d_out)
    Cs, W = d.cap_send, cfg.n_waves
    for s in range(cfg.n_ranks):
        d_ret, d_g = CB[s][0], CB[s][1]
        assert (d_g[S[s]["slot"] < 0] == 0).all()
        for p, f in enumerate(S[s]["fill"]):
            assert (d_ret[p * Cs + f:(p + 1) * Cs] == 0).all()
            assert (np.abs(f64(d_ret[p * Cs:p * Cs + f])).sum(1) > 0).all()
    for r in range(cfg.n_ranks):
        kept = np.zeros(len(EB[r][0]), bool)
        kept[BK[r]["bank_src"][BK[r]["bank_src"] >= 0]] = True
        assert (EB[r][0][~kept] == 0).all()
    # d_returned of kept rows is exactly bf16(g * d_ylat): rows of one token are parallel
    s = 0
    t = int(np.nonzero((S[s]["slot"] >= 0).sum(1) >= 2)[0][0])
    js = np.nonzero(S[s]["slot"][t] >= 0)[0][:2]
    vecs = []
    for j in js:
        e, sl = int(S[s]["topk"][t, j]), int(S[s]["slot"][t, j])
        row = ((e // cfg.experts_per_rank) * W + t // int(np.ceil(cfg.T / W))) * Cs + sl
        vecs.append(f64(CB[s][0][row]) / float(S[s]["gates"][t, j]))
    np.testing.assert_allclose(vecs[0], vecs[1], rtol=1e-2, atol=1e-6 * np.abs(vecs[0]).max())


@pytest.mark.parametrize("waves", ["tokens", "chunks"])
def test_sampled_backward_equals_full(orc, waves):
    """The sampled-output functions (full-size GPU checks) give the full
    functions' values bit for bit, on random stage inputs."""
    from dataclasses import replace
    from synth import gen
    cfg = replace(configs.TINY, waves=waves)
    d = orc.dims(cfg)
    T, L, D, S, Fs, k = cfg.T, cfg.latent, cfg.d_model, cfg.n_shared, cfg.d_ff_shared, cfg.top_k
    El, F = cfg.experts_per_rank, cfg.d_ff
    rng = np.random.default_rng(70)
    pay = lambda n, w, i: u16(gen.payload_rows(n, w, i))
    n_rows = cfg.n_ranks * cfg.n_waves * d.cap_send
    x, lg = pay(T, D, 1), (rng.standard_normal((T, cfg.n_experts)) * 2).astype(np.float32)
    topk, gates = orc.route(lg, k)
    slot = orc.sender(d, topk)["slot"]
    returned, ylat, d_out = pay(n_rows, L, 2), pay(T, L, 3), pay(T, D, 4)
    wlu, wld = u16(gen.latent_up(cfg)), u16(gen.latent_down(cfg))
    wsg, wsu, wsd = (u16(w) for w in gen.shared(cfg))
    full = orc.combine_backward(d, returned, topk, slot, gates, x, ylat, wlu, wsg, wsu, wsd, d_out)
    tok = np.array([0, 5, 21, 22, 43, T - 1])
    rows, dg, dsh = orc.combine_backward_tokens(d, returned, topk, slot, gates, x, wlu, wsg, wsu,
                                                wsd, d_out, tok)
    Cs, W = d.cap_send, cfg.n_waves
    for r, t in enumerate(tok):
        assert np.array_equal(dg[r], full[1][t])
        assert np.array_equal(dsh[r], full[2][t])
        for j in range(k):
            s = slot[t, j]
            if s < 0:
                assert (rows[r, j] == 0).all()
                continue
            dst = topk[t, j] // El
            Tw = -(-T // W)
            row = dst * W * Cs + s if waves == "chunks" else (dst * W + t // Tw) * Cs + s
            assert np.array_equal(rows[r, j], full[0][row])
    ra, cb = rng.integers(0, D, 9), rng.integers(0, L, 9)
    assert np.array_equal(orc.combine_wgrad_entries(d, x, ylat, wsg, wsu, d_out, 0, ra, cb),
                          full[3][ra, cb])
    sh, cf = rng.integers(0, S, 9), rng.integers(0, Fs, 9)
    assert np.array_equal(orc.combine_wgrad_entries(d, x, ylat, wsg, wsu, d_out, 1, ra, cf, sh),
                          full[4][sh, ra, cf])
    # receiver
    hdr = np.concatenate([rng.integers(0, El, n_rows // 2), -np.ones(n_rows - n_rows // 2, int)])
    hdr = rng.permutation(hdr).astype(np.int32)
    bo = orc.bank_slots(d, 0, hdr, None)
    bank, d_ret = pay(len(bo["bank_src"]), L, 5), pay(n_rows, L, 6)
    wg, wu, wdn = (u16(w) for w in gen.rank_experts(cfg, 0))
    fe = orc.expert_ffn_backward(d, bank, bo["bank_src"], bo["bfill"], wg, wu, wdn, d_ret)
    pos = np.nonzero(bo["bank_src"] >= 0)[0][::7]
    du = orc.expert_ffn_backward_rows(d, bank, bo["bank_src"], wg, wu, wdn, d_ret, pos)
    assert np.array_equal(du, fe[0][bo["bank_src"][pos]])
    for which, ref in ((0, fe[1]), (1, fe[2]), (2, fe[3])):
        for j in range(El):
            a = rng.integers(0, ref.shape[1], 5)
            b = rng.integers(0, ref.shape[2], 5)
            got = orc.expert_wgrad_entries(d, bank, bo["bank_src"], bo["bfill"], wg, wu, wdn,
                                           d_ret, j, which, a, b)
            assert np.array_equal(got, ref[j, a, b]), (which, j)
    # sender
    d_pools, d_shared = pay(n_rows, L, 7), pay(T, 2 * S * Fs, 8).reshape(T, 2, S, Fs)
    fp = orc.pack_backward(d, d_pools, topk, slot, x, d_shared, wld, wsg, wsu)
    dz, dx = orc.pack_backward_tokens(d, d_pools, topk, slot, d_shared, wld, wsg, wsu, tok)
    assert np.array_equal(dz, fp[0][tok]) and np.array_equal(dx, fp[1][tok])
    ra, cb = rng.integers(0, L, 9), rng.integers(0, D, 9)
    assert np.array_equal(orc.pack_wgrad_entries(d, d_pools, topk, slot, x, d_shared, 0, ra, cb),
                          fp[2][ra, cb])
    for which, ref in ((1, fp[3]), (2, fp[4])):
        got = orc.pack_wgrad_entries(d, d_pools, topk, slot, x, d_shared, which, cf, cb, sh)
        assert np.array_equal(got, ref[sh, cf, cb])


def test_ragged_backward_bounds_and_sampled(orc):
    """Ragged mode: a choice whose slot lies past its returned segment (the
    forward read it as zero) gets gate gradient 0, writes no row and adds
    nothing to dz; every other d_returned row stays 0.  The sampled-output
    functions equal the full ones on the same ragged inputs."""
    from synth import gen
    T, D, L, E, R, k, W, S, Fs = 3, 8, 8, 8, 2, 2, 1, 1, 8
    d = orc.Dims(T, D, L, E, R, k, W, 8, S, Fs, 0, 0, 0, 0)
    topk = np.array([[0, 4], [1, 5], [2, 6]], np.int32)   # dest 0 and dest 1
    slot = np.array([[0, 0], [1, 5], [2, 1]], np.int32)
    gates = np.array([[0.5, 0.25], [1.0, 2.0], [0.75, 1.5]], np.float32)
    offs = np.array([0, 3, 5], np.int64)                  # seg 0: 3 rows, seg 1: 2 rows
    pay = lambda n, w, i: u16(gen.payload_rows(n, w, i))
    returned, x, ylat, d_out = pay(5, L, 1), pay(T, D, 2), pay(T, L, 3), pay(T, D, 4)
    wlu, wsg, wsu, wsd = pay(D, L, 5), pay(S * Fs, D, 6), pay(S * Fs, D, 7), pay(S * D, Fs, 8)
    wsg, wsu, wsd = wsg.reshape(S, Fs, D), wsu.reshape(S, Fs, D), wsd.reshape(S, D, Fs)
    d_ret, dg, dsh, _, _ = orc.combine_backward(d, returned, topk, slot, gates, x, ylat, wlu, wsg,
                                                wsu, wsd, d_out, ret_offsets=offs)
    assert dg[1, 1] == 0.0 and (dg[[0, 0, 1, 2, 2], [0, 1, 0, 0, 1]] != 0).all()
    dyl = f64(u16(torch.from_numpy(f64(d_out) @ f64(wlu)).float().to(torch.bfloat16)))
    for t, j, row in ((0, 0, 0), (0, 1, 3), (1, 0, 1), (2, 0, 2), (2, 1, 4)):
        np.testing.assert_allclose(f64(d_ret[row]), gates[t, j] * dyl[t], rtol=1e-2, atol=1e-6)
    rows, dgt, dsht = orc.combine_backward_tokens(d, returned, topk, slot, gates, x, wlu, wsg, wsu,
                                                  wsd, d_out, np.arange(T), ret_offsets=offs)
    assert np.array_equal(dgt, dg) and np.array_equal(dsht, dsh) and (rows[1, 1] == 0).all()
    d_pools = pay(5, L, 9)
    dz, dx, dwld, dwsg, dwsu = orc.pack_backward(d, d_pools, topk, slot, x, dsh, wld_t := pay(L, D, 10),
                                                 wsg, wsu, pool_offsets=offs)
    np.testing.assert_array_equal(f64(dz[1]), f64(d_pools[1]))   # slot 5 of seg 1 adds nothing
    dzt, dxt = orc.pack_backward_tokens(d, d_pools, topk, slot, dsh, wld_t, wsg, wsu, np.arange(T),
                                        pool_offsets=offs)
    assert np.array_equal(dzt, dz) and np.array_equal(dxt, dx)
    ra, cb = np.array([0, 3, 7]), np.array([1, 0, 6])
    assert np.array_equal(orc.pack_wgrad_entries(d, d_pools, topk, slot, x, dsh, 0, ra, cb,
                                                 pool_offsets=offs), dwld[ra, cb])
    # receiver: ragged bank of 2 waves x 1 expert... one rank's groups at offsets
    d2 = orc.Dims(T, D, L, E, R, k, 2, 8, S, Fs, 0, 0, 0, 0)
    El = E // R
    hdr = np.array([0, 1, 2, 3, 1, 0, 2, 2, 3, 1], np.int32)       # rank 0's experts
    ro = np.array([0, 3, 5, 8, 10], np.int64)                      # (source, wave) segments
    bo = orc.bank_slots(d2, 0, hdr, ro)
    bank = pay(len(bo["bank_src"]), L, 11)
    d_ret2 = pay(len(hdr), L, 12)
    wg, wu, wdn = pay(El * 8, L, 13).reshape(El, 8, L), pay(El * 8, L, 14).reshape(El, 8, L), \
        pay(El * L, 8, 15).reshape(El, L, 8)
    fe = orc.expert_ffn_backward(d2, bank, bo["bank_src"], bo["bfill"], wg, wu, wdn, d_ret2,
                                 bank_offsets=bo["bank_offsets"])
    pos = np.arange(len(hdr))
    du = orc.expert_ffn_backward_rows(d2, bank, bo["bank_src"], wg, wu, wdn, d_ret2, pos,
                                      bank_offsets=bo["bank_offsets"])
    assert np.array_equal(du, fe[0][bo["bank_src"][pos]])
    for which, ref in ((0, fe[1]), (1, fe[2]), (2, fe[3])):
        for j in range(El):
            a, b = np.array([0, 5, 7]), np.array([0, 3, 7])
            got = orc.expert_wgrad_entries(d2, bank, bo["bank_src"], bo["bfill"], wg, wu, wdn,
                                           d_ret2, j, which, a, b,
                                           bank_offsets=bo["bank_offsets"])
            assert np.array_equal(got, ref[j, a, b]), (which, j)
