"""ctypes front end of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg.  The product path never imports it.

Arrays are numpy: bf16 tensors travel as uint16 bit patterns.  Weights are
stored output-major ([out, in]); see oracle.h for every layout.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "d_model", "latent", "n_experts", "n_ranks", "top_k", "n_waves",
        "d_ff", "n_shared", "d_ff_shared", "cap_send", "cap_recv", "wave_mode", "dedup")]


def build() -> str:
    """Compile liboracle.so with gcc (single-threaded, IEEE, no fast-math)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared",
                           _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The loaded oracle.  ORACLE_LIB names another build of oracle.c to load
    instead (the sanitizer build of tests/test_oracle_sanitized.py)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        dp = ctypes.POINTER(Dims)
        vp = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        sig = {
            "orc_bf16_from_double": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_tokens_per_wave": (i32, [i32, i32]),
            "orc_capacity": (i64, [i64, i32, i32, i64, i64]),
            "orc_route": (None, [_f32p, i64, i32, i32, _i32p, _f32p]),
            "orc_route_biased": (None, [_f32p, _f32p, i64, i32, i32, _i32p, _f32p]),
            "orc_expert_counts": (None, [_i32p, i64, i32, _i32p]),
            "orc_route_ex": (None, [_f32p, vp, i64, i32, i32, i32, _i32p, _f32p]),
            "orc_balance_bias": (None, [_i32p, i32, i32, ctypes.c_double, _f32p]),
            "orc_latent_rows": (None, [_u16p, i32, _u16p, i32, vp, i64, _u16p]),
            "orc_sender": (i64, [dp, _i32p, _i32p, _i32p, _i32p, vp]),
            "orc_pack_rows": (None, [dp, _u16p, _i32p, _i32p, vp, _u8p, i64]),
            "orc_bank_slots": (i64, [dp, i32, _i32p, vp, i64, vp, _i32p, _i32p,
                                     _i32p, ctypes.POINTER(i32)]),
            "orc_bank_rows": (None, [dp, _u8p, vp, _i32p, _i32p, _u16p]),
            "orc_ffn_row": (None, [i32, i32, _u16p, _u16p, _u16p, _u16p, _u16p]),
            "orc_expert_ffn": (None, [dp, _u16p, vp, _i32p, _i32p, _u16p, _u16p,
                                      _u16p, _u16p, i64]),
            "orc_combine_tokens": (None, [dp, _u16p, vp, _i32p, _i32p, _f32p,
                                          _u16p, _u16p, _u16p, _u16p, _u16p, vp,
                                          i64, _u16p, _u16p]),
            "orc_route_backward": (None, [_f32p, vp, i64, i32, i32, i32, _i32p, _f32p,
                                          _f32p]),
            "orc_combine_backward": (None, [dp, _u16p, vp, i64, _i32p, _i32p, _f32p, _u16p,
                                            _u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p,
                                            _f32p, _u16p, _u16p, _u16p]),
            "orc_expert_ffn_backward": (None, [dp, _u16p, vp, _i32p, _i32p, _u16p, _u16p,
                                               _u16p, _u16p, i64, _u16p, _u16p, _u16p,
                                               _u16p]),
            "orc_pack_backward": (None, [dp, _u16p, vp, _i32p, _i32p, _u16p, _u16p, _u16p,
                                         _u16p, _u16p, _u16p, _u16p, _u16p, _u16p, _u16p]),
            "orc_combine_backward_tokens": (None, [dp, _u16p, vp, _i32p, _i32p, _f32p, _u16p,
                                                   _u16p, _u16p, _u16p, _u16p, _u16p, _i64p, i64,
                                                   _u16p, _f32p, _u16p]),
            "orc_combine_wgrad_entries": (None, [dp, _u16p, _u16p, _u16p, _u16p, _u16p, i32,
                                                 _i32p, _i32p, _i32p, i64, _u16p]),
            "orc_expert_ffn_backward_rows": (None, [dp, _u16p, vp, _i32p, _u16p, _u16p, _u16p,
                                                    _u16p, _i64p, i64, _u16p]),
            "orc_expert_wgrad_entries": (None, [dp, _u16p, vp, _i32p, _i32p, _u16p, _u16p,
                                                _u16p, _u16p, i32, i32, _i32p, _i32p, i64,
                                                _u16p]),
            "orc_pack_backward_tokens": (None, [dp, _u16p, vp, _i32p, _i32p, _u16p, _u16p,
                                                _u16p, _u16p, _i64p, i64, _u16p, _u16p]),
            "orc_pack_wgrad_entries": (None, [dp, _u16p, vp, _i32p, _i32p, _u16p, _u16p, i32,
                                              _i32p, _i32p, _i32p, i64, _u16p]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------
# dims and sizes
# ----------------------------------------------------------------------------

def tokens_per_wave(T: int, W: int) -> int:
    return lib().orc_tokens_per_wave(T, W)


def capacity(tokens_per_wave_: int, top_k: int, groups: int, num: int, den: int) -> int:
    return lib().orc_capacity(tokens_per_wave_, top_k, groups, num, den)


def dims(cfg, T=None) -> Dims:
    """Dims of a workload, capacities from the oracle's own formula."""
    T = cfg.T if T is None else T
    tw = tokens_per_wave(T, cfg.n_waves)
    if cfg.cf_send is None:
        cs = cr = 0
    else:
        cs = capacity(tw, cfg.top_k, cfg.n_ranks, cfg.cf_send.numerator, cfg.cf_send.denominator)
        cr = capacity(tw, cfg.top_k, cfg.experts_per_rank, cfg.cf_recv.numerator,
                      cfg.cf_recv.denominator)
    if (cfg.waves == "chunks" or cfg.dedup) and not cs:
        raise ValueError("chunked waves and dedup need a fixed sender capacity")
    return Dims(T, cfg.d_model, cfg.latent, cfg.n_experts, cfg.n_ranks, cfg.top_k,
                cfg.n_waves, cfg.d_ff, cfg.n_shared, cfg.d_ff_shared, cs, cr,
                1 if cfg.waves == "chunks" else 0, 1 if cfg.dedup else 0)


def row_bytes(d: Dims) -> int:
    return d.latent * 2 + 16


def n_pool_rows(d: Dims) -> int:
    return d.n_ranks * d.n_waves * d.cap_send if d.cap_send else d.T * d.top_k


def n_bank_rows(d: Dims, n_recv_rows: int) -> int:
    El = d.n_experts // d.n_ranks
    return d.n_waves * El * d.cap_recv if d.cap_send else n_recv_rows


# ----------------------------------------------------------------------------
# stages
# ----------------------------------------------------------------------------

def bf16_from_double(v: float) -> int:
    return lib().orc_bf16_from_double(v)


def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(b)


def route(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    topk = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float32)
    lib().orc_route(logits, T, E, k, topk, gates)
    return topk, gates


def route_biased(logits: np.ndarray, bias: np.ndarray, k: int):
    """Router on fp32(logits + bias) ([P1] section 四, appendix A.2)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    bias = np.ascontiguousarray(bias, dtype=np.float32)
    T, E = logits.shape
    topk = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float32)
    lib().orc_route_biased(logits, bias, T, E, k, topk, gates)
    return topk, gates


def route_ex(logits: np.ndarray, k: int, bias=None, renorm=False):
    """Router with an optional bias and optionally renormalised gates."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    topk = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().orc_route_ex(logits, None if b is None else b.ctypes.data, T, E, k, int(renorm),
                       topk, gates)
    return topk, gates


def expert_counts(topk: np.ndarray, E: int) -> np.ndarray:
    """Selections of each expert in one batch ([P1] appendix A.2)."""
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    counts = np.empty(E, np.int32)
    lib().orc_expert_counts(topk.reshape(-1), topk.size, E, counts)
    return counts


def balance_bias(window: np.ndarray, alpha: float) -> np.ndarray:
    """b_i = -alpha (f_i - 1/E) over the batches of `window` [N, E] ([P1] appendix A.2)."""
    window = np.ascontiguousarray(window, dtype=np.int32)
    n, E = window.shape
    bias = np.empty(E, np.float32)
    lib().orc_balance_bias(window.reshape(-1), n, E, float(alpha), bias)
    return bias


def latent(x: np.ndarray, w_ld_t: np.ndarray, rows=None) -> np.ndarray:
    x = np.ascontiguousarray(x, np.uint16)
    w = np.ascontiguousarray(w_ld_t, np.uint16)
    L, D = w.shape
    r = None if rows is None else np.ascontiguousarray(rows, np.int64)
    n = x.shape[0] if r is None else len(r)
    z = np.empty((n, L), np.uint16)
    lib().orc_latent_rows(x, D, w, L, _ptr(r), n, z)
    return z


def sender(d: Dims, topk: np.ndarray):
    topk = np.ascontiguousarray(topk, np.int32)
    P = d.n_ranks * d.n_waves
    slot = np.empty((d.T, d.top_k), np.int32)
    fill = np.empty(P, np.int32)
    demand = np.empty(P, np.int32)
    offs = np.zeros(P + 1, np.int64) if d.cap_send == 0 else None
    drops = lib().orc_sender(ctypes.byref(d), topk, slot, fill, demand, _ptr(offs))
    return dict(slot=slot, fill=fill, demand=demand, pool_offsets=offs, drops=drops)


def pack_rows(d: Dims, z, topk, slot, pool_offsets=None) -> np.ndarray:
    n = n_pool_rows(d)
    pools = np.empty((n, row_bytes(d)), np.uint8)
    lib().orc_pack_rows(ctypes.byref(d), np.ascontiguousarray(z, np.uint16),
                        np.ascontiguousarray(topk, np.int32),
                        np.ascontiguousarray(slot, np.int32), _ptr(pool_offsets),
                        pools, n)
    return pools


def headers(rows: np.ndarray, latent_: int) -> np.ndarray:
    """Tail ids of a [n, row_bytes] uint8 array of pool / receive rows."""
    return np.ascontiguousarray(rows[:, latent_ * 2:latent_ * 2 + 4]).view(np.int32).reshape(-1)


def row_ids(rows: np.ndarray, latent_: int) -> np.ndarray:
    """All four tail ids of each row: [n, 4] (the dedup variant's headers)."""
    return np.ascontiguousarray(rows[:, latent_ * 2:latent_ * 2 + 16]).view(np.int32).reshape(-1, 4)


def recv_ids(d: Dims, rows: np.ndarray) -> np.ndarray:
    """What orc_bank_slots reads of receive rows: the first tail id of each,
    or all four with dedup."""
    return row_ids(rows, d.latent) if d.dedup else headers(rows, d.latent)


def bank_slots(d: Dims, rank: int, hdr: np.ndarray, recv_offsets=None):
    hdr = np.ascontiguousarray(hdr, np.int32)
    El = d.n_experts // d.n_ranks
    G = d.n_waves * El
    n_recv = len(hdr)                       # rows ([n, 4] ids with dedup)
    nb = n_bank_rows(d, n_recv)
    bank_src = np.empty(nb, np.int32)
    bfill = np.empty(G, np.int32)
    bdemand = np.empty(G, np.int32)
    boffs = np.zeros(G + 1, np.int64) if d.cap_send == 0 else None
    bad = ctypes.c_int32(0)
    ro = None if recv_offsets is None else np.ascontiguousarray(recv_offsets, np.int64)
    drops = lib().orc_bank_slots(ctypes.byref(d), rank, hdr, _ptr(ro), n_recv,
                                 _ptr(boffs), bank_src, bfill, bdemand, ctypes.byref(bad))
    return dict(bank_src=bank_src, bfill=bfill, bdemand=bdemand, bank_offsets=boffs,
                bad_rows=bad.value, drops=drops)


def bank_rows(d: Dims, recv: np.ndarray, bank_offsets, bank_src, bfill) -> np.ndarray:
    bank = np.zeros((len(bank_src), d.latent), np.uint16)
    lib().orc_bank_rows(ctypes.byref(d), np.ascontiguousarray(recv, np.uint8),
                        _ptr(bank_offsets), np.ascontiguousarray(bank_src, np.int32),
                        np.ascontiguousarray(bfill, np.int32), bank)
    return bank


def ffn_row(u, wg_t, wu_t, wd_t) -> np.ndarray:
    F, L = wg_t.shape
    y = np.empty(L, np.uint16)
    lib().orc_ffn_row(L, F, np.ascontiguousarray(u, np.uint16),
                      np.ascontiguousarray(wg_t, np.uint16),
                      np.ascontiguousarray(wu_t, np.uint16),
                      np.ascontiguousarray(wd_t, np.uint16), y)
    return y


def expert_ffn(d: Dims, bank, bank_offsets, bank_src, bfill, w_gate, w_up, w_down,
               n_ret_rows: int) -> np.ndarray:
    ret = np.empty((n_ret_rows, d.latent), np.uint16)
    lib().orc_expert_ffn(ctypes.byref(d), np.ascontiguousarray(bank, np.uint16),
                         _ptr(bank_offsets), np.ascontiguousarray(bank_src, np.int32),
                         np.ascontiguousarray(bfill, np.int32),
                         np.ascontiguousarray(w_gate, np.uint16),
                         np.ascontiguousarray(w_up, np.uint16),
                         np.ascontiguousarray(w_down, np.uint16), ret, n_ret_rows)
    return ret


def combine(d: Dims, returned, ret_offsets, topk, slot, gates, x, w_lu_t,
            ws_gate, ws_up, ws_down, tokens=None):
    tk = None if tokens is None else np.ascontiguousarray(tokens, np.int64)
    n = d.T if tk is None else len(tk)
    ylat = np.empty((n, d.latent), np.uint16)
    out = np.empty((n, d.d_model), np.uint16)
    lib().orc_combine_tokens(
        ctypes.byref(d), np.ascontiguousarray(returned, np.uint16), _ptr(ret_offsets),
        np.ascontiguousarray(topk, np.int32), np.ascontiguousarray(slot, np.int32),
        np.ascontiguousarray(gates, np.float32), np.ascontiguousarray(x, np.uint16),
        np.ascontiguousarray(w_lu_t, np.uint16), np.ascontiguousarray(ws_gate, np.uint16),
        np.ascontiguousarray(ws_up, np.uint16), np.ascontiguousarray(ws_down, np.uint16),
        _ptr(tk), n, ylat, out)
    return ylat, out


# ----------------------------------------------------------------------------
# backward of the branch (ragged mode: pass the segment / group offsets)
# ----------------------------------------------------------------------------

def _u16(a):
    return np.ascontiguousarray(a, np.uint16)


def route_backward(logits, topk, d_gates, bias=None, renorm=False):
    """d_logits [T, E] fp32 from the gradient of the gates."""
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    k = topk.shape[1]
    out = np.empty((T, E), np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().orc_route_backward(logits, None if b is None else b.ctypes.data, T, E, k, int(renorm),
                             np.ascontiguousarray(topk, np.int32),
                             np.ascontiguousarray(d_gates, np.float32), out)
    return out


def combine_backward(d: Dims, returned, topk, slot, gates, x, ylat, w_lu_t, ws_gate, ws_up,
                     ws_down, d_out, ret_offsets=None):
    """(d_returned (returned's rows), d_gates, d_shared [T, 2, S, Fs], dw_lat_up,
    dws_down); ret_offsets: returned's segments in ragged mode."""
    T, L, D, S, Fs = d.T, d.latent, d.d_model, d.n_shared, d.d_ff_shared
    n_rows = len(returned)
    ro = None if ret_offsets is None else np.ascontiguousarray(ret_offsets, np.int64)
    d_ret = np.empty((n_rows, L), np.uint16)
    d_gates = np.empty((T, d.top_k), np.float32)
    d_shared = np.empty((T, 2, S, Fs), np.uint16)
    dw_lu = np.empty((D, L), np.uint16)
    dws_down = np.empty((S, D, Fs), np.uint16)
    lib().orc_combine_backward(
        ctypes.byref(d), _u16(returned), _ptr(ro), n_rows, np.ascontiguousarray(topk, np.int32),
        np.ascontiguousarray(slot, np.int32), np.ascontiguousarray(gates, np.float32), _u16(x),
        _u16(ylat), _u16(w_lu_t), _u16(ws_gate), _u16(ws_up), _u16(ws_down), _u16(d_out),
        d_ret, d_gates, d_shared, dw_lu, dws_down)
    return d_ret, d_gates, d_shared, dw_lu, dws_down


def expert_ffn_backward(d: Dims, bank, bank_src, bfill, w_gate, w_up, w_down, d_ret,
                        bank_offsets=None):
    """(d_recv, dw_gate, dw_up, dw_down) of one rank's experts; bank_offsets:
    the bank's groups in ragged mode."""
    bo = None if bank_offsets is None else np.ascontiguousarray(bank_offsets, np.int64)
    El = d.n_experts // d.n_ranks
    n_ret = len(d_ret)
    d_recv = np.empty((n_ret, d.latent), np.uint16)
    dwg = np.empty((El, d.d_ff, d.latent), np.uint16)
    dwu = np.empty_like(dwg)
    dwd = np.empty((El, d.latent, d.d_ff), np.uint16)
    lib().orc_expert_ffn_backward(
        ctypes.byref(d), _u16(bank), _ptr(bo), np.ascontiguousarray(bank_src, np.int32),
        np.ascontiguousarray(bfill, np.int32), _u16(w_gate), _u16(w_up), _u16(w_down),
        _u16(d_ret), n_ret, d_recv, dwg, dwu, dwd)
    return d_recv, dwg, dwu, dwd


def pack_backward(d: Dims, d_pools, topk, slot, x, d_shared, w_ld_t, ws_gate, ws_up,
                  pool_offsets=None):
    """(dz, dx, dw_lat_down, dws_gate, dws_up); pool_offsets: d_pools'
    segments in ragged mode."""
    po = None if pool_offsets is None else np.ascontiguousarray(pool_offsets, np.int64)
    T, L, D, S, Fs = d.T, d.latent, d.d_model, d.n_shared, d.d_ff_shared
    dz = np.empty((T, L), np.uint16)
    dx = np.empty((T, D), np.uint16)
    dw_ld = np.empty((L, D), np.uint16)
    dwsg = np.empty((S, Fs, D), np.uint16)
    dwsu = np.empty_like(dwsg)
    lib().orc_pack_backward(
        ctypes.byref(d), _u16(d_pools), _ptr(po), np.ascontiguousarray(topk, np.int32),
        np.ascontiguousarray(slot, np.int32), _u16(x), _u16(d_shared), _u16(w_ld_t),
        _u16(ws_gate), _u16(ws_up), dz, dx, dw_ld, dwsg, dwsu)
    return dz, dx, dw_ld, dwsg, dwsu


# sampled outputs (full-size checks)

def _i32(a):
    return np.ascontiguousarray(a, np.int32)


def _i64(a):
    return np.ascontiguousarray(a, np.int64)


def combine_backward_tokens(d: Dims, returned, topk, slot, gates, x, w_lu_t, ws_gate, ws_up,
                            ws_down, d_out, tokens, ret_offsets=None):
    """(d_ret_rows [n, k, L], d_gates [n, k], d_shared [n, 2, S, Fs]) for tokens."""
    tk = _i64(tokens)
    ro = None if ret_offsets is None else _i64(ret_offsets)
    n, k, L = len(tk), d.top_k, d.latent
    rows = np.empty((n, k, L), np.uint16)
    dg = np.empty((n, k), np.float32)
    dsh = np.empty((n, 2, d.n_shared, d.d_ff_shared), np.uint16)
    lib().orc_combine_backward_tokens(
        ctypes.byref(d), _u16(returned), _ptr(ro), _i32(topk), _i32(slot),
        np.ascontiguousarray(gates, np.float32), _u16(x), _u16(w_lu_t), _u16(ws_gate),
        _u16(ws_up), _u16(ws_down), _u16(d_out), tk, n, rows, dg, dsh)
    return rows, dg, dsh


def combine_wgrad_entries(d: Dims, x, ylat, ws_gate, ws_up, d_out, which, ra, cb, sh=None):
    """which 0: dw_lat_up[ra, cb]; 1: dws_down[sh, ra, cb]."""
    n = len(ra)
    out = np.empty(n, np.uint16)
    shi = _i32(np.zeros(n) if sh is None else sh)
    lib().orc_combine_wgrad_entries(ctypes.byref(d), _u16(x), _u16(ylat), _u16(ws_gate),
                                    _u16(ws_up), _u16(d_out), which, shi, _i32(ra), _i32(cb), n,
                                    out)
    return out


def expert_ffn_backward_rows(d: Dims, bank, bank_src, w_gate, w_up, w_down, d_ret, pos,
                             bank_offsets=None):
    """d_u [n, L] of kept bank positions pos (written to d_recv[bank_src[pos]])."""
    p = _i64(pos)
    bo = None if bank_offsets is None else _i64(bank_offsets)
    out = np.empty((len(p), d.latent), np.uint16)
    lib().orc_expert_ffn_backward_rows(ctypes.byref(d), _u16(bank), _ptr(bo), _i32(bank_src),
                                       _u16(w_gate), _u16(w_up), _u16(w_down), _u16(d_ret), p,
                                       len(p), out)
    return out


def expert_wgrad_entries(d: Dims, bank, bank_src, bfill, w_gate, w_up, w_down, d_ret, j, which,
                         ra, cb, bank_offsets=None):
    """which 0: dw_gate[j, ra, cb]; 1: dw_up[j, ra, cb]; 2: dw_down[j, ra, cb]."""
    n = len(ra)
    bo = None if bank_offsets is None else _i64(bank_offsets)
    out = np.empty(n, np.uint16)
    lib().orc_expert_wgrad_entries(ctypes.byref(d), _u16(bank), _ptr(bo), _i32(bank_src),
                                   _i32(bfill),
                                   _u16(w_gate), _u16(w_up), _u16(w_down), _u16(d_ret), j, which,
                                   _i32(ra), _i32(cb), n, out)
    return out


def pack_backward_tokens(d: Dims, d_pools, topk, slot, d_shared, w_ld_t, ws_gate, ws_up, tokens,
                         pool_offsets=None):
    """(dz [n, L], dx [n, D]) for tokens."""
    tk = _i64(tokens)
    po = None if pool_offsets is None else _i64(pool_offsets)
    dz = np.empty((len(tk), d.latent), np.uint16)
    dx = np.empty((len(tk), d.d_model), np.uint16)
    lib().orc_pack_backward_tokens(ctypes.byref(d), _u16(d_pools), _ptr(po), _i32(topk),
                                   _i32(slot),
                                   _u16(d_shared), _u16(w_ld_t), _u16(ws_gate), _u16(ws_up), tk,
                                   len(tk), dz, dx)
    return dz, dx


def pack_wgrad_entries(d: Dims, d_pools, topk, slot, x, d_shared, which, ra, cb, sh=None,
                       pool_offsets=None):
    """which 0: dw_lat_down[ra, cb]; 1: dws_gate[sh, ra, cb]; 2: dws_up[sh, ra, cb]."""
    n = len(ra)
    po = None if pool_offsets is None else _i64(pool_offsets)
    out = np.empty(n, np.uint16)
    shi = _i32(np.zeros(n) if sh is None else sh)
    lib().orc_pack_wgrad_entries(ctypes.byref(d), _u16(d_pools), _ptr(po), _i32(topk),
                                 _i32(slot), _u16(x), _u16(d_shared), which, shi, _i32(ra),
                                 _i32(cb), n, out)
    return out
