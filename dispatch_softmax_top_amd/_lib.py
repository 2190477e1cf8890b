"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch device tensors (PyTorch supplies memory and the
stream); each function passes their raw pointers and the current HIP stream
and raises MoeError on a negative status.  There is no fallback: if the
library is missing or was not built, importing the functions raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

(MOE_CALL_ROUTE, MOE_CALL_PACK, MOE_CALL_BANK, MOE_CALL_FFN, MOE_CALL_COMBINE,
 MOE_CALL_COMBINE_SHARED, MOE_CALL_COMBINE_BWD, MOE_CALL_FFN_BWD, MOE_CALL_PACK_BWD) = range(9)


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class MoeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "d_model", "latent", "n_experts", "n_ranks", "top_k", "n_waves",
        "d_ff", "n_shared", "d_ff_shared", "cap_send", "cap_recv", "wave_mode", "dedup")]

    def __repr__(self):
        return "MoeDims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None

_VP = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
_DP = ctypes.POINTER(MoeDims)

_SIGS = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_capacity": (ctypes.c_int, [_DP, _I64, _I64, _I64, _I64, ctypes.POINTER(_I32),
                                    ctypes.POINTER(_I32)]),
    "moe_workspace_bytes": (_I64, [_DP, ctypes.c_int, _I64]),
    "moe_route": (ctypes.c_int, [_VP, _I32, _I32, _I32, _VP, _VP, _VP]),
    "moe_route_biased": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _VP, _VP]),
    "moe_expert_counts": (ctypes.c_int, [_VP, _I32, _I32, _I32, _VP, _VP]),
    "moe_balance_bias": (ctypes.c_int, [_VP, _I32, _I32, ctypes.c_double, _VP, _VP]),
    "moe_pack_waves": (ctypes.c_int, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                      _I64, _VP]),
    "moe_pack_waves_noalloc": (ctypes.c_int, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                              _VP, _VP]),
    "moe_bank": (ctypes.c_int, [_DP, _I32, _VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                _I64, _VP]),
    "moe_expert_ffn": (ctypes.c_int, [_DP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP, _VP, _I64,
                                      _VP, _I64, _VP]),
    "moe_combine": (ctypes.c_int, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                   _VP, _VP, _I64, _VP]),
    "moe_shared_swiglu": (ctypes.c_int, [_DP, _VP, _VP, _VP, _VP, _VP]),
    "moe_combine_shared": (ctypes.c_int, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          _VP, _I64, _VP]),
    "moe_route_backward": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP]),
    "moe_combine_backward": (ctypes.c_int, [_DP, _VP, _VP, _I64] + [_VP] * 17 + [_I64, _VP]),
    "moe_expert_ffn_backward": (ctypes.c_int, [_DP, _VP, _VP, _I64] + [_VP] * 6 +
                                [_I64] + [_VP] * 5 + [_I64, _VP]),
    "moe_pack_backward": (ctypes.c_int, [_DP] + [_VP] * 15 + [_I64, _VP]),
    "moe_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "moe_profile_collect": (ctypes.c_int, []),
    "moe_profile_get": (ctypes.c_int, [ctypes.c_int, ctypes.c_char_p, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I64)]),
    "moe_profile_reset": (None, []),
}

EXPORTS = tuple(_SIGS)


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc < 0:
        raise MoeError(rc, lib().moe_last_error().decode())
    return rc


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_capacity(d: MoeDims, cf_send, cf_recv):
    """(cap_send, cap_recv) from rational factors (fractions.Fraction or int)."""
    from fractions import Fraction
    fs, fr = Fraction(cf_send), Fraction(cf_recv)
    cs, cr = _I32(), _I32()
    _check(lib().moe_capacity(ctypes.byref(d), fs.numerator, fs.denominator, fr.numerator,
                              fr.denominator, ctypes.byref(cs), ctypes.byref(cr)))
    return cs.value, cr.value


def moe_workspace_bytes(d: MoeDims, call: int, n_rows: int = 0) -> int:
    return _check(lib().moe_workspace_bytes(ctypes.byref(d), call, n_rows))


def moe_route(logits, k, topk, gates, stream=None):
    T, E = logits.shape
    _check(lib().moe_route(_p(logits), T, E, k, _p(topk), _p(gates), _stream(stream)))


MOE_ROUTE_RENORM = 1
MOE_WAVES_TOKENS, MOE_WAVES_CHUNKS = 0, 1


def moe_route_biased(logits, bias, k, topk, gates, stream=None, flags=0):
    T, E = logits.shape
    _check(lib().moe_route_biased(_p(logits), _p(bias), T, E, k, flags, _p(topk), _p(gates),
                                  _stream(stream)))


def moe_expert_counts(topk, E, counts, stream=None):
    T, k = topk.shape
    _check(lib().moe_expert_counts(_p(topk), T, k, E, _p(counts), _stream(stream)))


def moe_balance_bias(window, alpha, bias, stream=None):
    n, E = window.shape
    _check(lib().moe_balance_bias(_p(window), n, E, float(alpha), _p(bias), _stream(stream)))


def moe_pack_waves(d, x, w_lat_down, topk, z, pools, pool_offsets, slot, fill, demand, ws,
                   stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_pack_waves(ctypes.byref(d), _p(x), _p(w_lat_down), _p(topk), _p(z),
                                _p(pools), _p(pool_offsets), _p(slot), _p(fill), _p(demand),
                                _p(ws), nbytes, _stream(stream)))


def moe_pack_waves_noalloc(d, x, w_lat_down, topk, z, pools, pool_offsets, slot, fill, demand,
                           stream=None):
    """moe_pack_waves with its scratch in the library's fixed device array."""
    _check(lib().moe_pack_waves_noalloc(ctypes.byref(d), _p(x), _p(w_lat_down), _p(topk),
                                        _p(z), _p(pools), _p(pool_offsets), _p(slot), _p(fill),
                                        _p(demand), _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 1 << 20


def moe_bank(d, rank, recv, recv_offsets, n_recv_rows, bank, bank_offsets, bank_src, bfill,
             bdemand, bad_rows, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_bank(ctypes.byref(d), rank, _p(recv), _p(recv_offsets), n_recv_rows,
                          _p(bank), _p(bank_offsets), _p(bank_src), _p(bfill), _p(bdemand),
                          _p(bad_rows), _p(ws), nbytes, _stream(stream)))


def moe_expert_ffn(d, bank, bank_offsets, bank_src, bfill, n_bank_rows, w_gate, w_up, w_down,
                   ret, n_ret_rows, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_expert_ffn(ctypes.byref(d), _p(bank), _p(bank_offsets), _p(bank_src),
                                _p(bfill), n_bank_rows, _p(w_gate), _p(w_up), _p(w_down),
                                _p(ret), n_ret_rows, _p(ws), nbytes, _stream(stream)))


def moe_combine(d, returned, ret_offsets, topk, slot, gates, x, w_lat_up, ws_gate, ws_up,
                ws_down, ylat, out, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_combine(ctypes.byref(d), _p(returned), _p(ret_offsets), _p(topk),
                             _p(slot), _p(gates), _p(x), _p(w_lat_up), _p(ws_gate), _p(ws_up),
                             _p(ws_down), _p(ylat), _p(out), _p(ws), nbytes, _stream(stream)))


def moe_shared_swiglu(d, x, ws_gate, ws_up, h_shared, stream=None):
    _check(lib().moe_shared_swiglu(ctypes.byref(d), _p(x), _p(ws_gate), _p(ws_up), _p(h_shared),
                                   _stream(stream)))


def moe_combine_shared(d, returned, ret_offsets, topk, slot, gates, w_lat_up, h_shared, ws_down,
                       ylat, out, ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_combine_shared(ctypes.byref(d), _p(returned), _p(ret_offsets), _p(topk),
                                    _p(slot), _p(gates), _p(w_lat_up), _p(h_shared),
                                    _p(ws_down), _p(ylat), _p(out), _p(ws), nbytes,
                                    _stream(stream)))


def moe_route_backward(logits, topk, d_gates, d_logits, bias=None, stream=None, flags=0):
    T, E = logits.shape
    k = topk.shape[1]
    _check(lib().moe_route_backward(_p(logits), _p(bias), T, E, k, flags, _p(topk), _p(d_gates),
                                    _p(d_logits), _stream(stream)))


def moe_combine_backward(d, returned, topk, slot, gates, fill, x, ylat, w_lat_up, ws_gate, ws_up,
                         ws_down, d_out, d_returned, d_gates, d_shared, dw_lat_up, dws_down, ws,
                         stream=None, ret_offsets=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_combine_backward(
        ctypes.byref(d), _p(returned), _p(ret_offsets), returned.shape[0], _p(topk), _p(slot),
        _p(gates), _p(fill), _p(x), _p(ylat),
        _p(w_lat_up), _p(ws_gate), _p(ws_up), _p(ws_down), _p(d_out), _p(d_returned),
        _p(d_gates), _p(d_shared), _p(dw_lat_up), _p(dws_down), _p(ws), nbytes,
        _stream(stream)))


def moe_expert_ffn_backward(d, bank, bank_src, bfill, w_gate, w_up, w_down, d_ret, d_recv,
                            dw_gate, dw_up, dw_down, ws, stream=None, bank_offsets=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_expert_ffn_backward(
        ctypes.byref(d), _p(bank), _p(bank_offsets), bank.shape[0], _p(bank_src), _p(bfill),
        _p(w_gate), _p(w_up), _p(w_down), _p(d_ret), d_ret.shape[0], _p(d_recv), _p(dw_gate),
        _p(dw_up), _p(dw_down), _p(ws), nbytes, _stream(stream)))


def moe_pack_backward(d, d_pools, topk, slot, x, d_shared, w_lat_down, ws_gate, ws_up, dz, dx,
                      dw_lat_down, dws_gate, dws_up, ws, stream=None, pool_offsets=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().moe_pack_backward(
        ctypes.byref(d), _p(d_pools), _p(pool_offsets), _p(topk), _p(slot), _p(x), _p(d_shared),
        _p(w_lat_down),
        _p(ws_gate), _p(ws_up), _p(dz), _p(dx), _p(dw_lat_down), _p(dws_gate), _p(dws_up),
        _p(ws), nbytes, _stream(stream)))


def moe_profile_enable(on: bool):
    _check(lib().moe_profile_enable(1 if on else 0))


def moe_profile_collect():
    _check(lib().moe_profile_collect())


def moe_profile_read():
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    out = {}
    i = 0
    buf = ctypes.create_string_buffer(128)
    while True:
        ms, n = ctypes.c_double(), _I64()
        if lib().moe_profile_get(i, buf, 128, ctypes.byref(ms), ctypes.byref(n)) != 0:
            break
        out[buf.value.decode()] = (ms.value, n.value)
        i += 1
    return out


def moe_profile_reset():
    lib().moe_profile_reset()
