"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/moe.h declares, and rejects bad arguments on the host
(returning a negative status and an error text) before any launch."""
import ctypes
import os
import re
from fractions import Fraction

import pytest

from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def moe():
    import dispatch_softmax_top_amd as m
    m.lib()
    return m


def test_exports_every_declared_symbol(moe):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(moe.lib(), n), n
    assert set(names) == set(moe.EXPORTS)


def test_abi_version(moe):
    assert moe.moe_abi_version() == 7


def test_capacity_matches_table(moe):
    from dispatch_softmax_top_amd import share
    for cfg, cs, cr in ((configs.TINY, 25, 34), (configs.SHARE_4K, 188, 2095),
                        (configs.ZIPF_16K, 752, 8376), (configs.LONG_65K, 3004, 33498),
                        (configs.SWEEP_16K["1.5/1.5"], 1025, 10924),
                        (configs.SWEEP_16K["2.0/2.0"], 1366, 14566)):
        d = share.make_dims(cfg)
        assert (d.cap_send, d.cap_recv) == (cs, cr), cfg.name


def test_capacity_agrees_with_oracle(moe, orc):
    from dispatch_softmax_top_amd import share
    import itertools
    for T, cs, cr in itertools.product((1, 7, 64, 601, 4096, 65536), ("11/10", "3/2", "7/3"),
                                       ("23/20", "1", "5/2")):
        cfg = configs.scaled(configs.SHARE_4K, "x", T=T, cf_send=Fraction(cs),
                             cf_recv=Fraction(cr))
        d, dd = share.make_dims(cfg), orc.dims(cfg)
        assert (d.cap_send, d.cap_recv) == (dd.cap_send, dd.cap_recv)


def _dims(moe, **kw):
    from dispatch_softmax_top_amd import share
    d = share.make_dims(configs.TINY)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value", [("latent", 100), ("d_model", 0), ("n_ranks", 5),
                                         ("top_k", 60), ("d_ff", 200), ("cap_recv", 0),
                                         ("n_experts", 2048), ("wave_mode", 2),
                                         ("dedup", 3)])
def test_bad_dims_rejected(moe, field, value):
    d = _dims(moe, **{field: value})
    rc = moe.lib().moe_workspace_bytes(ctypes.byref(d), moe.MOE_CALL_FFN, 0)
    assert rc < 0
    assert moe.lib().moe_last_error().decode()


@pytest.mark.parametrize("value,ok", [("64", True), ("200", True), ("8", True), ("", True),
                                      ("12", False), ("0", False), ("-8", False), ("64x", False)])
def test_planned_cus_variable_checked_before_any_launch(moe, monkeypatch, value, ok):
    monkeypatch.setenv("MOE_GEMM_CUS", value)
    d = _dims(moe)
    rc = moe.lib().moe_workspace_bytes(ctypes.byref(d), moe.MOE_CALL_FFN, 0)
    assert (rc >= 0) == ok
    if not ok:
        assert "MOE_GEMM_CUS" in moe.lib().moe_last_error().decode()


def test_chunked_waves_need_fixed_capacities(moe):
    d = _dims(moe, wave_mode=moe.MOE_WAVES_CHUNKS)
    assert moe.moe_workspace_bytes(d, moe.MOE_CALL_PACK, 0) >= 0
    d = _dims(moe, wave_mode=moe.MOE_WAVES_CHUNKS, cap_send=0, cap_recv=0)
    assert moe.lib().moe_workspace_bytes(ctypes.byref(d), moe.MOE_CALL_PACK, 0) < 0
    assert "chunk" in moe.lib().moe_last_error().decode()


def test_dedup_needs_fixed_capacities(moe):
    d = _dims(moe, dedup=1)
    assert moe.moe_workspace_bytes(d, moe.MOE_CALL_BANK, 0) >= 0
    d = _dims(moe, dedup=1, cap_send=0, cap_recv=0)
    assert moe.lib().moe_workspace_bytes(ctypes.byref(d), moe.MOE_CALL_PACK, 0) < 0
    d = _dims(moe, dedup=1)                        # the backward calls do not take it
    assert moe.lib().moe_workspace_bytes(ctypes.byref(d), moe.MOE_CALL_FFN_BWD, 0) == -2


def test_calls_reject_null_and_misaligned(moe):
    L = moe.lib()
    d = _dims(moe)
    assert L.moe_route(None, 4, 16, 8, None, None, None) == -1
    assert L.moe_route(ctypes.c_void_p(16), 4, 16, 17, ctypes.c_void_p(16), ctypes.c_void_p(16),
                       None) == -1
    assert L.moe_route(ctypes.c_void_p(18), 4, 16, 8, ctypes.c_void_p(16), ctypes.c_void_p(16),
                       None) == -1                                  # misaligned
    assert "aligned" in L.moe_last_error().decode()
    p = ctypes.c_void_p(256)
    assert L.moe_pack_waves(ctypes.byref(d), p, p, p, p, p, None, p, p, p, None, 0, None) < 0
    assert L.moe_bank(ctypes.byref(d), 99, p, None, 0, p, None, p, p, p, p, None, 0, None) == -1
    assert L.moe_bank(ctypes.byref(d), 0, p, None, 5, p, None, p, p, p, p, None, 0, None) == -1
    assert L.moe_expert_ffn(ctypes.byref(d), p, None, p, p, 1, p, p, p, p, 1, p, 1 << 30,
                            None) == -1
    assert L.moe_combine(ctypes.byref(d), p, None, p, p, p, p, p, p, p, p, p, p, None, 0,
                         None) == -4                                # workspace too small
    assert L.moe_shared_swiglu(ctypes.byref(d), None, p, p, p, None) == -1
    assert L.moe_shared_swiglu(ctypes.byref(d), p, p, p, None, None) == -1   # h_shared
    assert L.moe_combine_shared(ctypes.byref(d), p, None, p, p, p, p, None, p, p, p,
                                None, 0, None) == -1               # h_shared
    assert L.moe_combine_shared(ctypes.byref(d), p, None, p, p, p, p, p, p, None, p,
                                None, 0, None) == -1               # ylat
    assert L.moe_combine_shared(ctypes.byref(d), p, None, p, p, p, p, p, p, p, p,
                                p, 16, None) == -4                 # workspace too small


def test_workspace_sizes_grow_with_rows(moe):
    d = _dims(moe, cap_send=0, cap_recv=0)
    a = moe.moe_workspace_bytes(d, moe.MOE_CALL_FFN, 100)
    b = moe.moe_workspace_bytes(d, moe.MOE_CALL_FFN, 1000)
    assert 0 < a < b


def test_balancing_calls_reject_bad_arguments(moe):
    L = moe.lib()
    p = ctypes.c_void_p(256)
    assert L.moe_route_biased(p, ctypes.c_void_p(18), 4, 16, 8, 0, p, p, None) == -1  # misaligned
    assert L.moe_route_biased(p, p, 4, 16, 17, 0, p, p, None) == -1                # k > E
    assert L.moe_route_biased(p, p, 4, 16, 8, 6, p, p, None) == -1                 # unknown flag
    assert L.moe_expert_counts(p, 4, 8, 2000, p, None) == -2                       # E > 1024
    assert L.moe_expert_counts(p, 0, 8, 16, p, None) == -1
    assert L.moe_expert_counts(None, 4, 8, 16, p, None) == -1
    assert L.moe_balance_bias(p, 0, 16, 1.0, p, None) == -1                        # empty window
    assert L.moe_balance_bias(p, 2, 16, float("nan"), p, None) == -1
    assert L.moe_balance_bias(p, 2, 16, 1.0, None, None) == -1
    assert "bias" in L.moe_last_error().decode()


def test_backward_calls_check_arguments(moe):
    L = moe.lib()
    d = _dims(moe)
    for call in (moe.MOE_CALL_COMBINE_BWD, moe.MOE_CALL_FFN_BWD, moe.MOE_CALL_PACK_BWD):
        assert moe.moe_workspace_bytes(d, call, 0) > 0
    rg = _dims(moe, cap_send=0, cap_recv=0)
    # ragged: the expert call's workspace grows with its bank rows
    small = L.moe_workspace_bytes(ctypes.byref(rg), moe.MOE_CALL_FFN_BWD, 100)
    assert 0 < small < L.moe_workspace_bytes(ctypes.byref(rg), moe.MOE_CALL_FFN_BWD, 10000)
    dd = _dims(moe, dedup=1)
    assert L.moe_workspace_bytes(ctypes.byref(dd), moe.MOE_CALL_FFN_BWD, 0) == -2
    p = ctypes.c_void_p(256)
    big = 1 << 40
    n_ret = d.n_ranks * d.n_waves * d.cap_send
    n_bank = d.n_waves * (d.n_experts // d.n_ranks) * d.cap_recv
    # ragged without offsets; fixed with the wrong row count; fixed, small workspace
    assert L.moe_combine_backward(ctypes.byref(rg), p, None, 100, *([p] * 17), big, None) == -1
    assert L.moe_combine_backward(ctypes.byref(d), p, None, n_ret + 1, *([p] * 17), big,
                                  None) == -1
    assert L.moe_combine_backward(ctypes.byref(d), p, None, n_ret, *([p] * 17), 16, None) == -4
    assert "workspace" in L.moe_last_error().decode()
    assert L.moe_expert_ffn_backward(ctypes.byref(d), p, None, n_bank, *([p] * 5), None, n_ret,
                                     *([p] * 5), big, None) == -1                    # d_ret
    assert L.moe_expert_ffn_backward(ctypes.byref(rg), p, None, 100, *([p] * 6), 100,
                                     *([p] * 5), big, None) == -1                    # offsets
    assert L.moe_expert_ffn_backward(ctypes.byref(rg), p, p, 100, *([p] * 6), 99,
                                     *([p] * 5), big, None) == -1                    # rows
    assert L.moe_pack_backward(ctypes.byref(d), *([p] * 14), None, big, None) == -1  # ws NULL
    assert L.moe_route_backward(p, None, 4, 16, 17, 0, p, p, p, None) == -1          # k > E
    assert L.moe_route_backward(p, None, 4, 16, 8, 2, p, p, p, None) == -1           # flags
