"""Pins of oracle/dense.py, the whole-matrix form of the oracle's products.

dense.py does the products of oracle.c with float64 matrix products instead
of written-out loops.  It is pinned here against oracle.c (an independent
implementation of the same definitions, itself pinned in
test_oracle_pins.py), against closed forms, and its bf16 rounding against
torch and oracle.c bit for bit.  The float64 sums run in another order than
oracle.c's, so a product may differ from it by one bf16 unit where a sum
lands next to a rounding boundary; the tests allow that and require almost
every value to be equal.
"""
import math

import numpy as np
import pytest
import torch

from conftest import f64, u16, ulp_diff
from oracle import dense


def _bits(a):
    return u16(torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16))


def _rand_bits(rng, shape, scale=1.0):
    return _bits(rng.standard_normal(shape) * scale)


def _close_to_c(got, want, min_equal=0.995):
    """At most one bf16 unit apart everywhere, and equal almost everywhere."""
    ud = ulp_diff(got, want)
    assert ud.max() <= 1, f"{int((ud > 1).sum())} values more than one unit apart"
    assert (ud == 0).mean() >= min_equal, f"only {(ud == 0).mean():.4f} equal"


# ----------------------------------------------------------------------------
# bf16 rounding straight from the double
# ----------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-37, 37, 20000),
                           [0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38, 1e-39, -2e-41]])
    vals = vals.astype(np.float32)
    want = u16(torch.from_numpy(vals).to(torch.bfloat16))
    assert np.array_equal(dense.bf16_from_f64(vals.astype(np.float64)), want)


def test_bf16_rounding_ties_subnormals_overflow_match_c(orc):
    rng = np.random.default_rng(1)
    e = rng.integers(-140, 127, 3000).astype(np.float64)
    k = rng.integers(0, 128, 3000).astype(np.float64)
    ties = (128 + k + 0.5) * 2.0 ** (e - 7)            # exactly halfway between bf16 values
    near = ties * (1 + 2.0 ** -40)                     # just above a tie
    below = ties * (1 - 2.0 ** -40)
    wide = rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 39, 3000)
    special = np.array([0.0, -0.0, 1e39, -1e39, 3.3895313892515355e38, 3.39e38, 1e-45,
                        2.0 ** -133 * 0.5, 2.0 ** -133 * 1.5, 2.0 ** -126 * (1 - 2 ** -9)])
    vals = np.concatenate([ties, -ties, near, below, wide, special])
    want = np.array([orc.bf16_from_double(float(v)) for v in vals], np.uint16)
    assert np.array_equal(dense.bf16_from_f64(vals), want)
    # hand-checked cases: a tie to the even neighbour, and no double rounding
    assert dense.bf16_from_f64(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert dense.bf16_from_f64(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
    assert dense.bf16_from_f64(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81


# ----------------------------------------------------------------------------
# products against oracle.c
# ----------------------------------------------------------------------------

def test_latent_matches_c_oracle_and_identity(orc):
    rng = np.random.default_rng(2)
    T, D, L = 37, 320, 192
    x = _rand_bits(rng, (T, D))
    w = _rand_bits(rng, (L, D), D ** -0.5)
    _close_to_c(dense.latent(x, w), orc.latent(x, w))
    eye = np.zeros((L, D), np.float32)
    eye[np.arange(L), np.arange(L)] = 1.0              # W_ld = [I; 0]: z = x[:, :L]
    assert np.array_equal(dense.latent(x, _bits(eye)), x[:, :L])


def test_ffn_rows_match_c_oracle(orc):
    rng = np.random.default_rng(3)
    n, L, F = 41, 128, 256
    u = _rand_bits(rng, (n, L))
    wg = _rand_bits(rng, (F, L), L ** -0.5)
    wu = _rand_bits(rng, (F, L), L ** -0.5)
    wd = _rand_bits(rng, (L, F), F ** -0.5)
    want = np.stack([orc.ffn_row(u[i], wg, wu, wd) for i in range(n)])
    _close_to_c(dense.ffn_rows(u, wg, wu, wd), want)


def test_ffn_rows_closed_form():
    """u = e_0 makes a_f and b_f the chosen weights; W_d = I returns h."""
    L = F = 8
    u = _bits(np.eye(L)[:1])
    alpha = np.array([0, 1, 64, -64, 2, 1, 0.5, -1], np.float32)
    beta = np.array([5, 1, 2, 3, 0, -1, 4, 2], np.float32)
    wg = np.zeros((F, L), np.float32); wg[:, 0] = alpha
    wu = np.zeros((F, L), np.float32); wu[:, 0] = beta
    eye = np.eye(L, F, dtype=np.float32)
    y = dense.ffn_rows(u, _bits(wg), _bits(wu), _bits(eye))[0]
    sig = lambda a: 1.0 / (1.0 + math.exp(-a))
    want = [a * sig(a) * b for a, b in zip(alpha.astype(float), beta.astype(float))]
    assert np.array_equal(y, dense.bf16_from_f64(np.array(want)))
    assert f64(y)[2] == 128.0                           # silu(64) * 2, not silu(2) * 64


def _tiny_dims(orc, T=30, D=64, L=64, E=12, R=4, k=3, W=3, F=128, S=2, Fs=128, cap=(0, 0)):
    return orc.Dims(T, D, L, E, R, k, W, F, S, Fs, cap[0], cap[1], 0, 0)


@pytest.mark.parametrize("ragged", [False, True])
def test_expert_ffn_matches_c_oracle(orc, ragged):
    rng = np.random.default_rng(4 + ragged)
    d = _tiny_dims(orc, cap=(0, 0) if ragged else (5, 7))
    El = d.n_experts // d.n_ranks
    topk = np.stack([rng.choice(d.n_experts, d.top_k, replace=False)
                     for _ in range(d.T)]).astype(np.int32)
    snd = orc.sender(d, topk)
    pools = orc.pack_rows(d, _rand_bits(rng, (d.T, d.latent)), topk, snd["slot"],
                          snd["pool_offsets"])
    rank = 1
    # every source sends this shard's pools for `rank` (a valid receive buffer)
    if ragged:
        offs = snd["pool_offsets"]
        segs = [pools[offs[rank * d.n_waves + w]:offs[rank * d.n_waves + w + 1]]
                for w in range(d.n_waves)] * d.n_ranks
        recv = np.concatenate(segs)
        roffs = np.concatenate([[0], np.cumsum([len(x) for x in segs])]).astype(np.int64)
    else:
        C = d.cap_send
        recv = np.concatenate([pools.reshape(d.n_ranks, d.n_waves * C, -1)[rank]] * d.n_ranks)
        roffs = None
    bo = orc.bank_slots(d, rank, orc.headers(recv, d.latent), roffs)
    bank = orc.bank_rows(d, recv, bo.get("bank_offsets"), bo["bank_src"], bo["bfill"])
    wg = _rand_bits(rng, (El, d.d_ff, d.latent), d.latent ** -0.5)
    wu = _rand_bits(rng, (El, d.d_ff, d.latent), d.latent ** -0.5)
    wd = _rand_bits(rng, (El, d.latent, d.d_ff), d.d_ff ** -0.5)
    want = orc.expert_ffn(d, bank, bo.get("bank_offsets"), bo["bank_src"], bo["bfill"], wg, wu,
                          wd, len(recv))
    got = dense.expert_ffn(d, bank, bo.get("bank_offsets"), bo["bank_src"], bo["bfill"], wg, wu,
                           wd, len(recv))
    assert int(bo["bfill"].sum()) > 10 and int((bo["bdemand"] - bo["bfill"]).sum()) > 0 or ragged
    _close_to_c(got, want)


@pytest.mark.parametrize("ragged", [False, True])
def test_combine_matches_c_oracle(orc, ragged):
    rng = np.random.default_rng(6 + ragged)
    d = _tiny_dims(orc, T=40, cap=(0, 0) if ragged else (6, 8))
    topk = np.stack([rng.choice(d.n_experts, d.top_k, replace=False)
                     for _ in range(d.T)]).astype(np.int32)
    snd = orc.sender(d, topk)
    gates = rng.random((d.T, d.top_k)).astype(np.float32)
    n_ret = d.n_ranks * d.n_waves * d.cap_send if not ragged else int(snd["pool_offsets"][-1])
    # ragged: segments shorter than the sender's demand, so some slots fall past them
    roffs = None
    if ragged:
        lens = np.maximum(np.diff(snd["pool_offsets"]) - rng.integers(0, 2, d.n_ranks * d.n_waves),
                          0)
        roffs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        n_ret = int(roffs[-1])
    returned = _rand_bits(rng, (n_ret, d.latent))
    x = _rand_bits(rng, (d.T, d.d_model))
    wlu = _rand_bits(rng, (d.d_model, d.latent), d.latent ** -0.5)
    wsg = _rand_bits(rng, (d.n_shared, d.d_ff_shared, d.d_model), d.d_model ** -0.5)
    wsu = _rand_bits(rng, (d.n_shared, d.d_ff_shared, d.d_model), d.d_model ** -0.5)
    wsd = _rand_bits(rng, (d.n_shared, d.d_model, d.d_ff_shared), d.d_ff_shared ** -0.5)
    yo, oo = orc.combine(d, returned, roffs, topk, snd["slot"], gates, x, wlu, wsg, wsu, wsd)
    yg, og = dense.combine_tokens(d, returned, roffs, topk, snd["slot"], gates, x, wlu, wsg,
                                  wsu, wsd)
    _close_to_c(yg, yo)
    _close_to_c(og, oo)
    toks = np.array([39, 0, 17])
    yt, ot = dense.combine_tokens(d, returned, roffs, topk, snd["slot"], gates, x, wlu, wsg,
                                  wsu, wsd, tokens=toks)
    assert np.array_equal(yt, yg[toks]) and np.array_equal(ot, og[toks])


def test_combine_dropped_and_shared_only(orc):
    """Every choice dropped: ylat = 0 and out = the shared experts alone."""
    rng = np.random.default_rng(8)
    d = _tiny_dims(orc, T=9, cap=(4, 4))
    topk = np.stack([rng.choice(d.n_experts, d.top_k, replace=False)
                     for _ in range(d.T)]).astype(np.int32)
    slot = -np.ones((d.T, d.top_k), np.int32)
    returned = _rand_bits(rng, (d.n_ranks * d.n_waves * 4, d.latent))
    x = _rand_bits(rng, (d.T, d.d_model))
    wsg = _rand_bits(rng, (d.n_shared, d.d_ff_shared, d.d_model), 0.1)
    wsu = _rand_bits(rng, (d.n_shared, d.d_ff_shared, d.d_model), 0.1)
    sd = np.zeros((d.n_shared, d.d_model, d.d_ff_shared), np.float32)
    sd[0, np.arange(d.d_ff_shared // 2), np.arange(d.d_ff_shared // 2)] = 1.0
    ylat, out = dense.combine_tokens(d, returned, None, topk, slot,
                                     np.ones((d.T, d.top_k), np.float32), x,
                                     _rand_bits(rng, (d.d_model, d.latent)), wsg, wsu, _bits(sd))
    assert (ylat == 0).all()
    h = dense.shared_h(x, wsg, wsu)
    half = d.d_ff_shared // 2
    assert np.array_equal(out[:, :half], h[:, :half]) and (out[:, half:] == 0).all()


# ----------------------------------------------------------------------------
# backward: whole rows of the weight gradients against oracle.c's full backward
# ----------------------------------------------------------------------------

def _bwd_case(orc, seed):
    rng = np.random.default_rng(seed)
    d = _tiny_dims(orc, T=36, cap=(6, 9))
    El = d.n_experts // d.n_ranks
    topk = np.stack([rng.choice(d.n_experts, d.top_k, replace=False)
                     for _ in range(d.T)]).astype(np.int32)
    snd = orc.sender(d, topk)
    gates = rng.random((d.T, d.top_k)).astype(np.float32)
    n_rows = d.n_ranks * d.n_waves * d.cap_send
    w = dict(
        x=_rand_bits(rng, (d.T, d.d_model)), ylat=_rand_bits(rng, (d.T, d.latent)),
        returned=_rand_bits(rng, (n_rows, d.latent)), d_out=_rand_bits(rng, (d.T, d.d_model)),
        wlu=_rand_bits(rng, (d.d_model, d.latent), d.latent ** -0.5),
        wld=_rand_bits(rng, (d.latent, d.d_model), d.d_model ** -0.5),
        wsg=_rand_bits(rng, (d.n_shared, d.d_ff_shared, d.d_model), d.d_model ** -0.5),
        wsu=_rand_bits(rng, (d.n_shared, d.d_ff_shared, d.d_model), d.d_model ** -0.5),
        wsd=_rand_bits(rng, (d.n_shared, d.d_model, d.d_ff_shared), d.d_ff_shared ** -0.5),
        wg=_rand_bits(rng, (El, d.d_ff, d.latent), d.latent ** -0.5),
        wu=_rand_bits(rng, (El, d.d_ff, d.latent), d.latent ** -0.5),
        wd=_rand_bits(rng, (El, d.latent, d.d_ff), d.d_ff ** -0.5),
        d_pools=_rand_bits(rng, (n_rows, d.latent)),
        d_shared=_rand_bits(rng, (d.T, 2, d.n_shared, d.d_ff_shared)),
        d_ret=_rand_bits(rng, (n_rows, d.latent)))
    return rng, d, topk, snd, gates, w


def test_combine_wgrad_rows_match_c_oracle(orc):
    rng, d, topk, snd, gates, w = _bwd_case(orc, 20)
    _, _, _, dwlu, dwsd = orc.combine_backward(d, w["returned"], topk, snd["slot"], gates, w["x"],
                                               w["ylat"], w["wlu"], w["wsg"], w["wsu"], w["wsd"],
                                               w["d_out"])
    rows = np.array([0, 5, d.d_model - 1])
    _close_to_c(dense.outer_rows(f64(w["d_out"][:, rows]), f64(w["ylat"])), dwlu[rows])
    for sh in range(d.n_shared):
        f = np.array([0, 3, d.d_ff_shared - 1])
        got = dense.shared_down_wgrad_cols(w["x"], w["wsg"], w["wsu"], w["d_out"], sh, f)
        _close_to_c(got, dwsd[sh][:, f].T)


def test_expert_wgrad_rows_match_c_oracle(orc):
    rng, d, topk, snd, gates, w = _bwd_case(orc, 21)
    El = d.n_experts // d.n_ranks
    n_rows = d.n_ranks * d.n_waves * d.cap_send
    hdr = np.where(rng.random(n_rows) < 0.8, 1 * El + rng.integers(0, El, n_rows), -1)
    bo = orc.bank_slots(d, 1, hdr.astype(np.int32), None)
    bank = _rand_bits(rng, (len(bo["bank_src"]), d.latent))
    _, dwg, dwu, dwd = orc.expert_ffn_backward(d, bank, bo["bank_src"], bo["bfill"], w["wg"],
                                               w["wu"], w["wd"], w["d_ret"])
    f = np.array([0, 7, d.d_ff - 1])
    for j in range(El):
        pos = np.concatenate([np.arange(g * d.cap_recv, g * d.cap_recv + bo["bfill"][g])
                              for g in range(j, d.n_waves * El, El)])
        u, dy = bank[pos], w["d_ret"][bo["bank_src"][pos]]
        g, up, dn = dense.expert_wgrad_rows(u, dy, w["wg"][j], w["wu"][j], w["wd"][j], f)
        _close_to_c(g, dwg[j][f])
        _close_to_c(up, dwu[j][f])
        _close_to_c(dn, dwd[j][:, f].T)


def test_pack_wgrad_rows_match_c_oracle(orc):
    rng, d, topk, snd, gates, w = _bwd_case(orc, 22)
    dz, _, dwld, dwsg, dwsu = orc.pack_backward(d, w["d_pools"], topk, snd["slot"], w["x"],
                                                w["d_shared"], w["wld"], w["wsg"], w["wsu"])
    assert np.array_equal(dense.pack_dz(d, w["d_pools"], topk, snd["slot"]), dz)
    rows = np.array([0, 9, d.latent - 1])
    _close_to_c(dense.outer_rows(f64(dz[:, rows]), f64(w["x"])), dwld[rows])
    for sh in range(d.n_shared):
        f = np.array([1, d.d_ff_shared - 1])
        _close_to_c(dense.outer_rows(f64(w["d_shared"][:, 0, sh, f]), f64(w["x"])), dwsg[sh][f])
        _close_to_c(dense.outer_rows(f64(w["d_shared"][:, 1, sh, f]), f64(w["x"])), dwsu[sh][f])


def test_expert_wgrad_rows_over_chunks_match_c_oracle(orc):
    """More bank rows than one float64 chunk of dense.py: the sums over
    chunks still give oracle.c's entries."""
    rng = np.random.default_rng(23)
    n, L, F = 4500, 64, 128
    d = orc.Dims(8, 64, L, 4, 4, 1, 1, F, 0, 128, 4500, n, 0, 0)   # one expert per rank, one wave
    bank = _rand_bits(rng, (n, L))
    d_ret = _rand_bits(rng, (n, L))
    wg = _rand_bits(rng, (1, F, L), L ** -0.5)
    wu = _rand_bits(rng, (1, F, L), L ** -0.5)
    wd = _rand_bits(rng, (1, L, F), F ** -0.5)
    src, fill = np.arange(n, dtype=np.int32), np.array([n], np.int32)
    f = np.array([0, 77, F - 1])
    g, u, dn = dense.expert_wgrad_rows(bank, d_ret, wg[0], wu[0], wd[0], f)
    cols = np.arange(L)
    for which, got in ((0, g), (1, u)):
        ref = np.stack([orc.expert_wgrad_entries(d, bank, src, fill, wg, wu, wd, d_ret, 0, which,
                                                 np.full(L, fi), cols) for fi in f])
        _close_to_c(got, ref, min_equal=0.98)
    ref = np.stack([orc.expert_wgrad_entries(d, bank, src, fill, wg, wu, wd, d_ret, 0, 2, cols,
                                             np.full(L, fi)) for fi in f])
    _close_to_c(dn, ref, min_equal=0.98)
