"""GPU parity of the backward calls, on inputs shared with the oracle.

Each call gets exactly the inputs the oracle gets (generator tensors, oracle
routing, sender and bank decisions, stand-in payload and gradient rows), so
errors do not compound between stages.  bf16 outputs: per row within
2e-2 * max|ref| of the row (weight gradients per weight row); fp32 gate and
logit gradients: within 1e-4 of the row's scale; rows that must be zero are
exactly zero.
"""
import numpy as np
import pytest
import torch

import gpucase as gc
from conftest import f64, u16
from synth import configs, gen

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": configs.TINY,
    "mid": gc.MID,
    "mid_tight": gc.with_cf(gc.MID, "1/2", "3/5"),
    "mid_chunks": gc.chunked(gc.MID),
    "mid_ragged": gc.ragged(gc.MID),
    # degenerate shapes: top-1 routing, one wave, no shared experts
    "tiny_k1_w1_s0": configs.scaled(configs.TINY, configs.TINY.name + "_k1_W1_S0", top_k=1,
                                    n_waves=1, n_shared=0),
}


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dispatch_softmax_top_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def share():
    from dispatch_softmax_top_amd import share
    return share


def _ws(moe, d, call, n_rows=0):
    n = moe.moe_workspace_bytes(d, call, n_rows)
    return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")


def _seg_offsets(s0, rng, shorten):
    """Segments of a pools-layout buffer in ragged mode: the sender's pool
    offsets, with some segments a row shorter when `shorten` (slots past a
    segment's end have no row: the single-GPU identity return)."""
    lens = np.diff(s0["pool_offsets"])
    if shorten:
        lens = np.maximum(lens - rng.integers(0, 2, len(lens)), 0)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _rows(got, ref, what):
    """bf16 [.., n] tensors compared per last-axis row."""
    n = ref.shape[-1]
    gc.assert_rows_close(np.ascontiguousarray(got).reshape(-1, n),
                         np.ascontiguousarray(ref).reshape(-1, n), what)


def _grad_rows(rng_idx, shape):
    return u16(gen.payload_rows(int(np.prod(shape[:-1])), shape[-1], rng_idx)).reshape(shape)


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("biased", [False, True])
def test_route_backward(moe, orc, renorm, biased):
    rng = np.random.default_rng(60 + renorm + 2 * biased)
    for T, E, k in ((257, 384, 8), (64, 48, 8), (33, 1024, 32), (5, 8, 8)):
        lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
        bias = rng.standard_normal(E).astype(np.float32) if biased else None
        topk, _ = orc.route_ex(lg, k, bias=bias, renorm=renorm)
        dg = rng.standard_normal((T, k)).astype(np.float32)
        ref = orc.route_backward(lg, topk, dg, bias=bias, renorm=renorm)
        out = torch.full((T, E), 7.0, device="cuda")
        moe.moe_route_backward(gc.dev(lg), gc.dev(topk), gc.dev(dg), out,
                               bias=None if bias is None else gc.dev(bias),
                               flags=moe.MOE_ROUTE_RENORM if renorm else 0)
        torch.cuda.synchronize()
        got = gc.host(out)
        scale = np.abs(ref).max(1, keepdims=True) + 1e-30
        assert (np.abs(got - ref) <= 1e-4 * scale).all(), (T, E, k)
        if renorm:
            mask = np.zeros((T, E), bool)
            np.put_along_axis(mask, topk, True, 1)
            assert (got[~mask] == 0).all()


# ----------------------------------------------------------------------------
# combine side
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
def test_combine_backward(moe, orc, share, name):
    cfg = CASES[name]
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    T, L, D, S, Fs = cfg.T, cfg.latent, cfg.d_model, cfg.n_shared, cfg.d_ff_shared
    s0 = gc.oracle_sender_all(orc, cfg, d_orc, n_shards=1)[0]
    roffs = None if d.cap_send else _seg_offsets(s0, np.random.default_rng(30), True)
    n_rows = cfg.n_ranks * cfg.n_waves * d.cap_send if d.cap_send else int(roffs[-1])
    returned = u16(gen.payload_rows(n_rows, L, 31))
    ylat = u16(gen.payload_rows(T, L, 32))
    d_out = u16(gen.payload_rows(T, D, 33))
    x = u16(s0["x"])
    wlu = u16(gen.latent_up(cfg))
    wsg, wsu, wsd = (u16(w) for w in gen.shared(cfg))
    ref = orc.combine_backward(d_orc, returned, s0["topk"], s0["slot"], s0["gates"], x, ylat,
                               wlu, wsg, wsu, wsd, d_out, ret_offsets=roffs)
    o_dret, o_dg, o_dsh, o_dwlu, o_dwsd = ref

    dev = lambda a: gc.dev(np.ascontiguousarray(a))
    d_ret = torch.full((n_rows, L), 3.0, dtype=torch.bfloat16, device="cuda")  # poison
    d_g = torch.full((T, cfg.top_k), 5.0, device="cuda")
    d_sh = torch.empty((T, 2, S, Fs), dtype=torch.bfloat16, device="cuda")
    dwlu = torch.empty((D, L), dtype=torch.bfloat16, device="cuda")
    dwsd = torch.empty((S, D, Fs), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_backward(d, dev(returned), dev(s0["topk"]), dev(s0["slot"]), dev(s0["gates"]),
                             dev(s0["fill"]), dev(x), dev(ylat), dev(wlu), dev(wsg), dev(wsu),
                             dev(wsd), dev(d_out), d_ret, d_g, d_sh, dwlu, dwsd,
                             _ws(moe, d, moe.MOE_CALL_COMBINE_BWD),
                             ret_offsets=None if roffs is None else dev(roffs))
    torch.cuda.synchronize()
    g_dret = gc.host(d_ret)
    zero = ~np.abs(f64(o_dret)).any(1)
    assert (g_dret[zero] == 0).all()
    _rows(g_dret[~zero], o_dret[~zero], "d_returned")
    gd = gc.host(d_g)
    assert (gd[s0["slot"] < 0] == 0).all()
    assert (gd[o_dg == 0] == 0).all()             # ragged: slots past their segment too
    # each gate gradient is a dot product of a returned row with d_ylat[t]:
    # allow 2e-3 of max|returned| * sum|d_ylat[t]| (fp32 against fp64
    # accumulation, and one-unit differences in the bf16 d_ylat)
    y = f64(d_out) @ f64(wlu)
    tol = 2e-3 * np.abs(f64(returned)).max() * np.abs(y).sum(1, keepdims=True)
    assert (np.abs(gd - o_dg) <= tol).all()
    _rows(gc.host(d_sh), o_dsh, "d_shared")
    _rows(gc.host(dwlu), o_dwlu, "dw_lat_up")
    _rows(gc.host(dwsd), o_dwsd, "dws_down")


# ----------------------------------------------------------------------------
# receiver side
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
def test_expert_ffn_backward(moe, orc, share, name):
    cfg = CASES[name]
    rank = 1
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    L, F, El = cfg.latent, cfg.d_ff, cfg.experts_per_rank
    senders = gc.oracle_sender_all(orc, cfg, d_orc)
    hdr, offs = gc.recv_headers(cfg, d_orc, senders, rank)
    n = len(hdr)
    bo = orc.bank_slots(d_orc, rank, hdr, offs)
    nb = len(bo["bank_src"])
    bank = u16(gen.payload_rows(nb, L, 41))
    d_ret = u16(gen.payload_rows(n, L, 42))
    wg, wu, wd = (u16(w) for w in gen.rank_experts(cfg, rank))
    o_drecv, o_dwg, o_dwu, o_dwd = orc.expert_ffn_backward(d_orc, bank, bo["bank_src"],
                                                           bo["bfill"], wg, wu, wd, d_ret,
                                                           bank_offsets=bo["bank_offsets"])
    dev = lambda a: gc.dev(np.ascontiguousarray(a))
    d_recv = torch.full((n, L), 2.0, dtype=torch.bfloat16, device="cuda")
    dwg = torch.empty((El, F, L), dtype=torch.bfloat16, device="cuda")
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((El, L, F), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn_backward(d, dev(bank), dev(bo["bank_src"]), dev(bo["bfill"]), dev(wg),
                                dev(wu), dev(wd), dev(d_ret), d_recv, dwg, dwu, dwd,
                                _ws(moe, d, moe.MOE_CALL_FFN_BWD, 0 if d.cap_send else nb),
                                bank_offsets=None if d.cap_send else dev(bo["bank_offsets"]))
    torch.cuda.synchronize()
    kept = np.zeros(n, bool)
    kept[bo["bank_src"][bo["bank_src"] >= 0]] = True
    g = gc.host(d_recv)
    assert (g[~kept] == 0).all()
    _rows(g[kept], o_drecv[kept], "d_recv")
    for got, want, what in ((dwg, o_dwg, "dw_gate"), (dwu, o_dwu, "dw_up"), (dwd, o_dwd, "dw_down")):
        gg = gc.host(got)
        for j in range(El):
            if not np.abs(f64(want[j])).any():           # an expert with no kept rows
                assert (gg[j] == 0).all(), what
            else:
                _rows(gg[j], want[j], f"{what} expert {j}")


# ----------------------------------------------------------------------------
# sender side
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
def test_pack_backward(moe, orc, share, name):
    cfg = CASES[name]
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    T, L, D, S, Fs = cfg.T, cfg.latent, cfg.d_model, cfg.n_shared, cfg.d_ff_shared
    s0 = gc.oracle_sender_all(orc, cfg, d_orc, n_shards=1)[0]
    poffs = None if d.cap_send else _seg_offsets(s0, np.random.default_rng(50), True)
    n_rows = cfg.n_ranks * cfg.n_waves * d.cap_send if d.cap_send else int(poffs[-1])
    d_pools = u16(gen.payload_rows(n_rows, L, 51))
    d_shared = _grad_rows(52, (T, 2, S, Fs))
    x = u16(s0["x"])
    wld = u16(gen.latent_down(cfg))
    wsg, wsu, _ = (u16(w) for w in gen.shared(cfg))
    o_dz, o_dx, o_dwld, o_dwsg, o_dwsu = orc.pack_backward(d_orc, d_pools, s0["topk"], s0["slot"],
                                                           x, d_shared, wld, wsg, wsu,
                                                           pool_offsets=poffs)
    dev = lambda a: gc.dev(np.ascontiguousarray(a))
    dz = torch.empty((T, L), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    dwld = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
    dwsg = torch.empty((S, Fs, D), dtype=torch.bfloat16, device="cuda")
    dwsu = torch.empty_like(dwsg)
    moe.moe_pack_backward(d, dev(d_pools), dev(s0["topk"]), dev(s0["slot"]), dev(x),
                          dev(d_shared), dev(wld), dev(wsg), dev(wsu), dz, dx, dwld, dwsg, dwsu,
                          _ws(moe, d, moe.MOE_CALL_PACK_BWD),
                          pool_offsets=None if poffs is None else dev(poffs))
    torch.cuda.synchronize()
    gz = gc.host(dz)
    none = ~np.abs(f64(o_dz)).any(1)        # every choice dropped (or past its segment)
    assert (gz[none] == 0).all()
    _rows(gz[~none], o_dz[~none], "dz")
    _rows(gc.host(dx), o_dx, "dx")
    _rows(gc.host(dwld), o_dwld, "dw_lat_down")
    _rows(gc.host(dwsg), o_dwsg, "dws_gate")
    _rows(gc.host(dwsu), o_dwsu, "dws_up")


def test_backward_rejects_dedup_and_small_workspace(moe, share):
    d = share.make_dims(gc.deduped(configs.TINY))
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_bytes(d, moe.MOE_CALL_FFN_BWD, 0)
    d = share.make_dims(configs.TINY)
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_pack_backward(d, t, t, t, t, t, t, t, t, t, t, t, t, t,
                              torch.empty(16, dtype=torch.uint8, device="cuda"))


# ----------------------------------------------------------------------------
# whole backward chain on each side, after each side's own forward chain
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "mid_chunks", "tiny_k1_w1_s0", "mid_ragged"])
def test_backward_chain(moe, orc, share, name):
    """Forward then backward for rank 0 on each side: GPU calls only on the
    GPU, oracle calls only in the oracle, both exchanges as loopback
    identities (ragged: the receive layout and its offsets serve as the
    returned rows and the pool-row gradients).  Upstream differences of a
    bf16 unit propagate, so rows are compared with the same per-row
    tolerance."""
    cfg = CASES[name]
    rank = 0
    rg = cfg.cf_send is None
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    wld, wlu = gen.latent_down(cfg), gen.latent_up(cfg)
    wg, wu, wd = gen.rank_experts(cfg, rank)
    wsg, wsu, wsd = gen.shared(cfg)
    cu = lambda t: t.cuda()
    # GPU forward
    pools, poffs = [], []
    for s in range(cfg.n_shards):
        x, lg = gc.shard_inputs(cfg, s)
        snd = share.Sender(d)
        snd.route(lg.cuda())
        snd.pack(x.cuda(), cu(wld))
        pools.append(snd.pools)
        poffs.append(snd.pool_offsets)
        if s == rank:
            own, x_own, lg_own = snd, x, lg
    if rg:
        recv, roffs = share.loopback_recv_ragged(d, pools, poffs, rank)
    else:
        recv, roffs = share.loopback_recv_fixed(d, pools, rank), None
    rcv = share.Receiver(d, recv.shape[0])
    rcv.bank_rows(rank, recv, roffs)
    rcv.ffn(cu(wg), cu(wu), cu(wd))
    cmb = share.Combiner(d)
    cmb.combine(rcv.ret, roffs, own, cu(x_own), cu(wlu), cu(wsg), cu(wsu), cu(wsd))
    # GPU backward
    d_out = gen.payload_rows(cfg.T, cfg.d_model, 61)
    b = share.Backward(d, recv.shape[0])
    b.combine(rcv.ret, own, cmb, cu(x_own), cu(wlu), cu(wsg), cu(wsu), cu(wsd), cu(d_out),
              ret_offsets=roffs)
    b.route(lg_own.cuda(), own)
    b.ffn(rcv, cu(wg), cu(wu), cu(wd), b.d_returned)
    b.pack(b.d_recv, own, cu(x_own), cu(wld), cu(wsg), cu(wsu), pool_offsets=roffs)
    torch.cuda.synchronize()

    # oracle forward
    W, Cs = cfg.n_waves, d.cap_send
    o_pools, o_sh, s0 = [], [], None
    for s in range(cfg.n_shards):
        x, lg = gc.shard_inputs(cfg, s)
        topk, gates = orc.route(lg.numpy(), cfg.top_k)
        z = orc.latent(u16(x), u16(wld))
        sn = orc.sender(d_orc, topk)
        o_pools.append(orc.pack_rows(d_orc, z, topk, sn["slot"], sn["pool_offsets"]))
        o_sh.append(sn)
        if s == rank:
            s0 = dict(topk=topk, gates=gates, **sn)
    segs, lens = [], []
    for s in range(cfg.n_shards):
        for w in range(W):
            if rg:
                o = o_sh[s]["pool_offsets"]
                a, e = int(o[rank * W + w]), int(o[rank * W + w + 1])
            else:
                a, e = (rank * W + w) * Cs, (rank * W + w + 1) * Cs
            segs.append(o_pools[s][a:e])
            lens.append(e - a)
    o_recv = np.concatenate(segs)
    o_roffs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64) if rg else None
    bo = orc.bank_slots(d_orc, rank, orc.headers(o_recv, d.latent), o_roffs)
    o_bank = orc.bank_rows(d_orc, o_recv, bo["bank_offsets"], bo["bank_src"], bo["bfill"])
    ex = [u16(w) for w in (wg, wu, wd)]
    o_ret = orc.expert_ffn(d_orc, o_bank, bo["bank_offsets"], bo["bank_src"], bo["bfill"], *ex,
                           len(o_recv))
    sh = [u16(w) for w in (wsg, wsu, wsd)]
    o_ylat, _ = orc.combine(d_orc, o_ret, o_roffs, s0["topk"], s0["slot"], s0["gates"],
                            u16(x_own), u16(wlu), *sh)
    # oracle backward
    o_dret, o_dg, o_dsh, o_dwlu, o_dwsd = orc.combine_backward(
        d_orc, o_ret, s0["topk"], s0["slot"], s0["gates"], u16(x_own), o_ylat, u16(wlu), *sh,
        u16(d_out), ret_offsets=o_roffs)
    o_dl = orc.route_backward(lg_own.numpy(), s0["topk"], o_dg)
    o_drecv, o_dwg, o_dwu, o_dwd = orc.expert_ffn_backward(d_orc, o_bank, bo["bank_src"],
                                                           bo["bfill"], *ex, o_dret,
                                                           bank_offsets=bo["bank_offsets"])
    o_dz, o_dx, o_dwld, o_dwsg, o_dwsu = orc.pack_backward(d_orc, o_drecv, s0["topk"], s0["slot"],
                                                           u16(x_own), o_dsh, u16(wld), sh[0], sh[1],
                                                           pool_offsets=o_roffs)

    assert np.array_equal(gc.host(own.slot), s0["slot"])
    assert np.array_equal(gc.host(rcv.bank_src), bo["bank_src"])
    for got, want, what in ((b.d_returned, o_dret, "d_returned"), (b.d_recv, o_drecv, "d_recv"),
                            (b.dz, o_dz, "dz")):
        g = gc.host(got)
        nz = np.abs(f64(want)).any(1)
        assert (g[~nz] == 0).all(), what
        _rows(g[nz], want[nz], what)
    for got, want, what in ((b.d_shared, o_dsh, "d_shared"), (b.dx, o_dx, "dx"),
                            (b.dw_lat_up, o_dwlu, "dw_lat_up"), (b.dws_down, o_dwsd, "dws_down"),
                            (b.dw_lat_down, o_dwld, "dw_lat_down"), (b.dws_gate, o_dwsg, "dws_gate"),
                            (b.dws_up, o_dwsu, "dws_up"), (b.dw_gate, o_dwg, "dw_gate"),
                            (b.dw_up, o_dwu, "dw_up"), (b.dw_down, o_dwd, "dw_down")):
        g, w_ = gc.host(got), np.asarray(want)
        nz = np.abs(f64(w_)).reshape(-1, w_.shape[-1]).any(1)
        g2 = g.reshape(-1, w_.shape[-1])
        assert (g2[~nz] == 0).all(), what
        _rows(g2[nz], w_.reshape(-1, w_.shape[-1])[nz], what)
    gl = gc.host(b.d_logits)
    scale = np.abs(o_dl).max(1, keepdims=True) + 1e-30
    assert (np.abs(gl - o_dl) <= 2e-2 * scale).all()
