"""Whole path on the GPU against the whole path in the oracle.

Both sides start from the same generator inputs and each runs its own chain
(route -> pack -> loopback -> bank -> FFN -> combine) for rank 0, so this
also checks that the stages fit together.  Integer decisions are compared
bit for bit; bf16 tensors per row within 2e-2 * max|ref| (upstream bf16
rounding may differ by one unit between the sides, which the per-row
tolerance absorbs).
"""
import numpy as np
import pytest
import torch

import gpucase as gc
from conftest import u16
from synth import configs, gen

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": configs.TINY,
    "mid": gc.MID,
    "mid_ragged": gc.ragged(gc.MID),
    "mid_zipf": gc.skewed(gc.MID),
    "mid_zipf_chunks": gc.chunked(gc.skewed(gc.MID)),
    "mid_dedup": gc.deduped(gc.MID),
    # degenerate shapes: one rank holding every expert, one wave, no capacity,
    # no shared experts (a plain top-k MoE layer); top-1 routing
    "tiny_dense_r1_w1_s0": configs.scaled(configs.TINY, configs.TINY.name + "_R1_W1_S0",
                                          n_ranks=1, n_waves=1, n_shared=0, cf_send=None,
                                          cf_recv=None),
    "mid_k1": configs.scaled(gc.MID, gc.MID.name + "_k1", top_k=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_chain(orc, name):
    from dispatch_softmax_top_amd import share
    cfg = CASES[name]
    rank = 0
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    R, W = cfg.n_ranks, cfg.n_waves
    wld = gen.latent_down(cfg)
    wg, wu, wd = gen.rank_experts(cfg, rank)
    wlu = gen.latent_up(cfg)
    wsg, wsu, wsd = gen.shared(cfg)

    # ---- GPU chain
    g_pools, g_offs, own = [], [], None
    for s in range(cfg.n_shards):
        x, lg = gc.shard_inputs(cfg, s)
        snd = share.Sender(d)
        snd.route(lg.cuda())
        snd.pack(x.cuda(), wld.cuda())
        g_pools.append(snd.pools)
        g_offs.append(snd.pool_offsets)
        if s == rank:
            own, x_own = snd, x
    if d.cap_send:
        recv = share.loopback_recv_fixed(d, g_pools, rank)
        roffs = None
    else:
        recv, roffs = share.loopback_recv_ragged(d, g_pools, g_offs, rank)
    rcv = share.Receiver(d, recv.shape[0])
    rcv.bank_rows(rank, recv, roffs)
    rcv.ffn(wg.cuda(), wu.cuda(), wd.cuda())
    cmb = share.Combiner(d)
    cmb.combine(rcv.ret, roffs, own, x_own.cuda(), wlu.cuda(), wsg.cuda(), wsu.cuda(),
                wsd.cuda())
    torch.cuda.synchronize()

    # ---- oracle chain
    o_pools, o_snd = [], []
    for s in range(cfg.n_shards):
        x, lg = gc.shard_inputs(cfg, s)
        topk, gates = orc.route(lg.numpy(), cfg.top_k)
        z = orc.latent(u16(x), u16(wld))
        sn = orc.sender(d_orc, topk)
        o_pools.append(orc.pack_rows(d_orc, z, topk, sn["slot"], sn["pool_offsets"]))
        o_snd.append(dict(topk=topk, gates=gates, z=z, **sn))
    parts, lens = [], []
    for s in range(cfg.n_shards):
        for w in range(W):
            if d.cap_send:
                a = (rank * W + w) * d.cap_send
                b = a + d.cap_send
            else:
                a, b = o_snd[s]["pool_offsets"][rank * W + w], o_snd[s]["pool_offsets"][rank * W + w + 1]
            parts.append(o_pools[s][a:b])
            lens.append(b - a)
    o_recv = np.concatenate(parts)
    o_roffs = None if d.cap_send else np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    bo = orc.bank_slots(d_orc, rank, orc.recv_ids(d_orc, o_recv), o_roffs)
    o_bank = orc.bank_rows(d_orc, o_recv, bo["bank_offsets"], bo["bank_src"], bo["bfill"])
    o_ret = orc.expert_ffn(d_orc, o_bank, bo["bank_offsets"], bo["bank_src"], bo["bfill"],
                           u16(wg), u16(wu), u16(wd), len(o_recv) * (4 if d.dedup else 1))
    s0 = o_snd[rank]
    o_ylat, o_out = orc.combine(d_orc, o_ret, o_roffs, s0["topk"], s0["slot"], s0["gates"],
                                u16(x_own), u16(wlu), u16(wsg), u16(wsu), u16(wsd))

    # ---- compare
    assert np.array_equal(gc.host(own.topk), s0["topk"])
    assert np.array_equal(gc.host(own.slot), s0["slot"])
    assert np.array_equal(gc.host(own.fill), s0["fill"])
    assert np.array_equal(gc.host(own.demand), s0["demand"])
    gc.assert_rows_close(gc.host(own.z), s0["z"], "z")
    g_recv = gc.host(recv)
    assert g_recv.shape == o_recv.shape
    assert np.array_equal(orc.recv_ids(d_orc, g_recv), orc.recv_ids(d_orc, o_recv))
    if roffs is not None:
        assert np.array_equal(gc.host(roffs), o_roffs)
    assert np.array_equal(gc.host(rcv.bank_src), bo["bank_src"])
    assert np.array_equal(gc.host(rcv.bfill), bo["bfill"])
    assert np.array_equal(gc.host(rcv.bdemand), bo["bdemand"])
    assert int(gc.host(rcv.bad_rows)[0]) == 0
    used = bo["bank_src"] >= 0
    gc.assert_rows_close(gc.host(rcv.bank)[used], o_bank[used], "bank")
    gc.assert_rows_close(gc.host(rcv.ret), o_ret, "ret")
    gc.assert_rows_close(gc.host(cmb.ylat), o_ylat, "ylat")
    gc.assert_rows_close(gc.host(cmb.out), o_out, "out")


def test_repeat_determinism():
    """Same inputs, several runs and a different launch history: bitwise equal."""
    from dispatch_softmax_top_amd import share
    cfg = gc.MID
    d = share.make_dims(cfg)
    x, lg = gc.shard_inputs(cfg, 0)
    wld = gen.latent_down(cfg).cuda()
    ref = None
    for it in range(4):
        snd = share.Sender(d)
        snd.route(lg.cuda())
        snd.pack(x.cuda(), wld)
        torch.cuda.synchronize()
        cur = [gc.host(t).copy() for t in (snd.topk, snd.slot, snd.fill, snd.z)]
        cur.append(orc_headers(snd.pools, d.latent))
        if ref is None:
            ref = cur
        else:
            for a, b in zip(ref, cur):
                assert np.array_equal(a, b)


def orc_headers(pools, latent):
    p = gc.host(pools)
    return np.ascontiguousarray(p[:, 2 * latent:2 * latent + 4]).view(np.int32).reshape(-1)
