"""Full-size parity in the launch configuration bench.py times.

One rank's share with the receive buffer built from all 64 source shards
(config 1: T=4096, 6144/3072, 384 experts on 64 ranks; configs 2-4: T=16384
Zipf-skewed routing, T=65536 correlated routing, and the capacity sweep
including the ragged / dropless path).  The GPU runs bench.setup + one
bench.step.  The oracle gets only generator tensors (each shard's logits,
x rows, weights) and redoes every integer decision in full -- top-k of the
own shard, sender slots of every shard, the receive headers, bank slots --
and the GEMM outputs on sampled rows it recomputes one by one from x.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import gpucase as gc
from conftest import u16
from synth import configs, gen

pytestmark = pytest.mark.gpu


def hottest_rank(cfg):
    b = gen.zipf_bias(cfg).numpy()
    return int(np.argmax(b)) // cfg.experts_per_rank


CASES = [
    ("share4k", configs.SHARE_4K, 0, dict(z=12, ffn=16, comb=4)),
    ("zipf16k_r0", configs.ZIPF_16K, 0, dict(z=6, ffn=8, comb=2)),
    ("zipf16k_hot", configs.ZIPF_16K, "hot", dict(z=6, ffn=8, comb=2)),
    ("long65k", configs.LONG_65K, 0, dict(z=4, ffn=6, comb=2)),
    ("sweep16k_cf1.5", configs.SWEEP_16K["1.5/1.5"], "hot", dict(z=4, ffn=6, comb=2)),
    ("sweep16k_cf2.0", configs.SWEEP_16K["2.0/2.0"], "hot", dict(z=4, ffn=6, comb=2)),
    ("sweep16k_ragged", configs.SWEEP_16K["inf"], "hot", dict(z=4, ffn=6, comb=2)),
]


def _headers_for_rank(cfg, d_orc, topk, slot, demand, rank):
    """Receive-segment ids that shard (topk, slot) sends to `rank`, per wave."""
    El, W = cfg.experts_per_rank, cfg.n_waves
    Tw = math.ceil(cfg.T / W)
    wave = (np.arange(cfg.T) // Tw)[:, None].repeat(cfg.top_k, 1)
    m = (topk // El == rank) & (slot >= 0)
    segs = []
    for w in range(W):
        n = d_orc.cap_send if d_orc.cap_send else int(demand[rank * W + w])
        h = -np.ones(n, np.int32)
        sel = m & (wave == w)
        h[slot[sel]] = topk[sel]
        segs.append(h)
    return segs


def _token_of(cfg, topk, slot, rank, w, i):
    """(t, j) of the assignment that holds slot i of pool (rank, wave w)."""
    El, Tw = cfg.experts_per_rank, math.ceil(cfg.T / cfg.n_waves)
    t0, t1 = w * Tw, min(cfg.T, (w + 1) * Tw)
    sub = (topk[t0:t1] // El == rank) & (slot[t0:t1] == i)
    t, j = np.argwhere(sub)[0]
    return t0 + int(t), int(j)


@pytest.mark.parametrize("name,cfg,rank,ns", CASES, ids=[c[0] for c in CASES])
def test_full_share(orc, name, cfg, rank, ns):
    import bench
    if rank == "hot":
        rank = hottest_rank(cfg)
    print(f"\n[full] {name}: setup rank {rank}", flush=True)
    st = bench.setup(cfg, rank, keep_logits=True)
    bench.step(st)
    torch.cuda.synchronize()
    d = st.d
    d_orc = orc.dims(cfg)
    assert (d.cap_send, d.cap_recv) == (d_orc.cap_send, d_orc.cap_recv)
    R, W, L, El = cfg.n_ranks, cfg.n_waves, cfg.latent, cfg.experts_per_rank
    rng = np.random.default_rng(zlib.crc32(name.encode()))

    # ---- integer decisions, in full
    shards = []
    for s in range(cfg.n_shards):
        topk, gates = orc.route(st.host_logits[s], cfg.top_k)
        sn = orc.sender(d_orc, topk)
        shards.append(dict(topk=topk, gates=gates, **sn))
    own = shards[rank]
    assert np.array_equal(gc.host(st.snd.topk), own["topk"])
    np.testing.assert_allclose(gc.host(st.snd.gates), own["gates"], rtol=2e-5)
    assert np.array_equal(gc.host(st.snd.slot), own["slot"])
    assert np.array_equal(gc.host(st.snd.fill), own["fill"])
    assert np.array_equal(gc.host(st.snd.demand), own["demand"])
    if d.cap_send == 0:
        assert np.array_equal(gc.host(st.snd.pool_offsets), own["pool_offsets"])
    print(f"[full] {name}: routing and sender slots match", flush=True)

    segs, seg_src = [], []
    for s, sh in enumerate(shards):
        for w, h in enumerate(_headers_for_rank(cfg, d_orc, sh["topk"], sh["slot"],
                                                sh["demand"], rank)):
            segs.append(h)
            seg_src.append((s, w))
    hdr = np.concatenate(segs)
    lens = np.array([len(h) for h in segs])
    starts = np.concatenate([[0], np.cumsum(lens)])
    roffs = None if d.cap_send else starts.astype(np.int64)
    assert st.n_recv_rows == len(hdr)
    g_recv = st.recv.view(-1, 2 * L + 16)
    g_hdr = g_recv[:, 2 * L:2 * L + 4].contiguous().view(torch.int32).reshape(-1).cpu().numpy()
    assert np.array_equal(g_hdr, hdr)
    if roffs is not None:
        assert np.array_equal(gc.host(st.recv_offsets), roffs)
    bo = orc.bank_slots(d_orc, rank, hdr, roffs)
    assert np.array_equal(gc.host(st.rcv.bank_src), bo["bank_src"])
    assert np.array_equal(gc.host(st.rcv.bfill), bo["bfill"])
    assert np.array_equal(gc.host(st.rcv.bdemand), bo["bdemand"])
    assert int(gc.host(st.rcv.bad_rows)[0]) == bo["bad_rows"] == 0
    if roffs is not None:
        assert np.array_equal(gc.host(st.rcv.bank_offsets), bo["bank_offsets"])
    print(f"[full] {name}: receive headers and bank slots match "
          f"(kept {int(bo['bfill'].sum())} of {int(bo['bdemand'].sum())})", flush=True)

    # ---- copies: every kept pool row of the own shard is its z row; every
    # used bank row is its receive row (device-side comparisons, all rows)
    bsrc = st.rcv.bank_src.long()
    used = bsrc >= 0
    got = st.rcv.bank[used].view(torch.int16)
    want = g_recv[bsrc[used], :2 * L].contiguous().view(torch.int16).view(-1, L)
    assert torch.equal(got, want)
    slot_t = st.snd.slot.long()
    keep = slot_t >= 0
    tok_all = torch.arange(cfg.T, device="cuda")
    tok = tok_all[:, None].expand_as(slot_t)[keep]
    wave_t = tok_all // math.ceil(cfg.T / W)
    p = ((st.snd.topk.long() // El) * W + wave_t[:, None])[keep]
    if d.cap_send:
        prow = p * d.cap_send + slot_t[keep]
    else:
        prow = st.snd.pool_offsets[p] + slot_t[keep]
    pools = st.snd.pools
    assert torch.equal(pools[prow, :2 * L].contiguous().view(torch.int16).view(-1, L),
                       st.snd.z.view(torch.int16)[tok])

    # ---- GEMM outputs on sampled rows, recomputed from generator inputs
    wld = u16(st.wld)
    xcache = {}

    def xrow(s, t):
        if s not in xcache:
            xcache.clear()
            xcache[s] = gen.hidden(cfg, s, "cuda")
        return u16(xcache[s][t:t + 1])

    zt = rng.choice(cfg.T, ns["z"], replace=False)
    zo = orc.latent(u16(st.x), wld, rows=zt)
    gc.assert_rows_close(gc.host(st.snd.z)[zt], zo, "z (sampled)")

    wg, wu, wd = (u16(w) for w in (st.wg, st.wu, st.wd))

    def seg_of(row):
        k = int(np.searchsorted(starts, row, side="right")) - 1
        return seg_src[k][0], seg_src[k][1], int(row - starts[k])

    def oracle_ret_row(row):
        """FFN output the oracle expects at receive row `row` (0 if not kept)."""
        s, w, i = seg_of(row)
        e = int(hdr[row])
        t, j = _token_of(cfg, shards[s]["topk"], shards[s]["slot"], rank, w, i)
        assert shards[s]["topk"][t, j] == e
        z = orc.latent(xrow(s, t), wld)[0]
        j_loc = e % El
        return orc.ffn_row(z, wg[j_loc], wu[j_loc], wd[j_loc])

    kept_rows = bo["bank_src"][bo["bank_src"] >= 0]
    if len(kept_rows):
        pick = rng.choice(kept_rows, min(ns["ffn"], len(kept_rows)), replace=False)
        pick = sorted(pick, key=lambda r: seg_of(r)[0])
        ret_g = gc.host(st.rcv.ret)
        ref = np.stack([oracle_ret_row(r) for r in pick])
        gc.assert_rows_close(ret_g[pick], ref, "ret (sampled)")
        dropped = np.setdiff1d(np.arange(len(hdr)), kept_rows)
        if len(dropped):
            assert (ret_g[dropped] == 0).all()
    print(f"[full] {name}: sampled z and FFN rows match", flush=True)

    # combine: sampled tokens of the own shard, with the returned rows they read
    kept_set = set(kept_rows.tolist())
    Tw = math.ceil(cfg.T / W)
    toks = rng.choice(cfg.T, ns["comb"], replace=False)
    returned = np.zeros((len(hdr), L), np.uint16)
    for t in toks:
        for j in range(cfg.top_k):
            sl = own["slot"][t, j]
            if sl < 0:
                continue
            dd, w = own["topk"][t, j] // El, t // Tw
            seg = dd * W + w
            if sl >= lens[seg]:
                continue
            row = starts[seg] + sl
            if row in kept_set and not returned[row].any():
                returned[row] = oracle_ret_row(row)
    wlu = u16(st.wlu)
    wsg, wsu, wsd = (u16(w) for w in (st.wsg, st.wsu, st.wsd))
    yo, oo = orc.combine(d_orc, returned, roffs, own["topk"], own["slot"], own["gates"],
                         u16(st.x), wlu, wsg, wsu, wsd, tokens=toks)
    gc.assert_rows_close(gc.host(st.cmb.ylat)[toks], yo, "ylat (sampled)")
    gc.assert_rows_close(gc.host(st.cmb.out)[toks], oo, "out (sampled)")
    print(f"[full] {name}: sampled combine rows match", flush=True)
