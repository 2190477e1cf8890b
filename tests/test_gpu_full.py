"""Full-size parity in the launch configuration bench.py times.

One rank's share with the receive buffer built from all 64 source shards
(4096 tokens per shard at 6144/3072, 384 experts on 64 ranks; 16384 tokens
with Zipf-skewed routing; 65536 tokens with correlated routing; the capacity
sweep including the ragged / dropless path).  The GPU runs bench.setup and
one bench.step.  The oracle gets only generator tensors (each shard's
logits, x rows, weights) and redoes every integer decision in full: top-k of
every shard, sender slots of every shard, the receive headers, bank slots;
"hot" is the rank with the most kept received rows, found from the oracle's
own decisions and checked to be the rank bench.py measures as hot.

Floating-point outputs are checked against oracle/dense.py (the oracle's
definitions as float64 matrix products), row by row within 2e-2 * max|ref|:
  - 4096 tokens: every row of z, of the return buffer, of ylat and of out;
  - the larger workloads: every row of z, and of the return buffer and of
    ylat / out a selection that reaches every kind of tile the GEMMs run --
    the first and last row of every (wave, expert) bank group; a row of every
    32-row MFMA group of every tile the K-split last round of the expert
    SwiGLU or down GEMM cuts; the first and last row of every 256-row M tile
    of every product group; the first and last token of every wave and of
    every M tile of the up-projection; tokens with a choice dropped at the
    sender or reading a zero return row (a seeded 1024 of them when there are
    more); every return row those tokens read; and seeded random rows and
    tokens up to 1024 of each.  The test asserts that the selection holds
    every such row.
Every return row no kept bank row writes must be zero (all rows, on the
device).  The 4096-token case also runs the step ten times and once more
with every call on one stream, and requires every output bit-identical, and
runs the backward of the share three times, every gradient bit-identical.
"""
import math
import os
import zlib

import numpy as np
import pytest
import torch

import fullcheck as fc
import gpucase as gc
from conftest import u16
from oracle import dense
from synth import configs, gen

pytestmark = pytest.mark.gpu

NMIN = 1024        # rows per output at least, outside the every-row case

CASES = [
    # name, workload, rank (or "hot"), every row
    ("share4k", configs.SHARE_4K, 0, True),
    ("zipf16k_r0", configs.ZIPF_16K, 0, False),
    ("zipf16k_hot", configs.ZIPF_16K, "hot", False),
    ("long65k", configs.LONG_65K, 0, False),
    ("long65k_hot", configs.LONG_65K, "hot", False),
    ("sweep16k_cf1.5", configs.SWEEP_16K["1.5/1.5"], "hot", False),
    ("sweep16k_cf2.0", configs.SWEEP_16K["2.0/2.0"], "hot", False),
    ("sweep16k_ragged", configs.SWEEP_16K["inf"], "hot", False),
]


def _outputs(st):
    """Every output of a step, as device tensors (copies)."""
    L = st.d.latent
    s, r, c = st.snd, st.rcv, st.cmb
    used = r.bank_src >= 0
    ids = s.pools[:, 2 * L:2 * L + 4].contiguous().view(torch.int32).reshape(-1)
    out = dict(topk=s.topk, gates=s.gates, slot=s.slot, fill=s.fill, demand=s.demand, z=s.z,
               pool_tails=s.pools[:, 2 * L:], pool_rows=s.pools[ids >= 0, :2 * L],
               bank_src=r.bank_src, bfill=r.bfill, bdemand=r.bdemand, bank=r.bank[used],
               ret=r.ret, ylat=c.ylat, out=c.out)
    return {k: v.clone() for k, v in out.items()}


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _check_planned_cus(st, name, groups, split_mtiles, up_mtiles, bank_src, n_ret, rows_all):
    """The step with the GEMM launchers planning for 64 and for 200 CUs
    (MOE_GEMM_CUS) instead of the device's: other persistent grids, another
    work-queue spread, and no K-split last round at these counts.  Outputs of
    tiles that the device-count run does not split must be bit-identical;
    rows those split tiles touch (their bank rows' return rows, the tokens
    that read them, the up-projection's split tiles) agree within the
    floating-point tolerance.  The device-count step runs again after."""
    import bench
    ref = _outputs(st)
    hit = np.zeros(n_ret, bool)
    for pg, mt in split_mtiles:
        pos = groups[pg][mt * fc.GBM:(mt + 1) * fc.GBM]
        src = bank_src[pos]
        hit[src[src >= 0]] = True
    tok_hit = ((rows_all >= 0) & hit[np.maximum(rows_all, 0)]).any(1)
    for mt in up_mtiles:
        tok_hit[mt * fc.GBM:(mt + 1) * fc.GBM] = True
    exact = ("topk", "gates", "slot", "fill", "demand", "z", "pool_tails", "pool_rows",
             "bank_src", "bfill", "bdemand", "bank")
    try:
        for cus in ("64", "200"):
            os.environ["MOE_GEMM_CUS"] = cus
            bench.step(st)
            torch.cuda.synchronize()
            now = _outputs(st)
            bad = [k for k in exact if not _same(ref[k], now[k])]
            assert not bad, f"planned for {cus} CUs: {bad} differ"
            for k, rows in (("ret", hit), ("ylat", tok_hit), ("out", tok_hit)):
                keep = torch.from_numpy(~rows).cuda()
                assert _same(ref[k][keep], now[k][keep]), f"planned for {cus} CUs: {k} differs"
                if rows.any():
                    sel = torch.from_numpy(rows).cuda()
                    gc.assert_rows_close(gc.host(now[k][sel]), gc.host(ref[k][sel]),
                                         f"{k} planned for {cus} CUs, split rows")
            print(f"[full] {name}: planned for {cus} CUs: bit-identical outside the "
                  f"{int(hit.sum())} return rows and {int(tok_hit.sum())} tokens of split tiles, "
                  f"close on those", flush=True)
    finally:
        os.environ.pop("MOE_GEMM_CUS", None)
    bench.step(st)
    torch.cuda.synchronize()
    assert all(_same(ref[k], v) for k, v in _outputs(st).items()), "device-count step changed"


@pytest.mark.parametrize("name,cfg,which,full", CASES, ids=[c[0] for c in CASES])
def test_full_share(orc, name, cfg, which, full):
    import bench
    import dispatch_softmax_top_amd as moe
    print(f"\n[full] {name}: setup rank 0", flush=True)
    st = bench.setup(cfg, 0, keep_logits=True)
    logits = st.host_logits
    st.host_logits = None
    d_orc = orc.dims(cfg)
    assert (st.d.cap_send, st.d.cap_recv) == (d_orc.cap_send, d_orc.cap_recv)
    shards = fc.oracle_shards(orc, cfg, d_orc, logits)
    r_star = fc.hot_rank(cfg, d_orc, shards)
    assert bench.receiver_stats(st)[1] == r_star, "bench's hot rank differs from the oracle's"
    rank = r_star if which == "hot" else which
    if rank != 0:
        print(f"[full] {name}: setup rank {rank} (the hot rank)", flush=True)
        del st
        torch.cuda.empty_cache()
        st = bench.setup(cfg, rank)
        assert np.array_equal(st.logits.cpu().numpy(), logits[rank])
    del logits
    bench.step(st)
    torch.cuda.synchronize()
    d = st.d
    T, R, W, L, El = cfg.T, cfg.n_ranks, cfg.n_waves, cfg.latent, cfg.experts_per_rank
    D, F, S, Fs = cfg.d_model, cfg.d_ff, cfg.n_shared, cfg.d_ff_shared
    Tw = math.ceil(T / W)
    rng = np.random.default_rng(zlib.crc32(name.encode()))

    # ---- integer decisions, in full
    own = shards[rank]
    assert np.array_equal(gc.host(st.snd.topk), own["topk"])
    np.testing.assert_allclose(gc.host(st.snd.gates), own["gates"], rtol=2e-5)
    assert np.array_equal(gc.host(st.snd.slot), own["slot"])
    assert np.array_equal(gc.host(st.snd.fill), own["fill"])
    assert np.array_equal(gc.host(st.snd.demand), own["demand"])
    if d.cap_send == 0:
        assert np.array_equal(gc.host(st.snd.pool_offsets), own["pool_offsets"])
    print(f"[full] {name}: routing and sender slots match", flush=True)

    rm = fc.RecvMap(cfg, d_orc, shards, rank)
    assert st.n_recv_rows == rm.n
    g_recv = st.recv.view(-1, 2 * L + 16)
    g_hdr = g_recv[:, 2 * L:2 * L + 4].contiguous().view(torch.int32).reshape(-1).cpu().numpy()
    assert np.array_equal(g_hdr, rm.hdr)
    if rm.offsets is not None:
        assert np.array_equal(gc.host(st.recv_offsets), rm.offsets)
    bo = orc.bank_slots(d_orc, rank, rm.hdr, rm.offsets)
    assert np.array_equal(gc.host(st.rcv.bank_src), bo["bank_src"])
    assert np.array_equal(gc.host(st.rcv.bfill), bo["bfill"])
    assert np.array_equal(gc.host(st.rcv.bdemand), bo["bdemand"])
    assert int(gc.host(st.rcv.bad_rows)[0]) == bo["bad_rows"] == 0
    if rm.offsets is not None:
        assert np.array_equal(gc.host(st.rcv.bank_offsets), bo["bank_offsets"])
    print(f"[full] {name}: receive headers and bank slots match "
          f"(kept {int(bo['bfill'].sum())} of {int(bo['bdemand'].sum())})", flush=True)

    # ---- copies: every kept pool row of the own shard is its z row; every
    # used bank row is its receive row (device-side comparisons, all rows)
    bsrc = st.rcv.bank_src.long()
    used = bsrc >= 0
    assert torch.equal(st.rcv.bank[used].view(torch.int16),
                       g_recv[bsrc[used], :2 * L].contiguous().view(torch.int16).view(-1, L))
    slot_t = st.snd.slot.long()
    keep = slot_t >= 0
    tok_all = torch.arange(T, device="cuda")
    tok = tok_all[:, None].expand_as(slot_t)[keep]
    p = ((st.snd.topk.long() // El) * W + (tok_all // Tw)[:, None])[keep]
    prow = p * d.cap_send + slot_t[keep] if d.cap_send else st.snd.pool_offsets[p] + slot_t[keep]
    assert torch.equal(st.snd.pools[prow, :2 * L].contiguous().view(torch.int16).view(-1, L),
                       st.snd.z.view(torch.int16)[tok])

    # ---- repeats: ten steps on two streams, one on one stream, bit-identical
    if full:
        ref = _outputs(st)
        for i in range(9):
            bench.step(st)
            torch.cuda.synchronize()
            now = _outputs(st)
            bad = [k for k in ref if not _same(ref[k], now[k])]
            assert not bad, f"step {i + 2} differs from step 1 in {bad}"
        moe.moe_profile_reset()
        moe.moe_profile_enable(True)
        bench.step_serial(st)
        moe.moe_profile_collect()
        moe.moe_profile_enable(False)
        prof = moe.moe_profile_read()
        now = _outputs(st)
        bad = [k for k in ref if not _same(ref[k], now[k])]
        assert not bad, f"the one-stream step differs in {bad}"
        print(f"[full] {name}: 10 steps and the one-stream step bit-identical", flush=True)
        # the backward of the same share (as bench.py runs it), three times:
        # every gradient bit-identical (work-queue tile order, split tails)
        from dispatch_softmax_top_amd import share
        st.bwd = share.Backward(d, st.n_recv_rows)
        st.d_out = gen.payload_rows(d.T, d.d_model, 71, "cuda")
        grads = ("d_returned", "d_gates", "d_shared", "dw_lat_up", "dws_down", "d_logits",
                 "d_recv", "dw_gate", "dw_up", "dw_down", "dz", "dx", "dw_lat_down", "dws_gate",
                 "dws_up")
        bref = None
        for i in range(3):
            bench.backward_step(st)
            torch.cuda.synchronize()
            cur = {k: getattr(st.bwd, k).clone() for k in grads}
            if bref is None:
                bref = cur
            else:
                bad = [k for k in grads if not _same(bref[k], cur[k])]
                assert not bad, f"backward run {i + 1} differs from run 1 in {bad}"
        print(f"[full] {name}: backward three times bit-identical", flush=True)

    # ---- which rows: tiles of the GEMMs as the kernels cut them
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    bank_src, bfill, boffs = bo["bank_src"], bo["bfill"], bo["bank_offsets"]
    kept_pos = np.nonzero(bank_src >= 0)[0]
    groups = fc.product_groups(d_orc, bfill, boffs, max(L, F), len(bank_src))
    S_sw, sw_tiles = fc.grouped_split_tiles(groups, F // 128, L, ncu)
    S_dn, dn_tiles = fc.grouped_split_tiles(groups, math.ceil(L / fc.GBN), F, ncu)
    S_up, up_mtiles = fc.dense_split_mtiles(T, D, L + S * Fs, ncu)
    print(f"[full] {name}: K-split last rounds: expert SwiGLU {len(sw_tiles)} M tiles x{S_sw}, "
          f"down {len(dn_tiles)} x{S_dn}, up-projection {len(up_mtiles)} x{S_up}", flush=True)
    if name == "share4k":       # the split path is reached on purpose here
        assert S_sw > 1 and S_dn > 1 and S_up > 1
        assert ("gemm_up_shared_tail" in prof) and ("gemm_expert_swiglu_tail" in prof)

    if full:
        _check_planned_cus(st, name, groups, sw_tiles + dn_tiles, up_mtiles, bank_src, rm.n,
                           dense.returned_rows(d_orc, rm.offsets, own["topk"], own["slot"],
                                               np.arange(T)))

    must_pos = set()
    for g in range(W * El):
        if bfill[g]:
            start = int(boffs[g]) if boffs is not None else g * d.cap_recv
            must_pos |= {start, start + int(bfill[g]) - 1}
    for pg, mt in sw_tiles + dn_tiles:
        must_pos |= set(groups[pg][fc.mtile_probe_rows(len(groups[pg]), mt)].tolist())
    for pos in groups:
        for mt in range(math.ceil(len(pos) / fc.GBM)):
            must_pos |= {int(pos[mt * fc.GBM]), int(pos[min(len(pos), (mt + 1) * fc.GBM) - 1])}

    rows_all = dense.returned_rows(d_orc, rm.offsets, own["topk"], own["slot"], np.arange(T))
    pos_of_row = -np.ones(rm.n, np.int64)
    pos_of_row[bank_src[kept_pos]] = kept_pos
    reads_zero = ((rows_all >= 0) & (pos_of_row[np.maximum(rows_all, 0)] < 0)).any(1)
    drop_toks = np.nonzero((own["slot"] < 0).any(1) | reads_zero)[0]
    must_tok = {0, T - 1}
    for w in range(1, W):
        must_tok |= {w * Tw - 1, w * Tw}
    for mt in range(math.ceil(T / fc.GBM)):
        must_tok |= {mt * fc.GBM, min(T, (mt + 1) * fc.GBM) - 1}
    for mt in up_mtiles:
        must_tok |= set(fc.mtile_probe_rows(T, mt))
    if full:
        ffn_pos, toks = kept_pos, np.arange(T)
    else:
        ffn_pos = np.union1d(np.fromiter(must_pos, np.int64), fc.pick(rng, kept_pos, NMIN))
        toks = np.union1d(np.fromiter(must_tok, np.int64),
                          np.union1d(fc.pick(rng, drop_toks, NMIN), fc.pick(rng, np.arange(T), NMIN)))
    need = rows_all[toks]
    need = pos_of_row[need[need >= 0]]
    ffn_pos = np.union1d(ffn_pos, need[need >= 0]).astype(np.int64)
    assert must_pos <= set(ffn_pos.tolist()) and must_tok <= set(toks.tolist())
    assert len(ffn_pos) >= min(NMIN, len(kept_pos)) and len(toks) >= min(NMIN, T)

    # ---- z: every row of the own shard
    wld = u16(st.wld)
    x_own = u16(st.x)
    gc.assert_rows_close(gc.host(st.snd.z), dense.latent(x_own, wld), "z")
    print(f"[full] {name}: every z row matches", flush=True)

    # ---- return rows: the expert FFN of the oracle's z of each source token
    recv_rows = bank_src[ffn_pos]
    u = fc.source_latent(cfg, rm, recv_rows, wld,
                         lambda s, t: u16(gen.hidden_rows(cfg, s, t, "cuda")))
    wg, wu, wd = (u16(w) for w in (st.wg, st.wu, st.wd))
    ref = np.empty((len(ffn_pos), L), np.uint16)
    ej = rm.hdr[recv_rows] % El
    for j in range(El):
        sel = np.nonzero(ej == j)[0]
        if len(sel):
            ref[sel] = dense.ffn_rows(u[sel], wg[j], wu[j], wd[j])
    got = gc.host(st.rcv.ret[torch.from_numpy(recv_rows).cuda()])
    gc.assert_rows_close(got, ref, "ret")
    written = torch.zeros(rm.n, dtype=torch.bool, device="cuda")
    written[torch.from_numpy(bank_src[kept_pos]).cuda().long()] = True
    assert bool((st.rcv.ret[~written].view(torch.int16) == 0).all()), "unwritten return rows"
    print(f"[full] {name}: {len(ffn_pos)} of {len(kept_pos)} kept return rows match "
          f"({len(must_pos)} required by tile), the other {rm.n - len(kept_pos)} rows are zero",
          flush=True)

    # ---- combine: ylat and out of the chosen tokens
    returned = np.zeros((rm.n, L), np.uint16)
    returned[recv_rows] = ref
    wlu = u16(st.wlu)
    wsg, wsu, wsd = (u16(w) for w in (st.wsg, st.wsu, st.wsd))
    yo, oo = dense.combine_tokens(d_orc, returned, rm.offsets, own["topk"], own["slot"],
                                  own["gates"], x_own, wlu, wsg, wsu, wsd, tokens=toks)
    gc.assert_rows_close(gc.host(st.cmb.ylat)[toks], yo, "ylat")
    gc.assert_rows_close(gc.host(st.cmb.out)[toks], oo, "out")
    print(f"[full] {name}: ylat and out match on {len(toks)} of {T} tokens "
          f"({len(must_tok)} required by tile or wave, {len(drop_toks)} with a drop)", flush=True)
