"""Full-size parity of the wave and dedup variants, in the launch
configuration bench.py times (bench.py --waves chunks / --dedup: the 4096-token
shard, model width 6144, latent 3072, 384 experts on 64 ranks).

As in the default mode's full-size test, the GPU runs bench.setup + one
bench.step and the oracle gets only generator tensors: it redoes every
integer decision in full (top-k of every shard, sender slots, the receive
tails of rank r's buffer, bank slots) and the GEMM outputs on sampled rows,
one by one from x.
"""
import math
import zlib
from dataclasses import replace

import numpy as np
import pytest
import torch

import gpucase as gc
from conftest import u16
from synth import configs, gen

pytestmark = pytest.mark.gpu

CASES = [
    ("share4k_chunks", replace(configs.SHARE_4K, waves="chunks"), 0),
    ("share4k_dedup", replace(configs.SHARE_4K, dedup=True), 5),
    ("zipf16k_chunks_dedup", replace(configs.ZIPF_16K, waves="chunks", dedup=True), 35),
]


def _row_index(cfg, d_orc, topk, slot):
    """Pool row of every (t, j) (-1 if dropped) and, with dedup, its id index
    in the row (its rank among the token's same-destination choices, mod 4)."""
    El, W, C = cfg.experts_per_rank, cfg.n_waves, d_orc.cap_send
    dest = topk // El
    if cfg.waves == "chunks":
        row = dest * W * C + slot
    else:
        row = (dest * W + (np.arange(cfg.T) // math.ceil(cfg.T / W))[:, None]) * C + slot
    row = np.where(slot >= 0, row, -1)
    idx = np.zeros_like(topk)
    if cfg.dedup:
        for j in range(cfg.top_k):
            idx[:, j] = (dest[:, :j] == dest[:, j:j + 1]).sum(1) % 4
    return row, idx


def _tails_for_rank(cfg, d_orc, topk, slot, rank):
    """The receive tails shard (topk, slot) sends to `rank`: [W*C] first ids,
    or [W*C, 4] ids with dedup."""
    El, W, C = cfg.experts_per_rank, cfg.n_waves, d_orc.cap_send
    row, idx = _row_index(cfg, d_orc, topk, slot)
    mine = (topk // El == rank) & (row >= 0)
    ids = -np.ones((W * C, 4), np.int32)
    ids[row[mine] - rank * W * C, idx[mine]] = topk[mine]
    return ids if cfg.dedup else ids[:, 0].copy()


@pytest.mark.parametrize("name,cfg,rank", CASES, ids=[c[0] for c in CASES])
def test_full_variant(orc, name, cfg, rank):
    import bench
    print(f"\n[full variant] {name}: setup rank {rank}", flush=True)
    st = bench.setup(cfg, rank, keep_logits=True)
    bench.step(st)
    torch.cuda.synchronize()
    d = st.d
    d_orc = orc.dims(cfg)
    assert (d.cap_send, d.cap_recv, d.wave_mode, d.dedup) == \
        (d_orc.cap_send, d_orc.cap_recv, d_orc.wave_mode, d_orc.dedup)
    R, W, L, El, C = cfg.n_ranks, cfg.n_waves, cfg.latent, cfg.experts_per_rank, d.cap_send
    per = 4 if cfg.dedup else 1
    rng = np.random.default_rng(zlib.crc32(name.encode()))

    # ---- integer decisions, in full
    shards = []
    for s in range(cfg.n_shards):
        topk, gates = orc.route(st.host_logits[s], cfg.top_k)
        sn = orc.sender(d_orc, topk)
        shards.append(dict(topk=topk, gates=gates, **sn))
    own = shards[rank]
    assert np.array_equal(gc.host(st.snd.topk), own["topk"])
    assert np.array_equal(gc.host(st.snd.slot), own["slot"])
    assert np.array_equal(gc.host(st.snd.fill), own["fill"])
    assert np.array_equal(gc.host(st.snd.demand), own["demand"])
    tails = np.concatenate([_tails_for_rank(cfg, d_orc, sh["topk"], sh["slot"], rank)
                            for sh in shards])
    g_recv = st.recv.view(-1, 2 * L + 16)
    g_tails = g_recv[:, 2 * L:2 * L + 4 * per].contiguous().view(torch.int32).cpu().numpy()
    assert np.array_equal(g_tails.reshape(tails.shape), tails)
    bo = orc.bank_slots(d_orc, rank, tails, None)
    assert np.array_equal(gc.host(st.rcv.bank_src), bo["bank_src"])
    assert np.array_equal(gc.host(st.rcv.bfill), bo["bfill"])
    assert np.array_equal(gc.host(st.rcv.bdemand), bo["bdemand"])
    assert int(gc.host(st.rcv.bad_rows)[0]) == bo["bad_rows"] == 0
    print(f"[full variant] {name}: routing, sender slots, tails and bank slots match "
          f"(kept {int(bo['bfill'].sum())} of {int(bo['bdemand'].sum())})", flush=True)

    # ---- copies: kept pool rows of the own shard hold their token's z row;
    # used bank rows hold their receive row's payload
    orow, _ = _row_index(cfg, d_orc, own["topk"], own["slot"])
    keep = orow >= 0
    tok = np.broadcast_to(np.arange(cfg.T)[:, None], orow.shape)[keep]
    pools = st.snd.pools
    rows_t = torch.from_numpy(orow[keep]).cuda()
    assert torch.equal(pools[rows_t, :2 * L].contiguous().view(torch.int16).view(-1, L),
                       st.snd.z.view(torch.int16)[torch.from_numpy(tok).cuda()])
    bsrc = st.rcv.bank_src.long()
    used = bsrc >= 0
    want = g_recv[bsrc[used] // per, :2 * L].contiguous().view(torch.int16).view(-1, L)
    assert torch.equal(st.rcv.bank[used].view(torch.int16), want)

    # ---- GEMM outputs on sampled rows, recomputed from generator inputs
    wld = u16(st.wld)
    wg, wu, wd = (u16(w) for w in (st.wg, st.wu, st.wd))
    # which (shard, token) sent each receive row of rank r
    row_token = {}
    for s, sh in enumerate(shards):
        r_, _ = _row_index(cfg, d_orc, sh["topk"], sh["slot"])
        m = (sh["topk"] // El == rank) & (r_ >= 0)
        for t, rr in zip(np.nonzero(m)[0], r_[m]):
            row_token[s * W * C + int(rr) - rank * W * C] = (s, int(t))
    xcache = {}

    def xrow(s, t):
        if s not in xcache:
            xcache.clear()
            xcache[s] = gen.hidden(cfg, s, "cuda")
        return u16(xcache[s][t:t + 1])

    def oracle_ret_slot(q):
        """FFN output the oracle expects at return slot q."""
        row, i = divmod(q, per)
        e = int(tails[row, i] if cfg.dedup else tails[row])
        s, t = row_token[row]
        z = orc.latent(xrow(s, t), wld)[0]
        return orc.ffn_row(z, wg[e % El], wu[e % El], wd[e % El])

    kept = bo["bank_src"][bo["bank_src"] >= 0]
    pick = sorted(rng.choice(kept, 12, replace=False), key=lambda q: row_token[q // per][0])
    ret_g = gc.host(st.rcv.ret)
    gc.assert_rows_close(ret_g[pick], np.stack([oracle_ret_slot(q) for q in pick]),
                         "ret (sampled)")
    present = np.nonzero((tails >= 0).reshape(-1))[0] if cfg.dedup else np.nonzero(tails >= 0)[0]
    dropped = np.setdiff1d(present, kept)
    assert (ret_g[dropped] == 0).all()             # sent but not banked: zero return
    print(f"[full variant] {name}: sampled FFN rows match", flush=True)

    # combine: sampled tokens; under the loopback identity a choice of pool
    # row p (id index i) reads return slot p * per + i of rank r's buffer,
    # which the oracle rebuilds (0 where that slot was not banked)
    toks = rng.choice(cfg.T, 3, replace=False)
    kept_set = set(kept.tolist())
    returned = np.zeros((len(tails) * per, L), np.uint16)
    orow, oidx = _row_index(cfg, d_orc, own["topk"], own["slot"])
    for t in toks:
        for j in range(cfg.top_k):
            if orow[t, j] < 0:
                continue
            q = int(orow[t, j]) * per + int(oidx[t, j])
            if q in kept_set and not returned[q].any():
                returned[q] = oracle_ret_slot(q)
    wlu = u16(st.wlu)
    wsg, wsu, wsd = (u16(w) for w in (st.wsg, st.wsu, st.wsd))
    yo, oo = orc.combine(d_orc, returned, None, own["topk"], own["slot"], own["gates"],
                         u16(st.x), wlu, wsg, wsu, wsd, tokens=toks)
    gc.assert_rows_close(gc.host(st.cmb.ylat)[toks], yo, "ylat (sampled)")
    gc.assert_rows_close(gc.host(st.cmb.out)[toks], oo, "out (sampled)")
    print(f"[full variant] {name}: sampled combine rows match", flush=True)
