"""GPU parity per C-ABI call, on inputs shared with the oracle.

Each call gets exactly the inputs the oracle gets (generator tensors and
oracle-made routing / headers), so errors cannot compound between stages.
Integer outputs must match bit for bit; bf16 outputs within 2e-2 * max|ref|
per row.
"""
import math

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
    "mid_ragged": gc.ragged(gc.MID),
    "mid_zipf": gc.skewed(gc.MID),
    "mid_tight": gc.with_cf(gc.MID, "1/2", "3/5"),
    "mid_chunks": gc.chunked(gc.MID),
    "mid_chunks_tight": gc.chunked(gc.with_cf(gc.MID, "1/2", "3/5")),
    "mid_dedup": gc.deduped(gc.MID),
    "mid_dedup_tight": gc.deduped(gc.chunked(gc.with_cf(gc.MID, "1/2", "3/5"))),
    # more waves than the grouped GEMM merges into one product group: every
    # (wave, expert) bank group is its own product group
    "mid_w5": configs.scaled(gc.MID, gc.MID.name + "_W5", n_waves=5),
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


def _dims(orc, share, cfg):
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    assert (d.cap_send, d.cap_recv) == (d_orc.cap_send, d_orc.cap_recv)
    return d_orc, d


# ----------------------------------------------------------------------------
# route
# ----------------------------------------------------------------------------

def _route_check(moe, orc, lg_np, k):
    T, E = lg_np.shape
    topk = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route(gc.dev(lg_np), k, topk, gates)
    torch.cuda.synchronize()
    ot, og = orc.route(lg_np, k)
    assert np.array_equal(gc.host(topk), ot)
    np.testing.assert_allclose(gc.host(gates), og, rtol=2e-5, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_zipf"])
def test_route(moe, orc, name):
    cfg = CASES[name]
    _, lg = gc.shard_inputs(cfg, 0)
    _route_check(moe, orc, lg.numpy(), cfg.top_k)


def test_route_ties_and_edges(moe, orc):
    rng = np.random.default_rng(0)
    for E, k in ((384, 8), (48, 8), (64, 1), (130, 32), (1024, 8), (8, 8)):
        lg = rng.integers(-2, 3, (257, E)).astype(np.float32)   # heavy ties
        lg[0] = 0.0
        lg[1, ::2] = -0.0                                        # -0 ties +0
        _route_check(moe, orc, lg, k)
    _route_check(moe, orc, rng.standard_normal((1, 384)).astype(np.float32), 8)   # T = 1
    # chosen experts crowded on a few lanes (a lane's best three run out with
    # rounds left, so the rounds start again over every candidate)
    for E, k in ((384, 8), (384, 32), (1024, 8), (130, 32)):
        ramp = np.arange(E, dtype=np.float32)
        lg = np.stack([-ramp, ramp, np.roll(-ramp, 7), np.roll(ramp, -100 % E)] * 16)
        _route_check(moe, orc, lg, k)


def test_route_errors(moe):
    lg = torch.zeros(4, 16, device="cuda")
    t = torch.empty(4, 8, dtype=torch.int32, device="cuda")
    g = torch.empty(4, 8, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_route(lg, 17, t, g)                    # k > E
    with pytest.raises(moe.MoeError):
        moe.moe_route(torch.zeros(4, 2000, device="cuda"), 8, t, g)   # E > 1024


# ----------------------------------------------------------------------------
# pack
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
def test_pack(moe, orc, share, name):
    cfg = CASES[name]
    d_orc, d = _dims(orc, share, cfg)
    x, lg = gc.shard_inputs(cfg, 0)
    wld = gen.latent_down(cfg)
    topk, _ = orc.route(lg.numpy(), cfg.top_k)
    # GPU
    snd = share.Sender(d)
    snd.topk.copy_(torch.from_numpy(topk))
    snd.pools.fill_(0xAB)                        # poison: every checked byte must be written
    snd.slot.fill_(-7)
    snd.pack(x.cuda(), wld.cuda())
    torch.cuda.synchronize()
    # oracle
    zo = orc.latent(u16(x), u16(wld))
    so = orc.sender(d_orc, topk)
    po = orc.pack_rows(d_orc, zo, topk, so["slot"], so["pool_offsets"])
    assert np.array_equal(gc.host(snd.slot), so["slot"])
    assert np.array_equal(gc.host(snd.fill), so["fill"])
    assert np.array_equal(gc.host(snd.demand), so["demand"])
    if d.cap_send == 0:
        assert np.array_equal(gc.host(snd.pool_offsets), so["pool_offsets"])
    zg = gc.host(snd.z)
    gc.assert_rows_close(zg, zo, "z")
    pg = gc.host(snd.pools)
    hg, ho = orc.headers(pg, d.latent), orc.headers(po, d.latent)
    assert np.array_equal(hg, ho)
    if d.dedup:
        assert np.array_equal(orc.row_ids(pg, d.latent), orc.row_ids(po, d.latent))
    if not d.dedup:
        assert (pg[:, 2 * d.latent + 4:] == 0).all()      # header tail zeros
    kept = ho >= 0
    # kept rows carry the GPU's own z rows bit for bit
    El, Tw = cfg.experts_per_rank, math.ceil(cfg.T / cfg.n_waves)
    for t in range(cfg.T):
        for j in range(cfg.top_k):
            s = so["slot"][t, j]
            if s < 0:
                continue
            p = (topk[t, j] // El) * cfg.n_waves + t // Tw
            if d.wave_mode == 1:
                row = (topk[t, j] // El) * cfg.n_waves * d.cap_send + s
            else:
                row = p * d.cap_send + s if d.cap_send else so["pool_offsets"][p] + s
            assert np.array_equal(pg[row, :2 * d.latent].view(np.uint16), zg[t])
    assert kept.sum() == so["fill"].sum()


def test_pack_errors(moe, share):
    d = share.make_dims(configs.TINY)
    snd = share.Sender(d)
    x = torch.zeros(d.T, d.d_model, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(d.latent, d.d_model, dtype=torch.bfloat16, device="cuda")
    bad = share.make_dims(configs.TINY)
    bad.latent = 100                                     # not a multiple of 64
    with pytest.raises(moe.MoeError):
        moe.moe_pack_waves(bad, x, w, snd.topk, snd.z, snd.pools, None, snd.slot, snd.fill,
                           snd.demand, snd.ws)
    with pytest.raises(moe.MoeError):                    # workspace too small
        moe.moe_pack_waves(d, x, w, snd.topk, snd.z, snd.pools, None, snd.slot, snd.fill,
                           snd.demand, snd.ws[:16])


# ----------------------------------------------------------------------------
# bank
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("rank", [0, 5])
def test_bank(moe, orc, share, name, rank):
    cfg = CASES[name]
    d_orc, d = _dims(orc, share, cfg)
    senders = gc.oracle_sender_all(orc, cfg, d_orc)
    hdr, offs = gc.recv_headers(cfg, d_orc, senders, rank)
    n = len(hdr)
    if d.cap_send and name == "mid":                 # rows that claim another rank's expert
        empty = np.nonzero(hdr < 0)[0][:5]
        hdr[empty] = ((rank + 1) % cfg.n_ranks) * cfg.experts_per_rank
    payload = u16(gen.payload_rows(n, d.latent, 7))
    recv = gc.rows_with_headers(payload, hdr)
    rcv = share.Receiver(d, n)
    rcv.bank_src.fill_(-9)
    rcv.bank_rows(rank, gc.dev(recv), None if offs is None else gc.dev(offs))
    torch.cuda.synchronize()
    bo = orc.bank_slots(d_orc, rank, hdr, offs)
    assert np.array_equal(gc.host(rcv.bank_src), bo["bank_src"])
    assert np.array_equal(gc.host(rcv.bfill), bo["bfill"])
    assert np.array_equal(gc.host(rcv.bdemand), bo["bdemand"])
    assert int(gc.host(rcv.bad_rows)[0]) == bo["bad_rows"]
    if d.cap_send == 0:
        assert np.array_equal(gc.host(rcv.bank_offsets), bo["bank_offsets"])
    bank_o = orc.bank_rows(d_orc, recv, bo["bank_offsets"], bo["bank_src"], bo["bfill"])
    used = bo["bank_src"] >= 0
    assert np.array_equal(gc.host(rcv.bank)[used], bank_o[used])


# ----------------------------------------------------------------------------
# expert FFN
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
def test_expert_ffn(moe, orc, share, name):
    cfg = CASES[name]
    rank = 1
    d_orc, d = _dims(orc, share, cfg)
    senders = gc.oracle_sender_all(orc, cfg, d_orc)
    hdr, offs = gc.recv_headers(cfg, d_orc, senders, rank)
    n = len(hdr)
    bo = orc.bank_slots(d_orc, rank, hdr, offs)
    nb = len(bo["bank_src"])
    bank = u16(gen.payload_rows(nb, d.latent, 11))
    wg, wu, wd = gen.rank_experts(cfg, rank)
    rcv = share.Receiver(d, n)
    rcv.bank.copy_(gc.dev(bank))
    rcv.bank_src.copy_(torch.from_numpy(bo["bank_src"]))
    rcv.bfill.copy_(torch.from_numpy(bo["bfill"]))
    if d.cap_send == 0:
        rcv.bank_offsets.copy_(torch.from_numpy(bo["bank_offsets"]))
    rcv.ret.fill_(1.5)                               # poison: non-kept rows must become zero
    rcv.ffn(wg.cuda(), wu.cuda(), wd.cuda())
    torch.cuda.synchronize()
    n_ret = n * (4 if d.dedup else 1)
    ro = orc.expert_ffn(d_orc, bank, bo["bank_offsets"], bo["bank_src"], bo["bfill"],
                        u16(wg), u16(wu), u16(wd), n_ret)
    rg = gc.host(rcv.ret)
    kept = np.zeros(n_ret, bool)
    kept[bo["bank_src"][bo["bank_src"] >= 0]] = True
    assert (rg[~kept] == 0).all()
    gc.assert_rows_close(rg[kept], ro[kept], "ret")


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CASES))
def test_combine(moe, orc, share, name):
    cfg = CASES[name]
    d_orc, d = _dims(orc, share, cfg)
    senders = gc.oracle_sender_all(orc, cfg, d_orc)
    hdr, offs = gc.recv_headers(cfg, d_orc, senders, 0)
    n = len(hdr) * (4 if d.dedup else 1)                # return rows
    s0 = senders[0]
    returned = u16(gen.payload_rows(n, d.latent, 13))
    x = s0["x"]
    wlu = gen.latent_up(cfg)
    wsg, wsu, wsd = gen.shared(cfg)
    snd = share.Sender(d)
    snd.topk.copy_(torch.from_numpy(s0["topk"]))
    snd.slot.copy_(torch.from_numpy(s0["slot"]))
    snd.gates.copy_(torch.from_numpy(s0["gates"]))
    cmb = share.Combiner(d)
    cmb.combine(gc.dev(returned), None if offs is None else gc.dev(offs), snd, x.cuda(),
                wlu.cuda(), wsg.cuda(), wsu.cuda(), wsd.cuda())
    torch.cuda.synchronize()
    yo, oo = orc.combine(d_orc, returned, offs, s0["topk"], s0["slot"], s0["gates"], u16(x),
                         u16(wlu), u16(wsg), u16(wsu), u16(wsd))
    gc.assert_rows_close(gc.host(cmb.ylat), yo, "ylat")
    gc.assert_rows_close(gc.host(cmb.out), oo, "out")


@pytest.mark.parametrize("name", ["tiny", "mid_ragged"])
def test_combine_split_equals_combine(moe, share, name):
    """moe_shared_swiglu + moe_combine_shared give moe_combine's outputs bit
    for bit (same kernels, the shared intermediate in a caller buffer)."""
    cfg = CASES[name]
    d = share.make_dims(cfg)
    R, W = cfg.n_ranks, cfg.n_waves
    n = R * W * d.cap_send if d.cap_send else 3 * R * W
    returned = gen.payload_rows(n, d.latent, 21, "cuda")
    offs = None if d.cap_send else torch.arange(0, n + 1, 3, dtype=torch.int64, device="cuda")
    g = torch.Generator().manual_seed(5)
    snd = share.Sender(d)
    snd.topk.copy_(torch.randint(0, cfg.n_experts, (cfg.T, cfg.top_k), generator=g))
    snd.slot.copy_(torch.randint(-1, 3, (cfg.T, cfg.top_k), generator=g))
    snd.gates.copy_(torch.rand(cfg.T, cfg.top_k, generator=g))
    x = gen.hidden(cfg, 0, "cuda")
    wlu = gen.latent_up(cfg, "cuda")
    wsg, wsu, wsd = gen.shared(cfg, "cuda")
    a = share.Combiner(d)
    a.combine(returned, offs, snd, x, wlu, wsg, wsu, wsd)
    b = share.Combiner(d)
    b.shared(x, wsg, wsu)
    b.combine_shared(returned, offs, snd, wlu, wsd)
    torch.cuda.synchronize()
    assert torch.equal(a.ylat.view(torch.int16), b.ylat.view(torch.int16))
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))



@pytest.mark.parametrize("name", ["mid", "mid_ragged", "mid_w5"])
def test_planned_cus_bit_identical(moe, orc, share, monkeypatch, name):
    """The GEMM launchers planning for 8 or 24 CUs (MOE_GEMM_CUS) instead of
    the device's: one or three persistent blocks per XCD, the expert GEMMs'
    later tiles drawn from the work queue.  No last round is split at these
    sizes (K < 1024), so the pack, expert FFN and combine outputs equal the
    device-count run's bit for bit."""
    cfg, rank = CASES[name], 1
    d_orc, d = _dims(orc, share, cfg)
    senders = gc.oracle_sender_all(orc, cfg, d_orc)
    hdr, offs = gc.recv_headers(cfg, d_orc, senders, rank)
    n = len(hdr)
    bo = orc.bank_slots(d_orc, rank, hdr, offs)
    bank = gen.payload_rows(len(bo["bank_src"]), d.latent, 11, "cuda")
    wg, wu, wd = (w.cuda() for w in gen.rank_experts(cfg, rank))
    wr = gen.router_weight(cfg)
    x = gen.hidden(cfg, 0)
    logits = gen.logits(cfg, 0, x, wr).cuda()
    x = x.cuda()
    wld, wlu = gen.latent_down(cfg).cuda(), gen.latent_up(cfg).cuda()
    wsg, wsu, wsd = (w.cuda() for w in gen.shared(cfg))
    returned = gen.payload_rows(n, d.latent, 13, "cuda")
    r_offs = None if offs is None else gc.dev(offs)

    def run():
        snd = share.Sender(d)
        snd.route(logits)
        snd.pack(x, wld)
        rcv = share.Receiver(d, n)
        rcv.bank.copy_(bank)
        rcv.bank_src.copy_(torch.from_numpy(bo["bank_src"]))
        rcv.bfill.copy_(torch.from_numpy(bo["bfill"]))
        if d.cap_send == 0:
            rcv.bank_offsets.copy_(torch.from_numpy(bo["bank_offsets"]))
        rcv.ffn(wg, wu, wd)
        cmb = share.Combiner(d)
        cmb.combine(returned, r_offs, snd, x, wlu, wsg, wsu, wsd)
        torch.cuda.synchronize()
        # pool slots past the segments (ragged) and payloads of empty slots
        # are unspecified: the tails of every slot, the payloads of kept rows
        L = d.latent
        total = snd.pools.shape[0] if d.cap_send else int(snd.pool_offsets[-1])
        tails = snd.pools[:total, 2 * L:]
        ids = tails[:, :4].contiguous().view(torch.int32).reshape(-1)
        return {"z": snd.z.clone(), "pool_tails": tails.clone(),
                "pool_rows": snd.pools[:total][ids >= 0, :2 * L].clone(), "ret": rcv.ret.clone(),
                "ylat": cmb.ylat.clone(), "out": cmb.out.clone()}

    ref = run()
    for cus in ("8", "24"):
        monkeypatch.setenv("MOE_GEMM_CUS", cus)
        now = run()
        bad = [k for k in ref if not torch.equal(ref[k].contiguous().view(torch.uint8),
                                                  now[k].contiguous().view(torch.uint8))]
        assert not bad, f"planned for {cus} CUs: {bad} differ"


# ----------------------------------------------------------------------------
# K-split last rounds at a size where every row is checked
# ----------------------------------------------------------------------------

# K = 2048 and 3072 with few block tiles: the expert SwiGLU, the expert down
# GEMM and the up-projection all cut their (only) round along K
SPLIT = configs.scaled(gc.MID, "moe_split_T256_D2048_L2048_E48_R8", T=256, d_model=2048,
                       latent=2048, d_ff=1024, d_ff_shared=512)


def test_split_rounds_every_row(moe, orc, share):
    """Expert FFN and combine on a shape whose GEMMs split their last round
    along K; every row against oracle/dense.py, and the split tiles' tail
    kernels seen running."""
    import fullcheck as fc
    from oracle import dense
    cfg, rank = SPLIT, 1
    d_orc, d = _dims(orc, share, cfg)
    L, F, D, S, Fs, El = cfg.latent, cfg.d_ff, cfg.d_model, cfg.n_shared, cfg.d_ff_shared, \
        cfg.experts_per_rank
    senders = gc.oracle_sender_all(orc, cfg, d_orc)
    hdr, offs = gc.recv_headers(cfg, d_orc, senders, rank)
    n = len(hdr)
    bo = orc.bank_slots(d_orc, rank, hdr, offs)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    groups = fc.product_groups(d_orc, bo["bfill"], None, max(L, F), len(bo["bank_src"]))
    S_sw, sw = fc.grouped_split_tiles(groups, F // 128, L, ncu)
    S_dn, dn = fc.grouped_split_tiles(groups, L // 256, F, ncu)
    S_up, up = fc.dense_split_mtiles(cfg.T, D, L + S * Fs, ncu)
    assert S_sw > 1 and S_dn > 1 and S_up > 1, (S_sw, S_dn, S_up)
    # expert FFN on generator bank rows
    bank = u16(gen.payload_rows(len(bo["bank_src"]), L, 31))
    wg, wu, wd = gen.rank_experts(cfg, rank)
    rcv = share.Receiver(d, n)
    rcv.bank.copy_(gc.dev(bank))
    rcv.bank_src.copy_(torch.from_numpy(bo["bank_src"]))
    rcv.bfill.copy_(torch.from_numpy(bo["bfill"]))
    rcv.ret.fill_(1.5)
    moe.moe_profile_reset()
    moe.moe_profile_enable(True)
    rcv.ffn(wg.cuda(), wu.cuda(), wd.cuda())
    # combine of shard 0 over generator returned rows
    s0 = senders[0]
    returned = u16(gen.payload_rows(n, L, 33))
    wlu = gen.latent_up(cfg)
    wsg, wsu, wsd = gen.shared(cfg)
    snd = share.Sender(d)
    snd.topk.copy_(torch.from_numpy(s0["topk"]))
    snd.slot.copy_(torch.from_numpy(s0["slot"]))
    snd.gates.copy_(torch.from_numpy(s0["gates"]))
    cmb = share.Combiner(d)
    cmb.combine(gc.dev(returned), None, snd, s0["x"].cuda(), wlu.cuda(), wsg.cuda(), wsu.cuda(),
                wsd.cuda())
    moe.moe_profile_collect()
    moe.moe_profile_enable(False)
    prof = moe.moe_profile_read()
    torch.cuda.synchronize()
    assert "gemm_up_shared_tail" in prof
    ro = dense.expert_ffn(d_orc, bank, None, bo["bank_src"], bo["bfill"], u16(wg), u16(wu),
                          u16(wd), n)
    rg = gc.host(rcv.ret)
    kept = np.zeros(n, bool)
    kept[bo["bank_src"][bo["bank_src"] >= 0]] = True
    assert (rg[~kept] == 0).all()
    gc.assert_rows_close(rg[kept], ro[kept], "ret")
    yo, oo = dense.combine_tokens(d_orc, returned, None, s0["topk"], s0["slot"], s0["gates"],
                                  u16(s0["x"]), u16(wlu), u16(wsg), u16(wsu), u16(wsd))
    gc.assert_rows_close(gc.host(cmb.ylat), yo, "ylat")
    gc.assert_rows_close(gc.host(cmb.out), oo, "out")
    print(f"\n[split] expert SwiGLU {len(sw)} split M tiles x{S_sw}, down {len(dn)} x{S_dn}, "
          f"up-projection {len(up)} x{S_up}: every row matches", flush=True)
