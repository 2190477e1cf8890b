"""Full-size parity of the backward calls, in the launch configuration
bench.py times (the same entry points and sizes: T = 4096 / 16384 / 65536
tokens, model width 6144, latent 3072, 384 experts on 64 ranks).

Stage inputs come from the generators at full size (payload rows, made on
the device and copied to the host for the oracle, stand in
for returned rows, ylat, the bank, the gradients), routing and sender slots
from the oracle on the shard's own logits, the bank decisions from the
oracle on seeded receive headers.  Integer-exact properties are checked in
full (zero rows where nothing was kept, zero gate gradients of dropped
choices, the router's gradient everywhere); floating outputs on sampled
tokens and bank rows that the oracle computes one by one, and on sampled
rows of every weight gradient, each compared whole against the oracle's row
(oracle/dense.py) with the tolerance scaled by that oracle row: 2e-2 *
max|ref| per row, as for every other output.  For dw_down and dws_down the
rows are those of the transposes (one intermediate unit each), which the
oracle computes from one column of the recomputed intermediate.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import gpucase as gc
from conftest import f64, u16
from oracle import dense
from synth import configs, gen

pytestmark = pytest.mark.gpu

CASES = [
    ("share4k", configs.SHARE_4K, dict(tok=6, rows=10, ent=3, experts=3)),
    ("zipf16k", configs.ZIPF_16K, dict(tok=4, rows=6, ent=2, experts=2)),
    ("long65k", configs.LONG_65K, dict(tok=3, rows=4, ent=1, experts=1)),
]


def _group_positions(bfill, cap, j, W, El):
    """Bank positions of local expert j, in (wave, position) order."""
    return np.concatenate([np.arange(g * cap, g * cap + bfill[g]) for g in range(j, W * El, El)])


def _sample_tokens(cfg, slot, n, rng):
    Tw = math.ceil(cfg.T / cfg.n_waves)
    fixed = [0, cfg.T - 1, Tw - 1, Tw, min(cfg.T - 1, 2 * Tw)]
    dropped = np.nonzero((slot < 0).any(1))[0]
    if len(dropped):
        fixed.append(int(dropped[0]))
    return np.unique(np.concatenate([fixed, rng.integers(0, cfg.T, n)]))


@pytest.mark.parametrize("name,cfg,ns", CASES, ids=[c[0] for c in CASES])
def test_full_backward(moe_lib, orc, name, cfg, ns):
    from dispatch_softmax_top_amd import share
    moe = moe_lib
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    T, L, D, S, Fs, k = cfg.T, cfg.latent, cfg.d_model, cfg.n_shared, cfg.d_ff_shared, cfg.top_k
    El, F, R, W = cfg.experts_per_rank, cfg.d_ff, cfg.n_ranks, cfg.n_waves
    n_rows = R * W * d.cap_send
    print(f"\n[full backward] {name}: routing", flush=True)
    x_t, lg_t = gc.shard_inputs(cfg, 0)
    x, lg = u16(x_t), lg_t.numpy()
    topk, gates = orc.route(lg, k)
    so = orc.sender(d_orc, topk)
    slot, fill = so["slot"], so["fill"]
    wlu, wld = u16(gen.latent_up(cfg)), u16(gen.latent_down(cfg))
    wsg, wsu, wsd = (u16(w) for w in gen.shared(cfg))
    dev = lambda a: gc.dev(np.ascontiguousarray(a))
    b = share.Backward(d, n_rows)

    # ---- combine side
    print(f"[full backward] {name}: combine", flush=True)
    returned = gen.payload_rows(n_rows, L, 81, "cuda")
    ylat, d_out = gen.payload_rows(T, L, 82, "cuda"), gen.payload_rows(T, D, 83, "cuda")
    h_returned, h_ylat, h_dout = u16(returned), u16(ylat), u16(d_out)
    moe.moe_combine_backward(d, returned, dev(topk), dev(slot), dev(gates), dev(fill),
                             x_t.cuda(), ylat, dev(wlu), dev(wsg), dev(wsu), dev(wsd), d_out, b.d_returned, b.d_gates, b.d_shared, b.dw_lat_up,
                             b.dws_down, b.ws_combine)
    moe.moe_route_backward(lg_t.cuda(), dev(topk), b.d_gates, b.d_logits)
    torch.cuda.synchronize()
    g_dret, g_dg = gc.host(b.d_returned), gc.host(b.d_gates)
    for p in range(R * W):                                # rows past each pool's fill: zero
        assert (g_dret[p * d.cap_send + fill[p]:(p + 1) * d.cap_send] == 0).all()
    assert (g_dg[slot < 0] == 0).all()
    # the router's gradient in full, from the GPU's gate gradients
    o_dl = orc.route_backward(lg, topk, g_dg)
    scale = np.abs(o_dl).max(1, keepdims=True) + 1e-30
    assert (np.abs(gc.host(b.d_logits) - o_dl) <= 1e-4 * scale).all()
    tok = _sample_tokens(cfg, slot, ns["tok"], rng)
    rows, dg, dsh = orc.combine_backward_tokens(d_orc, h_returned, topk, slot, gates, x, wlu,
                                                wsg, wsu, wsd, h_dout, tok)
    Tw = math.ceil(T / W)
    used = []
    for r, t in enumerate(tok):
        for j in range(k):
            if slot[t, j] < 0:
                continue
            row = ((topk[t, j] // El) * W + t // Tw) * d.cap_send + slot[t, j]
            used.append(row)
            gc.assert_rows_close(g_dret[row][None], rows[r, j][None], f"d_returned t={t}")
    y = f64(h_dout[tok]) @ f64(wlu)
    tol = 2e-3 * np.abs(f64(h_returned[used])).max() * np.abs(y).sum(1, keepdims=True)
    assert (np.abs(g_dg[tok] - dg) <= tol).all()
    gc.assert_rows_close(gc.host(b.d_shared)[tok].reshape(len(tok), -1),
                         dsh.reshape(len(tok), -1), "d_shared")
    g_dwlu = gc.host(b.dw_lat_up)
    ra = np.unique(np.concatenate([[0, D - 1], rng.integers(0, D, ns["ent"] * 3)]))
    gc.assert_rows_close(g_dwlu[ra], dense.outer_rows(f64(h_dout[:, ra]), f64(h_ylat)),
                         "dw_lat_up rows")
    g_dwsd = gc.host(b.dws_down)
    for sh in range(S):
        cf = np.unique(np.concatenate([[0, Fs - 1], rng.integers(0, Fs, ns["ent"])]))
        ref = dense.shared_down_wgrad_cols(x, wsg, wsu, h_dout, sh, cf)
        gc.assert_rows_close(np.ascontiguousarray(g_dwsd[sh][:, cf].T), ref,
                             f"dws_down[{sh}] columns")

    # ---- receiver side (rank 1's experts on seeded receive headers)
    print(f"[full backward] {name}: experts", flush=True)
    rank = 1
    hdr = np.where(rng.random(n_rows) < 0.9, rank * El + rng.integers(0, El, n_rows), -1)
    bo = orc.bank_slots(d_orc, rank, hdr.astype(np.int32), None)
    nb = len(bo["bank_src"])
    bank, d_ret = gen.payload_rows(nb, L, 84, "cuda"), gen.payload_rows(n_rows, L, 85, "cuda")
    h_bank, h_dret = u16(bank), u16(d_ret)
    wg, wu, wdn = gen.rank_experts(cfg, rank)
    moe.moe_expert_ffn_backward(d, bank, dev(bo["bank_src"]), dev(bo["bfill"]), wg.cuda(),
                                wu.cuda(), wdn.cuda(), d_ret, b.d_recv, b.dw_gate,
                                b.dw_up, b.dw_down, b.ws_ffn)
    torch.cuda.synchronize()
    g_drecv = gc.host(b.d_recv)
    kept = np.zeros(n_rows, bool)
    kept[bo["bank_src"][bo["bank_src"] >= 0]] = True
    assert (g_drecv[~kept] == 0).all()
    filled = np.nonzero(bo["bank_src"] >= 0)[0]
    cap = d.cap_recv
    edges = [p for g in range(W * El) for p in (g * cap, g * cap + bo["bfill"][g] - 1)
             if bo["bfill"][g] > 0]
    pos = np.unique(np.concatenate([rng.choice(filled, ns["rows"]), rng.choice(edges, 4)]))
    ex = [u16(w) for w in (wg, wu, wdn)]
    du = orc.expert_ffn_backward_rows(d_orc, h_bank, bo["bank_src"], *ex, h_dret, pos)
    gc.assert_rows_close(g_drecv[bo["bank_src"][pos]], du, "d_recv")
    gw = [gc.host(t) for t in (b.dw_gate, b.dw_up, b.dw_down)]
    for j in rng.choice(El, ns["experts"], replace=False):
        fi = np.unique(np.concatenate([[0, F - 1], rng.integers(0, F, ns["ent"])]))
        pos_j = _group_positions(bo["bfill"], cap, int(j), W, El)
        refs = dense.expert_wgrad_rows(h_bank[pos_j], h_dret[bo["bank_src"][pos_j]],
                                       *(w[j] for w in ex), fi)
        gots = (gw[0][j][fi], gw[1][j][fi], np.ascontiguousarray(gw[2][j][:, fi].T))
        for what, got, ref in zip(("dw_gate", "dw_up", "dw_down^T"), gots, refs):
            gc.assert_rows_close(got, ref, f"{what} rows of expert {j}")

    # ---- sender side
    print(f"[full backward] {name}: pack", flush=True)
    d_pools = gen.payload_rows(n_rows, L, 86, "cuda")
    d_shared = gen.payload_rows(T, 2 * S * Fs, 87, "cuda")
    h_dpools, h_dshared = u16(d_pools), u16(d_shared)
    moe.moe_pack_backward(d, d_pools, dev(topk), dev(slot), x_t.cuda(), d_shared,
                          dev(wld), dev(wsg), dev(wsu), b.dz, b.dx, b.dw_lat_down, b.dws_gate,
                          b.dws_up, b.ws_pack)
    torch.cuda.synchronize()
    dz, dx = orc.pack_backward_tokens(d_orc, h_dpools, topk, slot, h_dshared, wld, wsg,
                                      wsu, tok)
    gz = gc.host(b.dz)
    none = (slot < 0).all(1)
    assert (gz[none] == 0).all()
    keep = ~none[tok]
    gc.assert_rows_close(gz[tok][keep], dz[keep], "dz")
    gc.assert_rows_close(gc.host(b.dx)[tok], dx, "dx")
    g_dwld = gc.host(b.dw_lat_down)
    dz_all = dense.pack_dz(d_orc, h_dpools, topk, slot)
    assert np.array_equal(dz_all[tok], dz)
    ra = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, ns["ent"] * 3)]))
    gc.assert_rows_close(g_dwld[ra], dense.outer_rows(f64(dz_all[:, ra]), f64(x)),
                         "dw_lat_down rows")
    dsh4 = h_dshared.reshape(T, 2, S, Fs)
    for which, got in ((0, b.dws_gate), (1, b.dws_up)):
        gw = gc.host(got)
        for sh in range(S):
            ra = np.unique(np.concatenate([[0, Fs - 1], rng.integers(0, Fs, ns["ent"])]))
            gc.assert_rows_close(gw[sh][ra], dense.outer_rows(f64(dsh4[:, which, sh, ra]), f64(x)),
                                 f"shared weight {which} rows of expert {sh}")


@pytest.fixture(scope="module")
def moe_lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dispatch_softmax_top_amd as m
    m.lib()
    return m


def test_full_expert_backward_skewed(moe_lib, orc):
    """The hottest Zipf rank's pattern at full size (16384 tokens): two of the
    six local experts saturated in every wave, four with no rows, so the
    weight-gradient launch mixes products of 786 K tiles with products of the
    minimum K.  Sampled receive rows and weight entries against the oracle;
    the empty experts' weight gradients exactly zero."""
    from dispatch_softmax_top_amd import share
    moe = moe_lib
    cfg = configs.ZIPF_16K
    rng = np.random.default_rng(zlib.crc32(b"skewed experts"))
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    L, El, R, W = cfg.latent, cfg.experts_per_rank, cfg.n_ranks, cfg.n_waves
    n_rows = R * W * d.cap_send
    rank, hot = 35, np.array([2, 5])
    print("\n[full backward] skewed experts: bank slots", flush=True)
    hdr = np.where(rng.random(n_rows) < 0.9, rank * El + rng.choice(hot, n_rows), -1)
    bo = orc.bank_slots(d_orc, rank, hdr.astype(np.int32), None)
    fills = bo["bfill"].reshape(W, El)
    assert (fills[:, hot] == d.cap_recv).all() and fills.sum() == W * len(hot) * d.cap_recv
    nb = len(bo["bank_src"])
    b = share.Backward(d, n_rows)
    bank, d_ret = gen.payload_rows(nb, L, 94, "cuda"), gen.payload_rows(n_rows, L, 95, "cuda")
    h_bank, h_dret = u16(bank), u16(d_ret)
    wg, wu, wdn = gen.rank_experts(cfg, rank)
    dev = lambda a: gc.dev(np.ascontiguousarray(a))
    print("[full backward] skewed experts: GPU", flush=True)
    moe.moe_expert_ffn_backward(d, bank, dev(bo["bank_src"]), dev(bo["bfill"]), wg.cuda(),
                                wu.cuda(), wdn.cuda(), d_ret, b.d_recv, b.dw_gate,
                                b.dw_up, b.dw_down, b.ws_ffn)
    torch.cuda.synchronize()
    g_drecv = gc.host(b.d_recv)
    kept = np.zeros(n_rows, bool)
    kept[bo["bank_src"][bo["bank_src"] >= 0]] = True
    assert (g_drecv[~kept] == 0).all()
    print("[full backward] skewed experts: oracle rows", flush=True)
    filled = np.nonzero(bo["bank_src"] >= 0)[0]
    cap = d.cap_recv
    edges = [g * cap + p for g in range(W * El) if bo["bfill"][g] > 0 for p in (0, bo["bfill"][g] - 1)]
    pos = np.unique(np.concatenate([rng.choice(filled, 6), rng.choice(edges, 4)]))
    ex = [u16(w) for w in (wg, wu, wdn)]
    du = orc.expert_ffn_backward_rows(d_orc, h_bank, bo["bank_src"], *ex, h_dret, pos)
    gc.assert_rows_close(g_drecv[bo["bank_src"][pos]], du, "d_recv")
    cold = np.setdiff1d(np.arange(El), hot)
    gw = [gc.host(t) for t in (b.dw_gate, b.dw_up, b.dw_down)]
    for which in range(3):
        assert (gw[which][cold] == 0).all(), f"weight {which}: an expert without rows has a gradient"
    print("[full backward] skewed experts: oracle weight rows", flush=True)
    F = cfg.d_ff
    for j in hot:
        fi = np.unique(np.concatenate([[0, F - 1], rng.integers(0, F, 2)]))
        pos_j = _group_positions(bo["bfill"], cap, int(j), W, El)
        refs = dense.expert_wgrad_rows(h_bank[pos_j], h_dret[bo["bank_src"][pos_j]],
                                       *(w[j] for w in ex), fi)
        gots = (gw[0][j][fi], gw[1][j][fi], np.ascontiguousarray(gw[2][j][:, fi].T))
        for what, got, ref in zip(("dw_gate", "dw_up", "dw_down^T"), gots, refs):
            gc.assert_rows_close(got, ref, f"{what} rows of expert {j}")


def _threaded(fn, tokens, parts=16):
    """fn(tokens chunk) -> tuple of arrays, run on chunks in threads (the C
    oracle releases the interpreter lock), results concatenated."""
    from concurrent.futures import ThreadPoolExecutor
    chunks = [c for c in np.array_split(np.asarray(tokens), parts) if len(c)]
    with ThreadPoolExecutor(len(chunks)) as ex:
        res = list(ex.map(fn, chunks))
    return tuple(np.concatenate([r[i] for r in res]) for i in range(len(res[0])))


def test_full_backward_ragged_hot(moe_lib, orc):
    """Dropless (ragged) backward at full size: the 16384-token Zipf
    workload's most-loaded rank, with the receive layout the oracle's routing
    of all 64 shards gives it, a few experts taking most of its rows.  The
    expert backward runs over that receive layout (segments per source shard
    and wave); the combine and pack backwards over the rank's own shard as a
    sender (segments per destination and wave, at its pool offsets).  Stage
    inputs are generator rows in those layouts.  Zero rows and zero gate
    gradients in full; sampled tokens and bank rows against the oracle; whole
    rows of every weight gradient against oracle/dense.py."""
    import fullcheck as fc
    from dispatch_softmax_top_amd import share
    moe = moe_lib
    cfg = configs.SWEEP_16K["inf"]
    rng = np.random.default_rng(zlib.crc32(b"ragged backward"))
    d_orc, d = orc.dims(cfg), share.make_dims(cfg)
    T, L, D, S, Fs, k = cfg.T, cfg.latent, cfg.d_model, cfg.n_shared, cfg.d_ff_shared, cfg.top_k
    El, F, W = cfg.experts_per_rank, cfg.d_ff, cfg.n_waves
    print("\n[full backward] ragged hot rank: routing of every shard", flush=True)
    wr = gen.router_weight(cfg, "cuda")
    logits = [gen.logits(cfg, s, gen.hidden(cfg, s, "cuda"), wr).cpu().numpy()
              for s in range(cfg.n_shards)]
    shards = fc.oracle_shards(orc, cfg, d_orc, logits)
    rank = fc.hot_rank(cfg, d_orc, shards)
    rm = fc.RecvMap(cfg, d_orc, shards, rank)
    own, lg = shards[rank], logits[rank]
    del logits
    topk, slot, gates, fill = own["topk"], own["slot"], own["gates"], own["fill"]
    po, n_s, n = own["pool_offsets"], int(own["pool_offsets"][-1]), rm.n
    x_t = gen.hidden(cfg, rank, "cuda")
    x = u16(x_t)
    wlu, wld = u16(gen.latent_up(cfg)), u16(gen.latent_down(cfg))
    wsg, wsu, wsd = (u16(w) for w in gen.shared(cfg))
    dev = lambda a: gc.dev(np.ascontiguousarray(a))
    ws = lambda call, rows=0: torch.empty(max(moe.moe_workspace_bytes(d, call, rows), 16),
                                          dtype=torch.uint8, device="cuda")
    Tw = math.ceil(T / W)
    tok = np.unique(np.concatenate([[0, T - 1], [w * Tw - 1 for w in range(1, W)],
                                    [w * Tw for w in range(1, W)], rng.integers(0, T, 96)]))
    print(f"[full backward] ragged: rank {rank}, {n} receive rows, {n_s} sent rows, combine",
          flush=True)

    # ---- combine side
    returned = gen.payload_rows(n_s, L, 91, "cuda")
    ylat, d_out = gen.payload_rows(T, L, 92, "cuda"), gen.payload_rows(T, D, 93, "cuda")
    d_ret = torch.full((n_s, L), 3.0, dtype=torch.bfloat16, device="cuda")
    d_g = torch.full((T, k), 5.0, device="cuda")
    d_sh = torch.empty((T, 2, S, Fs), dtype=torch.bfloat16, device="cuda")
    dwlu = torch.empty((D, L), dtype=torch.bfloat16, device="cuda")
    dwsd = torch.empty((S, D, Fs), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_backward(d, returned, dev(topk), dev(slot), dev(gates), dev(fill), x_t, ylat,
                             dev(wlu), dev(wsg), dev(wsu), dev(wsd), d_out, d_ret, d_g, d_sh,
                             dwlu, dwsd, ws(moe.MOE_CALL_COMBINE_BWD), ret_offsets=dev(po))
    torch.cuda.synchronize()
    h_ret, h_ylat, h_dout = u16(returned), u16(ylat), u16(d_out)
    del returned
    rows_all = dense.returned_rows(d_orc, po, topk, slot, np.arange(T))
    written = torch.zeros(n_s, dtype=torch.bool, device="cuda")
    w_rows = rows_all[rows_all >= 0]
    written[torch.from_numpy(w_rows).cuda()] = True
    assert bool((d_ret[~written].view(torch.int16) == 0).all()), "unwritten d_returned rows"
    g_dg = gc.host(d_g)
    assert (g_dg[rows_all < 0] == 0).all()
    o_rows, o_dg, o_dsh = _threaded(
        lambda c: orc.combine_backward_tokens(d_orc, h_ret, topk, slot, gates, x, wlu, wsg, wsu,
                                              wsd, h_dout, c, ret_offsets=po), tok)
    g_dret = gc.host(d_ret[torch.from_numpy(np.maximum(rows_all[tok], 0)).cuda().reshape(-1)])
    g_dret = g_dret.reshape(len(tok), k, L)
    live = rows_all[tok] >= 0
    gc.assert_rows_close(g_dret[live], o_rows[live], "d_returned (sampled tokens)")
    y = f64(h_dout[tok]) @ f64(wlu)
    tol = 2e-3 * np.abs(f64(h_ret[w_rows])).max() * np.abs(y).sum(1, keepdims=True)
    assert (np.abs(g_dg[tok] - o_dg) <= tol).all()
    gc.assert_rows_close(gc.host(d_sh)[tok].reshape(len(tok), -1), o_dsh.reshape(len(tok), -1),
                         "d_shared")
    ra = np.unique(np.concatenate([[0, D - 1], rng.integers(0, D, 6)]))
    gc.assert_rows_close(gc.host(dwlu)[ra], dense.outer_rows(f64(h_dout[:, ra]), f64(h_ylat)),
                         "dw_lat_up rows")
    g_dwsd = gc.host(dwsd)
    for sh in range(S):
        cf = np.unique(np.concatenate([[0, Fs - 1], rng.integers(0, Fs, 3)]))
        gc.assert_rows_close(np.ascontiguousarray(g_dwsd[sh][:, cf].T),
                             dense.shared_down_wgrad_cols(x, wsg, wsu, h_dout, sh, cf),
                             f"dws_down[{sh}] columns")
    del d_ret, h_ret
    torch.cuda.empty_cache()

    # ---- receiver side
    print("[full backward] ragged: experts", flush=True)
    bo = orc.bank_slots(d_orc, rank, rm.hdr, rm.starts)
    nb = len(bo["bank_src"])
    assert nb == n and int(bo["bfill"].sum()) == int((rm.hdr >= 0).sum())
    bank, dret = gen.payload_rows(nb, L, 94, "cuda"), gen.payload_rows(n, L, 95, "cuda")
    wg, wu, wdn = gen.rank_experts(cfg, rank)
    d_recv = torch.full((n, L), 2.0, dtype=torch.bfloat16, device="cuda")
    dwg = torch.empty((El, F, L), dtype=torch.bfloat16, device="cuda")
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((El, L, F), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn_backward(d, bank, dev(bo["bank_src"]), dev(bo["bfill"]), wg.cuda(),
                                wu.cuda(), wdn.cuda(), dret, d_recv, dwg, dwu, dwd,
                                ws(moe.MOE_CALL_FFN_BWD, nb),
                                bank_offsets=dev(bo["bank_offsets"]))
    torch.cuda.synchronize()
    kept = torch.zeros(n, dtype=torch.bool, device="cuda")
    kept[torch.from_numpy(bo["bank_src"][bo["bank_src"] >= 0]).cuda().long()] = True
    assert bool((d_recv[~kept].view(torch.int16) == 0).all())
    h_bank, h_dret = u16(bank), u16(dret)
    del bank, dret
    boff, bfill = bo["bank_offsets"], bo["bfill"]
    edges = [int(boff[g]) + p for g in range(W * El) if bfill[g] > 0
             for p in (0, int(bfill[g]) - 1)]
    pos = np.unique(np.concatenate([edges, rng.choice(np.nonzero(bo["bank_src"] >= 0)[0], 48)]))
    ex = [u16(w) for w in (wg, wu, wdn)]
    (du,) = _threaded(lambda c: (orc.expert_ffn_backward_rows(d_orc, h_bank, bo["bank_src"], *ex,
                                                             h_dret, c, bank_offsets=boff),), pos)
    gc.assert_rows_close(gc.host(d_recv[torch.from_numpy(bo["bank_src"][pos]).cuda().long()]),
                         du, "d_recv (sampled bank rows)")
    gw = [gc.host(t) for t in (dwg, dwu, dwd)]
    rows_j = [int(bfill[j::El].sum()) for j in range(El)]
    for j in range(El):
        if rows_j[j] == 0:
            assert all((g_[j] == 0).all() for g_ in gw), f"expert {j} has no rows"
            continue
        fi = np.unique(np.concatenate([[0, F - 1], rng.integers(0, F, 2)]))
        pos_j = np.concatenate([np.arange(int(boff[g]), int(boff[g]) + int(bfill[g]))
                                for g in range(j, W * El, El)])
        refs = dense.expert_wgrad_rows(h_bank[pos_j], h_dret[bo["bank_src"][pos_j]],
                                       *(w[j] for w in ex), fi)
        gots = (gw[0][j][fi], gw[1][j][fi], np.ascontiguousarray(gw[2][j][:, fi].T))
        for what, got, ref in zip(("dw_gate", "dw_up", "dw_down^T"), gots, refs):
            gc.assert_rows_close(got, ref, f"{what} rows of expert {j} ({rows_j[j]} rows)")
    del d_recv, h_bank
    torch.cuda.empty_cache()

    # ---- sender side (pool-row gradients in the receive layout)
    print("[full backward] ragged: pack", flush=True)
    d_pools = gen.payload_rows(n_s, L, 96, "cuda")
    d_shared = gen.payload_rows(T, 2 * S * Fs, 97, "cuda")
    b = share.Backward(d, 1)
    moe.moe_pack_backward(d, d_pools, dev(topk), dev(slot), x_t, d_shared, dev(wld), dev(wsg),
                          dev(wsu), b.dz, b.dx, b.dw_lat_down, b.dws_gate, b.dws_up,
                          ws(moe.MOE_CALL_PACK_BWD), pool_offsets=dev(po))
    torch.cuda.synchronize()
    h_dp, h_dsh = u16(d_pools), u16(d_shared)
    dz_all = dense.pack_dz(d_orc, h_dp, topk, slot, pool_offsets=po)
    gz = gc.host(b.dz)
    nz = np.abs(f64(dz_all)).any(1)
    assert (gz[~nz] == 0).all()
    gc.assert_rows_close(gz[nz], dz_all[nz], "dz (every token)")
    o_dz, o_dx = _threaded(lambda c: orc.pack_backward_tokens(d_orc, h_dp, topk, slot, h_dsh, wld,
                                                              wsg, wsu, c, pool_offsets=po), tok)
    assert np.array_equal(o_dz, dz_all[tok])
    gc.assert_rows_close(gc.host(b.dx)[tok], o_dx, "dx (sampled tokens)")
    ra = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, 6)]))
    gc.assert_rows_close(gc.host(b.dw_lat_down)[ra], dense.outer_rows(f64(dz_all[:, ra]), f64(x)),
                         "dw_lat_down rows")
    dsh4 = h_dsh.reshape(T, 2, S, Fs)
    for which, got in ((0, b.dws_gate), (1, b.dws_up)):
        g_ = gc.host(got)
        for sh in range(S):
            r2 = np.unique(np.concatenate([[0, Fs - 1], rng.integers(0, Fs, 3)]))
            gc.assert_rows_close(g_[sh][r2], dense.outer_rows(f64(dsh4[:, which, sh, r2]), f64(x)),
                                 f"shared weight {which} rows of expert {sh}")
    print(f"[full backward] ragged hot rank {rank}: every check passes", flush=True)
