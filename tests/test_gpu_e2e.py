"""Whole layer on the GPU: every rank of the tiny workload (T=64 tokens per
shard, 48 experts on 8 ranks) through the C ABI, with the exact return
exchange, against the oracle's 8-rank simulation and the per-token brute
force of test_oracle_e2e.

Each of the 8 source shards is routed and packed on the GPU; each rank banks
the rows every shard sent it (forward exchange: device copies of pool
segments) and runs its own six experts; each shard's combine then reads, for
destination d and wave w, the rows rank d computed for it (return exchange:
device copies of return-buffer segments) -- so every token's routed output
is the real one, not the single-GPU identity stand-in.  Integer decisions of
every shard and rank must equal the oracle's bit for bit; ylat and out of
every token of every shard match the oracle within 2e-2 * max|ref| per row
and the brute force likewise.
"""
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest
import torch

import gpucase as gc
from synth import configs, gen
from test_oracle_e2e import bits_of, brute_force, simulate

pytestmark = pytest.mark.gpu

VARIANTS = {
    "cf1.10_1.15": {},
    "tight": dict(cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2)),
    "ragged": dict(cf_send=None, cf_recv=None),
    "chunks_tight": dict(waves="chunks", cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2)),
    "dedup_tight": dict(dedup=True, cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2)),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_e2e_all_ranks_exact_return(orc, name):
    from dispatch_softmax_top_amd import share
    cfg = replace(configs.TINY, name=configs.TINY.name + "_" + name, **VARIANTS[name])
    print(f"\n[e2e] {cfg.name}: 8 ranks on the GPU", flush=True)
    d = share.make_dims(cfg)
    R, W, El = cfg.n_ranks, cfg.n_waves, cfg.experts_per_rank
    per = 4 if d.dedup else 1
    # the same generator tensors as the oracle's simulation (made on the host)
    wr = gen.router_weight(cfg)
    wld, wlu = gen.latent_down(cfg).cuda(), gen.latent_up(cfg).cuda()
    wsg, wsu, wsd = (w.cuda() for w in gen.shared(cfg))

    # senders: every shard routed and packed
    snd, xs = [], []
    for s in range(R):
        x = gen.hidden(cfg, s)
        lg = gen.logits(cfg, s, x, wr).cuda()
        sd = share.Sender(d)
        sd.route(lg)
        sd.pack(x.cuda(), wld)
        snd.append(sd)
        xs.append(x.cuda())

    # receivers: forward exchange, bank, each rank's own experts
    rcv, roffs = [], []
    for r in range(R):
        if d.cap_send:
            recv = share.loopback_recv_fixed(d, [sd.pools for sd in snd], r)
            ro = None
        else:
            recv, ro = share.loopback_recv_ragged(d, [sd.pools for sd in snd],
                                                  [sd.pool_offsets for sd in snd], r)
        rc = share.Receiver(d, recv.shape[0])
        rc.bank_rows(r, recv, ro)
        wg, wu, wd = (w.cuda() for w in gen.rank_experts(cfg, r))
        rc.ffn(wg, wu, wd)
        rcv.append(rc)
        roffs.append(ro)

    # return exchange: shard s reads, for destination dst and wave w, the
    # rows rank dst computed for source s; then each shard's combine
    cmb = []
    for s in range(R):
        parts = []
        for dst in range(R):
            for w in range(W):
                if d.cap_send:
                    a = (s * W + w) * d.cap_send * per
                    parts.append(rcv[dst].ret[a:a + d.cap_send * per])
                else:
                    o = roffs[dst].cpu().tolist()
                    parts.append(rcv[dst].ret[o[s * W + w]:o[s * W + w + 1]])
        returned = torch.cat(parts).contiguous()
        cb = share.Combiner(d)
        cb.combine(returned, snd[s].pool_offsets, snd[s], xs[s], wlu, wsg, wsu, wsd)
        cmb.append(cb)
    torch.cuda.synchronize()

    # oracle: the same 8-rank simulation with its own stages, and brute force
    d_orc, W_, S, BK, OUT = simulate(orc, cfg)
    ref = brute_force(cfg, d_orc, W_, S)
    n_drop = 0
    for s in range(R):
        assert np.array_equal(gc.host(snd[s].topk), S[s]["topk"]), f"topk of shard {s}"
        assert np.array_equal(gc.host(snd[s].slot), S[s]["slot"]), f"slot of shard {s}"
        assert np.array_equal(gc.host(snd[s].fill), S[s]["fill"])
        assert np.array_equal(gc.host(snd[s].demand), S[s]["demand"])
        n_drop += int((~ref[s][2]).sum())
    for r in range(R):
        assert np.array_equal(gc.host(rcv[r].bank_src), BK[r]["bank_src"]), f"bank of rank {r}"
        assert np.array_equal(gc.host(rcv[r].bfill), BK[r]["bfill"])
        assert np.array_equal(gc.host(rcv[r].bdemand), BK[r]["bdemand"])
    for s in range(R):
        ylat, out = gc.host(cmb[s].ylat), gc.host(cmb[s].out)
        gc.assert_rows_close(ylat, OUT[s][0], f"ylat of shard {s} vs oracle")
        gc.assert_rows_close(out, OUT[s][1], f"out of shard {s} vs oracle")
        gc.assert_rows_close(ylat, bits_of(ref[s][0]), f"ylat of shard {s} vs brute force")
        gc.assert_rows_close(out, bits_of(ref[s][1]), f"out of shard {s} vs brute force")
    if name == "ragged":
        assert n_drop == 0
    if name.endswith("tight"):
        assert n_drop > 0
    print(f"[e2e] {cfg.name}: every token of every shard matches ({n_drop} assignments "
          f"dropped)", flush=True)
