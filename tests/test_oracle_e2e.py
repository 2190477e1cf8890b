"""Whole-layer pin: 8-rank simulation from oracle stages vs per-token brute force.

All ranks of the tiny workload (T=64, d_model=256, latent=128, 48 experts on
8 ranks) are simulated with the oracle's stage functions and an exact return
exchange.  Independently, numpy computes each token's output straight from
the definition -- no pools, banks or slots: an assignment survives if its
position in its sender pool and in its receiver expert queue are both within
capacity, and a token's output is the gate-weighted sum of its surviving
experts' SwiGLU outputs, projected up, plus the two shared experts.
With infinite capacity (ragged mode) this is a textbook dense-dispatch top-k
MoE layer.
"""
import math

import numpy as np
import pytest
import torch

from conftest import f64, u16, ulp_diff
from synth import configs, gen


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), float64 result; written apart
    from the oracle's conversion."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(np.abs(v))                 # |v| = m 2^e, m in [0.5, 1)
    q = np.where(e - 1 >= -126, e - 8, -133)
    r = np.rint(np.ldexp(np.abs(v), -q))       # numpy rint: ties to even
    return np.copysign(np.ldexp(r, q), v)


def bits_of(v: np.ndarray) -> np.ndarray:
    return u16(torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16))


def silu(a):
    return a / (1.0 + np.exp(-a))


def simulate(orc, cfg):
    d = orc.dims(cfg)
    R, W, El, k, L = cfg.n_ranks, cfg.n_waves, cfg.experts_per_rank, cfg.top_k, cfg.latent
    wr = gen.router_weight(cfg)
    xs = [gen.hidden(cfg, s) for s in range(R)]
    lgs = [gen.logits(cfg, s, xs[s], wr).numpy() for s in range(R)]
    wld = u16(gen.latent_down(cfg))
    wlu = u16(gen.latent_up(cfg))
    wsg, wsu, wsd = (u16(w) for w in gen.shared(cfg))
    ex = [tuple(u16(w) for w in gen.rank_experts(cfg, r)) for r in range(R)]
    x = [u16(v) for v in xs]

    # sender side, every shard
    S = []
    for s in range(R):
        topk, gates = orc.route(lgs[s], k)
        z = orc.latent(x[s], wld)
        snd = orc.sender(d, topk)
        pools = orc.pack_rows(d, z, topk, snd["slot"], snd["pool_offsets"])
        S.append(dict(topk=topk, gates=gates, z=z, pools=pools, **snd))

    def seg(s, dst, w):      # rows of shard s's pool (dst, w)
        if d.cap_send:
            a = (dst * W + w) * d.cap_send
            return a, a + d.cap_send
        o = S[s]["pool_offsets"]
        return int(o[dst * W + w]), int(o[dst * W + w + 1])

    # receiver side, every rank
    RET, RO, BK = [], [], []
    for r in range(R):
        parts, lens = [], []
        for s in range(R):
            for w in range(W):
                a, b = seg(s, r, w)
                parts.append(S[s]["pools"][a:b])
                lens.append(b - a)
        recv = np.concatenate(parts)
        ro = None if d.cap_send else np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        bs = orc.bank_slots(d, r, orc.recv_ids(d, recv), ro)
        assert bs["bad_rows"] == 0
        bank = orc.bank_rows(d, recv, bs["bank_offsets"], bs["bank_src"], bs["bfill"])
        ret = orc.expert_ffn(d, bank, bs["bank_offsets"], bs["bank_src"], bs["bfill"],
                             *ex[r], len(recv) * (4 if d.dedup else 1))
        RET.append(ret); RO.append(ro); BK.append(dict(bs, bank=bank))

    # exact return and combine (with dedup, four return slots per row)
    OUT = []
    per = 4 if d.dedup else 1
    for s in range(R):
        parts = []
        for dst in range(R):
            for w in range(W):
                if d.cap_send:
                    a = (s * W + w) * d.cap_send * per
                    parts.append(RET[dst][a:a + d.cap_send * per])
                else:
                    parts.append(RET[dst][RO[dst][s * W + w]:RO[dst][s * W + w + 1]])
        returned = np.concatenate(parts)
        ylat, out = orc.combine(d, returned, S[s]["pool_offsets"], S[s]["topk"],
                                S[s]["slot"], S[s]["gates"], x[s], wlu, wsg, wsu, wsd)
        S[s]["returned"] = returned
        OUT.append((ylat, out))
    return d, dict(x=x, wld=wld, wlu=wlu, wsg=wsg, wsu=wsu, wsd=wsd, ex=ex, logits=lgs), S, BK, OUT


def brute_force(cfg, d, W_, S):
    """Per-token definition, from routing decisions (topk, gates) only."""
    R, Wv, El, k, L = cfg.n_ranks, cfg.n_waves, cfg.experts_per_rank, cfg.top_k, cfg.latent
    T = cfg.T
    Tw = math.ceil(T / Wv)
    Cs = d.cap_send or 10 ** 9
    Cr = d.cap_recv or 10 ** 9
    chunks = cfg.waves == "chunks"
    # sender position: rank of (t, j) among same (dest, wave) items in (t, j) order;
    # with chunked waves among same-dest items (one pool of Wv * Cs rows per dest)
    send_pos = []
    for s in range(R):
        topk = S[s]["topk"]
        key = topk // El if chunks else (topk // El) * Wv + (np.arange(T) // Tw)[:, None]
        if cfg.dedup:   # rows: groups of up to 4 same-destination choices of a token
            pos = np.zeros((T, k), int)
            nxt = {}
            for t in range(T):
                lead = {}
                for j in range(k):
                    dst = int(topk[t, j]) // El
                    c = int((topk[t, :j] // El == dst).sum())
                    if c % 4 == 0:
                        kk = int(key[t, j])
                        lead[(dst, c // 4)] = nxt.get(kk, 0)
                        nxt[kk] = lead[(dst, c // 4)] + 1
                    pos[t, j] = lead[(dst, c // 4)]
            send_pos.append(pos)
            continue
        flat = key.reshape(-1)
        pos = np.zeros_like(flat)
        for kk in np.unique(flat):
            idx = np.nonzero(flat == kk)[0]
            pos[idx] = np.arange(len(idx))
        send_pos.append(pos.reshape(T, k))
    # receiver position: within (expert, wave), order by (source shard, sender slot)
    recs = []
    for s in range(R):
        for t in range(T):
            for j in range(k):
                p = int(send_pos[s][t, j])
                if p < (Wv * Cs if chunks else Cs):
                    w = p // Cs if chunks else t // Tw
                    recs.append((int(S[s]["topk"][t, j]), w, s, p, t, j))
    recs.sort()
    keep = [np.zeros((T, k), bool) for _ in range(R)]
    cur, n = None, 0
    for e, w, s, sp, t, j in recs:
        if (e, w) != cur:
            cur, n = (e, w), 0
        keep[s][t, j] = n < Cr
        n += 1
    # outputs
    outs = []
    for s in range(R):
        x = f64(W_["x"][s])
        z = bf16_round(x @ f64(W_["wld"]).T)
        yl = np.zeros((T, L))
        for t in range(T):
            for j in range(k):
                if not keep[s][t, j]:
                    continue
                e = int(S[s]["topk"][t, j])
                wg, wu, wd = (f64(w[e % El]) for w in W_["ex"][e // El])
                h = bf16_round(silu(z[t] @ wg.T) * (z[t] @ wu.T))
                y = bf16_round(h @ wd.T)
                yl[t] += float(S[s]["gates"][t, j]) * y
        yl = bf16_round(yl)
        o = yl @ f64(W_["wlu"]).T
        for sh in range(cfg.n_shared):
            hs = bf16_round(silu(x @ f64(W_["wsg"][sh]).T) * (x @ f64(W_["wsu"][sh]).T))
            o = o + hs @ f64(W_["wsd"][sh]).T
        outs.append((yl, bf16_round(o), keep[s]))
    return outs


@pytest.mark.parametrize("cf", ["1.10/1.15", "inf", "tight", "chunks", "chunks_tight", "dedup_tight",
                                "dedup_chunks", "dense_r1_w1_s0", "k1_w1", "k1_tight"])
def test_e2e_tiny_matches_brute_force(orc, cf):
    from dataclasses import replace
    from fractions import Fraction
    cfg = configs.TINY
    if cf == "dense_r1_w1_s0":
        # one rank, one wave, no capacity, no shared experts: a plain top-k
        # MoE layer with every expert local
        cfg = replace(cfg, n_ranks=1, n_waves=1, n_shared=0, cf_send=None, cf_recv=None)
    elif cf.startswith("k1"):    # top-1 routing (a gate per token)
        cfg = replace(cfg, top_k=1, n_waves=1 if cf == "k1_w1" else cfg.n_waves)
        if cf == "k1_tight":
            cfg = replace(cfg, cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2))
    if cf == "inf":
        cfg = replace(cfg, cf_send=None, cf_recv=None)
    elif cf.endswith("tight"):   # forces sender and receiver drops
        cfg = replace(cfg, cf_send=Fraction(1, 2), cf_recv=Fraction(1, 2))
    if "chunks" in cf:           # the other reading of the waves
        cfg = replace(cfg, waves="chunks")
    if cf.startswith("dedup"):   # one row per destination group of a token's choices
        cfg = replace(cfg, dedup=True)
    d, W_, S, BK, OUT = simulate(orc, cfg)
    ref = brute_force(cfg, d, W_, S)
    El, W, Tw = cfg.experts_per_rank, cfg.n_waves, math.ceil(cfg.T / cfg.n_waves)
    n_exact = n_all = 0
    total_drop = 0
    for s in range(cfg.n_ranks):
        yl_ref, out_ref, keep = ref[s]
        ylat, out = OUT[s]
        # the oracle's keep decisions: kept at the sender and present in the bank
        kept_o = np.zeros_like(keep)
        for t in range(cfg.T):
            for j in range(cfg.top_k):
                sl = S[s]["slot"][t, j]
                if sl < 0:
                    continue
                r, w = S[s]["topk"][t, j] // El, t // Tw
                if d.wave_mode == 1:
                    row = (s * W + sl // d.cap_send) * d.cap_send + sl % d.cap_send
                elif d.cap_send:
                    row = (s * W + w) * d.cap_send + sl
                else:
                    lens = [S[q]["demand"][r * W + ww] for q in range(cfg.n_ranks) for ww in range(W)]
                    row = int(np.sum(lens[:s * W + w])) + sl
                if d.dedup:           # bank_src holds return slots: row * 4 + index in the row
                    c = int((S[s]["topk"][t, :j] // El == r).sum())
                    row = row * 4 + c % 4
                kept_o[t, j] = row in set(BK[r]["bank_src"].tolist())
        assert (kept_o == keep).all()
        total_drop += (~keep).sum()
        for got, want in ((ylat, bits_of(yl_ref)), (out, bits_of(out_ref))):
            du = ulp_diff(got, want)
            assert du.max() <= 1
            n_exact += (du == 0).sum()
            n_all += du.size
    assert n_exact / n_all > 0.999
    if cf == "inf":
        assert total_drop == 0
    if cf.endswith("tight"):
        assert total_drop > 0
