"""Shared inputs for the GPU parity tests.

Every input here comes from synth (seeded generator) or from the oracle;
nothing produced by libmoe ever feeds the oracle.
"""
import math
from dataclasses import replace
from fractions import Fraction

import numpy as np
import torch

from conftest import bf16_from_u16, f64, row_rel_err, u16
from synth import configs, gen

TOL = 2e-2   # per output row: max|err| <= TOL * max|ref|

# between tiny and full: several 256-row GEMM tiles, ragged tails everywhere
# (T_w = 201 with a short last wave, latent 384 = 1.5 column tiles)
MID = configs.scaled(configs.TINY, "moe_mid_T601_D512_L384_E48_R8", T=601, d_model=512,
                     latent=384, d_ff=256, d_ff_shared=256)


def ragged(cfg):
    return replace(cfg, name=cfg.name + "_ragged", cf_send=None, cf_recv=None)


def with_cf(cfg, cs, cr):
    return replace(cfg, name=cfg.name + f"_cf{cs}_{cr}", cf_send=Fraction(cs), cf_recv=Fraction(cr))


def skewed(cfg):
    """Zipf routing bias (cold experts, hot ranks, empty groups)."""
    return replace(cfg, name=cfg.name + "_zipf", routing="zipf")


def chunked(cfg):
    """The other reading of the waves: one pool per destination cut into chunks."""
    return replace(cfg, name=cfg.name + "_chunks", waves="chunks")


def deduped(cfg):
    """The dedup variant: a token's same-destination choices share rows."""
    return replace(cfg, name=cfg.name + "_dedup", dedup=True)


def shard_inputs(cfg, s, device="cpu"):
    x = gen.hidden(cfg, s, device)
    wr = gen.router_weight(cfg, device)
    lg = gen.logits(cfg, s, x, wr)
    return x, lg


def assert_rows_close(got_u16, ref_u16, what, tol=TOL):
    e = row_rel_err(got_u16, ref_u16)
    bad = np.nonzero(e > tol)[0]
    assert len(bad) == 0, f"{what}: {len(bad)} rows over tolerance, worst {e.max():.3g} at row {int(e.argmax())}"


def dev(a, device="cuda"):
    """numpy array (uint16 = bf16 bits) -> device tensor."""
    if a.dtype == np.uint16:
        return bf16_from_u16(a).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    if t.dtype == torch.bfloat16:
        return u16(t)
    return t.detach().cpu().numpy()


def oracle_sender_all(orc, cfg, d_orc, n_shards=None):
    """Oracle route + sender for every source shard (integer part only)."""
    out = []
    for s in range(n_shards or cfg.n_shards):
        x, lg = shard_inputs(cfg, s)
        topk, gates = orc.route(lg.numpy(), cfg.top_k)
        snd = orc.sender(d_orc, topk)
        out.append(dict(x=x, logits=lg, topk=topk, gates=gates, **snd))
    return out


def recv_headers(cfg, d_orc, senders, rank):
    """Tail ids of rank's receive buffer, built from the oracle's sender
    decisions of every source shard; plus recv_offsets in ragged mode."""
    R, W, El = cfg.n_ranks, cfg.n_waves, cfg.experts_per_rank
    Tw = math.ceil(cfg.T / W)
    if d_orc.dedup:      # four ids per row: read them off the oracle's own pools
        import oracle as orc
        C = d_orc.cap_send
        ids = []
        for snd in senders:
            z = np.zeros((cfg.T, cfg.latent), np.uint16)
            pools = orc.pack_rows(d_orc, z, snd["topk"], snd["slot"])
            ids.append(orc.row_ids(pools, cfg.latent)[rank * W * C:(rank + 1) * W * C])
        return np.concatenate(ids), None
    segs, lens = [], []
    for snd in senders:
        topk, slot = snd["topk"], snd["slot"]
        if d_orc.wave_mode == 1:         # one pool of W * C_s rows; slot = row in it
            h = -np.ones(W * d_orc.cap_send, np.int32)
            mine = (topk // El == rank) & (slot >= 0)
            h[slot[mine]] = topk[mine]
            segs.append(h)
            continue
        for w in range(W):
            n = d_orc.cap_send if d_orc.cap_send else int(snd["demand"][rank * W + w])
            h = -np.ones(n, np.int32)
            for t in range(w * Tw, min(cfg.T, (w + 1) * Tw)):
                for j in range(cfg.top_k):
                    e = int(topk[t, j])
                    if e // El == rank and slot[t, j] >= 0:
                        h[slot[t, j]] = e
            segs.append(h)
            lens.append(n)
    hdr = np.concatenate(segs)
    offs = None if d_orc.cap_send else np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return hdr, offs


def rows_with_headers(payload_u16, hdr):
    """uint8 [n, 2L+16] rows: payload bits then {id, 0, 0, 0}, or the four
    ids of a [n, 4] hdr (dedup)."""
    n, L = payload_u16.shape
    rows = np.zeros((n, 2 * L + 16), np.uint8)
    rows[:, :2 * L] = payload_u16.view(np.uint8).reshape(n, 2 * L)
    h = np.ascontiguousarray(hdr, np.int32)
    w = 16 if h.ndim == 2 else 4
    rows[:, 2 * L:2 * L + w] = h.view(np.uint8).reshape(n, w)
    return rows
