"""Helpers of the full-size parity tests: the oracle's decisions for every
source shard, where each receive row came from, a row selection that reaches
every kind of GEMM tile the kernels run, and the oracle's values of the
selected rows.

Everything the oracle computes here starts from generator tensors (synth)
and the oracle's own integer decisions; nothing produced by libmoe feeds it.

The tiling constants and formulas below mirror the GEMM kernels' (256 x 256
block tiles, K tiles of 32, the split of a partly filled last round along K,
groups of 8 tile-rows in the tile order).  They are used only to choose which
rows to check and to assert that the choice reached every split tile; no
expected value depends on them.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import dense

WORKERS = max(1, min(16, os.cpu_count() or 1))

# --- mirror of the GEMM tiling (row selection only) ------------------------
GBM = GBN = 256        # block tile rows / columns
GBK = 32               # K tile
MFMA_ROWS = 32         # rows of one MFMA row group
GSPLIT_MAX = 8         # parts per split tile at most
GSPLIT_MIN_KT = 16     # K tiles per part at least
GSPLIT_UNITS = 256     # partial tiles the split buffer holds
TILE_GROUP = 8         # tile-rows per group in the tile order
MERGE_WAVES = 4        # waves merged into one product group at most


def split_parts(total: int, ktiles: int, ncu: int) -> int:
    """Parts each tile of the last round is cut into (1: no split)."""
    max_parts = min(GSPLIT_MAX, ktiles // GSPLIT_MIN_KT)
    if max_parts < 2:
        return 1
    r = total % ncu
    if r == 0 or 2 * r > ncu:
        return 1
    return max(1, min(ncu // r, max_parts, GSPLIT_UNITS // r))


def tile_coords(logical: int, tm: int, tn: int):
    """(M tile, N tile) of a logical tile: groups of TILE_GROUP tile-rows,
    column-major inside a group."""
    per_group = TILE_GROUP * tn
    g = logical // per_group
    first = g * TILE_GROUP
    gs = min(tm - first, TILE_GROUP)
    r = logical - g * per_group
    return first + r % gs, r // gs


def dense_split_mtiles(M: int, N: int, K: int, ncu: int):
    """(parts, sorted M tiles holding a split tile) of a dense product."""
    tm, tn = math.ceil(M / GBM), math.ceil(N / GBN)
    total = tm * tn
    S = split_parts(total, K // GBK, ncu)
    if S == 1:
        return 1, []
    first = total - total % ncu
    return S, sorted({tile_coords(t, tm, tn)[0] for t in range(first, total)})


def product_groups(d, bfill, bank_offsets, width: int, n_bank_rows: int):
    """Bank positions of each product group of the grouped expert GEMMs, in
    group row order: one local expert over all waves (when the waves are few
    and the bank small enough for 32-bit copy offsets), else every (wave,
    expert) bank group alone."""
    El = d.n_experts // d.n_ranks
    W = d.n_waves

    def rows(g):
        start = int(bank_offsets[g]) if bank_offsets is not None else g * d.cap_recv
        return np.arange(start, start + int(bfill[g]), dtype=np.int64)

    if W <= MERGE_WAVES and n_bank_rows * width * 2 < 2 ** 31 - 1:
        return [np.concatenate([rows(w * El + j) for w in range(W)]) for j in range(El)]
    return [rows(g) for g in range(W * El)]


def grouped_split_tiles(groups, tn: int, K: int, ncu: int):
    """(parts, [(group, M tile)] of the split tiles) of a grouped product."""
    tiles = []
    for pg, pos in enumerate(groups):
        tmg = math.ceil(len(pos) / GBM)
        tiles += [(pg,) + tile_coords(rem, tmg, tn) for rem in range(tmg * tn)]
    total = len(tiles)
    S = split_parts(total, K // GBK, ncu)
    if S == 1:
        return 1, []
    return S, sorted({(pg, mt) for pg, mt, _ in tiles[total - total % ncu:]})


def mtile_probe_rows(n: int, mt: int):
    """Row indices (0 .. n-1) of M tile mt: the first row of each of its
    32-row MFMA groups, and its last row."""
    lo, hi = mt * GBM, min(n, (mt + 1) * GBM)
    return sorted(set(range(lo, hi, MFMA_ROWS)) | {hi - 1})


# --- the oracle's decisions -------------------------------------------------

def oracle_shards(orc, cfg, d_orc, logits):
    """Route + sender of every source shard (threads: the C oracle releases
    the interpreter lock while it runs)."""
    def one(s):
        topk, gates = orc.route(logits[s], cfg.top_k)
        return dict(topk=topk, gates=gates, **orc.sender(d_orc, topk))
    with ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(one, range(cfg.n_shards)))


def hot_rank(cfg, d_orc, shards):
    """Rank with the most kept received rows: kept sender rows per (rank,
    wave, local expert) over every shard, each clamped at the receiver
    capacity, summed per rank (waves by token)."""
    R, W, El = cfg.n_ranks, cfg.n_waves, cfg.experts_per_rank
    Tw = math.ceil(cfg.T / W)
    counts = np.zeros(R * W * El, np.int64)
    for sh in shards:
        t, j = np.nonzero(sh["slot"] >= 0)
        e = sh["topk"][t, j].astype(np.int64)
        counts += np.bincount(((e // El) * W + t // Tw) * El + e % El, minlength=R * W * El)
    c = counts.reshape(R, -1)
    kept = np.minimum(c, d_orc.cap_recv) if d_orc.cap_recv else c
    return int(kept.sum(1).argmax())


class RecvMap:
    """Rank `rank`'s receive buffer as the oracle's sender decisions make it
    (waves by token): per row its expert id (-1 empty), source shard and
    source token; segment starts and lengths in (source, wave) order."""

    def __init__(self, cfg, d_orc, shards, rank):
        R, W, El = cfg.n_ranks, cfg.n_waves, cfg.experts_per_rank
        Tw = math.ceil(cfg.T / W)
        lens = np.array([d_orc.cap_send if d_orc.cap_send else int(sh["demand"][rank * W + w])
                         for sh in shards for w in range(W)], np.int64)
        self.lens = lens
        self.starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        n = int(self.starts[-1])
        self.hdr = -np.ones(n, np.int32)
        self.shard = -np.ones(n, np.int32)
        self.tok = -np.ones(n, np.int64)
        for s, sh in enumerate(shards):
            t, j = np.nonzero((sh["topk"] // El == rank) & (sh["slot"] >= 0))
            row = self.starts[s * W + t // Tw] + sh["slot"][t, j]
            self.hdr[row] = sh["topk"][t, j]
            self.shard[row] = s
            self.tok[row] = t
        self.offsets = None if d_orc.cap_send else self.starts

    @property
    def n(self):
        return len(self.hdr)


def source_latent(cfg, rm: RecvMap, rows: np.ndarray, w_ld_t: np.ndarray, hidden) -> np.ndarray:
    """Oracle z of the source token of each receive row (dense.latent on the
    generator's x rows).  hidden(s) -> that shard's x as uint16 rows source
    (an object indexable by token arrays)."""
    out = np.zeros((len(rows), cfg.latent), np.uint16)
    shards = rm.shard[rows]
    for s in np.unique(shards):
        if s < 0:
            continue
        sel = np.nonzero(shards == s)[0]
        out[sel] = dense.latent(hidden(int(s), rm.tok[rows[sel]]), w_ld_t)
    return out


def pick(rng, pool, n):
    """n seeded picks from pool (all of it if smaller), sorted."""
    pool = np.asarray(pool)
    if len(pool) <= n:
        return np.sort(pool)
    return np.sort(rng.choice(pool, n, replace=False))
