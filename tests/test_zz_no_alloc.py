"""moe_pack_waves_noalloc: the sender call with its slot-assignment scratch
in the library's fixed device array instead of a caller workspace.

Each case runs the same inputs through moe_pack_waves (with a workspace) and
moe_pack_waves_noalloc, into separately poisoned output buffers, and asserts
every output equal bit for bit: z, slot, fill, demand, pool_offsets, every
pool row's tail, and the payload of every kept pool row.  The integer
outputs are also checked against the oracle's sender.  The calls run in a
row, the later ones on fewer tokens than the first, so the fixed scratch
still holds the first call's larger count table when they run.
"""
import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

import dispatch_softmax_top_amd as moe
import gpucase as gc
from dispatch_softmax_top_amd import share
from synth import configs, gen

# (name, workload, tokens): 4096 tokens fill 16 count tiles of 2048
# assignments; the later calls use fewer tiles and other pool counts
SEQUENCE = [
    ("share_T4096", configs.SHARE_4K, 4096),
    ("share_T1500", configs.SHARE_4K, 1500),
    ("mid_ragged_T601", gc.ragged(gc.MID), 601),
    ("mid_T333", gc.MID, 333),
]


def _run(cfg, T, noalloc):
    d = share.make_dims(cfg, T)
    x = gen.hidden(replace(cfg, T=T), 0, "cuda")
    wr = gen.router_weight(cfg, "cuda")
    lg = gen.logits(replace(cfg, T=T), 0, x, wr)
    snd = share.Sender(d)
    for t in (snd.z, snd.pools, snd.slot, snd.fill, snd.demand, snd.pool_offsets):
        if t is not None:
            t.view(torch.uint8).fill_(0xAB)
    snd.route(lg)
    if noalloc:
        moe.moe_pack_waves_noalloc(d, x, gen.latent_down(cfg, "cuda"), snd.topk, snd.z,
                                   snd.pools, snd.pool_offsets, snd.slot, snd.fill, snd.demand)
    else:
        snd.pack(x, gen.latent_down(cfg, "cuda"))
    torch.cuda.synchronize()
    return d, snd, lg


@pytest.mark.gpu
def test_noalloc_matches_workspace_call(orc):
    for name, cfg, T in SEQUENCE:
        print(f"\n[noalloc] {name}: T={T}", flush=True)
        d, ref, lg = _run(cfg, T, noalloc=False)
        _, got, _ = _run(cfg, T, noalloc=True)
        for what in ("topk", "z", "slot", "fill", "demand", "pool_offsets"):
            a, b = getattr(ref, what), getattr(got, what)
            if a is None:
                continue
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name}: {what}"
        L = d.latent
        assert torch.equal(ref.pools[:, 2 * L:], got.pools[:, 2 * L:]), f"{name}: pool tails"
        ids = ref.pools[:, 2 * L:2 * L + 4].contiguous().view(torch.int32).reshape(-1)
        kept = ids >= 0
        assert torch.equal(ref.pools[kept, :2 * L], got.pools[kept, :2 * L]), f"{name}: rows"
        # integer decisions against the oracle, on the same fp32 logits
        dd = orc.dims(cfg, T)
        topk, _ = orc.route(lg.cpu().numpy(), cfg.top_k)
        sn = orc.sender(dd, topk)
        assert np.array_equal(gc.host(got.slot), sn["slot"]), f"{name}: slot vs oracle"
        assert np.array_equal(gc.host(got.fill), sn["fill"]), f"{name}: fill vs oracle"
        assert np.array_equal(gc.host(got.demand), sn["demand"]), f"{name}: demand vs oracle"
        print(f"[noalloc] {name}: equal ({int(kept.sum())} kept rows)", flush=True)


def test_noalloc_rejects_oversize_before_launch():
    """A shape whose count table exceeds the fixed scratch is refused on the
    host (no device is touched: the pointers are never read)."""
    cfg = configs.SHARE_4K
    T = 400_000                       # 3.2M assignments: 1563 tiles x 193 counts
    d = share.make_dims(replace(cfg, T=T), T)
    need = moe.moe_workspace_bytes(d, moe.MOE_CALL_PACK)
    assert need > moe.MOE_NOALLOC_SCRATCH_BYTES
    fake = [ctypes.c_void_p(4096 * (i + 1)) for i in range(9)]
    rc = moe.lib().moe_pack_waves_noalloc(ctypes.byref(d), *fake, None)
    assert rc == -2
    assert b"fixed scratch" in moe.lib().moe_last_error()
    # the largest table that fits is accepted by the same size rule
    T_ok = 2_781_184 // cfg.top_k
    d_ok = share.make_dims(replace(cfg, T=T_ok), T_ok)
    assert moe.moe_workspace_bytes(d_ok, moe.MOE_CALL_PACK) <= moe.MOE_NOALLOC_SCRATCH_BYTES
    T_no = T_ok + 1
    d_no = share.make_dims(replace(cfg, T=T_no), T_no)
    assert moe.moe_workspace_bytes(d_no, moe.MOE_CALL_PACK) > moe.MOE_NOALLOC_SCRATCH_BYTES
