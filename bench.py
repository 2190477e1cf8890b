"""Benchmark: routed tokens/s through one MI355X's share of the pooled-wave
MoE layer (route -> pack_waves -> bank -> expert_ffn -> combine), with the
roofline position of the dominant kernel and the oracle timed on the host.

One step = the whole path for one rank over one source shard of T tokens:
route the shard's logits, project and pack its pools, bank the receive
buffer (pools that all source shards packed for this rank -- built once,
untimed, by a device-copy loopback that stands in for the all-to-all),
run the six local experts, and combine (identity return loopback).  Bank +
expert FFN run on a second stream beside route + pack + the shared experts
(no data dependence between them); the combine waits for both.

The line's value is the 4096-token shard at rank 0 (mean over the K timed
steps; the median and the spread are in step_ms).  Beside it: the dominant
kernel's roofline, the oracle's rate on the host, the same steps after a
1 GiB read sweep each (cold_cache, with the copy kernels' and the router's
per-kernel rates after such a sweep), the backward of the share, and the
figures of three more workloads, forward and backward (the 65536-token
long-context shard at rank 0, and the most-loaded rank of the Zipf-skewed
16384-token shard and of its dropless form).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--rank R|hot]
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "routed tokens/s through MoE layer on 1 MI355X; % HBM/MFMA roofline; drop %"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class State:
    pass


def setup(cfg, rank=0, device="cuda", seed=0, progress=False, keep_logits=False):
    """Inputs in HBM for one rank: its own shard, its experts' weights, and
    the receive buffer made from every source shard's pools (loopback).
    keep_logits: also keep a host copy of every shard's router logits."""
    import torch
    from dispatch_softmax_top_amd import share
    from synth import gen

    st = State()
    st.cfg, st.rank = cfg, rank
    d = st.d = share.make_dims(cfg)
    st.wr = gen.router_weight(cfg, device, seed)
    st.wld = gen.latent_down(cfg, device, seed)
    st.wg, st.wu, st.wd = gen.rank_experts(cfg, rank, device, seed)
    st.wlu = gen.latent_up(cfg, device, seed)
    st.wsg, st.wsu, st.wsd = gen.shared(cfg, device, seed)

    snd = share.Sender(d, device)
    R, W = d.n_ranks, d.n_waves
    El = cfg.experts_per_rank
    st.sent_demand = 0     # pool rows asked for, all shards
    st.sent_fill = 0       # pool rows sent
    st.sent_dropped = 0    # assignments dropped at the sender (a row may carry several: dedup)
    # kept sender rows per (destination rank, wave, local expert), all shards:
    # what every rank's bank step would see (drop statistics, hottest rank)
    st.recv_counts = torch.zeros(R * W * El, dtype=torch.int64, device=device)
    wave_of = torch.arange(cfg.T, device=device) // -(-cfg.T // W)
    st.host_logits = [] if keep_logits else None
    if d.cap_send:
        st.n_recv_rows = R * W * d.cap_send
        st.recv = torch.empty(st.n_recv_rows, share.row_bytes(d), dtype=torch.uint8,
                              device=device)
        rv = st.recv.view(R, W, d.cap_send, -1)
    else:
        parts, lens = [], []
    t0 = time.time()
    for s in range(cfg.n_shards):
        x = gen.hidden(cfg, s, device, seed)
        lg = gen.logits(cfg, s, x, st.wr, seed)
        snd.route(lg)
        snd.pack(x, st.wld)
        st.sent_demand += int(snd.demand.sum())
        st.sent_fill += int(snd.fill.sum())
        st.sent_dropped += int((snd.slot < 0).sum())
        e = snd.topk.long()
        if d.wave_mode == moe_waves_chunks():   # the wave is the chunk of the slot
            wv = snd.slot.long().clamp(min=0) // d.cap_send
        else:
            wv = wave_of[:, None]
        key = ((e // El) * W + wv) * El + e % El
        st.recv_counts += torch.bincount(key[snd.slot >= 0], minlength=R * W * El)
        if d.cap_send:
            rv[s].copy_(snd.pools.view(R, W, d.cap_send, -1)[rank])
        else:
            o = snd.pool_offsets.cpu().tolist()
            for w in range(W):
                a, b = o[rank * W + w], o[rank * W + w + 1]
                parts.append(snd.pools[a:b].clone())
                lens.append(b - a)
        if s == rank:
            st.x, st.logits = x, lg
        if keep_logits:
            st.host_logits.append(lg.cpu().numpy())
        if progress and (s % 16 == 15 or s == cfg.n_shards - 1):
            log(f"setup: shard {s + 1}/{cfg.n_shards} packed ({time.time() - t0:.1f}s)")
    if d.cap_send:
        st.recv_offsets = None
    else:
        st.recv = torch.cat(parts)
        st.n_recv_rows = st.recv.shape[0]
        import itertools
        st.recv_offsets = torch.tensor([0] + list(itertools.accumulate(lens)),
                                       dtype=torch.int64, device=device)
    st.snd = share.Sender(d, device)
    st.rcv = share.Receiver(d, st.n_recv_rows, device)
    st.cmb = share.Combiner(d, device)
    st.s_ffn = torch.cuda.Stream(device)
    st.ev_start, st.ev_ffn = torch.cuda.Event(), torch.cuda.Event()
    torch.cuda.synchronize()
    st.bal = None  # quantile balancing state (bench --balance-alpha)
    return st


def moe_waves_chunks():
    from dispatch_softmax_top_amd import MOE_WAVES_CHUNKS
    return MOE_WAVES_CHUNKS


def receiver_stats(st):
    """(receiver drop % over all ranks, rank with the most kept received rows)
    from the kept sender rows of every shard."""
    d = st.d
    c = st.recv_counts.view(d.n_ranks, -1)
    kept = c.clamp(max=d.cap_recv) if d.cap_recv else c
    total = int(c.sum())
    pct = 100.0 * (total - int(kept.sum())) / max(total, 1)
    return pct, int(kept.sum(1).argmax())


def path_roofline(kernels, work, ms):
    """Time the step's kernels would take at the HBM or MFMA peak (whichever
    bounds each), over the measured step time.  Kernels without an
    algorithmic figure (slot ranking, flag kernels) count as zero."""
    t = 0.0
    for name, (kind, amount) in work.items():
        n = kernels.get(name, {}).get("launches_per_step", 0)
        if kind == "flop":
            t += n * amount / (PEAK_BF16_TFLOPS * 1e12)
        else:
            t += n * amount / (PEAK_HBM_GBS * 1e9)
    return {"ms_at_peaks": round(t * 1e3, 4), "frac": round(t * 1e3 / ms, 4)}


def sweep_buffer(flush_bytes):
    """A device buffer of flush_bytes for cache sweeps (written once here)."""
    import torch
    return torch.ones(flush_bytes // 2, dtype=torch.bfloat16, device="cuda")


def sweep(buf):
    """Read every byte of buf (a reduction): L2 and the 256 MB MALL then hold
    only clean lines of buf, so the next kernels find their inputs in HBM and
    write back nothing of the sweep's."""
    import torch
    torch.sum(buf, dtype=torch.float32)


def cold_steps(st, steps, stepper=None, flush_bytes=1 << 30):
    """ms per step when every step starts after a read sweep of flush_bytes
    (inputs and weights evicted from L2 and the 256 MB MALL, still in HBM);
    each step is timed alone on the stream the kernels run on."""
    import torch
    stepper = stepper or step
    stream = torch.cuda.current_stream()
    buf = sweep_buffer(flush_bytes)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        sweep(buf)
        e0.record(stream)
        stepper(st)
        e1.record(stream)
    torch.cuda.synchronize()
    del buf
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps


def host_cpu():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def step(st):
    """One pass of the path.  Bank + expert FFN read the receive buffer of the
    last exchange, not this step's route and pack, so they run on a second
    stream, started behind everything already on the main stream, which runs
    route, pack and then the shared experts; the combine waits for the FFN.
    Measured against one stream, three streams (the shared experts on their
    own) and other splits at four workloads, this one was fastest or within
    1.5% of the fastest at each."""
    import torch
    main = torch.cuda.current_stream()
    st.ev_start.record(main)
    st.s_ffn.wait_event(st.ev_start)
    with torch.cuda.stream(st.s_ffn):
        st.rcv.bank_rows(st.rank, st.recv, st.recv_offsets)
        st.rcv.ffn(st.wg, st.wu, st.wd)
        st.ev_ffn.record(st.s_ffn)
    route_shard(st)
    st.snd.pack(st.x, st.wld)
    st.cmb.shared(st.x, st.wsg, st.wsu)
    main.wait_event(st.ev_ffn)
    st.cmb.combine_shared(st.rcv.ret, st.recv_offsets, st.snd, st.wlu, st.wsd)


def route_shard(st):
    """Route the shard; with quantile balancing on, on the logits plus the bias
    of the past batches, then count this batch's choices and set the bias the
    next step routes with."""
    if st.bal is None:
        st.snd.route(st.logits)
    else:
        st.snd.route(st.logits, bias=st.bal.bias)
        st.bal.update(st.snd.topk)


def step_serial(st):
    """The same path with every call on one stream, in path order (moe_combine
    as one call): each kernel runs alone."""
    route_shard(st)
    st.snd.pack(st.x, st.wld)
    st.rcv.bank_rows(st.rank, st.recv, st.recv_offsets)
    st.rcv.ffn(st.wg, st.wu, st.wd)
    st.cmb.combine(st.rcv.ret, st.recv_offsets, st.snd, st.x, st.wlu, st.wsg, st.wsu, st.wsd)


def algorithmic_work(st):
    """Per-kernel algorithmic flops / bytes of one step from the actual counts."""
    d = st.d
    T, k, L, D, F, S, Fs = d.T, d.top_k, d.latent, d.d_model, d.d_ff, d.n_shared, d.d_ff_shared
    kept_s = int(st.snd.fill.sum())
    n_slots = int(st.snd.pools.shape[0])
    kept_r = int(st.rcv.bfill.sum())
    w = {}
    w["gemm_latent_down"] = ("flop", 2.0 * T * D * L)
    w["gemm_expert_swiglu"] = ("flop", 4.0 * kept_r * L * F)
    w["gemm_expert_down"] = ("flop", 2.0 * kept_r * F * L)
    w["gemm_shared_swiglu"] = ("flop", 4.0 * T * D * S * Fs)
    w["gemm_up_shared"] = ("flop", 2.0 * T * (L + S * Fs) * D)
    w["route_topk_softmax"] = ("byte", T * d.n_experts * 4.0 + T * k * 8.0)
    w["pack_rows"] = ("byte", T * L * 2.0 + kept_s * (2 * L + 16) + (n_slots - kept_s) * 16.0)
    w["bank_rows"] = ("byte", 2.0 * kept_r * 2 * L)
    kept_a = int((st.snd.slot >= 0).sum())  # kept assignments (one return row each)
    w["combine_gather"] = ("byte", kept_a * 2.0 * L + T * k * 8.0 + T * L * 2.0)
    return w


def backward_step(st):
    """Backward of the same share, every call on one stream: combine side,
    router, experts (the return exchange reversed: a loopback identity, as in
    the forward return), pack side (the forward exchange reversed, likewise)."""
    b = st.bwd
    # ragged mode: both loopbacks keep the receive layout, as the forward's
    b.combine(st.rcv.ret, st.snd, st.cmb, st.x, st.wlu, st.wsg, st.wsu, st.wsd, st.d_out,
              ret_offsets=st.recv_offsets)
    b.route(st.logits, st.snd, bias=None if st.bal is None else st.bal.bias)
    b.ffn(st.rcv, st.wg, st.wu, st.wd, b.d_returned)
    b.pack(b.d_recv, st.snd, st.x, st.wld, st.wsg, st.wsu, pool_offsets=st.recv_offsets)


def backward_work(st):
    """Algorithmic flops / bytes of the backward's kernels, from the actual
    counts (the same bookkeeping as the forward's)."""
    d = st.d
    T, k, L, D, F, S, Fs, E = (d.T, d.top_k, d.latent, d.d_model, d.d_ff, d.n_shared,
                               d.d_ff_shared, d.n_experts)
    El = E // d.n_ranks
    SF = S * Fs
    Tp = -(-T // 32) * 32
    kept_s = int(st.snd.fill.sum())
    kept_r = int(st.rcv.bfill.sum())
    n_slots = int(st.n_recv_rows)
    if d.cap_send:   # every expert's K block: its capacity over all waves
        kpad = El * (-(-(d.n_waves * d.cap_recv) // 32) * 32)
    else:            # packed: each expert's rows rounded up to K tiles, at least 256
        rows = st.rcv.bfill.view(d.n_waves, El).sum(0).tolist()
        kpad = sum(max(-(-r // 32) * 32, 256) for r in rows)
    # the backward SwiGLU writes h and d_a | d_b transposed itself when the
    # bank's product groups are one per local expert (at most 4 waves and
    # 32-bit copy offsets over the bank), leaving dy and u to transpose
    merged = d.n_waves <= 4 and st.rcv.n_bank_rows * max(L, F) * 2 < 2**31 - 1
    tcols = 2 * L if merged else 2 * L + 3 * F
    f = lambda v: ("flop", float(v))
    b = lambda v: ("byte", float(v))
    return {
        "gemm_bwd_d_ylat": f(2 * T * D * (L + SF)),
        "gemm_shared_swiglu_bwd": f(4 * T * D * SF),
        "gemm_bwd_dw_combine": f(2 * D * (L + SF) * T),     # dW_lu and dW_sd, one launch
        "gemm_bwd_d_h": f(2 * kept_r * L * F),
        "gemm_expert_swiglu_bwd": f(4 * kept_r * L * F),
        "gemm_bwd_d_u": f(2 * kept_r * 2 * F * L),
        "gemm_bwd_dw_experts": f(3 * 2 * L * F * kept_r),  # dW_d, dW_g, dW_u, one launch
        "gemm_bwd_dx": f(2 * T * D * (L + 2 * SF)),
        "gemm_bwd_dw_pack": f(2 * (L + 2 * SF) * D * T),    # dW_ld, dW_sg, dW_su, one launch
        # d_ylat row + kept returned rows read; every d_returned row written
        "combine_backward": b(T * L * 2 + kept_s * L * 2 + n_slots * L * 2 + T * k * 16),
        "route_backward": b(T * E * 8 + T * k * 12),
        "gather_bank_grad": b(kept_r * L * 4),
        "combine_gather": b(kept_s * L * 2 + T * k * 8 + T * L * 2),
        # transposes (batched launches): elements read + elements written, padding included
        "transpose_combine_weights": b(4 * D * L + 4 * D * SF),
        "transpose_combine_acts": b(2 * T * (D + L + SF) + 2 * Tp * (D + L + SF)),
        "transpose_expert_weights": b(3 * 4 * El * L * F),
        "transpose_bank": b(2 * kept_r * tcols + 2 * kpad * tcols),
        "transpose_pack_weights": b(4 * L * D + 8 * SF * D),
        "transpose_pack_acts": b(2 * T * (D + L + 2 * SF) + 2 * Tp * (D + L + 2 * SF)),
    }


def kernel_table(prof, work, steps):
    """Per-kernel entries from the library's event timing; a split GEMM's
    rate is taken over the kernel and its _tail launch."""
    per_step = {name: tot / steps for name, (tot, n) in prof.items()}
    kernels = {}
    for name, (tot, n) in prof.items():
        avg = tot / n
        kind, amount = work.get(name, (None, 0.0))
        entry = {"avg_us": round(avg * 1e3, 3), "launches_per_step": n // steps}
        tail = name + "_tail"
        if tail in per_step:
            entry["tail_us"] = round(per_step[tail] * 1e3, 3)
            avg = per_step[name] + per_step[tail]
            entry["with_tail_us"] = round(avg * 1e3, 3)
        if kind == "flop":
            entry["tflops"] = round(amount / (avg * 1e-3) / 1e12, 2)
            entry["mfma_frac"] = round(entry["tflops"] / PEAK_BF16_TFLOPS, 4)
        elif kind == "byte":
            entry["gbs"] = round(amount / (avg * 1e-3) / 1e9, 1)
            entry["hbm_frac"] = round(entry["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = entry
    return kernels, per_step


def bench_backward(st, steps, warmup):
    """Backward timing (its own timed region, after the forward's), the
    per-kernel pass and the roofline of its dominant kernel."""
    import torch
    import dispatch_softmax_top_amd as moe
    from dispatch_softmax_top_amd import share
    from synth import gen
    d = st.d
    st.bwd = share.Backward(d, st.n_recv_rows)
    # stand-in gradient of the layer output: seeded N(0, 1) bf16
    st.d_out = gen.payload_rows(d.T, d.d_model, 71, "cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        backward_step(st)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        backward_step(st)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    log(f"bench: backward {steps} steps, {ms:.3f} ms/step")
    moe.moe_profile_reset()
    moe.moe_profile_enable(True)
    for _ in range(steps):
        backward_step(st)
    moe.moe_profile_collect()
    moe.moe_profile_enable(False)
    work = backward_work(st)
    kernels, per_step = kernel_table(moe.moe_profile_read(), work, steps)
    gemms = [n for n, (kind, _) in work.items() if kind == "flop" and n in per_step]
    dom = max(gemms, key=lambda n: per_step[n] + per_step.get(n + "_tail", 0.0))
    dom_s = (per_step[dom] + per_step.get(dom + "_tail", 0.0)) * 1e-3
    achieved = work[dom][1] / dom_s / 1e12
    flops = sum(a for kind, a in work.values() if kind == "flop")
    return {
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(d.T / (ms * 1e-3), 1),
        "tflops_per_step": round(flops / 1e12, 4),
        "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "data": "d_out: seeded N(0,1) bf16; both exchanges reversed as loopback identities",
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counted_traffic(dom, st.cfg.name)},
        "path_roofline": path_roofline(kernels, work, ms),
        "kernels": kernels,
    }


TRAFFIC_SOURCES = ("dispatch_softmax_top_amd/csrc/gemm.h", "dispatch_softmax_top_amd/csrc/gemm.hip",
                   "dispatch_softmax_top_amd/csrc/common.h")


def counted_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading),
    or None if none was taken for this workload or the kernel's sources have
    changed since."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    sha = h.hexdigest()
    for f in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_bytes.txt")):
        for line in open(f):
            if not line.startswith(f"traffic {kernel} "):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[2:])
            if kv.get("workload") == workload and kv.get("source_sha256") == sha:
                return int(kv["bytes_per_launch"])
    return None


def _u16(t):
    import numpy as np
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_cpu_baseline(st, rows=(64, 160, 32)):
    """Oracle timing on the host.  Sample: route + sender slots of the whole
    shard (full), latent rows for `rows[0]` tokens, expert FFN for `rows[1]`
    bank rows, combine (gather + up-projection + shared experts) for
    `rows[2]` tokens; each sampled stage is scaled linearly to its full row
    count.  Returns (tokens/s, description)."""
    import numpy as np
    import oracle as orc
    cfg = st.cfg
    dd = orc.dims(cfg)
    lg = st.logits.cpu().numpy()
    x = _u16(st.x)
    est = 0.0
    t0 = time.perf_counter()
    topk, gates = orc.route(lg, cfg.top_k)
    snd = orc.sender(dd, topk)
    t1 = time.perf_counter()
    est += t1 - t0
    rng = np.random.default_rng(0)
    toks = rng.choice(cfg.T, rows[0], replace=False)
    wld = _u16(st.wld)
    t0 = time.perf_counter()
    orc.latent(x, wld, rows=toks)
    t1 = time.perf_counter()
    est += (t1 - t0) * cfg.T / rows[0]
    # pack rows + bank copy: memcpy-class work, timed in full on the oracle
    z = np.zeros((cfg.T, cfg.latent), np.uint16)
    t0 = time.perf_counter()
    pools = orc.pack_rows(dd, z, topk, snd["slot"], snd["pool_offsets"])
    t1 = time.perf_counter()
    est += t1 - t0
    recv = st.recv.cpu().numpy()
    hdr = orc.headers(recv, cfg.latent)
    t0 = time.perf_counter()
    bo = orc.bank_slots(dd, st.rank, hdr, None if st.recv_offsets is None else st.recv_offsets.cpu().numpy())
    bank = orc.bank_rows(dd, recv, bo["bank_offsets"], bo["bank_src"], bo["bfill"])
    t1 = time.perf_counter()
    est += t1 - t0
    kept = int(bo["bfill"].sum())
    wg, wu, wd = (_u16(w) for w in (st.wg, st.wu, st.wd))
    t0 = time.perf_counter()
    for r in range(rows[1]):
        orc.ffn_row(bank[r], wg[0], wu[0], wd[0])
    t1 = time.perf_counter()
    est += (t1 - t0) * kept / rows[1]
    ret = np.zeros((st.n_recv_rows, cfg.latent), np.uint16)
    wlu = _u16(st.wlu)
    wsg, wsu, wsd = (_u16(w) for w in (st.wsg, st.wsu, st.wsd))
    t0 = time.perf_counter()
    orc.combine(dd, ret, None if st.recv_offsets is None else st.recv_offsets.cpu().numpy(),
                topk, snd["slot"], gates, x, wlu, wsg, wsu, wsd, tokens=toks[:rows[2]])
    t1 = time.perf_counter()
    est += (t1 - t0) * cfg.T / rows[2]
    desc = (f"oracle, 1 thread: route+sender slots+pack rows+bank slots/copy in full for the "
            f"{cfg.T}-token shard; latent on {rows[0]} tokens, expert FFN on {rows[1]} of "
            f"{kept} bank rows, combine on {rows[2]} tokens; sampled stages scaled by rows")
    return cfg.T / est, desc


def setup_rank(cfg, which, progress=False):
    """Setup for rank `which`: an int, or "hot" -- the rank with the most kept
    received rows, found from a first pass over every shard."""
    import torch
    if which != "hot":
        return setup(cfg, int(which), progress=progress)
    st = setup(cfg, 0, progress=progress)
    rank = receiver_stats(st)[1]
    if rank == 0:
        return st
    log(f"bench: {cfg.name}: hottest rank is {rank}: setup again")
    del st
    torch.cuda.empty_cache()
    return setup(cfg, rank, progress=progress)


def time_steps(st, stepfn, steps):
    """(mean ms per step over the whole timed region, [ms of each step]):
    events on the main stream, which every step's other streams join before
    its combine, so consecutive events bracket exactly one step."""
    import torch
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        stepfn(st)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]) / steps, per


def step_stats(per):
    s = sorted(per)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"mean": round(sum(s) / n, 4), "median": round(med, 4), "min": round(s[0], 4),
            "max": round(s[-1], 4)}


def kernel_pass(st, steps):
    """Per-kernel durations: the library brackets each launch with hipEvents.
    The calls go on one stream, so that each kernel runs alone (in the
    two-stream step a kernel's duration depends on what it happens to share
    the GPU with)."""
    import dispatch_softmax_top_amd as moe
    moe.moe_profile_reset()
    moe.moe_profile_enable(True)
    for _ in range(steps):
        step_serial(st)
    moe.moe_profile_collect()
    moe.moe_profile_enable(False)
    work = algorithmic_work(st)
    # A GEMM whose last round was split along K finishes in a second kernel
    # (<name>_tail: sum of the partial tiles and the epilogue); its rate is
    # taken over both launches.
    kernels, per_step = kernel_table(moe.moe_profile_read(), work, steps)
    return kernels, per_step, work


COLD_KERNELS = ("route_topk_softmax", "pack_rows", "bank_rows", "combine_gather")


def cold_kernel_pass(st, steps, flush_bytes=1 << 30):
    """The per-kernel pass with a read sweep of flush_bytes before every step
    (outside the timed launches): inputs that no earlier kernel of the step
    wrote (logits, the receive buffer, weights) come from HBM.  Returns the
    entries of the copy kernels and the router."""
    import torch
    import dispatch_softmax_top_amd as moe
    buf = sweep_buffer(flush_bytes)
    moe.moe_profile_reset()
    for _ in range(steps):
        sweep(buf)
        moe.moe_profile_enable(True)
        step_serial(st)
        moe.moe_profile_enable(False)
    moe.moe_profile_collect()
    torch.cuda.synchronize()
    del buf
    kernels, _ = kernel_table(moe.moe_profile_read(), algorithmic_work(st), steps)
    return {n: kernels[n] for n in COLD_KERNELS if n in kernels}


def gemm_frac(kernels, name):
    k = kernels.get(name, {})
    return k.get("mfma_frac")


def drop_stats(st):
    cfg, d = st.cfg, st.d
    kept_r, dem_r = int(st.rcv.bfill.sum()), int(st.rcv.bdemand.sum())
    return {
        "sender_pct_own_shard": round(100.0 * int((st.snd.slot < 0).sum()) / (d.T * d.top_k), 3),
        "sender_pct_all_shards": round(100.0 * st.sent_dropped / (cfg.n_shards * d.T * d.top_k), 3),
        "pool_rows_sent_per_shard": round(st.sent_fill / cfg.n_shards, 1),
        "receiver_pct_rank": round(100.0 * (dem_r - kept_r) / max(dem_r, 1), 3),
        "receiver_pct_all_ranks": round(receiver_stats(st)[0], 3),
        "bad_rows": int(st.rcv.bad_rows[0]),
    }


# The other workloads of the line: the 65536-token long-context shard at rank
# 0, and the most-loaded rank of the Zipf-skewed 16384-token shard and of its
# dropless (ragged) form.
OTHER_WORKLOADS = ((3, "0"), (2, "hot"), (4, "hot"))


def workload_summary(cfg, which, steps, warmup, backward=True):
    """Figures of one more workload: forward step time (mean, median, cold
    caches), routed tokens/s, path roofline, the expert GEMMs' MFMA fractions
    and the drop rates; with backward, the backward's step time, path
    roofline and dominant kernel."""
    import torch
    t0 = time.time()
    st = setup_rank(cfg, which)
    for _ in range(warmup):
        step(st)
    ms, per = time_steps(st, step, steps)
    kernels, per_step, work = kernel_pass(st, steps)
    cold = cold_steps(st, steps)
    out = {
        "workload": cfg.name, "rank": st.rank, "rank_choice": which, "T": st.d.T,
        "cap_send": st.d.cap_send, "cap_recv": st.d.cap_recv, "steps": steps,
        "ms_per_step": round(ms, 4), "step_ms": step_stats(per),
        "tokens_per_s": round(st.d.T / (ms * 1e-3), 1),
        "cold_cache_ms_per_step": round(cold, 4),
        "path_roofline": path_roofline(kernels, work, ms),
        "gemm_expert_swiglu_mfma_frac": gemm_frac(kernels, "gemm_expert_swiglu"),
        "gemm_expert_down_mfma_frac": gemm_frac(kernels, "gemm_expert_down"),
        "kept_rows_at_rank": int(st.rcv.bfill.sum()),
        "drops": drop_stats(st),
    }
    if backward and not st.d.dedup:
        bw = bench_backward(st, steps, warmup)
        out["backward"] = {k: bw[k] for k in ("ms_per_step", "tokens_per_s", "achieved_tflops",
                                               "roofline", "path_roofline")}
    out["wall_s"] = round(time.time() - t0, 1)
    del st
    torch.cuda.empty_cache()
    log(f"bench: {cfg.name} rank {out['rank']}: {ms:.3f} ms/step")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1,
                    help="workload: 0 tiny (64 tokens, 48 experts), 1 the 4096-token share, "
                         "2 Zipf 16384 tokens, 3 long context 65536 tokens, 4 Zipf 16384 "
                         "tokens dropless")
    ap.add_argument("--rank", default="0",
                    help="rank to measure, or 'hot': the rank with the most kept received rows")
    ap.add_argument("--serial", action="store_true",
                    help="issue the step's calls on one stream (each kernel alone)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the steps timed after a 1 GiB read sweep each (cold caches)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' forward figures (65536 tokens at rank 0, "
                         "the Zipf 16384-token hot rank, its dropless hot rank)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward measurements")
    ap.add_argument("--balance-alpha", type=float, default=None, metavar="ALPHA",
                    help="quantile balancing on: route with the bias -ALPHA (f - 1/E) from the "
                         "selection counts of the past --balance-window batches")
    ap.add_argument("--balance-window", type=int, default=8)
    ap.add_argument("--dedup", action="store_true",
                    help="variant: a token's choices on one destination share rows (up to four "
                         "ids per row); the backward is not measured")
    ap.add_argument("--waves", choices=("tokens", "chunks"), default="tokens",
                    help="tokens: wave(t) = t / T_w, a pool per (destination, wave); chunks: "
                         "one pool of n_waves * C_s rows per destination cut into n_waves chunks")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise device copy of MIB mebibytes, three "
                         "times: the reference for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the expert-parallel layer; the exchange "
              "between GPUs is a loopback and runs on one GPU only. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import dispatch_softmax_top_amd as moe
    from synth import configs

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)   # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n}))
        return

    cfg = configs.WORKLOADS[args.config]
    if args.waves != cfg.waves or args.dedup:
        import dataclasses
        cfg = dataclasses.replace(cfg, waves=args.waves, dedup=args.dedup or cfg.dedup)
    log(f"bench: {cfg.name} rank {args.rank}: setup")
    st = setup_rank(cfg, args.rank, progress=True)
    rank = st.rank
    if args.balance_alpha is not None:
        from dispatch_softmax_top_amd import share
        st.bal = share.Balancer(cfg.n_experts, args.balance_window, args.balance_alpha)
    stepfn = step_serial if args.serial else step
    for _ in range(args.warmup):
        stepfn(st)
    torch.cuda.synchronize()
    log("bench: warmup done")

    # timed region: K steps, events on the stream the kernels run on
    ms, per = time_steps(st, stepfn, args.steps)
    log(f"bench: {args.steps} steps, {ms:.3f} ms/step")
    kernels, per_step, work = kernel_pass(st, args.steps)
    dom = "gemm_expert_swiglu"
    dom_avg_s = (per_step[dom] + per_step.get(dom + "_tail", 0.0)) * 1e-3
    achieved = work[dom][1] / dom_avg_s / 1e12
    d = st.d
    kept_r = int(st.rcv.bfill.sum())
    drops = drop_stats(st)

    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        val, desc = run_cpu_baseline(st)
        cpu = {"value": round(val, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": desc, "wall_s": round(time.time() - t0, 1),
               "cpu_model": host_cpu(), "host_cpus": os.cpu_count()}

    backward = None
    if not args.no_backward and not d.dedup:
        backward = bench_backward(st, args.steps, args.warmup)
        backward["train_step_ms"] = round(ms + backward["ms_per_step"], 4)
        backward["train_tokens_per_s"] = round(d.T / ((ms + backward["ms_per_step"]) * 1e-3), 1)

    cold = None
    if not args.no_cold:
        cms = cold_steps(st, args.steps, stepfn)
        cold = {"ms_per_step": round(cms, 4), "tokens_per_s": round(d.T / (cms * 1e-3), 1),
                "flush_bytes": 1 << 30, "kernels": cold_kernel_pass(st, args.steps)}
        log(f"bench: cold-cache {cms:.3f} ms/step")

    workloads = None
    if not args.no_workloads and args.balance_alpha is None and not args.dedup \
            and args.waves == "tokens":
        del st      # every figure of the main workload is taken above
        torch.cuda.empty_cache()
        workloads = [workload_summary(configs.WORKLOADS[c], w, min(args.steps, 10), 2,
                                      backward=not args.no_backward)
                     for c, w in OTHER_WORKLOADS if (c, w) != (args.config, args.rank)]

    tok_s = d.T / (ms * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": step_stats(per),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs; random-init weights)",
        "config": {"workload": cfg.name, "rank": rank, "T": d.T, "d_model": d.d_model,
                   "latent": d.latent, "n_experts": d.n_experts, "n_ranks": d.n_ranks,
                   "top_k": d.top_k, "n_waves": d.n_waves, "d_ff": d.d_ff,
                   "n_shared": d.n_shared, "cap_send": d.cap_send, "cap_recv": d.cap_recv,
                   "source_shards": cfg.n_shards, "streams": 1 if args.serial else 2,
                   "waves": cfg.waves, "dedup": bool(d.dedup),
                   "balance": None if args.balance_alpha is None else
                   {"alpha": args.balance_alpha, "window": args.balance_window}},
        "roofline": {"kernel": dom, "bound": "mfma", "measured": "per-kernel pass after the "
                     "timed steps, calls on one stream (each kernel alone); duration of the "
                     "kernel plus its split-tail kernel",
                     "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": counted_traffic(dom, cfg.name)},
        "cpu_baseline": cpu,
        "path_roofline": path_roofline(kernels, work, ms),
        "rates": {"assignments_per_s": round(d.T * d.top_k / (ms * 1e-3), 1),
                  "kept_rows_per_s": round(kept_r / (ms * 1e-3), 1)},
        "cold_cache": cold,
        "backward": backward,
        "drops": drops,
        "kernels": kernels,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
