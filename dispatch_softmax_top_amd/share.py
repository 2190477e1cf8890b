"""One GPU's share of the layer: buffers (torch allocations) and the call
sequence route -> pack_waves -> bank -> expert_ffn -> combine.

Plumbing only.  Every step runs in libmoe's HIP kernels; torch allocates the
device memory and supplies the stream.  The exchange between GPUs is not
here: ``loopback_recv`` builds a receive buffer from pools of several
source shards with device copies (a stand-in for the all-to-all), and the
return path is the identity (the combine reads ``ret`` in place, taking
source index s as destination index s).
"""
from fractions import Fraction

import torch

from . import _lib as L


def make_dims(cfg, T=None) -> L.MoeDims:
    """Dims of a workload; capacities from the library's own formula."""
    T = cfg.T if T is None else T
    waves = {"tokens": L.MOE_WAVES_TOKENS, "chunks": L.MOE_WAVES_CHUNKS}[cfg.waves]
    d = L.MoeDims(T, cfg.d_model, cfg.latent, cfg.n_experts, cfg.n_ranks, cfg.top_k,
                  cfg.n_waves, cfg.d_ff, cfg.n_shared, cfg.d_ff_shared, 0, 0, waves,
                  int(getattr(cfg, "dedup", False)))
    if cfg.cf_send is not None:
        d.cap_send, d.cap_recv = L.moe_capacity(d, Fraction(cfg.cf_send), Fraction(cfg.cf_recv))
    return d


def row_bytes(d) -> int:
    return 2 * d.latent + 16


def n_pool_rows(d) -> int:
    return d.n_ranks * d.n_waves * d.cap_send if d.cap_send else d.T * d.top_k


def experts_per_rank(d) -> int:
    return d.n_experts // d.n_ranks


def _ws(d, call, n_rows, dev):
    n = L.moe_workspace_bytes(d, call, n_rows)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=dev) if n > 0 else None


class Sender:
    """Route + pack buffers of one source shard."""

    def __init__(self, d, device="cuda"):
        self.d = d
        T, k, L_, R, W = d.T, d.top_k, d.latent, d.n_ranks, d.n_waves
        dev = torch.device(device)
        self.topk = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.gates = torch.empty(T, k, dtype=torch.float32, device=dev)
        self.z = torch.empty(T, L_, dtype=torch.bfloat16, device=dev)
        self.pools = torch.empty(n_pool_rows(d), row_bytes(d), dtype=torch.uint8, device=dev)
        self.pool_offsets = (torch.empty(R * W + 1, dtype=torch.int64, device=dev)
                             if d.cap_send == 0 else None)
        self.slot = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.fill = torch.empty(R * W, dtype=torch.int32, device=dev)
        self.demand = torch.empty(R * W, dtype=torch.int32, device=dev)
        self.ws = _ws(d, L.MOE_CALL_PACK, 0, dev)

    def route(self, logits, stream=None, bias=None, renorm=False):
        if bias is None and not renorm:
            L.moe_route(logits, self.d.top_k, self.topk, self.gates, stream)
        else:
            L.moe_route_biased(logits, bias, self.d.top_k, self.topk, self.gates, stream,
                               L.MOE_ROUTE_RENORM if renorm else 0)

    def pack(self, x, w_lat_down, stream=None):
        L.moe_pack_waves(self.d, x, w_lat_down, self.topk, self.z, self.pools, self.pool_offsets,
                         self.slot, self.fill, self.demand, self.ws, stream)


class Receiver:
    """Bank + FFN buffers of one rank, for a receive buffer of n_recv_rows rows."""

    def __init__(self, d, n_recv_rows, device="cuda"):
        self.d = d
        dev = torch.device(device)
        El = experts_per_rank(d)
        G = d.n_waves * El
        self.n_recv_rows = n_recv_rows
        self.n_bank_rows = G * d.cap_recv if d.cap_send else n_recv_rows
        self.bank = torch.empty(self.n_bank_rows, d.latent, dtype=torch.bfloat16, device=dev)
        self.bank_offsets = (torch.empty(G + 1, dtype=torch.int64, device=dev)
                             if d.cap_send == 0 else None)
        self.bank_src = torch.empty(self.n_bank_rows, dtype=torch.int32, device=dev)
        self.bfill = torch.empty(G, dtype=torch.int32, device=dev)
        self.bdemand = torch.empty(G, dtype=torch.int32, device=dev)
        self.bad_rows = torch.empty(4, dtype=torch.int32, device=dev)
        # return rows: one per receive row, four (one per tail id) with dedup
        self.n_ret_rows = n_recv_rows * (4 if d.dedup else 1)
        self.ret = torch.empty(self.n_ret_rows, d.latent, dtype=torch.bfloat16, device=dev)
        self.ws_bank = _ws(d, L.MOE_CALL_BANK, n_recv_rows, dev)
        self.ws_ffn = _ws(d, L.MOE_CALL_FFN, self.n_bank_rows, dev)

    def bank_rows(self, rank, recv, recv_offsets=None, stream=None):
        L.moe_bank(self.d, rank, recv, recv_offsets, self.n_recv_rows, self.bank,
                   self.bank_offsets, self.bank_src, self.bfill, self.bdemand, self.bad_rows,
                   self.ws_bank, stream)

    def ffn(self, w_gate, w_up, w_down, stream=None):
        L.moe_expert_ffn(self.d, self.bank, self.bank_offsets, self.bank_src, self.bfill,
                         self.n_bank_rows, w_gate, w_up, w_down, self.ret, self.n_ret_rows,
                         self.ws_ffn, stream)


class Balancer:
    """Quantile balancing state of one router: the selection counts of the
    last `window` batches (a ring of rows) and the bias they give."""

    def __init__(self, n_experts, window, alpha, device="cuda"):
        dev = torch.device(device)
        self.E, self.window, self.alpha = n_experts, window, alpha
        self.counts = torch.zeros(window, n_experts, dtype=torch.int32, device=dev)
        self.bias = torch.zeros(n_experts, dtype=torch.float32, device=dev)
        self.batches = 0

    def update(self, topk, stream=None):
        """Count this batch's choices into the ring, then recompute the bias."""
        row = self.batches % self.window
        L.moe_expert_counts(topk, self.E, self.counts[row], stream)
        self.batches += 1
        n = min(self.batches, self.window)
        L.moe_balance_bias(self.counts[:n], self.alpha, self.bias, stream)


class Combiner:
    def __init__(self, d, device="cuda"):
        self.d = d
        dev = torch.device(device)
        self.ylat = torch.empty(d.T, d.latent, dtype=torch.bfloat16, device=dev)
        self.out = torch.empty(d.T, d.d_model, dtype=torch.bfloat16, device=dev)
        self.ws = _ws(d, L.MOE_CALL_COMBINE, 0, dev)
        # the shared experts' intermediate and the split partial tiles when
        # the combine runs as two calls
        self.h_shared = torch.empty(d.T, max(d.n_shared * d.d_ff_shared, 1), dtype=torch.bfloat16,
                                    device=dev)
        self.ws_shared = _ws(d, L.MOE_CALL_COMBINE_SHARED, 0, dev)

    def combine(self, returned, ret_offsets, snd: Sender, x, w_lat_up, ws_gate, ws_up, ws_down,
                stream=None):
        L.moe_combine(self.d, returned, ret_offsets, snd.topk, snd.slot, snd.gates, x, w_lat_up,
                      ws_gate, ws_up, ws_down, self.ylat, self.out, self.ws, stream)

    def shared(self, x, ws_gate, ws_up, stream=None):
        L.moe_shared_swiglu(self.d, x, ws_gate, ws_up, self.h_shared, stream)

    def combine_shared(self, returned, ret_offsets, snd: Sender, w_lat_up, ws_down, stream=None):
        L.moe_combine_shared(self.d, returned, ret_offsets, snd.topk, snd.slot, snd.gates,
                             w_lat_up, self.h_shared, ws_down, self.ylat, self.out,
                             self.ws_shared, stream)


class Backward:
    """Gradient buffers and workspaces of one rank's share (fixed or ragged
    mode): the sender's combine and pack sides, the receiver's experts and
    the router.  On one GPU both exchanges are loopbacks, read as identities
    like the forward return: the receiver's return-row gradients are the
    sender's d_returned, and the sender's pool-row gradients are the
    receiver's d_recv (in ragged mode both keep the receive layout: its
    offsets go with them)."""

    def __init__(self, d, n_recv_rows, device="cuda"):
        self.d = d
        dev = torch.device(device)
        T, L_, D, E = d.T, d.latent, d.d_model, d.n_experts
        S, Fs, F, El = d.n_shared, d.d_ff_shared, d.d_ff, experts_per_rank(d)
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.d_returned = torch.empty(n_recv_rows, L_, **bf)
        self.d_gates = torch.empty(T, d.top_k, dtype=torch.float32, device=dev)
        self.d_logits = torch.empty(T, E, dtype=torch.float32, device=dev)
        self.d_shared = torch.empty(T, 2, max(S, 1), Fs, **bf)
        self.dw_lat_up = torch.empty(D, L_, **bf)
        self.dws_down = torch.empty(max(S, 1), D, Fs, **bf)
        self.d_recv = torch.empty(n_recv_rows, L_, **bf)
        self.dw_gate = torch.empty(El, F, L_, **bf)
        self.dw_up = torch.empty(El, F, L_, **bf)
        self.dw_down = torch.empty(El, L_, F, **bf)
        self.dz = torch.empty(T, L_, **bf)
        self.dx = torch.empty(T, D, **bf)
        self.dw_lat_down = torch.empty(L_, D, **bf)
        self.dws_gate = torch.empty(max(S, 1), Fs, D, **bf)
        self.dws_up = torch.empty(max(S, 1), Fs, D, **bf)
        self.ws_combine = _ws(d, L.MOE_CALL_COMBINE_BWD, 0, dev)
        self.ws_ffn = _ws(d, L.MOE_CALL_FFN_BWD, 0 if d.cap_send else n_recv_rows, dev)
        self.ws_pack = _ws(d, L.MOE_CALL_PACK_BWD, 0, dev)

    def combine(self, returned, snd: Sender, cmb: Combiner, x, w_lat_up, ws_gate, ws_up, ws_down,
                d_out, stream=None, ret_offsets=None):
        L.moe_combine_backward(self.d, returned, snd.topk, snd.slot, snd.gates, snd.fill, x,
                               cmb.ylat, w_lat_up, ws_gate, ws_up, ws_down, d_out,
                               self.d_returned, self.d_gates, self.d_shared, self.dw_lat_up,
                               self.dws_down, self.ws_combine, stream, ret_offsets=ret_offsets)

    def route(self, logits, snd: Sender, bias=None, renorm=False, stream=None):
        L.moe_route_backward(logits, snd.topk, self.d_gates, self.d_logits, bias=bias,
                             stream=stream, flags=L.MOE_ROUTE_RENORM if renorm else 0)

    def ffn(self, rcv: Receiver, w_gate, w_up, w_down, d_ret, stream=None):
        L.moe_expert_ffn_backward(self.d, rcv.bank, rcv.bank_src, rcv.bfill, w_gate, w_up, w_down,
                                  d_ret, self.d_recv, self.dw_gate, self.dw_up, self.dw_down,
                                  self.ws_ffn, stream, bank_offsets=rcv.bank_offsets)

    def pack(self, d_pools, snd: Sender, x, w_lat_down, ws_gate, ws_up, stream=None,
             pool_offsets=None):
        L.moe_pack_backward(self.d, d_pools, snd.topk, snd.slot, x, self.d_shared, w_lat_down,
                            ws_gate, ws_up, self.dz, self.dx, self.dw_lat_down, self.dws_gate,
                            self.dws_up, self.ws_pack, stream, pool_offsets=pool_offsets)


# ----------------------------------------------------------------------------
# loopback exchange (harness side, stand-in for the all-to-all)
# ----------------------------------------------------------------------------

def loopback_recv_fixed(d, pools_by_source, rank, recv=None):
    """recv[s] = pools_s[dest = rank] for every source shard s (fixed mode)."""
    R, W, C, RB = d.n_ranks, d.n_waves, d.cap_send, row_bytes(d)
    if recv is None:
        recv = torch.empty(R * W * C, RB, dtype=torch.uint8, device=pools_by_source[0].device)
    rv = recv.view(R, W, C, RB)
    for s, pools in enumerate(pools_by_source):
        rv[s].copy_(pools.view(R, W, C, RB)[rank])
    return recv


def loopback_recv_ragged(d, pools_by_source, offsets_by_source, rank):
    """Ragged mode: concatenate segment (rank, w) of every source s in (s, w) order."""
    R, W = d.n_ranks, d.n_waves
    parts, lens = [], []
    for pools, offs in zip(pools_by_source, offsets_by_source):
        o = offs.cpu().tolist()
        for w in range(W):
            a, b = o[rank * W + w], o[rank * W + w + 1]
            parts.append(pools[a:b])
            lens.append(b - a)
    recv = torch.cat(parts) if parts else None
    offs = torch.tensor([0] + list(torch.tensor(lens).cumsum(0).tolist()), dtype=torch.int64,
                        device=pools_by_source[0].device)
    return recv, offs
