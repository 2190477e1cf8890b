"""Seeded synthetic inputs, shared by the oracle side and the HIP side.

Every tensor is a pure function of (seed, tensor id, index).  Uniforms come
from SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014): the i-th output of a stream with state ``s`` is
``mix64(s + (i + 1) * 0x9E3779B97F4A7C15)``.  Normals come from the
Box-Muller transform (Box & Muller, 1958) in float64, then are scaled,
rounded to float32 and then to bfloat16 (round to nearest even both times).

The arithmetic is expressed in torch int64 (two's-complement wrap equals
uint64 arithmetic) so the same code runs on the host or on a device.  A test
generates each input once and hands copies of that one tensor to both sides;
nothing here depends on the method under test.

Recipe (workload shapes in ``synth.configs``):
  x        bf16 N(0,1)          [T, d_model]        per shard
  W_r      bf16 N(0,1/d_model)  [E, d_model]        router weight
  logits   fp32 x.W_r^T (+ routing bias)            per shard
  W_ld     bf16 N(0,1/d_model)  [latent, d_model]   latent down (out x in)
  W_g,W_u  bf16 N(0,1/latent)   [d_ff, latent]      per global expert id
  W_d      bf16 N(0,1/d_ff)     [latent, d_ff]      per global expert id
  W_lu     bf16 N(0,1/latent)   [d_model, latent]   latent up
  W_sg,W_su bf16 N(0,1/d_model) [d_ff_sh, d_model]  per shared expert
  W_sd     bf16 N(0,1/d_ff_sh)  [d_model, d_ff_sh]  per shared expert
Routing skew: "zipf" adds b_e = 1.5 ln(w_rho), w_rho = rho^-1.1 / H over a
seeded permutation of the experts; "longctx" adds a per-shard N(0,1.5^2)
vector plus a piecewise-constant N(0,0.5^2) vector per 4096-token chunk.
"""
import math

import torch

GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1

# tensor ids
X, WR, WLD, WG, WU, WD, WLU, WSG, WSU, WSD, PERM, BSEQ, BCHUNK, PAYLOAD = range(1, 15)

_CHUNK = 1 << 24  # elements per generation chunk


def _s64(u: int) -> int:
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _mix_int(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def stream_state(seed: int, tid: int, idx: int) -> int:
    """Initial SplitMix64 state of the stream for (seed, tensor id, index)."""
    return _mix_int(_mix_int(seed * GOLDEN + 1) ^ _mix_int((tid << 32) ^ idx))


def uniform_bits(state: int, start: int, n: int, device) -> torch.Tensor:
    """Outputs start .. start+n-1 of the SplitMix64 stream, as int64 bit patterns."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix(i * _s64(GOLDEN) + _s64(state))


def _normals_f64(state: int, start: int, n: int, device) -> torch.Tensor:
    """Box-Muller normals for elements start .. start+n-1 (start even)."""
    assert start % 2 == 0
    npair = (n + 1) // 2
    bits = uniform_bits(state, start, 2 * npair, device).view(npair, 2)
    u = (_lsr(bits, 11).to(torch.float64) + 0.5) * (2.0 ** -53)
    r = torch.sqrt(-2.0 * torch.log(u[:, 0]))
    th = (2.0 * math.pi) * u[:, 1]
    out = torch.stack((r * torch.cos(th), r * torch.sin(th)), dim=1).reshape(-1)
    return out[:n]


def normal_f64(shape, sigma: float, tid: int, idx: int, seed: int = 0,
               device="cpu") -> torch.Tensor:
    n = math.prod(shape)
    st = stream_state(seed, tid, idx)
    return (_normals_f64(st, 0, n, device) * sigma).view(*shape)


def normal_bf16(shape, sigma: float, tid: int, idx: int, seed: int = 0,
                device="cpu") -> torch.Tensor:
    """bf16(fp32(sigma * N(0,1))) with the stream of (seed, tid, idx)."""
    n = math.prod(shape)
    st = stream_state(seed, tid, idx)
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        v = _normals_f64(st, s, m, device) * sigma
        out[s:s + m] = v.to(torch.float32).to(torch.bfloat16)
    return out.view(*shape)


# ----------------------------------------------------------------------------
# Workload tensors
# ----------------------------------------------------------------------------

def hidden(cfg, shard: int, device="cpu", seed: int = 0) -> torch.Tensor:
    return normal_bf16((cfg.T, cfg.d_model), 1.0, X, shard, seed, device)


def hidden_rows(cfg, shard: int, rows, device="cpu", seed: int = 0) -> torch.Tensor:
    """Rows ``rows`` of hidden(cfg, shard), bit for bit, without generating
    the others: element (t, i) is output t*d_model + i of the shard's stream,
    and with d_model even every row starts a Box-Muller pair."""
    D = cfg.d_model
    assert D % 2 == 0
    st = stream_state(seed, X, shard)
    r = torch.as_tensor(rows, dtype=torch.int64, device=device).reshape(-1)
    out = torch.empty(len(r), D, dtype=torch.bfloat16, device=device)
    step = max(1, _CHUNK // D)
    for a in range(0, len(r), step):
        rr = r[a:a + step]
        # stream positions 2p and 2p+1 feed the pair p = element index / 2
        pair = rr[:, None] * (D // 2) + torch.arange(D // 2, dtype=torch.int64, device=device)
        pos = torch.stack((2 * pair, 2 * pair + 1), dim=-1)
        bits = _mix((pos + 1) * _s64(GOLDEN) + _s64(st))
        u = (_lsr(bits, 11).to(torch.float64) + 0.5) * (2.0 ** -53)
        rad = torch.sqrt(-2.0 * torch.log(u[..., 0]))
        th = (2.0 * math.pi) * u[..., 1]
        v = torch.stack((rad * torch.cos(th), rad * torch.sin(th)), dim=-1).reshape(len(rr), D)
        out[a:a + step] = v.to(torch.float32).to(torch.bfloat16)
    return out


def router_weight(cfg, device="cpu", seed: int = 0) -> torch.Tensor:
    return normal_bf16((cfg.n_experts, cfg.d_model), cfg.d_model ** -0.5, WR, 0,
                       seed, device)


def zipf_bias(cfg, seed: int = 0) -> torch.Tensor:
    """[E] fp32: 1.5 ln(w_rho), w_rho = rho^-1.1 / H, over a seeded permutation."""
    E = cfg.n_experts
    keys = uniform_bits(stream_state(seed, PERM, 0), 0, E, "cpu")
    perm = torch.argsort(keys, stable=True)          # perm[rho-1] = expert
    rho = torch.arange(1, E + 1, dtype=torch.float64)
    w = rho ** -1.1
    w = w / w.sum()
    b = torch.empty(E, dtype=torch.float64)
    b[perm] = 1.5 * torch.log(w)
    return b.to(torch.float32)


def longctx_bias(cfg, shard: int, seed: int = 0) -> torch.Tensor:
    """[n_chunks, E] fp32: per-shard N(0,1.5^2) + per-4096-chunk N(0,0.5^2)."""
    E = cfg.n_experts
    nch = (cfg.T + 4095) // 4096
    seq = normal_f64((E,), 1.5, BSEQ, shard, seed)
    chunk = normal_f64((nch, E), 0.5, BCHUNK, shard, seed)
    return (seq.to(torch.float32)[None, :] + chunk.to(torch.float32))


def logits(cfg, shard: int, x: torch.Tensor, w_r: torch.Tensor,
           seed: int = 0) -> torch.Tensor:
    """fp32 router logits of one shard: x.W_r^T in fp32 plus the workload's bias."""
    lg = x.float() @ w_r.float().t()
    if cfg.routing == "zipf":
        lg += zipf_bias(cfg, seed).to(lg.device)[None, :]
    elif cfg.routing == "longctx":
        b = longctx_bias(cfg, shard, seed).to(lg.device)
        tok_chunk = torch.arange(cfg.T, device=lg.device) // 4096
        lg += b[tok_chunk]
    return lg.contiguous()


def latent_down(cfg, device="cpu", seed: int = 0) -> torch.Tensor:
    return normal_bf16((cfg.latent, cfg.d_model), cfg.d_model ** -0.5, WLD, 0,
                       seed, device)


def latent_up(cfg, device="cpu", seed: int = 0) -> torch.Tensor:
    return normal_bf16((cfg.d_model, cfg.latent), cfg.latent ** -0.5, WLU, 0,
                       seed, device)


def expert(cfg, e: int, device="cpu", seed: int = 0):
    """(W_g [F,L], W_u [F,L], W_d [L,F]) of global expert e."""
    F, L = cfg.d_ff, cfg.latent
    return (normal_bf16((F, L), L ** -0.5, WG, e, seed, device),
            normal_bf16((F, L), L ** -0.5, WU, e, seed, device),
            normal_bf16((L, F), F ** -0.5, WD, e, seed, device))


def rank_experts(cfg, rank: int, device="cpu", seed: int = 0):
    """Stacked weights of the experts hosted by ``rank``: [E_l, ...] each."""
    El = cfg.experts_per_rank
    ws = [expert(cfg, rank * El + j, device, seed) for j in range(El)]
    return tuple(torch.stack([w[i] for w in ws]).contiguous() for i in range(3))


def shared(cfg, device="cpu", seed: int = 0):
    """(W_sg [S,Fs,D], W_su [S,Fs,D], W_sd [S,D,Fs])."""
    S, Fs, D = cfg.n_shared, cfg.d_ff_shared, cfg.d_model
    if S == 0:
        e = torch.empty((0, Fs, D), dtype=torch.bfloat16, device=device)
        return e, e.clone(), torch.empty((0, D, Fs), dtype=torch.bfloat16, device=device)
    g = torch.stack([normal_bf16((Fs, D), D ** -0.5, WSG, s, seed, device) for s in range(S)])
    u = torch.stack([normal_bf16((Fs, D), D ** -0.5, WSU, s, seed, device) for s in range(S)])
    d = torch.stack([normal_bf16((D, Fs), Fs ** -0.5, WSD, s, seed, device) for s in range(S)])
    return g.contiguous(), u.contiguous(), d.contiguous()


def payload_rows(n: int, width: int, idx: int, device="cpu", seed: int = 0):
    """bf16 N(0,1) rows used as stand-in payloads in stage-level tests."""
    return normal_bf16((n, width), 1.0, PAYLOAD, idx, seed, device)
