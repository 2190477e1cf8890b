"""GPU parity of quantile balancing ("从玩具到前沿:训练一个真正的大模型,到底难在哪里",
section 四 and appendix A.2): routing on logits + bias, per-expert selection
counts, and the bias from a window of counts.  Routing choices, counts and
the bias are compared bit for bit (the bias is computed in double on both
sides and rounded once to fp32); gates within the router's tolerance."""
import numpy as np
import pytest
import torch

import gpucase as gc
from synth import configs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dispatch_softmax_top_amd as m
    m.lib()
    return m


def _route_biased(moe, lg, bias, k):
    T = lg.shape[0]
    topk = torch.full((T, k), -9, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route_biased(gc.dev(lg), gc.dev(bias), k, topk, gates)
    torch.cuda.synchronize()
    return gc.host(topk), gc.host(gates)


@pytest.mark.parametrize("T,E,k,scale", [(601, 48, 8, 0.3), (4096, 384, 8, 1.0),
                                         (257, 1024, 32, 0.5), (1, 8, 8, 2.0)])
def test_route_biased(moe, orc, T, E, k, scale):
    rng = np.random.default_rng(T + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = (scale * rng.standard_normal(E)).astype(np.float32)
    topk, gates = _route_biased(moe, lg, bias, k)
    ot, og = orc.route_biased(lg, bias, k)
    assert np.array_equal(topk, ot)
    np.testing.assert_allclose(gates, og, rtol=2e-5, atol=1e-12)


def test_route_biased_ties_and_null_bias(moe, orc):
    rng = np.random.default_rng(1)
    lg = rng.integers(-2, 3, (300, 64)).astype(np.float32)       # heavy ties
    bias = rng.integers(-1, 2, 64).astype(np.float32)
    topk, _ = _route_biased(moe, lg, bias, 8)
    assert np.array_equal(topk, orc.route_biased(lg, bias, 8)[0])
    t2 = torch.empty(300, 8, dtype=torch.int32, device="cuda")
    g2 = torch.empty(300, 8, device="cuda")
    moe.moe_route_biased(gc.dev(lg), None, 8, t2, g2)             # NULL bias = plain router
    torch.cuda.synchronize()
    assert np.array_equal(gc.host(t2), orc.route(lg, 8)[0])


@pytest.mark.parametrize("T,k,E", [(4096, 8, 384), (65536, 8, 384), (601, 8, 48), (1, 1, 1),
                                   (5000, 32, 1024)])
def test_expert_counts(moe, orc, T, k, E):
    rng = np.random.default_rng(T * k)
    topk = rng.integers(-1, E + 1, (T, k)).astype(np.int32)      # -1 and E are not experts
    counts = torch.full((E,), -5, dtype=torch.int32, device="cuda")
    moe.moe_expert_counts(gc.dev(topk), E, counts)
    torch.cuda.synchronize()
    assert np.array_equal(gc.host(counts), orc.expert_counts(topk, E))


@pytest.mark.parametrize("n,E,alpha", [(1, 4, 0.5), (8, 384, 1e-3), (3, 48, 40.0),
                                       (16, 1024, 2.5)])
def test_balance_bias(moe, orc, n, E, alpha):
    rng = np.random.default_rng(n * E)
    window = rng.integers(0, 4096, (n, E)).astype(np.int32)
    window[0, : E // 3] = 0
    bias = torch.full((E,), 7.0, device="cuda")
    moe.moe_balance_bias(gc.dev(window), alpha, bias)
    torch.cuda.synchronize()
    ref = orc.balance_bias(window, alpha)
    assert np.array_equal(gc.host(bias).view(np.uint32), ref.view(np.uint32))
    zero = np.zeros((n, E), np.int32)                             # nothing chosen: no bias
    moe.moe_balance_bias(gc.dev(zero), alpha, bias)
    torch.cuda.synchronize()
    assert np.array_equal(gc.host(bias), orc.balance_bias(zero, alpha))


def test_balancing_loop_in_lockstep(moe, orc):
    """Route -> count -> bias, six batches of a skewed workload, GPU and oracle
    side by side from the same logits: every choice, count and bias agrees."""
    from dispatch_softmax_top_amd import share
    cfg = gc.skewed(gc.MID)
    E, k = cfg.n_experts, cfg.top_k
    bal = share.Balancer(E, window=4, alpha=40.0)
    o_bias, o_window, loads = np.zeros(E, np.float32), [], []
    snd = share.Sender(share.make_dims(cfg))
    for step in range(6):
        _, lg = gc.shard_inputs(cfg, step)
        snd.route(lg.cuda(), bias=bal.bias)
        bal.update(snd.topk)
        torch.cuda.synchronize()
        ot, _ = orc.route_biased(lg.numpy(), o_bias, k)
        assert np.array_equal(gc.host(snd.topk), ot), f"step {step}: choices differ"
        c = orc.expert_counts(ot, E)
        assert np.array_equal(gc.host(bal.counts[step % 4]), c), f"step {step}: counts differ"
        o_window = (o_window + [c])[-4:]
        o_bias = orc.balance_bias(np.array(o_window), 40.0)
        assert np.array_equal(gc.host(bal.bias).view(np.uint32), o_bias.view(np.uint32)), \
            f"step {step}: bias differs"
        loads.append(c.max() / c.mean())
    assert np.mean(loads[1:]) < loads[0]


def test_balance_errors(moe):
    t = torch.zeros(4, 8, dtype=torch.int32, device="cuda")
    c = torch.zeros(2000, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_expert_counts(t, 2000, c)                          # E > 1024
    b = torch.zeros(16, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_balance_bias(torch.zeros(0, 16, dtype=torch.int32, device="cuda"), 1.0, b)
    with pytest.raises(moe.MoeError):
        moe.moe_balance_bias(torch.zeros(2, 16, dtype=torch.int32, device="cuda"), float("nan"), b)


@pytest.mark.parametrize("with_bias", [False, True])
def test_route_renormalised_gates(moe, orc, with_bias):
    rng = np.random.default_rng(11)
    T, E, k = 4096, 384, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if with_bias else None
    topk = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gates = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route_biased(gc.dev(lg), None if bias is None else gc.dev(bias), k, topk, gates,
                         flags=moe.MOE_ROUTE_RENORM)
    torch.cuda.synchronize()
    ot, og = orc.route_ex(lg, k, bias=bias, renorm=True)
    assert np.array_equal(gc.host(topk), ot)
    np.testing.assert_allclose(gc.host(gates), og, rtol=2e-5, atol=1e-12)
