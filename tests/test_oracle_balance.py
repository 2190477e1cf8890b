"""Pins of the oracle's quantile balancing ("从玩具到前沿:训练一个真正的大模型,到底难在
哪里", section 四 and appendix A.2): selection counts, the bias
b_i = -alpha (f_i - 1/E) from a window of counts, and routing on the biased
logits.  Each is checked against something other than the oracle itself:
numpy's bincount and argsort, a hand-worked example, invariants of the
formula, and the property the pages give the method (routing tends to
uniform)."""
import numpy as np
import pytest


def test_counts_are_a_bincount(orc):
    rng = np.random.default_rng(3)
    E = 48
    topk = rng.integers(-2, E + 2, size=(300, 8)).astype(np.int32)  # some outside [0, E)
    valid = topk[(topk >= 0) & (topk < E)]
    assert np.array_equal(orc.expert_counts(topk, E), np.bincount(valid, minlength=E))


def test_bias_worked_example(orc):
    # E = 4, 8 choices: f = (6/8, 2/8, 0, 0), alpha = 1/2:
    # b = -1/2 (f - 1/4) = (-1/4, 0, 1/8, 1/8), exact in binary
    b = orc.balance_bias(np.array([[6, 2, 0, 0]]), 0.5)
    assert np.array_equal(b, np.array([-0.25, 0.0, 0.125, 0.125], np.float32))
    # the same selections spread over a window of three batches
    w = np.array([[1, 0, 0, 0], [3, 2, 0, 0], [2, 0, 0, 0]])
    assert np.array_equal(orc.balance_bias(w, 0.5), b)


def test_bias_invariants(orc):
    rng = np.random.default_rng(4)
    E = 384
    w = rng.integers(0, 500, size=(5, E)).astype(np.int32)
    b = orc.balance_bias(w, 0.7).astype(np.float64)
    H = w.sum(0).astype(np.float64)
    ref = -0.7 * (H / H.sum() - 1.0 / E)                      # the formula in numpy, fp64
    assert np.abs(b - ref).max() <= 1e-7 * np.abs(ref).max()
    assert abs(b.sum()) < 1e-6 * 0.7                          # frequencies sum to 1
    assert np.all(np.sign(b) == -np.sign(H / H.sum() - 1.0 / E))  # hot down, cold up
    assert np.array_equal(orc.balance_bias(3 * w, 0.7), orc.balance_bias(w, 0.7))  # scale-free
    assert np.array_equal(orc.balance_bias(np.full((2, E), 7), 0.7), np.zeros(E, np.float32))
    assert np.array_equal(orc.balance_bias(np.zeros((3, E), np.int32), 0.7),
                          np.zeros(E, np.float32))                # nothing chosen: no bias
    assert np.array_equal(orc.balance_bias(w, 0.0), np.zeros(E, np.float32) * -0.0)


def _brute_route(lb, k):
    order = np.lexsort((np.arange(lb.shape[1])[None, :].repeat(lb.shape[0], 0), -lb), axis=1)
    topk = order[:, :k].astype(np.int32)
    z = np.exp(lb.astype(np.float64) - lb.max(1, keepdims=True))
    g = np.take_along_axis(z / z.sum(1, keepdims=True), topk, 1)
    return topk, g


@pytest.mark.parametrize("integer_logits", [False, True])
def test_biased_route_is_route_on_fp32_sum(orc, integer_logits):
    rng = np.random.default_rng(5)
    T, E, k = 200, 48, 8
    if integer_logits:  # many ties, broken toward the lower index
        lg = rng.integers(-3, 3, size=(T, E)).astype(np.float32)
        bias = rng.integers(-1, 2, size=E).astype(np.float32)
    else:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        bias = (0.3 * rng.standard_normal(E)).astype(np.float32)
    lb = lg + bias[None, :]                      # numpy float32 add: one fp32 rounding
    topk, gates = orc.route_biased(lg, bias, k)
    ref_k, ref_g = _brute_route(lb, k)
    assert np.array_equal(topk, ref_k)
    assert np.abs(gates - ref_g).max() <= 1e-6 * ref_g.max()


def test_biased_route_can_exclude_an_expert(orc):
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((100, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    bias[3] = -1e4
    topk, _ = orc.route_biased(lg, bias, 4)
    assert not (topk == 3).any()
    assert (orc.route(lg, 4)[0] == 3).any()


def test_balancing_evens_out_skewed_routing(orc):
    """The method's purpose: with the bias of the previous batches fed back,
    the most-chosen expert's load falls toward the mean (skew of Zipf-like
    expert preferences, as in the skewed workloads)."""
    rng = np.random.default_rng(0)
    E, T, k, steps = 48, 512, 8, 12
    w = np.arange(1, E + 1) ** -1.1
    skew = np.zeros(E, np.float32)
    skew[rng.permutation(E)] = 1.5 * np.log(w / w.sum())
    ratio = {}
    for alpha in (0.0, 40.0):
        bias, window, r = np.zeros(E, np.float32), [], []
        for _ in range(steps):
            lg = (rng.standard_normal((T, E)) + skew).astype(np.float32)
            c = orc.expert_counts(orc.route_biased(lg, bias, k)[0], E)
            window = (window + [c])[-4:]
            bias = orc.balance_bias(np.array(window), alpha)
            r.append(c.max() / c.mean())
        ratio[alpha] = np.mean(r[1:])
    assert ratio[0.0] > 5.5                  # unbalanced: the hottest expert takes every token
    assert ratio[40.0] < 0.85 * ratio[0.0]


def test_renormalised_gates_are_softmax_over_the_chosen(orc):
    """Gate variant: with renormalisation the k gates of a token are the
    softmax over its k chosen logits (closed form), sum to 1, and keep the
    ratios of the full-softmax gates; the choices do not change."""
    rng = np.random.default_rng(8)
    T, E, k = 150, 48, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.2 * rng.standard_normal(E)).astype(np.float32)
    for b in (None, bias):
        t0, g0 = orc.route_ex(lg, k, bias=b)
        t1, g1 = orc.route_ex(lg, k, bias=b, renorm=True)
        assert np.array_equal(t0, t1)
        lb = lg if b is None else lg + b[None, :]
        chosen = np.take_along_axis(lb, t1, 1).astype(np.float64)
        z = np.exp(chosen - chosen.max(1, keepdims=True))
        assert np.abs(g1 - z / z.sum(1, keepdims=True)).max() < 1e-7
        assert np.abs(g1.astype(np.float64).sum(1) - 1).max() < 1e-6
        np.testing.assert_allclose(g1 / g1[:, :1], g0 / g0[:, :1], rtol=1e-6)
    assert np.array_equal(orc.route_ex(lg, k)[1], orc.route(lg, k)[1])
    assert np.array_equal(orc.route_ex(lg, k, bias=bias)[1], orc.route_biased(lg, bias, k)[1])
