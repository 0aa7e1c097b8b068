"""Pins of the oracle's SiTU-GLU and router.

SiTU: "Kimi K3 engine (c/kimi_k3.c)", "Architecture notes":
h = 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25). The identities below hold for that
formula only: a swapped constant, a sigmoid of -g or a dropped factor breaks
one of them.

Router: same section (sigmoid scores, score-correction bias, top-16 on the
biased scores, weights = raw scores renormalised) and "kimi-k3-in-c" README,
"Three invariants" (the bias steers selection only).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import read_table

GU = [(-30.0, 7.0), (-3.0, -2.0), (-0.5, 40.0), (0.25, 0.1), (1.0, -1.0), (2.5, 12.0), (9.0, 100.0)]


def test_situ_vec_is_the_scalar_formula_elementwise():
    g = synth.normal_f32(13, 500, 6.0, key=1)
    u = synth.normal_f32(13, 500, 40.0, key=2)
    h = oracle.situ_vec(g, u)
    want = np.array([np.float32(oracle.situ(float(a), float(b))) for a, b in zip(g, u)])
    assert np.array_equal(h, want)


@pytest.mark.parametrize("g,u", GU)
def test_situ_odd_even_parts(g, u):
    hp = oracle.situ(g, u)
    hm = oracle.situ(-g, u)
    # sigmoid(g) + sigmoid(-g) = 1  =>  h(g) - h(-g) = 100 tanh(g/4) tanh(u/25)
    assert math.isclose(hp - hm, 100 * math.tanh(g / 4) * math.tanh(u / 25), rel_tol=1e-13, abs_tol=1e-300)
    # sigmoid(g) - sigmoid(-g) = tanh(g/2)  =>  h(g) + h(-g) = 100 tanh(g/4) tanh(g/2) tanh(u/25)
    assert math.isclose(hp + hm, 100 * math.tanh(g / 4) * math.tanh(g / 2) * math.tanh(u / 25),
                        rel_tol=1e-12, abs_tol=1e-13)
    # odd in u
    assert oracle.situ(g, -u) == -hp


def test_situ_zeros_and_limits():
    assert oracle.situ(0.0, 3.0) == 0.0
    assert oracle.situ(3.0, 0.0) == 0.0
    # g -> +inf: 4 * 1 * 1 * 25 tanh(u/25); g, u -> +inf: 100
    assert math.isclose(oracle.situ(200.0, 25.0), 100 * math.tanh(1.0), rel_tol=1e-15)
    assert oracle.situ(1e3, 1e4) == 100.0
    # g -> -inf: the sigmoid kills it
    assert abs(oracle.situ(-200.0, 25.0)) < 1e-80


def test_bias_fixture():
    rows = read_table("route_bias_fixture.txt")
    bias = np.array([0, 0, 0, 0, 0, 0, 0.5, 0.9], np.float32)
    logits, want_b, want_u, want_w = [], [], [], []
    for r in rows:
        a, b, c, d = r.split("|")
        logits.append([float(v) for v in a.split()])
        want_b.append([int(v) for v in b.split()])
        want_u.append([int(v) for v in c.split()])
        want_w.append([float(v) for v in d.split()])
    logits = np.array(logits)
    idx, wts, _ = oracle.route_select(logits, bias, 2)
    assert np.array_equal(idx, np.array(want_b))
    # wts are float32: within half an ulp of the 9-digit values
    assert np.allclose(wts, np.array(want_w), rtol=0, atol=6e-8)
    idx0, _, _ = oracle.route_select(logits, np.zeros(8, np.float32), 2)
    assert np.array_equal(idx0, np.array(want_u))
    # the bias reorders the selection on five of the six rows
    assert sum(not np.array_equal(a, b) for a, b in zip(idx, idx0)) == 5


def test_zero_bias_selects_top_logits_and_weights_ignore_bias():
    W, b = synth.router(21, 896, 256, 0.1)
    x = synth.activations(21, 8, 256)
    lg = oracle.route_logits(x, W)
    idx0, w0, _ = oracle.route_select(lg, np.zeros(896, np.float32), 16)
    for t in range(8):
        order = np.lexsort((np.arange(896), -lg[t]))[:16]
        assert np.array_equal(idx0[t], order)
    assert np.allclose(w0.sum(1), 1.0, atol=1e-6)
    idx, w, bsel = oracle.route_select(lg, b, 16)
    # descending biased score
    assert np.all(np.diff(bsel, axis=1) <= 0)
    # weights: the unbiased sigmoid scores of the selected set, renormalised
    sig = 1.0 / (1.0 + np.exp(-lg))
    for t in range(8):
        sc = sig[t, idx[t]]
        assert np.allclose(w[t], sc / sc.sum(), rtol=1e-6, atol=0)
        # the same selection with another bias gives the same weights
    idx2, w2, _ = oracle.route_select(lg, b * 0, 16)
    same = [t for t in range(8) if set(idx2[t]) == set(idx[t])]
    for t in same:
        assert np.allclose(np.sort(w2[t]), np.sort(w[t]), rtol=1e-7)


def test_logits_fixed_order_and_exactness():
    rng = np.random.default_rng(5)
    # integer inputs: every partial sum is exact, so any order gives the same value
    W = rng.integers(-50, 51, size=(30, 77)).astype(np.float32)
    x = rng.integers(-50, 51, size=(3, 77)).astype(np.float32)
    lg = oracle.route_logits(x, W)
    assert np.array_equal(lg, x.astype(np.float64) @ W.astype(np.float64).T)
    # random floats: products exact in double, so within a few ulp of the exact sum
    W, _ = synth.router(9, 64, 3584, 0.1)
    x = synth.activations(9, 2, 3584)
    lg = oracle.route_logits(x, W)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.all(np.abs(lg - ref) <= 1e-13 * (np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T))
    # exactly rounded reference (math.fsum of the exact double products): the
    # in-order double sum stays within n*2^-53 of sum|w x| (the standard bound)
    import math
    for t in range(2):
        for e in range(0, 64, 7):
            exact = math.fsum((x[t].astype(np.float64) * W[e].astype(np.float64)).tolist())
            ab = float(np.abs(x[t].astype(np.float64)) @ np.abs(W[e].astype(np.float64)))
            assert abs(lg[t, e] - exact) <= 3584 * 2.0 ** -53 * ab
    # the documented order (index order, one double accumulator), on a case
    # where the order decides the result: 2^53 + 1 rounds back to 2^53 (ties to
    # even), so 1 + 2^53 - 2^53 gives 0 in index order while the exact sum is 1
    w = np.array([1.0, 2.0 ** 53, -(2.0 ** 53), 1.0], np.float32)
    xv = np.ones((1, 4), np.float32)
    assert oracle.route_logits(xv, w[None, :])[0, 0] == 1.0  # 0 + 1 at the end
    assert oracle.route_logits(xv[:, :3], w[None, :3])[0, 0] == 0.0


# ---- K3_TOPP ("Kimi K3 engine (c/kimi_k3.c)", "Streaming design" and its table of
# environment variables): keep the routed experts up to cumulative weight p,
# drop the low-weight tail of the top-k, renormalise; p = 0 is off.

def _logits_for(scores):
    """Logits whose sigmoid is the given scores."""
    s = np.asarray(scores, np.float64)
    return np.log(s / (1.0 - s))[None, :]


def _topp(logits, top_k, p, bias=None):
    bias = np.zeros(logits.shape[1], np.float32) if bias is None else bias
    idx, wts, _ = oracle.route_select(logits, bias, top_k)
    return oracle.route_topp(idx, wts, logits, p)


def test_topp_hand_example():
    # scores 0.8, 0.6, 0.4, 0.2 selected (top 4 of 6): weights 0.4, 0.3, 0.2, 0.1
    lg = _logits_for([0.8, 0.6, 0.4, 0.2, 0.1, 0.05])
    idx, wts = _topp(lg, 4, 0.5)  # 0.4 taken; 0.3 taken (0.4 < 0.5); 0.2 not (0.7 >= 0.5)
    assert np.array_equal(idx[0], [0, 1, -1, -1])
    assert np.allclose(wts[0], [4 / 7, 3 / 7, 0, 0], rtol=0, atol=1e-7)
    idx, wts = _topp(lg, 4, 0.85)  # 0.9 before the last weight: it is dropped
    assert np.array_equal(idx[0], [0, 1, 2, -1])
    assert np.allclose(wts[0], [0.8 / 1.8, 0.6 / 1.8, 0.4 / 1.8, 0], rtol=0, atol=1e-7)
    for p in (0.95, 1.0, 0.0):  # everything kept: the weights are the top-k ones
        idx, wts = _topp(lg, 4, p)
        assert np.array_equal(idx[0], [0, 1, 2, 3])
        assert np.allclose(wts[0], [0.4, 0.3, 0.2, 0.1], rtol=0, atol=1e-7)


def test_topp_boundary_keeps_the_expert_that_reaches_p():
    lg = _logits_for([0.8, 0.6, 0.4, 0.2, 0.1, 0.05])
    w0 = 0.8 / (0.8 + 0.6 + 0.4 + 0.2)
    idx, _ = _topp(lg, 4, w0 - 1e-9)  # p reached by the first expert alone
    assert np.array_equal(idx[0], [0, -1, -1, -1])
    idx, _ = _topp(lg, 4, w0 + 1e-9)  # the second expert is needed to reach p
    assert np.array_equal(idx[0], [0, 1, -1, -1])


def test_topp_order_is_by_weight_with_ties_in_route_order():
    # experts 0 and 1 have equal scores (equal weights); the bias puts expert 1
    # ahead of expert 0 in the route, and expert 2 (largest weight) behind both
    lg = _logits_for([0.3, 0.3, 0.4, 0.01])
    bias = np.array([0.0, 0.05, -0.2, 0.0], np.float32)
    idx, wts, _ = oracle.route_select(lg, bias, 3)
    assert np.array_equal(idx[0], [1, 0, 2])  # route order: biased score
    t_idx, t_wts = oracle.route_topp(idx, wts, lg, 0.4 + 1e-9)
    # by weight: expert 2 (0.4) first; then the tie 1, 0 in route order: 1 is taken
    assert np.array_equal(t_idx[0], [1, -1, 2])
    assert np.allclose(t_wts[0], [0.3 / 0.7, 0, 0.4 / 0.7], rtol=0, atol=1e-7)


def test_topp_invariants_on_random_routings():
    W, b = synth.router(33, 896, 512, 0.1)
    x = synth.activations(33, 40, 512)
    lg = oracle.route_logits(x, W)
    idx, wts, _ = oracle.route_select(lg, b, 16)
    sig = 1.0 / (1.0 + np.exp(-lg))
    rng = np.random.default_rng(33)
    for p in rng.uniform(0.05, 0.99, 6):
        t_idx, t_wts = oracle.route_topp(idx, wts, lg, p)
        for t in range(x.shape[0]):
            w = sig[t, idx[t]] / sig[t, idx[t]].sum()
            kept = t_idx[t] >= 0
            assert np.all(t_idx[t][kept] == idx[t][kept])  # kept entries stay in place
            assert np.all(t_wts[t][~kept] == 0)
            # the kept set is a prefix of the weight order (ties: route order) ...
            order = np.lexsort((np.arange(16), -w))
            n = kept.sum()
            assert set(order[:n]) == set(np.flatnonzero(kept))
            # ... the shortest one that reaches p
            cum = np.cumsum(w[order])
            assert n == 16 or cum[n - 1] >= p - 1e-12
            assert n == 1 or cum[n - 2] < p + 1e-12
            # renormalised over the kept experts
            assert abs(t_wts[t][kept].sum() - 1.0) < 1e-6
            assert np.allclose(t_wts[t][kept], w[kept] / w[kept].sum(), rtol=2e-7, atol=0)


def test_layer_skips_dropped_pairs():
    # a dropped pair (idx -1) adds nothing: the same as a kept expert with weight 0
    from tests.helpers import ExpertSource
    E, latent, inter = 5, 64, 64
    src = ExpertSource(35, latent, inter, 120, 123, 0.0)
    ex = {e: src(e) for e in range(E)}
    x = synth.activations(35, 3, latent)
    idx = np.array([[0, -1, 2], [-1, -1, 4], [1, 3, -1]], np.int32)
    wts = np.array([[0.6, 0.0, 0.4], [0.0, 0.0, 1.0], [0.5, 0.5, 0.0]], np.float32)
    y = oracle.moe_layer(x, idx, wts, ex, E)
    idx0 = np.where(idx < 0, 0, idx).astype(np.int32)
    y0 = oracle.moe_layer(x, idx0, wts, ex, E)
    assert np.array_equal(y, y0)
