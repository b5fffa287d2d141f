"""Pins for the fp64 oracle: closed forms, identities, special cases and
hand-worked examples that fix what the method computes independently of the
oracle's own code.

Sources are on "The Hedgehog & the Porcupine: Expressive Linear Attentions
with Softmax Mimicry": Eq. 2 and its running-sum form (sections 2 and 3.4,
"Complexity Analysis"), the Hedgehog map (section 3.4, "The Hedgehog MLP
Feature Map", Choices 1-3) and the degree-2 Taylor map (section 3.4, "The
Taylor Exponential as a Bridge Result").

Each pin is chosen so that a plausible slip in the oracle fails at least one:
  - wrong causal boundary (j < i instead of j <= i): first-row, prefix-mean,
    worked examples;
  - W transposed or a bias dropped / not negated: cosh identity, worked
    examples with bias, identity-init feature map;
  - missing 1/sqrt(2) or a missing Taylor term: Taylor closed form and the
    Taylor worked examples;
  - S transposed or a wrong index in the read-out: quadratic form vs running
    sums, convex-hull bound;
  - state not carried or double counted: split-resume, decode chain;
  - distillation loss (Eq. 4, section 3.4 "The Attention Weight Distillation
    Loss"): a key beyond the causal boundary or a wrong normaliser (first-query
    loss, uniform cases), a missing 1/sqrt(d) or a misplaced softmax (two-key
    logistic case), a loss below the target's entropy (Gibbs inequality), and
    the Taylor kernel's agreement with exp at small scores.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HH, TAY = oracle.MAP_HEDGEHOG, oracle.MAP_TAYLOR2
MAPS = {"hedgehog": HH, "taylor2": TAY}


def _val(s):
    """Evaluate the small expressions used in the golden fixtures."""
    if isinstance(s, (int, float)):
        return float(s)
    s = s.strip()
    if s.startswith("e^"):
        return math.exp(_val(s[2:]))
    if s == "ln2":
        return math.log(2.0)
    if s == "-ln2":
        return -math.log(2.0)
    if s.endswith("/sqrt2"):
        return _val(s[: -len("/sqrt2")]) / math.sqrt(2.0)
    if "/" in s:
        a, b = s.split("/")
        return float(a) / float(b)
    return float(s)


def _vals(lst):
    return np.array([_val(x) for x in lst], dtype=np.float64)


def _rand_case(rng, map_, B, H, N, d, wscale=0.5, bscale=0.2, xscale=1.0):
    q = rng.standard_normal((B, H, N, d)) * xscale
    k = rng.standard_normal((B, H, N, d)) * xscale
    v = rng.standard_normal((B, H, N, d))
    if map_ == HH:
        W = rng.standard_normal((H, d, d)) * wscale
        b = rng.standard_normal((H, d)) * bscale
    else:
        W, b = None, None
    return q, k, v, W, b


# ---------------------------------------------------------------- golden ----

def test_golden_feature_dims():
    g = json.load(open(os.path.join(GOLDEN, "taylor_feature_dim.json")))
    for c in g["cases"]:
        assert oracle.feature_dim(MAPS[c["map"]], c["d"]) == c["feature_dim"]


def test_golden_worked_examples():
    g = json.load(open(os.path.join(GOLDEN, "worked_examples.json")))
    for c in g["cases"]:
        m = MAPS[c["map"]]
        d = c["d"]
        N = len(c["q"])
        q = _vals(c["q"]).reshape(1, 1, N, d)
        k = _vals(c["k"]).reshape(1, 1, N, d)
        v = _vals(c["v"]).reshape(1, 1, N, d)
        W = np.array(c["W"], np.float64).reshape(1, d, d) if "W" in c else None
        b = _vals(c["b"]).reshape(1, d) if "b" in c else None
        y = oracle.causal(m, q, k, v, W, b)
        np.testing.assert_allclose(y.ravel(), _vals(c["causal_y"]), rtol=1e-13, atol=0, err_msg=c["name"])
        yq = oracle.quadratic(m, q, k, v, W, b, causal=True)
        np.testing.assert_allclose(yq.ravel(), _vals(c["causal_y"]), rtol=1e-13, atol=0, err_msg=c["name"])
        if "bidir_y" in c:
            yb = oracle.bidir(m, q, k, v, W, b)
            np.testing.assert_allclose(yb.ravel(), _vals(c["bidir_y"]), rtol=1e-13, err_msg=c["name"])
    for f in g["featuremaps"]:
        m = MAPS[f["map"]]
        d = f["d"]
        x = _vals(f["x"]).reshape(1, 1, 1, d)
        W = np.array(f["W"], np.float64).reshape(1, d, d) if "W" in f else None
        b = _vals(f["b"]).reshape(1, d) if "b" in f else None
        phi = oracle.featuremap(m, x, W, b)
        np.testing.assert_allclose(phi.ravel(), _vals(f["phi"]), rtol=1e-14, err_msg=f["name"])


# ------------------------------------------------------ closed forms ----

def test_taylor_kernel_closed_form():
    # phi(q).phi(k) = 1 + q.k + (q.k)^2 / 2 exactly (up to rounding)
    rng = np.random.default_rng(11)
    for d in (1, 2, 4, 16):
        x = rng.standard_normal((1, 1, 64, d))
        phi = oracle.featuremap(TAY, x)[0, 0]
        for i in range(0, 64, 2):
            s = float(x[0, 0, i] @ x[0, 0, i + 1])
            assert phi[i] @ phi[i + 1] == pytest.approx(1 + s + s * s / 2, rel=1e-13, abs=1e-13)


def test_hedgehog_kernel_cosh_identity():
    # phi(q).phi(k) = sum_l e^{w_l.q+b_l} e^{w_l.k+b_l} + e^{-w_l.q-b_l} e^{-w_l.k-b_l}
    #              = 2 sum_l cosh(w_l.(q + k) + 2 b_l),  w_l = l-th row of W
    rng = np.random.default_rng(12)
    for d in (1, 2, 4, 16):
        W = rng.standard_normal((1, d, d)) * 0.4
        b = rng.standard_normal((1, d)) * 0.3
        x = rng.standard_normal((1, 1, 32, d))
        phi = oracle.featuremap(HH, x, W, b)[0, 0]
        for i in range(0, 32, 2):
            s = x[0, 0, i] + x[0, 0, i + 1]
            want = 2.0 * sum(math.cosh(float(W[0, l] @ s) + 2.0 * b[0, l]) for l in range(d))
            assert phi[i] @ phi[i + 1] == pytest.approx(want, rel=1e-13)
        if d > 1:  # the identity tells rows from columns: W^T must not satisfy it
            s = x[0, 0, 0] + x[0, 0, 1]
            wrong = 2.0 * sum(math.cosh(float(W[0, :, l] @ s) + 2.0 * b[0, l]) for l in range(d))
            assert abs(phi[0] @ phi[1] - wrong) > 1e-6 * abs(wrong)


def test_identity_init_feature_map():
    rng = np.random.default_rng(13)
    d = 8
    x = rng.standard_normal((1, 1, 5, d))
    W = np.eye(d)[None]
    b = np.zeros((1, d))
    phi = oracle.featuremap(HH, x, W, b)[0, 0]
    np.testing.assert_allclose(phi, np.concatenate([np.exp(x[0, 0]), np.exp(-x[0, 0])], axis=1), rtol=1e-15)


# ------------------------------------------------ equivalent forms ----

@pytest.mark.parametrize("map_", [HH, TAY])
@pytest.mark.parametrize("d", [1, 2, 4, 16])
def test_running_sums_equal_quadratic_form(map_, d):
    rng = np.random.default_rng(100 + d + 7 * map_)
    N = 33 if d < 16 else 20
    q, k, v, W, b = _rand_case(rng, map_, 2, 2, N, d, xscale=0.5 if map_ == TAY else 1.0)
    y = oracle.causal(map_, q, k, v, W, b)
    yq = oracle.quadratic(map_, q, k, v, W, b, causal=True)
    np.testing.assert_allclose(y, yq, rtol=1e-11, atol=1e-12)
    yb = oracle.bidir(map_, q, k, v, W, b)
    yqb = oracle.quadratic(map_, q, k, v, W, b, causal=False)
    np.testing.assert_allclose(yb, yqb, rtol=1e-11, atol=1e-12)
    # bidirectional last row sees the same keys as the causal last row
    np.testing.assert_allclose(yb[:, :, -1], y[:, :, -1], rtol=1e-11, atol=1e-12)
    # selected rows of the quadratic form equal the full form
    rows = [0, N // 2, N - 1]
    np.testing.assert_allclose(oracle.quadratic(map_, q, k, v, W, b, causal=True, rows=rows),
                               yq[:, :, rows], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("map_", [HH, TAY])
def test_split_forward_resumes_from_state(map_):
    rng = np.random.default_rng(21 + map_)
    d, N, N1 = 4, 40, 17
    q, k, v, W, b = _rand_case(rng, map_, 1, 3, N, d)
    y, S, z = oracle.causal(map_, q, k, v, W, b, want_state=True)
    y1, S1, z1 = oracle.causal(map_, q[:, :, :N1], k[:, :, :N1], v[:, :, :N1], W, b, want_state=True)
    y2, S2, z2 = oracle.causal(map_, q[:, :, N1:], k[:, :, N1:], v[:, :, N1:], W, b, S0=S1, z0=z1,
                               want_state=True)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=2), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z, rtol=1e-12)
    # the final state is the plain sum over all keys of phi(k_j) v_j^T and phi(k_j)
    phik = oracle.featuremap(map_, k, W, b)
    np.testing.assert_allclose(S, np.einsum("bhnf,bhnc->bhfc", phik, v), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, phik.sum(axis=2), rtol=1e-12)


@pytest.mark.parametrize("map_", [HH, TAY])
def test_decode_chain_equals_forward(map_):
    rng = np.random.default_rng(31 + map_)
    d, N = 4, 12
    q, k, v, W, b = _rand_case(rng, map_, 2, 2, N, d)
    y, S_end, z_end = oracle.causal(map_, q, k, v, W, b, want_state=True)
    dp = oracle.feature_dim(map_, d)
    S = np.zeros((2, 2, dp, d))
    z = np.zeros((2, 2, dp))
    for i in range(N):
        yi, S, z = oracle.decode_step(map_, q[:, :, i], k[:, :, i], v[:, :, i], W, b, S, z)
        np.testing.assert_allclose(yi, y[:, :, i], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, S_end, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z_end, rtol=1e-12)


# ------------------------------------------------- special cases ----

def test_zero_map_gives_prefix_and_global_means():
    # W = 0, b = 0: every feature is e^0 = 1, all weights equal.
    rng = np.random.default_rng(41)
    d, N = 16, 50
    q, k, v, _, _ = _rand_case(rng, HH, 1, 2, N, d)
    W = np.zeros((2, d, d))
    b = np.zeros((2, d))
    y = oracle.causal(HH, q, k, v, W, b)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(y, prefix_mean, rtol=1e-13, atol=1e-14)
    yb = oracle.bidir(HH, q, k, v, W, b)
    np.testing.assert_allclose(yb, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), rtol=1e-13,
                               atol=1e-14)


def test_taylor_zero_query_gives_prefix_mean():
    # q = 0: kernel 1 + 0 + 0 = 1 for every key.
    rng = np.random.default_rng(42)
    d, N = 16, 30
    _, k, v, _, _ = _rand_case(rng, TAY, 1, 1, N, d)
    q = np.zeros_like(k)
    y = oracle.causal(TAY, q, k, v)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(y, prefix_mean, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("map_", [HH, TAY])
def test_first_row_and_convex_hull(map_):
    rng = np.random.default_rng(51 + map_)
    d, N = 8, 40
    q, k, v, W, b = _rand_case(rng, map_, 2, 2, N, d)
    y = oracle.causal(map_, q, k, v, W, b)
    np.testing.assert_allclose(y[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-15)
    lo = np.minimum.accumulate(v, axis=2)
    hi = np.maximum.accumulate(v, axis=2)
    assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)
    yb = oracle.bidir(map_, q, k, v, W, b)
    assert np.all(yb >= v.min(axis=2, keepdims=True) - 1e-12)
    assert np.all(yb <= v.max(axis=2, keepdims=True) + 1e-12)


def test_single_key_weight_is_kernel_value():
    # With two keys, y_1 = (a0 v0 + a1 v1) / (a0 + a1); a_j from the Taylor closed form.
    rng = np.random.default_rng(61)
    d = 3
    q = rng.standard_normal((1, 1, 2, d)) * 0.7
    k = rng.standard_normal((1, 1, 2, d)) * 0.7
    v = rng.standard_normal((1, 1, 2, d))
    y = oracle.causal(TAY, q, k, v)
    s0 = float(q[0, 0, 1] @ k[0, 0, 0])
    s1 = float(q[0, 0, 1] @ k[0, 0, 1])
    a0, a1 = 1 + s0 + s0 * s0 / 2, 1 + s1 + s1 * s1 / 2
    np.testing.assert_allclose(y[0, 0, 1], (a0 * v[0, 0, 0] + a1 * v[0, 0, 1]) / (a0 + a1), rtol=1e-13)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(71)
    q, k, v, W, b = _rand_case(rng, HH, 2, 3, 25, 8)
    y1 = oracle.causal(HH, q, k, v, W, b, nthreads=1)
    y8 = oracle.causal(HH, q, k, v, W, b, nthreads=8)
    assert np.array_equal(y1, y8)


@pytest.mark.parametrize("map_", [HH, TAY])
def test_prefix_state_equals_running_sums(map_):
    rng = np.random.default_rng(81 + map_)
    q, k, v, W, b = _rand_case(rng, map_, 2, 3, 30, 4)
    _, S, z = oracle.causal(map_, q, k, v, W, b, want_state=True)
    S2, z2 = oracle.prefix_state(map_, k, v, W, b)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z, rtol=1e-12)


# ---- attention-weight distillation loss (Eq. 4 of the walkthrough's section 3.4) ----

def _softmax_rows(logits):
    from scipy.special import softmax
    return softmax(logits, axis=-1)


@pytest.mark.parametrize("map_,d", [(HH, 8), (TAY, 4)])
def test_distill_first_query_loss_is_zero(map_, d):
    # one key: both distributions put all weight on it
    rng = np.random.default_rng(61)
    q = rng.standard_normal((2, 3, 20, d))
    k = rng.standard_normal((2, 3, 20, d))
    W = rng.standard_normal((3, d, d)) / math.sqrt(d)
    L = oracle.distill_loss(map_, q, k, W, None)
    assert np.all(np.abs(L[:, :, 0]) < 1e-12)


def test_distill_uniform_cases_give_log_count():
    # q = 0 makes the softmax uniform; W = b = 0 (Hedgehog) or q = 0 (Taylor: phi(0).phi(k) = 1)
    # makes the linear weights uniform too: L_i = log(i + 1)
    rng = np.random.default_rng(62)
    N, d = 40, 8
    k = rng.standard_normal((1, 2, N, d))
    q0 = np.zeros((1, 2, N, d))
    want = np.log(np.arange(1, N + 1))
    L = oracle.distill_loss(HH, q0, k, np.zeros((2, d, d)), np.zeros((2, d)))
    assert np.allclose(L[0, 0], want, rtol=0, atol=1e-12) and np.allclose(L[0, 1], want, rtol=0, atol=1e-12)
    L = oracle.distill_loss(TAY, q0, k)
    assert np.allclose(L[0, 0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("map_,d", [(HH, 8), (TAY, 4)])
def test_distill_gibbs_inequality(map_, d):
    # a cross-entropy is at least the entropy of its target distribution
    rng = np.random.default_rng(63)
    N = 30
    q = rng.standard_normal((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    W = rng.standard_normal((1, d, d)) / math.sqrt(d)
    L = oracle.distill_loss(map_, q, k, W, None)[0, 0]
    for i in range(N):
        p = _softmax_rows(q[0, 0, i] @ k[0, 0, : i + 1].T / math.sqrt(d))
        H = -np.sum(p * np.log(p))
        assert L[i] >= H - 1e-12


def test_distill_taylor_small_scores_match_softmax():
    # d = 1: the Taylor kernel 1 + s + s^2/2 equals exp(s) up to s^3/6, and the softmax logits are
    # s / sqrt(1) = s, so the predicted weights are the softmax weights up to that remainder and the
    # loss is the softmax entropy up to a few times max|s|^3 / 6
    rng = np.random.default_rng(64)
    N = 25
    q = rng.uniform(-0.3, 0.3, (1, 1, N, 1))
    k = rng.uniform(-0.3, 0.3, (1, 1, N, 1))
    L = oracle.distill_loss(TAY, q, k)[0, 0]
    smax = float(np.max(np.abs(q))) * float(np.max(np.abs(k)))
    for i in range(N):
        p = _softmax_rows(q[0, 0, i] @ k[0, 0, : i + 1].T)
        H = -np.sum(p * np.log(p))
        assert abs(L[i] - H) <= 4 * smax ** 3 / 6 + 1e-12


def test_distill_two_keys_logistic():
    # with two keys the softmax is the logistic function of the logit difference; the linear
    # weights come from the (separately pinned) feature map
    from scipy.special import expit
    rng = np.random.default_rng(65)
    d = 8
    q = rng.standard_normal((1, 1, 2, d))
    k = rng.standard_normal((1, 1, 2, d))
    W = rng.standard_normal((1, d, d)) / math.sqrt(d)
    b = rng.standard_normal((1, d)) * 0.1
    L = oracle.distill_loss(HH, q, k, W, b)[0, 0, 1]
    fq = oracle.featuremap(HH, q, W, b)[0, 0, 1]
    fk = oracle.featuremap(HH, k, W, b)[0, 0]
    a = fk @ fq
    p1 = expit((q[0, 0, 1] @ k[0, 0, 1] - q[0, 0, 1] @ k[0, 0, 0]) / math.sqrt(d))
    want = -((1 - p1) * math.log(a[0] / a.sum()) + p1 * math.log(a[1] / a.sum()))
    assert abs(L - want) < 1e-12


def test_distill_rows_subset_matches_all_rows():
    rng = np.random.default_rng(66)
    q = rng.standard_normal((2, 2, 50, 8))
    k = rng.standard_normal((2, 2, 50, 8))
    W = rng.standard_normal((2, 8, 8)) / math.sqrt(8)
    full = oracle.distill_loss(HH, q, k, W, None)
    rows = [49, 0, 17, 33]
    part = oracle.distill_loss(HH, q, k, W, None, rows=rows)
    assert np.array_equal(part, full[:, :, rows])
