"""Pins for the oracle's feature-map variants and its backward.

Feature maps (section 3.4, "The Hedgehog MLP Feature Map"): the single-sided exponential
exp(W x + b) with d' = d (Choice 1, default d' = d), the softmax over the d feature directions
without bias (Choice 4), single-sided and with the negation mapping of Choice 3 as one softmax
per half.  Pins: hand-worked fractions (tests/golden/feature_map_variants.json), the kernel
identity printed under Choice 1, W = t I giving exp(t x) (the fixed phi_t map of the section 3.2
diagnostics), each softmax half summing to one, invariance of the softmax maps to adding one
vector to every row of W (and its failure for the exp maps), and W = 0 giving prefix means.

Backward (gradients of sum(dy * y), the quantities training from scratch needs, section 3.4,
"Training Protocols for the Three Regimes"): central finite differences of the oracle's own
forward for every input and parameter, every map, causal and bidirectional; and the closed
form of dv when every feature vector is the same (prefix means).

A slip these catch: a bias in a softmax map, a softmax over all 2d features instead of per
half, a softmax over tokens, W transposed, a gradient sign or a missing term of the quotient
rule (dL/da_ij without the -y_i part), a causal boundary off by one in the backward.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
HH, TAY, HS, EXP, SM = (oracle.MAP_HEDGEHOG, oracle.MAP_TAYLOR2, oracle.MAP_HEDGEHOG_SOFTMAX, oracle.MAP_EXP,
                        oracle.MAP_SOFTMAX)
MAPS = {"hedgehog": HH, "taylor2": TAY, "hedgehog_softmax": HS, "exp": EXP, "softmax": SM}


def _val(s):
    if isinstance(s, (int, float)):
        return float(s)
    s = s.strip()
    if s == "ln2":
        return math.log(2.0)
    if s == "-ln2":
        return -math.log(2.0)
    if "/" in s:
        a, b = s.split("/")
        return float(a) / float(b)
    return float(s)


def _arr(x):
    return np.array([[_val(e) for e in row] if isinstance(row, list) else _val(row) for row in x], np.float64)


def test_feature_dims():
    assert oracle.feature_dim(HS, 64) == 128
    assert oracle.feature_dim(EXP, 64) == 64
    assert oracle.feature_dim(SM, 16) == 16


def test_golden_variants():
    g = json.load(open(os.path.join(GOLDEN, "feature_map_variants.json")))
    for c in g["cases"]:
        m, d = MAPS[c["map"]], c["d"]
        q = _arr(c["q"]).reshape(1, 1, -1, d)
        k = _arr(c["k"]).reshape(1, 1, -1, d)
        v = _arr(c["v"]).reshape(1, 1, -1, d)
        W = np.array(c["W"], np.float64).reshape(1, d, d)
        b = _arr(c["b"]).reshape(1, d) if "b" in c else None
        want = _arr(c["causal_y"]).reshape(1, 1, -1, d)
        np.testing.assert_allclose(oracle.causal(m, q, k, v, W, b), want, rtol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(oracle.quadratic(m, q, k, v, W, b), want, rtol=1e-13, err_msg=c["name"])
    for f in g["featuremaps"]:
        m, d = MAPS[f["map"]], f["d"]
        x = _arr(f["x"]).reshape(1, 1, 1, d)
        W = np.array(f["W"], np.float64).reshape(1, d, d)
        b = _arr(f["b"]).reshape(1, d) if "b" in f else None
        np.testing.assert_allclose(oracle.featuremap(m, x, W, b).ravel(), _arr(f["phi"]), rtol=1e-14,
                                   err_msg=f["name"])


def test_exp_map_kernel_identity():
    # printed under Choice 1: phi(q).phi(k) = sum_l exp(w_l.(q + k) + 2 b_l), w_l the l-th row of W
    rng = np.random.default_rng(41)
    for d in (1, 2, 4, 16):
        W = rng.standard_normal((1, d, d)) * 0.4
        b = rng.standard_normal((1, d)) * 0.3
        x = rng.standard_normal((1, 1, 2, d))
        phi = oracle.featuremap(EXP, x, W, b)[0, 0]
        s = x[0, 0, 0] + x[0, 0, 1]
        want = sum(math.exp(float(W[0, l] @ s) + 2.0 * b[0, l]) for l in range(d))
        assert phi[0] @ phi[1] == pytest.approx(want, rel=1e-13)
        if d > 1:
            wrong = sum(math.exp(float(W[0, :, l] @ s) + 2.0 * b[0, l]) for l in range(d))
            assert abs(phi[0] @ phi[1] - wrong) > 1e-6 * abs(wrong)


def test_exp_map_with_scaled_identity_is_phi_t():
    rng = np.random.default_rng(42)
    d, t = 8, 1.7
    x = rng.standard_normal((1, 1, 5, d))
    phi = oracle.featuremap(EXP, x, t * np.eye(d)[None], np.zeros((1, d)))
    np.testing.assert_allclose(phi, np.exp(t * x), rtol=1e-14)


@pytest.mark.parametrize("m", [HS, SM])
def test_softmax_maps_normalise_per_half_and_ignore_shifts(m):
    rng = np.random.default_rng(43 + m)
    d = 8
    x = rng.standard_normal((2, 3, 7, d))
    W = rng.standard_normal((3, d, d)) * 0.6
    phi = oracle.featuremap(m, x, W)
    halves = phi.reshape(2, 3, 7, -1, d)
    np.testing.assert_allclose(halves.sum(axis=-1), 1.0, rtol=1e-14)
    assert (phi > 0).all() and (phi < 1).all()
    # the same vector added to every row of W moves every projection of x by the same amount:
    # a softmax over the directions does not change (per half: the negated half moves too)
    a = rng.standard_normal((3, 1, d))
    np.testing.assert_allclose(oracle.featuremap(m, x, W + a), phi, rtol=1e-12)
    # a bias would be ignored by definition (Choice 4 omits it)
    np.testing.assert_allclose(oracle.featuremap(m, x, W, rng.standard_normal((3, d))), phi, rtol=0)
    # the exponential maps are not shift invariant
    e1 = oracle.featuremap(EXP, x, W, np.zeros((3, d)))
    e2 = oracle.featuremap(EXP, x, W + a, np.zeros((3, d)))
    assert np.abs(e1 - e2).max() > 1e-3
    if m == HS:  # the two halves are different distributions (not one softmax over 2d entries)
        assert np.abs(halves[..., 0, :] - halves[..., 1, :]).max() > 1e-3


@pytest.mark.parametrize("m", [HS, EXP, SM])
def test_variants_zero_W_give_prefix_means(m):
    rng = np.random.default_rng(44 + m)
    B, H, N, d = 2, 2, 9, 4
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    W = np.zeros((H, d, d))
    b = np.zeros((H, d))
    y = oracle.causal(m, q, k, v, W, b)
    np.testing.assert_allclose(y, np.cumsum(v, axis=2) / np.arange(1, N + 1)[:, None], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.bidir(m, q, k, v, W, b), np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape),
                               rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("m", [HS, EXP, SM])
def test_variants_running_sums_equal_quadratic_form(m):
    rng = np.random.default_rng(45 + m)
    q, k, v = (rng.standard_normal((1, 2, 17, 4)) for _ in range(3))
    W = rng.standard_normal((2, 4, 4)) * 0.5
    b = rng.standard_normal((2, 4)) * 0.2
    np.testing.assert_allclose(oracle.causal(m, q, k, v, W, b), oracle.quadratic(m, q, k, v, W, b), rtol=1e-11)
    y, S, z = oracle.causal(m, q, k, v, W, b, want_state=True)
    phik = oracle.featuremap(m, k, W, b)
    np.testing.assert_allclose(S, np.einsum("bhnf,bhnc->bhfc", phik, v), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.causal_features(oracle.featuremap(m, q, W, b), phik, v), y, rtol=1e-12)


# ---------------------------------------------------------------- backward ----

def _loss(m, causal, dy, q, k, v, W, b):
    y = oracle.causal(m, q, k, v, W, b) if causal else oracle.bidir(m, q, k, v, W, b)
    return float((dy * y).sum())


@pytest.mark.parametrize("m", [HH, TAY, HS, EXP, SM])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 2, 5, 3), (2, 1, 1, 2), (1, 1, 4, 1)])
def test_backward_matches_central_differences(m, causal, shape):
    B, H, N, d = shape
    rng = np.random.default_rng(hash((m, causal, shape)) % 2 ** 32)
    q, k, v = (rng.standard_normal(shape) * 0.7 for _ in range(3))
    W = rng.standard_normal((H, d, d)) * 0.5
    b = rng.standard_normal((H, d)) * 0.3
    dy = rng.standard_normal(shape)
    dq, dk, dv, dW, db = oracle.backward(m, q, k, v, W, b, dy, causal=causal)
    args = {"q": q, "k": k, "v": v, "W": W, "b": b}
    grads = {"q": dq, "k": dk, "v": dv, "W": dW, "b": db}
    assert (dW is None) == (m == TAY)
    assert (db is None) == (m not in (HH, EXP))
    h = 1e-6
    for name, g in grads.items():
        if g is None:
            continue
        fd = np.zeros_like(args[name])
        for idx in np.ndindex(fd.shape):
            a = dict(args)
            xp = args[name].copy()
            xp[idx] += h
            a[name] = xp
            lp = _loss(m, causal, dy, **a)
            xm = args[name].copy()
            xm[idx] -= h
            a[name] = xm
            lm = _loss(m, causal, dy, **a)
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(np.abs(fd).max(), 1e-3)
        assert np.abs(fd - g).max() <= 1e-6 * scale, (name, np.abs(fd - g).max(), scale)


def test_backward_prefix_mean_closed_form():
    # W = 0: every feature vector is the same, y_i is the mean of v_0..v_i, so
    # dL/dv_j = sum_{i >= j} dy_i / (i + 1) and nothing depends on q or k
    rng = np.random.default_rng(46)
    B, H, N, d = 1, 2, 7, 3
    q, k, v, dy = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    W = np.zeros((H, d, d))
    b = rng.standard_normal((H, d)) * 0.3
    dq, dk, dv, dW, db = oracle.backward(HH, q, k, v, W, b, dy)
    want = np.flip(np.cumsum(np.flip(dy / np.arange(1, N + 1)[:, None], axis=2), axis=2), axis=2)
    np.testing.assert_allclose(dv, want, rtol=1e-12)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk, 0.0, atol=1e-13)
    dq, dk, dv, dW, db = oracle.backward(HH, q, k, v, W, b, dy, causal=False)
    np.testing.assert_allclose(dv, np.broadcast_to(dy.sum(axis=2, keepdims=True) / N, dv.shape), rtol=1e-12)
