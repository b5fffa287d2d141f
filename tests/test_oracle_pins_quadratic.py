"""Pins for the oracle's generalised quadratic map.

The learned global quadratic kernel p(s) = a + b s + c s^2 of the paperlayer.ai summary of
arXiv 2610.13674 (section 2; App. D, "Global Reference and HD Realization"), realised here by the
feature map [sqrt(a), sqrt(b) x, sqrt(c) x_i x_j] with per-head coefficients.  Pins:
  * the kernel identity phi(q).phi(k) = a + b s + c s^2, s = q.k, checked against the
    polynomial evaluated directly (a wrong root, a dropped term or a transposed pair index fails);
  * (a, b, c) = (1, 1, 1/2) is the degree-2 Taylor map of the walkthrough's section 3.4, "The
    Taylor Exponential as a Bridge Result": same features, same causal outputs and states;
  * b = c = 0 makes every weight equal: y_i is the mean of v_0 .. v_i;
  * causal and bidirectional outputs equal a brute-force softmax-free attention whose weights
    p(q_i.k_j) are formed directly from the polynomial, on tiny inputs;
  * scaling (a, b, c) by one factor leaves every output unchanged (the weights are normalised);
  * coefficients act per head: a two-head call equals two one-head calls;
  * chained decode steps reproduce the causal forward rows and its final state.
"""

import numpy as np
import pytest

import oracle

QD, TAY = oracle.MAP_QUADRATIC, oracle.MAP_TAYLOR2


def _qkv(seed, B=1, H=2, N=9, d=16, scale=0.35):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((B, H, N, d)) * s for s in (scale, scale, 1.0))


def _poly(abc, s):
    return abc[0] + abc[1] * s + abc[2] * s * s


COEFS = [np.array([0.7, 0.9, 0.4]), np.array([2.0, 0.0, 1.5]), np.array([0.25, 3.0, 0.05])]


@pytest.mark.parametrize("ci", range(len(COEFS)))
def test_kernel_identity(ci):
    abc = COEFS[ci]
    q, k, _ = _qkv(1, H=1)
    W = abc.reshape(1, 3)
    fq, fk = oracle.featuremap(QD, q, W)[0, 0], oracle.featuremap(QD, k, W)[0, 0]
    assert fq.shape[-1] == 1 + 16 + 256
    s = q[0, 0] @ k[0, 0].T
    np.testing.assert_allclose(fq @ fk.T, _poly(abc, s), rtol=1e-13, atol=1e-13)


def test_taylor_case_is_the_taylor_map():
    q, k, v = _qkv(2)
    W = np.tile([1.0, 1.0, 0.5], (2, 1))
    np.testing.assert_allclose(oracle.featuremap(QD, q, W), oracle.featuremap(TAY, q), rtol=0, atol=1e-15)
    yq, Sq, zq = oracle.causal(QD, q, k, v, W, want_state=True)
    yt, St, zt = oracle.causal(TAY, q, k, v, want_state=True)
    np.testing.assert_allclose(yq, yt, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Sq, St, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(zq, zt, rtol=1e-13, atol=1e-13)


def test_constant_kernel_gives_prefix_means():
    q, k, v = _qkv(3)
    W = np.tile([1.3, 0.0, 0.0], (2, 1))
    y = oracle.causal(QD, q, k, v, W)
    ref = np.cumsum(v, axis=2) / np.arange(1, v.shape[2] + 1)[None, None, :, None]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def _brute(abc_h, q, k, v, causal):
    B, H, N, d = q.shape
    y = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            s = q[b, h] @ k[b, h].T
            w = _poly(abc_h[h], s)
            if causal:
                w = np.tril(w)
            y[b, h] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
    return y


@pytest.mark.parametrize("causal", [True, False])
def test_matches_brute_force_weights(causal):
    q, k, v = _qkv(4, B=2, H=2, N=11)
    W = np.stack([COEFS[0], COEFS[2]])
    y = oracle.causal(QD, q, k, v, W) if causal else oracle.bidir(QD, q, k, v, W)
    np.testing.assert_allclose(y, _brute(W, q, k, v, causal), rtol=1e-12, atol=1e-12)


def test_scaled_coefficients_leave_outputs_unchanged():
    q, k, v = _qkv(5)
    W = np.stack([COEFS[0], COEFS[1]])
    np.testing.assert_allclose(oracle.causal(QD, q, k, v, 3.5 * W), oracle.causal(QD, q, k, v, W),
                               rtol=1e-12, atol=1e-12)


def test_coefficients_are_per_head():
    q, k, v = _qkv(6)
    W = np.stack([COEFS[0], COEFS[2]])
    y = oracle.causal(QD, q, k, v, W)
    for h in range(2):
        yh = oracle.causal(QD, q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], W[h:h + 1])
        np.testing.assert_allclose(y[:, h:h + 1], yh, rtol=0, atol=0)


def test_decode_chain_equals_forward():
    q, k, v = _qkv(7, N=6)
    W = np.stack([COEFS[0], COEFS[1]])
    yf, Sf, zf = oracle.causal(QD, q, k, v, W, want_state=True)
    dp = oracle.feature_dim(QD, 16)
    S = np.zeros((1, 2, dp, 16))
    z = np.zeros((1, 2, dp))
    for i in range(6):
        yi, S, z = oracle.decode_step(QD, q[:, :, i:i + 1], k[:, :, i:i + 1], v[:, :, i:i + 1], W, None, S, z)
        np.testing.assert_allclose(yi, yf[:, :, i], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, Sf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, zf, rtol=1e-12, atol=1e-12)
