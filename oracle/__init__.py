"""fp64 CPU oracle for Hedgehog-style linear attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never touch it.  The arithmetic lives in ``hh_oracle.c`` (plain C, double
precision); this module builds it with gcc and marshals numpy arrays.

What each function computes, with its source on the pages ("The Hedgehog &
the Porcupine: Expressive Linear Attentions with Softmax Mimicry"):
  featuremap  -- Hedgehog map exp(+-(W x + b)) (section 3.4, "The Hedgehog MLP
                 Feature Map", Choices 1 and 3) or the degree-2 Taylor map
                 (section 3.4, "The Taylor Exponential as a Bridge Result");
                 the single-sided exp(W x + b) with d' = d (Choice 1 and the
                 default d' = d of the same section); the softmax over the d
                 feature directions, no bias (Choice 4), single-sided (d' = d)
                 or with the negation mapping as one softmax per half (d' = 2d);
                 the generalised quadratic [sqrt a, sqrt b x, sqrt c x_i x_j] of
                 the kernel p(s) = a + b s + c s^2, coefficients per head
                 (paperlayer.ai summary of arXiv 2610.13674, section 2 and
                 App. D, "Global Reference and HD Realization").
  causal      -- Eq. 2 by running sums S_i, z_i (section 3.4, "Complexity
                 Analysis"), with optional initial and final state.
  bidir       -- the same sums over all keys (bidirectional encoders).
  decode_step -- one running-sum update followed by the read-out.
  quadratic   -- Eq. 2 as an explicit sum over key positions (no running sums),
                 used to pin the running-sum form and for sampled rows.
  causal_features -- the running-sum form from given features phi(q_i), phi(k_j).
  backward    -- gradients of sum(dy * y) with respect to q, k, v, W and b,
                 from the explicit form by the chain rule.
Parity status: every function is pinned by the closed forms and invariants in
tests/test_oracle_pins.py (no function is "parity unpinned").
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hh_oracle.c")
LIB = os.path.join(HERE, "libhh_oracle.so")

MAP_HEDGEHOG = 0
MAP_TAYLOR2 = 1
MAP_HEDGEHOG_SOFTMAX = 2
MAP_EXP = 3
MAP_SOFTMAX = 4
MAP_QUADRATIC = 5

_lib = None


def build(force: bool = True) -> str:
    """Compile hh_oracle.c into libhh_oracle.so next to it (gcc, -O2, IEEE fp64)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        lib = ctypes.CDLL(LIB)
        D = ctypes.c_void_p
        L = ctypes.c_long
        I = ctypes.c_int
        lib.hho_feature_dim.argtypes = [I, I]
        lib.hho_feature_dim.restype = I
        lib.hho_causal.argtypes = [I, I, L, L, L, D, D, D, D, D, D, D, D, D, D, I]
        lib.hho_bidir.argtypes = [I, I, L, L, L, D, D, D, D, D, D, I]
        lib.hho_decode_step.argtypes = [I, I, L, L, D, D, D, D, D, D, D, D, I]
        lib.hho_quadratic.argtypes = [I, I, L, L, L, I, D, D, D, D, D, L, D, D, I]
        lib.hho_featuremap.argtypes = [I, I, L, L, L, D, D, D, D, I]
        lib.hho_distill.argtypes = [I, I, L, L, L, D, D, D, D, L, D, D, I]
        lib.hho_causal_features.argtypes = [I, I, L, L, D, D, D, D, D, D, D, D, I]
        lib.hho_backward.argtypes = [I, I, L, L, L, I, D, D, D, D, D, D, D, D, D, D, D, I]
        for f in (lib.hho_causal, lib.hho_bidir, lib.hho_decode_step, lib.hho_quadratic,
                  lib.hho_featuremap, lib.hho_distill, lib.hho_causal_features, lib.hho_backward):
            f.restype = None
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def feature_dim(map_: int, d: int) -> int:
    return int(_load().hho_feature_dim(map_, d))


def _params(map_, W, b, H, d):
    if map_ == MAP_TAYLOR2:
        return None, None
    if map_ == MAP_QUADRATIC:  # W holds the coefficients (a, b, c) of each head
        return _f64(W).reshape(H, 3), None
    W = _f64(W).reshape(H, d, d)
    if map_ in (MAP_HEDGEHOG, MAP_EXP):
        b = None if b is None or np.size(b) == 0 else _f64(b).reshape(H, d)
    else:  # the softmax maps have no bias
        b = None
    return W, b


def featuremap(map_: int, x, W=None, b=None, nthreads: Optional[int] = None) -> np.ndarray:
    """x [B,H,N,d] -> phi [B,H,N,d'] in float64."""
    x = _f64(x)
    B, H, N, d = x.shape
    W, b = _params(map_, W, b, H, d)
    dp = feature_dim(map_, d)
    out = np.empty((B, H, N, dp), np.float64)
    _load().hho_featuremap(map_, d, B, H, N, _ptr(x), _ptr(W), _ptr(b), _ptr(out),
                           nthreads or default_threads())
    return out


def causal(map_: int, q, k, v, W=None, b=None, S0=None, z0=None, want_state: bool = False,
           nthreads: Optional[int] = None):
    """Causal Eq. 2 by running sums.  q,k,v [B,H,N,d] -> y [B,H,N,d] (float64).

    With want_state, also returns the final (S [B,H,d',d], z [B,H,d'])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    W, b = _params(map_, W, b, H, d)
    dp = feature_dim(map_, d)
    S0 = None if S0 is None else _f64(S0).reshape(B, H, dp, d)
    z0 = None if z0 is None else _f64(z0).reshape(B, H, dp)
    y = np.empty_like(q)
    S = np.empty((B, H, dp, d), np.float64) if want_state else None
    z = np.empty((B, H, dp), np.float64) if want_state else None
    _load().hho_causal(map_, d, B, H, N, _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b), _ptr(S0),
                       _ptr(z0), _ptr(y), _ptr(S), _ptr(z), nthreads or default_threads())
    return (y, S, z) if want_state else y


def causal_features(phiq, phik, v, S0=None, z0=None, want_state: bool = False, nthreads: Optional[int] = None):
    """Causal Eq. 2 by running sums from given features phi(q_i), phi(k_j) [B,H,N,d'] and values
    v [B,H,N,d] (the recurrence of section 3.4, "Complexity Analysis", with the feature map
    already applied).  Returns y [B,H,N,d], and the final (S, z) with want_state."""
    phiq, phik, v = _f64(phiq), _f64(phik), _f64(v)
    B, H, N, d = v.shape
    dp = phiq.shape[-1]
    assert phiq.shape == (B, H, N, dp) and phik.shape == (B, H, N, dp)
    S0 = None if S0 is None else _f64(S0).reshape(B, H, dp, d)
    z0 = None if z0 is None else _f64(z0).reshape(B, H, dp)
    y = np.empty_like(v)
    S = np.empty((B, H, dp, d), np.float64) if want_state else None
    z = np.empty((B, H, dp), np.float64) if want_state else None
    _load().hho_causal_features(d, dp, B * H, N, _ptr(phiq), _ptr(phik), _ptr(v), _ptr(S0), _ptr(z0), _ptr(y),
                                _ptr(S), _ptr(z), nthreads or default_threads())
    return (y, S, z) if want_state else y


def bidir(map_: int, q, k, v, W=None, b=None, nthreads: Optional[int] = None) -> np.ndarray:
    """Bidirectional Eq. 2 (all keys).  q,k,v [B,H,N,d] -> y [B,H,N,d] (float64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    W, b = _params(map_, W, b, H, d)
    y = np.empty_like(q)
    _load().hho_bidir(map_, d, B, H, N, _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b), _ptr(y),
                      nthreads or default_threads())
    return y


def decode_step(map_: int, q, k, v, W, b, S, z, nthreads: Optional[int] = None):
    """One step from (S, z).  q,k,v [B,H,1,d] or [B,H,d]; returns (y [B,H,d], S', z') in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H = q.shape[:2]
    d = q.shape[-1]
    W, b = _params(map_, W, b, H, d)
    dp = feature_dim(map_, d)
    S = _f64(S).reshape(B, H, dp, d).copy()
    z = _f64(z).reshape(B, H, dp).copy()
    y = np.empty((B, H, d), np.float64)
    _load().hho_decode_step(map_, d, B, H, _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b), _ptr(S),
                            _ptr(z), _ptr(y), nthreads or default_threads())
    return y, S, z


def quadratic(map_: int, q, k, v, W=None, b=None, causal: bool = True, rows=None,
              nthreads: Optional[int] = None) -> np.ndarray:
    """Explicit quadratic form.  Returns y [B,H,N,d], or [B,H,len(rows),d] for selected rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    W, b = _params(map_, W, b, H, d)
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        assert rows.ndim == 1 and (rows.size == 0 or (rows.min() >= 0 and rows.max() < N))
        nr = rows.size
    else:
        nr = N
    y = np.empty((B, H, nr, d), np.float64)
    _load().hho_quadratic(map_, d, B, H, N, int(bool(causal)), _ptr(q), _ptr(k), _ptr(v), _ptr(W),
                          _ptr(b), nr if rows is not None else 0,
                          _ptr(rows) if rows is not None else None, _ptr(y),
                          nthreads or default_threads())
    return y


def prefix_state(map_: int, k, v, W=None, b=None, nthreads: Optional[int] = None):
    """Running sums after a whole prefix: S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j) (float64).

    The definition of S_N, z_N in section 3.4, "Complexity Analysis", evaluated with the
    oracle's feature map and a library matrix product per (b, h); one batch row at a time
    to bound memory.  k, v: [B,H,N,d] -> S [B,H,d',d], z [B,H,d']."""
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, N, d = k.shape
    dp = feature_dim(map_, d)
    S = np.empty((B, H, dp, d), np.float64)
    z = np.empty((B, H, dp), np.float64)
    for bi in range(B):
        phi = featuremap(map_, k[bi:bi + 1], W, b, nthreads=nthreads)[0]     # [H,N,dp]
        S[bi] = np.matmul(phi.transpose(0, 2, 1), _f64(v[bi]))
        z[bi] = phi.sum(axis=1)
    return S, z


def backward(map_: int, q, k, v, W=None, b=None, dy=None, causal: bool = True, nthreads: Optional[int] = None):
    """Gradients of L = sum(dy * y) with y the forward of Eq. 2 (causal or bidirectional).

    Written from the explicit form a_ij = phi(q_i).phi(k_j): dL/da_ij = dy_i.(v_j - y_i) / den_i,
    then the chain rule through a_ij to the features and through the feature map to q, k and the
    map's parameters (the gradients that training from scratch needs, section 3.4, "Training
    Protocols for the Three Regimes").  Returns (dq, dk, dv [B,H,N,d], dW [H,d,d], db [H,d]);
    dW and db sum over the batch, the tokens and both q and k (None for the Taylor map; db None
    for the maps without a bias)."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, H, N, d = q.shape
    W, b = _params(map_, W, b, H, d)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dWp = np.empty((B, H, d, d), np.float64)
    dbp = np.empty((B, H, d), np.float64)
    _load().hho_backward(map_, d, B, H, N, int(bool(causal)), _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b),
                         _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dWp), _ptr(dbp), nthreads or default_threads())
    dW = None if map_ in (MAP_TAYLOR2, MAP_QUADRATIC) else dWp.sum(axis=0)
    db = dbp.sum(axis=0) if map_ in (MAP_HEDGEHOG, MAP_EXP) else None
    return dq, dk, dv, dW, db


def distill_loss(map_: int, q, k, W=None, b=None, rows=None, nthreads: Optional[int] = None) -> np.ndarray:
    """Attention-weight distillation loss (Eq. 4 of the walkthrough's section 3.4) per query:
    q, k [B,H,N,d] -> L [B,H,N] (float64), or [B,H,len(rows)] for the listed query rows.

    L_i = -sum_{j<=i} p_ij log(a_ij / sum_{m<=i} a_im), with p_ij the causal softmax of
    q_i.k_j / sqrt(d) and a_ij = phi(q_i).phi(k_j)."""
    q, k = _f64(q), _f64(k)
    B, H, N, d = q.shape
    W, b = _params(map_, W, b, H, d)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nr = N if r is None else len(r)
    out = np.empty((B, H, nr), np.float64)
    _load().hho_distill(map_, d, B, H, N, _ptr(q), _ptr(k), _ptr(W), _ptr(b), 0 if r is None else nr,
                        _ptr(r), _ptr(out), nthreads or default_threads())
    return out
