"""GPU parity of the generalised quadratic map against the fp64 oracle.

The kernel a + b s + c s^2 with per-head coefficients (paperlayer.ai summary of arXiv 2610.13674,
section 2 and App. D, "Global Reference and HD Realization") runs on the packed-state kernels of
the Taylor map (bf16, head dim 16) and on the fp32 token path.  The coefficients are drawn per
head so that every weight is positive (workloads.make_inputs).  Cases: the C5 shape (B2 H16 N8192
d16) in full, ragged lengths causal and bidirectional, many segments with resume from an
arbitrary state, the fp32 path, the feature map in both dtypes, a decode step from an oracle
state, and the Taylor coefficients (1, 1, 1/2) against the Taylor map itself.  Tolerances are
those of the Taylor tests: the bf16 rule on y (rtol 2e-2, atol 1e-2), the state rule scaled by
max|S| for bf16 inputs, fp32 rtol 1e-4 / atol 1e-5 on the fp32 path.
"""

import sys

import numpy as np
import pytest

import oracle
from softmax_mimicking_feature_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

QD = wl.MAP_QUADRATIC


def hh():
    import softmax_mimicking_feature_amd as m
    return m


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


TORCH_DT = {wl.DT_BF16: torch.bfloat16, wl.DT_F32: torch.float32}


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, want, rtol, atol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = np.abs(got - want)
    bad = err > atol + rtol * np.abs(want)
    nrm = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    msg = f"{what}: {int(bad.sum())}/{bad.size} out of tolerance; max abs err {err.max():.3e}, normwise {nrm:.3e}"
    print("  " + msg, flush=True)
    assert not bad.any(), msg


def wload(**kw):
    return wl.CONFIGS["c5_taylor_causal"].replace(map=QD, **kw)


def coef_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x["W"], np.float32)).cuda()


def state_tol(w, S):
    if w.dtype == wl.DT_BF16:
        return 2e-2, 1e-2 * float(np.abs(S).max())
    return 1e-5, 1e-6 * float(np.abs(S).max())


def check_fwd(w, x, S0=None, z0=None):
    m = hh()
    dt = TORCH_DT[w.dtype]
    S0t = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, np.float32)).cuda()
    z0t = None if z0 is None else torch.from_numpy(np.ascontiguousarray(z0, np.float32)).cuda()
    r = m.hh_linattn_fwd(dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt), coef_dev(x), None, causal=w.causal,
                         map=QD, S0=S0t, z0=z0t, want_state=w.causal)
    torch.cuda.synchronize()
    rtol, atol = wl.tolerance(w.dtype)
    if w.causal:
        y, S, z = r
        yo, So, zo = oracle.causal(QD, x["q"], x["k"], x["v"], x["W"], S0=S0, z0=z0, want_state=True)
        sr, sa = state_tol(w, So)
        assert_close(host(S), So, sr, sa, "S_out")
        zr, za = state_tol(w, zo)
        assert_close(host(z), zo, zr, za, "z_out")
    else:
        y = r
        yo = oracle.bidir(QD, x["q"], x["k"], x["v"], x["W"])
    assert_close(host(y), yo, rtol, atol, "y")
    return y


def test_full_c5_shape():
    w = wload(seed=5501)
    say(f"quadratic map at the C5 shape B{w.B} H{w.H} N{w.N} d{w.d}")
    check_fwd(w, wl.make_inputs(w))


@pytest.mark.parametrize("N", [1, 17, 100, 1000, 3000])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged(N, causal):
    w = wload(B=1, H=3, N=N, causal=causal, seed=5600 + N)
    say(f"quadratic bf16 causal={causal} N={N}")
    check_fwd(w, wl.make_inputs(w))


@pytest.mark.parametrize("B,H,N", [(1, 1, 3000), (2, 8, 700)])
def test_segments_and_resume(B, H, N):
    # one head: many segments; then resume from an oracle state plus an antisymmetric part in
    # the quadratic rows (the packed basis keeps it aside and returns it in S_out)
    w = wload(B=B, H=H, N=N, seed=5700 + N)
    say(f"quadratic resume B={B} H={H} N={N}")
    x = wl.make_inputs(w)
    pre = wl.make_inputs(w.replace(N=64, seed=5701))
    pre["W"] = x["W"]
    _, S1, z1 = oracle.causal(QD, pre["q"], pre["k"], pre["v"], pre["W"], want_state=True)
    rng = np.random.default_rng(5702)
    R = rng.standard_normal((B, H, 16, 16, w.d)) * float(np.abs(S1).mean())
    S0 = S1.copy()
    S0[:, :, 17:273] += (R - R.transpose(0, 1, 3, 2, 4)).reshape(B, H, 256, w.d)
    check_fwd(w, x, S0=S0.astype(np.float32).astype(np.float64), z0=z1.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("causal", [True, False])
def test_fp32_path(causal):
    w = wload(dtype=wl.DT_F32, B=1, H=2, N=150, causal=causal, seed=5800)
    say(f"quadratic fp32 causal={causal}")
    check_fwd(w, wl.make_inputs(w))


@pytest.mark.parametrize("dtype", [wl.DT_BF16, wl.DT_F32])
def test_featuremap(dtype):
    w = wload(B=2, H=3, N=333, dtype=dtype, seed=5900)
    say(f"quadratic featuremap dtype={dtype}")
    x = wl.make_inputs(w)
    phi = hh().hh_featuremap(dev(x["q"], TORCH_DT[dtype]), coef_dev(x), None, map=QD)
    torch.cuda.synchronize()
    want = oracle.featuremap(QD, x["q"], x["W"])
    rtol, atol = (1e-2, 1e-6) if dtype == wl.DT_BF16 else (1e-5, 1e-7)
    assert_close(host(phi), want, rtol, atol, "phi")


def test_decode_step():
    w = wload(B=2, H=2, N=50, seed=6000)
    say("quadratic decode step")
    x = wl.make_inputs(w)
    S64, z64 = oracle.prefix_state(QD, x["k"], x["v"], x["W"])
    tok = wl.make_decode_token(w, B=2, H=2)
    dt = TORCH_DT[w.dtype]
    S = torch.from_numpy(S64.astype(np.float32)).cuda()
    z = torch.from_numpy(z64.astype(np.float32)).cuda()
    y = hh().hh_linattn_decode_step(dev(tok["q"], dt), dev(tok["k"], dt), dev(tok["v"], dt), coef_dev(x), None, S, z,
                                    map=QD)
    torch.cuda.synchronize()
    yo, So, zo = oracle.decode_step(QD, tok["q"], tok["k"], tok["v"], x["W"], None, S64.astype(np.float32),
                                    z64.astype(np.float32))
    rtol, atol = wl.tolerance(w.dtype)
    assert_close(host(y), yo, rtol, atol, "decode y")
    assert_close(S.cpu().numpy(), So, 1e-5, 1e-4, "decode S")
    assert_close(z.cpu().numpy(), zo, 1e-5, 1e-4, "decode z")


def test_taylor_coefficients_match_taylor_map():
    # (a, b, c) = (1, 1, 1/2) runs the same arithmetic as the Taylor map: identical bits
    w = wload(B=2, H=4, N=777, seed=6100)
    say("quadratic (1, 1, 1/2) against the Taylor map")
    x = wl.make_inputs(w)
    m = hh()
    dt = TORCH_DT[w.dtype]
    q, k, v = dev(x["q"], dt), dev(x["k"], dt), dev(x["v"], dt)
    coef = torch.tensor([[1.0, 1.0, 0.5]] * w.H, dtype=torch.float32, device="cuda")
    yq, Sq, zq = m.hh_linattn_fwd(q, k, v, coef, None, map=QD, want_state=True)
    yt, St, zt = m.hh_linattn_fwd(q, k, v, None, None, map=wl.MAP_TAYLOR2, want_state=True)
    torch.cuda.synchronize()
    assert torch.equal(yq, yt)
    assert torch.equal(Sq, St)
    assert torch.equal(zq, zt)
