"""GPU parity of the backward (dq, dk, dv, dW, db given dL/dy) against the fp64 oracle's backward,
which is written from the explicit form of Eq. 2 by the chain rule and pinned by central finite
differences (tests/test_oracle_pins_variants.py).

Tolerance.  The kernels take the features, g = dy / den and the intra-chunk weights as bf16
matrix-core operands (relative rounding 2^-9 each) and sum in fp32; a gradient entry is a sum of
many such terms with mixed signs, so its error scales with the largest entry of the gradient
rather than with the entry itself: a few 2^-9 relative roundings of the largest terms.  Rule per
tensor: |gpu - oracle| <= 2e-2 |oracle| + 3e-2 max|oracle| elementwise (measured up to 1.7e-2 max|oracle|), and normwise
||gpu - oracle|| / ||oracle|| <= 1e-2 (measured at most 6.7e-3 over these cases).  A gradient that
is exactly zero (a one-token sequence: y_0 = v_0 whatever q and k are, so dq = dk = dW = db = 0)
is instead held to the rounding level of the terms that cancel in it: max|gpu| <= 2^-7 max|dv|
(times B N for dW and db, which sum over the tokens)."""

import sys

import numpy as np
import pytest

import oracle
from softmax_mimicking_feature_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HH, HS, EXP, SM = oracle.MAP_HEDGEHOG, oracle.MAP_HEDGEHOG_SOFTMAX, oracle.MAP_EXP, oracle.MAP_SOFTMAX


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def close_grad(got, want, what, zero_floor=None):
    got = np.asarray(got, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    scale = float(np.abs(want).max())
    if zero_floor is not None and scale < 1e-6 * zero_floor:
        print(f"  {what}: exactly zero by the method; max|gpu| {np.abs(got).max():.3e} (bound {zero_floor:.3e})")
        assert np.abs(got).max() <= zero_floor, what
        return
    err = np.abs(got - want)
    bad = err > 2e-2 * np.abs(want) + 3e-2 * scale
    nrm = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    print(f"  {what}: max abs err {err.max():.3e} (max|ref| {scale:.3e}), normwise {nrm:.3e}, "
          f"{int(bad.sum())}/{bad.size} out", flush=True)
    assert not bad.any() and nrm <= 1e-2, what


def run_case(map_, causal, B, H, N, d, seed, b_std=0.1):
    w = wl.CONFIGS["c2_gpt2_causal"].replace(B=B, H=H, N=N, d=d, w_std=d ** -0.5,
                                             b_std=b_std if map_ in (HH, EXP) else 0.0, seed=seed)
    x = wl.make_inputs(w)
    b = x["b"] if map_ in (HH, EXP) else None
    rng = np.random.default_rng(seed + 1)
    dy = wl.round_to_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))
    import softmax_mimicking_feature_amd as m
    q, k, v, W = (dev(x[n]) for n in ("q", "k", "v", "W"))
    bt = None if b is None else dev(b)
    y = m.hh_linattn_fwd(q, k, v, W, bt, map=map_, causal=causal)
    dq, dk, dv, dW, db = m.hh_linattn_bwd(q, k, v, W, bt, y, dev(dy), map=map_, causal=causal)
    torch.cuda.synchronize()
    oq, ok_, ov, oW, ob = oracle.backward(map_, x["q"], x["k"], x["v"], x["W"], b, dy, causal=causal)
    close_grad(host(dv), ov, "dv")
    floor = 2.0 ** -7 * float(np.abs(ov).max())
    close_grad(host(dq), oq, "dq", floor)
    close_grad(host(dk), ok_, "dk", floor)
    close_grad(host(dW), oW, "dW", floor * N * B)
    if ob is not None:
        close_grad(host(db), ob, "db", floor * N * B)
    else:
        assert db is None


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("N", [1, 65, 700])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_hedgehog(d, N, causal):
    say(f"backward hedgehog d={d} N={N} causal={causal}")
    run_case(HH, causal, 2, 3, N, d, seed=16000 + d + N)


@pytest.mark.parametrize("map_", [HS, EXP, SM])
@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_variants(map_, d, causal):
    say(f"backward map={map_} d={d} causal={causal}")
    run_case(map_, causal, 1, 2, 300, d, seed=17000 + 10 * map_ + d)


def test_backward_many_segments():
    # one sequence cut into many segments: forward and reverse sums handed across 40+ segments
    say("backward hedgehog B1 H1 N3000 d64, many segments")
    run_case(HH, True, 1, 1, 3000, 64, seed=18000)


@pytest.mark.parametrize("d,H", [(64, 12), (128, 2)])
def test_backward_model_shapes(d, H):
    # GPT-2 heads (d 64, N 1024, all 12 heads of one sequence) and two Llama-2-7B heads (d 128,
    # N 4096): the oracle's explicit form costs N^2 per head
    N = 1024 if d == 64 else 4096
    say(f"backward hedgehog B1 H{H} N{N} d{d}")
    run_case(HH, True, 1, H, N, d, seed=18100 + d, b_std=0.1 if d == 64 else 0.0)


def test_backward_llama2_bench_shape_sampled_heads():
    # the backward workload as timed (B1 H32 N4096 d128: eight segments of 512 tokens per head,
    # the launch configuration of that head count), every gradient of three heads against the
    # oracle, which treats the heads independently (dW, db are per head at B = 1)
    w = wl.CONFIGS["c3_llama2_backward"]
    say(f"backward hedgehog B{w.B} H{w.H} N{w.N} d{w.d}, heads 0, 17, 31 against the oracle")
    x = wl.make_inputs(w)
    rng = np.random.default_rng(19000)
    dy = wl.round_to_bf16(rng.standard_normal((w.B, w.H, w.N, w.d)).astype(np.float32))
    import softmax_mimicking_feature_amd as m
    q, k, v, W, b = (dev(x[n]) for n in ("q", "k", "v", "W", "b"))
    y = m.hh_linattn_fwd(q, k, v, W, b, map=HH, causal=True)
    dq, dk, dv, dW, db = m.hh_linattn_bwd(q, k, v, W, b, y, dev(dy), map=HH, causal=True)
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    sel = lambda a: a[:, heads]
    oq, ok_, ov, oW, ob = oracle.backward(HH, sel(x["q"]), sel(x["k"]), sel(x["v"]), x["W"][heads], x["b"][heads],
                                          sel(dy), causal=True)
    close_grad(host(dv)[:, heads], ov, "dv")
    close_grad(host(dq)[:, heads], oq, "dq")
    close_grad(host(dk)[:, heads], ok_, "dk")
    close_grad(host(dW)[heads], oW, "dW")
    close_grad(host(db)[heads], ob, "db")
