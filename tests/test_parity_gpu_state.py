"""GPU checks of the carried state and of long recurrences.

* fp32 carry across segments.  A sequence is cut into segments whose aggregates are handed to
  the later segments; these hand-offs are fp32 (the running sums S_i, z_i of section 3.4,
  "Complexity Analysis", carried without rounding).  Two checks that bf16 hand-offs would fail:
  - the same head run alone (cut into many segments) and inside a 256-head batch (one segment
    per sequence) returns the same final state to fp32 summation accuracy;
  - the final state equals the oracle's running sums of the very features the kernels use
    (bf16-rounded phi(k), which is what the matrix cores multiply), again to fp32 accuracy.
  A bf16 hand-off rounds 7/8 of the sum to 8 significant bits: normwise error ~1e-3.
* NaN containment (Eq. 2 is causal, j <= i): a NaN in v_j[c] reaches y_i[c] for i >= j and no
  other column; rows before the 32-token block holding j are bit-identical to a run without
  the NaN.  Inside that block the matrix cores multiply the masked-out (exactly zero) weights
  of later keys by their values, and IEEE 0 * NaN = NaN, so earlier rows of the same block see
  the NaN in column c as well; no other output does.
* 4096 chained decode steps at d = 128 reproduce the forward rows and its final state.
"""

import sys

import numpy as np
import pytest

import oracle
from softmax_mimicking_feature_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def hh():
    import softmax_mimicking_feature_amd as m
    return m


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype or torch.bfloat16).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def normwise(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def bf16(a):
    return wl.round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)


def close(got, want, rtol, atol, what):
    err = np.abs(np.asarray(got, np.float64) - want)
    bad = err > atol + rtol * np.abs(want)
    print(f"  {what}: max abs err {err.max():.3e}, normwise {normwise(got, want):.3e}, "
          f"{int(bad.sum())}/{bad.size} out of tolerance", flush=True)
    assert not bad.any(), what


@pytest.mark.parametrize("d", [128, 64])
def test_fp32_carry_segmented_equals_one_segment(d):
    m = hh()
    w = wl.CONFIGS["c3_llama2_causal"].replace(B=1, H=1, N=4096, d=d, w_std=d ** -0.5, seed=9700 + d)
    say(f"fp32 carry d={d}: one head alone (many segments) vs in a 256-head batch (one segment)")
    x = wl.make_inputs(w)
    q, k, v, W, b = (dev(x[n]) for n in ("q", "k", "v", "W", "b"))
    y1, S1, z1 = m.hh_linattn_fwd(q, k, v, W, b, want_state=True)
    nb = 256 if d == 128 else 512    # enough sequences that each one is a single segment
    rep = lambda t: t.expand(nb, -1, -1, -1).contiguous()  # noqa: E731
    y2, S2, z2 = m.hh_linattn_fwd(rep(q), rep(k), rep(v), W, b, want_state=True)
    torch.cuda.synchronize()
    ws1 = m.hh_linattn_fwd_workspace(w.map, w.dtype, 1, 1, 1, w.N, d)
    ws2 = m.hh_linattn_fwd_workspace(w.map, w.dtype, 1, nb, 1, w.N, d)
    assert ws1 > 0, "the single head must be cut into segments"
    assert ws2 == 0, "each sequence of the batch must be one segment (no slots)"
    Sa, Sb = host(S1)[0, 0], host(S2)[0, 0]
    za, zb = host(z1)[0, 0], host(z2)[0, 0]
    # every sequence of the batch is the same head: same result everywhere
    assert torch.equal(S2[:1].expand(nb, -1, -1, -1), S2)
    e_s, e_z = normwise(Sa, Sb), normwise(za, zb)
    print(f"  segmented vs one segment: S normwise {e_s:.3e}, z normwise {e_z:.3e}", flush=True)
    assert e_s <= 2e-6 and e_z <= 2e-6  # measured ~4e-7 (fp32 sums in another order); bf16 hand-offs ~1e-3
    rtol, atol = wl.tolerance(w.dtype)
    close(host(y1)[0, 0], host(y2)[0, 0], rtol, atol, "y segmented vs one segment")

    # against the oracle's running sums of the bf16-rounded features the kernels multiply
    phik = bf16(oracle.featuremap(w.map, x["k"], x["W"], x["b"]))
    phiq = bf16(oracle.featuremap(w.map, x["q"], x["W"], x["b"]))
    _, So, zo = oracle.causal_features(phiq, phik, x["v"], want_state=True)
    e_so, e_zo = normwise(Sa, So[0, 0]), normwise(za, zo[0, 0])
    print(f"  vs oracle sums of bf16 features: S normwise {e_so:.3e}, z normwise {e_zo:.3e}", flush=True)
    assert e_so <= 5e-5 and e_zo <= 5e-5  # measured ~1.2e-5: rare 1-ulp differences of bf16 features
    close(Sa, So[0, 0], 1e-3, 1e-4 * float(np.abs(So).max()), "S_out vs oracle (bf16 features)")


def test_fp32_carry_softmax_map_d128():
    # The per-half softmax map at d = 128 runs on the fused kernels, which normalise each token's
    # features themselves (per-wave maxima and sums combined across waves); its segment hand-offs
    # are the same fp32 slots.  Same two checks as above.
    m = hh()
    w = wl.CONFIGS["c3_llama2_softmax_map"].replace(B=1, H=1, seed=9811)
    say("fp32 carry, softmax map per half d=128: one head alone (many segments) vs in a 256-head batch")
    x = wl.make_inputs(w)
    q, k, v, W = (dev(x[n]) for n in ("q", "k", "v", "W"))
    y1, S1, z1 = m.hh_linattn_fwd(q, k, v, W, None, map=w.map, want_state=True)
    rep = lambda t: t.expand(256, -1, -1, -1).contiguous()  # noqa: E731
    y2, S2, z2 = m.hh_linattn_fwd(rep(q), rep(k), rep(v), W, None, map=w.map, want_state=True)
    torch.cuda.synchronize()
    assert m.hh_linattn_fwd_workspace(w.map, w.dtype, 1, 1, 1, w.N, w.d) > 0, "the single head must be cut into segments"
    assert m.hh_linattn_fwd_workspace(w.map, w.dtype, 1, 256, 1, w.N, w.d) == 0, "one segment per sequence, no features in memory"
    assert torch.equal(S2[:1].expand(256, -1, -1, -1), S2)
    Sa, Sb = host(S1)[0, 0], host(S2)[0, 0]
    za, zb = host(z1)[0, 0], host(z2)[0, 0]
    e_s, e_z = normwise(Sa, Sb), normwise(za, zb)
    print(f"  segmented vs one segment: S normwise {e_s:.3e}, z normwise {e_z:.3e}", flush=True)
    # The segment-state pass and the chunked pass form a key's features with different partial
    # maxima (8 waves of 16 directions vs 2 of 64), so a feature's last bf16 bit can differ between
    # the two runs: up to a few 1e-5 normwise, where a bf16 hand-off of the aggregates gives ~1e-3.
    assert e_s <= 1e-4 and e_z <= 1e-4
    rtol, atol = wl.tolerance(w.dtype)
    close(host(y1)[0, 0], host(y2)[0, 0], rtol, atol, "y segmented vs one segment")
    # each half of every feature vector sums to 1, so z_out sums to N per half up to the bf16
    # rounding of the features
    assert abs(za[:w.d].sum() / w.N - 1.0) < 2e-3 and abs(za[w.d:].sum() / w.N - 1.0) < 2e-3
    phik = bf16(oracle.featuremap(w.map, x["k"], x["W"], None))
    phiq = bf16(oracle.featuremap(w.map, x["q"], x["W"], None))
    _, So, zo = oracle.causal_features(phiq, phik, x["v"], want_state=True)
    for what, Sx, zx in (("segmented", Sa, za), ("one segment", Sb, zb)):
        e_so, e_zo = normwise(Sx, So[0, 0]), normwise(zx, zo[0, 0])
        print(f"  {what} vs oracle sums of bf16 features: S normwise {e_so:.3e}, z normwise {e_zo:.3e}", flush=True)
        assert e_so <= 1e-4 and e_zo <= 1e-4
        close(Sx, So[0, 0], 1e-3, 1e-4 * float(np.abs(So).max()), f"S_out {what} vs oracle (bf16 features)")


@pytest.mark.parametrize("d,B,H", [(128, 1, 4), (64, 2, 3)])
def test_nan_in_values_stays_causal(d, B, H):
    m = hh()
    N = 1500
    w = wl.CONFIGS["c3_llama2_causal"].replace(B=B, H=H, N=N, d=d, w_std=d ** -0.5, seed=9800 + d)
    x = wl.make_inputs(w)
    # NaN entries: mid-block, first row of a block, a later segment, and the last token
    spots = [(0, 0, 37, 5), (0, min(1, H - 1), 64, 0), (B - 1, H - 1, 1100, d - 1), (0, 0, N - 1, 3)]
    say(f"NaN containment d={d} B={B} H={H} N={N} spots={spots}")
    v_nan = x["v"].copy()
    v_zero = x["v"].copy()
    for bb, hh_, j, c in spots:
        v_nan[bb, hh_, j, c] = np.nan
        v_zero[bb, hh_, j, c] = 0.0
    W, b = dev(x["W"]), dev(x["b"])
    q, k = dev(x["q"]), dev(x["k"])
    y_nan = host(m.hh_linattn_fwd(q, k, dev(v_nan), W, b))
    y_ref = host(m.hh_linattn_fwd(q, k, dev(v_zero), W, b))
    torch.cuda.synchronize()
    yo = oracle.causal(w.map, x["q"], x["k"], v_nan, x["W"], x["b"])
    rtol, atol = wl.tolerance(w.dtype)
    for bb in range(B):
        for hh_ in range(H):
            mine = [(j, c) for (b2, h2, j, c) in spots if (b2, h2) == (bb, hh_)]
            expect_nan = np.zeros((N, d), bool)
            for j, c in mine:
                expect_nan[j:, c] = True
            assert np.array_equal(np.isnan(yo[bb, hh_]), expect_nan), "oracle: NaN exactly at i >= j, column c"
            g = y_nan[bb, hh_]
            got_nan = np.isnan(g)
            assert not np.isinf(g).any()
            allowed = expect_nan.copy()
            for j, c in mine:
                allowed[32 * (j // 32):, c] = True
            assert not (got_nan & ~allowed).any(), f"NaN outside its column / before its block (b={bb}, h={hh_})"
            assert got_nan[expect_nan].all(), f"missing NaN at i >= j (b={bb}, h={hh_})"
            first = min([32 * (j // 32) for j, _ in mine], default=N)
            # rows before the earliest poisoned block: identical to the run without the NaN
            assert np.array_equal(g[:first], y_ref[bb, hh_][:first])
            fin = ~allowed
            err = np.abs(g[fin] - yo[bb, hh_][fin])
            assert (err <= atol + rtol * np.abs(yo[bb, hh_][fin])).all()


def test_decode_chain_4096_steps_d128():
    m = hh()
    w = wl.CONFIGS["c3_llama2_causal"].replace(B=1, H=2, N=4096, seed=9900)
    say("4096 chained decode steps, B1 H2 d128, against the oracle forward")
    x = wl.make_inputs(w)
    dt = torch.bfloat16
    # token-major copies so that step i reads contiguous [B,H,d] slices
    qs, ks, vs = (dev(np.ascontiguousarray(x[n].transpose(2, 0, 1, 3)), dt) for n in ("q", "k", "v"))
    W, b = dev(x["W"]), dev(x["b"])
    dp = 2 * w.d
    S = torch.zeros((w.B, w.H, dp, w.d), dtype=torch.float32, device="cuda")
    z = torch.zeros((w.B, w.H, dp), dtype=torch.float32, device="cuda")
    ys = torch.empty((w.N, w.B, w.H, w.d), dtype=dt, device="cuda")
    for i in range(w.N):
        m.hh_linattn_decode_step(qs[i], ks[i], vs[i], W, b, S, z, out=ys[i])
    torch.cuda.synchronize()
    y = host(ys).transpose(1, 2, 0, 3)
    yo, So, zo = oracle.causal(w.map, x["q"], x["k"], x["v"], x["W"], x["b"], want_state=True)
    rtol, atol = wl.tolerance(w.dtype)
    close(y, yo, rtol, atol, "decode chain y")
    # the decode step maps features in fp32 and sums in fp32: 4096 steps of fp32 rounding
    close(S.cpu().numpy(), So, 1e-3, 1e-5 * float(np.abs(So).max()), "decode chain S")
    close(z.cpu().numpy(), zo, 1e-4, 0.0, "decode chain z")
    assert normwise(S.cpu().numpy(), So) <= 1e-5
