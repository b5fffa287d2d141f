"""hh_linattn_fwd_noalloc (the forward with the library's own scratch instead of a caller
workspace) against hh_linattn_fwd, through the C ABI: the same kernels run, so the outputs
and final states must be identical bit for bit.  Two calls in a row, the second with a smaller
problem (the scratch keeps the first call's contents), for d = 128 and d = 64, causal and
bidirectional, and the per-half softmax map at d = 128 (whose kernels form its features)."""

import sys

import numpy as np
import pytest

from softmax_mimicking_feature_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("d,causal,map_", [(128, True, wl.MAP_HEDGEHOG), (64, True, wl.MAP_HEDGEHOG),
                                           (64, False, wl.MAP_HEDGEHOG), (128, True, wl.MAP_HEDGEHOG_SOFTMAX)])
def test_noalloc_matches_workspace_forward(d, causal, map_):
    import softmax_mimicking_feature_amd as m
    for i, (B, H, N) in enumerate([(1, 32, 4096), (1, 4, 1000)]):
        w = wl.CONFIGS["c3_llama2_causal"].replace(B=B, H=H, N=N, d=d, w_std=d ** -0.5, seed=9950 + i + d,
                                                    causal=causal, map=map_)
        say(f"noalloc call {i + 1}: map {map_} B{B} H{H} N{N} d{d} causal={causal}")
        need = m.hh_linattn_fwd_workspace(w.map, w.dtype, int(causal), B, H, N, d)
        assert need > 0, "the case must use segment slots"
        x = wl.make_inputs(w)
        q, k, v, W, b = (dev(x[n]) for n in ("q", "k", "v", "W", "b"))
        if map_ != wl.MAP_HEDGEHOG:
            b = None  # the softmax maps take no bias
        if causal:
            y0, S0, z0 = m.hh_linattn_fwd(q, k, v, W, b, map=map_, want_state=True)
            y1 = torch.empty_like(q)
            S1, z1 = torch.empty_like(S0), torch.empty_like(z0)
            m.hh_linattn_fwd_noalloc(q, k, v, W, b, map=map_, out=y1, S_out=S1, z_out=z1)
            torch.cuda.synchronize()
            assert torch.equal(y0, y1) and torch.equal(S0, S1) and torch.equal(z0, z1)
        else:
            y0 = m.hh_linattn_fwd(q, k, v, W, b, causal=False)
            y1 = torch.empty_like(q)
            m.hh_linattn_fwd_noalloc(q, k, v, W, b, causal=False, out=y1)
            torch.cuda.synchronize()
            assert torch.equal(y0, y1)
