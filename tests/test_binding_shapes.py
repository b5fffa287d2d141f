"""The Python binding checks every tensor's shape on the host before anything is launched.

The C ABI receives raw pointers and sizes only, so an undersized W, b, output or state buffer
would otherwise be read or written out of bounds by the kernels.  These tests need no GPU:
the shape checks run before the device checks, so a mis-shaped CPU tensor is rejected with a
message naming its expected shape, and a correctly shaped CPU tensor gets past them and is
then rejected as not being on the GPU."""

import pytest

torch = pytest.importorskip("torch")

import softmax_mimicking_feature_amd as hh  # noqa: E402

B, H, N, d = 2, 3, 10, 16
dp = 2 * d


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def good_fwd():
    return dict(q=t(B, H, N, d), k=t(B, H, N, d), v=t(B, H, N, d), W=t(H, d, d), b=t(H, d))


def test_fwd_correct_shapes_pass_to_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        hh.hh_linattn_fwd(**good_fwd())


@pytest.mark.parametrize("arg,bad", [
    ("W", (d, d)),                 # one head's W for H heads
    ("W", (H, d, d // 2)),
    ("b", (d,)),
    ("out", (B, H, N - 1, d)),
    ("S0", (B, H, dp, d - 1)),
    ("z0", (B, H, dp - 1)),
    ("S_out", (B, H, d, d)),       # d' rows missing
    ("z_out", (B, 1, dp)),
])
def test_fwd_rejects_bad_shapes(arg, bad):
    kw = good_fwd()
    dtype = torch.float32 if arg in ("S0", "z0", "S_out", "z_out") else torch.bfloat16
    kw[arg] = t(*bad, dtype=dtype)
    if arg in ("S0", "S_out"):   # the partner must be present and well formed
        kw["z0" if arg == "S0" else "z_out"] = t(B, H, dp, dtype=torch.float32)
    if arg in ("z0", "z_out"):
        kw["S0" if arg == "z0" else "S_out"] = t(B, H, dp, d, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        hh.hh_linattn_fwd(**kw)


def test_fwd_rejects_mismatched_qkv_and_missing_W():
    kw = good_fwd()
    kw["v"] = t(B, H, N + 1, d)
    with pytest.raises(ValueError, match="same shape"):
        hh.hh_linattn_fwd(**kw)
    kw = good_fwd()
    kw["W"] = None
    with pytest.raises(ValueError, match="W is required"):
        hh.hh_linattn_fwd(**kw)


def good_dec():
    return dict(q=t(B, H, d), k=t(B, H, d), v=t(B, H, d), W=t(H, d, d), b=t(H, d),
                S=t(B, H, dp, d, dtype=torch.float32), z=t(B, H, dp, dtype=torch.float32))


def test_decode_correct_shapes_pass_to_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        hh.hh_linattn_decode_step(**good_dec())


@pytest.mark.parametrize("arg,bad", [
    ("W", (d, d)), ("b", (H, d + 1)), ("S", (B, H, d, d)), ("z", (B, H, d)), ("k", (B, H, d - 1)),
    ("v", (B, H + 1, d)), ("out", (B, H, d - 1)),
])
def test_decode_rejects_bad_shapes(arg, bad):
    kw = good_dec()
    dtype = torch.float32 if arg in ("S", "z") else torch.bfloat16
    kw[arg] = t(*bad, dtype=dtype)
    with pytest.raises(ValueError, match="shape|same shape|elements"):
        hh.hh_linattn_decode_step(**kw)


def test_featuremap_and_distill_reject_bad_shapes():
    x = t(B, H, N, d)
    with pytest.raises(ValueError, match="shape"):
        hh.hh_featuremap(x, t(1, d, d), t(H, d))
    with pytest.raises(ValueError, match="shape"):
        hh.hh_featuremap(x, t(H, d, d), t(H, d), out=t(B, H, N, d))
    with pytest.raises(ValueError, match="GPU tensor"):
        hh.hh_featuremap(x, t(H, d, d), t(H, d))
    with pytest.raises(ValueError, match="shape"):
        hh.hh_distill_loss(x, x, t(H, d, d), t(H, d), out=t(B, H, N - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        hh.hh_distill_loss(x, x, t(H, d, 1), t(H, d))
    with pytest.raises(ValueError, match="GPU tensor"):
        hh.hh_distill_loss(x, x, t(H, d, d), t(H, d))


def test_quadratic_map_takes_per_head_coefficients():
    kw = dict(q=t(B, H, N, d), k=t(B, H, N, d), v=t(B, H, N, d), map=hh.HH_MAP_QUADRATIC)
    with pytest.raises(ValueError, match="shape"):
        hh.hh_linattn_fwd(W=t(H, d, d, dtype=torch.float32), **kw)    # a Hedgehog W, not [H,3]
    with pytest.raises(ValueError, match="no bias"):
        hh.hh_linattn_fwd(W=t(H, 3, dtype=torch.float32), b=t(H, d), **kw)
    with pytest.raises(ValueError, match="GPU tensor"):
        hh.hh_linattn_fwd(W=t(H, 3, dtype=torch.float32), **kw)
