"""Hedgehog-style linear attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of libhh (include/hh.h), with the same
entry-point names.  It only marshals arguments: torch supplies device memory
and the current stream, every step of the computation runs in the HIP
kernels of libhh.  There is no fallback: if libhh.so is missing, every call
raises.

    y = hh_linattn_fwd(q, k, v, W, b, causal=True)            # [B,H,N,d]
    y, S, z = hh_linattn_fwd(q, k, v, W, b, want_state=True)   # + final fp32 state
    y = hh_linattn_decode_step(q1, k1, v1, W, b, S, z)         # S, z updated in place
    phi = hh_featuremap(x, W, b)                               # [B,H,N,d']
    loss = hh_distill_loss(q, k, W, b)                         # [B,H,N] per-query Eq. 4 loss
"""

from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import (HH_BF16, HH_EHIP, HH_EINVAL, HH_EUNSUPPORTED, HH_EWORKSPACE, HH_F32, HH_MAP_EXP, HH_MAP_HEDGEHOG,
                   HH_MAP_HEDGEHOG_SOFTMAX, HH_MAP_QUADRATIC, HH_MAP_SOFTMAX, HH_MAP_TAYLOR2, HH_OK, LibraryMissing)

__all__ = ["hh_feature_dim", "hh_featuremap", "hh_linattn_fwd_workspace", "hh_linattn_fwd", "hh_linattn_fwd_noalloc",
           "hh_linattn_bwd_workspace", "hh_linattn_bwd",
           "hh_linattn_decode_step", "hh_distill_loss_workspace", "hh_distill_loss", "hh_status_str", "hh_last_error", "hh_abi_version", "HHError",
           "LibraryMissing", "HH_F32", "HH_BF16", "HH_MAP_HEDGEHOG", "HH_MAP_TAYLOR2", "HH_MAP_HEDGEHOG_SOFTMAX",
           "HH_MAP_EXP", "HH_MAP_SOFTMAX", "HH_MAP_QUADRATIC", "HH_OK", "HH_EINVAL",
           "HH_EUNSUPPORTED", "HH_EWORKSPACE", "HH_EHIP"]


class HHError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _check(status: int) -> None:
    if status != HH_OK:
        lib = _lib.load()
        raise HHError(status, f"{lib.hh_status_str(status).decode()}: {lib.hh_last_error().decode()}")


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HH_BF16
    if t.dtype == torch.float32:
        return HH_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _dev(t, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _map_params(map: int, W, b, H: int, d: int):
    """Check W and b for a map (W [H,d,d] for every map with a W, b [H,d] or None where the map has
    a bias, None for the softmax maps; for the generalised quadratic map W is the coefficients
    (a, b, c) of each head, [H,3]); returns them, or (None, None) for the Taylor map."""
    if map == HH_MAP_TAYLOR2:
        return None, None
    if W is None:
        raise ValueError(f"W is required for map {map}")
    if map == HH_MAP_QUADRATIC:
        _shape(W, "W", (H, 3))
        if b is not None:
            raise ValueError("the quadratic map has no bias: b must be None")
        return W, None
    _shape(W, "W", (H, d, d))
    if map in (HH_MAP_HEDGEHOG_SOFTMAX, HH_MAP_SOFTMAX):
        if b is not None:
            raise ValueError("the softmax maps have no bias: b must be None")
    else:
        _shape(b, "b", (H, d))
    return W, b


def _w_dtype(map: int, dtype):
    """Element type of W: the generalised quadratic map's coefficients are fp32 in every dtype."""
    return _torch().float32 if map == HH_MAP_QUADRATIC else dtype


def _shape(t, name: str, shape) -> None:
    """Host-side size check: the C ABI receives raw pointers and cannot tell an undersized
    buffer from a valid one, so every tensor's shape is checked before anything is launched."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def hh_abi_version() -> int:
    return _lib.load().hh_abi_version()


def hh_feature_dim(map: int, d: int) -> int:
    return _lib.load().hh_feature_dim(map, d)


def hh_status_str(status: int) -> str:
    return _lib.load().hh_status_str(status).decode()


def hh_last_error() -> str:
    return _lib.load().hh_last_error().decode()


def hh_featuremap(x, W=None, b=None, *, map: int = HH_MAP_HEDGEHOG, out=None, stream=None):
    """phi(x) for x [B,H,N,d]; returns [B,H,N,d'] in x's dtype."""
    lib = _lib.load()
    torch = _torch()
    if x.dim() != 4:
        raise ValueError(f"x must be [B,H,N,d], got {list(x.shape)}")
    B, H, N, d = x.shape
    dp = lib.hh_feature_dim(map, d)
    if dp < 0:
        raise ValueError(f"invalid map/head dim ({map}, {d})")
    W, b = _map_params(map, W, b, H, d)
    _shape(out, "out", (B, H, N, dp))
    _dev(x, "x")
    if out is None:
        out = torch.empty((B, H, N, dp), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype)
    _dev(W, "W", _w_dtype(map, x.dtype))
    _dev(b, "b", x.dtype)
    _check(lib.hh_featuremap(map, _dtype_code(x), B, H, N, d, _ptr(x), _ptr(W), _ptr(b), _ptr(out),
                             _stream(stream)))
    return out


def hh_linattn_fwd_workspace(map: int, dtype: int, causal: bool, B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().hh_linattn_fwd_workspace(map, dtype, int(bool(causal)), B, H, N, d))


def hh_linattn_fwd(q, k, v, W=None, b=None, *, causal: bool = True, map: int = HH_MAP_HEDGEHOG, S0=None, z0=None,
                   out=None, want_state: bool = False, S_out=None, z_out=None, workspace=None, stream=None):
    """Eq. 2 forward with the feature map included.  q, k, v: [B,H,N,d].

    Returns y, or (y, S_out, z_out) when want_state (fp32 final state)."""
    lib = _lib.load()
    torch = _torch()
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,N,d], got {list(q.shape)}")
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape [B,H,N,d]")
    dp = lib.hh_feature_dim(map, d)
    if dp < 0:
        raise ValueError(f"invalid map/head dim ({map}, {d})")
    W, b = _map_params(map, W, b, H, d)
    _shape(out, "out", q.shape)
    for t, nm in ((S0, "S0"), (S_out, "S_out")):
        _shape(t, nm, (B, H, dp, d))
    for t, nm in ((z0, "z0"), (z_out, "z_out")):
        _shape(t, nm, (B, H, dp))
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm, q.dtype)
    dt = _dtype_code(q)
    _dev(W, "W", _w_dtype(map, q.dtype))
    _dev(b, "b", q.dtype)
    _dev(S0, "S0", torch.float32)
    _dev(z0, "z0", torch.float32)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if want_state and S_out is None:
        S_out = torch.empty((B, H, dp, d), dtype=torch.float32, device=q.device)
        z_out = torch.empty((B, H, dp), dtype=torch.float32, device=q.device)
    _dev(S_out, "S_out", torch.float32)
    _dev(z_out, "z_out", torch.float32)
    need = lib.hh_linattn_fwd_workspace(map, dt, int(bool(causal)), B, H, N, d)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.hh_linattn_fwd(map, dt, int(bool(causal)), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b),
                              _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_out), _ptr(z_out), _ptr(workspace), ws_bytes,
                              _stream(stream)))
    if S_out is not None:
        return out, S_out, z_out
    return out


def hh_linattn_fwd_noalloc(q, k, v, W=None, b=None, *, causal: bool = True, map: int = HH_MAP_HEDGEHOG, S0=None,
                           z0=None, out=None, S_out=None, z_out=None, stream=None):
    """hh_linattn_fwd with the library's own scratch instead of a workspace: allocates nothing
    when `out` (and S_out, z_out if wanted) are given.  Returns out, or (out, S_out, z_out)."""
    lib = _lib.load()
    torch = _torch()
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,N,d], got {list(q.shape)}")
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape [B,H,N,d]")
    dp = lib.hh_feature_dim(map, d)
    if dp < 0:
        raise ValueError(f"invalid map/head dim ({map}, {d})")
    W, b = _map_params(map, W, b, H, d)
    _shape(out, "out", q.shape)
    for t, nm in ((S0, "S0"), (S_out, "S_out")):
        _shape(t, nm, (B, H, dp, d))
    for t, nm in ((z0, "z0"), (z_out, "z_out")):
        _shape(t, nm, (B, H, dp))
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm, q.dtype)
    dt = _dtype_code(q)
    _dev(W, "W", _w_dtype(map, q.dtype))
    _dev(b, "b", q.dtype)
    for t, nm in ((S0, "S0"), (z0, "z0"), (S_out, "S_out"), (z_out, "z_out")):
        _dev(t, nm, torch.float32)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    _check(lib.hh_linattn_fwd_noalloc(map, dt, int(bool(causal)), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(W),
                                      _ptr(b), _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_out), _ptr(z_out),
                                      _stream(stream)))
    if S_out is not None:
        return out, S_out, z_out
    return out


def hh_linattn_bwd_workspace(map: int, dtype: int, causal: bool, B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().hh_linattn_bwd_workspace(map, dtype, int(bool(causal)), B, H, N, d))


def hh_linattn_bwd(q, k, v, W, b, y, dy, *, causal: bool = True, map: int = HH_MAP_HEDGEHOG, dq=None, dk=None,
                   dv=None, dW=None, db=None, workspace=None, stream=None):
    """Backward of hh_linattn_fwd given y (its output) and dy = dL/dy, all [B,H,N,d] bf16.

    Returns (dq, dk, dv, dW, db): dq, dk, dv bf16 [B,H,N,d]; dW [H,d,d] and db [H,d] fp32 (db
    None for the maps without a bias or when b is None)."""
    lib = _lib.load()
    torch = _torch()
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,N,d], got {list(q.shape)}")
    B, H, N, d = q.shape
    for t, nm in ((k, "k"), (v, "v"), (y, "y"), (dy, "dy"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _shape(t, nm, q.shape)
    W, b = _map_params(map, W, b, H, d)
    if W is None:
        raise ValueError("the backward needs a map with a W")
    has_db = b is not None
    _shape(dW, "dW", (H, d, d))
    _shape(db, "db", (H, d))
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (y, "y"), (dy, "dy")):
        _dev(t, nm, q.dtype)
    dt = _dtype_code(q)
    _dev(W, "W", _w_dtype(map, q.dtype))
    _dev(b, "b", q.dtype)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    dW = torch.empty((H, d, d), dtype=torch.float32, device=q.device) if dW is None else dW
    if has_db and db is None:
        db = torch.empty((H, d), dtype=torch.float32, device=q.device)
    if not has_db:
        db = None
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _dev(t, nm, q.dtype)
    _dev(dW, "dW", torch.float32)
    _dev(db, "db", torch.float32)
    need = lib.hh_linattn_bwd_workspace(map, dt, int(bool(causal)), B, H, N, d)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.hh_linattn_bwd(map, dt, int(bool(causal)), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b),
                              _ptr(y), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), _ptr(db), _ptr(workspace),
                              ws_bytes, _stream(stream)))
    return dq, dk, dv, dW, db


def hh_linattn_decode_step(q, k, v, W, b, S, z, *, map: int = HH_MAP_HEDGEHOG, out=None, stream=None):
    """One recurrent step.  q, k, v: [B,H,d] or [B,H,1,d]; S [B,H,d',d], z [B,H,d'] fp32 updated in place."""
    lib = _lib.load()
    torch = _torch()
    if q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[2] != 1):
        raise ValueError(f"decode expects q of shape [B,H,d] or [B,H,1,d], got {list(q.shape)}")
    B, H = q.shape[:2]
    d = q.shape[-1]
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    dp = lib.hh_feature_dim(map, d)
    if dp < 0:
        raise ValueError(f"invalid map/head dim ({map}, {d})")
    W, b = _map_params(map, W, b, H, d)
    _shape(S, "S", (B, H, dp, d))
    _shape(z, "z", (B, H, dp))
    if out is not None and out.numel() != B * H * d:
        raise ValueError(f"out must hold B*H*d = {B * H * d} elements, got {list(out.shape)}")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm, q.dtype)
    dt = _dtype_code(q)
    _dev(W, "W", _w_dtype(map, q.dtype))
    _dev(b, "b", q.dtype)
    _dev(S, "S", torch.float32)
    _dev(z, "z", torch.float32)
    if out is None:
        out = torch.empty((B, H, d), dtype=q.dtype, device=q.device)
    _dev(out, "out", q.dtype)
    _check(lib.hh_linattn_decode_step(map, dt, B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(b), _ptr(S),
                                      _ptr(z), _ptr(out), _stream(stream)))
    return out


def hh_distill_loss_workspace(map: int, dtype: int, B: int, H: int, N: int, d: int) -> int:
    return int(_lib.load().hh_distill_loss_workspace(map, dtype, B, H, N, d))


def hh_distill_loss(q, k, W=None, b=None, *, map: int = HH_MAP_HEDGEHOG, out=None, workspace=None, stream=None):
    """Attention-weight distillation loss (Eq. 4) per query.  q, k: [B,H,N,d] bf16 -> loss [B,H,N] fp32."""
    lib = _lib.load()
    torch = _torch()
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,N,d], got {list(q.shape)}")
    B, H, N, d = q.shape
    if k.shape != q.shape:
        raise ValueError("q and k must have the same shape [B,H,N,d]")
    W, b = _map_params(map, W, b, H, d)
    _shape(out, "out", (B, H, N))
    for t, nm in ((q, "q"), (k, "k")):
        _dev(t, nm, q.dtype)
    dt = _dtype_code(q)
    _dev(W, "W", _w_dtype(map, q.dtype))
    _dev(b, "b", q.dtype)
    if out is None:
        out = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    need = lib.hh_distill_loss_workspace(map, dt, B, H, N, d)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.hh_distill_loss(map, dt, B, H, N, d, _ptr(q), _ptr(k), _ptr(W), _ptr(b), _ptr(out), _ptr(workspace),
                               ws_bytes, _stream(stream)))
    return out
