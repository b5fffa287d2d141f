"""ctypes loader for libhh.so.  Fails loudly when the library has not been built."""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhh.so")

HH_OK, HH_EINVAL, HH_EUNSUPPORTED, HH_EWORKSPACE, HH_EHIP = 0, 1, 2, 3, 4
HH_F32, HH_BF16 = 0, 1
HH_MAP_HEDGEHOG, HH_MAP_TAYLOR2, HH_MAP_HEDGEHOG_SOFTMAX, HH_MAP_EXP, HH_MAP_SOFTMAX, HH_MAP_QUADRATIC = 0, 1, 2, 3, 4, 5

# Every function declared in include/hh.h.
EXPORTS = ("hh_abi_version", "hh_feature_dim", "hh_featuremap", "hh_linattn_fwd_workspace",
           "hh_linattn_fwd", "hh_linattn_fwd_noalloc", "hh_linattn_bwd_workspace", "hh_linattn_bwd",
           "hh_linattn_decode_step", "hh_distill_loss_workspace", "hh_distill_loss",
           "hh_status_str", "hh_last_error")


class LibraryMissing(RuntimeError):
    pass


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    # libhh links libamdhip64.so.7.  torch ships its own copy of the HIP runtime; if torch
    # is imported after libhh, the process ends up with two runtimes and the second one sees
    # no device.  Importing torch first makes libhh bind to the runtime torch already loaded
    # (same soname), so there is one runtime per process.
    try:
        import torch  # noqa: F401
    except ImportError:  # plain C/ctypes use without torch: libhh brings its own runtime
        pass
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} is missing: build it with "
                             "`python -m softmax_mimicking_feature_amd.build` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    I, P, Z = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.hh_abi_version.argtypes = []
    lib.hh_abi_version.restype = I
    lib.hh_feature_dim.argtypes = [I, I]
    lib.hh_feature_dim.restype = I
    lib.hh_featuremap.argtypes = [I, I, I, I, I, I, P, P, P, P, P]
    lib.hh_featuremap.restype = I
    lib.hh_linattn_fwd_workspace.argtypes = [I, I, I, I, I, I, I]
    lib.hh_linattn_fwd_workspace.restype = Z
    lib.hh_linattn_fwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.hh_linattn_fwd.restype = I
    lib.hh_linattn_fwd_noalloc.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P]
    lib.hh_linattn_fwd_noalloc.restype = I
    lib.hh_linattn_bwd_workspace.argtypes = [I, I, I, I, I, I, I]
    lib.hh_linattn_bwd_workspace.restype = Z
    lib.hh_linattn_bwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
    lib.hh_linattn_bwd.restype = I
    lib.hh_linattn_decode_step.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P]
    lib.hh_linattn_decode_step.restype = I
    lib.hh_distill_loss_workspace.argtypes = [I, I, I, I, I, I]
    lib.hh_distill_loss_workspace.restype = Z
    lib.hh_distill_loss.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, Z, P]
    lib.hh_distill_loss.restype = I
    lib.hh_status_str.argtypes = [I]
    lib.hh_status_str.restype = ctypes.c_char_p
    lib.hh_last_error.argtypes = []
    lib.hh_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib
