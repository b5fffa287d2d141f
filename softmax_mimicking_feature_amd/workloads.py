"""Seeded synthetic inputs for the Hedgehog linear-attention path.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no feature map, no attention), so
that both the HIP library and the CPU oracle can be fed the same bytes without
sharing any computation.

Workload shapes follow the model families that the Hedgehog paper evaluates
("The Hedgehog & the Porcupine: Expressive Linear Attentions with Softmax
Mimicry", Experiments: GPT-2 125M with 12 heads of dimension 64, BERT-base,
Llama-2 7B with 32 heads of dimension 128) and its degree-2 Taylor baseline
(head dimension 16 gives d' = 1 + 16 + 256).  The pages evaluate on
WikiText-103, GLUE and SAMSum; those datasets and trained weights are not
used here: i.i.d. Gaussian inputs of the same shapes stand in for them, since
kernel cost depends only on shapes and parity is checked against the oracle
on identical inputs.

Drawing order (fixed): q, k, v, W, b, each a block of standard normals from
``numpy.random.default_rng(seed)`` (PCG64), scaled, cast to float32, and for
bf16 workloads rounded to bfloat16 with round-to-nearest-even on the host.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

MAP_HEDGEHOG = 0
MAP_TAYLOR2 = 1
MAP_HEDGEHOG_SOFTMAX = 2
MAP_EXP = 3
MAP_SOFTMAX = 4
MAP_QUADRATIC = 5
DT_F32 = 0
DT_BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    map: int            # MAP_HEDGEHOG, MAP_TAYLOR2, MAP_HEDGEHOG_SOFTMAX, MAP_EXP, MAP_SOFTMAX or MAP_QUADRATIC
    dtype: int          # DT_F32 or DT_BF16
    causal: bool
    B: int
    H: int
    N: int
    d: int
    seed: int
    qk_scale: float     # multiplier on N(0,1) draws for q and k
    v_scale: float      # multiplier on N(0,1) draws for v
    w_std: float        # std of W entries (0 for the Taylor map: no W)
    b_std: float        # std of b entries
    description: str = ""

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _cfg() -> Dict[str, Workload]:
    c = {}
    c["c1_tiny_f32"] = Workload(
        "c1_tiny_f32", MAP_HEDGEHOG, DT_F32, True, B=1, H=1, N=256, d=16, seed=1001,
        qk_scale=1.0, v_scale=1.0, w_std=16 ** -0.5, b_std=0.0,
        description="tiny causal Hedgehog, fp32, B1 H1 N256 d16 d'32")
    c["c2_gpt2_causal"] = Workload(
        "c2_gpt2_causal", MAP_HEDGEHOG, DT_BF16, True, B=8, H=12, N=1024, d=64, seed=1002,
        qk_scale=1.0, v_scale=1.0, w_std=64 ** -0.5, b_std=0.1,
        description="GPT-2-125M-shaped causal, bf16, B8 H12 N1024 d64 d'128")
    c["c2_gpt2_softmax_map"] = Workload(
        "c2_gpt2_softmax_map", MAP_HEDGEHOG_SOFTMAX, DT_BF16, True, B=8, H=12, N=1024, d=64, seed=1002,
        qk_scale=1.0, v_scale=1.0, w_std=64 ** -0.5, b_std=0.0,
        description="GPT-2-125M-shaped causal with the softmax-over-features map per half (no bias), bf16, "
                    "B8 H12 N1024 d64 d'128")
    s3 = 128 ** -0.25
    c["c3_llama2_causal"] = Workload(
        "c3_llama2_causal", MAP_HEDGEHOG, DT_BF16, True, B=1, H=32, N=4096, d=128, seed=1003,
        qk_scale=s3, v_scale=s3, w_std=128 ** -0.5, b_std=0.0,
        description="Llama-2-7B-shaped causal, bf16, B1 H32 N4096 d128 d'256")
    c["c3_llama2_decode"] = Workload(
        "c3_llama2_decode", MAP_HEDGEHOG, DT_BF16, True, B=16, H=32, N=4096, d=128, seed=2003,
        qk_scale=s3, v_scale=s3, w_std=128 ** -0.5, b_std=0.0,
        description="Llama-2-7B-shaped decode step over a 4096-token fp32 state, batch 16")
    c["c3_llama2_distill"] = Workload(
        "c3_llama2_distill", MAP_HEDGEHOG, DT_BF16, True, B=1, H=32, N=4096, d=128, seed=1003,
        qk_scale=s3, v_scale=s3, w_std=128 ** -0.5, b_std=0.0,
        description="attention-weight distillation loss (Eq. 4) at the Llama-2-7B head shapes, bf16, "
                    "B1 H32 N4096 d128 (the causal workload's inputs; v unused)")
    c["c3_llama2_softmax_map"] = Workload(
        "c3_llama2_softmax_map", MAP_HEDGEHOG_SOFTMAX, DT_BF16, True, B=1, H=32, N=4096, d=128, seed=1003,
        qk_scale=s3, v_scale=s3, w_std=128 ** -0.5, b_std=0.0,
        description="Llama-2-7B-shaped causal with the softmax-over-features map per half (no bias), bf16, "
                    "B1 H32 N4096 d128 d'256 (the causal workload's inputs)")
    c["c3_llama2_backward"] = Workload(
        "c3_llama2_backward", MAP_HEDGEHOG, DT_BF16, True, B=1, H=32, N=4096, d=128, seed=1003,
        qk_scale=s3, v_scale=s3, w_std=128 ** -0.5, b_std=0.0,
        description="backward (dq, dk, dv, dW, db) of the Llama-2-7B-shaped causal forward, bf16, "
                    "B1 H32 N4096 d128 (the causal workload's inputs; dL/dy ~ N(0,1))")
    c["c4_bert_bidir"] = Workload(
        "c4_bert_bidir", MAP_HEDGEHOG, DT_BF16, False, B=32, H=12, N=512, d=64, seed=1004,
        qk_scale=1.0, v_scale=1.0, w_std=64 ** -0.5, b_std=0.0,
        description="BERT-base-shaped bidirectional, bf16, B32 H12 N512 d64 d'128")
    c["c5_taylor_causal"] = Workload(
        "c5_taylor_causal", MAP_TAYLOR2, DT_BF16, True, B=2, H=16, N=8192, d=16, seed=1005,
        qk_scale=16 ** -0.5, v_scale=1.0, w_std=0.0, b_std=0.0,
        description="degree-2 Taylor map causal, bf16, B2 H16 N8192 d16 d'273")
    return c


CONFIGS: Dict[str, Workload] = _cfg()

# Seed of the single decode token that follows the 4096-token prefix.
DECODE_STEP_SEED = 3003


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _store(a: np.ndarray, dtype: int) -> np.ndarray:
    a = a.astype(np.float32)
    return round_to_bf16(a) if dtype == DT_BF16 else a


def make_inputs(w: Workload, *, B: Optional[int] = None, H: Optional[int] = None,
                N: Optional[int] = None, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw q, k, v [B,H,N,d], W [H,d,d] (row = output direction), b [H,d].

    All arrays are float32 holding values exactly representable in the
    workload's storage dtype.  For the Taylor map W and b are returned as
    empty arrays (the map has no parameters); the softmax maps use no b.  For
    the generalised quadratic map W is the fp32 coefficients (a, b, c) of each
    head, [H,3] (never rounded), drawn so that every weight is positive:
    a ~ U(0.5, 1.5), b ~ U(0.2, 1.2), c = b^2 / (4 a) times U(1.5, 3), and b
    is empty.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    seed = w.seed if seed is None else seed
    d = w.d
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)) * w.qk_scale
    k = rng.standard_normal((B, H, N, d)) * w.qk_scale
    v = rng.standard_normal((B, H, N, d)) * w.v_scale
    out = {"q": _store(q, w.dtype), "k": _store(k, w.dtype), "v": _store(v, w.dtype)}
    if w.map == MAP_QUADRATIC:
        a = rng.uniform(0.5, 1.5, H)
        bb = rng.uniform(0.2, 1.2, H)
        c = bb * bb / (4.0 * a) * rng.uniform(1.5, 3.0, H)
        out["W"] = np.stack([a, bb, c], axis=1).astype(np.float32)
        out["b"] = np.zeros((0,), np.float32)
    elif w.map != MAP_TAYLOR2:
        W = rng.standard_normal((H, d, d)) * w.w_std
        b = rng.standard_normal((H, d)) * w.b_std
        out["W"] = _store(W, w.dtype)
        out["b"] = _store(b, w.dtype)
    else:
        out["W"] = np.zeros((0,), np.float32)
        out["b"] = np.zeros((0,), np.float32)
    return out


def make_decode_token(w: Workload, *, B: Optional[int] = None, H: Optional[int] = None,
                      seed: int = DECODE_STEP_SEED) -> Dict[str, np.ndarray]:
    """One new token per (b, h): q, k, v of shape [B,H,1,d], same distributions as the prefix."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    rng = np.random.default_rng(seed)
    d = w.d
    q = rng.standard_normal((B, H, 1, d)) * w.qk_scale
    k = rng.standard_normal((B, H, 1, d)) * w.qk_scale
    v = rng.standard_normal((B, H, 1, d)) * w.v_scale
    return {"q": _store(q, w.dtype), "k": _store(k, w.dtype), "v": _store(v, w.dtype)}


def feature_dim(map_: int, d: int) -> int:
    """Length of a feature vector: 2d (Hedgehog, per-half softmax), 1 + d + d*d (Taylor), d
    (single-sided maps)."""
    if map_ in (MAP_HEDGEHOG, MAP_HEDGEHOG_SOFTMAX):
        return 2 * d
    if map_ in (MAP_TAYLOR2, MAP_QUADRATIC):
        return 1 + d + d * d
    return d


def map_has_bias(map_: int) -> bool:
    """Whether a map takes the bias b (the softmax maps and the Taylor map do not)."""
    return map_ in (MAP_HEDGEHOG, MAP_EXP)


def random_state(w: Workload, *, B: Optional[int] = None, H: Optional[int] = None,
                 seed: int = 7) -> Dict[str, np.ndarray]:
    """A positive synthetic (S, z) pair of plausible magnitude, for edge-case tests.

    Not a state produced by the method: only used where any fp32 state is a
    valid input (resume from a caller-supplied state).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    dp = feature_dim(w.map, w.d)
    rng = np.random.default_rng(seed)
    z = (rng.random((B, H, dp)) + 0.5).astype(np.float32) * 8.0
    S = (rng.standard_normal((B, H, dp, w.d)) * 2.0).astype(np.float32)
    return {"S": S, "z": z}


def tolerance(dtype: int):
    """(rtol, atol) for outputs: bf16 inputs 2e-2 / 1e-2, fp32 inputs 1e-4 / 1e-5."""
    return (2e-2, 1e-2) if dtype == DT_BF16 else (1e-4, 1e-5)


def bytes_per_elem(dtype: int) -> int:
    return 2 if dtype == DT_BF16 else 4
