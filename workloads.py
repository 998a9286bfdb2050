"""Seeded synthetic inputs for starting-node triangular self-attention.

This module only draws random numbers and rounds them to the storage type;
it holds none of the method's arithmetic, so both the CPU oracle and the GPU
path can take their inputs from it without sharing any computation.

Shapes follow the benchmark problem the two l2_p6 transcripts work on
(POPCORNBENCH, problem l2_p6: pair representation (B, N, N, D), pair mask
(B, N, N), parameters in nn.LayerNorm / nn.Linear layouts). The default size
of that problem is the first workload below (B=2, N=32, D=64, h=4). The other
four workloads widen it to the sizes the build is measured on.

Recipe (fixed, so that results are reproducible):

* generator: numpy ``Generator(PCG64(seed))``; the default seed of workload k
  is ``1000 + k``;
* draw order: pair_repr, mask, ln gamma, ln beta, Wq, Wk, Wv, Wg, bg, Wz, Wo,
  bo;
* pair_repr ~ N(0, 1); gamma = 1 + 0.1 N(0, 1); beta = 0.1 N(0, 1);
  every weight matrix ~ N(0, 1/D) (standard deviation 1/sqrt(D));
  every bias ~ N(0, 0.02) (standard deviation sqrt(0.02));
* all draws are float32; for bf16 workloads every array is then rounded to
  bfloat16 with round-to-nearest-even, so that the oracle (which widens them
  to float64) and the GPU see bit-identical values;
* masks are uint8 with 1 = attend, 0 = masked:
  - ``bernoulli``: i.i.d. Bernoulli(p) per (b, j, k), then the diagonal is set
    to 1 so that every query column has a valid key;
  - ``pad``: a valid length L per batch, mask[b, j, k] = (j < L and k < L);
    L is fixed, or drawn per batch uniformly from an inclusive range.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "make_inputs",
    "round_to_bf16",
    "WEIGHT_NAMES",
]

# Parameter names in the order of the C-ABI weight struct.
WEIGHT_NAMES = (
    "ln_weight",
    "ln_bias",
    "w_query",
    "w_key",
    "w_value",
    "w_gate",
    "b_gate",
    "w_bias_proj",
    "w_out",
    "b_out",
)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One input configuration: shapes, storage type and mask recipe."""

    name: str
    B: int
    N: int
    D: int
    h: int
    dtype: str  # "f32" or "bf16"
    mask: Tuple  # ("bernoulli", p) | ("pad", L) | ("pad_range", lo, hi) | ("ones",)
    seed: int = 0

    @property
    def d(self) -> int:
        return self.D // self.h

    @property
    def positions(self) -> int:
        return self.B * self.N * self.N

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload("c1_B2_N32_D64_h4_f32", 2, 32, 64, 4, "f32", ("bernoulli", 0.9), 1001),
    2: Workload("c2_B1_N128_D128_h4_f32", 1, 128, 128, 4, "f32", ("bernoulli", 0.9), 1002),
    3: Workload("c3_B1_N256_D128_h4_bf16", 1, 256, 128, 4, "bf16", ("pad", 240), 1003),
    4: Workload("c4_B1_N384_D128_h4_bf16", 1, 384, 128, 4, "bf16", ("bernoulli", 0.95), 1004),
    5: Workload("c5_B4_N512_D128_h8_bf16", 4, 512, 128, 8, "bf16", ("pad_range", 384, 512), 1005),
}


def workload(k: int) -> Workload:
    return WORKLOADS[k]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs here are always finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    u = ((u + bias) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _mask(rng: np.random.Generator, B: int, N: int, spec: Sequence) -> np.ndarray:
    kind = spec[0]
    if kind == "ones":
        return np.ones((B, N, N), dtype=np.uint8)
    if kind == "bernoulli":
        m = (rng.random((B, N, N), dtype=np.float32) < np.float32(spec[1])).astype(np.uint8)
        idx = np.arange(N)
        m[:, idx, idx] = 1
        return m
    if kind in ("pad", "pad_range"):
        if kind == "pad":
            lengths = np.full(B, int(spec[1]), dtype=np.int64)
        else:
            lengths = rng.integers(int(spec[1]), int(spec[2]), size=B, endpoint=True)
        lengths = np.minimum(lengths, N)
        r = np.arange(N)
        m = np.zeros((B, N, N), dtype=np.uint8)
        for b in range(B):
            valid = r < lengths[b]
            m[b] = (valid[:, None] & valid[None, :]).astype(np.uint8)
        return m
    if kind == "zeros":
        return np.zeros((B, N, N), dtype=np.uint8)
    raise ValueError(f"unknown mask recipe {spec!r}")


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw one workload's inputs.

    Returns a dict with float32 numpy arrays ``pair_repr`` (B,N,N,D) and every
    name in ``WEIGHT_NAMES`` (nn.Linear layout: weight (out, in)), plus the
    uint8 ``pair_mask`` (B,N,N), ``num_heads`` and ``dtype``. For bf16
    workloads every float array already holds bf16-representable values.
    """
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    B, N, D, h = w.B, w.N, w.D, w.h
    if D % h:
        raise ValueError("pair_dim must be divisible by num_heads")
    f32 = np.float32
    w_std = f32(1.0 / np.sqrt(D))
    b_std = f32(np.sqrt(0.02))

    def normal(shape, std=f32(1.0)):
        return rng.standard_normal(shape, dtype=f32) * std

    out = {}
    out["pair_repr"] = normal((B, N, N, D))
    out["pair_mask"] = _mask(rng, B, N, w.mask)
    out["ln_weight"] = f32(1.0) + f32(0.1) * normal((D,))
    out["ln_bias"] = f32(0.1) * normal((D,))
    out["w_query"] = normal((D, D), w_std)
    out["w_key"] = normal((D, D), w_std)
    out["w_value"] = normal((D, D), w_std)
    out["w_gate"] = normal((D, D), w_std)
    out["b_gate"] = normal((D,), b_std)
    out["w_bias_proj"] = normal((h, D), w_std)
    out["w_out"] = normal((D, D), w_std)
    out["b_out"] = normal((D,), b_std)
    if w.dtype == "bf16":
        for k, v in list(out.items()):
            if v.dtype == np.float32:
                out[k] = round_to_bf16(v)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    for k, v in out.items():
        out[k] = np.ascontiguousarray(v)
    out["num_heads"] = h
    out["dtype"] = w.dtype
    return out
