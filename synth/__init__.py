"""Seeded synthetic inputs for the streamed AllGather+GEMM workloads.

This module only draws random numbers.  It holds none of the method's
arithmetic, so both the CPU oracle and the HIP path can take their inputs
from it without sharing any computation.

Recipe (numpy ``Generator(PCG64(seed))``):
  * seed = 1000 * case_id + {1: A, 2: B, 3: bias, 4: scale}
  * A is drawn whole (gathered M x K) and then split into n_shards row
    blocks, shard s holding rows [s*S, (s+1)*S) with S = M / n_shards.
  * fp16 values are drawn in float32 (normal or uniform) and rounded to
    float16 with numpy's round-to-nearest-even cast.
  * int8 values are integers in [-127, 127] (both ends included, -128 never
    drawn); bias is an int32 integer in [-1000, 1000]; scale is a float32
    drawn uniformly in [1e-4, 1e-3].

The shapes and distributions follow the workloads on the pages:
PTO-ISA AllGather+GEMM README ("measured performance" tables: fp16 A/B,
fp32 C), Triton-distributed AllGather GEMM tutorial (host test: randn fp16),
catccos AllGatherMatmulDequant design doc (section 8.3 test shapes, int8 A/B,
int32 bias, fp32 per-channel scale) and the Pallas collective matmul page
(normal f16 data, 1024-row shards).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Case", "CASES", "make_f16", "make_bf16", "make_fp8", "make_i8", "make_case",
           "split_rows"]


@dataclass(frozen=True)
class Case:
    """One synthetic workload: gathered shape, shard count and value recipe."""

    case_id: int
    kind: str            # "f16" or "i8"
    n_shards: int
    M: int
    K: int
    N: int
    dist: str = "normal"  # "normal" -> N(0,1), "uniform" -> U[-1,1] (fp16 only)
    chunk_rows: int = 0   # 0 -> automatic choice (64..128 chunks per source)
    link_gbps: float = 0.0  # 0 -> unthrottled producer
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def shard_rows(self) -> int:
        return self.M // self.n_shards

    @property
    def name(self) -> str:
        return (f"{self.kind} {self.n_shards}x{self.shard_rows} rows "
                f"M={self.M} K={self.K} N={self.N}")


# The five workloads: a small one the oracle finishes in a blink, the
# 2-shard 2048x2048x1024 row of the PTO-ISA table, the 4096^3 row with a
# producer paced to one xGMI link, the 8-shard 8192x4096x4096 row (Pallas and
# PTO-ISA 8-card workload) and the first int8 row of the catccos shapes.
CASES: dict[int, Case] = {
    1: Case(1, "f16", 2, 256, 256, 128, "normal", chunk_rows=32,
            note="2 shards of 128 rows, chunk of 32 rows"),
    2: Case(2, "f16", 2, 2048, 2048, 1024, "uniform",
            note="2 shards of 1024 rows, automatic chunk size"),
    3: Case(3, "f16", 4, 4096, 4096, 4096, "normal", link_gbps=153.0,
            note="4 shards, producer paced to 153 GB/s per emulated link"),
    4: Case(4, "f16", 8, 8192, 4096, 4096, "normal",
            note="8 shards of 1024 rows"),
    5: Case(5, "i8", 2, 16384, 27392, 4096,
            note="int8 + bias + per-channel dequant, 2 shards of 8192 rows"),
    # the other two rows of the catccos test-shape table (section 8.3),
    # read like the first: M is the gathered row count, over 2 shards
    6: Case(6, "i8", 2, 131072, 8192, 3072,
            note="int8 + dequant, 2 shards of 65536 rows"),
    7: Case(7, "i8", 2, 64, 16384, 7168,
            note="int8 + dequant, small-M (decode-like), 2 shards of 32 rows"),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def split_rows(A: np.ndarray, n_shards: int) -> list[np.ndarray]:
    """Split a gathered M x K matrix into n_shards contiguous row blocks."""
    M = A.shape[0]
    if M % n_shards:
        raise ValueError("M must be a multiple of n_shards")
    S = M // n_shards
    return [np.ascontiguousarray(A[s * S:(s + 1) * S]) for s in range(n_shards)]


def make_f16(M: int, K: int, N: int, n_shards: int, dist: str = "normal",
             seed_base: int = 0):
    """fp16 shards of A (list of S x K) and B (K x N), both C-contiguous."""
    def draw(seed, shape):
        g = _rng(seed)
        if dist == "normal":
            x = g.standard_normal(shape, dtype=np.float32)
        elif dist == "uniform":
            x = g.uniform(-1.0, 1.0, shape).astype(np.float32)
        else:
            raise ValueError(dist)
        return x.astype(np.float16)

    A = draw(seed_base + 1, (M, K))
    B = draw(seed_base + 2, (K, N))
    return split_rows(A, n_shards), B


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> bfloat16 bit patterns (uint16), round to nearest
    even on the dropped 16 bits; for finite inputs only (how the draws are
    stored, like the fp16 cast above)."""
    bits = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return bits.astype(np.uint16)


def make_bf16(M: int, K: int, N: int, n_shards: int, dist: str = "normal",
              seed_base: int = 0):
    """bfloat16 shards of A and B, as uint16 bit patterns (numpy has no
    bfloat16 type); drawn like make_f16, then rounded to bfloat16."""
    def draw(seed, shape):
        g = _rng(seed)
        if dist == "normal":
            x = g.standard_normal(shape, dtype=np.float32)
        elif dist == "uniform":
            x = g.uniform(-1.0, 1.0, shape).astype(np.float32)
        else:
            raise ValueError(dist)
        return to_bf16_bits(x)

    A = draw(seed_base + 1, (M, K))
    B = draw(seed_base + 2, (K, N))
    return split_rows(A, n_shards), B


def _e4m3_values() -> np.ndarray:
    """Values of the non-negative finite OCP FP8 E4M3 codes 0x00..0x7E, in
    code order (which is also increasing value order)."""
    c = np.arange(0x7F)
    e, f = c >> 3, c & 7
    return np.where(e == 0, f * 2.0 ** -9, (8 + f) * np.exp2(e - 10.0))


def to_fp8e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> OCP FP8 E4M3 bit patterns (uint8), round to nearest
    even; finite inputs of magnitude below 464 only (464 and above would
    round past the largest value, 448)."""
    x = np.asarray(x, np.float32)
    a = np.abs(x.astype(np.float64))
    if not np.all(a < 464.0):
        raise ValueError("value outside the E4M3 range")
    vals = _e4m3_values()
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(a == vals[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def make_fp8(M: int, K: int, N: int, n_shards: int, dist: str = "normal",
             seed_base: int = 0):
    """OCP FP8 E4M3 shards of A and B, as uint8 bit patterns; drawn like
    make_f16, then rounded to E4M3."""
    def draw(seed, shape):
        g = _rng(seed)
        if dist == "normal":
            x = g.standard_normal(shape, dtype=np.float32)
        elif dist == "uniform":
            x = g.uniform(-1.0, 1.0, shape).astype(np.float32)
        else:
            raise ValueError(dist)
        return to_fp8e4m3_bits(x)

    A = draw(seed_base + 1, (M, K))
    B = draw(seed_base + 2, (K, N))
    return split_rows(A, n_shards), B


def make_i8(M: int, K: int, N: int, n_shards: int, seed_base: int = 0):
    """int8 shards, int8 B, int32 bias [N] and fp32 per-channel scale [N]."""
    A = _rng(seed_base + 1).integers(-127, 128, (M, K), dtype=np.int8)
    B = _rng(seed_base + 2).integers(-127, 128, (K, N), dtype=np.int8)
    bias = _rng(seed_base + 3).integers(-1000, 1001, (N,), dtype=np.int32)
    scale = _rng(seed_base + 4).uniform(1e-4, 1e-3, (N,)).astype(np.float32)
    return split_rows(A, n_shards), B, bias, scale


def make_case(case: Case | int):
    """Inputs of one of the seeded workloads, seeded by its id."""
    if isinstance(case, int):
        case = CASES[case]
    base = 1000 * case.case_id
    if case.kind == "f16":
        return make_f16(case.M, case.K, case.N, case.n_shards, case.dist, base)
    return make_i8(case.M, case.K, case.N, case.n_shards, base)
