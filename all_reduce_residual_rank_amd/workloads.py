"""Seeded synthetic inputs for the fused all-reduce + residual + RMSNorm epilogue.

This module only draws random numbers and casts them to the storage type; it
holds none of the epilogue's arithmetic. Both the HIP path's tests and the
CPU oracle take their inputs from here, as raw host tensors (CPU torch).

Recipe (the same for every workload): a CPU ``torch.Generator`` seeded with
``seed`` draws fp32 normals in this order -- rank 0 .. R-1 inputs ``[M][H]``,
then per-(rank, row) scales when the workload has them, then the residual
``[M][H]``, then the weight ``[H]`` -- and each tensor is cast to T with
round-to-nearest-even. The workloads are the row/hidden/rank shapes the
pages measure (tensor-parallel decode and prefill rows at hidden 6144, 7168,
2880 and 512).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
DT_CODE = {"bf16": 0, "fp16": 1, "fp32": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    R: int
    M: int
    H: int
    dtype: str = "bf16"
    eps: float = 1e-6
    gemma: bool = False
    fp8: bool = False
    mirror: bool = True            # write the T output (with FP8: the optional mirror)
    x_sigma: float = 1.0           # inputs ~ N(0, x_sigma) ...
    row_scale: tuple | None = None  # ... times U(lo, hi) per (rank, row) when set
    w_mean: float = 1.0            # weight ~ N(w_mean, w_sigma)
    w_sigma: float = 0.1
    note: str = field(default="", compare=False)

    @property
    def flags(self) -> int:
        return DT_CODE[self.dtype] | (4 if self.gemma else 0) | (8 if self.fp8 else 0)

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def make_inputs(wl: Workload, seed: int = 0, M: int | None = None):
    """Draw the inputs of ``wl`` (optionally with a different row count M).

    Returns (xs, residual, weight): R tensors [M][H], [M][H] and [H] in T, on CPU.
    """
    M = wl.M if M is None else M
    g = torch.Generator().manual_seed(seed)
    T = DTYPES[wl.dtype]
    xs32 = [torch.randn(M, wl.H, generator=g) * wl.x_sigma for _ in range(wl.R)]
    if wl.row_scale is not None:
        lo, hi = wl.row_scale
        s = torch.rand(wl.R, M, 1, generator=g) * (hi - lo) + lo
        xs32 = [x * s[r] for r, x in enumerate(xs32)]
    res32 = torch.randn(M, wl.H, generator=g)
    w32 = torch.randn(wl.H, generator=g) * wl.w_sigma + wl.w_mean
    return [x.to(T) for x in xs32], res32.to(T), w32.to(T)


def exact_integer_inputs(R: int, M: int, H: int, seed: int, dtype: str = "bf16"):
    """Small-integer rank inputs whose sums are exact in every T.

    Rank r holds ((i * (r + 1) + seed * (r + 3)) mod 31) - 15 at flat index i,
    the generator of the tail-specialisation reproducer in ROCm/aiter PR #5807
    ("Standalone microbenchmark reproducer"). Values lie in [-15, 15].
    """
    T = DTYPES[dtype]
    idx = torch.arange(M * H, dtype=torch.int64).reshape(M, H)
    return [(((idx * (r + 1) + seed * (r + 3)) % 31) - 15).to(T) for r in range(R)]


# The five workloads: small decode case, the headline prefill case, FP8 +
# gemma_norm in fp16, a wide-row R=8 case, and a tail/decode sweep.
SMALL = Workload("r4_m16_h6144_bf16", R=4, M=16, H=6144)
HEADLINE = Workload("r4_m1024_h6144_bf16_rowscale", R=4, M=1024, H=6144, row_scale=(0.1, 10.0))
FP8_GEMMA = Workload("r4_m2800_h6144_fp16_gemma_fp8", R=4, M=2800, H=6144, dtype="fp16",
                     gemma=True, fp8=True, mirror=False, x_sigma=2.0, w_mean=0.0, w_sigma=0.1)
WIDE_R8 = Workload("r8_m2048_h7168_bf16", R=8, M=2048, H=7168, eps=1e-5)
TAIL_SHAPES = [(1, 2880), (64, 2880), (121, 2880), (1023, 512), (1024, 512), (1025, 512)]
TAILS = [Workload(f"r4_m{m}_h{h}_bf16", R=4, M=m, H=h) for m, h in TAIL_SHAPES]
TAIL_FP32 = Workload("r4_m1025_h512_fp32", R=4, M=1025, H=512, dtype="fp32")

ALL = [SMALL, HEADLINE, FP8_GEMMA, WIDE_R8, *TAILS, TAIL_FP32]
BY_NAME = {w.name: w for w in ALL}


# ---- the plain rank all-reduce (no norm epilogue) ---------------------------
# Message sizes of the flattened sweep in ROCm/aiter PR #5807 (benchmark case
# sets): representative byte sizes, the 1 MiB tile boundary and its
# neighbours (+-64 B, 63/64/65 packs-of-64 B), the (M, 2880) upstream rows and
# the (1023/1024/1025, 512) regression rows. Sizes that give an element count
# already listed are dropped, as the sweep does.
SUM_BYTES = (8192, 65536, 262144, 524288, 1048576, 4194304, 8388608)
SUM_TILE_OFFSETS = (-64, 0, 64, 63 * 64, 64 * 64, 65 * 64)
SUM_UPSTREAM_M = (120, 121, 127, 157, 160, 161, 256, 512)
SUM_REGRESSION_M = (1023, 1024, 1025)


@dataclass(frozen=True)
class SumCase:
    name: str
    dtype: str
    numel: int

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def nbytes(self) -> int:
        return self.numel * self.esize


def sum_cases(dtype: str) -> list[SumCase]:
    e = 4 if dtype == "fp32" else 2
    cand = [(f"shape_{m}x512", m * 512) for m in SUM_REGRESSION_M]
    cand += [(f"bytes_{n}", n // e) for n in SUM_BYTES]
    cand += [(f"tile_boundary_{o:+d}", (1048576 + o) // e) for o in SUM_TILE_OFFSETS]
    cand += [(f"upstream_{m}x2880", m * 2880) for m in SUM_UPSTREAM_M]
    seen, cases = set(), []
    for name, numel in cand:
        if numel in seen:
            continue
        seen.add(numel)
        cases.append(SumCase(name, dtype, numel))
    return cases


def make_sum_inputs(R: int, numel: int, seed: int, dtype: str = "bf16", sigma: float = 1.0):
    """R rank tensors of numel elements, N(0, sigma) cast to T (RNE)."""
    g = torch.Generator().manual_seed(seed)
    T = DTYPES[dtype]
    return [(torch.randn(numel, generator=g) * sigma).to(T) for _ in range(R)]


# The sum-only benchmark message: the rank inputs of the prefill rows
# (R=4, 1024 x 6144 bf16, 12 MiB per rank).
SUM_HEADLINE = SumCase("sum_r4_n6291456_bf16", "bf16", 1024 * 6144)
