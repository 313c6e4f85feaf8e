"""Seeded synthetic inputs for the GEMM workloads (shared by tests, bench and smoke).

This module draws random matrices and nothing else: it holds none of the
product's arithmetic, so it can feed both the CPU oracle and the HIP library
the very same bytes.  Every generator returns CPU ``torch`` tensors in the
input dtype; ``bits()`` gives their raw bit patterns as numpy arrays.

Workload families (all row-major, A is [M,K], B is [K,N]) follow the shapes
the pages discuss: square fp16/fp8 products (Insight Edge cuTile blog,
"TileGymで行列積ベンチマーク" tables), decode-time products with a single or
few rows and the few-tiles/huge-K case (Tencent deterministic-inference
article, "Split-K"), and the fused-QKV projection shape N=6144, K=4096
(same article, "チューニングのトレードオフ").

Seeds: ``torch.Generator('cpu')`` seeded with ``1000*family + size_index``;
A is drawn before B.  Smaller-M inputs of one family are row prefixes of the
largest A, so batch-invariance checks compare like with like.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "e4m3": torch.float8_e4m3fn,
    "e5m2": torch.float8_e5m2,
    "f32": torch.float32,
}
_BITS_VIEW = {torch.float16: torch.uint16, torch.bfloat16: torch.uint16,
              torch.float8_e4m3fn: torch.uint8, torch.float8_e5m2: torch.uint8,
              torch.float32: torch.uint32}


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU tensor as a numpy array (no copy if contiguous)."""
    t = t.detach().cpu().contiguous()
    return t.view(_BITS_VIEW[t.dtype]).numpy()


def gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return g


def uniform(shape, dtype, g, lo=-1.0, hi=1.0) -> torch.Tensor:
    """i.i.d. uniform[lo, hi) drawn in fp32, cast to ``dtype`` (round to nearest even)."""
    x = torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo
    return x.to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def normal(shape, dtype, g, std=1.0) -> torch.Tensor:
    """i.i.d. N(0, std^2) drawn in fp32, cast to ``dtype`` (round to nearest even)."""
    x = torch.randn(shape, generator=g, dtype=torch.float32) * std
    return x.to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def integers(shape, dtype, g, lo=-4, hi=4) -> torch.Tensor:
    """i.i.d. uniform integers in [lo, hi] (inclusive), stored exactly in ``dtype``,
    on the generator's device (a CUDA generator draws very large inputs in place)."""
    x = torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32, device=g.device)
    return x.to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def grid(shape, dtype, g, mag=255, exp=-6) -> torch.Tensor:
    """Values n * 2^exp with integer |n| <= mag: full 8-bit significands on one grid."""
    n = torch.randint(-mag, mag + 1, shape, generator=g, dtype=torch.int32)
    x = n.to(torch.float64) * (2.0 ** exp)
    return x.to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def uniform64(shape, g, lo=-1.0, hi=1.0) -> torch.Tensor:
    """i.i.d. uniform[lo, hi) in fp64 (53 random significand bits)."""
    return torch.rand(shape, generator=g, dtype=torch.float64) * (hi - lo) + lo


def wide64(shape, g, spread=20) -> torch.Tensor:
    """fp64 N(0,1) values times 2^e, e uniform integers in [-spread, spread]:
    full significands over a wide exponent range."""
    x = torch.randn(shape, generator=g, dtype=torch.float64)
    e = torch.randint(-spread, spread + 1, shape, generator=g, dtype=torch.int32)
    return torch.ldexp(x, e.to(torch.float64))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str           # input dtype
    out: str             # output dtype
    seed: int
    kind: str            # "int", "uniform", "normal_scaled", "normal"
    api: str             # "run" or "splitk"
    split_k: tuple = (0,)  # 0 = plan default
    m_slices: tuple = ()   # row prefixes used for invariance checks
    gen_rows: int = 0      # A is drawn with this many rows (>= M) and sliced

    def make(self):
        """(A, B) as CPU tensors of the input dtype."""
        g = gen(self.seed)
        rows = max(self.gen_rows, self.M)
        if self.kind == "int":
            A = integers((rows, self.K), self.dtype, g)
            B = integers((self.K, self.N), self.dtype, g)
        elif self.kind == "uniform":
            A = uniform((rows, self.K), self.dtype, g)
            B = uniform((self.K, self.N), self.dtype, g)
        elif self.kind == "normal_scaled":
            s = 1.0 / math.sqrt(self.K)
            A = normal((rows, self.K), self.dtype, g, std=s)
            B = normal((self.K, self.N), self.dtype, g, std=s)
        elif self.kind == "normal":
            A = normal((rows, self.K), self.dtype, g)
            B = normal((self.K, self.N), self.dtype, g)
        else:
            raise ValueError(self.kind)
        return A[: self.M].contiguous(), B

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self) -> int:
        """Bytes of A, B and C that one product must move at least once."""
        isz = DTYPES[self.dtype].itemsize
        osz = DTYPES[self.out].itemsize
        return (self.M * self.K + self.K * self.N) * isz + self.M * self.N * osz


def _registry():
    w = {}
    # Tiny exact product: integers in [-4, 4], fp16 in, fp32 out.
    w["exact256"] = Workload("exact256", 256, 256, 256, "f16", "f32", 1000, "int", "run",
                             split_k=(1, 4), m_slices=(1, 7, 64))
    # Square fp16 products, uniform[-1, 1), fp32 out, no split-K.
    for i, n in enumerate((1024, 4096, 8192)):
        w[f"square_f16_{n}"] = Workload(f"square_f16_{n}", n, n, n, "f16", "f32", 2000 + i,
                                        "uniform", "run")
    # Decode-shaped bf16 products: A drawn once as 128 x K; M uses row prefixes.
    for m in (1, 8, 32, 128):
        w[f"decode_bf16_m{m}"] = Workload(f"decode_bf16_m{m}", m, 4096, 14336, "bf16", "f32",
                                          3000, "normal_scaled", "splitk",
                                          m_slices=(1, 8, 32, 128), gen_rows=128)
    # Few output tiles, huge K: split-K through a workspace.
    w["hugek_f16"] = Workload("hugek_f16", 256, 256, 131072, "f16", "f32", 4000, "uniform",
                              "splitk", split_k=(1, 8, 32, 128))
    # Square fp8 e5m2 products, N(0,1) cast to e5m2 (scale 1.0), bf16 out.
    for i, n in enumerate((4096, 8192, 16384)):
        w[f"square_e5m2_{n}"] = Workload(f"square_e5m2_{n}", n, n, n, "e5m2", "bf16", 5000 + i,
                                         "normal", "run")
    return w


WORKLOADS = _registry()


@dataclasses.dataclass(frozen=True)
class OzakiWorkload:
    """Square fp64 product by the Ozaki scheme (the Insight Edge blog's FP64
    emulation tables run square sizes 1024 .. 16384)."""
    name: str
    n: int
    type2: str
    seed: int

    def make(self):
        """(A, B) fp64 CPU tensors, uniform[-1, 1)."""
        g = gen(self.seed)
        return uniform64((self.n, self.n), g), uniform64((self.n, self.n), g)

    @property
    def flops(self) -> int:
        """fp64 flops of the product it emulates (2 n^3)."""
        return 2 * self.n ** 3


def _ozaki_registry():
    w = {}
    for t, t2 in enumerate(("bf16", "e4m3", "i8")):
        for i, n in enumerate((1024, 4096, 8192, 16384)):
            w[f"ozaki_{t2}_{n}"] = OzakiWorkload(f"ozaki_{t2}_{n}", n, t2, 6000 + 10 * t + i)
    return w


OZAKI_WORKLOADS = _ozaki_registry()
