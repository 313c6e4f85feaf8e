"""Shared helpers for the GPU tests: run the library, fetch bits, check bounds.

The error bound for fp32 output is the one the deterministic-GEMM target
fixes: |C - C_ref| <= K * 2^-24 * (|A||B|)_ij, with C_ref the exact (fp64)
product.  For bf16 output it adds the final rounding to bf16 (unit roundoff
2^-8): K u (|A||B|)(1 + 2^-8) + 2^-8 |C_ref|; fp16 output likewise with
2^-11 plus half the smallest fp16 subnormal (2^-25).  A bias adds one fp32
rounding of the sum: the accumulated bound times (1 + 2^-24) plus
2^-24 |C_ref|, with |A||B| + |bias| in place of |A||B|.

fp8 inputs can need one more term, from how the gfx950 fp8 matrix instruction
(16x16x128) sums the products of one K step (measured, and pinned by
tests/test_gpu_fp8_step.py): the products of each aligned group of 8
consecutive K positions are added in a window that ends 13 binades below the
largest product of that group, and what falls below it is truncated toward
zero.  Other groups, and the fp32 accumulator, are not in that window.  So
each group can lose at most sum_k min(|a_k b_k|, 2^(E-13)), E the binade of
its largest product; ``fp8_step_window`` computes that sum per element.
``fp8_check_bound`` adds it only for K below FP8_PLAIN_BOUND_MIN_K: longer
fp8 sums are held to the plain bound.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import invariant_matmul_amd as imm
import oracle
import workloads as wl

U32 = 2.0 ** -24
U_BF16 = 2.0 ** -8
U_F16 = 2.0 ** -11


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def out_torch_dtype(code: int):
    return {imm.DTYPE["f32"]: torch.float32, imm.DTYPE["bf16"]: torch.bfloat16,
            imm.DTYPE["f16"]: torch.float16}[code]


def run(plan, A, B, split: bool, stream=None):
    """Run the plan on device tensors A, B; returns the device output."""
    info = plan.info
    C = torch.empty((info["M"], info["N"]), dtype=out_torch_dtype(info["out_dtype"]),
                    device=A.device)
    if split:
        ws = torch.empty(max(1, imm.gemm_workspace_size(plan) // 4), dtype=torch.float32,
                         device=A.device)
        imm.gemm_splitk_run(plan, A, B, C, ws, stream)
    else:
        imm.gemm_run(plan, A, B, C, stream)
    return C


def bits_of(C: torch.Tensor) -> np.ndarray:
    """Raw output bits on the host (uint32 for fp32, uint16 for bf16)."""
    torch.cuda.synchronize()
    return wl.bits(C.cpu())


def values_of(C: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return C.cpu().to(torch.float64).numpy()


def expected_bits(C64: np.ndarray, out: str) -> np.ndarray:
    return oracle.round_rne(out, C64)


def bound(K: int, C64: np.ndarray, Cabs: np.ndarray, out: str, bias: bool = False) -> np.ndarray:
    b = K * U32 * Cabs
    if bias:
        b = b * (1.0 + U32) + U32 * np.abs(C64)
    if out == "bf16":
        b = b * (1.0 + U_BF16) + U_BF16 * np.abs(C64)
    elif out == "f16":
        b = b * (1.0 + U_F16) + U_F16 * np.abs(C64) + 2.0 ** -25
    return b


FP8 = ("e4m3", "e5m2")
FP8_GROUP = 8        # K positions added in one window by the fp8 matrix step
FP8_WINDOW = 13      # binades kept below the largest product of a group


def fp8_step_window(A_vals: np.ndarray, B_vals: np.ndarray, ii=None, jj=None,
                    scale: float = 1.0, chunk: int = 256) -> np.ndarray:
    """Per element, the most the fp8 step window can drop: for every group of
    8 K positions (aligned from the start of K; slices start at multiples of
    128, so the groups are the same with or without a split),
    sum_k min(|p_k|, 2^(E-13)) with p_k = a_ik b_kj and
    2^E <= max_k |p_k| < 2^(E+1); times |scale|.  With ii, jj given, only
    those elements (flat arrays); else all of M x N."""
    A = np.abs(np.asarray(A_vals, dtype=np.float64))
    B = np.abs(np.asarray(B_vals, dtype=np.float64))
    K = A.shape[1]
    pad = (-K) % FP8_GROUP
    if pad:
        A = np.pad(A, ((0, 0), (0, pad)))
        B = np.pad(B, ((0, pad), (0, 0)))
    if ii is None:
        ii, jj = np.meshgrid(np.arange(A.shape[0]), np.arange(B.shape[1]), indexing="ij")
        shape = ii.shape
        ii, jj = ii.ravel(), jj.ravel()
    else:
        ii, jj = np.asarray(ii), np.asarray(jj)
        shape = ii.shape
    out = np.empty(ii.size, dtype=np.float64)
    Bt = B.T
    for s in range(0, ii.size, chunk):
        P = A[ii[s:s + chunk]] * Bt[jj[s:s + chunk]]          # n x K products
        P = P.reshape(P.shape[0], -1, FP8_GROUP)             # n x groups x 8
        mx = P.max(axis=2, keepdims=True)
        with np.errstate(divide="ignore"):
            lsb = np.where(mx > 0, 2.0 ** (np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - FP8_WINDOW), 0.0)
        out[s:s + chunk] = np.minimum(P, lsb).sum(axis=(1, 2))
    return abs(scale) * out.reshape(shape)


def check_bound(C: np.ndarray, C64: np.ndarray, Cabs: np.ndarray, K: int, out: str,
                bias: bool = False, window=None) -> float:
    """Assert every element is within the bound (plus ``window``, the fp8 step
    allowance, when given); returns max |err| / bound."""
    err = np.abs(C - C64)
    b = bound(K, C64, Cabs, out, bias)
    if window is not None:
        w = np.asarray(window, dtype=np.float64)
        if out == "bf16":
            w = w * (1.0 + U_BF16)
        elif out == "f16":
            w = w * (1.0 + U_F16)
        b = b + w
    bad = err > b
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{int(bad.sum())} elements outside the bound; first {idx.tolist()}: "
            f"got {C[bad][:5]}, want {C64[bad][:5]}, bound {b[bad][:5]}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(b > 0, err / b, 0.0)
    return float(r.max()) if r.size else 0.0


# fp8 products are checked against the plain bound from this K on; below it
# the step window is added to the bound (the departure from the fp32-accumulation
# bound that the fp8 matrix step causes on short sums).  Measured on random
# N(0, 1) e4m3 / e5m2 inputs (3 x 256 x 256 outputs per K, fp32 out): the
# plain bound fails at K <= 128 (up to 99 times the bound at K = 16), holds at
# K = 256 with a worst ratio of 0.58 - 0.76, at K = 512 with 0.15 - 0.18 and
# at K >= 4096 with at most 0.007.
FP8_PLAIN_BOUND_MIN_K = 512


def fp8_check_bound(C, C64, Cabs, K, out, dt, a_bits=None, b_bits=None, ii=None, jj=None,
                    bias=False) -> float:
    """check_bound for any input dtype.  16-bit inputs, and fp8 inputs with
    K >= FP8_PLAIN_BOUND_MIN_K, get the plain bound; fp8 inputs with a shorter
    K get the plain bound plus the step window of their own products (A and B
    bit patterns, and the element positions ii, jj when C holds a sample)."""
    if dt not in FP8 or K >= FP8_PLAIN_BOUND_MIN_K:
        return check_bound(C, C64, Cabs, K, out, bias=bias)
    win = fp8_step_window(oracle.decode(dt, a_bits), oracle.decode(dt, b_bits), ii, jj)
    return check_bound(C, C64, Cabs, K, out, bias=bias, window=win)


NARROW_TILES = ("32x64", "64x64", "32x32")   # DMA tiles of 64 and 32 columns: fp16 / bf16 inputs only


def tiles_for(dt: str, tiles):
    """The tiles of `tiles` that take input dtype dt (the narrow tiles take
    16-bit inputs only)."""
    return [t for t in tiles if dt in ("f16", "bf16") or t not in NARROW_TILES]


def dtype_name(code: int) -> str:
    return {v: k for k, v in imm.DTYPE.items()}[code]
