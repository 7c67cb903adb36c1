"""fp64 CPU oracle for the few-row quantized GEMV  y[M,N] = x[M,K] * dequant(W[N,K])^T.

TEST INFRASTRUCTURE ONLY.  This module is the parity reference for the HIP
path.  Only the test suite, the package smoke check and the benchmark's CPU
baseline leg may import it; the product path never does.  It shares no code
with the HIP path (no kernels, headers, helpers or tables) and imports nothing
from the product package.

What it computes is the plain definition of the operation, written out:

* Affine group quantization (MLX quantized_matmul small-M verify kernels,
  Facts: "group-size mechanism" -- 4 B of fp16 scale+bias per group; the
  affine mode listed with qmv_wide): each weight is w[n,k] = s[n,g]*q[n,k] +
  b[n,g] with g = k // group_size, one fp16 scale and one fp16 bias per output
  row n and group g.  Read plainly as scale times code plus bias, not
  scale*(q - zero).
* Weights stored [out, in] and the product taken as x @ W^T (same page, Facts:
  the (M,5120)@(17408,5120)^T microbench).
* Codes packed little-endian along K: 4-bit codes two per byte, low nibble
  first; 2-bit codes four per byte, lowest crumb first (the 2-bit order is not
  stated on the pages; this is the reading that matches the 4-bit convention);
  8-bit codes one per byte (the int8 affine mode of qmv_wide, MLX page,
  Facts: the int8 M=8 speedup; the code is the unsigned byte).
* Every weight group is used once for all M rows (metal : few-row MMA mat-mul
  and batched copies for speculative decoding, Overview: each weight is
  dequantized once for all rows).  That is an evaluation-order property of the
  fast path; the value it reaches is exactly this dequantize-then-matmul.

Precision: fp16 -> fp64 and bf16 -> fp64 are exact.  s*q is exact (11-bit
significand times a 4-bit integer).  Adding b is exact whenever s*q and b lie
within ~38 binades of each other, which holds for every workload here (s and
|b| are within a factor of ~100); each product x*w is then exact too (8-bit
times <= ~45-bit significands; 8-bit codes give an 19-bit s*q, still exact).  So in practice only the K-term summation
rounds, at K * 2^-53 relative at worst -- twelve orders of magnitude below the
1e-3 tolerance.

The fused residual sum ("metal : few-row MMA mat-mul and batched copies for
speculative decoding", Overview: a fusion table entry where MUL_MAT + ADD
writes the residual sum from the MMA store) is the same product plus an fp32
residual tensor of the output's shape [M, N]: y[m,n] = (x W^T)[m,n] + r[m,n],
computed here in fp64 (fp32 -> fp64 is exact).  The residual is read as
having the output's layout, since the ADD consumes the mat-mul's result
element by element.

Parity of y is pinned by closed forms, invariants and exact rational brute
force (the pages print no worked y values); see tests/test_oracle.py.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "fp16_bits_to_f64",
    "bf16_bits_to_f64",
    "unpack_codes",
    "dequantize",
    "qgemv_reference",
    "residual_f64",
    "qgemv_add_reference",
    "abs_product_sum",
    "tolerance",
    "check_close",
    "FP_FORMATS",
    "e2m1_to_f64",
    "e4m3_to_f64",
    "e8m0_to_f64",
    "fp_elements",
    "fp_dequantize",
    "qgemv_fp_reference",
    "fp_abs_product_sum",
    "qgemv_gather_reference",
    "gather_abs_product_sum",
]


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (the top half of a binary32) -> float64 (exact)."""
    u32 = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def unpack_codes(codes: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Packed codes [N, K*bits/8] uint8 -> integer codes q [N, K] uint8.

    For column k: byte = codes[n, (k*bits) // 8], shift = (k*bits) % 8,
    q = (byte >> shift) & (2**bits - 1).
    """
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    codes = np.asarray(codes, dtype=np.uint8)
    N = codes.shape[0]
    if codes.shape[1] * 8 != K * bits:
        raise ValueError("codes row length does not match K*bits/8")
    k = np.arange(K)
    byte_idx = (k * bits) // 8
    shift = ((k * bits) % 8).astype(np.uint8)
    mask = np.uint8((1 << bits) - 1)
    q = (codes[:, byte_idx] >> shift[None, :]) & mask
    assert q.shape == (N, K)
    return q.astype(np.uint8)


def dequantize(q: np.ndarray, scales: np.ndarray, biases: np.ndarray, group_size: int) -> np.ndarray:
    """w[n,k] = s[n, k//gs] * q[n,k] + b[n, k//gs] in fp64.  scales/biases are fp16 bits."""
    q = np.asarray(q)
    N, K = q.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    s = fp16_bits_to_f64(scales)
    b = fp16_bits_to_f64(biases)
    if s.shape != (N, K // group_size) or b.shape != s.shape:
        raise ValueError("scales/biases must be [N, K/group_size]")
    g = np.arange(K) // group_size
    return s[:, g] * q.astype(np.float64) + b[:, g]


def _row_chunks(N: int, K: int, rows: Optional[Sequence[int]], budget_elems: int = 1 << 23):
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    step = max(1, budget_elems // max(K, 1))
    for i in range(0, len(idx), step):
        yield i, idx[i:i + step]


def qgemv_reference(codes, scales, biases, x_bits, M: int, N: int, K: int, bits: int,
                    group_size: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """y_ref[m, j] = sum_k x[m,k] * w[n_j, k] in fp64, n_j = rows[j] (default: all N).

    x_bits: bf16 bit patterns [>=M, K]; the first M rows are used.
    Dequantization is done in row chunks to bound memory (fp64 W of a
    17408x5120 matrix would be 713 MB); chunking over output rows does not
    reorder any sum.
    """
    x = bf16_bits_to_f64(np.asarray(x_bits)[:M])
    if x.shape != (M, K):
        raise ValueError("x must have at least M rows of length K")
    n_out = N if rows is None else len(rows)
    y = np.empty((M, n_out), dtype=np.float64)
    for start, idx in _row_chunks(N, K, rows):
        q = unpack_codes(codes[idx], K, bits)
        w = dequantize(q, scales[idx], biases[idx], group_size)
        y[:, start:start + len(idx)] = x @ w.T
    return y


def residual_f64(residual, M: int, N: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp32 residual [>=M, N] -> float64 [M, len(rows)] (exact), columns `rows` (default all N)."""
    r = np.asarray(residual, dtype=np.float32)
    if r.ndim != 2 or r.shape[0] < M or r.shape[1] != N:
        raise ValueError("residual must be [>=M, N] float32")
    r = r[:M].astype(np.float64)
    return r if rows is None else r[:, np.asarray(rows, dtype=np.int64)]


def qgemv_add_reference(codes, scales, biases, x_bits, residual, M: int, N: int, K: int, bits: int,
                        group_size: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Fused residual sum in fp64: y_ref[m, j] = sum_k x[m,k] w[n_j,k] + r[m, n_j].

    residual: float32 [>=M, N], the output's layout; the first M rows are used.
    """
    prod = qgemv_reference(codes, scales, biases, x_bits, M, N, K, bits, group_size, rows=rows)
    return prod + residual_f64(residual, M, N, rows)


def abs_product_sum(codes, scales, biases, x_bits, M: int, N: int, K: int, bits: int,
                    group_size: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """sum_k |x[m,k] * w[n,k]| in fp64 (the scale of the tolerance)."""
    x = np.abs(bf16_bits_to_f64(np.asarray(x_bits)[:M]))
    n_out = N if rows is None else len(rows)
    out = np.empty((M, n_out), dtype=np.float64)
    for start, idx in _row_chunks(N, K, rows):
        q = unpack_codes(codes[idx], K, bits)
        w = np.abs(dequantize(q, scales[idx], biases[idx], group_size))
        out[:, start:start + len(idx)] = x @ w.T
    return out


# Relative size of the rounding that adding the residual in fp32 may add: the
# sum is rounded once or twice (half an fp32 ulp, 2^-24 relative, each time)
# and its magnitude is at most |r| + sum_k |x_k w_k|.
ADD_ROUNDING = 2.0 ** -23


def tolerance(abs_sum: np.ndarray, rel: float = 1e-3, abs_floor: float = 1e-6,
              residual_abs: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-element bound |y - y_ref| <= rel * sum_k |x_k w_k| + abs_floor, plus,
    for the fused residual sum, 2^-23 * (|r| + sum_k |x_k w_k|)."""
    a = np.asarray(abs_sum, dtype=np.float64)
    tol = rel * a + abs_floor
    if residual_abs is not None:
        tol = tol + ADD_ROUNDING * (np.abs(np.asarray(residual_abs, dtype=np.float64)) + a)
    return tol


def check_close(y_test, y_ref, abs_sum, rel: float = 1e-3, abs_floor: float = 1e-6,
                residual_abs: Optional[np.ndarray] = None):
    """Return (ok, worst_ratio, index).  worst_ratio = max |dy| / tol (<= 1 passes).
    NaN/Inf in y_test fail.  residual_abs: |r| for the fused residual sum."""
    y_test = np.asarray(y_test, dtype=np.float64)
    if not np.all(np.isfinite(y_test)):
        bad = np.argwhere(~np.isfinite(y_test))[0]
        return False, float("inf"), tuple(int(i) for i in bad)
    tol = tolerance(abs_sum, rel, abs_floor, residual_abs)
    ratio = np.abs(y_test - y_ref) / tol
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    worst = float(ratio[idx])
    return worst <= 1.0, worst, tuple(int(i) for i in idx)


# ---------------------------------------------------------------- FP block formats
#
# The block-scaled floating-point modes of qmv_wide (MLX page, Facts: qmv_wide
# covers affine, nvfp4, mxfp4 and mxfp8; their M=8 speedups on the Gemma-4-12B
# gate/up shape).  The pages name the modes but not their encodings; these
# decoders follow the public OCP Microscaling Formats (MX) v1.0 specification
# (element types FP4 E2M1 and FP8 E4M3, shared scale E8M0, block of 32) and,
# for nvfp4, the same E2M1 elements with an FP8 E4M3 scale per block of 16.
# Each weight is w[n,k] = scale[n, k // block] * element[n,k]; there is no
# bias.  Elements are packed along K like the affine codes: two FP4 elements
# per byte, low nibble first; one FP8 element per byte.

FP_FORMATS = {
    # name: (element bits, block size, scale type)
    "mxfp4": (4, 32, "e8m0"),
    "nvfp4": (4, 16, "e4m3"),
    "mxfp8": (8, 32, "e8m0"),
}


def e2m1_to_f64(nibbles: np.ndarray) -> np.ndarray:
    """FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
    Exponent 0 is subnormal (0 or 0.5); no infinities or NaNs."""
    v = np.asarray(nibbles, dtype=np.int64) & 0xF
    sign = np.where(v & 0x8, -1.0, 1.0)
    e = (v >> 1) & 0x3
    m = v & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def e4m3_to_f64(bytes_: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (OCP): sign bit 7, exponent bits 6..3 (bias 7), mantissa bits
    2..0.  Exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no
    infinities (max 448)."""
    v = np.asarray(bytes_, dtype=np.int64) & 0xFF
    sign = np.where(v & 0x80, -1.0, 1.0)
    e = (v >> 3) & 0xF
    m = v & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e8m0_to_f64(bytes_: np.ndarray) -> np.ndarray:
    """E8M0 shared scale: 2^(e - 127); e = 255 is NaN."""
    e = np.asarray(bytes_, dtype=np.int64) & 0xFF
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def fp_elements(codes: np.ndarray, K: int, fmt: str) -> np.ndarray:
    """Packed elements [N, K*bits/8] -> element values [N, K] in fp64 (exact)."""
    bits, _, _ = FP_FORMATS[fmt]
    q = unpack_codes(codes, K, bits)  # the raw 4- or 8-bit fields, same packing as affine codes
    return e2m1_to_f64(q) if bits == 4 else e4m3_to_f64(q)


def fp_scales(scales: np.ndarray, fmt: str) -> np.ndarray:
    _, _, stype = FP_FORMATS[fmt]
    return e8m0_to_f64(scales) if stype == "e8m0" else e4m3_to_f64(scales)


def fp_dequantize(codes: np.ndarray, scales: np.ndarray, K: int, fmt: str) -> np.ndarray:
    """w[n,k] = scale[n, k // block] * element[n,k] in fp64 (exact: the product
    of a <= 4-bit and a power-of-two or 4-bit significand)."""
    _, block, _ = FP_FORMATS[fmt]
    el = fp_elements(codes, K, fmt)
    s = fp_scales(scales, fmt)
    if s.shape != (el.shape[0], K // block):
        raise ValueError("scales must be [N, K/block]")
    return s[:, np.arange(K) // block] * el


def qgemv_fp_reference(codes, scales, x_bits, M: int, N: int, K: int, fmt: str,
                       rows: Optional[Sequence[int]] = None, residual=None) -> np.ndarray:
    """y_ref[m, j] = sum_k x[m,k] * w[n_j, k] (+ residual[m, n_j]) in fp64."""
    x = bf16_bits_to_f64(np.asarray(x_bits)[:M])
    if x.shape != (M, K):
        raise ValueError("x must have at least M rows of length K")
    n_out = N if rows is None else len(rows)
    y = np.empty((M, n_out), dtype=np.float64)
    for start, idx in _row_chunks(N, K, rows):
        w = fp_dequantize(codes[idx], scales[idx], K, fmt)
        y[:, start:start + len(idx)] = x @ w.T
    if residual is not None:
        y += residual_f64(residual, M, N, rows)
    return y


def fp_abs_product_sum(codes, scales, x_bits, M: int, N: int, K: int, fmt: str,
                       rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """sum_k |x[m,k] * w[n,k]| in fp64 (the scale of the tolerance)."""
    x = np.abs(bf16_bits_to_f64(np.asarray(x_bits)[:M]))
    n_out = N if rows is None else len(rows)
    out = np.empty((M, n_out), dtype=np.float64)
    for start, idx in _row_chunks(N, K, rows):
        out[:, start:start + len(idx)] = x @ np.abs(fp_dequantize(codes[idx], scales[idx], K, fmt)).T
    return out


# ---------------------------------------------------------------- gathered (MoE) verify
#
# The MoE form of the verify product (MLX page, Facts: dense and MoE
# gather_qmm verify; the expert-union cost per verify row is named as
# unstudied).  Read plainly, as a gathered product over (activation row,
# expert) pairs: pair p takes activation row x_idx[p] and expert e_idx[p] and
# yields y[p] = x[x_idx[p]] . dequant(W[e_idx[p]])^T, with the experts'
# weights stored as E affine-quantized matrices of the same shape.  A fast
# path reads every expert in the union of e_idx once for all the pairs that
# use it; the value it reaches is this per-pair product.

def qgemv_gather_reference(codes, scales, biases, x_bits, x_idx, e_idx, N: int, K: int,
                           bits: int, group_size: int,
                           rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """y[p, j] = sum_k x[x_idx[p], k] * w_{e_idx[p]}[n_j, k] in fp64.

    codes [E, N, K*bits/8]; scales, biases [E, N, K/gs] fp16 bits; x_bits
    [X, K] bf16 bits; x_idx, e_idx [P] integers.  Experts are dequantized once
    each (pairs grouped by expert only to avoid recomputing w; the sums are per
    pair)."""
    x_idx = np.asarray(x_idx, dtype=np.int64)
    e_idx = np.asarray(e_idx, dtype=np.int64)
    P = len(e_idx)
    n_out = N if rows is None else len(rows)
    y = np.empty((P, n_out), dtype=np.float64)
    x_bits = np.asarray(x_bits)
    for e in np.unique(e_idx):
        sel = np.nonzero(e_idx == e)[0]
        y[sel] = qgemv_reference(codes[e], scales[e], biases[e], x_bits[x_idx[sel]], len(sel), N, K,
                                 bits, group_size, rows=rows)
    return y


def gather_abs_product_sum(codes, scales, biases, x_bits, x_idx, e_idx, N: int, K: int, bits: int,
                           group_size: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """sum_k |x[x_idx[p], k] * w_{e_idx[p]}[n, k]| per pair (the tolerance scale)."""
    x_idx = np.asarray(x_idx, dtype=np.int64)
    e_idx = np.asarray(e_idx, dtype=np.int64)
    x_bits = np.asarray(x_bits)
    n_out = N if rows is None else len(rows)
    out = np.empty((len(e_idx), n_out), dtype=np.float64)
    for e in np.unique(e_idx):
        sel = np.nonzero(e_idx == e)[0]
        out[sel] = abs_product_sum(codes[e], scales[e], biases[e], x_bits[x_idx[sel]], len(sel), N, K,
                                   bits, group_size, rows=rows)
    return out
