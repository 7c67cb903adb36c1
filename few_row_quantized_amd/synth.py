"""Seeded synthetic inputs for the few-row quantized GEMV.

This module only draws random inputs in the storage formats the kernels and
the oracle consume; it contains none of the product's arithmetic (no unpack,
no dequantization, no dot products).  Both the HIP path's tests/bench and the
CPU oracle's tests take their inputs from here.

Workloads follow the matrix shapes the pages measure on (MLX quantized_matmul
small-M verify kernels, Facts: the (M,5120)@(17408,5120)^T microbench and the
4096x4096 / 4096x12288 residual shapes) with the value distributions of the
affine group format (w = scale*q + bias, one fp16 scale and one fp16 bias per
output row and group of `group_size` along K):

* 4-bit: q ~ U{0..15}, two codes per byte, low nibble first.
  scale ~ U[0.001, 0.01] rounded to fp16; bias = fp16(-8*scale + N(0, 1e-3)).
* 2-bit: q ~ U{0..3}, four codes per byte, least-significant crumb first.
  scale ~ U[0.005, 0.03]; bias = fp16(-1.5*scale + N(0, 1e-3)).
* 8-bit: q ~ U{0..255}, one code per byte.  scale ~ U[1e-4, 1e-3];
  bias = fp16(-128*scale + N(0, 1e-3)): the zero point in the middle of the
  code range as for the other widths, and weights of about the 4-bit range.
* x ~ N(0, 1) rounded to bf16 (round to nearest even); the decoder-layer sweep
  scales round(1% of K) channels by 20 (in fp32, before rounding) as outliers.

Because the codes are i.i.d. uniform, the packed bytes are i.i.d. uniform over
0..255 for both widths, so codes are drawn directly as bytes.

Draw order per problem: codes, scales, bias noise, x, outlier channels.  The
second parameter of N(0, 1e-3) is read as a standard deviation.

Block-scaled FP formats (mxfp4, nvfp4, mxfp8) draw element codes and scale
bytes directly in their storage encodings (see _draw_fp), then x.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    """One projection: y[M,N] = x[M,K] * dequant(W[N,K])^T."""

    name: str
    K: int
    N: int
    bits: int
    group_size: int
    m_values: Tuple[int, ...]
    seed: int
    outliers: bool = False
    # Problems that share `share_key` share codes and x (only scales and
    # biases are redrawn), as in the group-size sweep.
    share_key: Optional[str] = None
    # Block-scaled floating-point format ("mxfp4", "nvfp4", "mxfp8"); None for
    # the affine codes.  For these, `bits` is the element width, `group_size`
    # the scale block, `scales` holds one scale byte per block and `biases` is
    # empty.
    fmt: Optional[str] = None


def _layer(name: str, K: int, N: int, idx: int) -> Shape:
    return Shape(f"layer27b_{name}", K, N, 4, 128, tuple(range(1, 17)),
                 seed=40000 + 100 * idx, outliers=True)


# Element width and scale block of the FP block formats.
FP_BITS = {"mxfp4": 4, "nvfp4": 4, "mxfp8": 8}
FP_BLOCK = {"mxfp4": 32, "nvfp4": 16, "mxfp8": 32}

# Workloads.  Names say what they are; seeds are fixed per workload.
WORKLOADS: Dict[str, Shape] = {s.name: s for s in [
    Shape("tiny_k256_n512_4b_g64", 256, 512, 4, 64, (1, 2, 3, 4), seed=0),
    Shape("square_k4096_n4096_4b_g64", 4096, 4096, 4, 64, (1, 2, 3, 4, 5, 8), seed=10000),
    Shape("ffnup_k4096_n12288_4b_g32", 4096, 12288, 4, 32, (4, 8), seed=20000, share_key="ffnup"),
    Shape("ffnup_k4096_n12288_4b_g64", 4096, 12288, 4, 64, (4, 8), seed=20001, share_key="ffnup"),
    Shape("ffnup_k4096_n12288_4b_g128", 4096, 12288, 4, 128, (4, 8), seed=20002, share_key="ffnup"),
    Shape("lowram27b_gateup_k5120_n17408_2b_g64", 5120, 17408, 2, 64, tuple(range(2, 13)), seed=30000),
    Shape("lowram27b_down_k17408_n5120_2b_g64", 17408, 5120, 2, 64, tuple(range(2, 13)), seed=30100),
    _layer("q", 5120, 6144, 0),
    _layer("k", 5120, 1024, 1),
    _layer("v", 5120, 1024, 2),
    _layer("o", 6144, 5120, 3),
    _layer("gate", 5120, 17408, 4),
    _layer("up", 5120, 17408, 5),
    _layer("down", 17408, 5120, 6),
    # 8-bit affine gs64 (MLX page, Facts: int8 qmv_wide on Gemma-4-12B gate/up
    # 15360x3840; the (M,5120)@(17408,5120)^T microbench also run at 8 bits)
    Shape("square_k4096_n4096_8b_g64", 4096, 4096, 8, 64, (1, 2, 3, 4, 5, 8), seed=50000),
    Shape("gemma12b_gateup_k3840_n15360_8b_g64", 3840, 15360, 8, 64, (1, 2, 4, 8), seed=50100),
    Shape("mlxbench_k5120_n17408_8b_g64", 5120, 17408, 8, 64, tuple(range(1, 17)), seed=50200),
    # block-scaled FP modes of qmv_wide (MLX page, Facts: nvfp4, mxfp4 and
    # mxfp8 speedups on the Gemma-4-12B gate/up shape 15360x3840)
    *[Shape(f"{pre}_{fmt}", K, N, FP_BITS[fmt], FP_BLOCK[fmt], ms, seed=seed + off, fmt=fmt)
      for off, fmt in enumerate(("mxfp4", "nvfp4", "mxfp8"))
      for pre, K, N, ms, seed in (("square_k4096_n4096", 4096, 4096, (1, 2, 3, 4, 5, 8), 60000),
                                  ("gemma12b_gateup_k3840_n15360", 3840, 15360, (1, 2, 4, 8), 60100))],
]}

LAYER27B = [f"layer27b_{p}" for p in ("q", "k", "v", "o", "gate", "up", "down")]


@dataclasses.dataclass
class Problem:
    """Inputs in device storage formats (all numpy, C-contiguous).

    codes  uint8  [N, K*bits/8]
    scales uint16 [N, K/group_size]   (fp16 bit patterns)
    biases uint16 [N, K/group_size]   (fp16 bit patterns)
    x      uint16 [Mmax, K]           (bf16 bit patterns)
    """

    shape: Shape
    codes: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    x: np.ndarray
    outlier_channels: Optional[np.ndarray]
    seed: int

    @property
    def K(self) -> int:
        return self.shape.K

    @property
    def N(self) -> int:
        return self.shape.N

    @property
    def bits(self) -> int:
        return self.shape.bits

    @property
    def group_size(self) -> int:
        return self.shape.group_size

    def x_rows(self, M: int) -> np.ndarray:
        return np.ascontiguousarray(self.x[:M])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite; NaN handling is not needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f64_to_fp16_bits(a: np.ndarray) -> np.ndarray:
    """Round to IEEE half precision (numpy's conversion, nearest-even); uint16 bits."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def _draw_meta(rng: np.random.Generator, N: int, G: int, bits: int):
    if bits == 4:
        lo, hi, zero_point = 0.001, 0.01, 8.0
    elif bits == 2:
        lo, hi, zero_point = 0.005, 0.03, 1.5
    elif bits == 8:
        lo, hi, zero_point = 1e-4, 1e-3, 128.0
    else:
        raise ValueError(f"unsupported bits {bits}")
    s16 = rng.uniform(lo, hi, size=(N, G)).astype(np.float16)
    noise = rng.normal(0.0, 1e-3, size=(N, G))
    b16 = (-zero_point * s16.astype(np.float64) + noise).astype(np.float16)
    return s16.view(np.uint16).copy(), b16.view(np.uint16).copy()


def _draw_codes(rng: np.random.Generator, N: int, K: int, bits: int) -> np.ndarray:
    return rng.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)


def _draw_x(rng: np.random.Generator, M: int, K: int, outliers: bool):
    x32 = rng.standard_normal(size=(M, K)).astype(np.float32)
    chans = None
    if outliers:
        n_out = int(round(0.01 * K))
        chans = np.sort(rng.choice(K, size=n_out, replace=False))
        x32[:, chans] *= np.float32(20.0)
    return f32_to_bf16_bits(x32), chans


def _draw_fp(rng: np.random.Generator, N: int, K: int, fmt: str):
    """Elements and scale bytes of a block-scaled FP format.

    FP4 elements: uniform nibbles (every E2M1 value, both zeros).  FP8
    elements: uniform over the 254 finite E4M3 bytes.  E8M0 scales: exponent
    uniform in 116..121 (mxfp4, 2^-11..2^-6) or 110..115 (mxfp8, 2^-17..2^-12),
    so weights span about the 4-bit affine range.  nvfp4 E4M3 scales: exponent
    field 1..3, mantissa uniform (2^-6 .. 1.875*2^-4), positive."""
    bits, block = FP_BITS[fmt], FP_BLOCK[fmt]
    G = K // block
    if bits == 4:
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    else:
        v = rng.integers(0, 254, size=(N, K)).astype(np.int64)
        v = v + (v >= 0x7F)  # skip 0x7F (NaN); 0xFF is never reached
        codes = v.astype(np.uint8)
    if fmt == "nvfp4":
        e = rng.integers(1, 4, size=(N, G))
        m = rng.integers(0, 8, size=(N, G))
        scales = ((e << 3) | m).astype(np.uint8)
    else:
        lo = 116 if fmt == "mxfp4" else 110
        scales = rng.integers(lo, lo + 6, size=(N, G)).astype(np.uint8)
    return codes, scales


def make_problem(shape: Shape, m_max: Optional[int] = None, seed: Optional[int] = None) -> Problem:
    """Draw one problem.  x has m_max rows (default: the workload's largest M);
    an M-row call uses the first M rows.  FP formats: codes, scale bytes, x
    (draw order), biases empty."""
    m_max = m_max or max(shape.m_values)
    base_seed = shape.seed if seed is None else seed
    if shape.fmt is not None:
        rng = np.random.default_rng(base_seed)
        codes, scales = _draw_fp(rng, shape.N, shape.K, shape.fmt)
        x, chans = _draw_x(rng, m_max, shape.K, shape.outliers)
        return Problem(shape, codes, scales, np.zeros((shape.N, 0), np.uint16), x, chans, base_seed)
    if shape.share_key is not None and seed is None:
        # Shared codes and x across the group-size sweep; scales/biases per gs.
        shared_seed = min(s.seed for s in WORKLOADS.values() if s.share_key == shape.share_key)
        rng_shared = np.random.default_rng(shared_seed)
        codes = _draw_codes(rng_shared, shape.N, shape.K, shape.bits)
        rng_meta = np.random.default_rng(base_seed)
        scales, biases = _draw_meta(rng_meta, shape.N, shape.K // shape.group_size, shape.bits)
        x, chans = _draw_x(rng_shared, m_max, shape.K, shape.outliers)
    else:
        rng = np.random.default_rng(base_seed)
        codes = _draw_codes(rng, shape.N, shape.K, shape.bits)
        scales, biases = _draw_meta(rng, shape.N, shape.K // shape.group_size, shape.bits)
        x, chans = _draw_x(rng, m_max, shape.K, shape.outliers)
    return Problem(shape, codes, scales, biases, x, chans, base_seed)


def custom_shape(K: int, N: int, bits: int, group_size: int, m_values: Sequence[int] = (1,),
                 seed: int = 1234, outliers: bool = False, name: Optional[str] = None) -> Shape:
    """A shape outside the named workloads (tests: ragged tails, edge cases)."""
    return Shape(name or f"custom_k{K}_n{N}_{bits}b_g{group_size}", K, N, bits, group_size,
                 tuple(m_values), seed, outliers)


def custom_fp_shape(K: int, N: int, fmt: str, m_values: Sequence[int] = (1,), seed: int = 1234,
                    outliers: bool = False) -> Shape:
    """An FP-format shape outside the named workloads."""
    return Shape(f"custom_k{K}_n{N}_{fmt}", K, N, FP_BITS[fmt], FP_BLOCK[fmt], tuple(m_values),
                 seed, outliers, fmt=fmt)


def special_problem(K: int, N: int, bits: int, group_size: int, M: int, kind: str,
                    seed: int = 7, outliers: bool = False) -> Problem:
    """Structured inputs with closed-form results.

    kind = "zero_codes": every code 0 (w = bias).
    kind = "unit_scale_onehot": scale 1.0, bias 0.0, random codes, x row m = e_{k_m}
      (one-hot at column k_m = (m * 37 + 5) % K); then y[m, n] = q[n, k_m] exactly.
    kind = "zero_weights": every code of row n equals the zero point z_n = n mod 2^bits
      (rows cycle through all code values) and b = -z_n * s exactly: each scale is
      drawn as usual, then rounded to the 11 - bitlength(z_n) significant bits that
      keep z_n * s exact in fp16.  Every weight dequantizes to exactly 0, so
      y[m, n] = 0 (x keeps its outlier channels when `outliers`).
    """
    shape = custom_shape(K, N, bits, group_size, (M,), seed=seed, name=f"{kind}_k{K}_n{N}",
                         outliers=outliers)
    p = make_problem(shape, m_max=M, seed=seed)
    if kind == "zero_weights":
        z = np.arange(N, dtype=np.int64) % (1 << bits)
        per_byte = 8 // bits
        byte = np.zeros(N, dtype=np.int64)
        for j in range(per_byte):
            byte |= z << (bits * j)
        p.codes[:] = byte.astype(np.uint8)[:, None]
        s = p.scales.view(np.float16).astype(np.float64)
        keep = 11 - np.array([int(v).bit_length() for v in z])  # significant bits of s
        mant, expo = np.frexp(s)
        s = np.ldexp(np.round(np.ldexp(mant, keep[:, None])), expo - keep[:, None])
        p.scales[:] = f64_to_fp16_bits(s)
        p.biases[:] = f64_to_fp16_bits(-z[:, None] * s)
        assert np.array_equal(p.biases.view(np.float16).astype(np.float64), -z[:, None] * s)
    elif kind == "zero_codes":
        p.codes[:] = 0
    elif kind == "unit_scale_onehot":
        p.scales[:] = np.float16(1.0).view(np.uint16)
        p.biases[:] = np.float16(0.0).view(np.uint16)
        p.x[:] = 0
        for m in range(M):
            p.x[m, onehot_column(m, K)] = f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    else:
        raise ValueError(kind)
    return p


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """One MoE expert projection: E experts of [N, K], affine codes; M verify
    rows, each routed to `topk` distinct experts."""

    name: str
    E: int
    K: int
    N: int
    bits: int
    group_size: int
    topk: int
    m_values: Tuple[int, ...]
    seed: int


# Qwen3-30B-A3B's expert FFN (named on the MLX page, Facts: the group-size
# decode study): 128 experts, 8 active per token, hidden size 2048, expert
# intermediate size 768; gate and up fused into one [1536, 2048] matrix.
MOE_WORKLOADS: Dict[str, MoeShape] = {s.name: s for s in [
    MoeShape("moe30b_gateup_e128_k2048_n1536_4b_g64_top8", 128, 2048, 1536, 4, 64, 8,
             tuple(range(1, 17)), seed=70000),
    MoeShape("moe30b_down_e128_k768_n2048_4b_g64_top8", 128, 768, 2048, 4, 64, 8,
             tuple(range(1, 17)), seed=70100),
]}


@dataclasses.dataclass
class MoeProblem:
    """codes [E, N, K*bits/8]; scales, biases [E, N, K/gs] fp16 bits; x [Mmax, K]
    bf16 bits; routing [Mmax, topk] expert ids (distinct per row).  An M-row
    verify uses pairs p = m*topk + j for m < M: x_idx[p] = m,
    e_idx[p] = routing[m, j]."""

    shape: MoeShape
    codes: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    x: np.ndarray
    routing: np.ndarray

    def pairs(self, M: int):
        k = self.shape.topk
        x_idx = np.repeat(np.arange(M, dtype=np.int32), k)
        e_idx = self.routing[:M].reshape(-1).astype(np.int32)
        return x_idx, e_idx


def make_moe_problem(shape: MoeShape, m_max: Optional[int] = None) -> MoeProblem:
    """Expert weights with the 4-bit affine distributions of the dense
    workloads (drawn expert by expert), x ~ N(0, 1) in bf16, then the routing:
    each row picks `topk` distinct experts uniformly at random.  Draw order:
    codes, scales, bias noise, x, routing."""
    m_max = m_max or max(shape.m_values)
    rng = np.random.default_rng(shape.seed)
    codes = _draw_codes(rng, shape.E * shape.N, shape.K, shape.bits).reshape(shape.E, shape.N, -1)
    s, b = _draw_meta(rng, shape.E * shape.N, shape.K // shape.group_size, shape.bits)
    scales = s.reshape(shape.E, shape.N, -1)
    biases = b.reshape(shape.E, shape.N, -1)
    x, _ = _draw_x(rng, m_max, shape.K, False)
    routing = np.stack([rng.choice(shape.E, size=shape.topk, replace=False) for _ in range(m_max)])
    return MoeProblem(shape, codes, scales, biases, x, routing.astype(np.int32))


def make_residual(M: int, N: int, seed: int) -> np.ndarray:
    """Residual input of the fused residual sum: float32 [M, N] ~ N(0, 1), drawn
    from its own stream (seed + 1_000_003) so the problem's other draws do not
    change.  Its magnitude is that of y on the 4-bit workloads (|y| ~ 1-2)."""
    rng = np.random.default_rng(seed + 1_000_003)
    return rng.standard_normal(size=(M, N)).astype(np.float32)


def onehot_column(m: int, K: int) -> int:
    return (m * 37 + 5) % K


def list_workloads() -> List[str]:
    return list(WORKLOADS)
