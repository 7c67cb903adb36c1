"""Algorithmic byte and flop counts for one few-row quantized GEMV call.

The weight stream W = packed codes + fp16 scales + fp16 biases is what the
method reads once per call instead of once per activation row.  "Effective
weight GB/s" divides W by the kernel time.  That is the byte model behind the
roofline figure of the MLX quantized_matmul small-M verify kernels page
(Facts: the M3 Ultra microbench puts (M,5120)@(17408,5120)^T, 4-bit g64, at
about 0.074 ms at 677 GB/s -- W alone, 50,135,040 B, gives 0.0741 ms) and of
its group-size bullet (scale+bias are 20% / 11% / 5.9% of the stream at
g32 / g64 / g128).

Total algorithmic bytes add the activations (bf16, read once) and the fp32
output (written once).
"""
from __future__ import annotations

__all__ = ["code_bytes", "meta_bytes", "weight_bytes", "algorithmic_bytes", "useful_flops",
           "metadata_share", "fp_weight_bytes", "fp_algorithmic_bytes"]


def code_bytes(N: int, K: int, bits: int) -> int:
    return N * K * bits // 8


def meta_bytes(N: int, K: int, group_size: int) -> int:
    # one fp16 scale + one fp16 bias per (row, group)
    return 4 * N * (K // group_size)


def weight_bytes(N: int, K: int, bits: int, group_size: int) -> int:
    return code_bytes(N, K, bits) + meta_bytes(N, K, group_size)


def algorithmic_bytes(M: int, N: int, K: int, bits: int, group_size: int) -> int:
    return weight_bytes(N, K, bits, group_size) + 2 * M * K + 4 * M * N


def fp_weight_bytes(N: int, K: int, bits: int, block: int) -> int:
    """Block-scaled FP formats: packed elements plus one scale byte per block."""
    return code_bytes(N, K, bits) + N * (K // block)


def fp_algorithmic_bytes(M: int, N: int, K: int, bits: int, block: int) -> int:
    return fp_weight_bytes(N, K, bits, block) + 2 * M * K + 4 * M * N


def useful_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def metadata_share(bits: int, group_size: int) -> float:
    """Fraction of the weight stream taken by scale+bias."""
    per_group_codes = group_size * bits / 8.0
    return 4.0 / (per_group_codes + 4.0)
