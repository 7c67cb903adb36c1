"""The byte model behind the bench's GB/s and roofline figures against the
buffers the library is handed (no GPU): the weight stream is exactly the
packed codes plus the per-group (or per-block) metadata the generator lays
out, and the algorithmic bytes of an M-row call add M bf16 activation rows
and M fp32 output rows."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from few_row_quantized_amd import accounting, synth  # noqa: E402

AFFINE = [(2, 64), (2, 128), (4, 32), (4, 64), (4, 128), (8, 32), (8, 64)]
FP = [("mxfp4", 4, 32), ("nvfp4", 4, 16), ("mxfp8", 8, 32)]
K, N, M = 1024, 48, 5


@pytest.mark.parametrize("bits,gs", AFFINE)
def test_affine_weight_stream_is_the_buffers(bits, gs):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs), m_max=M)
    assert p.codes.nbytes == accounting.code_bytes(N, K, bits)
    assert p.scales.nbytes + p.biases.nbytes == accounting.meta_bytes(N, K, gs)
    w = p.codes.nbytes + p.scales.nbytes + p.biases.nbytes
    assert w == accounting.weight_bytes(N, K, bits, gs)
    y_bytes = 4 * M * N
    assert accounting.algorithmic_bytes(M, N, K, bits, gs) == w + p.x[:M].nbytes + y_bytes


@pytest.mark.parametrize("fmt,bits,block", FP)
def test_fp_weight_stream_is_the_buffers(fmt, bits, block):
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt), m_max=M)
    assert p.biases.nbytes == 0
    w = p.codes.nbytes + p.scales.nbytes
    assert w == accounting.fp_weight_bytes(N, K, bits, block)
    assert accounting.fp_algorithmic_bytes(M, N, K, bits, block) == w + p.x[:M].nbytes + 4 * M * N


def test_metadata_share_is_the_buffers_share():
    for bits, gs in AFFINE:
        p = synth.make_problem(synth.custom_shape(K, N, bits, gs), m_max=1)
        meta = p.scales.nbytes + p.biases.nbytes
        share = meta / (meta + p.codes.nbytes)
        assert abs(accounting.metadata_share(bits, gs) - share) < 1e-12, (bits, gs)
