"""GPU parity at the size limits of the C ABI: the longest K (QGEMV_MAX_K) and
the widest N (QGEMV_MAX_N), every path, against the fp64 oracle, every
element."""
import numpy as np
import pytest

import oracle
from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import DeviceProblem, OracleRows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


def _check(p, y, M, cols, label):
    ref = oracle.qgemv_reference(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits,
                                 p.group_size, rows=cols)
    absum = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits,
                                   p.group_size, rows=cols)
    yy = y if cols is None else y[:, cols]
    assert np.all(np.isfinite(yy)), f"{label}: non-finite output"
    ok, worst, idx = oracle.check_close(yy, ref, absum)
    assert ok, f"{label}: worst |dy|/tol = {worst:.3g} at {idx}"


@pytest.mark.parametrize("N,bits,gs", [(40, 4, 128), (24, 2, 64), (20, 8, 64)])
def test_longest_k_every_element(N, bits, gs):
    K = q.MAX_K
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=11 + N, outliers=True), m_max=16)
    d = DeviceProblem(p)
    for path in ("dot", "mfma", "auto"):
        if not q.qgemv_path_supported(path, 1, N, K, bits, gs):
            continue
        for M in (1, 5, 16):
            say(f"max K {path} K={K} N={N} bits={bits} gs={gs} M={M}")
            _check(p, d.run_host(M, path), M, None, f"{path} K={K} N={N} M={M}")


@pytest.mark.parametrize("K,bits,gs", [(128, 4, 32), (256, 2, 64), (128, 8, 32)])
def test_widest_n_every_element(K, bits, gs):
    N = q.MAX_N
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=13 + K), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, 16)
    for path in ("dot", "mfma", "auto"):
        if not q.qgemv_path_supported(path, 1, N, K, bits, gs):
            continue
        for M in (1, 8, 16):
            say(f"max N {path} K={K} N={N} bits={bits} gs={gs} M={M}")
            y = d.run_host(M, path)
            assert np.all(np.isfinite(y)), "non-finite output"
            orc.check(y, M, label=f"{path} K={K} N={N} M={M}")
