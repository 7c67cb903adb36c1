"""GPU parity on rows whose weights dequantize to exactly zero.

Every code of row n equals a zero point z_n (rows cycle through all code
values) and its bias is -z_n * s exactly, so y = 0 and the tolerance is the
absolute floor 1e-6 alone: the case where a decode that carries an offset, or a
scale term and a bias term that cancel in fp32, loses to rounding.  The kernels
decode codes without an offset, and each lane keeps traces of nonzero weights
in the groups it folds (codes that differ within a group, or a group weight
s*c + b that is not exactly zero) and contributes exactly 0 when there are
none, so:
* every element is exactly 0, and with a residual exactly the residual;
* hence within the tolerance (the worst |dy|/tol is printed).
Both paths and the dispatcher, 2-, 4- and 8-bit codes, every group size, short
and long K (a partial last bias block included), single-pass and persistent
MFMA kernels, plain and fused sums, activations with x20 outlier channels.
"""
import numpy as np
import pytest

from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import DeviceProblem, OracleRows, say

pytestmark = pytest.mark.gpu

# K, N, bits, gs: N = 300 runs the single-pass MFMA kernel (K split over two
# workgroups), N = 4200 / 4128 the persistent kernels (registers for K 3840 to
# 5120, half of K in LDS for 17408)
SHAPES = [
    (4096, 300, 4, 32), (4096, 300, 4, 64), (4096, 300, 4, 128),
    (17408, 300, 4, 32), (17408, 300, 4, 64), (17408, 300, 4, 128),
    (4096, 300, 2, 32), (4096, 300, 2, 64), (4096, 300, 2, 128),
    (17408, 300, 2, 64), (17408, 300, 2, 128),
    (4096, 4200, 4, 64), (5120, 4200, 2, 64), (17408, 4200, 4, 128), (17408, 4128, 2, 64),
    (4096, 300, 8, 32), (4096, 300, 8, 64), (4096, 300, 8, 128),
    (4096, 4200, 8, 32), (3840, 4200, 8, 64), (5120, 4200, 8, 64),
    # a partial last bias block (single-pass MFMA kernel)
    (640, 300, 4, 128), (11008, 300, 4, 128), (768, 300, 2, 128), (4864, 4200, 4, 128),
]
MS = (1, 2, 8, 16)


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


@pytest.mark.parametrize("K,N,bits,gs", SHAPES)
def test_zero_weight_rows(K, N, bits, gs):
    import torch
    p = synth.special_problem(K, N, bits, gs, max(MS), "zero_weights", seed=K + N + bits, outliers=True)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, max(MS))
    assert np.all(orc.ref == 0.0)
    r = synth.make_residual(max(MS), N, seed=K + N)
    r_dev = torch.from_numpy(r).to("cuda:0")
    worst = 0.0
    for path in ("dot", "mfma", "auto"):
        if not q.qgemv_path_supported(path, 1, N, K, bits, gs):
            continue
        for M in MS:
            say(f"zero weights {path} K={K} N={N} bits={bits} gs={gs} M={M}")
            y = d.run_host(M, path)
            worst = max(worst, orc.check(y, M, label=f"{path} M={M}"))
            assert np.all(y == 0.0), f"{path} M={M}: a zero row is not exactly 0"
            ya = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
            q.qgemv_run_path_add(path, d.codes, d.scales, d.biases, d.x, r_dev, ya, M, N, K, bits, gs)
            torch.cuda.synchronize()
            ya = ya.cpu().numpy()
            worst = max(worst, orc.check(ya, M, label=f"{path} add M={M}", residual=r))
            assert np.array_equal(ya, r[:M]), f"{path} add M={M}: zero rows plus r are not r"
    say(f"zero weights K={K} N={N} bits={bits} gs={gs}: worst |dy|/tol = {worst:.3g}")
