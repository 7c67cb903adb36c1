"""GPU parity on seeded random shapes: every path that runs the shape, at
random row counts, against the fp64 oracle, every element; and, within a
forced path, row 0 of every M-row call bitwise equal to the single-row call
(K <= 4096, where no kernel configuration depends on M).  The affine formats,
the block-scaled FP formats, and the fused residual sum (bitwise the plain
call plus r).

The shapes are drawn to cross the kernels' choices: N from a few columns (one
ragged tile) to past 256 tiles (the persistent kernels), K from one bias block
to 4096, every supported bit width and group size, outlier channels on half of
them."""
import numpy as np
import pytest

from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import DeviceProblem, OracleRows, say

pytestmark = pytest.mark.gpu

FORMATS = [(2, 32), (2, 64), (2, 128), (4, 32), (4, 64), (4, 128), (8, 32), (8, 64), (8, 128)]


def draw_cases(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        bits, gs = FORMATS[rng.integers(len(FORMATS))]
        step = int(np.lcm(64, 4 * gs))  # K a multiple of a bias block (and of 64)
        K = step * int(rng.integers(1, 4096 // step + 1))
        N = int(rng.choice([rng.integers(1, 48), rng.integers(48, 1200), rng.integers(4096, 6000)]))
        Ms = sorted(set(int(m) for m in rng.integers(1, 17, size=3)))
        cases.append((i, bits, gs, K, N, Ms, bool(rng.integers(2))))
    return cases


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


@pytest.mark.parametrize("i,bits,gs,K,N,Ms,outliers", draw_cases(24, seed=20261202))
def test_random_shape_every_element(i, bits, gs, K, N, Ms, outliers):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=5000 + i, outliers=outliers), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, max(Ms))
    for path in ("dot", "mfma", "auto"):
        if not q.qgemv_path_supported(path, 1, N, K, bits, gs):
            continue
        y1 = None
        for M in [1] + Ms:
            say(f"random case {i}: {path} bits={bits} gs={gs} K={K} N={N} M={M}")
            y = d.run_host(M, path)
            orc.check(y, M, label=f"case {i} {path} M={M}")
            if M == 1:
                y1 = y
            elif path != "auto":  # the dispatcher may pick another path at another M
                assert np.array_equal(y[:1], y1), f"case {i} {path}: row 0 of M={M} differs from M=1"
        torch.cuda.synchronize()


def draw_partial_cases(n_cases: int, seed: int):
    # K a whole number of super-chunks (128 codes at 4 bits, 256 at 2) with
    # at least 4 groups but not a whole number of 4-group bias blocks: the
    # single-pass MFMA kernel's partial-block variant
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        bits, gs = [(4, 64), (4, 128), (2, 128)][rng.integers(3)]
        scw = 512 // bits
        K = scw * int(rng.integers(1, 12288 // scw + 1))
        if K % gs or K // gs < 4 or K % (4 * gs) == 0:
            continue
        N = int(rng.choice([rng.integers(1, 48), rng.integers(48, 1200), rng.integers(4096, 6000)]))
        Ms = sorted(set(int(m) for m in rng.integers(1, 17, size=3)))
        cases.append((len(cases), bits, gs, K, N, Ms, bool(rng.integers(2))))
    return cases


@pytest.mark.parametrize("i,bits,gs,K,N,Ms,outliers", draw_partial_cases(12, seed=20261204))
def test_random_partial_block_shape_every_element(i, bits, gs, K, N, Ms, outliers):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=7000 + i, outliers=outliers), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, max(Ms))
    for path in ("dot", "mfma", "auto"):
        assert q.qgemv_path_supported(path, 1, N, K, bits, gs)
        y1 = None
        for M in [1] + Ms:
            say(f"random partial-block case {i}: {path} bits={bits} gs={gs} K={K} N={N} M={M}")
            y = d.run_host(M, path)
            orc.check(y, M, label=f"case {i} {path} M={M}")
            if M == 1:
                y1 = y
            elif path != "auto":
                assert np.array_equal(y[:1], y1), f"case {i} {path}: row 0 of M={M} differs from M=1"


def draw_fp_cases(n_cases: int, seed: int):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        fmt = ["mxfp4", "nvfp4", "mxfp8"][rng.integers(3)]
        K = 64 * int(rng.integers(1, 64 + 1))  # 64..4096 (the MFMA path needs K % 128 == 0)
        N = int(rng.choice([rng.integers(1, 48), rng.integers(48, 1200), rng.integers(4096, 6000)]))
        Ms = sorted(set(int(m) for m in rng.integers(1, 17, size=3)))
        cases.append((i, fmt, K, N, Ms))
    return cases


@pytest.mark.parametrize("i,fmt,K,N,Ms", draw_fp_cases(12, seed=20261203))
def test_random_fp_shape_every_element(i, fmt, K, N, Ms):
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=6000 + i), m_max=16)
    d_codes, d_scales, d_x, torch = _fp_device(p)
    orc = OracleRows.fp(p, max(Ms))
    for path in ("dot", "mfma", "auto"):
        if not q.qgemv_path_supported_fp(path, 1, N, K, fmt):
            continue
        y1 = None
        for M in [1] + Ms:
            say(f"random fp case {i}: {path} {fmt} K={K} N={N} M={M}")
            y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
            q.qgemv_run_path_fp(path, d_codes, d_scales, d_x, None, y, M, N, K, fmt)
            torch.cuda.synchronize()
            yh = y.cpu().numpy()
            orc.check(yh, M, label=f"fp case {i} {path} M={M}")
            if M == 1:
                y1 = yh
            elif path != "auto":
                assert np.array_equal(yh[:1], y1), f"fp case {i} {path}: row 0 of M={M} differs from M=1"


def _fp_device(p):
    import torch
    return (torch.from_numpy(p.codes).to("cuda:0"), torch.from_numpy(p.scales).to("cuda:0"),
            torch.from_numpy(p.x.view(np.int16)).to("cuda:0"), torch)


@pytest.mark.parametrize("i,bits,gs,K,N,Ms,outliers", draw_cases(12, seed=20261204))
def test_random_shape_fused_residual(i, bits, gs, K, N, Ms, outliers):
    # y = x W^T + r through the fused entry point, every path, against the
    # oracle's product plus r, and bitwise equal to the plain call plus r
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=7000 + i, outliers=outliers), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, max(Ms))
    r = synth.make_residual(16, N, seed=p.seed)
    for path in ("dot", "mfma", "auto"):
        if not q.qgemv_path_supported(path, 1, N, K, bits, gs):
            continue
        for M in Ms:
            say(f"random residual case {i}: {path} bits={bits} gs={gs} K={K} N={N} M={M}")
            r_dev = torch.from_numpy(r[:M].copy()).to("cuda:0")
            y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
            q.qgemv_run_path_add(path, d.codes, d.scales, d.biases, d.x, r_dev, y, M, N, K, bits, gs)
            torch.cuda.synchronize()
            yh = y.cpu().numpy()
            orc.check(yh, M, label=f"residual case {i} {path} M={M}", residual=r)
            plain = d.run_host(M, path)
            assert np.array_equal(yh, (plain + r[:M]).astype(np.float32)), f"residual case {i} {path} M={M}"
