"""GPU parity of the fused residual sum y = x W^T + r (qgemv_small_add /
qgemv_run_path_add) through the C ABI.

Bars:
* every element within 1e-3 * sum|x w| + 1e-6 + 2^-23 * (|r| + sum|x w|) of
  the fp64 oracle, full sizes included;
* bit for bit the plain product of the same path followed by one fp32 add
  (numpy's IEEE round-to-nearest-even add), out of place and in place -- the
  in-place call on a shape where the MFMA path splits K is held to the
  tolerance only (it runs the unsplit kernel);
* row m of an M-row call equals the M=1 call on x[m], r[m] bitwise.
"""
import numpy as np
import pytest

import oracle
from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import DeviceProblem, OracleRows, say

pytestmark = pytest.mark.gpu

PATHS = ["dot", "mfma", "auto"]


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


def run_add(d: DeviceProblem, M: int, r_dev, path="auto", y=None):
    import torch
    p = d.p
    if y is None:
        y = torch.full((M, p.N), float("nan"), dtype=torch.float32, device=d.device)
    q.qgemv_run_path_add(path, d.codes, d.scales, d.biases, d.x, r_dev, y, M, p.N, p.K, p.bits,
                         p.group_size)
    torch.cuda.synchronize()
    return y


def check_add(p, y, r, M, cols=None, label=""):
    ref = oracle.qgemv_add_reference(p.codes, p.scales, p.biases, p.x, r, M, p.N, p.K, p.bits,
                                     p.group_size, rows=cols)
    absum = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits,
                                   p.group_size, rows=cols)
    rr = r[:M] if cols is None else r[:M][:, cols]
    yy = y if cols is None else y[:, cols]
    ok, worst, idx = oracle.check_close(yy, ref, absum, residual_abs=rr)
    assert ok, f"{label}: worst |dy|/tol = {worst:.3g} at {idx}"


def supported(path, p, M=1):
    return q.qgemv_path_supported(path, M, p.N, p.K, p.bits, p.group_size)


def fp32_add(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return (a.astype(np.float32) + b.astype(np.float32)).astype(np.float32)


SHAPES = [
    # K, N, bits, gs: ragged N, several K stages, many tiles per CU, K split
    (256, 512, 4, 64), (640, 40, 4, 32), (1024, 300, 4, 64), (2048, 97, 4, 128),
    (8192, 33, 4, 64), (512, 72, 2, 32), (1280, 300, 2, 64), (17408, 23, 2, 64),
    (64, 5, 2, 64), (2048, 4500, 4, 64), (1280, 4700, 2, 64), (5120, 1024, 4, 128),
    (1024, 300, 8, 64), (2048, 4500, 8, 32), (5120, 1024, 8, 64), (2048, 97, 8, 128),
    (3840, 4200, 8, 64), (5120, 4150, 8, 64),
    # long K, many tiles: halves of K with their activations in LDS
    (6656, 4200, 4, 128), (8192, 4130, 2, 64),
]


@pytest.mark.parametrize("K,N,bits,gs", SHAPES)
@pytest.mark.parametrize("path", PATHS)
def test_add_every_element_and_bitwise_plain_plus_add(path, K, N, bits, gs):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=7 * K + N, outliers=True), m_max=16)
    if not supported(path, p):
        pytest.skip("path does not support this shape")
    d = DeviceProblem(p)
    r = synth.make_residual(16, N, seed=p.seed)
    for M in (1, 2, 5, 8, 16):
        say(f"add {path} K={K} N={N} bits={bits} gs={gs} M={M}")
        r_dev = torch.from_numpy(r[:M].copy()).to(d.device)
        y = run_add(d, M, r_dev, path).cpu().numpy()
        check_add(p, y, r, M, label=f"add {path} K={K} N={N} M={M}")
        plain = d.run_host(M, path)
        assert np.array_equal(y, fp32_add(plain, r[:M])), f"M={M}: not plain + r bit for bit"


def _mfma_splits_k(p, M) -> bool:
    # the MFMA kernels that split K over two workgroups add the halves into a
    # prefilled y, which an in-place call cannot have: it takes the unsplit
    # single-pass kernel, whose sums are ordered otherwise.  The single-pass
    # kernel splits K when its 16-column tile groups are few for the CUs; the
    # register-resident persistent kernel (more tiles than CUs) for 8-bit
    # codes in groups of 64 with more than 16 bias blocks.  The shapes are
    # chosen on either side of these rules (256 CUs).
    tiles = (p.N + 15) // 16
    single = (tiles < 512 and p.K >= 8192) or (4 * tiles <= 256 and p.K >= 2048)
    persist = tiles > 256 and p.bits == 8 and p.group_size == 64 and p.K > 16 * 256
    return single or persist


@pytest.mark.parametrize("K,N,bits,gs", [(2048, 97, 4, 128), (1024, 300, 4, 64),
                                         (2048, 4500, 4, 64), (17408, 23, 2, 64),
                                         (5120, 1024, 4, 128), (5120, 4150, 8, 64)])
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_add_in_place(path, K, N, bits, gs):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=11 * K + N), m_max=16)
    d = DeviceProblem(p)
    r = synth.make_residual(16, N, seed=p.seed)
    for M in (1, 4, 16):
        say(f"add in place {path} K={K} N={N} M={M}")
        y = torch.from_numpy(r[:M].copy()).to(d.device)
        run_add(d, M, y, path, y=y)
        yh = y.cpu().numpy()
        check_add(p, yh, r, M, label=f"in place {path} K={K} N={N} M={M}")
        if path == "dot" or not _mfma_splits_k(p, M):
            assert np.array_equal(yh, fp32_add(d.run_host(M, path), r[:M])), f"M={M}"


@pytest.mark.parametrize("path", ["dot", "mfma"])
@pytest.mark.parametrize("K,N,bits,gs", [(2048, 200, 4, 64), (2048, 4500, 2, 128), (10240, 150, 2, 64)])
def test_add_row_of_m_row_call_equals_single_row_call(path, K, N, bits, gs):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=79), m_max=16)
    d = DeviceProblem(p)
    r = synth.make_residual(16, N, seed=p.seed)
    r_all = torch.from_numpy(r).to(d.device)
    say(f"add row invariance {path} K={K} N={N} bits={bits} gs={gs}")
    singles = []
    for m in range(16):
        y1 = torch.empty((1, N), dtype=torch.float32, device=d.device)
        q.qgemv_run_path_add(path, d.codes, d.scales, d.biases, d.x[m:m + 1].clone(),
                             r_all[m:m + 1].clone(), y1, 1, N, K, bits, gs)
        singles.append(y1)
    torch.cuda.synchronize()
    singles = torch.cat(singles).cpu().numpy()
    for M in (2, 5, 8, 16):
        y = run_add(d, M, r_all[:M].clone(), path).cpu().numpy()
        assert np.array_equal(y, singles[:M]), f"M={M}"


FULL = [("square_k4096_n4096_4b_g64", (1, 4, 8)), ("layer27b_k", (1, 8, 16)),
        ("layer27b_gate", (2, 8, 16)), ("layer27b_down", (1, 4, 8, 16)),
        ("lowram27b_down_k17408_n5120_2b_g64", (2, 12)), ("ffnup_k4096_n12288_4b_g32", (4, 8)),
        ("mlxbench_k5120_n17408_8b_g64", (1, 8, 16))]


@pytest.mark.parametrize("name,ms", FULL)
def test_add_full_size_every_element(name, ms):
    import torch
    s = synth.WORKLOADS[name]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    r = synth.make_residual(max(ms), s.N, seed=p.seed)
    orc = OracleRows.affine(p, max(ms))
    for path in PATHS:
        if not supported(path, p):
            continue
        for M in ms:
            say(f"add full {name} {path} M={M}")
            r_dev = torch.from_numpy(r[:M].copy()).to(d.device)
            y = run_add(d, M, r_dev, path).cpu().numpy()
            assert np.all(np.isfinite(y)), "non-finite output"
            orc.check(y, M, label=f"{name} {path} M={M}", residual=r)
            assert np.array_equal(y, fp32_add(d.run_host(M, path), r[:M]))


def test_add_auto_matches_select_and_small_add():
    import torch
    s = synth.WORKLOADS["square_k4096_n4096_4b_g64"]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    r = synth.make_residual(8, s.N, seed=p.seed)
    for M in s.m_values:
        r_dev = torch.from_numpy(r[:M].copy()).to(d.device)
        name = {q.PATH_DOT: "dot", q.PATH_MFMA: "mfma"}[q.qgemv_select(M, s.N, s.K, s.bits, s.group_size)]
        say(f"add auto vs {name} M={M}")
        y = torch.empty((M, s.N), dtype=torch.float32, device=d.device)
        q.qgemv_small_add(d.codes, d.scales, d.biases, d.x, r_dev, y, M, s.N, s.K, s.bits, s.group_size)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), run_add(d, M, r_dev, name).cpu().numpy())


def test_add_torch_helper_and_overlap_rejected():
    import torch
    s = synth.WORKLOADS["tiny_k256_n512_4b_g64"]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    M = 4
    r = synth.make_residual(M, s.N, seed=p.seed)
    r_dev = torch.from_numpy(r).to(d.device)
    say("add torch helper")
    y = q.small(d.codes, d.scales, d.biases, d.x[:M], 4, 64, residual=r_dev)
    torch.cuda.synchronize()
    check_add(p, y.cpu().numpy(), r, M, label="helper")
    big = torch.zeros((2 * M, s.N), dtype=torch.float32, device=d.device)
    with pytest.raises(q.QgemvError) as e:
        q.qgemv_small_add(d.codes, d.scales, d.biases, d.x, big[1:M + 1], big[:M], M, s.N, s.K, 4, 64)
    assert e.value.status == q.EINVAL
