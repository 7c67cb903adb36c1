"""GPU parity where K is not a whole number of bias blocks (4 groups): the
single-pass MFMA kernel takes a partial last block (2- and 4-bit codes, K a
whole number of 64-byte super-chunks and of at least 4 groups), the
persistent kernels do not run, and the dot path covers the same shapes.

Bars: every element within 1e-3 * sum|x w| + 1e-6 of the oracle on both
paths and the dispatcher (plain and fused residual sums, K split over two
workgroups on small N, more tiles than CUs); on the MFMA path row m of an
M-row call equals the M=1 call on x[m] bit for bit.
"""
import numpy as np
import pytest

import oracle
from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import DeviceProblem, OracleRows, say

pytestmark = pytest.mark.gpu

# K, N, bits, gs: the last block holds 1 to 3 of its 4 groups
SHAPES = [
    (640, 200, 4, 128),     # 5 groups: a block and one group
    (384, 96, 4, 64),       # 6 groups: a block and two
    (768, 130, 2, 128),     # 2-bit, 6 groups
    (1280, 72, 2, 64),      # 2-bit, 20 groups: 5 blocks (whole: control)
    (2176, 64, 4, 64),      # 34 groups over two workgroups (K split)
    (8960, 300, 4, 128),    # 70 groups
    (11008, 1000, 4, 128),  # 86 groups
    (4864, 4500, 4, 128),   # 38 groups, 282 tiles: more tiles than CUs
]
MS = (1, 2, 3, 5, 8, 13, 16)


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


def test_support_rules():
    sup = q.qgemv_path_supported
    for K, N, bits, gs in SHAPES:
        assert sup("mfma", 1, N, K, bits, gs), (K, bits, gs)
    assert not sup("mfma", 1, 64, 384, 4, 128)   # 3 groups
    assert not sup("mfma", 1, 64, 4352, 8, 128)  # 8-bit codes: whole blocks only


@pytest.mark.parametrize("K,N,bits,gs", SHAPES)
def test_partial_block_every_element(K, N, bits, gs):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=9 * K + N, outliers=True), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, 16)
    r = synth.make_residual(16, N, seed=K + 3 * N)
    r_dev = torch.from_numpy(r).to("cuda:0")
    for path in ("mfma", "dot", "auto"):
        for M in MS:
            say(f"partial block {path} K={K} N={N} bits={bits} gs={gs} M={M}")
            orc.check(d.run_host(M, path), M, label=f"{path} M={M}")
        for M in (1, 8):
            ya = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
            q.qgemv_run_path_add(path, d.codes, d.scales, d.biases, d.x, r_dev, ya, M, N, K, bits, gs)
            torch.cuda.synchronize()
            orc.check(ya.cpu().numpy(), M, label=f"{path} add M={M}", residual=r)


@pytest.mark.parametrize("K,N,bits,gs", SHAPES)
def test_partial_block_rows_equal_single_row_calls_bitwise(K, N, bits, gs):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=13 * K + N), m_max=16)
    d = DeviceProblem(p)
    say(f"partial block row invariance K={K} N={N} bits={bits} gs={gs}")
    singles = []
    for m in range(16):
        y1 = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        q.qgemv_run_path("mfma", d.codes, d.scales, d.biases, d.x[m:m + 1].clone(), y1, 1, N, K, bits, gs)
        singles.append(y1)
    torch.cuda.synchronize()
    singles = torch.cat(singles).cpu().numpy()
    for M in (2, 4, 5, 8, 9, 16):
        assert np.array_equal(d.run_host(M, "mfma"), singles[:M]), f"M={M}"


def test_partial_block_gathered_verify():
    # experts with a partial last block: the gathered verify's single-pass
    # kernel at every row count (the persistent form needs whole blocks)
    import torch
    s = synth.MoeShape("moe_partial", 6, 640, 200, 4, 128, 4, (16,), 43)
    p = synth.make_moe_problem(s, m_max=16)
    rng = np.random.default_rng(47)
    codes = torch.from_numpy(p.codes).to("cuda:0")
    scales = torch.from_numpy(p.scales.view(np.int16)).to("cuda:0")
    biases = torch.from_numpy(p.biases.view(np.int16)).to("cuda:0")
    x = torch.from_numpy(p.x.view(np.int16)).to("cuda:0")
    for X in (1, 2, 4, 16):
        P = 24
        x_idx = rng.integers(0, X, size=P)
        e_idx = rng.integers(0, s.E, size=P)
        y = torch.full((P, s.N), float("nan"), dtype=torch.float32, device="cuda:0")
        say(f"partial block gather X={X}")
        q.qgemv_gather(codes, scales, biases, x, torch.from_numpy(x_idx.astype(np.int32)).to("cuda:0"),
                       torch.from_numpy(e_idx.astype(np.int32)).to("cuda:0"), y, P, X, s.E, s.N, s.K, s.bits,
                       s.group_size)
        torch.cuda.synchronize()
        ref = oracle.qgemv_gather_reference(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K, s.bits,
                                            s.group_size)
        absum = oracle.gather_abs_product_sum(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K,
                                              s.bits, s.group_size)
        ok, worst, idx = oracle.check_close(y.cpu().numpy(), ref, absum)
        assert ok, f"X={X}: worst |dy|/tol = {worst:.3g} at {idx}"
