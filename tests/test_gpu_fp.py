"""GPU parity of the block-scaled FP formats (mxfp4, nvfp4, mxfp8) through the
C ABI against the fp64 oracle.

Bars:
* decoded elements bit-exact: the unpack probe of each path writes the bf16
  pattern of every element, equal to the oracle's decoded value (all E2M1 and
  E4M3 values are bf16 values); through the real kernels, unit scales and
  one-hot x give y equal to the element exactly;
* y: |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-6 per element (plus the
  residual term for the fused residual sum), every element on small, ragged
  and full-size shapes;
* row m of an M-row call equals the M=1 call on x[m] bitwise; the fused
  residual sum equals the plain product plus r rounded once, bit for bit.
"""
import numpy as np
import pytest

import oracle
from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import OracleRows, say

pytestmark = pytest.mark.gpu

FMTS = ["mxfp4", "nvfp4", "mxfp8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


class FpDevice:
    def __init__(self, p, device="cuda:0"):
        import torch
        self.p = p
        self.codes = torch.from_numpy(p.codes).to(device)
        self.scales = torch.from_numpy(p.scales).to(device)
        self.x = torch.from_numpy(p.x.view(np.int16)).to(device)
        self.device = device

    def run(self, M, path="auto", residual=None, y=None):
        import torch
        p = self.p
        if y is None:
            y = torch.full((M, p.N), float("nan"), dtype=torch.float32, device=self.device)
        q.qgemv_run_path_fp(path, self.codes, self.scales, self.x, residual, y, M, p.N, p.K,
                            p.shape.fmt)
        torch.cuda.synchronize()
        return y.cpu().numpy()


def check(p, y, M, cols=None, residual=None, label=""):
    ref = oracle.qgemv_fp_reference(p.codes, p.scales, p.x, M, p.N, p.K, p.shape.fmt, rows=cols,
                                    residual=residual)
    absum = oracle.fp_abs_product_sum(p.codes, p.scales, p.x, M, p.N, p.K, p.shape.fmt, rows=cols)
    yy = y if cols is None else y[:, cols]
    rabs = None
    if residual is not None:
        rabs = residual[:M] if cols is None else residual[:M][:, cols]
    ok, worst, idx = oracle.check_close(yy, ref, absum, residual_abs=rabs)
    assert ok, f"{label}: worst |dy|/tol = {worst:.3g} at {idx}"


def paths_for(p, M=1):
    return [pt for pt in ("dot", "mfma", "auto")
            if q.qgemv_path_supported_fp(pt, M, p.N, p.K, p.shape.fmt)]


def bf16_bits_of(values: np.ndarray) -> np.ndarray:
    # exact: every decoded element is a bf16 value
    b = values.astype(np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)
    return (b >> 16).astype(np.uint16)


def same_elements(got_bits: np.ndarray, want: np.ndarray) -> bool:
    """Decoded bf16 patterns equal the oracle's values bit for bit, except that
    a zero may carry either sign (+0 and -0 give the same products)."""
    want_bits = bf16_bits_of(want)
    zero = want == 0
    return bool(np.array_equal(got_bits[~zero], want_bits[~zero]) and
                np.all((got_bits[zero] & 0x7FFF) == 0))


# ---------------------------------------------------------------- decoding: bit-exact

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K,N", [(256, 40), (1024, 17), (512, 5)])
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_unpack_probe_is_bit_exact(path, K, N, fmt):
    import torch
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=K + N), m_max=1)
    if not q.qgemv_path_supported_fp(path, 1, N, K, fmt):
        pytest.skip("path does not support this format")
    say(f"fp unpack probe {path} {fmt} K={K} N={N}")
    d = FpDevice(p)
    out = torch.full((N, K), 0x7FFF, dtype=torch.int16, device="cuda:0")
    q.qgemv_unpack_probe_fp(path, d.codes, out, N, K, fmt)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert same_elements(got, oracle.fp_elements(p.codes, K, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_every_byte_value_decodes_exactly(fmt):
    # all 256 byte values of the element encoding (FP8: the finite ones)
    import torch
    K, N = 256, 16
    bits = synth.FP_BITS[fmt]
    vals = np.arange(256, dtype=np.uint8)
    if bits == 8:
        vals = vals[(vals != 0x7F) & (vals != 0xFF)]
    codes = np.resize(vals, N * K * bits // 8).astype(np.uint8).reshape(N, K * bits // 8)
    d_codes = torch.from_numpy(codes).to("cuda:0")
    for path in ("dot", "mfma"):
        if not q.qgemv_path_supported_fp(path, 1, N, K, fmt):
            continue
        say(f"fp every byte {path} {fmt}")
        out = torch.zeros((N, K), dtype=torch.int16, device="cuda:0")
        q.qgemv_unpack_probe_fp(path, d_codes, out, N, K, fmt)
        torch.cuda.synchronize()
        assert same_elements(out.cpu().numpy().view(np.uint16), oracle.fp_elements(codes, K, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_unit_scale_onehot_gives_elements_exactly(fmt):
    K, N, M = 512, 48, 16
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=17), m_max=M)
    p.scales[:] = 0x38 if fmt == "nvfp4" else 127  # scale 1.0 (E4M3 / E8M0)
    p.x[:] = 0
    for m in range(M):
        p.x[m, synth.onehot_column(m, K)] = 0x3F80
    els = oracle.fp_elements(p.codes, K, fmt)
    d = FpDevice(p)
    for path in paths_for(p, M):
        say(f"fp onehot {path} {fmt}")
        y = d.run(M, path)
        for m in range(M):
            assert np.array_equal(y[m], els[:, synth.onehot_column(m, K)].astype(np.float32)), f"{path} row {m}"


@pytest.mark.parametrize("fmt", FMTS)
def test_every_scale_byte_decodes_exactly(fmt):
    # every E8M0 scale byte 0..254 (0x00 is 2^-127, an fp32 subnormal) and
    # every finite E4M3 scale byte (negative and subnormal included), through
    # the real kernels: row n's blocks all carry scale byte n, every element
    # is 1.0 and row m of x is one-hot, so y[m, n] is the decoded scale itself
    K, M = 256, 16
    vals = np.arange(255, dtype=np.uint8) if fmt.startswith("mx") else \
        np.array([v for v in range(256) if v not in (0x7F, 0xFF)], dtype=np.uint8)
    N = len(vals)
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=23), m_max=M)
    p.codes[:] = 0x22 if synth.FP_BITS[fmt] == 4 else 0x38  # E2M1 / E4M3 1.0
    p.scales[:] = vals[:, None]
    p.x[:] = 0
    for m in range(M):
        p.x[m, synth.onehot_column(m, K)] = 0x3F80
    want = (oracle.e8m0_to_f64(vals) if fmt.startswith("mx") else oracle.e4m3_to_f64(vals)).astype(np.float32)
    assert np.all(np.isfinite(want))
    d = FpDevice(p)
    for path in paths_for(p, M):
        for MM in (1, 2, 5, 16):
            say(f"fp every scale byte {path} {fmt} M={MM}")
            y = d.run(MM, path)
            for m in range(MM):
                # float equality: bit equality except that the product of a
                # -0 scale may be stored as +0
                assert np.array_equal(y[m], want), f"{path} M={MM} row {m}: scale bytes {vals[y[m] != want][:8]}"


# ---------------------------------------------------------------- every element

RAGGED = [(256, 512), (640, 40), (1024, 300), (2048, 97), (8192, 33), (128, 16), (3840, 200)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K,N", RAGGED)
def test_ragged_shapes_every_element(K, N, fmt):
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=3 * K + N, outliers=True), m_max=16)
    d = FpDevice(p)
    for path in paths_for(p):
        for M in (1, 2, 5, 8, 13, 16):
            say(f"fp ragged {path} {fmt} K={K} N={N} M={M}")
            check(p, d.run(M, path), M, label=f"{fmt} {path} K={K} N={N} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_many_tiles_every_element(fmt):
    K, N = 1024, 4500
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=41), m_max=16)
    d = FpDevice(p)
    for path in paths_for(p):
        for M in (1, 8, 16):
            say(f"fp many tiles {path} {fmt} M={M}")
            check(p, d.run(M, path), M, label=f"{fmt} {path} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_row_of_m_row_call_equals_single_row_call_bitwise(path, fmt):
    import torch
    K, N = 2048, 300
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=77), m_max=16)
    if not q.qgemv_path_supported_fp(path, 1, N, K, fmt):
        pytest.skip("path does not support this format")
    d = FpDevice(p)
    say(f"fp row invariance {path} {fmt}")
    singles = []
    for m in range(16):
        y1 = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        q.qgemv_run_path_fp(path, d.codes, d.scales, d.x[m:m + 1].clone(), None, y1, 1, N, K, fmt)
        singles.append(y1)
    torch.cuda.synchronize()
    singles = torch.cat(singles).cpu().numpy()
    for M in (2, 3, 4, 5, 6, 7, 8, 9, 16):
        assert np.array_equal(d.run(M, path), singles[:M]), f"M={M}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K,N", [(1024, 4500), (5120, 1024)])  # the second splits K on the MFMA path
def test_residual_sum_is_plain_plus_r_bitwise(fmt, K, N):
    import torch
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=91), m_max=16)
    d = FpDevice(p)
    r = synth.make_residual(16, N, seed=p.seed)
    for path in paths_for(p):
        for M in (1, 4, 16):
            say(f"fp residual {path} {fmt} M={M}")
            r_dev = torch.from_numpy(r[:M].copy()).to("cuda:0")
            y = d.run(M, path, residual=r_dev)
            check(p, y, M, residual=r, label=f"{fmt} {path} + r M={M}")
            plain = d.run(M, path)
            assert np.array_equal(y, (plain + r[:M]).astype(np.float32))
            yi = r_dev.clone()
            d.run(M, path, residual=yi, y=yi)  # in place (unsplit kernel where K would be split)
            yh = yi.cpu().numpy()
            check(p, yh, M, residual=r, label=f"{fmt} {path} in place M={M}")
            if K < 2048:
                assert np.array_equal(yh, y)


# ---------------------------------------------------------------- full size

FULL = [(n, s.m_values) for n, s in synth.WORKLOADS.items() if s.fmt is not None]


@pytest.mark.parametrize("name,ms", FULL)
def test_full_size_every_element(name, ms):
    import torch
    s = synth.WORKLOADS[name]
    p = synth.make_problem(s)
    d = FpDevice(p)
    orc = OracleRows.fp(p, max(ms))
    for path in paths_for(p):
        for M in ms:
            say(f"fp full {name} {path} M={M}")
            y = d.run(M, path)
            assert np.all(np.isfinite(y))
            orc.check(y, M, label=f"{name} {path} M={M}")
    say(f"fp full unpack {name}")
    for path in ("dot", "mfma"):
        if not q.qgemv_path_supported_fp(path, 1, s.N, s.K, s.fmt):
            continue
        out = torch.empty((s.N, s.K), dtype=torch.int16, device="cuda:0")
        q.qgemv_unpack_probe_fp(path, d.codes, out, s.N, s.K, s.fmt)
        torch.cuda.synchronize()
        assert same_elements(out.cpu().numpy().view(np.uint16), oracle.fp_elements(p.codes, s.K, s.fmt))
