"""Pins for the oracle's block-scaled FP formats (mxfp4, nvfp4, mxfp8), against
things other than the oracle itself:

* the element and scale encodings stated by the OCP Microscaling Formats v1.0
  specification (tests/golden/ocp_mx_elements.json);
* torch's own CPU decoders of float8_e4m3fn and float8_e8m0fnu for every byte;
* exact rational brute force on tiny shapes, with bit-level decoders written
  here independently of the oracle's;
* closed forms (one-hot activations select one scaled element);
* planted mistakes that must fail at least one pin.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import qgemv_oracle as qo
from few_row_quantized_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_mx_elements.json")
FMTS = ["mxfp4", "nvfp4", "mxfp8"]


def golden():
    return json.load(open(GOLDEN))


# ---------------------------------------------------------------- independent decoders (exact)

def frac_e2m1(v: int) -> Fraction:
    # table lookup of the magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    return -mags[v & 7] if v & 8 else mags[v & 7]


def frac_e4m3(v: int) -> Fraction:
    sign = -1 if v & 0x80 else 1
    e, m = (v >> 3) & 0xF, v & 7
    assert not (e == 15 and m == 7)
    if e == 0:
        return sign * Fraction(m, 8 * 64)
    return sign * Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def frac_e8m0(v: int) -> Fraction:
    assert v != 255
    return Fraction(2) ** (v - 127)


def frac_bf16(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** -133
    return sign * Fraction(128 + f) * Fraction(2) ** (e - 134)


def exact_fp_y(p, M):
    fmt, K, N = p.shape.fmt, p.K, p.N
    bits, block = synth.FP_BITS[fmt], synth.FP_BLOCK[fmt]
    xs = [[frac_bf16(int(v)) for v in p.x[m]] for m in range(M)]
    y = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        big = int.from_bytes(bytes(p.codes[n].tolist()), "little")
        els = [(big >> (bits * k)) & ((1 << bits) - 1) for k in range(K)]
        dec = frac_e2m1 if bits == 4 else frac_e4m3
        sdec = frac_e8m0 if fmt.startswith("mx") else frac_e4m3
        w = [sdec(int(p.scales[n, k // block])) * dec(els[k]) for k in range(K)]
        for m in range(M):
            y[m][n] = sum(xs[m][k] * w[k] for k in range(K))
    return y


def run(p, M, rows=None):
    return oracle.qgemv_fp_reference(p.codes, p.scales, p.x, M, p.N, p.K, p.shape.fmt, rows=rows)


# ---------------------------------------------------------------- encodings

def test_e2m1_matches_the_specification_table():
    vals = golden()["e2m1"]["values"]
    got = oracle.e2m1_to_f64(np.arange(16))
    assert got.tolist() == vals
    assert np.array_equal(np.signbit(got), np.signbit(np.array(vals)))


def test_e4m3_matches_the_specification_points():
    g = golden()["e4m3"]
    for code, val in g["points"]:
        assert oracle.e4m3_to_f64(np.array([int(code, 16)]))[0] == val, code
    for code in g["nan"]:
        assert np.isnan(oracle.e4m3_to_f64(np.array([int(code, 16)]))[0])


def test_e8m0_matches_the_specification_points():
    g = golden()["e8m0"]
    for code, val in g["points"]:
        assert oracle.e8m0_to_f64(np.array([int(code, 16)]))[0] == val, code
    assert np.isnan(oracle.e8m0_to_f64(np.array([255]))[0])


def test_e4m3_matches_torch_for_every_byte():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_f64(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e8m0_matches_torch_for_every_byte():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_to_f64(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_elements_are_unpacked_like_the_affine_codes():
    # two FP4 elements per byte, low nibble first; one FP8 element per byte
    codes = np.array([[0x21, 0xF7]], np.uint8)
    assert oracle.fp_elements(codes, 4, "mxfp4").tolist() == [[0.5, 1.0, 6.0, -6.0]]
    assert oracle.fp_elements(codes, 2, "mxfp8").tolist() == [[frac_e4m3(0x21), frac_e4m3(0xF7)]]


# ---------------------------------------------------------------- closed forms and brute force

@pytest.mark.parametrize("fmt", FMTS)
def test_onehot_x_selects_one_scaled_element(fmt):
    K, N = 128, 12
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=31), m_max=1)
    bits, block = synth.FP_BITS[fmt], synth.FP_BLOCK[fmt]
    for k in (0, block - 1, block, K - 1):
        p.x[:] = 0
        p.x[0, k] = 0x3F80
        y = run(p, 1)
        for n in range(N):
            big = int.from_bytes(bytes(p.codes[n].tolist()), "little")
            el = (big >> (bits * k)) & ((1 << bits) - 1)
            dec = frac_e2m1 if bits == 4 else frac_e4m3
            sdec = frac_e8m0 if fmt.startswith("mx") else frac_e4m3
            assert y[0, n] == float(sdec(int(p.scales[n, k // block])) * dec(el))


@pytest.mark.parametrize("fmt,K,N,M", [("mxfp4", 64, 5, 2), ("nvfp4", 64, 4, 3), ("mxfp8", 96, 4, 2)])
def test_matches_exact_rational_brute_force(fmt, K, N, M):
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=300 + K + N), m_max=M)
    y = run(p, M)
    ex = exact_fp_y(p, M)
    absum = oracle.fp_abs_product_sum(p.codes, p.scales, p.x, M, N, K, fmt)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= Fraction(K) * Fraction(2) ** -52 * Fraction(absum[m, n])


def test_residual_is_added_in_the_output_layout():
    p = synth.make_problem(synth.custom_fp_shape(64, 6, "mxfp4", seed=5), m_max=2)
    p.x[:] = 0
    r = (np.arange(12, dtype=np.float32).reshape(2, 6) - 5) * np.float32(0.5)
    y = oracle.qgemv_fp_reference(p.codes, p.scales, p.x, 2, 6, 64, "mxfp4", residual=r)
    assert y.tolist() == r.astype(np.float64).tolist()


def test_sampled_rows_match_full_result():
    p = synth.make_problem(synth.custom_fp_shape(256, 40, "nvfp4", seed=9), m_max=3)
    y = run(p, 3)
    rows = [0, 17, 39]
    assert np.array_equal(run(p, 3, rows=rows), y[:, rows])


# ---------------------------------------------------------------- planted mistakes

def _pins():
    try:
        test_e2m1_matches_the_specification_table()
        test_e4m3_matches_torch_for_every_byte()
        test_e8m0_matches_torch_for_every_byte()
        test_elements_are_unpacked_like_the_affine_codes()
        for fmt in FMTS:
            test_onehot_x_selects_one_scaled_element(fmt)
        test_matches_exact_rational_brute_force("nvfp4", 64, 4, 3)
    except AssertionError:
        return False
    return True


def _e2m1_bias2(v):
    # exponent bias 2 instead of 1
    return qo._orig_e2m1(v) / np.where((np.asarray(v) >> 1) & 3, 2.0, 1.0)


def _e4m3_bias8(v):
    # the bias of the other common E4M3 variant
    return qo._orig_e4m3(v) / 2.0


def _e8m0_bias128(v):
    return qo._orig_e8m0(v) / 2.0


def _nvfp4_block32(codes, scales, K, fmt):
    el = qo.fp_elements(codes, K, fmt)
    s = qo.fp_scales(scales, fmt)
    blk = 32 if fmt == "nvfp4" else qo.FP_FORMATS[fmt][1]
    return s[:, np.minimum(np.arange(K) // blk, s.shape[1] - 1)] * el


def _high_nibble_first(codes, K, fmt):
    bits = qo.FP_FORMATS[fmt][0]
    q = qo.unpack_codes(codes, K, bits)
    if bits == 4:
        q = q.reshape(q.shape[0], -1, 2)[:, :, ::-1].reshape(q.shape[0], K)
    return qo.e2m1_to_f64(q) if bits == 4 else qo.e4m3_to_f64(q)


@pytest.mark.parametrize("target,mutant", [
    ("e2m1_to_f64", _e2m1_bias2), ("e4m3_to_f64", _e4m3_bias8), ("e8m0_to_f64", _e8m0_bias128),
    ("fp_dequantize", _nvfp4_block32), ("fp_elements", _high_nibble_first),
])
def test_pins_catch_planted_mistakes(monkeypatch, target, mutant):
    assert _pins(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(qo, "_orig_e2m1", qo.e2m1_to_f64, raising=False)
    monkeypatch.setattr(qo, "_orig_e4m3", qo.e4m3_to_f64, raising=False)
    monkeypatch.setattr(qo, "_orig_e8m0", qo.e8m0_to_f64, raising=False)
    monkeypatch.setattr(qo, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert not _pins(), f"planted mistake in {target} went unnoticed"


def test_generator_fp_distributions():
    s = synth.WORKLOADS["square_k4096_n4096_mxfp8"]
    p = synth.make_problem(s, m_max=1)
    assert p.codes.shape == (4096, 4096) and p.scales.shape == (4096, 128)
    assert not np.isin(p.codes, [0x7F, 0xFF]).any()  # no NaN elements
    assert p.scales.min() >= 110 and p.scales.max() <= 115
    s4 = synth.WORKLOADS["square_k4096_n4096_nvfp4"]
    p4 = synth.make_problem(s4, m_max=1)
    assert p4.scales.shape == (4096, 256)
    assert np.all(np.isfinite(oracle.e4m3_to_f64(p4.scales))) and (p4.scales < 0x80).all()


# ---------------------------------------------------------------- the tolerance scale
#
# fp_abs_product_sum sets the bound of every FP-format parity check, so it is
# pinned on its own: exact rational brute force with this file's decoders,
# closed forms (a one-hot row gives |w| of one column; flipping the sign of x
# changes nothing; with x >= 0 and w >= 0 it equals y), and planted mistakes.

def exact_fp_abs(p, M):
    fmt, K, N = p.shape.fmt, p.K, p.N
    bits, block = synth.FP_BITS[fmt], synth.FP_BLOCK[fmt]
    xs = [[frac_bf16(int(v)) for v in p.x[m]] for m in range(M)]
    out = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        big = int.from_bytes(bytes(p.codes[n].tolist()), "little")
        els = [(big >> (bits * k)) & ((1 << bits) - 1) for k in range(K)]
        dec = frac_e2m1 if bits == 4 else frac_e4m3
        sdec = frac_e8m0 if fmt.startswith("mx") else frac_e4m3
        w = [sdec(int(p.scales[n, k // block])) * dec(els[k]) for k in range(K)]
        for m in range(M):
            out[m][n] = sum(abs(xs[m][k] * w[k]) for k in range(K))
    return out


def abs_sum(p, M, rows=None):
    return oracle.fp_abs_product_sum(p.codes, p.scales, p.x, M, p.N, p.K, p.shape.fmt, rows=rows)


@pytest.mark.parametrize("fmt,K,N,M", [("mxfp4", 64, 5, 2), ("nvfp4", 64, 4, 3), ("mxfp8", 96, 4, 2)])
def test_abs_product_sum_matches_exact_rational(fmt, K, N, M):
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=400 + K + N), m_max=M)
    got = abs_sum(p, M)
    want = exact_fp_abs(p, M)
    for m in range(M):
        for n in range(N):
            assert want[m][n] > 0
            assert abs(Fraction(got[m, n]) - want[m][n]) <= Fraction(K) * Fraction(2) ** -52 * want[m][n]


@pytest.mark.parametrize("fmt", FMTS)
def test_abs_product_sum_onehot_gives_magnitude_of_one_weight(fmt):
    K, N = 64, 5
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=41), m_max=2)
    bits, block = synth.FP_BITS[fmt], synth.FP_BLOCK[fmt]
    k = 37  # second nvfp4 block of the first 32, second half of an mx block
    p.x[:] = 0
    p.x[0, k] = 0xC000  # -2.0: the sign of x must not matter
    p.x[1, k] = 0x3F80  # 1.0
    got = abs_sum(p, 2)
    for n in range(N):
        big = int.from_bytes(bytes(p.codes[n].tolist()), "little")
        el = (big >> (bits * k)) & ((1 << bits) - 1)
        dec = frac_e2m1 if bits == 4 else frac_e4m3
        sdec = frac_e8m0 if fmt.startswith("mx") else frac_e4m3
        w = abs(sdec(int(p.scales[n, k // block])) * dec(el))
        assert got[0, n] == float(2 * w) and got[1, n] == float(w), (fmt, n)


@pytest.mark.parametrize("fmt", FMTS)
def test_abs_product_sum_sign_and_same_sign_closed_forms(fmt):
    K, N = 128, 6
    p = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=43), m_max=2)
    base = abs_sum(p, 2)
    # flipping the sign bit of every activation leaves every |x*w| unchanged
    q = synth.make_problem(synth.custom_fp_shape(K, N, fmt, seed=43), m_max=2)
    q.x ^= np.uint16(0x8000)
    assert np.array_equal(abs_sum(q, 2), base)
    # non-negative x and non-negative weights: the sum of |x*w| is y itself
    bits = synth.FP_BITS[fmt]
    if bits == 4:
        q.codes &= np.uint8(0x77)  # clear both nibbles' sign bits
    else:
        q.codes &= np.uint8(0x7F)
        q.codes[q.codes == 0x7F] = 0x7E  # keep clear of the NaN pattern
    q.x &= np.uint16(0x7FFF)
    y = oracle.qgemv_fp_reference(q.codes, q.scales, q.x, 2, N, K, fmt)
    a = abs_sum(q, 2)
    assert np.allclose(a, y, rtol=K * 2.0 ** -52, atol=0)
    # and never below |y| (triangle inequality) on signed data
    ys = oracle.qgemv_fp_reference(p.codes, p.scales, p.x, 2, N, K, fmt)
    assert np.all(base >= np.abs(ys) * (1 - K * 2.0 ** -52))


def _abs_pins():
    try:
        for fmt, K, N, M in [("mxfp4", 64, 5, 2), ("nvfp4", 64, 4, 3), ("mxfp8", 96, 4, 2)]:
            test_abs_product_sum_matches_exact_rational(fmt, K, N, M)
        for fmt in FMTS:
            test_abs_product_sum_onehot_gives_magnitude_of_one_weight(fmt)
            test_abs_product_sum_sign_and_same_sign_closed_forms(fmt)
    except AssertionError:
        return False
    return True


def _abs_inflated(codes, scales, x_bits, M, N, K, fmt, rows=None):
    return 2.0 * qo._orig_fp_abs(codes, scales, x_bits, M, N, K, fmt, rows)


def _abs_dropped_on_w(codes, scales, x_bits, M, N, K, fmt, rows=None):
    # |x| @ w^T: the magnitude taken of the activations only
    x = np.abs(qo.bf16_bits_to_f64(np.asarray(x_bits)[:M]))
    idx = np.arange(N) if rows is None else np.asarray(rows)
    return x @ qo.fp_dequantize(codes[idx], scales[idx], K, fmt).T


def _abs_nvfp4_block32(codes, scales, x_bits, M, N, K, fmt, rows=None):
    x = np.abs(qo.bf16_bits_to_f64(np.asarray(x_bits)[:M]))
    idx = np.arange(N) if rows is None else np.asarray(rows)
    return x @ np.abs(_nvfp4_block32(codes[idx], scales[idx], K, fmt)).T


def _abs_x_row0(codes, scales, x_bits, M, N, K, fmt, rows=None):
    xb = np.repeat(np.asarray(x_bits)[:1], M, axis=0)
    return qo._orig_fp_abs(codes, scales, xb, M, N, K, fmt, rows)


@pytest.mark.parametrize("mutant", [_abs_inflated, _abs_dropped_on_w, _abs_nvfp4_block32, _abs_x_row0])
def test_abs_pins_catch_planted_mistakes(monkeypatch, mutant):
    assert _abs_pins(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(qo, "_orig_fp_abs", qo.fp_abs_product_sum, raising=False)
    monkeypatch.setattr(qo, "fp_abs_product_sum", mutant)
    monkeypatch.setattr(oracle, "fp_abs_product_sum", mutant)
    assert not _abs_pins(), f"planted mistake {mutant.__name__} went unnoticed"
