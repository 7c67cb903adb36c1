"""Pins for the fp64 oracle, checked against things other than the oracle itself.

The pages print no worked value of y, so the oracle is pinned by:
* closed forms of the storage format (nibble/crumb order, fp16/bf16 decoding
  of textbook bit patterns);
* closed forms of the product (all-zero codes; one-hot activations);
* invariants (row independence of the M-row result; linearity in x);
* exact rational brute force on tiny shapes (fractions.Fraction, with its own
  bit-level decoders and its own bit-stream unpacking);
* planted mistakes: mutated copies of the oracle must fail at least one pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import qgemv_oracle as qo
from few_row_quantized_amd import accounting, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- independent decoders

def frac_fp16(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    assert e != 0x1F, "inf/nan not expected"
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f) * Fraction(2) ** (e - 25)


def frac_bf16(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f) * Fraction(2) ** -133
    return sign * Fraction(128 + f) * Fraction(2) ** (e - 134)


def bitstream_codes(row_bytes: np.ndarray, K: int, bits: int):
    """Codes read as consecutive `bits`-wide fields of a little-endian bit stream."""
    big = int.from_bytes(bytes(row_bytes.tolist()), "little")
    mask = (1 << bits) - 1
    return [(big >> (bits * k)) & mask for k in range(K)]


def independent_pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [N, K] little-endian into bytes (test-local packer)."""
    N, K = q.shape
    out = np.zeros((N, K * bits // 8), np.uint8)
    for n in range(N):
        acc = 0
        for k in range(K):
            acc |= int(q[n, k]) << (bits * k)
        out[n] = np.frombuffer(acc.to_bytes(K * bits // 8, "little"), np.uint8)
    return out


def exact_y(p: synth.Problem, M: int):
    """Exact rational y[m][n] for a tiny problem, from the definition."""
    K, N, gs, bits = p.K, p.N, p.group_size, p.bits
    xs = [[frac_bf16(int(v)) for v in p.x[m]] for m in range(M)]
    y = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        q = bitstream_codes(p.codes[n], K, bits)
        w = [frac_fp16(int(p.scales[n, k // gs])) * q[k] + frac_fp16(int(p.biases[n, k // gs]))
             for k in range(K)]
        for m in range(M):
            y[m][n] = sum(xs[m][k] * w[k] for k in range(K))
    return y


def run_oracle(p: synth.Problem, M: int, rows=None):
    return oracle.qgemv_reference(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits,
                                  p.group_size, rows=rows)


# ---------------------------------------------------------------- storage format

def test_unpack_4bit_closed_form_bytes():
    codes = np.array([[0x21, 0xF0, 0x0F, 0xA5]], np.uint8)
    q = oracle.unpack_codes(codes, 8, 4)
    assert q.tolist() == [[1, 2, 0, 15, 15, 0, 5, 10]]


def test_unpack_2bit_closed_form_bytes():
    codes = np.array([[0xE4, 0x1B]], np.uint8)
    q = oracle.unpack_codes(codes, 8, 2)
    assert q.tolist() == [[0, 1, 2, 3, 3, 2, 1, 0]]


def test_unpack_8bit_closed_form_bytes():
    # one code per byte, the byte itself (unsigned)
    codes = np.array([[0x00, 0xFF, 0x80, 0x7F, 0x21]], np.uint8)
    q = oracle.unpack_codes(codes, 5 * 8 // 8, 8)
    assert q.tolist() == [[0, 255, 128, 127, 33]]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_unpack_matches_bitstream_and_packer(bits):
    rng = np.random.default_rng(3)
    K, N = 128, 5
    q = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    packed = independent_pack(q, bits)
    assert np.array_equal(oracle.unpack_codes(packed, K, bits), q)
    for n in range(N):
        assert bitstream_codes(packed[n], K, bits) == q[n].tolist()


def test_fp16_decode_textbook_values():
    pats = np.array([0x3C00, 0xC000, 0x7BFF, 0x0001, 0x0400, 0x3555, 0x8000], np.uint16)
    want = [1.0, -2.0, 65504.0, 2.0 ** -24, 2.0 ** -14, 0.333251953125, -0.0]
    got = oracle.fp16_bits_to_f64(pats)
    assert got.tolist() == want
    for p, w in zip(pats.tolist(), want):
        assert float(frac_fp16(p)) == w


def test_bf16_decode_textbook_values():
    pats = np.array([0x3F80, 0xC0A0, 0x0001, 0x7F7F, 0x3EAB, 0x4300], np.uint16)
    want = [1.0, -5.0, 2.0 ** -133, 3.3895313892515355e38, 0.333984375, 128.0]
    got = oracle.bf16_bits_to_f64(pats)
    assert got.tolist() == want
    for p, w in zip(pats.tolist(), want):
        assert float(frac_bf16(p)) == w


def test_dequant_special_cases():
    q = np.array([[0, 1, 15, 7]], np.uint8)
    one = np.float16(1.0).view(np.uint16)
    zero = np.float16(0.0).view(np.uint16)
    s = np.array([[one, one]], np.uint16)
    b = np.array([[zero, zero]], np.uint16)
    assert oracle.dequantize(q, s, b, 2).tolist() == [[0.0, 1.0, 15.0, 7.0]]
    s2 = np.array([[np.float16(0.5).view(np.uint16), np.float16(0.25).view(np.uint16)]], np.uint16)
    b2 = np.array([[np.float16(-3.0).view(np.uint16), np.float16(2.0).view(np.uint16)]], np.uint16)
    assert oracle.dequantize(q, s2, b2, 2).tolist() == [[-3.0, -2.5, 5.75, 3.75]]
    assert oracle.dequantize(np.zeros_like(q), s2, b2, 2).tolist() == [[-3.0, -3.0, 2.0, 2.0]]


# ---------------------------------------------------------------- closed forms of y

@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 32), (2, 64), (2, 128), (8, 64)])
def test_zero_codes_gives_bias_times_group_sums(bits, gs):
    K, N, M = 256, 24, 3
    p = synth.special_problem(K, N, bits, gs, M, "zero_codes")
    y = run_oracle(p, M)
    # y[m,n] = sum_g b[n,g] * (sum over group g of x[m,k]) -- computed with
    # python floats from the textbook decoders, group by group.
    for m in range(M):
        xrow = [float(frac_bf16(int(v))) for v in p.x[m]]
        gsum = [math.fsum(xrow[g * gs:(g + 1) * gs]) for g in range(K // gs)]
        for n in range(N):
            want = math.fsum(float(frac_fp16(int(p.biases[n, g]))) * gsum[g] for g in range(K // gs))
            assert abs(y[m, n] - want) <= 1e-12 * (1 + abs(want))


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 128), (2, 32), (2, 64), (8, 32), (8, 128)])
def test_onehot_x_selects_one_dequantized_column(bits, gs):
    K, N = 256, 16
    shape = synth.custom_shape(K, N, bits, gs, seed=11)
    p = synth.make_problem(shape, m_max=1)
    cols = [0, gs - 1, gs, K // 2 + 1, K - 1]
    for k in cols:
        p.x[:] = 0
        p.x[0, k] = 0x3F80  # bf16 1.0
        y = run_oracle(p, 1)
        for n in range(N):
            qk = bitstream_codes(p.codes[n], K, bits)[k]
            want = frac_fp16(int(p.scales[n, k // gs])) * qk + frac_fp16(int(p.biases[n, k // gs]))
            assert y[0, n] == float(want)


def test_unit_scale_onehot_gives_codes():
    p = synth.special_problem(256, 32, 4, 64, 4, "unit_scale_onehot")
    y = run_oracle(p, 4)
    for m in range(4):
        k = synth.onehot_column(m, 256)
        want = [bitstream_codes(p.codes[n], 256, 4)[k] for n in range(32)]
        assert y[m].tolist() == [float(v) for v in want]


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("name", ["tiny_k256_n512_4b_g64"])
def test_row_of_m_row_result_equals_single_row_result(name):
    p = synth.make_problem(synth.WORKLOADS[name])
    M = max(p.shape.m_values)
    y = run_oracle(p, M)
    scale = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits, p.group_size)
    for m in range(M):
        sub = synth.Problem(p.shape, p.codes, p.scales, p.biases, p.x[m:m + 1].copy(), None, p.seed)
        y1 = run_oracle(sub, 1)
        assert np.all(np.abs(y1[0] - y[m]) <= 1e-12 * scale[m] + 1e-300)


def test_linearity_in_x():
    K, N = 256, 40
    p = synth.make_problem(synth.custom_shape(K, N, 4, 64, seed=5), m_max=2)
    # x1 on even columns, x2 on odd columns; alpha, beta powers of two keep
    # alpha*x1 + beta*x2 exactly representable in bf16.
    x1 = p.x[0].copy()
    x1[1::2] = 0
    x2 = p.x[1].copy()
    x2[0::2] = 0
    alpha, beta = 2.0, -0.5
    x1f = oracle.bf16_bits_to_f64(x1)
    x2f = oracle.bf16_bits_to_f64(x2)
    comb = synth.f32_to_bf16_bits((alpha * x1f + beta * x2f).astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(comb), alpha * x1f + beta * x2f)
    X = np.stack([x1, x2, comb])
    q = synth.Problem(p.shape, p.codes, p.scales, p.biases, X, None, p.seed)
    y = run_oracle(q, 3)
    scale = oracle.abs_product_sum(p.codes, p.scales, p.biases, X, 3, N, K, 4, 64)
    assert np.all(np.abs(y[2] - (alpha * y[0] + beta * y[1])) <= 1e-12 * (scale[2] + scale[0] + scale[1]))


def test_sampled_rows_match_full_result():
    p = synth.make_problem(synth.WORKLOADS["tiny_k256_n512_4b_g64"])
    y = run_oracle(p, 4)
    rows = [0, 7, 300, 511]
    assert np.array_equal(run_oracle(p, 4, rows=rows), y[:, rows])


# ---------------------------------------------------------------- exact brute force

@pytest.mark.parametrize("bits,gs,K,N,M", [
    (4, 32, 64, 5, 2), (4, 64, 192, 7, 3), (4, 128, 256, 4, 2),
    (2, 32, 128, 6, 3), (2, 64, 256, 5, 2), (2, 128, 128, 3, 1),
    (8, 32, 64, 5, 3), (8, 64, 192, 4, 2), (8, 128, 256, 3, 2),
])
def test_matches_exact_rational_brute_force(bits, gs, K, N, M):
    shape = synth.custom_shape(K, N, bits, gs, seed=100 + K + N + bits)
    p = synth.make_problem(shape, m_max=M)
    y = run_oracle(p, M)
    ex = exact_y(p, M)
    absum = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, N, K, bits, gs)
    for m in range(M):
        for n in range(N):
            # fp64 summation of exact products: |err| <= K * 2^-53 * sum|x w|
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= Fraction(K) * Fraction(2) ** -52 * Fraction(absum[m, n])


def test_tolerance_hand_value():
    # x = [1, -2], w = [0.5, 0.25]: sum |x w| = 0.5 + 0.5 = 1.0
    assert oracle.tolerance(np.array([1.0]))[0] == pytest.approx(1e-3 + 1e-6, rel=0, abs=1e-18)
    ok, worst, _ = oracle.check_close(np.array([1.0 + 0.9e-3]), np.array([1.0]), np.array([1.0]))
    assert ok and worst < 1
    ok, _, _ = oracle.check_close(np.array([1.0 + 1.2e-3]), np.array([1.0]), np.array([1.0]))
    assert not ok
    ok, _, _ = oracle.check_close(np.array([np.nan]), np.array([1.0]), np.array([1.0]))
    assert not ok


# ---------------------------------------------------------------- planted mistakes

def _pin_suite():
    """A compact run of the pins above; returns True when all pass."""
    try:
        test_unpack_4bit_closed_form_bytes()
        test_unpack_2bit_closed_form_bytes()
        test_zero_codes_gives_bias_times_group_sums(4, 64)
        test_onehot_x_selects_one_dequantized_column(4, 64)
        test_onehot_x_selects_one_dequantized_column(2, 32)
        test_matches_exact_rational_brute_force(4, 64, 192, 7, 3)
        test_matches_exact_rational_brute_force(2, 64, 256, 5, 2)
        test_unpack_8bit_closed_form_bytes()
        test_onehot_x_selects_one_dequantized_column(8, 32)
        test_matches_exact_rational_brute_force(8, 64, 192, 4, 2)
    except AssertionError:
        return False
    return True


def _mutant_high_nibble_first(codes, K, bits):
    q = qo._orig_unpack(codes, K, bits)
    if bits == 4:
        q = q.reshape(q.shape[0], -1, 2)[:, :, ::-1].reshape(q.shape[0], K)
    else:
        q = q.reshape(q.shape[0], -1, 4)[:, :, ::-1].reshape(q.shape[0], K)
    return q


def _mutant_signed_bytes(codes, K, bits):
    # 8-bit codes read as two's-complement int8 (q - 256 for q >= 128)
    q = qo._orig_unpack(codes, K, bits).astype(np.int16)
    if bits == 8:
        q = np.where(q >= 128, q - 256, q)
    return q


def _mutant_dropped_bias(q, scales, biases, gs):
    return qo._orig_dequant(q, scales, np.zeros_like(biases), gs)


def _mutant_bias_sign(q, scales, biases, gs):
    return qo._orig_dequant(q, scales, biases ^ np.uint16(0x8000), gs)


def _mutant_group_index(q, scales, biases, gs):
    s = oracle.fp16_bits_to_f64(scales)
    b = oracle.fp16_bits_to_f64(biases)
    K = q.shape[1]
    g = np.minimum((np.arange(K) + 1) // gs, K // gs - 1)
    return s[:, g] * q + b[:, g]


def _mutant_scale_bias_swapped(q, scales, biases, gs):
    return qo._orig_dequant(q, biases, scales, gs)


@pytest.mark.parametrize("target,mutant", [
    ("unpack_codes", _mutant_high_nibble_first),
    ("unpack_codes", _mutant_signed_bytes),
    ("dequantize", _mutant_dropped_bias),
    ("dequantize", _mutant_bias_sign),
    ("dequantize", _mutant_group_index),
    ("dequantize", _mutant_scale_bias_swapped),
])
def test_pins_catch_planted_mistakes(monkeypatch, target, mutant):
    assert _pin_suite(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(qo, "_orig_unpack", qo.unpack_codes, raising=False)
    monkeypatch.setattr(qo, "_orig_dequant", qo.dequantize, raising=False)
    monkeypatch.setattr(qo, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert not _pin_suite(), f"planted mistake in {target} went unnoticed"


def test_pins_catch_transposed_product(monkeypatch):
    orig = qo.qgemv_reference

    def transposed(codes, scales, biases, x_bits, M, N, K, bits, gs, rows=None):
        y = orig(codes, scales, biases, x_bits, M, N, K, bits, gs, rows=rows)
        return y[:, ::-1].copy()  # columns permuted: output rows attached to the wrong n

    monkeypatch.setattr(qo, "qgemv_reference", transposed)
    monkeypatch.setattr(oracle, "qgemv_reference", transposed)
    assert not _pin_suite()


# ---------------------------------------------------------------- fused residual sum

def run_add(p: synth.Problem, M: int, r, rows=None):
    return oracle.qgemv_add_reference(p.codes, p.scales, p.biases, p.x, r, M, p.N, p.K, p.bits,
                                      p.group_size, rows=rows)


def distinct_residual(M: int, N: int) -> np.ndarray:
    """Every element different and exactly representable: r[m, n] = (N*m + n)/4 - 3."""
    return (np.arange(M * N, dtype=np.float32).reshape(M, N) * np.float32(0.25) - np.float32(3.0))


def test_add_zero_activations_gives_the_residual():
    # x = 0: every product vanishes and y[m, n] is r[m, n] itself, in the
    # output's [M, N] layout
    K, N, M = 256, 24, 3
    p = synth.make_problem(synth.custom_shape(K, N, 4, 64, seed=21), m_max=M)
    p.x[:] = 0
    r = distinct_residual(M, N)
    y = run_add(p, M, r)
    assert y.tolist() == [[(N * m + n) / 4 - 3 for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("bits,gs", [(4, 64), (2, 32)])
def test_add_onehot_x_gives_dequantized_weight_plus_residual(bits, gs):
    K, N, M = 256, 16, 2
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=23), m_max=M)
    r = distinct_residual(M, N)
    ks = [gs - 1, K - 1]
    p.x[:] = 0
    for m, k in enumerate(ks):
        p.x[m, k] = 0x3F80  # bf16 1.0
    y = run_add(p, M, r)
    for m, k in enumerate(ks):
        for n in range(N):
            qk = bitstream_codes(p.codes[n], K, bits)[k]
            want = (frac_fp16(int(p.scales[n, k // gs])) * qk + frac_fp16(int(p.biases[n, k // gs]))
                    + Fraction(float(r[m, n])))
            assert y[m, n] == float(want)


@pytest.mark.parametrize("bits,gs,K,N,M", [(4, 64, 192, 7, 3), (2, 128, 256, 5, 2)])
def test_add_matches_exact_rational_brute_force(bits, gs, K, N, M):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=200 + K + N), m_max=M)
    r = synth.make_residual(M, N, seed=p.seed)
    y = run_add(p, M, r)
    ex = exact_y(p, M)
    absum = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, N, K, bits, gs)
    for m in range(M):
        for n in range(N):
            want = ex[m][n] + Fraction(float(r[m, n]))
            bound = Fraction(K + 1) * Fraction(2) ** -52 * (Fraction(absum[m, n]) + abs(Fraction(float(r[m, n]))))
            assert abs(Fraction(y[m, n]) - want) <= bound


def test_add_sampled_rows_match_full_result():
    p = synth.make_problem(synth.WORKLOADS["tiny_k256_n512_4b_g64"])
    r = synth.make_residual(4, p.N, seed=p.seed)
    y = run_add(p, 4, r)
    rows = [0, 7, 300, 511]
    assert np.array_equal(run_add(p, 4, r, rows=rows), y[:, rows])


def test_add_tolerance_hand_value():
    # sum |x w| = 1, |r| = 3: 1e-3 + 1e-6 + 2^-23 * (3 + 1)
    tol = oracle.tolerance(np.array([1.0]), residual_abs=np.array([-3.0]))[0]
    assert tol == 1e-3 + 1e-6 + 4.0 * 2.0 ** -23
    ok, _, _ = oracle.check_close(np.array([4.0 + 1.0005e-3]), np.array([4.0]), np.array([1.0]),
                                  residual_abs=np.array([3.0]))
    assert ok
    ok, _, _ = oracle.check_close(np.array([4.0 + 1.01e-3]), np.array([4.0]), np.array([1.0]),
                                  residual_abs=np.array([3.0]))
    assert not ok


def _add_pin_suite():
    try:
        test_add_zero_activations_gives_the_residual()
        test_add_onehot_x_gives_dequantized_weight_plus_residual(4, 64)
        test_add_matches_exact_rational_brute_force(4, 64, 192, 7, 3)
    except (AssertionError, ValueError):
        return False
    return True


def _res_negated(residual, M, N, rows=None):
    return -qo._orig_residual(residual, M, N, rows)


def _res_transposed(residual, M, N, rows=None):
    # the [M, N] buffer read as if it were [N, M]
    r = np.asarray(residual, dtype=np.float32)[:M].reshape(N, M).T.astype(np.float64)
    return r if rows is None else r[:, rows]


def _res_row0_broadcast(residual, M, N, rows=None):
    r = qo._orig_residual(residual, M, N, rows)
    return np.broadcast_to(r[:1], r.shape).copy()


def _res_dropped(residual, M, N, rows=None):
    return np.zeros_like(qo._orig_residual(residual, M, N, rows))


@pytest.mark.parametrize("mutant", [_res_negated, _res_transposed, _res_row0_broadcast, _res_dropped])
def test_add_pins_catch_planted_mistakes(monkeypatch, mutant):
    assert _add_pin_suite(), "pins must pass on the unmodified oracle"
    monkeypatch.setattr(qo, "_orig_residual", qo.residual_f64, raising=False)
    monkeypatch.setattr(qo, "residual_f64", mutant)
    assert not _add_pin_suite(), f"planted mistake {mutant.__name__} went unnoticed"


# ---------------------------------------------------------------- byte model (pages' printed values)

def test_byte_model_matches_pages_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "byte_model.json")))
    for gs, ent in g["metadata_share_4bit"].items():
        assert abs(accounting.metadata_share(4, int(gs)) - ent["printed"]) <= ent["abs_tol"]
    r = accounting.metadata_share(4, 32) / accounting.metadata_share(4, 128)
    assert abs(r - g["g32_over_g128_metadata"]["printed"]) <= g["g32_over_g128_metadata"]["abs_tol"]
    c = g["roofline_case"]
    w = accounting.weight_bytes(c["N"], c["K"], c["bits"], c["group_size"])
    assert w == 50_135_040
    ms = w / (c["bandwidth_GB_per_s"] * 1e9) * 1e3
    assert abs(ms - c["printed_ms"]) <= c["abs_tol_ms"]
    # the printed figure is the weight stream alone: adding x and an fp32 y at M=7 misses it
    ms_total = accounting.algorithmic_bytes(7, c["N"], c["K"], c["bits"], c["group_size"]) / (c["bandwidth_GB_per_s"] * 1e9) * 1e3
    assert abs(ms_total - c["printed_ms"]) > c["abs_tol_ms"]


# ---------------------------------------------------------------- generator

def test_generator_is_deterministic_and_shaped():
    s = synth.WORKLOADS["square_k4096_n4096_4b_g64"]
    a = synth.make_problem(s)
    b = synth.make_problem(s)
    assert np.array_equal(a.codes, b.codes) and np.array_equal(a.x, b.x)
    assert np.array_equal(a.scales, b.scales) and np.array_equal(a.biases, b.biases)
    assert a.codes.shape == (4096, 2048) and a.codes.dtype == np.uint8
    assert a.scales.shape == (4096, 64) and a.x.shape == (8, 4096)
    s16 = oracle.fp16_bits_to_f64(a.scales)
    assert s16.min() >= 0.001 - 1e-6 and s16.max() <= 0.01 + 1e-5
    b16 = oracle.fp16_bits_to_f64(a.biases)
    resid = b16 + 8 * s16
    assert abs(resid.mean()) < 1e-4 and 0.8e-3 < resid.std() < 1.2e-3
    # codes uniform: every nibble value appears with frequency ~1/16
    q = oracle.unpack_codes(a.codes[:64], 4096, 4)
    freq = np.bincount(q.ravel(), minlength=16) / q.size
    assert np.all(np.abs(freq - 1 / 16) < 0.005)


def test_generator_8bit_distributions():
    s = synth.WORKLOADS["square_k4096_n4096_8b_g64"]
    a = synth.make_problem(s)
    assert a.codes.shape == (4096, 4096) and a.scales.shape == (4096, 64)
    s16 = oracle.fp16_bits_to_f64(a.scales)
    assert s16.min() >= 1e-4 - 1e-7 and s16.max() <= 1e-3 + 1e-6
    resid = oracle.fp16_bits_to_f64(a.biases) + 128 * s16
    assert abs(resid.mean()) < 1e-4 and 0.8e-3 < resid.std() < 1.2e-3
    freq = np.bincount(a.codes[:64].ravel(), minlength=256) / a.codes[:64].size
    assert np.all(np.abs(freq - 1 / 256) < 0.001)


def test_group_size_sweep_shares_codes_and_x():
    ps = [synth.make_problem(synth.WORKLOADS[f"ffnup_k4096_n12288_4b_g{g}"]) for g in (32, 64, 128)]
    assert all(np.array_equal(ps[0].codes, p.codes) for p in ps)
    assert all(np.array_equal(ps[0].x, p.x) for p in ps)
    assert ps[0].scales.shape == (12288, 128) and ps[2].scales.shape == (12288, 32)


def test_outlier_channels():
    p = synth.make_problem(synth.WORKLOADS["layer27b_down"])
    assert len(p.outlier_channels) == 174
    x = oracle.bf16_bits_to_f64(p.x)
    mask = np.zeros(p.K, bool)
    mask[p.outlier_channels] = True
    assert np.abs(x[:, mask]).mean() > 10 * np.abs(x[:, ~mask]).mean()


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = synth.f32_to_bf16_bits(v).tolist()
    assert got == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


@pytest.mark.parametrize("bits,gs,K,N,M", [(4, 64, 128, 6, 2), (2, 32, 128, 5, 3)])
def test_abs_product_sum_matches_exact_rational(bits, gs, K, N, M):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=7 + K + N), m_max=M)
    got = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, N, K, bits, gs)
    for n in range(N):
        q = bitstream_codes(p.codes[n], K, bits)
        w = [frac_fp16(int(p.scales[n, k // gs])) * q[k] + frac_fp16(int(p.biases[n, k // gs]))
             for k in range(K)]
        for m in range(M):
            want = sum(abs(frac_bf16(int(p.x[m, k])) * w[k]) for k in range(K))
            assert abs(Fraction(got[m, n]) - want) <= Fraction(K) * Fraction(2) ** -52 * want
