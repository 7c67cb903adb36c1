"""Pins for the oracle's gathered (MoE) verify product, against things other
than the oracle itself: closed forms with one-hot activation rows (which
select one dequantized column of the routed expert), exact rational brute
force with this file's own decoders, structural invariants (permuting or
repeating pairs), and planted mistakes that must fail a pin."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import qgemv_oracle as qo
from few_row_quantized_amd import synth

from test_oracle import bitstream_codes, frac_bf16, frac_fp16


def tiny(E=5, N=6, K=128, bits=4, gs=64, X=3, seed=3):
    shape = synth.MoeShape("tiny_moe", E, K, N, bits, gs, 2, (X,), seed)
    return synth.make_moe_problem(shape, m_max=X)


def run(p, x_idx, e_idx, rows=None):
    s = p.shape
    return oracle.qgemv_gather_reference(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K,
                                         s.bits, s.group_size, rows=rows)


def test_onehot_rows_select_the_routed_experts_column():
    p = tiny()
    s = p.shape
    cols = [5, 64, 127]  # one-hot column of x row 0, 1, 2 (two groups)
    p.x[:] = 0
    for r, k in enumerate(cols):
        p.x[r, k] = 0x3F80
    x_idx = np.array([2, 0, 1, 0, 2, 1])
    e_idx = np.array([4, 4, 0, 2, 1, 3])
    y = run(p, x_idx, e_idx)
    for i in range(len(e_idx)):
        e, k = int(e_idx[i]), cols[x_idx[i]]
        for n in range(s.N):
            q = bitstream_codes(p.codes[e, n], s.K, s.bits)[k]
            want = frac_fp16(int(p.scales[e, n, k // s.group_size])) * q + \
                frac_fp16(int(p.biases[e, n, k // s.group_size]))
            assert y[i, n] == float(want), (i, n)


def test_matches_exact_rational_brute_force():
    p = tiny(E=4, N=3, K=64, gs=32, X=3, seed=8)
    s = p.shape
    x_idx = np.array([0, 1, 2, 1, 0])
    e_idx = np.array([3, 3, 0, 1, 3])
    y = run(p, x_idx, e_idx)
    for i in range(len(e_idx)):
        e, r = int(e_idx[i]), int(x_idx[i])
        xs = [frac_bf16(int(v)) for v in p.x[r]]
        for n in range(s.N):
            q = bitstream_codes(p.codes[e, n], s.K, s.bits)
            w = [frac_fp16(int(p.scales[e, n, k // s.group_size])) * q[k] +
                 frac_fp16(int(p.biases[e, n, k // s.group_size])) for k in range(s.K)]
            exact = sum(xs[k] * w[k] for k in range(s.K))
            bound = Fraction(s.K) * Fraction(2) ** -52 * sum(abs(xs[k] * w[k]) for k in range(s.K))
            assert abs(Fraction(y[i, n]) - exact) <= bound


def test_permuting_or_repeating_pairs_moves_rows():
    p = tiny()
    x_idx = np.array([0, 1, 2, 0, 1])
    e_idx = np.array([1, 1, 4, 3, 0])
    y = run(p, x_idx, e_idx)
    perm = np.array([3, 0, 4, 2, 1])
    assert np.array_equal(run(p, x_idx[perm], e_idx[perm]), y[perm])
    rep = np.array([0, 0, 2, 2])
    assert np.array_equal(run(p, x_idx[rep], e_idx[rep]), y[rep])
    assert np.array_equal(run(p, x_idx, e_idx, rows=[0, 5]), y[:, [0, 5]])


def _pins():
    try:
        test_onehot_rows_select_the_routed_experts_column()
        test_matches_exact_rational_brute_force()
    except AssertionError:
        return False
    return True


def _swapped_roles(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    return qo._orig_gather(codes, scales, biases, x_bits, np.minimum(e_idx, len(x_bits) - 1),
                           np.minimum(x_idx, len(codes) - 1), N, K, bits, gs, rows)


def _expert_off_by_one(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    return qo._orig_gather(codes, scales, biases, x_bits, x_idx, (np.asarray(e_idx) + 1) % len(codes),
                           N, K, bits, gs, rows)


def _pair_index_as_row(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    rows_ = np.arange(len(e_idx)) % len(x_bits)
    return qo._orig_gather(codes, scales, biases, x_bits, rows_, e_idx, N, K, bits, gs, rows)


@pytest.mark.parametrize("mutant", [_swapped_roles, _expert_off_by_one, _pair_index_as_row])
def test_pins_catch_planted_mistakes(monkeypatch, mutant):
    assert _pins()
    monkeypatch.setattr(qo, "_orig_gather", qo.qgemv_gather_reference, raising=False)
    monkeypatch.setattr(qo, "qgemv_gather_reference", mutant)
    monkeypatch.setattr(oracle, "qgemv_gather_reference", mutant)
    assert not _pins(), f"{mutant.__name__} went unnoticed"


def test_moe_generator_routing():
    s = synth.MOE_WORKLOADS["moe30b_down_e128_k768_n2048_4b_g64_top8"]
    p = synth.make_moe_problem(s)
    assert p.codes.shape == (128, 2048, 384) and p.scales.shape == (128, 2048, 12)
    for m in range(16):
        assert len(set(p.routing[m].tolist())) == 8  # distinct experts per row
    x_idx, e_idx = p.pairs(4)
    assert x_idx.tolist() == [0] * 8 + [1] * 8 + [2] * 8 + [3] * 8
    assert e_idx.tolist() == p.routing[:4].reshape(-1).tolist()


# ---------------------------------------------------------------- the tolerance scale
#
# gather_abs_product_sum sets the bound of every MoE parity check: pinned by
# exact rational brute force, a one-hot closed form (|w| of the routed
# expert's column, whatever the sign of x), and planted mistakes.

def abs_run(p, x_idx, e_idx, rows=None):
    s = p.shape
    return oracle.gather_abs_product_sum(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K,
                                         s.bits, s.group_size, rows=rows)


def test_abs_product_sum_matches_exact_rational_brute_force():
    p = tiny(E=4, N=3, K=64, gs=32, X=3, seed=11)
    s = p.shape
    x_idx = np.array([2, 1, 0, 1, 2])
    e_idx = np.array([0, 3, 3, 1, 2])
    got = abs_run(p, x_idx, e_idx)
    for i in range(len(e_idx)):
        e, r = int(e_idx[i]), int(x_idx[i])
        xs = [frac_bf16(int(v)) for v in p.x[r]]
        for n in range(s.N):
            q = bitstream_codes(p.codes[e, n], s.K, s.bits)
            w = [frac_fp16(int(p.scales[e, n, k // s.group_size])) * q[k] +
                 frac_fp16(int(p.biases[e, n, k // s.group_size])) for k in range(s.K)]
            want = sum(abs(xs[k] * w[k]) for k in range(s.K))
            assert want > 0
            assert abs(Fraction(got[i, n]) - want) <= Fraction(s.K) * Fraction(2) ** -52 * want, (i, n)


def test_abs_product_sum_onehot_gives_magnitude_of_the_routed_weight():
    p = tiny()
    s = p.shape
    cols = [3, 70, 126]
    p.x[:] = 0
    p.x[0, cols[0]] = 0xBF80  # -1.0
    p.x[1, cols[1]] = 0x4000  # 2.0
    p.x[2, cols[2]] = 0xC040  # -3.0
    mag = [1, 2, 3]
    x_idx = np.array([1, 0, 2, 2, 0, 1])
    e_idx = np.array([4, 4, 0, 3, 1, 2])
    got = abs_run(p, x_idx, e_idx)
    for i in range(len(e_idx)):
        e, r = int(e_idx[i]), int(x_idx[i])
        k = cols[r]
        for n in range(s.N):
            q = bitstream_codes(p.codes[e, n], s.K, s.bits)[k]
            w = frac_fp16(int(p.scales[e, n, k // s.group_size])) * q + \
                frac_fp16(int(p.biases[e, n, k // s.group_size]))
            assert got[i, n] == float(mag[r] * abs(w)), (i, n)


def test_abs_product_sum_is_at_least_the_magnitude_of_y():
    p = tiny(seed=12)
    x_idx = np.array([0, 1, 2, 0])
    e_idx = np.array([3, 3, 1, 0])
    a = abs_run(p, x_idx, e_idx)
    y = run(p, x_idx, e_idx)
    assert np.all(a >= np.abs(y) * (1 - 128 * 2.0 ** -52))
    assert np.array_equal(abs_run(p, x_idx, e_idx, rows=[1, 4]), a[:, [1, 4]])


def _abs_pins():
    try:
        test_abs_product_sum_matches_exact_rational_brute_force()
        test_abs_product_sum_onehot_gives_magnitude_of_the_routed_weight()
        test_abs_product_sum_is_at_least_the_magnitude_of_y()
    except AssertionError:
        return False
    return True


def _abs_inflated(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    return 2.0 * qo._orig_gabs(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows)


def _abs_wrong_row(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    return qo._orig_gabs(codes, scales, biases, x_bits, (np.asarray(x_idx) + 1) % len(x_bits), e_idx,
                         N, K, bits, gs, rows)


def _abs_wrong_expert(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    return qo._orig_gabs(codes, scales, biases, x_bits, x_idx, (np.asarray(e_idx) + 1) % len(codes),
                         N, K, bits, gs, rows)


def _abs_dropped_on_w(codes, scales, biases, x_bits, x_idx, e_idx, N, K, bits, gs, rows=None):
    out = []
    x = np.abs(qo.bf16_bits_to_f64(np.asarray(x_bits)))
    idx = np.arange(N) if rows is None else np.asarray(rows)
    for r, e in zip(np.asarray(x_idx), np.asarray(e_idx)):
        q = qo.unpack_codes(codes[e][idx], K, bits)
        w = qo.dequantize(q, scales[e][idx], biases[e][idx], gs)
        out.append(x[r] @ w.T)
    return np.array(out)


@pytest.mark.parametrize("mutant", [_abs_inflated, _abs_wrong_row, _abs_wrong_expert, _abs_dropped_on_w])
def test_abs_pins_catch_planted_mistakes(monkeypatch, mutant):
    assert _abs_pins()
    monkeypatch.setattr(qo, "_orig_gabs", qo.gather_abs_product_sum, raising=False)
    monkeypatch.setattr(qo, "gather_abs_product_sum", mutant)
    monkeypatch.setattr(oracle, "gather_abs_product_sum", mutant)
    assert not _abs_pins(), f"{mutant.__name__} went unnoticed"
