"""GPU parity of the gathered (MoE) verify, qgemv_gather, through the C ABI
against the fp64 oracle.

Bars: every element within 1e-3 * sum|x w| + 1e-6 of the oracle, full
sizes included; each pair's row bitwise equal to a call with the same
activation rows X and that pair alone (the kernel and its configuration depend
on the shape and X only, not on the other pairs: the single-pass kernel for
X <= 2, the persistent one from X = 3); repeated calls bitwise identical;
pairs with invalid indices leave their row of y untouched.
"""
import numpy as np
import pytest

import oracle
from few_row_quantized_amd import qgemv as q
from few_row_quantized_amd import synth

from gpu_util import OracleRows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import torch
    torch.cuda.init()
    yield


class MoeDevice:
    def __init__(self, p):
        import torch
        self.p = p
        d = "cuda:0"
        self.codes = torch.from_numpy(p.codes).to(d)
        self.scales = torch.from_numpy(p.scales.view(np.int16)).to(d)
        self.biases = torch.from_numpy(p.biases.view(np.int16)).to(d)
        self.x = torch.from_numpy(p.x.view(np.int16)).to(d)

    def run(self, x_idx, e_idx, fill=float("nan"), X=None):
        # X: activation rows passed to the call (the first X rows of x)
        import torch
        s = self.p.shape
        X = self.p.x.shape[0] if X is None else X
        P = len(e_idx)
        xi = torch.from_numpy(np.asarray(x_idx, np.int32)).to("cuda:0")
        ei = torch.from_numpy(np.asarray(e_idx, np.int32)).to("cuda:0")
        y = torch.full((P, s.N), fill, dtype=torch.float32, device="cuda:0")
        q.qgemv_gather(self.codes, self.scales, self.biases, self.x, xi, ei, y, P, X,
                       s.E, s.N, s.K, s.bits, s.group_size)
        torch.cuda.synchronize()
        return y.cpu().numpy()


def check(p, y, x_idx, e_idx, cols=None, label=""):
    s = p.shape
    ref = oracle.qgemv_gather_reference(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K,
                                        s.bits, s.group_size, rows=cols)
    absum = oracle.gather_abs_product_sum(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K,
                                          s.bits, s.group_size, rows=cols)
    yy = y if cols is None else y[:, cols]
    ok, worst, idx = oracle.check_close(yy, ref, absum)
    assert ok, f"{label}: worst |dy|/tol = {worst:.3g} at {idx}"


def small(E=12, K=1024, N=200, bits=4, gs=64, X=16, seed=5):
    return synth.make_moe_problem(synth.MoeShape("moe_small", E, K, N, bits, gs, 4, (X,), seed), m_max=X)


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 32), (4, 128), (2, 64), (8, 64)])
def test_random_routing_every_element(bits, gs):
    p = small(bits=bits, gs=gs, seed=bits * 100 + gs)
    d = MoeDevice(p)
    rng = np.random.default_rng(1)
    for P in (1, 7, 40, 128):
        x_idx = rng.integers(0, 16, size=P)
        e_idx = rng.integers(0, p.shape.E, size=P)
        say(f"gather random bits={bits} gs={gs} P={P}")
        check(p, d.run(x_idx, e_idx), x_idx, e_idx, label=f"P={P}")


def test_many_pairs_on_one_expert():
    # 40 pairs on expert 3: three chunks of at most 16 rows
    p = small(seed=11)
    d = MoeDevice(p)
    x_idx = np.arange(40) % 16
    e_idx = np.full(40, 3)
    e_idx[[5, 17, 33]] = [0, 11, 3]
    say("gather many pairs on one expert")
    check(p, d.run(x_idx, e_idx), x_idx, e_idx, label="one expert")


@pytest.mark.parametrize("bits,gs", [(4, 64), (2, 64), (8, 32)])
def test_few_activation_rows_every_element_and_bitwise(bits, gs):
    # at most 4 or 8 activation rows: compact activation loads, experts' pairs
    # taken 4 or 8 at a time (an expert with more pairs than rows gets several
    # chunks); each pair's row is the same float as with the most rows passed
    # to the same kernel (2 rows: the single-pass kernel; 16: the persistent)
    p = small(bits=bits, gs=gs, seed=19 + bits)
    d = MoeDevice(p)
    rng = np.random.default_rng(7)
    for X in (1, 2, 3, 4, 5, 8):
        for P in (1, 9, 40):
            x_idx = rng.integers(0, X, size=P)
            e_idx = rng.integers(0, 3 if P == 40 else p.shape.E, size=P)  # P = 40: ~13 pairs per expert
            say(f"gather few rows bits={bits} gs={gs} X={X} P={P}")
            y = d.run(x_idx, e_idx, X=X)
            check(p, y, x_idx, e_idx, label=f"X={X} P={P}")
            Xr = 2 if X <= 2 else 16
            assert np.array_equal(y, d.run(x_idx, e_idx, X=Xr)), f"X={X} P={P} against {Xr} rows"


def test_invalid_pairs_leave_rows_untouched():
    p = small(seed=13)
    d = MoeDevice(p)
    x_idx = np.array([0, 1, 99, 2, -1, 3])
    e_idx = np.array([1, 12, 2, -5, 4, 0])  # pairs 1 (expert 12 of 12), 2, 3, 4 are invalid
    say("gather invalid pairs")
    y = d.run(x_idx, e_idx, fill=7.25)
    bad = [1, 2, 3, 4]
    assert np.all(y[bad] == np.float32(7.25))
    good = [0, 5]
    check(p, y[good], x_idx[good], e_idx[good], label="valid pairs")


@pytest.mark.parametrize("X", [2, 16])
def test_pair_rows_do_not_depend_on_the_other_pairs_and_repeat(X):
    p = small(E=6, K=2048, N=1536, seed=17)  # 96 tiles, K=2048
    d = MoeDevice(p)
    rng = np.random.default_rng(3)
    x_idx = rng.integers(0, X, size=24)
    e_idx = rng.integers(0, 6, size=24)
    say(f"gather pair rows vs single-pair calls, bitwise, X={X}")
    y = d.run(x_idx, e_idx, X=X)
    check(p, y, x_idx, e_idx, label=f"X={X}")
    assert np.array_equal(y, d.run(x_idx, e_idx, X=X))
    for i in range(len(e_idx)):
        y1 = d.run(x_idx[i:i + 1], e_idx[i:i + 1], X=X)
        assert np.array_equal(y1[0], y[i]), f"pair {i}"


@pytest.mark.parametrize("name", list(synth.MOE_WORKLOADS))
def test_full_size_every_element(name):
    # pairs(M) are the first 8*M pairs of pairs(16): one oracle evaluation
    s = synth.MOE_WORKLOADS[name]
    p = synth.make_moe_problem(s)
    d = MoeDevice(p)
    xa, ea = p.pairs(16)
    orc = OracleRows.gather(p, xa, ea)
    # X = M activation rows, as a verify step passes them (M <= 2: the
    # single-pass kernel, M >= 3: the persistent one where the shape fits it),
    # and X = 16 rows passed for every M
    for M in (1, 2, 3, 4, 8, 16):
        x_idx, e_idx = p.pairs(M)
        assert np.array_equal(x_idx, xa[:len(x_idx)]) and np.array_equal(e_idx, ea[:len(e_idx)])
        for X in sorted({M, 16}):
            say(f"gather full {name} M={M} X={X} pairs={len(e_idx)} union={len(set(e_idx.tolist()))}")
            y = d.run(x_idx, e_idx, X=X)
            assert np.all(np.isfinite(y))
            orc.check(y, len(e_idx), label=f"{name} M={M} X={X}")


def test_full_size_pair_rows_do_not_depend_on_the_other_pairs():
    # 16 verify rows on the 128-expert gate/up shape: the union's (expert, tile)
    # items outnumber the resident workgroups, so each workgroup walks several;
    # sampled pairs computed alone give the same bits
    s = synth.MOE_WORKLOADS["moe30b_gateup_e128_k2048_n1536_4b_g64_top8"]
    p = synth.make_moe_problem(s)
    d = MoeDevice(p)
    x_idx, e_idx = p.pairs(16)
    say(f"gather full-size pair rows vs single-pair calls, pairs={len(e_idx)} union={len(set(e_idx.tolist()))}")
    y = d.run(x_idx, e_idx)
    rng = np.random.default_rng(11)
    for i in sorted(rng.choice(len(e_idx), size=24, replace=False).tolist()):
        y1 = d.run(x_idx[i:i + 1], e_idx[i:i + 1])
        assert np.array_equal(y1[0], y[i]), f"pair {i} (expert {int(e_idx[i])}, row {int(x_idx[i])})"


@pytest.mark.parametrize("X", [2, 3, 16])
def test_max_pairs_on_few_experts(X):
    # QGEMV_MAX_PAIRS pairs on 3 experts of a ragged N: ~85 pairs per expert,
    # so every expert takes several chunks (16 pairs each with 16 rows, 4 with
    # 3 rows) and a workgroup's item range crosses chunk and expert borders;
    # sampled pairs computed alone give the same bits
    p = small(E=5, K=1024, N=200, X=16, seed=23)
    d = MoeDevice(p)
    rng = np.random.default_rng(29)
    P = q.MAX_PAIRS
    x_idx = rng.integers(0, X, size=P)
    e_idx = rng.choice([0, 2, 4], size=P)
    say(f"gather max pairs X={X} P={P}")
    y = d.run(x_idx, e_idx, X=X)
    check(p, y, x_idx, e_idx, label=f"X={X} P={P}")
    for i in sorted(rng.choice(P, size=6, replace=False).tolist()):
        y1 = d.run(x_idx[i:i + 1], e_idx[i:i + 1], X=X)
        assert np.array_equal(y1[0], y[i]), f"pair {i}"


@pytest.mark.parametrize("X", [2, 8])
def test_many_experts(X):
    # QGEMV_MAX_EXPERTS experts stored, 64 pairs on random ones (the union
    # bitmap and the rank sort over ids up to 4095); small N and K
    p = small(E=q.MAX_EXPERTS, K=256, N=48, X=16, seed=31)
    d = MoeDevice(p)
    rng = np.random.default_rng(37)
    x_idx = rng.integers(0, X, size=64)
    e_idx = rng.integers(0, q.MAX_EXPERTS, size=64)
    e_idx[:4] = [0, q.MAX_EXPERTS - 1, q.MAX_EXPERTS - 1, 2048]
    say(f"gather many experts X={X}")
    check(p, d.run(x_idx, e_idx, X=X), x_idx, e_idx, label=f"X={X}")
