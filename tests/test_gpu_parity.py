"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars:
* decoded integer codes: bit-exact (unpack probe of each path, and the
  one-hot unit-scale product y == q exactly);
* y: |y - y_ref| <= 1e-3 * sum_k |x_k w_k| + 1e-6 per element, no NaN;
* within one path, row m of an M-row call is bitwise equal to the M=1 call on
  x[m], and repeated calls are bitwise identical.
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


def check_y(p, y, M, cols=None, label=""):
    ref = oracle.qgemv_reference(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits,
                                 p.group_size, rows=cols)
    absum = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, M, p.N, p.K, p.bits,
                                   p.group_size, rows=cols)
    yy = y if cols is None else y[:, cols]
    ok, worst, idx = oracle.check_close(yy, ref, absum)
    assert ok, f"{label}: worst |dy|/tol = {worst:.3g} at {idx}"
    return worst


def supported(path, p, M=1):
    return q.qgemv_path_supported(path, M, p.N, p.K, p.bits, p.group_size)


# ---------------------------------------------------------------- codes: bit-exact

UNPACK_SHAPES = [
    (256, 512, 4, 64), (512, 40, 4, 32), (1024, 17, 4, 128),
    (512, 40, 2, 64), (1024, 33, 2, 128), (512, 24, 2, 32),
    (256, 512, 8, 64), (512, 40, 8, 32), (1024, 17, 8, 128),
]


@pytest.mark.parametrize("K,N,bits,gs", UNPACK_SHAPES)
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_unpack_probe_is_bit_exact(path, K, N, bits, gs):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=K + N), m_max=1)
    if not q.qgemv_path_supported(path, 1, N, K, bits, gs):
        pytest.skip("path does not support this shape")
    say(f"unpack probe {path} K={K} N={N} bits={bits} gs={gs}")
    d = DeviceProblem(p)
    out = torch.full((N, K), 0xEE, dtype=torch.uint8, device="cuda:0")
    q.qgemv_unpack_probe(path, d.codes, out, N, K, bits, gs)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.unpack_codes(p.codes, K, bits)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", [n for n, w in synth.WORKLOADS.items() if w.fmt is None])
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_unpack_probe_full_size(path, name):
    import torch
    s = synth.WORKLOADS[name]
    if not q.qgemv_path_supported(path, 1, s.N, s.K, s.bits, s.group_size):
        pytest.skip("path does not support this shape")
    p = synth.make_problem(s, m_max=1)
    say(f"unpack probe {path} {name}")
    d = DeviceProblem(p)
    out = torch.empty((s.N, s.K), dtype=torch.uint8, device="cuda:0")
    q.qgemv_unpack_probe(path, d.codes, out, s.N, s.K, s.bits, s.group_size)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.unpack_codes(p.codes, s.K, s.bits))


@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 32), (4, 128), (2, 64), (2, 128), (2, 32),
                                     (8, 32), (8, 64), (8, 128)])
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_unit_scale_onehot_gives_codes_exactly(path, bits, gs):
    K, N, M = 1024, 48, 16
    p = synth.special_problem(K, N, bits, gs, M, "unit_scale_onehot")
    if not supported(path, p, M):
        pytest.skip("path does not support this shape")
    say(f"onehot {path} bits={bits} gs={gs}")
    y = DeviceProblem(p).run_host(M, path)
    codes = oracle.unpack_codes(p.codes, K, bits)
    for m in range(M):
        k = synth.onehot_column(m, K)
        assert np.array_equal(y[m], codes[:, k].astype(np.float32)), f"row {m}"


# ---------------------------------------------------------------- small shapes, every element

@pytest.mark.parametrize("path", PATHS)
def test_tiny_workload_all_m(path):
    s = synth.WORKLOADS["tiny_k256_n512_4b_g64"]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    for M in s.m_values:
        say(f"tiny {path} M={M}")
        check_y(p, d.run_host(M, path), M, label=f"tiny {path} M={M}")


RAGGED = [
    # K, N, bits, gs : N not a multiple of the tile sizes, several K stages
    (640, 40, 4, 32), (1024, 300, 4, 64), (2048, 97, 4, 128), (8192, 33, 4, 64),
    (512, 72, 2, 32), (1280, 300, 2, 64), (2048, 129, 2, 128), (17408, 23, 2, 64),
    (64, 16, 4, 32), (64, 5, 2, 64),
    (640, 40, 8, 32), (1024, 300, 8, 64), (2048, 97, 8, 128), (8192, 33, 8, 64), (64, 16, 8, 32),
    (3840, 200, 8, 64),
]


@pytest.mark.parametrize("K,N,bits,gs", RAGGED)
@pytest.mark.parametrize("path", PATHS)
def test_ragged_shapes_every_element(path, K, N, bits, gs):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=3 * K + N, outliers=True), m_max=16)
    if not supported(path, p):
        pytest.skip("path does not support this shape")
    d = DeviceProblem(p)
    for M in (1, 2, 5, 8, 13, 16):
        say(f"ragged {path} K={K} N={N} bits={bits} gs={gs} M={M}")
        check_y(p, d.run_host(M, path), M, label=f"{path} K={K} N={N} M={M}")


# More 16-column tiles than CUs: the MFMA path streams several tiles per
# workgroup (ranges of 1 to 3 tiles, ragged last tile) with the activations
# in registers, or, when K is too long for them, with one half of K's
# activations in LDS per workgroup (K 6656 and up: an odd number of bias
# blocks, halves of 7 to 24 blocks, 4 to 12 waves, 1 to 4 blocks per wave).
PERSIST = [
    (1024, 4113, 4, 32), (2048, 4500, 4, 64), (3072, 5000, 4, 128), (6144, 4200, 4, 128),
    (1280, 4700, 2, 64), (2048, 9000, 2, 128), (8192, 4500, 4, 128),
    (1024, 4113, 8, 32), (2048, 4500, 8, 64), (3840, 4200, 8, 64), (5120, 4150, 8, 64),
    (6656, 4200, 4, 128), (8192, 4130, 2, 64), (10240, 4500, 2, 128),
]

# Long K with the activations of half of K in LDS, at sizes where the LDS
# holds a whole half only up to M = 7 to 10: larger M restages the
# activations in two or three phases per half.
LONG_K_LDS = [(12288, 4104, 4, 64), (12288, 4100, 4, 32), (17408, 4128, 2, 64), (17408, 4200, 4, 128)]


@pytest.mark.parametrize("K,N,bits,gs", PERSIST)
def test_many_tiles_per_cu_every_element(K, N, bits, gs):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=5 * K + N, outliers=True), m_max=16)
    d = DeviceProblem(p)
    for M in (1, 3, 8, 16):
        say(f"many tiles mfma K={K} N={N} bits={bits} gs={gs} M={M}")
        check_y(p, d.run_host(M, "mfma"), M, label=f"mfma K={K} N={N} M={M}")


@pytest.mark.parametrize("K,N,bits,gs", LONG_K_LDS)
def test_long_k_lds_persistent_every_element(K, N, bits, gs):
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=9 * K + N, outliers=True), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, 16)
    for M in (1, 2, 7, 8, 9, 16):
        say(f"long K lds mfma K={K} N={N} bits={bits} gs={gs} M={M}")
        orc.check(d.run_host(M, "mfma"), M, label=f"mfma K={K} N={N} M={M}")


@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_zero_codes(path):
    K, N, M = 2048, 64, 8
    p = synth.special_problem(K, N, 4, 64, M, "zero_codes")
    say(f"zero codes {path}")
    check_y(p, DeviceProblem(p).run_host(M, path), M, label="zero codes")


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("bits,gs,N,K", [(4, 64, 200, 2048), (2, 64, 200, 2048), (4, 128, 200, 2048),
                                         (4, 64, 4500, 2048), (2, 128, 4500, 2048),
                                         (4, 128, 300, 8192), (2, 64, 150, 10240),
                                         (4, 128, 4200, 6656), (2, 64, 4130, 8192),
                                         (8, 64, 200, 2048), (8, 32, 4500, 1024), (8, 64, 150, 10240), (8, 64, 4150, 5120),
                                         (4, 64, 4096, 8192)])
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_row_of_m_row_call_equals_single_row_call_bitwise(path, bits, gs, N, K):
    import torch
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=77), m_max=16)
    d = DeviceProblem(p)
    say(f"row invariance {path} bits={bits} gs={gs} N={N} K={K}")
    singles = []
    for m in range(16):
        xm = d.x[m:m + 1].clone()
        y1 = torch.empty((1, N), dtype=torch.float32, device="cuda:0")
        q.qgemv_run_path(path, d.codes, d.scales, d.biases, xm, y1, 1, N, K, bits, gs)
        singles.append(y1)
    torch.cuda.synchronize()
    singles = torch.cat(singles).cpu().numpy()
    for M in (2, 3, 4, 5, 6, 7, 8, 9, 12, 16):
        y = d.run_host(M, path)
        assert np.array_equal(y, singles[:M]), f"M={M}"


@pytest.mark.parametrize("bits,gs,N,K", [(4, 128, 4200, 17408), (2, 64, 4130, 17408)])
def test_long_k_row_invariance_by_configuration(bits, gs, N, K):
    # Long K with more tiles than CUs: the long-K kernel's configuration
    # depends on M through its LDS budget (tests/kernel_config.py mirrors the
    # launch search).  Rows agree bit for bit within a configuration, and with
    # the oracle's tolerance across configurations.
    import torch
    from kernel_config import mfma_configuration
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = synth.make_problem(synth.custom_shape(K, N, bits, gs, seed=78), m_max=16)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, 16)
    say(f"long-K row invariance bits={bits} gs={gs} N={N} K={K} cus={cus}")
    first = {}  # configuration -> (M, y) of its smallest M
    configs = set()
    for M in range(1, 17):
        cfg = mfma_configuration(M, N, K, bits, gs, cus)
        configs.add(cfg)
        y = d.run_host(M, "mfma")
        orc.check(y, M, f"M={M} {cfg}")
        if cfg in first:
            M0, y0 = first[cfg]
            assert np.array_equal(y[:M0], y0), f"M={M} differs from M={M0} within {cfg}"
        else:
            first[cfg] = (M, y)
    assert len(configs) >= 2, "the shape should cross a configuration threshold"


@pytest.mark.parametrize("name", ["square_k4096_n4096_4b_g64", "layer27b_gate", "layer27b_down",
                                  "mlxbench_k5120_n17408_8b_g64"])
@pytest.mark.parametrize("path", ["dot", "mfma"])
def test_repeated_calls_are_bitwise_identical(path, name):
    s = synth.WORKLOADS[name]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    say(f"determinism {path} {name}")
    a = d.run_host(8, path)
    b = d.run_host(8, path)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- full sizes, every element

FULL_CASES = [(_n, tuple(_s.m_values)) for _n, _s in synth.WORKLOADS.items()
              if not _n.startswith("tiny") and _s.fmt is None]


@pytest.mark.parametrize("name,ms", FULL_CASES)
def test_full_size_every_element(name, ms):
    # one oracle evaluation at the largest M; every element of every M, on
    # both paths and the dispatcher (the bench's launch configuration)
    s = synth.WORKLOADS[name]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    orc = OracleRows.affine(p, max(ms))
    worst = 0.0
    for path in PATHS:
        if not supported(path, p):
            continue
        for M in ms:
            say(f"full {name} {path} M={M}")
            y = d.run_host(M, path)
            assert np.all(np.isfinite(y)), "non-finite output"
            worst = max(worst, orc.check(y, M, label=f"{name} {path} M={M}"))
    say(f"full {name}: worst |dy|/tol = {worst:.3g}")


def test_auto_path_matches_select():
    # the dispatcher's choice is what qgemv_small runs: compare bitwise
    s = synth.WORKLOADS["square_k4096_n4096_4b_g64"]
    p = synth.make_problem(s)
    d = DeviceProblem(p)
    for M in s.m_values:
        chosen = q.qgemv_select(M, s.N, s.K, s.bits, s.group_size)
        name = {q.PATH_DOT: "dot", q.PATH_MFMA: "mfma"}[chosen]
        say(f"auto vs {name} M={M}")
        assert np.array_equal(d.run_host(M, "auto"), d.run_host(M, name))


# ---------------------------------------------------------------- stream probe

def test_stream_probe_reads_every_byte():
    import torch
    nbytes = 9 * 1024 * 1024 + 4096
    rng = np.random.default_rng(9)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).to("cuda:0")
    nb = q.qgemv_stream_probe_blocks(nbytes)
    for layout in (0, 1):
        for u in (1, 2, 4, 8, 16):
            out = torch.zeros(nb, dtype=torch.int32, device="cuda:0")
            q.qgemv_stream_probe(buf, nbytes, out, u, layout)
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
            assert got == np.bitwise_xor.reduce(host), f"layout {layout}, loads per thread {u}"


# ---------------------------------------------------------------- concurrency

def test_concurrent_calls_from_host_threads_on_separate_streams():
    # the library keeps only caches of device properties: calls from several
    # host threads, each on its own stream (default priority), give the same
    # bits as the same calls made one after another
    import threading
    import torch
    cases = [(2048, 4500, 4, 64, "mfma"), (1024, 300, 4, 32, "dot"), (5120, 1024, 4, 128, "mfma"),
             (2048, 97, 8, 64, "auto"), (1280, 300, 2, 64, "dot"), (4096, 512, 8, 32, "mfma")]
    devs = [DeviceProblem(synth.make_problem(synth.custom_shape(K, N, b, g, seed=K + N), m_max=8))
            for K, N, b, g, _ in cases]
    say("concurrency: sequential reference")
    want = [d.run_host(M, path) for d, (_, _, _, _, path) in zip(devs, cases) for M in (1, 5, 8)]
    got = [None] * len(want)
    errors = []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            d, path = devs[i], cases[i][4]
            outs = []
            with torch.cuda.stream(st):
                for M in (1, 5, 8):
                    y = torch.full((M, d.p.N), float("nan"), dtype=torch.float32, device="cuda:0")
                    for _ in range(20):
                        q.qgemv_run_path(path, d.codes, d.scales, d.biases, d.x, y, M, d.p.N, d.p.K,
                                         d.p.bits, d.p.group_size, stream=st)
                    outs.append(y)
            st.synchronize()
            for j, y in enumerate(outs):
                got[3 * i + j] = y.cpu().numpy()
        except Exception as e:  # surfaced below
            errors.append(repr(e))

    say("concurrency: threads")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for a, b in zip(want, got):
        assert np.array_equal(a, b)
