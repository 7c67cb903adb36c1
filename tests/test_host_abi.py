"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/qgemv.h declares, and rejects invalid arguments with
the documented status before anything is launched."""
import ctypes
import os
import re

import pytest

from few_row_quantized_amd import qgemv as q

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qgemv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(qgemv_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("qgemv_small", "qgemv_select", "qgemv_run_path", "qgemv_unpack_probe",
                 "qgemv_stream_probe", "qgemv_strerror", "qgemv_small_add", "qgemv_run_path_add"):
        assert must in names


def test_binding_limits_match_the_header():
    src = open(HEADER).read()
    for name, val in (("QGEMV_MAX_M", q.MAX_M), ("QGEMV_MAX_K", q.MAX_K), ("QGEMV_MAX_N", q.MAX_N)):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, src)
        assert m and int(m.group(1)) == val, name


def test_shapes_at_the_limits_are_accepted_and_beyond_rejected():
    L = q.lib()
    # validation only (fake pointers): the limits pass shape checks, one past fails
    assert L.qgemv_select(q.MAX_M, 64, q.MAX_K, 4, 128) in (q.PATH_DOT, q.PATH_MFMA)
    assert L.qgemv_select(1, q.MAX_N, 128, 4, 32) in (q.PATH_DOT, q.PATH_MFMA)
    assert L.qgemv_select(1, q.MAX_N + 1, 128, 4, 32) == q.EINVAL
    assert L.qgemv_select(1, 64, q.MAX_K + 128, 4, 128) == q.EINVAL


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(q.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


# Fake, never-dereferenced addresses: every call below fails validation first.
A = 1 << 20  # 16-byte aligned
MIS = A + 4   # not 16-byte aligned


@pytest.mark.parametrize("M,N,K,bits,gs,want", [
    (0, 64, 256, 4, 64, q.EINVAL),        # M < 1
    (17, 64, 256, 4, 64, q.EINVAL),       # M > 16
    (1, 0, 256, 4, 64, q.EINVAL),         # N < 1
    (1, 64, 0, 4, 64, q.EINVAL),          # K < 64
    (1, 64, 96, 4, 32, q.EINVAL),         # K % 64 != 0
    (1, 64, 192, 4, 128, q.EINVAL),       # K % gs != 0
    (1, 64, 256, 3, 64, q.EINVAL),        # bits
    (1, 64, 256, 6, 64, q.EINVAL),        # bits
    (1, 64, 256, 16, 64, q.EINVAL),       # bits
    (1, 64, 256, 4, 16, q.EINVAL),        # group size
    (1, 64, 256, 4, 256, q.EINVAL),       # group size
    (1, 64, 262144, 4, 64, q.EINVAL),     # K above the limit
])
def test_invalid_shapes_rejected(M, N, K, bits, gs, want):
    L = q.lib()
    assert L.qgemv_small(A, A, A, A, A, M, N, K, bits, gs, None) == want
    assert L.qgemv_select(M, N, K, bits, gs) == want
    for path in (q.PATH_AUTO, q.PATH_DOT, q.PATH_MFMA):
        assert L.qgemv_run_path(path, A, A, A, A, A, M, N, K, bits, gs, None) == want


@pytest.mark.parametrize("which", range(5))
def test_null_pointers_rejected(which):
    ptrs = [A] * 5
    ptrs[which] = None
    assert q.lib().qgemv_small(*ptrs, 4, 64, 256, 4, 64, None) == q.EINVAL


@pytest.mark.parametrize("which", range(5))
def test_misaligned_pointers_rejected(which):
    ptrs = [A] * 5
    ptrs[which] = MIS
    assert q.lib().qgemv_small(*ptrs, 4, 64, 256, 4, 64, None) == q.EALIGN


# ---------------------------------------------------------------- fused residual sum

@pytest.mark.parametrize("M,N,K,bits,gs,want", [
    (0, 64, 256, 4, 64, q.EINVAL), (17, 64, 256, 4, 64, q.EINVAL), (1, 64, 96, 4, 32, q.EINVAL),
    (1, 64, 256, 6, 64, q.EINVAL), (1, 64, 256, 4, 16, q.EINVAL),
])
def test_add_invalid_shapes_rejected(M, N, K, bits, gs, want):
    L = q.lib()
    B = A + (1 << 24)  # residual apart from y
    assert L.qgemv_small_add(A, A, A, A, B, A, M, N, K, bits, gs, None) == want
    for path in (q.PATH_AUTO, q.PATH_DOT, q.PATH_MFMA):
        assert L.qgemv_run_path_add(path, A, A, A, A, B, A, M, N, K, bits, gs, None) == want


@pytest.mark.parametrize("which", range(6))
def test_add_null_and_misaligned_pointers_rejected(which):
    L = q.lib()
    ptrs = [A, A, A, A, A + (1 << 24), A]
    ptrs[which] = None
    assert L.qgemv_small_add(*ptrs, 4, 64, 256, 4, 64, None) == q.EINVAL
    ptrs = [A, A, A, A, A + (1 << 24), A]
    ptrs[which] = ptrs[which] + 4
    assert L.qgemv_small_add(*ptrs, 4, 64, 256, 4, 64, None) == q.EALIGN


def test_add_partially_overlapping_residual_rejected():
    L = q.lib()
    M, N = 4, 64
    row = N * 4
    # residual one row after y, or one row before: overlap, refused
    assert L.qgemv_small_add(A, A, A, A, A + row, A, M, N, 256, 4, 64, None) == q.EINVAL
    assert L.qgemv_small_add(A, A, A, A, A, A + row, M, N, 256, 4, 64, None) == q.EINVAL
    # an unknown path is refused before anything else
    assert L.qgemv_run_path_add(5, A, A, A, A, A, A, M, N, 256, 4, 64, None) == q.EINVAL


def test_unknown_path_rejected():
    L = q.lib()
    assert L.qgemv_run_path(3, A, A, A, A, A, 1, 64, 256, 4, 64, None) == q.EINVAL
    assert L.qgemv_run_path(-1, A, A, A, A, A, 1, 64, 256, 4, 64, None) == q.EINVAL
    assert L.qgemv_path_supported(7, 1, 64, 256, 4, 64) == q.EINVAL
    assert L.qgemv_unpack_probe(q.PATH_AUTO, A, A, 64, 256, 4, 64, None) == q.EINVAL


def test_mfma_path_shape_support():
    sup = q.qgemv_path_supported
    assert sup("mfma", 4, 4096, 4096, 4, 64)
    assert sup("mfma", 4, 4096, 4096, 2, 64)
    assert not sup("mfma", 4, 4096, 4096, 2, 32)   # 2-bit gs32: dot path only
    assert not sup("mfma", 4, 4096, 192, 4, 32)     # K not a multiple of 128
    assert sup("mfma", 4, 4096, 640, 4, 128)        # a partial last bias block (5 groups)
    assert not sup("mfma", 4, 4096, 384, 4, 128)    # fewer than 4 groups
    assert sup("dot", 4, 4096, 192, 4, 32)
    assert sup("mfma", 4, 4096, 4096, 8, 32) and sup("mfma", 4, 4096, 4096, 8, 64)
    assert sup("mfma", 4, 4096, 4096, 8, 128) and sup("dot", 4, 4096, 4096, 8, 128)
    assert not sup("mfma", 4, 4096, 4352, 8, 128)   # K not a multiple of 4*gs
    # a forced path that cannot run the shape is refused before launch
    assert q.lib().qgemv_run_path(q.PATH_MFMA, A, A, A, A, A, 4, 64, 192, 4, 32, None) == q.EUNSUPPORTED


def test_select_returns_a_supported_path_everywhere():
    for bits in (2, 4, 8):
        for gs in (32, 64, 128):
            for K in (256, 640, 4096, 5120, 17408):
                if K % gs:
                    continue
                for M in range(1, 17):
                    p = q.qgemv_select(M, 4096, K, bits, gs)
                    assert p in (q.PATH_DOT, q.PATH_MFMA)
                    assert q.qgemv_path_supported(p, M, 4096, K, bits, gs)


def test_select_keeps_the_dot_path_below_four_rows_on_partial_blocks():
    # K with a partial last bias block (11008 = 86 groups of 128): only the
    # single-pass MFMA kernel takes it, so the dot path up to M = 3; whole
    # blocks (11264 = 88 groups) follow the measured table
    for K, bits in ((11008, 4), (8960, 4), (11008, 2)):
        for M in range(1, 17):
            p = q.qgemv_select(M, 4096, K, bits, 128)
            if M < 4:
                assert p == q.PATH_DOT, (K, bits, M)
            assert q.qgemv_path_supported(p, M, 4096, K, bits, 128)
    assert any(q.qgemv_select(M, 4096, 11264, 4, 128) == q.PATH_MFMA for M in (2, 3))


def test_stream_probe_validation():
    L = q.lib()
    assert L.qgemv_stream_probe(None, 1024, A, 4, 0, None) == q.EINVAL
    assert L.qgemv_stream_probe(A, 1000, A, 4, 0, None) == q.EINVAL
    assert L.qgemv_stream_probe(A, 0, A, 4, 0, None) == q.EINVAL
    for bad in (0, 3, 32):
        assert L.qgemv_stream_probe(A, 1024, A, bad, 0, None) == q.EINVAL
    for bad in (-1, 2):
        assert L.qgemv_stream_probe(A, 1024, A, 4, bad, None) == q.EINVAL
    assert L.qgemv_stream_probe(MIS, 1024, A, 4, 1, None) == q.EALIGN
    assert 1 <= q.qgemv_stream_probe_blocks(16) <= q.qgemv_stream_probe_blocks(1 << 30)


def test_strerror_and_version():
    for s in (q.OK, q.EINVAL, q.EUNSUPPORTED, q.EALIGN, q.EHIP, -99):
        assert isinstance(q.qgemv_strerror(s), str) and q.qgemv_strerror(s)
    assert q.qgemv_version() >= 100


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(q, "_lib", None)
    monkeypatch.setattr(q, "LIB_PATH", "/nonexistent/libqgemv.so")
    with pytest.raises(RuntimeError):
        q.qgemv_version()


def test_product_path_does_not_import_oracle():
    import ast
    pkg = os.path.dirname(q.__file__)
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            tree = ast.parse(open(os.path.join(pkg, fn)).read())
            for node in ast.walk(tree):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                    assert not any(m.split(".")[0] == "oracle" for m in mods), fn


# ---------------------------------------------------------------- FP block formats

@pytest.mark.parametrize("M,N,K,fmt,want", [
    (1, 64, 256, 0, q.EINVAL), (1, 64, 256, 4, q.EINVAL),        # unknown format
    (0, 64, 256, 1, q.EINVAL), (17, 64, 256, 1, q.EINVAL),        # M
    (1, 0, 256, 1, q.EINVAL), (1, 64, 96, 1, q.EINVAL),           # N, K % 64
    (1, 64, q.MAX_K + 64, 3, q.EINVAL),                           # K above the limit
])
def test_fp_invalid_shapes_rejected(M, N, K, fmt, want):
    L = q.lib()
    assert L.qgemv_small_fp(A, A, A, None, A, M, N, K, fmt, None) == want
    assert L.qgemv_select_fp(M, N, K, fmt) == want
    for path in (q.PATH_AUTO, q.PATH_DOT, q.PATH_MFMA):
        assert L.qgemv_run_path_fp(path, A, A, A, None, A, M, N, K, fmt, None) == want


@pytest.mark.parametrize("which", range(4))
def test_fp_null_and_misaligned_pointers_rejected(which):
    L = q.lib()
    ptrs = [A, A, A, A]  # codes, scales, x, y (residual NULL)
    ptrs[which] = None
    args = ptrs[:3] + [None] + ptrs[3:]
    assert L.qgemv_small_fp(*args, 4, 64, 256, q.FMT_MXFP4, None) == q.EINVAL
    ptrs = [A, A, A, A]
    ptrs[which] += 4
    args = ptrs[:3] + [None] + ptrs[3:]
    assert L.qgemv_small_fp(*args, 4, 64, 256, q.FMT_MXFP4, None) == q.EALIGN


def test_fp_residual_overlap_and_alignment():
    L = q.lib()
    M, N = 4, 64
    assert L.qgemv_small_fp(A, A, A, A + N * 4, A, M, N, 256, q.FMT_MXFP8, None) == q.EINVAL
    assert L.qgemv_small_fp(A, A, A, A + (1 << 24) + 4, A, M, N, 256, q.FMT_MXFP8, None) == q.EALIGN


def test_fp_path_support():
    sup = q.qgemv_path_supported_fp
    for fmt in ("mxfp4", "nvfp4", "mxfp8"):
        assert sup("mfma", 4, 4096, 4096, fmt)
        assert not sup("mfma", 4, 4096, 192, fmt)       # K not a multiple of 128
    assert sup("dot", 4, 4096, 192, "nvfp4") and sup("dot", 4, 4096, 192, "mxfp8")
    for fmt in ("mxfp4", "nvfp4", "mxfp8"):
        for M in range(1, 17):
            p = q.qgemv_select_fp(M, 15360, 3840, fmt)
            assert p in (q.PATH_DOT, q.PATH_MFMA) and sup(p, M, 15360, 3840, fmt)
    assert q.lib().qgemv_unpack_probe_fp(q.PATH_MFMA, A, A, 64, 192, q.FMT_NVFP4, None) == q.EUNSUPPORTED


# ---------------------------------------------------------------- gathered (MoE) verify

def test_gather_validation():
    L = q.lib()
    g = L.qgemv_gather
    ok = dict(P=8, X=2, E=16, N=64, K=256, bits=4, gs=64)

    def call(**kw):
        a = dict(ok, **kw)
        ptrs = kw.pop("ptrs", None) or [A, A, A, A, A, A, A]
        return g(*ptrs, a["P"], a["X"], a["E"], a["N"], a["K"], a["bits"], a["gs"], None)

    assert call(P=0) == q.EINVAL and call(P=q.MAX_PAIRS + 1) == q.EINVAL
    assert call(E=0) == q.EINVAL and call(E=q.MAX_EXPERTS + 1) == q.EINVAL
    assert call(X=0) == q.EINVAL
    assert call(bits=3) == q.EINVAL and call(K=96) == q.EINVAL
    assert call(K=192, gs=32) == q.EUNSUPPORTED  # K not a multiple of 128: no MFMA path
    assert call(bits=2, gs=32) == q.EUNSUPPORTED
    for i in range(7):
        ptrs = [A] * 7
        ptrs[i] = None
        assert g(*ptrs, 8, 2, 16, 64, 256, 4, 64, None) == q.EINVAL
    ptrs = [A] * 7
    ptrs[4] = A + 2  # x_idx not 4-byte aligned
    assert g(*ptrs, 8, 2, 16, 64, 256, 4, 64, None) == q.EALIGN
