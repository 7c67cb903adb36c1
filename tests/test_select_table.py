"""The dispatcher table compiled into the library against the sweep it was
generated from (no GPU): the committed header is exactly what the generator
writes from the committed sweep, the sweep covers every workload at every M on
both paths, and the class rule reduces to a plain comparison where a class
holds one shape."""
import collections
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from few_row_quantized_amd import calibrate, synth  # noqa: E402

PKG = os.path.join(ROOT, "few_row_quantized_amd")
SWEEP = os.path.join(PKG, "calibration", "select_sweep.json")
HEADER = os.path.join(PKG, "csrc", "qgemv_select_table.h")


def _rows():
    with open(SWEEP) as f:
        return json.load(f)["rows"]


def test_header_is_generated_from_the_committed_sweep():
    src = os.path.relpath(SWEEP, ROOT)
    want = calibrate.emit_header(calibrate.table_from_sweep(_rows()), src)
    with open(HEADER) as f:
        assert f.read() == want


def test_sweep_covers_every_workload_at_every_m_on_both_paths():
    seen = collections.defaultdict(set)
    for r in _rows():
        assert r["dot_us"] > 0 and r["mfma_us"] > 0, r
        seen[r["workload"]].add(r["M"])
    for name in synth.WORKLOADS:
        if name.startswith("tiny"):
            continue
        assert seen[name] == set(range(1, 17)), name


def test_single_shape_classes_pick_the_faster_path():
    rows = _rows()
    key = lambda r: ((100 + calibrate.FP_CODES[r["fmt"]], 0) if "fmt" in r else
                     (r["bits"], r["group_size"])) + (calibrate.n_class(r["N"]),
                                                      calibrate.k_class(r["K"]))
    shapes = collections.defaultdict(set)
    for r in rows:
        shapes[key(r)].add((r["N"], r["K"]))
    table = calibrate.table_from_sweep(rows)
    checked = 0
    for r in rows:
        k = key(r)
        if len(shapes[k]) != 1:
            continue
        bit = (table[k] >> (r["M"] - 1)) & 1
        assert bit == (1 if r["mfma_us"] < r["dot_us"] else 0), (k, r["M"])
        checked += 1
    assert checked >= 16
