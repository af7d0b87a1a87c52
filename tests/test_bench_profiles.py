"""The profile summariser's assignment of traced dispatches to workloads (CPU)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _d(names):
    return [{"name": n, "ns": i} for i, n in enumerate(names)]


def test_match_skips_input_building_dispatches():
    order = [{"name": "a", "kernels": [("prefill_kernel", 1)], "reps": 2},
             {"name": "b", "kernels": [("zero_kernel", 2), ("rows_kernel", 1)], "reps": 2}]
    names = ["normal_kernel", "compress_kernel", "prefill_kernel<0>", "prefill_kernel<0>",
             "normal_kernel", "prefill_kernel<lse>",  # building b: not b's kernels
             "zero_kernel", "zero_kernel", "rows_kernel", "zero_kernel", "zero_kernel",
             "rows_kernel", "fill", "copy"]
    m = bench._match(_d(names), order)
    assert [[d["ns"] for d in l] for l in m["a"]] == [[2], [3]]
    assert [[d["ns"] for d in l] for l in m["b"]] == [[6, 7, 8], [9, 10, 11]]
    assert m["copy"][0][0]["name"] == "copy"


def test_match_needs_the_whole_run_of_launches():
    # a lone match of the first kernel (a build step) is skipped for the full run
    order = [{"name": "b", "kernels": [("zero_kernel", 1), ("rows_kernel", 1)], "reps": 1}]
    m = bench._match(_d(["zero_kernel", "x", "zero_kernel", "rows_kernel", "copy"]), order)
    assert [d["ns"] for d in m["b"][0]] == [2, 3]


def test_match_reports_missing_launches():
    order = [{"name": "a", "kernels": [("gate_kernel", 1)], "reps": 1}]
    with pytest.raises(SystemExit):
        bench._match(_d(["prefill_kernel", "copy"]), order)


def test_match_leaves_out_warm_up_launches():
    order = [{"name": "a", "kernels": [("gate_kernel", 1)], "reps": 2, "warm": 1}]
    m = bench._match(_d(["x", "gate_kernel", "gate_kernel", "gate_kernel", "copy"]), order)
    assert [[d["ns"] for d in l] for l in m["a"]] == [[2], [3]]


def test_copy_probe_library_exports_its_entry_point():
    """The copy-path probe behind bench.py --copy-rate is built and loadable (no
    GPU call here)."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "long_context_compressed_hca_amd", "libhca_probe.so")
    assert os.path.exists(path), "build() makes libhca_probe.so"
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "hca_probe_copy_rate")


def test_parity_figures_flag_a_planted_error():
    """The bench line's parity figures: exact rows pass, one row off by 5e-2 fails
    on max-abs and is named as the worst row."""
    import numpy as np
    import bench
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((4, 8, 512))
    ok = bench.parity_figures(ref.copy(), ref)
    assert ok["pass"] and ok["rel_l2"] == 0.0 and ok["rows"] == 32
    bad = ref.copy()
    bad[2, 3, 7] += 5e-2
    f = bench.parity_figures(bad, ref)
    assert not f["pass"] and abs(f["max_abs"] - 5e-2) < 1e-12
    assert f["worst_row_rel_l2"] > 1e-3
