"""bench.py's byte model: the per-kernel attribution of the algorithmic
(each stream and unique row once) and logical bytes sums exactly to the
step totals of its documented formulas, and those totals equal the formulas
written out independently here on a tiny hand-checked problem."""
import numpy as np

import bench
import tbe_workloads as wl

BWD_KERNELS = ("tile_map", "transpose", "radix_upsweep", "radix_scan", "radix_downsweep", "rle", "classify",
               "chunk_order", "bwd_single", "bwd_tiny", "bwd_medium", "bwd_chunk",
               "bwd_long_update", "dense_select", "dense_partial", "dense_update")


def _model(spec):
    off, idx = spec.offsets(), spec.indices()
    st = bench.workload_stats(spec, off, idx)
    return st, bench.byte_model(spec, st)


def test_attribution_sums_to_the_step_totals():
    for spec in (wl.config("C2", rows=20000, B=512, T=4), wl.config("C3", rows=50000, B=256, T=10),
                 wl.config("C5", rows=200000, B=2048, T=3), wl.config("C1")):
        st, (comp, logi, tot) = _model(spec)
        assert comp["fwd_pool"] == tot["fwd_comp"]
        assert logi["fwd_pool"] == tot["fwd_logi"]
        assert abs(sum(comp[k] for k in BWD_KERNELS) - tot["bwd_comp"]) < 1e-6 * tot["bwd_comp"]
        assert abs(sum(logi[k] for k in BWD_KERNELS) - tot["bwd_logi"]) < 1e-6 * tot["bwd_logi"]
        assert comp["bwd_chunk_fused"] == comp["bwd_chunk"] + comp["bwd_long_update"]


def test_totals_on_a_hand_checked_problem():
    """One table of 10 rows x D 8 fp16, B = 2, int64, no weights; bags
    [3, 0, 1] and [0, 0]: N = 5 lookups of U = 3 rows (row 0 three times,
    rows 1 and 3 once)."""
    spec = wl.Spec("hand", 1, [10], [8], [0], "f16", 2, "list:3,2", "const:3", "i64", False)
    off = spec.offsets()
    assert list(off) == [0, 3, 5]
    idx = np.array([3, 0, 1, 0, 0], np.int64)
    st = bench.workload_stats(spec, off, idx)
    comp, logi, tot = bench.byte_model(spec, st)
    N, U, si, sw, D, TB1, B = 5, 3, 8, 2, 8, 3, 2
    # forward: indices, offsets, each unique row once, the output
    assert tot["fwd_comp"] == N * si + TB1 * si + U * D * sw + B * D * 4
    assert tot["fwd_logi"] == N * si + TB1 * si + N * D * sw + B * D * 4
    # backward: 16 B of key/bag traffic per lookup, 24 B + a row read and
    # written per run, grad_out once (compulsory) or per lookup (logical)
    assert tot["bwd_comp"] == N * (si + 16) + TB1 * si + U * (2 * D * sw + 24) + B * D * 4
    assert tot["bwd_logi"] == N * (si + 16) + TB1 * si + U * (2 * D * sw + 24) + N * 4 * D
    # run classes: row 0 three times (tiny), rows 1 and 3 once (single)
    assert st[0]["n_single"] == 2 and st[0]["n_tiny"] == 1 and st[0]["N_tiny"] == 3


def test_hot_runs_move_between_kernels_not_out_of_the_step(monkeypatch):
    """With the hot-row contraction in force (its lookup threshold lowered to
    this small batch), the long runs it takes are attributed to it and the
    step totals are unchanged; the hot rows are the longest long runs, at
    most 128 per table."""
    spec = wl.config("C5", rows=200000, B=2048, T=3)
    st0, (comp0, logi0, tot0) = _model(spec)
    assert all(s["n_hot"] == 0 for s in st0)
    monkeypatch.setattr(bench, "DENSE_MIN_LOOKUPS", 0)
    st, (comp, logi, tot) = _model(spec)
    assert tot == tot0
    assert abs(sum(comp[k] for k in BWD_KERNELS) - tot["bwd_comp"]) < 1e-6 * tot["bwd_comp"]
    assert abs(sum(logi[k] for k in BWD_KERNELS) - tot["bwd_logi"]) < 1e-6 * tot["bwd_logi"]
    for s in st:
        assert 0 < s["n_hot"] <= min(128, s["n_long"]) and s["N_hot"] <= s["N_long"]
    assert comp["dense_partial"] > 0 and comp["bwd_chunk"] < comp0["bwd_chunk"]
    moved = comp["dense_partial"] + comp["bwd_chunk"]
    assert abs(moved - comp0["bwd_chunk"]) < 1e-9 * comp0["bwd_chunk"]
