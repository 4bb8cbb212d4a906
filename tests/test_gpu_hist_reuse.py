"""The histogram forward's row counts reused by the histogram backward
(tbe_forward_preprocess with TBE_FWD_SAVE_HIST, then
TBE_BWD_HIST | TBE_BWD_PREPROCESSED): the forward matches the oracle, the
backward is bit-identical to the histogram backward that reads the indices
and within the oracle's tolerances, counts saved for another batch are not
used, and shapes the histogram paths do not serve are refused."""
import numpy as np
import pytest
import torch

import tbe_workloads as wl
from tests import support as S
from tests.test_gpu_parity import _announce, _spec, _tables_bytes

pytestmark = pytest.mark.gpu


def _reuse_spec(name):
    if name == "c4":
        return wl.config("C4", B=2048)
    if name == "mean_long_bags":
        # bags past the 256 counted lookups (counted by the remainder path), mean
        return wl.Spec("mean_long_bags", 2021, [50], [96], [1], "f16", 300, "uniform:64:700",
                       "uniform", "i64", False)
    if name == "mean_empty_bags":
        # empty bags next to long ones under mean pooling (average length above 64)
        return wl.Spec("mean_empty_bags", 2023, [64], [128], [1], "f16", 700,
                       "list:0,130,0,200,64,0,120,1", "uniform", "i64", False)
    if name == "e33_d64_i32":
        return wl.Spec("e33_d64_i32", 2022, [33], [64], [0], "f16", 5000, "poisson:70:+1",
                       "zipf:1.1", "i32", False)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["c4", "mean_long_bags", "mean_empty_bags", "e33_d64_i32"])
def test_saved_histogram_reused_by_backward(name):
    import table_embedding_amd as te
    _announce(name, "saved histogram")
    case = S.Case(_reuse_spec(name), m_nonzero=True)
    spec = case.spec
    res = []
    for mode in ("indices", "saved"):
        case.reset_tables()
        tb = case.tbe()
        if mode == "saved":
            out = tb.forward_and_preprocess(spec.B, case.d_idx, case.d_off, None,
                                            flags=te.TBE_FWD_SAVE_HIST)
            flags = te.TBE_BWD_HIST | te.TBE_BWD_PREPROCESSED
        else:
            out = tb.forward(spec.B, case.d_idx, case.d_off, None)
            flags = te.TBE_BWD_HIST
        tb.backward(spec.B, case.d_idx, case.d_off, None, case.d_G, spec.lr, spec.eps,
                    flags=flags)
        torch.cuda.synchronize()
        S.check_forward(case, out)
        S.check_backward(case, tb)
        if mode == "saved":  # the saved counts: every bag's exact row counts, bit for bit
            v = te.tbe_workspace_views(tb.plan, spec.B, case.N)
            E = spec.rows[0]
            got = S.read_u32(tb._ws, v["hist_counts"], (spec.B * E + 1) // 2).view(np.uint16)
            want = np.zeros((spec.B, E), np.uint16)
            bag = np.repeat(np.arange(spec.B), np.diff(case.off.astype(np.int64)))
            np.add.at(want, (bag, case.idx.astype(np.int64)), 1)
            assert np.array_equal(got[:spec.B * E].reshape(spec.B, E), want), "saved counts"
        res.append(_tables_bytes(tb, spec.wdtype))
        tb.close()
    assert res[0] == res[1], "saved counts give other bits than the indices"


def test_counts_of_another_batch_are_not_used():
    """Counts saved for a batch of other size stay unused: the backward reads
    the indices (bit-identical to the plain histogram backward)."""
    import table_embedding_amd as te
    case = S.Case(_reuse_spec("c4"), m_nonzero=True)
    other = S.Case(wl.config("C4", B=1024))
    spec = case.spec
    tb = case.tbe()
    ws = tb.workspace(spec.B, case.N)
    te.tbe_forward_preprocess(tb.plan, other.spec.B, other.d_idx, other.d_off, other.N, None,
                              torch.empty((other.spec.B, 128), device="cuda"), ws,
                              te.TBE_FWD_SAVE_HIST)
    tb.backward(spec.B, case.d_idx, case.d_off, None, case.d_G, spec.lr, spec.eps,
                flags=te.TBE_BWD_HIST | te.TBE_BWD_PREPROCESSED)
    torch.cuda.synchronize()
    a = _tables_bytes(tb, spec.wdtype)
    tb.close()
    case.reset_tables()
    tb = case.tbe()
    tb.backward(spec.B, case.d_idx, case.d_off, None, case.d_G, spec.lr, spec.eps,
                flags=te.TBE_BWD_HIST)
    torch.cuda.synchronize()
    assert _tables_bytes(tb, spec.wdtype) == a
    S.check_backward(case, tb)
    tb.close()


def test_save_hist_refused_where_it_does_not_apply():
    import table_embedding_amd as te
    for name in ("C2s", "C3s"):   # many tables / per-sample weights
        case = S.Case(_spec(name))
        tb = case.tbe()
        with pytest.raises(te.TBEError) as ei:
            tb.forward_and_preprocess(case.spec.B, case.d_idx, case.d_off, case.d_psw,
                                      flags=te.TBE_FWD_SAVE_HIST)
        assert ei.value.code == te.TBE_E_UNSUPPORTED
        tb.close()
    with pytest.raises(te.TBEError) as ei:  # the plain forward has no workspace to save into
        case = S.Case(_reuse_spec("c4"))
        tb = case.tbe()
        tb.forward(case.spec.B, case.d_idx, case.d_off, None, flags=te.TBE_FWD_SAVE_HIST)
    assert ei.value.code == te.TBE_E_ARG
    torch.cuda.synchronize()
