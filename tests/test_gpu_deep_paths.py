"""The variants the library picks for deep batches (64 Mi lookups and more:
backward gathers with eight lookups in flight and non-temporal weight rows;
8 Mi and more: run-length tiles of four 4096-key groups; 1 Mi and more:
non-temporal rows alone), run at scaled sizes through the test knobs and compared with the
oracle like every other case: integer outputs of the preprocessing bit for
bit, weights and momentum within tolerance, fused = two-launch bit for bit.

Also the contract of a look-back wait that gives up: with the poll limit
forced to 0 from the host (every kernel still exits normally), the
preprocessing flags its error word and the backward writes nothing."""
import contextlib

import numpy as np
import pytest
import torch

from tests import support as S
from tests.test_gpu_parity import _announce, _spec, _tables_bytes

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def knobs(**kv):
    import table_embedding_amd as te
    names = {"rle_deep": te.TBE_KNOB_RLE_DEEP_LOOKUPS, "bwd_deep": te.TBE_KNOB_BWD_DEEP_LOOKUPS,
             "bwd_stream": te.TBE_KNOB_BWD_STREAM_LOOKUPS, "polls": te.TBE_KNOB_WAIT_POLLS,
             "dense": te.TBE_KNOB_DENSE_LOOKUPS}
    try:
        for k, v in kv.items():
            te.tbe_test_knob(names[k], v)
        yield
    finally:
        for k in names.values():
            te.tbe_test_knob(k, -1)


DEEP = ["C2s", "C3s", "C5s", "many_tables", "const257", "heavy_chunks", "wide_f32", "cut_bags",
        "dense_mean", "dense_many", "dense_half", "dense_wide"]


def _takes_dense(spec):
    """The backward takes the hot-row contraction (when its lookup threshold
    is met) for batches without per-sample weights on plans of at most 128
    tables with a table whose D is a multiple of 16 and at most 256."""
    return (not spec.weighted and spec.T <= 128
            and any(d % 16 == 0 and d <= 256 for d in spec.dims))


VARIANTS = {"deep": dict(rle_deep=0, bwd_deep=0, dense=1 << 40), "stream": dict(bwd_stream=0),
            "dense": dict(dense=0), "dense_deep": dict(rle_deep=0, bwd_deep=0, dense=0),
            "no_dense": dict(dense=1 << 40)}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", DEEP)
def test_deep_batch_variants_parity(name, variant):
    """Each variant at scaled sizes: "dense" runs the hot-row contraction of
    the long runs (which deep batches take from 8 Mi lookups on), "no_dense"
    keeps every long run on the chunk path."""
    import table_embedding_amd as te
    _announce(name, f"{variant} variants")
    kv = VARIANTS[variant]
    case = S.Case(_spec(name), m_nonzero=True)
    with knobs(**kv):
        tb = case.tbe()
        tb.preprocess(case.spec.B, case.d_idx, case.d_off, case.d_psw)
        torch.cuda.synchronize()
        S.check_preprocess(case, tb)
        tb.close()
        res = []
        for flags in (0, te.TBE_BWD_FUSED_LONG):
            case.reset_tables()
            tb = case.tbe()
            tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G,
                        case.spec.lr, case.spec.eps, flags=flags)
            torch.cuda.synchronize()
            if flags == 0:
                S.check_backward(case, tb)
            if kv.get("dense") == 0 and _takes_dense(case.spec):
                S.check_dense(case, tb)
            res.append(_tables_bytes(tb, case.spec.wdtype))
            tb.close()
        assert res[0] == res[1], "fused differs from two-launch"


@pytest.mark.parametrize("name", ["dense_many", "dense_mean"])
def test_dense_unaligned_indices_bitwise(name):
    """The contraction reads four lookups at once with 16-byte loads only when
    the indices are 16-byte aligned; indices one element off that alignment
    (legal: the boundary asks for element alignment) take element loads and
    give the same bits."""
    _announce(name, "dense, unaligned indices")
    case = S.Case(_spec(name), m_nonzero=True)
    spec = case.spec
    buf = torch.empty(case.N + 1, dtype=case.d_idx.dtype, device="cuda")
    buf[1:].copy_(case.d_idx)
    idx_u = buf[1:]
    assert idx_u.data_ptr() % 16 != 0 and idx_u.is_contiguous()
    res = []
    with knobs(dense=0):
        for idx in (case.d_idx, idx_u):
            case.reset_tables()
            tb = case.tbe()
            tb.backward(spec.B, idx, case.d_off, case.d_psw, case.d_G, spec.lr, spec.eps)
            torch.cuda.synchronize()
            res.append(_tables_bytes(tb, spec.wdtype))
            tb.close()
    assert res[0] == res[1], "unaligned indices changed the contraction's result"


@pytest.mark.parametrize("name", ["C2s", "C3s", "C5s"])
def test_wait_give_up_writes_nothing(name):
    """Poll limit 0: every tile with predecessors gives up its look-back at
    once; prep_error is set and neither the self-preprocessing backward nor
    one on the preprocessed workspace writes a weight, a momentum or a debug
    counter.  With the default limit restored the same inputs give the oracle's
    result."""
    import table_embedding_amd as te
    _announce(name, "look-back give-up")
    case = S.Case(_spec(name), m_nonzero=True)
    spec = case.spec
    assert case.N > 4096, "needs more than one run-length tile"
    W0 = [w.tobytes() for w in case.W]
    M0 = [m.tobytes() for m in case.M]
    with knobs(polls=0):
        for flags in (0, te.TBE_BWD_FUSED_LONG, te.TBE_BWD_PREPROCESSED):
            case.reset_tables()
            tb = case.tbe()
            if flags & te.TBE_BWD_PREPROCESSED:
                tb.preprocess(spec.B, case.d_idx, case.d_off, case.d_psw)
            dbg = torch.zeros(sum(spec.rows), dtype=torch.uint32, device="cuda")
            tb.backward(spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, spec.lr, spec.eps,
                        flags=flags, debug_row_updates=dbg)
            torch.cuda.synchronize()
            v = te.tbe_workspace_views(tb.plan, spec.B, case.N)
            assert int(S.read_u32(tb._ws, v["prep_error"], 1)[0]) != 0, "no give-up flagged"
            assert [S.to_host_storage(w, spec.wdtype).tobytes() for w in tb.weights] == W0
            assert [m.cpu().numpy().tobytes() for m in tb.momentum] == M0
            assert not dbg.cpu().numpy().any()
            tb.close()
    case.reset_tables()
    tb = case.tbe()
    tb.backward(spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, spec.lr, spec.eps)
    torch.cuda.synchronize()
    v = te.tbe_workspace_views(tb.plan, spec.B, case.N)
    assert int(S.read_u32(tb._ws, v["prep_error"], 1)[0]) == 0
    S.check_backward(case, tb)
    tb.close()


@pytest.mark.parametrize("name", ["dense_mean", "C5s", "heavy_chunks", "dense_wide"])
@pytest.mark.parametrize("optimizer", ["adagrad", "sgd"])
def test_dense_rows_with_other_optimizers(name, optimizer):
    """The hot rows' update takes the element-wise Adagrad and SGD epilogues
    too: against the oracle, each touched row once, fused = two-launch."""
    import oracle
    import table_embedding_amd as te
    from tests.test_gpu_optimizers import _gabs, _run, epilogue_weights_ok
    _announce(name, f"dense rows, {optimizer}")
    case = S.Case(_spec(name))
    spec = case.spec
    with knobs(dense=0):
        W, A, A0, cnt = _run(case, optimizer)
        Wf, Af, _, _ = _run(case, optimizer, te.TBE_BWD_FUSED_LONG)
    Wr = [w.copy() for w in case.W]
    Ar = [a.copy() for a in A0]
    oracle.backward(spec.rows, spec.dims, spec.pooling, spec.wdtype, Wr,
                    Ar if optimizer == "adagrad" else None, spec.B, spec.itype, case.idx,
                    case.off, case.psw, case.G, spec.lr, spec.eps, optimizer=optimizer)
    for t in range(spec.T):
        mask = np.zeros(spec.rows[t], bool)
        mask[S.touched_rows(case, t)] = True
        W0 = case.W[t].reshape(spec.rows[t], spec.dims[t])
        Aref = Ar[t][mask] if optimizer == "adagrad" else None
        ok, v = epilogue_weights_ok(W[t][mask], Wr[t].reshape(spec.rows[t], spec.dims[t])[mask],
                                    W0[mask], spec.wdtype, optimizer, spec.lr,
                                    _gabs(case, t)[mask], Aref)
        assert ok, f"table {t}: weight tolerance exceeded ({v})"
        assert np.array_equal(cnt[t], mask.astype(np.uint32)), f"table {t}: each touched row once"
        assert W[t].tobytes() == Wf[t].tobytes() and A[t].tobytes() == Af[t].tobytes()
