"""tbe_backward_rowwise_adagrad_noalloc (the library's static workspace, for
callers that cannot allocate) against tbe_backward_rowwise_adagrad with a
caller workspace, through the C ABI: two calls in a row on one device, the
second on a smaller batch, each giving bit-identical weights, momentum and
debug counters, and both within the oracle's tolerances.  Batches beyond the
static workspace and a preprocessed flag are refused on the host."""
import numpy as np
import pytest
import torch

import tbe_workloads as wl
from tests import support as S

pytestmark = pytest.mark.gpu


def _step(case, noalloc):
    import table_embedding_amd as te
    case.reset_tables()
    tb = case.tbe()
    spec = case.spec
    dbg = torch.zeros(sum(spec.rows), dtype=torch.uint32, device="cuda")
    if noalloc:
        te.tbe_backward_rowwise_adagrad_noalloc(tb.plan, spec.B, case.d_idx, case.d_off, case.N,
                                                case.d_psw, case.d_G, spec.lr, spec.eps, 0, dbg)
    else:
        ws = tb.workspace(spec.B, case.N)
        te.tbe_backward_rowwise_adagrad(tb.plan, spec.B, case.d_idx, case.d_off, case.N,
                                        case.d_psw, case.d_G, spec.lr, spec.eps, ws, 0, dbg)
    torch.cuda.synchronize()
    W = [S.to_host_storage(w, spec.wdtype) for w in tb.weights]
    M = [m.cpu().numpy() for m in tb.momentum]
    return tb, W, M, dbg.cpu().numpy()


def test_noalloc_equals_workspace_backward_twice():
    import table_embedding_amd as te
    # the first batch (every D bucket, mean and sum, per-sample weights, long
    # runs) is larger than the second, which then runs over the first's leftovers
    specs = [wl.config("C3", rows=50000, B=256, T=10), wl.config("C2", rows=20000, B=128, T=4)]
    sizes = []
    for spec in specs:
        case = S.Case(spec, m_nonzero=True)
        print(f"[gpu] no-alloc backward {spec.name}: {case.N} lookups", flush=True)
        sizes.append(case.N)
        tb = case.tbe()
        assert te.tbe_workspace_size(tb.plan, spec.B, case.N) <= te.TBE_STATIC_WS_BYTES
        tb.close()
        tb_ref, W_ref, M_ref, c_ref = _step(case, noalloc=False)
        tb_ref.close()
        tb_na, W_na, M_na, c_na = _step(case, noalloc=True)
        for t in range(spec.T):
            assert W_na[t].tobytes() == W_ref[t].tobytes(), f"table {t}: weights differ"
            assert M_na[t].tobytes() == M_ref[t].tobytes(), f"table {t}: momentum differs"
        assert np.array_equal(c_na, c_ref), "debug counters differ"
        S.check_backward(case, tb_na)
        tb_na.close()
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_what_it_cannot_serve():
    import table_embedding_amd as te
    spec = wl.config("C2", rows=20000, B=128, T=4)
    case = S.Case(spec)
    tb = case.tbe()
    # a preprocessed workspace cannot be handed in
    with pytest.raises(te.TBEError) as e:
        te.tbe_backward_rowwise_adagrad_noalloc(tb.plan, spec.B, case.d_idx, case.d_off, case.N,
                                                None, case.d_G, spec.lr, spec.eps,
                                                te.TBE_BWD_PREPROCESSED)
    assert e.value.code == te.TBE_E_ARG
    # a batch whose workspace exceeds the static array is refused on the host,
    # before anything is enqueued (the claimed count is never read on the device)
    big = 1
    while te.tbe_workspace_size(tb.plan, spec.B, big) <= te.TBE_STATIC_WS_BYTES:
        big *= 2
    with pytest.raises(te.TBEError) as e:
        te.tbe_backward_rowwise_adagrad_noalloc(tb.plan, spec.B, case.d_idx, case.d_off, big,
                                                None, case.d_G, spec.lr, spec.eps)
    assert e.value.code == te.TBE_E_TOO_LARGE
    # the hot-row contraction starts at 8 Mi lookups, past what the array holds
    assert big <= 8 << 20
    assert te.tbe_workspace_size(tb.plan, 1, 8 << 20) > te.TBE_STATIC_WS_BYTES
    torch.cuda.synchronize()
    tb.close()
