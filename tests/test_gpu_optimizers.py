"""Optimizer epilogue variants of the backward (tbe_backward): element-wise
Adagrad (HugeCTR walkthrough, step 5) and SGD on the same run pipeline, against
the oracle.  Bars: weights within 2 storage ulp (float32: 1e-6 max(1,|ref|)),
element-wise state within 1e-5 of its scale A_ref + gabs^2 (gabs[d]: the sum
of the absolute contributions to the entry's gradient; one entry's gradient
may cancel to far below its terms, and float32 summation errors scale with
the terms, not with the sum), untouched rows and their state
bit-identical, every touched row updated once, fused and two-launch long-run
paths bit-identical."""
import numpy as np
import pytest
import torch

import oracle
from tests import support as S
from tests.test_gpu_parity import _spec, _announce

pytestmark = pytest.mark.gpu

CASES = ["C1", "C2s", "C3s", "C5s", "empty_bags", "one_bag", "const257", "wide_f32", "wide_bf16",
         "many_tables"]


def _state0(spec, optimizer):
    if optimizer == "sgd":
        return [np.zeros(r, np.float32) for r in spec.rows]
    rng = np.random.default_rng(99)
    return [(np.abs(rng.standard_normal((r, d))) * 0.01).astype(np.float32)
            for r, d in zip(spec.rows, spec.dims)]


def _gabs(case, t):
    """Per entry of table t: sum over its lookups of |S[p] (1/L if mean) G[j, d]|."""
    spec = case.spec
    B, off, idx = spec.B, case.off, case.idx
    col = spec.col_offsets()[t]
    D = spec.dims[t]
    out = np.zeros((spec.rows[t], D), np.float64)
    lo, hi = int(off[t * B]), int(off[(t + 1) * B])
    if hi == lo:
        return out
    p = np.arange(lo, hi)
    j = np.searchsorted(off, p, side="right") - 1
    s = np.ones(len(p)) if case.psw is None else np.abs(case.psw[p].astype(np.float64))
    if spec.pooling[t] == 1:
        s = s / (off[j + 1] - off[j]).astype(np.float64)
    contrib = s[:, None] * np.abs(case.G[j - t * B, col:col + D].astype(np.float64))
    np.add.at(out, idx[p].astype(np.int64), contrib)
    return out


def epilogue_weights_ok(Wg, Wref, W0, wdtype, optimizer, lr, gabs, Aref=None):
    """Weights after the SGD or element-wise Adagrad epilogue.  16-bit: 2 ulp at
    operand scale (as for row-wise Adagrad on bfloat16).  float32: 1e-6 max(1,
    |ref|) plus the float32 summation bound of the gradient carried through
    the step: a row gradient is a float32 sum of every contribution, good to
    about 1e-6 of the sum of their magnitudes (gabs), and neither epilogue
    normalizes it away (SGD moves the weight by lr * g; element-wise Adagrad
    by lr * g / sqrt(A), whose error is at most lr * dg / sqrt(A))."""
    if wdtype != "f32":
        return S.weights_ok(Wg, Wref, wdtype, W0, literal_f16=False)
    a = Wg.view(np.float32).astype(np.float64)
    b = Wref.view(np.float32).astype(np.float64)
    step = lr * 1e-6 * gabs
    if optimizer == "adagrad":
        step = step / np.sqrt(np.maximum(Aref.astype(np.float64), 1e-30))
    v = np.abs(a - b) / (1e-6 * np.maximum(1.0, np.abs(b)) + step)
    worst = float(v.max(initial=0.0))
    return worst <= 1.0, worst


def _run(case, optimizer, flags=0):
    import table_embedding_amd as te
    spec = case.spec
    A0 = _state0(spec, optimizer)
    d_W = [S.from_host_storage(w, spec.wdtype) for w in case.W]
    d_A = [torch.from_numpy(a.copy()).cuda() for a in A0]
    tb = te.TBE(spec.rows, spec.dims, spec.pooling, d_W, d_A)
    dbg = torch.zeros(sum(spec.rows), dtype=torch.uint32, device="cuda")
    code = {"adagrad": te.TBE_OPT_ADAGRAD, "sgd": te.TBE_OPT_SGD}[optimizer]
    tb.backward(spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, spec.lr, spec.eps,
                flags=flags, debug_row_updates=dbg, optimizer=code)
    torch.cuda.synchronize()
    W = [S.to_host_storage(w, spec.wdtype).reshape(r, d)
         for w, r, d in zip(tb.weights, spec.rows, spec.dims)]
    A = [a.cpu().numpy() for a in d_A]
    kb = tb.key_bases()
    c = dbg.cpu().numpy()
    tb.close()
    return W, A, A0, [c[kb[t]:kb[t] + spec.rows[t]] for t in range(spec.T)]


@pytest.mark.parametrize("name", CASES)
@pytest.mark.parametrize("optimizer", ["adagrad", "sgd"])
def test_optimizer_parity(name, optimizer):
    _announce(name, f"optimizer {optimizer}")
    case = S.Case(_spec(name))
    spec = case.spec
    if case.N == 0:
        pytest.skip("no lookups")
    W, A, A0, cnt = _run(case, optimizer)
    Wr = [w.copy() for w in case.W]
    Ar = [a.copy() for a in A0]
    oracle.backward(spec.rows, spec.dims, spec.pooling, spec.wdtype, Wr,
                    Ar if optimizer == "adagrad" else None, spec.B, spec.itype, case.idx,
                    case.off, case.psw, case.G, spec.lr, spec.eps, optimizer=optimizer)
    for t in range(spec.T):
        rows = S.touched_rows(case, t)
        mask = np.zeros(spec.rows[t], bool)
        mask[rows] = True
        W0 = case.W[t].reshape(spec.rows[t], spec.dims[t])
        Wref = Wr[t].reshape(spec.rows[t], spec.dims[t])
        assert W[t][~mask].tobytes() == W0[~mask].tobytes(), f"table {t}: untouched rows"
        ok, v = epilogue_weights_ok(W[t][mask], Wref[mask], W0[mask], spec.wdtype, optimizer,
                                    spec.lr, _gabs(case, t)[mask],
                                    Ar[t][mask] if optimizer == "adagrad" else None)
        assert ok, f"table {t}: weight tolerance exceeded ({v})"
        assert A[t][~mask].tobytes() == A0[t][~mask].tobytes(), f"table {t}: untouched state"
        if optimizer == "adagrad":
            scale = Ar[t][mask].astype(np.float64) + _gabs(case, t)[mask] ** 2
            rel = np.abs(A[t][mask].astype(np.float64) - Ar[t][mask]) / scale
            assert float(rel.max(initial=0.0)) <= 1e-5, f"table {t}: state error {rel.max()}"
        else:
            assert A[t].tobytes() == A0[t].tobytes(), "SGD touched the state buffer"
        want = np.zeros(spec.rows[t], np.int32)
        want[rows] = 1
        assert np.array_equal(cnt[t], want), f"table {t}: each touched row once"


@pytest.mark.parametrize("name", ["C3s", "C5s", "const257"])
@pytest.mark.parametrize("optimizer", ["adagrad", "sgd"])
def test_optimizer_fused_equals_two_launch(name, optimizer):
    import table_embedding_amd as te
    case = S.Case(_spec(name))
    a = _run(case, optimizer)
    b = _run(case, optimizer, te.TBE_BWD_FUSED_LONG)
    for t in range(case.spec.T):
        assert a[0][t].tobytes() == b[0][t].tobytes()
        assert a[1][t].tobytes() == b[1][t].tobytes()


def test_unknown_optimizer_refused():
    import table_embedding_amd as te
    case = S.Case(_spec("C1"))
    tb = case.tbe()
    with pytest.raises(te.TBEError) as ei:
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, 0.01, 1e-8,
                    optimizer=7)
    assert ei.value.code == te.TBE_E_ARG
    tb.close()
