"""Input validation and repair (tbe_validate) on the GPU.

Valid workloads report nothing and stay untouched; planted contract breaks
(indices out of range, offsets out of order / out of range / wrong ends) are
reported with the right bits, count and first positions, computed here by a
plain numpy check of the contract; repair rewrites exactly what the header
says, and the forward over repaired indices matches the oracle.  Nothing but
the validation kernels ever reads the broken inputs.
"""
import numpy as np
import pytest
import torch

import tbe_workloads as wl
from tests import support as S
from tests.test_gpu_parity import _spec

pytestmark = pytest.mark.gpu
NONE = 0xFFFFFFFF


def _expect(spec, off, idx):
    """The error block a plain check of the contract gives."""
    import table_embedding_amd as te
    T, B = spec.T, spec.B
    N = len(idx)
    bits, bad, first_bag, first_pos = 0, 0, NONE, NONE
    # the start offset is bag 0's, the end offset the last bag's
    if off[0] != 0:
        bits |= te.TBE_INVALID_OFFSET_START
        first_bag = 0 if T * B else NONE
    if off[T * B] != N:
        bits |= te.TBE_INVALID_OFFSET_END
        first_bag = min(first_bag, T * B - 1) if T * B else NONE
    for j in range(T * B):
        lo, hi = int(off[j]), int(off[j + 1])
        f = 0
        if lo > hi:
            f |= te.TBE_INVALID_OFFSET_ORDER
        if lo < 0 or lo > N or hi < 0 or hi > N:
            f |= te.TBE_INVALID_OFFSET_RANGE
        if f:
            bits |= f
            first_bag = min(first_bag, j)
    # every index once, against the table whose (clamped) start offset is the
    # last one at or before its position
    starts = np.clip(off[0:T * B + 1:B][:T].astype(np.int64), 0, N)
    p = np.arange(N)
    t = np.clip(np.searchsorted(starts, p, side="right") - 1, 0, T - 1) if T else p * 0
    rows = np.asarray(spec.rows, np.int64)[t]
    r = idx.astype(np.int64)
    badp = np.nonzero((r < 0) | (r >= rows))[0]
    if len(badp):
        bits |= te.TBE_INVALID_INDEX
        bad = len(badp)
        first_pos = int(badp[0])
        tt = int(t[first_pos])
        seg = off[tt * B:tt * B + B].astype(np.int64)
        first_bag = min(first_bag, tt * B + int(np.searchsorted(seg, first_pos, side="right")) - 1)
    return [bits, bad, first_bag, first_pos]


def _run(spec, off, idx, flags=0):
    import table_embedding_amd as te
    tb = S.Case(spec).tbe()
    d_off = torch.from_numpy(off.copy()).cuda()
    d_idx = torch.from_numpy(idx.copy()).cuda()
    err = torch.zeros(te.TBE_VALIDATE_WORDS, dtype=torch.int32, device="cuda")
    te.tbe_validate(tb.plan, spec.B, d_idx, d_off, len(idx), err, flags)
    torch.cuda.synchronize()
    got = [int(x) & 0xFFFFFFFF for x in err.cpu().numpy()]
    out = (got, d_off.cpu().numpy(), d_idx.cpu().numpy())
    tb.close()
    return out


@pytest.mark.parametrize("name", ["C1", "C2s", "many_tables", "empty_bags", "all_empty", "one_row"])
def test_valid_inputs_report_nothing(name):
    import table_embedding_amd as te
    spec = _spec(name)
    off, idx = spec.offsets(), spec.indices()
    for flags in (0, te.TBE_VALIDATE_REPAIR):
        got, o2, i2 = _run(spec, off, idx, flags)
        assert got == [0, 0, NONE, NONE]
        assert np.array_equal(o2, off) and np.array_equal(i2, idx)


@pytest.mark.parametrize("name", ["C2s", "many_tables"])
def test_bad_indices_reported_and_repaired(name):
    import table_embedding_amd as te
    spec = _spec(name)
    off, idx = spec.offsets(), spec.indices().copy()
    rng = np.random.default_rng(7)
    pos = np.sort(rng.choice(len(idx), 37, replace=False))
    tab = np.searchsorted(off, pos, side="right") - 1
    tab = tab // spec.B
    rows = np.asarray(spec.rows)[tab]
    idx[pos[0::3]] = rows[0::3]                      # one past the table
    idx[pos[1::3]] = -1 if idx.dtype == np.int64 else -5
    idx[pos[2::3]] = rows[2::3] + 1000
    want = _expect(spec, off, idx)
    assert want[0] == te.TBE_INVALID_INDEX and want[1] == 37
    got, o2, i2 = _run(spec, off, idx)
    assert got == want
    assert np.array_equal(i2, idx), "check alone must not write"
    got, o2, i2 = _run(spec, off, idx, te.TBE_VALIDATE_REPAIR)
    assert got == want
    fixed = idx.copy()
    fixed[pos] = 0
    assert np.array_equal(i2, fixed) and np.array_equal(o2, off)
    # the repaired inputs keep the contract and pool as the oracle does
    case = S.Case(spec)
    case.idx = fixed
    case.d_idx = torch.from_numpy(fixed).cuda()
    out = case.tbe().forward(spec.B, case.d_idx, case.d_off, case.d_psw)
    torch.cuda.synchronize()
    S.check_forward(case, out)


def test_bad_offsets_reported_and_clamped():
    import table_embedding_amd as te
    spec = _spec("C2s")
    off0, idx = spec.offsets(), spec.indices()
    N, TB = len(idx), spec.T * spec.B
    cases = []
    o = off0.copy(); o[0] = 3; cases.append(o)                 # start
    o = off0.copy(); o[TB] = N - 2; cases.append(o)            # end
    o = off0.copy(); o[100], o[101] = o[101], o[100] + 1; cases.append(o)  # order
    o = off0.copy(); o[700] = N + 50; cases.append(o)          # range (and order)
    o = off0.copy(); o[5] = -4; cases.append(o)                # negative
    for o in cases:
        want = _expect(spec, o, idx)
        assert want[0] != 0
        got, o2, i2 = _run(spec, o, idx)
        assert got == want, (got, want)
        got, o2, i2 = _run(spec, o, idx, te.TBE_VALIDATE_REPAIR)
        assert got == want
        clamp = np.clip(o, 0, N)
        clamp[0], clamp[TB] = 0, N
        assert np.array_equal(o2, clamp)
