"""tbe_forward_checked: the forward with the input checks fused into the
generic kernels.  Valid inputs give tbe_forward's output bit for bit and an
empty error block; planted indices out of range (int32, int64, and int64
values whose low word is a valid row) are reported exactly as the plain numpy
check of the contract in test_gpu_validate reports them, and the pooled
output equals the oracle's with those lookups contributing nothing (bags keep
their lengths); planted offset breaks are reported the same way and give
finite outputs.  Both generic kernels (equal pieces, one bag per subgroup)."""
import numpy as np
import pytest
import torch

import oracle
from tests import support as S
from tests.test_gpu_parity import _announce, _spec
from tests.test_gpu_validate import NONE, _expect

pytestmark = pytest.mark.gpu
SPLITS = ["balanced", "one_bag"]


def _flags(split):
    import table_embedding_amd as te
    return te.TBE_FWD_NO_HIST | (te.TBE_FWD_BALANCE if split == "balanced" else
                                 te.TBE_FWD_NO_BALANCE)


def _checked(case, idx, off, split):
    import table_embedding_amd as te
    spec = case.spec
    tb = case.tbe()
    d_idx = torch.from_numpy(idx.copy()).cuda()
    d_off = torch.from_numpy(off.copy()).cuda()
    out = torch.full((spec.B, spec.dtot), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.full((te.TBE_VALIDATE_WORDS,), 7, dtype=torch.uint32, device="cuda")
    te.tbe_forward_checked(tb.plan, spec.B, d_idx, d_off, len(idx), case.d_psw, out, err,
                           _flags(split))
    torch.cuda.synchronize()
    res = out.cpu().numpy(), [int(x) for x in err.cpu().numpy()]
    tb.close()
    return res


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("name", ["C1", "C2s", "C3s", "C4s", "many_tables", "empty_bags",
                                  "cut_bags", "wide_f32", "one_row", "all_empty"])
def test_checked_forward_valid_inputs(name, split):
    import table_embedding_amd as te
    _announce(name, f"checked forward {split}")
    case = S.Case(_spec(name))
    got, err = _checked(case, case.idx, case.off, split)
    assert err == [0, 0, NONE, NONE]
    tb = case.tbe()
    ref = tb.forward(case.spec.B, case.d_idx, case.d_off, case.d_psw,
                     flags=_flags(split)).cpu().numpy()
    assert got.tobytes() == ref.tobytes(), "checked forward differs from tbe_forward"
    if case.N:
        S.check_forward(case, torch.from_numpy(got))


def _plant(spec, idx, off, n, seed, high_word=False):
    rng = np.random.default_rng(seed)
    pos = np.sort(rng.choice(len(idx), n, replace=False))
    tab = (np.searchsorted(off, pos, side="right") - 1) // spec.B
    rows = np.asarray(spec.rows, np.int64)[tab]
    idx = idx.copy()
    idx[pos[0::3]] = rows[0::3]                              # one past the table
    idx[pos[1::3]] = -1 if idx.dtype == np.int64 else -7     # negative
    if high_word:                                            # low word a valid row
        idx[pos[2::3]] = (np.int64(1) << 32) + 3
    else:
        idx[pos[2::3]] = rows[2::3] + 999
    return idx, pos


@pytest.mark.parametrize("split", SPLITS)
@pytest.mark.parametrize("name,high", [("C2s", False), ("C2s", True), ("many_tables", False),
                                       ("C3s", True), ("cut_bags", False)])
def test_checked_forward_bad_indices(name, high, split):
    import table_embedding_amd as te
    _announce(name, f"checked forward bad indices high={high} {split}")
    case = S.Case(_spec(name))
    spec = case.spec
    idx, pos = _plant(spec, case.idx, case.off, 40, 11, high_word=high)
    want = _expect(spec, case.off, idx)
    assert want[0] == te.TBE_INVALID_INDEX and want[1] == 40
    got, err = _checked(case, idx, case.off, split)
    assert err == want, (err, want)
    # the oracle with the bad lookups contributing nothing (weight 0, row 0)
    clean = idx.copy()
    clean[pos] = 0
    w = (np.ones(len(idx), np.float32) if case.psw is None else case.psw.copy())
    w[pos] = 0.0
    ref = oracle.forward(spec.rows, spec.dims, spec.pooling, spec.wdtype, case.W, spec.B,
                         spec.itype, clean, case.off, w).astype(np.float64)
    e = np.abs(got.astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    assert np.all(np.isfinite(got)) and float(e.max()) <= 1e-4


@pytest.mark.parametrize("split", SPLITS)
def test_checked_forward_bad_offsets(split):
    _announce("C2s", f"checked forward bad offsets {split}")
    case = S.Case(_spec("C2s"))
    spec = case.spec
    off0, idx = case.off, case.idx
    N, TB = len(idx), spec.T * spec.B
    cases = []
    o = off0.copy(); o[0] = 3; cases.append(o)                 # start
    o = off0.copy(); o[TB] = N - 2; cases.append(o)            # end
    o = off0.copy(); o[100], o[101] = o[101], o[100] + 1; cases.append(o)  # order
    o = off0.copy(); o[700] = N + 50; cases.append(o)          # range (and order)
    o = off0.copy(); o[5] = -4; cases.append(o)                # negative
    o = off0.copy(); o[TB] = N + 1000; cases.append(o)         # end past N
    for o in cases:
        want = _expect(spec, o, idx)
        assert want[0] != 0 and want[1] == 0
        got, err = _checked(case, idx, o, split)
        assert err == want, (err, want)
        assert np.all(np.isfinite(got))
