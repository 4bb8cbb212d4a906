"""Parity at the full workload sizes, in the launch configuration bench.py
times: tbe_forward, then tbe_backward_rowwise_adagrad with its own
preprocessing, one stream, default flags.  Inputs are bench.py's: the index
structure from the seeded numpy generators, weights / grad_out / per-sample
weights drawn on the device from seeded torch generators (momentum starts at
0).

Tables are independent in the forward and in the backward, and the
table-major layout makes each table's sorted lookups a segment of their own,
so the oracle run on one table alone (all of its bags with their real
lengths, per-sample weights and pooling, its grad_out columns, its weights
and momentum before the step) gives that table's whole result; the oracle
forms every contribution scale itself, in float64.  For each checked table:
  - forward: every pooled output of the table's columns;
  - backward: every row (touched rows within tolerance, untouched rows and
    their momentum bit-identical);
  - preprocessing: every integer output of the table's segment bit for bit
    (sorted keys and bags, run starts and keys, the five task lists and
    their counts, the chunk placement);
  - every touched row updated exactly once (debug counter).
C5 (138 M lookups: the 16384-key run-length tiles, the deep gathers and
streamed weight rows): tables 0, 31 and 63, and on them the fused long-run
path against the two-launch one, bit for bit.  C3: all 16 tables (every D
bucket, sum and mean, per-sample weights) and the per-bucket list begins.
C2 and C4: the oracle on the whole problem; C2 every integer output of the
preprocessing bit for bit.
"""
import types

import numpy as np
import pytest
import torch

import bench
import oracle
import tbe_workloads as wl
from tests import support as S

pytestmark = pytest.mark.gpu


class Full:
    """One bench-configuration step of a workload, with host copies of the
    checked tables taken before the step."""

    def __init__(self, cfg, tables):
        import table_embedding_amd as te
        self.te = te
        self.spec = spec = wl.config(cfg)
        print(f"[gpu] full-size {cfg}: generating", flush=True)
        (self.off, self.idx, self.d_off, self.d_idx, self.W, self.M, self.G,
         self.psw) = bench.device_inputs(spec, torch)
        self.N = int(self.off[-1])
        self.B = spec.B
        self.col = spec.col_offsets()
        self.tb = te.TBE(spec.rows, spec.dims, spec.pooling, self.W, self.M)
        self.tables = list(tables)
        self.W0 = {t: S.to_host_storage(self.W[t], spec.wdtype).reshape(spec.rows[t], spec.dims[t])
                   for t in self.tables}
        self.M0 = {t: self.M[t].cpu().numpy().copy() for t in self.tables}
        self.out = torch.empty((spec.B, spec.dtot), dtype=torch.float32, device="cuda")
        self.cnt = torch.zeros(sum(spec.rows), dtype=torch.uint32, device="cuda")
        print(f"[gpu] full-size {cfg}: step, {self.N} lookups", flush=True)
        self.ws = self.tb.workspace(spec.B, self.N)
        te.tbe_forward(self.tb.plan, spec.B, self.d_idx, self.d_off, self.N, self.psw, self.out)
        te.tbe_backward_rowwise_adagrad(self.tb.plan, spec.B, self.d_idx, self.d_off, self.N,
                                        self.psw, self.G, spec.lr, spec.eps, self.ws, 0,
                                        self.cnt)
        torch.cuda.synchronize()
        self.lists = S.WorkspaceLists(self.tb, spec, self.off, self.N)
        self.after = {}

    def table_inputs(self, t):
        B = self.B
        lo, hi = int(self.off[t * B]), int(self.off[(t + 1) * B])
        off_t = (self.off[t * B:(t + 1) * B + 1].astype(np.int64) - lo).astype(self.off.dtype)
        idx_t = np.ascontiguousarray(self.idx[lo:hi])
        psw_t = None if self.psw is None else self.psw[lo:hi].cpu().numpy()
        c, D = int(self.col[t]), self.spec.dims[t]
        G_t = self.G[:, c:c + D].contiguous().cpu().numpy()
        return idx_t, off_t, psw_t, G_t

    def check_table(self, t):
        spec, B = self.spec, self.B
        R, D, P = spec.rows[t], spec.dims[t], spec.pooling[t]
        idx_t, off_t, psw_t, G_t = self.table_inputs(t)
        n_t = len(idx_t)
        # forward: every pooled output of the table
        ref = oracle.forward([R], [D], [P], spec.wdtype, [self.W0[t]], B, spec.itype, idx_t,
                             off_t, psw_t).astype(np.float64)
        c = int(self.col[t])
        got = self.out[:, c:c + D].cpu().numpy().astype(np.float64)
        fw = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max(initial=0.0))
        assert fw <= 1e-4, f"table {t}: forward scaled error {fw}"
        # backward: every row
        Wr, Mr = self.W0[t].copy(), self.M0[t].copy()
        oracle.backward_rowwise_adagrad([R], [D], [P], spec.wdtype, [Wr], [Mr], B, spec.itype,
                                        idx_t, off_t, psw_t, G_t, spec.lr, spec.eps)
        Wg = S.to_host_storage(self.W[t], spec.wdtype).reshape(R, D)
        Mg = self.M[t].cpu().numpy()
        self.after[t] = (Wg.tobytes(), Mg.tobytes())
        touched = np.zeros(R, bool)
        touched[np.unique(idx_t.astype(np.int64))] = True
        assert Wg[~touched].tobytes() == self.W0[t][~touched].tobytes(), f"table {t}: untouched W"
        assert Mg[~touched].tobytes() == self.M0[t][~touched].tobytes(), f"table {t}: untouched M"
        ok, wv = S.weights_ok(Wg[touched], Wr[touched], spec.wdtype, self.W0[t][touched])
        assert ok, f"table {t}: weight tolerance exceeded ({wv})"
        mref = Mr[touched].astype(np.float64)
        rel = np.abs(Mg[touched].astype(np.float64) - mref) / np.maximum(np.abs(mref), 1e-30)
        mv = float(rel.max(initial=0.0))
        assert mv <= 1e-5, f"table {t}: momentum rel error {mv}"
        # preprocessing: the table's segment bit for bit
        r = oracle.preprocess([R], B, spec.itype, idx_t, off_t)
        g, kw = self.lists.table(t)
        spec_t = types.SimpleNamespace(rows=[R], pooling=[P], B=B)
        S.compare_preprocess(spec_t, off_t, psw_t, n_t, g, r, **kw)
        # every touched row once
        kb = self.tb.key_bases()
        seg = self.cnt[kb[t]:kb[t] + R].cpu().numpy()
        assert np.array_equal(seg, touched.astype(np.uint32)), f"table {t}: not exactly once"
        return fw, wv, mv

    def check_fused_equals_two_launch(self):
        """The checked tables restored to their state before the step, then the
        fused long-run backward on the same preprocessed workspace: bit for bit
        the two-launch result (the other tables take a second step, which does
        not touch the checked ones)."""
        te, spec = self.te, self.spec
        for t in self.tables:
            self.W[t].copy_(S.from_host_storage(self.W0[t].reshape(-1), spec.wdtype).view(
                self.W[t].shape))
            self.M[t].copy_(torch.from_numpy(self.M0[t]).cuda())
        te.tbe_backward_rowwise_adagrad(self.tb.plan, spec.B, self.d_idx, self.d_off, self.N,
                                        self.psw, self.G, spec.lr, spec.eps, self.ws,
                                        te.TBE_BWD_PREPROCESSED | te.TBE_BWD_FUSED_LONG)
        torch.cuda.synchronize()
        for t in self.tables:
            Wg = S.to_host_storage(self.W[t], spec.wdtype).tobytes()
            Mg = self.M[t].cpu().numpy().tobytes()
            assert (Wg, Mg) == self.after[t], f"table {t}: fused differs from two-launch"

    def close(self):
        self.tb.close()


def _run(cfg, tables, fused=False, begins=False):
    f = Full(cfg, tables)
    try:
        S.STATS["literal_ulp"] = 0.0
        worst = [0.0, 0.0, 0.0]
        for t in tables:
            fw, wv, mv = f.check_table(t)
            worst = [max(worst[0], fw), max(worst[1], wv), max(worst[2], mv)]
            print(f"[gpu] full-size {cfg} table {t}: forward err {fw:.2e}, weight {wv:.2f}, "
                  f"momentum rel {mv:.2e}", flush=True)
        if begins:
            f.lists.check_begins()
        if fused:
            f.check_fused_equals_two_launch()
        print(f"[gpu] full-size {cfg}: forward err {worst[0]:.2e}, weight {worst[1]:.2f} "
              f"(literal ulp {S.STATS['literal_ulp']:.0f}), momentum rel {worst[2]:.2e}",
              flush=True)
    finally:
        f.close()


@pytest.mark.timeout(900)
def test_fullsize_c3_all_tables():
    _run("C3", list(range(16)), begins=True)


@pytest.mark.timeout(900)
def test_fullsize_c5_tables_and_fused():
    _run("C5", [0, 31, 63], fused=True)


def _whole(cfg):
    """The oracle on the whole problem: pooled outputs, every row, every integer
    output of the preprocessing (C2)."""
    import table_embedding_amd as te
    spec = wl.config(cfg)
    print(f"[gpu] full-size {cfg}: generating", flush=True)
    off, idx, d_off, d_idx, W, M, G, psw_d = bench.device_inputs(spec, torch)
    N = int(off[-1])
    tb = te.TBE(spec.rows, spec.dims, spec.pooling, W, M)
    try:
        Wh = [S.to_host_storage(w, spec.wdtype) for w in W]
        out = torch.empty((spec.B, spec.dtot), dtype=torch.float32, device="cuda")
        cnt = torch.zeros(sum(spec.rows), dtype=torch.uint32, device="cuda")
        ws = tb.workspace(spec.B, N)
        te.tbe_forward(tb.plan, spec.B, d_idx, d_off, N, psw_d, out)
        te.tbe_backward_rowwise_adagrad(tb.plan, spec.B, d_idx, d_off, N, psw_d, G, spec.lr,
                                        spec.eps, ws, 0, cnt)
        torch.cuda.synchronize()
        psw = None if psw_d is None else psw_d.cpu().numpy()
        ref = oracle.forward(spec.rows, spec.dims, spec.pooling, spec.wdtype, Wh, spec.B,
                             spec.itype, idx, off, psw)
        got = out.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref.astype(np.float64)))
        assert float(err.max()) <= 1e-4, f"forward scaled error {err.max()}"
        Mh = [np.zeros(r, np.float32) for r in spec.rows]
        Wr = [w.copy() for w in Wh]
        oracle.backward_rowwise_adagrad(spec.rows, spec.dims, spec.pooling, spec.wdtype, Wr, Mh,
                                        spec.B, spec.itype, idx, off, psw, G.cpu().numpy(),
                                        spec.lr, spec.eps)
        S.STATS["literal_ulp"] = 0.0
        kb = tb.key_bases()
        c = cnt.cpu().numpy()
        for t in range(spec.T):
            R, D = spec.rows[t], spec.dims[t]
            Wg = S.to_host_storage(W[t], spec.wdtype).reshape(R, D)
            W0 = Wh[t].reshape(R, D)
            lo, hi = int(off[t * spec.B]), int(off[(t + 1) * spec.B])
            touched = np.zeros(R, bool)
            touched[np.unique(idx[lo:hi].astype(np.int64))] = True
            ok, v = S.weights_ok(Wg[touched], Wr[t].reshape(R, D)[touched], spec.wdtype,
                                 W0[touched])
            assert ok, f"table {t}: weight tolerance exceeded ({v})"
            Mg = M[t].cpu().numpy()
            assert Wg[~touched].tobytes() == W0[~touched].tobytes(), f"table {t}: untouched W"
            assert not Mg[~touched].any(), f"table {t}: untouched momentum"
            rel = np.abs(Mg[touched].astype(np.float64) - Mh[t][touched]) / np.abs(Mh[t][touched])
            assert float(rel.max(initial=0.0)) <= 1e-5, f"table {t}: momentum rel {rel.max()}"
            assert np.array_equal(c[kb[t]:kb[t] + R], touched.astype(np.uint32)), f"table {t}"
        if cfg == "C2":
            case = types.SimpleNamespace(spec=spec, off=off, idx=idx, N=N, psw=psw,
                                         oracle_preprocess=lambda: oracle.preprocess(
                                             spec.rows, spec.B, spec.itype, idx, off))
            S.check_preprocess(case, tb)
        print(f"[gpu] full-size {cfg}: whole problem ok (literal ulp "
              f"{S.STATS['literal_ulp']:.0f})", flush=True)
    finally:
        tb.close()


@pytest.mark.timeout(600)
def test_fullsize_c2_whole():
    _whole("C2")


@pytest.mark.timeout(600)
def test_fullsize_c4_whole():
    _whole("C4")
