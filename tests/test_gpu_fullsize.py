"""Parity at the full workload sizes, in the launch configuration bench.py times:
tbe_forward, then tbe_backward_rowwise_adagrad with its own preprocessing, one
stream, default flags.  Inputs are bench.py's: the index structure from the
seeded numpy generators, weights / grad_out / per-sample weights drawn on the
device from seeded torch generators (momentum starts at 0).

What the oracle computes one by one:
  - forward: sampled bags of sampled tables (first, last, longest, random), each
    pooled by the oracle from a copy of exactly the rows it reads;
  - backward: sampled rows of sampled tables (the hottest, runs of lengths 255,
    256, 257 and 512 when present, one long run of each size class, singles,
    2..31, 32..255, random): the oracle updates a copy of each row from all of
    its lookups, every lookup a one-lookup bag that carries its grad_out row and
    its contribution scale S[p] * (1/L if mean) (the same float32 scale the
    device folds in), so the oracle's float64 sum over the lookups is the row
    gradient of the definition;
and at any size:
  - every touched row of the sampled tables updated exactly once (debug
    counter), untouched rows' weights and momentum bit-identical (sampled);
  - C2 and C4 in full: the oracle on the whole problem, and for C2 every integer
    output of the preprocessing bit for bit.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import tbe_workloads as wl
from tests import support as S

pytestmark = pytest.mark.gpu


class Full:
    """One bench-configuration step of a workload, with host copies of what the
    checks need taken before the backward runs."""

    def __init__(self, cfg, sample_tables, rows_per_table=24, bags_per_table=16, seed=7,
                 snapshot_all=False):
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
        self.rng = np.random.default_rng(seed)
        self.tables = list(sample_tables)
        self.rows_per_table = rows_per_table
        self.bags_per_table = bags_per_table
        self.samples = {t: self._pick(t) for t in self.tables}
        # host copies before any update
        self.before = {}
        for t, smp in self.samples.items():
            r = torch.from_numpy(np.concatenate([smp["rows"], smp["untouched"]])).cuda()
            self.before[t] = (S.to_host_storage(self.W[t][r], spec.wdtype),
                              self.M[t][r].cpu().numpy().copy())
        self.forward_rows = {t: S.to_host_storage(self.W[t][torch.from_numpy(
            smp["fwd_rows"]).cuda()], spec.wdtype) for t, smp in self.samples.items()}
        self.W_init = ([S.to_host_storage(w, spec.wdtype) for w in self.W] if snapshot_all
                       else None)
        # the step
        self.out = torch.empty((spec.B, spec.dtot), dtype=torch.float32, device="cuda")
        self.cnt = torch.zeros(sum(spec.rows), dtype=torch.int32, device="cuda")
        print(f"[gpu] full-size {cfg}: step, {self.N} lookups", flush=True)
        self.ws = self.tb.workspace(spec.B, self.N)
        te.tbe_forward(self.tb.plan, spec.B, self.d_idx, self.d_off, self.N, self.psw, self.out)
        te.tbe_backward_rowwise_adagrad(self.tb.plan, spec.B, self.d_idx, self.d_off, self.N,
                                        self.psw, self.G, spec.lr, spec.eps, self.ws, 0,
                                        self.cnt)
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- samples
    def _segment(self, t):
        lo, hi = int(self.off[t * self.B]), int(self.off[(t + 1) * self.B])
        return lo, hi

    def _pick(self, t):
        lo, hi = self._segment(t)
        ix = self.idx[lo:hi].astype(np.int64)
        uniq, cnt = np.unique(ix, return_counts=True)
        rows = [int(uniq[np.argmax(cnt)])] if len(uniq) else []
        for want in (255, 256, 257, 512):
            hit = uniq[cnt == want]
            if len(hit):
                rows.append(int(hit[0]))
        for lo_c, hi_c in ((1, 2), (2, 32), (32, 256), (256, 512), (512, 1 << 30)):
            hit = uniq[(cnt >= lo_c) & (cnt < hi_c)]
            if len(hit):
                rows += [int(x) for x in self.rng.choice(hit, min(3, len(hit)), replace=False)]
        if len(uniq):
            rows += [int(x) for x in self.rng.choice(uniq, min(4, len(uniq)), replace=False)]
        rows = np.unique(np.array(rows, np.int64))[: self.rows_per_table]
        touched = np.zeros(self.spec.rows[t], bool)
        touched[uniq] = True
        free = np.flatnonzero(~touched)
        untouched = (self.rng.choice(free, min(64, len(free)), replace=False)
                     if len(free) else np.zeros(0, np.int64))
        lens = np.diff(self.off[t * self.B:(t + 1) * self.B + 1].astype(np.int64))
        bags = {0, self.B - 1, int(np.argmax(lens))}
        bags |= {int(b) for b in self.rng.choice(self.B, self.bags_per_table, replace=False)}
        bags = np.array(sorted(bags), np.int64)
        fwd_rows = np.unique(np.concatenate(
            [ix[int(self.off[t * self.B + b]) - lo:int(self.off[t * self.B + b + 1]) - lo]
             for b in bags] + [np.zeros(0, np.int64)]))
        return dict(rows=rows, untouched=np.sort(untouched).astype(np.int64), bags=bags,
                    fwd_rows=fwd_rows, uniq=uniq)

    # ----------------------------------------------------------------- checks
    def check_forward_samples(self):
        spec, worst = self.spec, 0.0
        for t, smp in self.samples.items():
            D, lo = spec.dims[t], self._segment(t)[0]
            bags, fr = smp["bags"], smp["fwd_rows"]
            if len(fr) == 0:
                continue
            sub_idx, sub_off, sub_psw = [], [0], []
            for b in bags:
                j = t * self.B + int(b)
                p0, p1 = int(self.off[j]), int(self.off[j + 1])
                sub_idx.append(np.searchsorted(fr, self.idx[p0:p1].astype(np.int64)))
                sub_off.append(sub_off[-1] + p1 - p0)
                if self.psw is not None:
                    sub_psw.append(self.psw[p0:p1].cpu().numpy())
            idx_a = np.concatenate(sub_idx).astype(np.int64)
            off_a = np.array(sub_off, np.int64)
            psw_a = np.concatenate(sub_psw).astype(np.float32) if self.psw is not None else None
            ref = oracle.forward([max(1, len(fr))], [D], [spec.pooling[t]], spec.wdtype,
                                 [self.forward_rows[t].reshape(len(fr), D)], len(bags), "i64",
                                 idx_a, off_a, psw_a).astype(np.float64)
            got = self.out[torch.from_numpy(bags).cuda(), int(self.col[t]):int(self.col[t]) + D]
            got = got.cpu().numpy().astype(np.float64)
            err = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max(initial=0.0))
            assert err <= 1e-4, f"table {t}: forward scaled error {err}"
            worst = max(worst, err)
        return worst

    def _scales(self, t, pos, bags):
        """Contribution scale of each lookup, in float32 as the device forms it."""
        sp = (np.ones(len(pos), np.float32) if self.psw is None
              else self.psw[torch.from_numpy(pos).cuda()].cpu().numpy().astype(np.float32))
        if self.spec.pooling[t] == wl.POOL_MEAN:
            L = (self.off[bags + 1] - self.off[bags]).astype(np.float32)
            sp = (sp / L).astype(np.float32)
        return sp

    def check_backward_samples(self):
        spec, worst_w, worst_m = self.spec, 0.0, 0.0
        for t, smp in self.samples.items():
            D, (lo, hi) = spec.dims[t], self._segment(t)
            rows, nr = smp["rows"], len(smp["rows"])
            ix = self.idx[lo:hi].astype(np.int64)
            sub_idx, pos_all = [], []
            for k, r in enumerate(rows):
                pos = lo + np.flatnonzero(ix == r)
                pos_all.append(pos)
                sub_idx.append(np.full(len(pos), k, np.int64))
            pos = np.concatenate(pos_all).astype(np.int64)
            bags = np.searchsorted(self.off, pos, side="right") - 1  # bag j of each lookup
            b = bags - t * self.B
            G = self.G[torch.from_numpy(b).cuda(), int(self.col[t]):int(self.col[t]) + D]
            G = np.ascontiguousarray(G.cpu().numpy(), np.float32)
            W0, M0 = self.before[t]
            Wr = np.ascontiguousarray(W0[:nr])
            Mr = np.ascontiguousarray(M0[:nr])
            oracle.backward_rowwise_adagrad([nr], [D], [wl.POOL_SUM], spec.wdtype, [Wr], [Mr],
                                            len(pos), "i64", np.concatenate(sub_idx),
                                            np.arange(len(pos) + 1, dtype=np.int64),
                                            self._scales(t, pos, bags), G, spec.lr, spec.eps)
            r_all = torch.from_numpy(np.concatenate([rows, smp["untouched"]])).cuda()
            Wg = S.to_host_storage(self.W[t][r_all], spec.wdtype)
            Mg = self.M[t][r_all].cpu().numpy()
            ok, v = S.weights_ok(Wg[:nr], Wr, spec.wdtype, W0[:nr])
            assert ok, f"table {t}: weight tolerance exceeded ({v})"
            rel = np.abs(Mg[:nr].astype(np.float64) - Mr) / np.maximum(np.abs(Mr), 1e-30)
            assert float(rel.max(initial=0.0)) <= 1e-5, f"table {t}: momentum rel {rel.max()}"
            assert Wg[nr:].tobytes() == W0[nr:].tobytes(), f"table {t}: untouched weights"
            assert Mg[nr:].tobytes() == M0[nr:].tobytes(), f"table {t}: untouched momentum"
            worst_w, worst_m = max(worst_w, v), max(worst_m, float(rel.max(initial=0.0)))
        return worst_w, worst_m

    def check_exactly_once(self):
        kb = self.tb.key_bases()
        for t, smp in self.samples.items():
            seg = self.cnt[kb[t]:kb[t] + self.spec.rows[t]].cpu().numpy()
            want = np.zeros(self.spec.rows[t], np.int32)
            want[smp["uniq"]] = 1
            assert np.array_equal(seg, want), f"table {t}: row updates not exactly once"

    def close(self):
        self.tb.close()


def _run(cfg, tables):
    f = Full(cfg, tables)
    try:
        fw = f.check_forward_samples()
        ww, wm = f.check_backward_samples()
        f.check_exactly_once()
        print(f"[gpu] full-size {cfg}: forward err {fw:.2e}, weight ulp {ww}, "
              f"momentum rel {wm:.2e}", flush=True)
    finally:
        f.close()


@pytest.mark.timeout(600)
def test_fullsize_c3_sampled():
    # D 32 sum, 96 mean, 128 sum, 160 mean, 256 sum: every bucket and both poolings
    _run("C3", [0, 1, 7, 8, 14])


@pytest.mark.timeout(900)
def test_fullsize_c5_sampled():
    _run("C5", [0, 31, 63])


class _CaseView:
    """The attributes support.check_preprocess reads, for a Full workload."""

    def __init__(self, f):
        self.spec, self.off, self.idx, self.N = f.spec, f.off, f.idx, f.N
        self.psw = None if f.psw is None else f.psw.cpu().numpy()

    def oracle_preprocess(self):
        return oracle.preprocess(self.spec.rows, self.spec.B, self.spec.itype, self.idx, self.off)


def _whole(cfg):
    """The oracle on the whole problem: pooled outputs, every row, every integer
    output of the preprocessing (C2)."""
    f = Full(cfg, [0], snapshot_all=True)
    try:
        spec = f.spec
        W0 = [S.to_host_storage(w, spec.wdtype) for w in f.W]  # after the step
        Wh = f.W_init
        psw = None if f.psw is None else f.psw.cpu().numpy()
        ref = oracle.forward(spec.rows, spec.dims, spec.pooling, spec.wdtype, Wh, spec.B,
                             spec.itype, f.idx, f.off, psw)
        got = f.out.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref.astype(np.float64)))
        assert float(err.max()) <= 1e-4, f"forward scaled error {err.max()}"
        Mh = [np.zeros(r, np.float32) for r in spec.rows]
        Wr = [w.copy() for w in Wh]
        oracle.backward_rowwise_adagrad(spec.rows, spec.dims, spec.pooling, spec.wdtype, Wr, Mh,
                                        spec.B, spec.itype, f.idx, f.off, psw,
                                        f.G.cpu().numpy(), spec.lr, spec.eps)
        for t in range(spec.T):
            Wg = W0[t].reshape(spec.rows[t], spec.dims[t])
            ok, v = S.weights_ok(Wg, Wr[t].reshape(spec.rows[t], spec.dims[t]), spec.wdtype,
                                 Wh[t].reshape(spec.rows[t], spec.dims[t]))
            assert ok, f"table {t}: weight tolerance exceeded ({v})"
            Mg = f.M[t].cpu().numpy()
            touched = Mh[t] != 0
            W0t, Wht = Wg, Wh[t].reshape(spec.rows[t], spec.dims[t])
            assert W0t[~touched].tobytes() == Wht[~touched].tobytes(), f"table {t}: untouched W"
            assert Mg[~touched].tobytes() == Mh[t][~touched].tobytes(), f"table {t}: momentum"
            rel = np.abs(Mg[touched].astype(np.float64) - Mh[t][touched]) / np.abs(Mh[t][touched])
            assert float(rel.max(initial=0.0)) <= 1e-5, f"table {t}: momentum rel {rel.max()}"
        if cfg == "C2":
            S.check_preprocess(_CaseView(f), f.tb)
        f.check_exactly_once()
    finally:
        f.close()


@pytest.mark.timeout(600)
def test_fullsize_c2_whole():
    _whole("C2")


@pytest.mark.timeout(600)
def test_fullsize_c4_whole():
    _whole("C4")
