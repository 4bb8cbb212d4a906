"""Shared helpers of the GPU parity tests: upload a workload, run the HIP path
through the C ABI, run the oracle on the same inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tbe_workloads as wl

TORCH_WD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def tolerance_weights(a_st, b_st, wdtype, ref_f64=None):
    """Max violation of the weight tolerance: 2 storage ulp for 16-bit types,
    1e-6*max(1,|ref|) for float32.  Returns the worst ulp distance or scaled error."""
    if wdtype == "f32":
        a = a_st.view(np.float32).astype(np.float64)
        b = b_st.view(np.float32).astype(np.float64)
        return float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b)), initial=0.0))
    a = a_st.astype(np.int64)
    b = b_st.astype(np.int64)
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return float(np.max(np.abs(a - b), initial=0))


def storage_ulp(mag, wdtype):
    """Spacing of the storage format at magnitude mag (subnormal spacing below)."""
    p, emin = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}[wdtype]
    e = np.floor(np.log2(np.maximum(mag, np.ldexp(1.0, emin))))
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))


# worst literal (bit-pattern) ulp distance of 16-bit weights seen by weights_ok,
# reported beside the enforced measure
STATS = {"literal_ulp": 0.0}


def literal_ulp(a_st, b_st, wdtype):
    """Distance in representable values between stored 16-bit weights (the
    ulp of the result itself); float32 tables give 0."""
    if wdtype == "f32":
        return 0.0
    return tolerance_weights(a_st, b_st, wdtype)


def weights_ok(a_st, b_st, wdtype, old_st=None, literal_f16=True):
    """Updated weights against the oracle's.  float16 after row-wise Adagrad:
    within 2 ulp of the result itself (representable values between the two
    bit patterns), the bar as written.  bfloat16, and float16 after the other
    optimizer epilogues (literal_f16=False: SGD and element-wise Adagrad,
    whose step is not normalized by the row's momentum): within 2 ulp taken at
    max(|W_before|, |W_ref|), the scale of the operands.  The device forms the
    step in float32, and where W - step cancels toward zero the result's own
    ulp is far finer than the float32 rounding of the operands (bfloat16: an
    8-bit exponent, no spacing floor near 0; float16: 2^-24 in the subnormal
    range, where an SGD step of lr * g with g a float32 sum of thousands of
    terms can land).  float32: within 1e-6 max(1, |ref|).  The literal
    distance of 16-bit weights is recorded in STATS either way."""
    lit = literal_ulp(a_st, b_st, wdtype)
    if wdtype != "f32":
        STATS["literal_ulp"] = max(STATS["literal_ulp"], lit)
    if wdtype == "f32":
        v = tolerance_weights(a_st, b_st, wdtype)
        return v <= 1e-6, v
    if (wdtype == "f16" and literal_f16) or old_st is None:
        return lit <= 2, lit
    import tbe_workloads as wl_
    a = wl_.storage_to_f64(a_st, wdtype)
    b = wl_.storage_to_f64(b_st, wdtype)
    o = wl_.storage_to_f64(old_st, wdtype)
    u = storage_ulp(np.maximum(np.abs(b), np.abs(o)), wdtype)
    v = float(np.max(np.abs(a - b) / u, initial=0.0))
    return v <= 2, v


def to_host_storage(t: torch.Tensor, wdtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if wdtype == "f32":
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def from_host_storage(a: np.ndarray, wdtype: str, device="cuda") -> torch.Tensor:
    if wdtype == "f32":
        return torch.from_numpy(a.copy()).to(device)
    return torch.from_numpy(a.view(np.int16).copy()).to(device).view(TORCH_WD[wdtype])


class Case:
    """Host inputs of one workload plus their device copies."""

    def __init__(self, spec: wl.Spec, m_nonzero=False, device="cuda"):
        self.spec = spec
        self.off = spec.offsets()
        self.idx = spec.indices()
        self.psw = spec.per_sample_weights()
        self.G = spec.grad_out()
        self.W = [wl.to_storage(spec.weights_f32(t), spec.wdtype) for t in range(spec.T)]
        self.M = [spec.momentum(t, nonzero=m_nonzero) for t in range(spec.T)]
        self.N = int(self.off[-1])
        d = device
        self.d_off = torch.from_numpy(self.off).to(d)
        self.d_idx = torch.from_numpy(self.idx).to(d)
        self.d_psw = None if self.psw is None else torch.from_numpy(self.psw).to(d)
        self.d_G = torch.from_numpy(self.G).to(d)
        self.reset_tables()

    def reset_tables(self):
        self.d_W = [from_host_storage(w, self.spec.wdtype) for w in self.W]
        self.d_M = [torch.from_numpy(m.copy()).cuda() for m in self.M]

    def tbe(self):
        import table_embedding_amd as te
        return te.TBE(self.spec.rows, self.spec.dims, self.spec.pooling, self.d_W, self.d_M)

    # ------------------------------------------------------------- oracle
    def oracle_forward(self):
        s = self.spec
        return oracle.forward(s.rows, s.dims, s.pooling, s.wdtype, self.W, s.B, s.itype,
                              self.idx, self.off, self.psw)

    def oracle_backward(self):
        s = self.spec
        W = [w.copy() for w in self.W]
        M = [m.copy() for m in self.M]
        oracle.backward_rowwise_adagrad(s.rows, s.dims, s.pooling, s.wdtype, W, M, s.B, s.itype,
                                        self.idx, self.off, self.psw, self.G, s.lr, s.eps)
        return W, M

    def oracle_preprocess(self):
        return oracle.preprocess(self.spec.rows, self.spec.B, self.spec.itype, self.idx, self.off)


def read_u32(ws: torch.Tensor, offset: int, count: int) -> np.ndarray:
    if count == 0:
        return np.zeros(0, np.uint32)
    return ws[offset:offset + 4 * count].cpu().numpy().view(np.uint32).copy()


def read_u32x4(ws, offset, count):
    return read_u32(ws, offset, 4 * count).reshape(count, 4)


def check_forward(case: Case, out_gpu: torch.Tensor):
    ref = case.oracle_forward().astype(np.float64)
    got = out_gpu.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    assert np.all(np.isfinite(got))
    worst = float(err.max(initial=0.0))
    assert worst <= 1e-4, f"forward max scaled error {worst}"
    return worst


def touched_rows(case: Case, t: int) -> np.ndarray:
    s = case.spec
    lo, hi = int(case.off[t * s.B]), int(case.off[(t + 1) * s.B])
    return np.unique(case.idx[lo:hi].astype(np.int64))


def check_backward(case: Case, tbe_obj):
    """Touched rows within tolerance of the oracle, untouched rows bit-identical."""
    Wr, Mr = case.oracle_backward()
    s = case.spec
    worst_w, worst_m = 0.0, 0.0
    for t in range(s.T):
        Wg = to_host_storage(tbe_obj.weights[t], s.wdtype).reshape(s.rows[t], s.dims[t])
        Mg = tbe_obj.momentum[t].cpu().numpy()
        W0 = case.W[t].reshape(s.rows[t], s.dims[t])
        rows = touched_rows(case, t)
        mask = np.zeros(s.rows[t], bool)
        mask[rows] = True
        assert Wg[~mask].tobytes() == W0[~mask].tobytes(), f"table {t}: untouched rows changed"
        assert Mg[~mask].tobytes() == case.M[t][~mask].tobytes(), f"table {t}: untouched M"
        ok, v = weights_ok(Wg[mask], Wr[t].reshape(s.rows[t], s.dims[t])[mask], s.wdtype,
                           W0[mask])
        assert ok, f"table {t}: weight tolerance exceeded ({v})"
        worst_w = max(worst_w, v)
        rel = np.abs(Mg[mask].astype(np.float64) - Mr[t][mask]) / np.maximum(
            np.abs(Mr[t][mask].astype(np.float64)), 1e-30)
        worst = float(rel.max(initial=0.0))
        assert worst <= 1e-5, f"table {t}: momentum rel error {worst}"
        worst_m = max(worst_m, worst)
    return worst_w, worst_m


def bucket_of_table(spec) -> np.ndarray:
    w = [1 << max(0, (d - 1).bit_length()) for d in spec.dims]
    uw = sorted(set(w))
    return np.array([uw.index(x) for x in w], np.int64)


def gpu_preprocess_views(tbe_obj, case: Case):
    """Read the workspace after tbe_preprocess and map it to the oracle's key order."""
    import table_embedding_amd as te
    s = case.spec
    v = te.tbe_workspace_views(tbe_obj.plan, s.B, case.N)
    ws = tbe_obj._ws
    N = case.N
    nb = v["num_buckets"]
    cnt = read_u32(ws, v["counters"], 6 + 5 * (nb + 1))
    assert int(read_u32(ws, v["prep_error"], 1)[0]) == 0, "a look-back wait gave up"
    U, n1, nt, nm, nl, nc = (int(x) for x in cnt[:6])
    out = dict(
        sorted_key=read_u32(ws, v["sorted_key"], N).astype(np.int64),
        sorted_bag=read_u32(ws, v["sorted_bag"], N).astype(np.int64),
        sorted_scale=read_u32(ws, v["sorted_scale"], N).view(np.float32),
        run_start=read_u32(ws, v["run_start"], U + 1).astype(np.int64),
        run_key=read_u32(ws, v["run_key"], U).astype(np.int64),
        single_task=read_u32x4(ws, v["single_task"], n1).astype(np.int64),
        tiny_task=read_u32x4(ws, v["tiny_task"], nt).astype(np.int64),
        medium_task=read_u32x4(ws, v["medium_task"], nm).astype(np.int64),
        long_task=read_u32x4(ws, v["long_task"], nl).astype(np.int64),
        long_cbeg=read_u32(ws, v["long_cbeg"], nl).astype(np.int64),
        chunk_task=read_u32x4(ws, v["chunk_task"], nc).astype(np.int64),
        U=U, n_single=n1, n_tiny=nt, n_medium=nm, n_long=nl, n_chunks=nc, nb=nb,
        begins=cnt[6:].reshape(5, nb + 1).astype(np.int64))
    kb = np.array(tbe_obj.key_bases(), np.int64)
    out["key_base"] = kb
    return out


def check_preprocess(case: Case, tbe_obj):
    """Bit-exact comparison of every integer output of the preprocessing."""
    g = gpu_preprocess_views(tbe_obj, case)
    r = case.oracle_preprocess()
    compare_preprocess(case.spec, case.off, case.psw, case.N, g, r)
    return g, r


def compare_preprocess(spec, off, psw, N, g, r, chunk_pos0=0, long_idx0=0):
    """Every integer output of the device preprocessing g against the oracle's r
    (bit for bit): sorted keys and bags, run starts, keys and lengths, the five
    task lists and their counts, the chunk placement, and (when g has them) the
    per-bucket list begins.  g may be one table's part of a larger workspace:
    chunk tasks then sit at positions [chunk_pos0, chunk_pos0 + n_chunks) and
    carry long-run indices from long_idx0 on."""
    kb = g["key_base"]
    base = np.concatenate([[0], np.cumsum(spec.rows)[:-1]]).astype(np.int64)
    order = np.argsort(kb, kind="stable")       # tables by linear key
    kb_sorted = kb[order]

    def to_oracle_key(k):
        i = np.searchsorted(kb_sorted, k, side="right") - 1
        t = order[i]
        return base[t] + (k - kb[t]), t

    okey, _ = to_oracle_key(g["sorted_key"])
    # GPU keys are ordered by (bucket, table); a stable re-sort by the oracle's table-major key
    # gives the oracle's order if and only if every table segment matches
    perm = np.argsort(okey, kind="stable")
    assert np.array_equal(okey[perm], r["sorted_key"].astype(np.int64)), "sorted keys differ"
    # the sort is stable and each bag's lookups are contiguous, so the bag ids of the sorted
    # lookups are the oracle's bag[sorted_pos] (equal keys in ascending position)
    assert np.array_equal(g["sorted_bag"][perm], r["bag"][r["sorted_pos"]]), "sorted bags differ"
    # run starts point at the first slot of each run in the GPU order
    assert g["U"] == r["U"]
    assert g["run_start"][-1] == N
    assert np.array_equal(g["sorted_key"][g["run_start"][:-1]], g["run_key"])
    lens_g = np.diff(g["run_start"])
    rk_o, _ = to_oracle_key(g["run_key"])
    p = np.argsort(rk_o, kind="stable")
    assert np.array_equal(rk_o[p], r["run_key"].astype(np.int64)), "run keys differ"
    assert np.array_equal(lens_g[p], np.diff(r["run_start"])), "run lengths differ"
    olens = np.diff(r["run_start"])
    assert g["n_single"] == int((olens == 1).sum()), "single-lookup run count differs"
    assert g["n_tiny"] == int(((olens >= 2) & (olens < 32)).sum()), "tiny run count differs"
    assert g["n_single"] + g["n_tiny"] + g["n_medium"] == r["n_short"], "short-run count differs"
    assert (g["n_long"], g["n_chunks"]) == (r["n_long"], r["n_chunks"])
    # bag and contribution scale of every sorted lookup
    if psw is not None or any(q == wl.POOL_MEAN for q in spec.pooling):
        L = np.diff(off.astype(np.int64))
        j = r["bag"][r["sorted_pos"]]
        sp = (np.ones(len(j), np.float32) if psw is None
              else psw[r["sorted_pos"]].astype(np.float32))
        mean = np.array(spec.pooling)[j // spec.B] == wl.POOL_MEAN
        want = np.where(mean, sp / L[j].astype(np.float32), sp).astype(np.float32)
        np.testing.assert_allclose(g["sorted_scale"][perm], want, rtol=2.5e-7, atol=0)
    # tasks: every run appears once, in ascending key order, with its table and row
    st = g["single_task"]     # {start, row, table, bag}
    tt = g["tiny_task"]       # {start, len, row, table}
    mt = g["medium_task"]     # {start, len, row, table}
    lt = g["long_task"]
    rs = g["run_start"][:-1]
    one = lens_g == 1
    if len(st):
        assert np.array_equal(st[:, 0], rs[one])
        assert np.array_equal(kb[st[:, 2]] + st[:, 1], g["sorted_key"][st[:, 0]])
        assert np.all(np.diff(kb[st[:, 2]] + st[:, 1]) > 0)
        assert np.array_equal(st[:, 3], g["sorted_bag"][st[:, 0]])
    else:
        assert not one.any()
    for tasks, sel in ((tt, (lens_g >= 2) & (lens_g < 32)), (mt, (lens_g >= 32) & (lens_g < 256))):
        if len(tasks):
            assert np.array_equal(tasks[:, 0], rs[sel])
            assert np.array_equal(tasks[:, 1], lens_g[sel])
            assert np.array_equal(kb[tasks[:, 3]] + tasks[:, 2], g["sorted_key"][tasks[:, 0]])
            assert np.all(np.diff(kb[tasks[:, 3]] + tasks[:, 2]) > 0)
        else:
            assert not sel.any()
    if len(lt):
        assert np.all(lt[:, 1] >= 256)
        assert np.array_equal(lt[:, 0], g["run_start"][:-1][lens_g >= 256])
        assert np.array_equal(lt[:, 1], lens_g[lens_g >= 256])
        assert np.array_equal(kb[lt[:, 3]] + lt[:, 2], g["sorted_key"][lt[:, 0]])
        nch = (lt[:, 1] + 255) // 256
        assert np.array_equal(g["long_cbeg"] - chunk_pos0,
                              np.concatenate([[0], np.cumsum(nch)[:-1]]))
        ct = g["chunk_task"]
        # a run's chunks fill its positions [cbeg, cbeg + nch); the positions are taken in
        # order of (position mod 8, position) and receive chunks 0, 1, 2, ... in turn, so
        # the chunks a residue class holds are consecutive in the run
        want = np.full((g["n_chunks"], 4), -1, np.int64)
        for l, (st0, ln, row, t) in enumerate(lt):
            nch = int((ln + 255) // 256)
            cb = int(g["long_cbeg"][l])
            slots = sorted(range(cb, cb + nch), key=lambda q: (q % 8, q))
            for k, q in enumerate(slots):
                want[q - chunk_pos0] = [st0 + 256 * k, min(256, ln - 256 * k), t, l + long_idx0]
        assert np.array_equal(ct, want), "chunk tasks differ"
    if "begins" not in g:
        return
    # per-bucket begins split the five lists exactly at bucket changes
    bt = bucket_of_table(spec)
    z = np.zeros(0, np.int64)
    for k, tab in enumerate((st[:, 2] if len(st) else z, tt[:, 3] if len(tt) else z,
                             mt[:, 3] if len(mt) else z, lt[:, 3] if len(lt) else z,
                             g["chunk_task"][:, 2] if g["n_chunks"] else z)):
        b = g["begins"][k]
        assert b[0] == 0 and b[-1] == len(tab)
        for q in range(g["nb"]):
            assert np.all(bt[tab[b[q]:b[q + 1]]] == q)


class WorkspaceLists:
    """The integer outputs of one preprocessing, read once from a (full-size)
    workspace, from which one table's part can be cut out and compared with
    the oracle run on that table alone (tables are independent, so the
    oracle's whole-problem result restricted to a table is its one-table
    result)."""

    def __init__(self, tbe_obj, spec, off, N):
        import table_embedding_amd as te
        self.spec, self.off, self.N = spec, off, N
        self.ws = tbe_obj._ws
        self.v = v = te.tbe_workspace_views(tbe_obj.plan, spec.B, N)
        nb = v["num_buckets"]
        cnt = read_u32(self.ws, v["counters"], 6 + 5 * (nb + 1))
        assert int(read_u32(self.ws, v["prep_error"], 1)[0]) == 0, "a look-back wait gave up"
        U, n1, nt, nm, nl, nc = (int(x) for x in cnt[:6])
        self.U = U
        self.kb = np.array(tbe_obj.key_bases(), np.int64)
        self.run_start = read_u32(self.ws, v["run_start"], U + 1).astype(np.int64)
        self.run_key = read_u32(self.ws, v["run_key"], U).astype(np.int64)
        self.lists = dict(
            single_task=read_u32x4(self.ws, v["single_task"], n1).astype(np.int64),
            tiny_task=read_u32x4(self.ws, v["tiny_task"], nt).astype(np.int64),
            medium_task=read_u32x4(self.ws, v["medium_task"], nm).astype(np.int64),
            long_task=read_u32x4(self.ws, v["long_task"], nl).astype(np.int64),
            chunk_task=read_u32x4(self.ws, v["chunk_task"], nc).astype(np.int64))
        self.long_cbeg = read_u32(self.ws, v["long_cbeg"], nl).astype(np.int64)
        self.nb = nb
        self.begins = cnt[6:].reshape(5, nb + 1).astype(np.int64)
        # output base of each table's segment: tables in key order
        per_table = np.array([int(off[(t + 1) * spec.B] - off[t * spec.B])
                              for t in range(spec.T)], np.int64)
        order = np.argsort(self.kb, kind="stable")
        base = np.zeros(spec.T, np.int64)
        base[order] = np.concatenate([[0], np.cumsum(per_table[order])[:-1]])
        self.base, self.per_table = base, per_table

    def table(self, t):
        """Table t's part, rebased to a one-table problem (keys are rows, bag
        ids are the table's own 0 .. B-1, slots count from the segment's
        start); chunk positions stay global (their residues place them)."""
        spec, B = self.spec, self.spec.B
        b0, n_t, kb_t = int(self.base[t]), int(self.per_table[t]), int(self.kb[t])
        v = self.v
        g = dict(
            sorted_key=read_u32(self.ws, v["sorted_key"] + 4 * b0, n_t).astype(np.int64) - kb_t,
            sorted_bag=read_u32(self.ws, v["sorted_bag"] + 4 * b0, n_t).astype(np.int64) - t * B,
            sorted_scale=read_u32(self.ws, v["sorted_scale"] + 4 * b0, n_t).view(np.float32))
        rs = self.run_start
        u0 = int(np.searchsorted(rs[:-1], b0, side="left"))
        u1 = int(np.searchsorted(rs[:-1], b0 + n_t, side="left"))
        g["run_start"] = rs[u0:u1 + 1] - b0
        g["run_key"] = self.run_key[u0:u1] - kb_t
        g["U"] = u1 - u0
        out = {}
        for name, tcol in (("single_task", 2), ("tiny_task", 3), ("medium_task", 3),
                           ("long_task", 3), ("chunk_task", 2)):
            a = self.lists[name]
            sel = np.flatnonzero(a[:, tcol] == t) if len(a) else np.zeros(0, np.int64)
            if len(sel):
                assert np.array_equal(sel, np.arange(sel[0], sel[-1] + 1)), f"{name}: not contiguous"
            out[name] = (a[sel].copy(), int(sel[0]) if len(sel) else 0)
        st, _ = out["single_task"]
        if len(st):
            st[:, 0] -= b0
            st[:, 2] = 0
            st[:, 3] -= t * B
        for name in ("tiny_task", "medium_task", "long_task"):
            a, _ = out[name]
            if len(a):
                a[:, 0] -= b0
                a[:, 3] = 0
        lt, l0 = out["long_task"]
        ct, c0 = out["chunk_task"]
        if len(ct):
            ct[:, 0] -= b0
            ct[:, 2] = 0
        g.update(single_task=st, tiny_task=out["tiny_task"][0], medium_task=out["medium_task"][0],
                 long_task=lt, chunk_task=ct, long_cbeg=self.long_cbeg[l0:l0 + len(lt)],
                 n_single=len(st), n_tiny=len(out["tiny_task"][0]),
                 n_medium=len(out["medium_task"][0]), n_long=len(lt), n_chunks=len(ct),
                 key_base=np.zeros(1, np.int64))
        if len(lt):
            assert c0 == int(g["long_cbeg"][0]), "chunk positions do not start at the first run's"
        return g, dict(chunk_pos0=c0, long_idx0=l0)

    def check_begins(self):
        """The per-bucket begins of the five lists split them exactly where the
        tables' D bucket changes."""
        bt = bucket_of_table(self.spec)
        for k, (name, tcol) in enumerate((("single_task", 2), ("tiny_task", 3),
                                          ("medium_task", 3), ("long_task", 3),
                                          ("chunk_task", 2))):
            tab = self.lists[name][:, tcol] if len(self.lists[name]) else np.zeros(0, np.int64)
            b = self.begins[k]
            assert b[0] == 0 and b[-1] == len(tab), name
            for q in range(self.nb):
                assert np.all(bt[tab[b[q]:b[q + 1]]] == q), name


DENSE_ROWS = 128


def expected_hot_rows(case: Case):
    """Per table, the (row, run length) pairs that the hot-row contraction
    takes, from the host inputs by the selection rule: among the table's long
    runs (run length >= 256), those that reach the smallest threshold of at
    least max(256, B / 256) that at most 128 runs reach; tables whose D is not
    a multiple of 16 or exceeds 256 take none.  Rows ascending (the long
    list's key order within a table)."""
    spec, B = case.spec, case.spec.B
    min_len = max(256, min(B // 256, 1 << 30))
    out = []
    for t in range(spec.T):
        D = spec.dims[t]
        if D % 16 or D > 256:
            out.append([])
            continue
        lo, hi = int(case.off[t * B]), int(case.off[(t + 1) * B])
        rows, lens = np.unique(case.idx[lo:hi].astype(np.int64), return_counts=True)
        keep = lens >= 256
        rows, lens = rows[keep], lens[keep]
        thr = min_len
        if int((lens >= thr).sum()) > DENSE_ROWS:
            # one more than the (DENSE_ROWS + 1)-th longest run
            thr = int(np.sort(lens)[::-1][DENSE_ROWS]) + 1
        sel = lens >= thr
        assert int(sel.sum()) <= DENSE_ROWS
        out.append(list(zip(rows[sel].tolist(), lens[sel].tolist())))
    return out


def check_dense(case: Case, tbe_obj):
    """After a backward that took the hot-row contraction: each table's hot
    rows and their count equal the host selection, each entry names its long
    run, and long_flag marks exactly the hot runs (integers, bit for bit)."""
    import table_embedding_amd as te
    spec = case.spec
    v = te.tbe_workspace_views(tbe_obj.plan, spec.B, case.N)
    ws = tbe_obj._ws
    nb = v["num_buckets"]
    cnt = read_u32(ws, v["counters"], 6 + 5 * (nb + 1))
    nl = int(cnt[4])
    lt = read_u32x4(ws, v["long_task"], nl).astype(np.int64)
    flag = read_u32(ws, v["long_flag"], nl)
    dcnt = read_u32(ws, v["dense_count"], spec.T)
    drows = read_u32x4(ws, v["dense_rows"], spec.T * DENSE_ROWS).reshape(
        spec.T, DENSE_ROWS, 4).astype(np.int64)
    exp = expected_hot_rows(case)
    hot = set()
    for t in range(spec.T):
        assert int(dcnt[t]) == len(exp[t]), f"table {t}: {int(dcnt[t])} hot rows, expected {len(exp[t])}"
        got = drows[t, :len(exp[t])]
        assert [(int(r[2]), int(r[1])) for r in got] == exp[t], f"table {t}: hot rows differ"
        for r in got:
            li = int(r[3])
            assert 0 <= li < nl and lt[li, 3] == t and np.array_equal(lt[li, :3], r[:3]), \
                f"table {t}: hot row {int(r[2])} does not name its long run"
            hot.add(li)
    want = np.zeros(nl, np.uint32)
    want[sorted(hot)] = 1
    assert np.array_equal(flag, want), "long_flag differs from the hot runs"
    return sum(len(e) for e in exp)
