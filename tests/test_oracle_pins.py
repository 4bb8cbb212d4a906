"""Pins of the CPU oracle to facts fixed outside the oracle itself.

- the worked example printed on the HugeCTR walkthrough (every intermediate
  array of the transposition, sort and run counting) and the FBTriton page's
  "a row used by three samples becomes one run of length three";
- closed forms of the row-wise Adagrad step;
- the counts-times-table identity (FBTriton page, "Forward", small-table
  histogram path) as a numpy float64 matrix product, for forward and for the
  row gradients;
- a pure-Python brute force without sorting on 500 random tiny problems;
- numpy / torch rounding of the storage formats;
- numpy's stable argsort and unique at full workload sizes.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import tbe_workloads as wl
from tests import brute

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


# ----------------------------------------------------------------- helpers

def bag_of_lookup(offsets):
    L = np.diff(np.asarray(offsets, np.int64))
    return np.repeat(np.arange(L.size), L)


def count_matrix(offsets, indices, psw, B, t, R):
    """A[b, r] = sum of S[p] over lookups p of bag (t, b) with I[p] = r."""
    off = np.asarray(offsets, np.int64)
    lo, hi = off[t * B], off[(t + 1) * B]
    bag = bag_of_lookup(off)[lo:hi] - t * B
    s = np.ones(hi - lo) if psw is None else np.asarray(psw[lo:hi], np.float64)
    A = np.zeros((B, R))
    np.add.at(A, (bag, np.asarray(indices[lo:hi], np.int64)), s)
    return A


def mean_scale(offsets, B, t, pooling):
    L = np.diff(np.asarray(offsets, np.int64))[t * B:(t + 1) * B].astype(np.float64)
    if pooling == wl.POOL_MEAN:
        return np.where(L > 0, 1.0 / np.maximum(L, 1), 0.0)
    return np.ones(B)


def f16(x):
    return np.float64(np.float16(x))


def ulp_diff(a_stored, b_stored, wdtype):
    """|a-b| in units of the storage format's ordered bit patterns."""
    if wdtype == "f32":
        a = a_stored.view(np.int32).astype(np.int64)
        b = b_stored.view(np.int32).astype(np.int64)
        a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
        b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    else:
        a = a_stored.astype(np.int64)
        b = b_stored.astype(np.int64)
        a = np.where(a & 0x8000, -(a & 0x7FFF), a)
        b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


# ----------------------------------------------------------- worked example

def _we():
    return np.array(GOLD["offsets"], np.int64), np.array(GOLD["indices"], np.int64)


def test_worked_example_preprocessing_arrays():
    off, idx = _we()
    r = oracle.preprocess([GOLD["rows"]], GOLD["B"], "i64", idx, off)
    assert r["bag"].tolist() == GOLD["bag"]
    assert r["sorted_key"].tolist() == GOLD["sorted_key"]
    assert r["bag"][r["sorted_pos"]].tolist() == GOLD["bag_of_sorted"]
    assert r["run_start"].tolist() == GOLD["run_start"]
    assert r["run_start"][:-1].tolist() == GOLD["run_start_printed"]
    assert r["U"] == GOLD["U"]
    flags = np.zeros(len(idx), np.int64)
    flags[r["run_start"][:-1]] = 1
    assert flags.tolist() == GOLD["flags"]
    assert np.cumsum(flags).tolist() == GOLD["scan"]
    assert r["n_short"] == 5 and r["n_long"] == 0 and r["n_chunks"] == 0


def test_row_used_by_three_samples_is_one_run_of_three():
    off, idx = _we()
    r = oracle.preprocess([GOLD["rows"]], GOLD["B"], "i64", idx, off)
    u = int(np.nonzero(r["run_key"] == 1)[0][0])
    lo, hi = r["run_start"][u], r["run_start"][u + 1]
    assert hi - lo == 3
    assert sorted(r["bag"][r["sorted_pos"][lo:hi]].tolist()) == [0, 1, 3]


def test_duplicate_lookups_count_separately():
    v = GOLD["duplicate_variant"]
    off, idx = np.array(v["offsets"], np.int64), np.array(v["indices"], np.int64)
    r = oracle.preprocess([GOLD["rows"]], GOLD["B"], "i64", idx, off)
    for row, want in ((2, v["row2_lookups_from_bag2"]), (3, v["row3_lookups_from_bag2"])):
        u = int(np.nonzero(r["run_key"] == row)[0][0])
        bags = r["bag"][r["sorted_pos"][r["run_start"][u]:r["run_start"][u + 1]]]
        assert int((bags == 2).sum()) == want


@pytest.mark.parametrize("wdtype", ["f32", "f16", "bf16"])
def test_worked_example_forward_bag2(wdtype):
    off, idx = _we()
    rng = np.random.default_rng(3)
    W = wl.to_storage(rng.random((GOLD["rows"], GOLD["dim"]), dtype=np.float32) - 0.5, wdtype)
    out = oracle.forward([GOLD["rows"]], [GOLD["dim"]], [0], wdtype, [W], GOLD["B"], "i64", idx, off)
    Wd = wl.storage_to_f64(W, wdtype)
    a, b = GOLD["forward_bag2_rows"]
    np.testing.assert_array_equal(out[2], (Wd[a] + Wd[b]).astype(np.float32))


ROW_GRAD = {1: 7.0, 2: 4.0, 3: 5.0, 4: 1.0, 5: 3.0}  # G[b, :] = b + 1 summed over each run's bags


@pytest.mark.parametrize("m0,eps", [(0.0, 1e-8), (1.0, 0.5)])
def test_worked_example_adagrad_closed_form(m0, eps):
    """Row-wise Adagrad: with every entry of a row gradient equal to c,
    M' = M + c^2 and W' = W - lr*c/(sqrt(M') + eps)."""
    off, idx = _we()
    R, D, B = GOLD["rows"], GOLD["dim"], GOLD["B"]
    rng = np.random.default_rng(4)
    W = (rng.random((R, D), dtype=np.float32) * 0.2 - 0.1).astype(np.float32)
    W0 = W.copy()
    M = np.full(R, m0, np.float32)
    G = np.repeat(np.arange(1, B + 1, dtype=np.float32)[:, None], D, axis=1)
    lr = 0.01
    oracle.backward_rowwise_adagrad([R], [D], [0], "f32", [W], [M], B, "i64", idx, off, None,
                                    G, lr, eps)
    assert W[0].tobytes() == W0[0].tobytes() and M[0] == np.float32(m0)
    for r, c in ROW_GRAD.items():
        m = np.float32(m0 + c * c)
        assert M[r] == m
        want = (W0[r].astype(np.float64)
                - float(np.float32(lr)) * c / (math.sqrt(float(m)) + float(np.float32(eps))))
        np.testing.assert_array_equal(W[r], want.astype(np.float32))


@pytest.mark.parametrize("a0,eps", [(0.0, 1e-8), (2.0, 0.5)])
def test_worked_example_elementwise_adagrad_and_sgd_closed_form(a0, eps):
    """With every entry of a row gradient equal to c: element-wise Adagrad
    A' = A + c^2 per entry and W' = W - lr*c/(sqrt(A') + eps); SGD W' = W - lr*c;
    untouched rows (and their state) unchanged."""
    off, idx = _we()
    R, D, B = GOLD["rows"], GOLD["dim"], GOLD["B"]
    rng = np.random.default_rng(5)
    W0 = (rng.random((R, D), dtype=np.float32) * 0.2 - 0.1).astype(np.float32)
    G = np.repeat(np.arange(1, B + 1, dtype=np.float32)[:, None], D, axis=1)
    lr = 0.01
    W = W0.copy()
    A = np.full((R, D), a0, np.float32)
    oracle.backward([R], [D], [0], "f32", [W], [A], B, "i64", idx, off, None, G, lr, eps,
                    optimizer="adagrad")
    assert W[0].tobytes() == W0[0].tobytes() and np.all(A[0] == np.float32(a0))
    for r, c in ROW_GRAD.items():
        a = np.float32(a0 + c * c)
        assert np.all(A[r] == a)
        want = (W0[r].astype(np.float64)
                - float(np.float32(lr)) * c / (math.sqrt(float(a)) + float(np.float32(eps))))
        np.testing.assert_array_equal(W[r], want.astype(np.float32))
    W = W0.copy()
    oracle.backward([R], [D], [0], "f32", [W], None, B, "i64", idx, off, None, G, lr, eps,
                    optimizer="sgd")
    assert W[0].tobytes() == W0[0].tobytes()
    for r, c in ROW_GRAD.items():
        want = W0[r].astype(np.float64) - float(np.float32(lr)) * c
        np.testing.assert_array_equal(W[r], want.astype(np.float32))


@pytest.mark.parametrize("optimizer", ["adagrad", "sgd"])
@pytest.mark.parametrize("chunk", range(3))
def test_brute_force_tiny_other_optimizers(optimizer, chunk):
    for seed in range(chunk * 40, chunk * 40 + 40):
        p = wl.random_tiny(seed)
        W_st = _tiny_to_oracle(p)
        Wn = [w.copy() for w in W_st]
        A0 = [(np.abs(np.random.default_rng(seed).standard_normal((r, d))) * 0.1).astype(np.float32)
              for r, d in zip(p["rows"], p["dims"])]
        An = [a.copy() for a in A0]
        oracle.backward(p["rows"], p["dims"], p["pooling"], p["wdtype"], Wn,
                        An if optimizer == "adagrad" else None, p["B"], p["itype"], p["indices"],
                        p["offsets"], p["psw"], p["G"], p["lr"], p["eps"], optimizer=optimizer)
        Wref, Aref, touched = brute.update(p, optimizer, A0)
        for t in range(p["T"]):
            rows_t = sorted(r for (tt, r) in touched if tt == t)
            untouched = np.setdiff1d(np.arange(p["rows"][t]), rows_t)
            assert Wn[t][untouched].tobytes() == W_st[t][untouched].tobytes(), seed
            if optimizer == "adagrad":
                assert An[t][untouched].tobytes() == A0[t][untouched].tobytes(), seed
            if rows_t:
                if optimizer == "adagrad":
                    np.testing.assert_allclose(An[t][rows_t], Aref[t][rows_t], rtol=1e-6)
                want = wl.to_storage(Wref[t][rows_t].astype(np.float32), p["wdtype"])
                assert ulp_diff(Wn[t][rows_t], want, p["wdtype"]).max() <= 1, seed


def test_worked_example_mean_pooling_gradient():
    """Mean pooling scales each bag's gradient by 1/L (bag lengths 4, 3, 2, 1)."""
    off, idx = _we()
    R, D, B = GOLD["rows"], 4, GOLD["B"]
    W = np.zeros((R, D), np.float32)
    M = np.zeros(R, np.float32)
    G = np.repeat(np.arange(1, B + 1, dtype=np.float32)[:, None], D, axis=1)
    oracle.backward_rowwise_adagrad([R], [D], [1], "f32", [W], [M], B, "i64", idx, off, None,
                                    G, 0.01, 1e-8)
    g1 = 1 / 4 + 2 / 3 + 4 / 1  # row 1 used by bags 0, 1, 3
    assert M[1] == np.float32(g1 * g1)


# ------------------------------------------------------- dense identities

def _dense_check(spec, W_st, psw, off, idx, check_bwd=True, m_nonzero=False):
    T, B, dims, rows = spec.T, spec.B, spec.dims, spec.rows
    out = oracle.forward(rows, dims, spec.pooling, spec.wdtype, W_st, B, spec.itype, idx, off, psw)
    col = spec.col_offsets()
    Wd = [wl.storage_to_f64(w, spec.wdtype) for w in W_st]
    As = []
    for t in range(T):
        A = mean_scale(off, B, t, spec.pooling[t])[:, None] * count_matrix(off, idx, psw, B, t,
                                                                           rows[t])
        As.append(A)
        ref = A @ Wd[t]
        got = out[:, col[t]:col[t] + dims[t]].astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref)))
    if not check_bwd:
        return
    G = spec.grad_out()
    M = [spec.momentum(t, nonzero=m_nonzero) for t in range(T)]
    W_new = [w.copy() for w in W_st]
    M_new = [m.copy() for m in M]
    oracle.backward_rowwise_adagrad(rows, dims, spec.pooling, spec.wdtype, W_new, M_new, B,
                                    spec.itype, idx, off, psw, G, spec.lr, spec.eps)
    lr, eps = float(np.float32(spec.lr)), float(np.float32(spec.eps))
    for t in range(T):
        touched = count_matrix(off, idx, None, B, t, rows[t]).sum(axis=0) > 0
        g = As[t].T @ G[:, col[t]:col[t] + dims[t]].astype(np.float64)  # [R, D]
        m = (M[t].astype(np.float64) + (g * g).sum(axis=1) / dims[t]).astype(np.float32)
        assert np.all(np.abs(M_new[t][touched] - m[touched])
                      <= 1e-6 * np.maximum(np.abs(m[touched]), 1e-30))
        assert M_new[t][~touched].tobytes() == M[t][~touched].tobytes()
        w = Wd[t] - lr * g / (np.sqrt(m.astype(np.float64))[:, None] + eps)
        want = wl.to_storage(w.astype(np.float32), spec.wdtype) if spec.wdtype != "f32" \
            else w.astype(np.float32)
        # the float32 step before storage rounding may flip one rounding: <= 1 ulp
        assert ulp_diff(W_new[t][touched], want[touched], spec.wdtype).max(initial=0) <= 1
        assert W_new[t][~touched].tobytes() == W_st[t][~touched].tobytes()


def test_dense_identity_c1_full():
    spec = wl.config("C1")
    W = [wl.to_storage(spec.weights_f32(t), spec.wdtype) for t in range(spec.T)]
    _dense_check(spec, W, spec.per_sample_weights(), spec.offsets(), spec.indices())


@pytest.mark.parametrize("wdtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("itype", ["i32", "i64"])
def test_dense_identity_mixed_tables(wdtype, itype):
    """Several tables, sum and mean, per-sample weights, empty bags, duplicates."""
    spec = wl.Spec("mixed", 77, [50, 7, 33], [4, 12, 20], [0, 1, 1], wdtype, 40,
                   "uniform:0:20", "zipf:1.1", itype, True, lr=0.05, eps=0.1)
    W = [wl.to_storage(spec.weights_f32(t), wdtype) for t in range(spec.T)]
    _dense_check(spec, W, spec.per_sample_weights(), spec.offsets(), spec.indices(),
                 m_nonzero=True)


def test_dense_identity_c3_scaled():
    spec = wl.config("C3", rows=300, B=64, T=5)
    W = [wl.to_storage(spec.weights_f32(t), spec.wdtype) for t in range(spec.T)]
    _dense_check(spec, W, spec.per_sample_weights(), spec.offsets(), spec.indices())


@pytest.mark.slow
def test_dense_identity_c4_full():
    spec = wl.config("C4")
    W = [wl.to_storage(spec.weights_f32(0), spec.wdtype)]
    _dense_check(spec, W, None, spec.offsets(), spec.indices())


# ------------------------------------------------------------ brute force

def _tiny_to_oracle(p):
    W_st = [wl.to_storage(w, p["wdtype"]) for w in p["W32"]]
    p["Wf64"] = [wl.storage_to_f64(w, p["wdtype"]) for w in W_st]
    return W_st


@pytest.mark.parametrize("chunk", range(10))
def test_brute_force_tiny(chunk):
    for seed in range(chunk * 50, chunk * 50 + 50):
        p = wl.random_tiny(seed)
        W_st = _tiny_to_oracle(p)
        out = oracle.forward(p["rows"], p["dims"], p["pooling"], p["wdtype"], W_st, p["B"],
                             p["itype"], p["indices"], p["offsets"], p["psw"])
        ref = brute.forward(p)
        assert np.all(np.abs(out - ref) <= 1e-6 * np.maximum(1, np.abs(ref))), seed
        Wn = [w.copy() for w in W_st]
        Mn = [m.copy() for m in p["M"]]
        oracle.backward_rowwise_adagrad(p["rows"], p["dims"], p["pooling"], p["wdtype"], Wn, Mn,
                                        p["B"], p["itype"], p["indices"], p["offsets"], p["psw"],
                                        p["G"], p["lr"], p["eps"])
        Wref, Mref, touched = brute.adagrad(p)
        for t in range(p["T"]):
            rows_t = sorted(r for (tt, r) in touched if tt == t)
            untouched = np.setdiff1d(np.arange(p["rows"][t]), rows_t)
            assert Wn[t][untouched].tobytes() == W_st[t][untouched].tobytes(), seed
            assert Mn[t][untouched].tobytes() == p["M"][t][untouched].tobytes(), seed
            if rows_t:
                np.testing.assert_allclose(Mn[t][rows_t], Mref[t][rows_t], rtol=1e-6)
                want = wl.to_storage(Wref[t][rows_t].astype(np.float32), p["wdtype"])
                assert ulp_diff(Wn[t][rows_t], want, p["wdtype"]).max() <= 1, seed


def test_brute_force_long_runs_cross_the_threshold():
    """Two rows, ~600 lookups: runs of length >= 256 split into chunks."""
    rng = np.random.default_rng(11)
    B, L = 30, 20
    off = np.arange(0, B * L + 1, L, dtype=np.int64)
    idx = (rng.random(B * L) < 0.7).astype(np.int64)  # row 1 ~ 420 times, row 0 ~ 180
    r = oracle.preprocess([2], B, "i64", idx, off)
    lens = np.diff(r["run_start"])
    assert r["n_long"] == int((lens >= 256).sum()) >= 1
    assert r["n_chunks"] == int(sum(-(-int(x) // 256) for x in lens if x >= 256))
    p = dict(T=1, rows=[2], dims=[3], pooling=[0], wdtype="f32", itype="i64", B=B, offsets=off,
             indices=idx, psw=None, W32=[np.zeros((2, 3), np.float32)],
             M=[np.zeros(2, np.float32)], G=rng.standard_normal((B, 3), dtype=np.float32),
             lr=0.01, eps=1e-8)
    W_st = _tiny_to_oracle(p)
    Mn = [np.zeros(2, np.float32)]
    oracle.backward_rowwise_adagrad([2], [3], [0], "f32", W_st, Mn, B, "i64", idx, off, None,
                                    p["G"], 0.01, 1e-8)
    Wref, Mref, _ = brute.adagrad(p)
    np.testing.assert_allclose(Mn[0], Mref[0], rtol=1e-6)
    np.testing.assert_allclose(W_st[0], Wref[0], rtol=1e-6, atol=1e-9)


# ------------------------------------------------------- storage formats

def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("f16", bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode("bf16", bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def _probe_values(rng, n):
    mant = rng.random(n) + 0.5
    expo = rng.integers(-30, 20, n)
    x = np.ldexp(mant, expo) * np.where(rng.random(n) < 0.5, -1, 1)
    specials = [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25, 2.0 ** -14, 1 + 2.0 ** -11,
                1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -40]
    return np.concatenate([x, specials])


def test_f16_rounding_matches_numpy():
    x = _probe_values(np.random.default_rng(5), 20000)
    got = np.array([oracle.round_to("f16", v) for v in x])
    want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)
    np.testing.assert_array_equal(oracle.encode("f16", x), x.astype(np.float16).view(np.uint16))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(6)
    x = np.ldexp(rng.random(20000) + 0.5, rng.integers(-140, 128, 20000)).astype(np.float32)
    x = np.concatenate([x, -x[:100], np.float32([0.0, 1.00390625, 1.01171875, 3.3895314e38,
                                                   3.4e38, 1e-40, 9.2e-41])])
    want = torch.from_numpy(x).to(torch.bfloat16)
    got = np.array([oracle.round_to("bf16", float(v)) for v in x])
    assert np.array_equal(got, want.double().numpy())
    np.testing.assert_array_equal(oracle.encode("bf16", x.astype(np.float64)),
                                  want.view(torch.int16).numpy().view(np.uint16))


# --------------------------------------------- full-size sort / RLE pins

def _linear_keys(spec, off, idx):
    base = np.concatenate([[0], np.cumsum(spec.rows)[:-1]]).astype(np.int64)
    t_of = bag_of_lookup(off) // spec.B
    return base[t_of] + idx.astype(np.int64)


def _sort_rle_vs_numpy(spec):
    off, idx = spec.offsets(), spec.indices()
    r = oracle.preprocess(spec.rows, spec.B, spec.itype, idx, off)
    key = _linear_keys(spec, off, idx)
    assert np.array_equal(r["key"].astype(np.int64), key)
    assert np.array_equal(r["bag"], bag_of_lookup(off))
    order = np.argsort(key, kind="stable")
    assert np.array_equal(r["sorted_pos"], order)
    uk, first, cnt = np.unique(key, return_index=True, return_counts=True)
    assert np.array_equal(r["run_key"].astype(np.int64), uk)
    # first occurrence of a key in original order = sorted position of its run start
    assert np.array_equal(r["sorted_pos"][r["run_start"][:-1]], first)
    lens = np.diff(r["run_start"])
    assert np.array_equal(lens, cnt)
    assert lens.sum() == len(idx)
    assert r["n_short"] == int((cnt < 256).sum()) and r["n_long"] == int((cnt >= 256).sum())
    assert r["n_chunks"] == int(np.sum((cnt[cnt >= 256] + 255) // 256))
    assert r["chunk_len"].sum() == cnt[cnt >= 256].sum()
    assert np.all(r["chunk_len"] <= 256) and np.all(r["chunk_len"] > 0)
    return r


def test_sort_rle_c1_full():
    _sort_rle_vs_numpy(wl.config("C1"))


@pytest.mark.slow
def test_sort_rle_c2_full():
    r = _sort_rle_vs_numpy(wl.config("C2"))
    assert r["n_long"] > 100  # Zipf 1.05 makes hot rows with SL >= 256


@pytest.mark.slow
def test_sort_rle_c4_full():
    r = _sort_rle_vs_numpy(wl.config("C4"))
    assert r["U"] == 64 and r["n_long"] == 64


@pytest.mark.slow
def test_sort_rle_c5_one_table():
    r = _sort_rle_vs_numpy(wl.config("C5", T=1))
    assert r["n_long"] > 100


@pytest.mark.parametrize("sl,kind,chunks", [(255, "short", []), (256, "long", [256]),
                                             (257, "long", [256, 1]), (513, "long", [256, 256, 1])])
def test_run_threshold_and_chunking_edges(sl, kind, chunks):
    """FBTriton page, "Backward": SL < 256 is an owner update, SL >= 256 is cut
    into chunks of 256 lookups in sorted order (the last one may be shorter)."""
    B = sl
    off = np.arange(B + 1, dtype=np.int64)       # one lookup per bag
    idx = np.full(sl, 3, np.int64)               # all on row 3
    r = oracle.preprocess([5], B, "i64", idx, off)
    assert r["U"] == 1
    assert (r["n_short"], r["n_long"]) == ((1, 0) if kind == "short" else (0, 1))
    assert r["chunk_len"].tolist() == chunks
    assert r["chunk_start"].tolist() == [256 * k for k in range(len(chunks))]
