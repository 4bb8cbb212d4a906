"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Workloads are the five configurations with every distribution kept and the
sizes scaled so the oracle finishes in seconds while still spanning several
4096-key tiles with a ragged tail, plus edge cases: empty bags, an all-empty
batch, B = 1, a one-row table, runs of exactly 255/256/257 lookups, D = 4 and
D = 1024, D not a multiple of 8, many tables over every bucket, int32 indices,
mean pooling with per-sample weights, non-zero initial momentum.

Bars: integer outputs bit-exact; pooled outputs |d| <= 1e-4 max(1,|ref|);
16-bit weights within 2 ulp, float32 weights within 1e-6 max(1,|ref|);
momentum within 1e-5 relative; untouched rows bit-identical; fused and
two-launch long-run paths bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import tbe_workloads as wl
from tests import support as S

pytestmark = pytest.mark.gpu


def _spec(name):
    if name == "C1":
        return wl.config("C1")
    if name == "C2s":
        return wl.config("C2", rows=20000, B=512, T=4)
    if name == "C3s":
        return wl.config("C3", rows=50000, B=256, T=10)
    if name == "C4s":
        return wl.config("C4", B=2048)
    if name == "C5s":
        return wl.config("C5", rows=200000, B=2048, T=3)
    if name == "empty_bags":
        return wl.Spec("empty_bags", 2001, [100, 37, 60], [8, 36, 4], [0, 1, 1], "f16", 33,
                       "list:0,3,0,5,1,0,0,9", "uniform", "i64", True)
    if name == "all_empty":
        return wl.Spec("all_empty", 2002, [10, 10], [16, 32], [0, 1], "bf16", 7, "list:0",
                       "uniform", "i64", False)
    if name == "one_bag":
        return wl.Spec("one_bag", 2003, [1000], [128], [1], "f16", 1, "fixed:700",
                       "zipf:1.3", "i32", True)
    if name == "one_row":
        return wl.Spec("one_row", 2004, [1], [16], [0], "f32", 3, "fixed:300", "uniform",
                       "i64", False)
    if name.startswith("const"):
        n = int(name[5:])
        return wl.Spec(name, 2005, [9], [64], [0], "bf16", n, "fixed:1", "const:5", "i64",
                       True)
    if name == "wide_f32":
        return wl.Spec("wide_f32", 2006, [300, 50], [1024, 512], [0, 1], "f32", 64,
                       "uniform:0:40", "zipf:1.2", "i64", True)
    if name == "wide_bf16":
        return wl.Spec("wide_bf16", 2007, [300, 20], [1024, 4], [1, 0], "bf16", 64,
                       "uniform:1:30", "zipf:1.1", "i32", False)
    if name == "many_tables":
        dims = [4, 12, 64, 100, 128, 256, 512, 1024, 36, 8]
        T = 40
        return wl.Spec("many_tables", 2008, [int(50 + 37 * t) for t in range(T)],
                       [dims[t % len(dims)] for t in range(T)], [t % 2 for t in range(T)],
                       "f16", 40, "uniform:0:12", "zipf:1.05", "i32", True)
    if name == "many_bags":
        # 12000 bags: the transposition gives each workgroup several bags
        return wl.Spec("many_bags", 2009, [3000, 500], [16, 64], [0, 1], "f16", 6000,
                       "uniform:0:20", "zipf:1.1", "i32", True)
    if name == "cut_bags":
        # bags of 0 .. 900 lookups next to each other: the forward's equal
        # pieces cut long bags many times and fall on empty bags (32 and 64
        # subgroups per wave with D = 16 and D = 8 f16 rows)
        return wl.Spec("cut_bags", 2011, [700, 90, 400], [16, 16, 8], [0, 1, 0], "f16", 200,
                       "list:0,0,1,900,0,2,0,0,150,3,0,64,0,0,0,0,33,1,1,2000,7",
                       "zipf:1.05", "i32", True)
    if name == "heavy_chunks":
        # 32 runs of 32768 lookups: one classification tile with 4096 chunks,
        # which the whole workgroup places
        return wl.Spec("heavy_chunks", 2010, [32], [16], [0], "f32", 4096, "fixed:256",
                       "uniform", "i32", False)
    if name == "dense_mean":
        # hot rows of mean and sum tables without per-sample weights (integer
        # counts times 1/L), D = 256 beside narrower tiles, and a D = 40
        # table that cannot take the contraction
        return wl.Spec("dense_mean", 2014, [5000, 3000, 800, 2000], [128, 64, 40, 256],
                       [1, 0, 1, 1], "f16", 2048, "uniform:1:64", "zipf:1.2", "i64", False)
    if name == "dense_many":
        # more long runs than the contraction takes: its threshold is searched
        return wl.Spec("dense_many", 2015, [3000], [32], [0], "bf16", 16384, "fixed:64",
                       "zipf:1.05", "i32", False)
    if name == "dense_half":
        # 223 long runs, all taken: the second 128 hot rows partly filled
        return wl.Spec("dense_half", 2017, [3000], [32], [0], "bf16", 8192, "fixed:64",
                       "zipf:1.05", "i32", False)
    if name == "dense_wide":
        # bags of up to 2000 lookups from 50 rows: hot-row counts above 255 in
        # a bag, which enter the contraction in 8-bit parts
        return wl.Spec("dense_wide", 2016, [50, 300], [64, 160], [0, 1], "f32", 512,
                       "list:300,1,2000,5,700,0,64", "zipf:1.5", "i64", False)
    if name == "sparse_bags":
        # one bag in ten holds lookups: a 4096-lookup sort tile spans more
        # than 4096 bags, so the first pass finds bags in global memory
        return wl.Spec("sparse_bags", 2018, [3000, 500], [16, 32], [1, 0], "f16", 20000,
                       "list:0,0,0,0,0,0,0,0,0,3", "zipf:1.1", "i32", True)
    if name == "thin_bags":
        # about 1.9 lookups per bag: a tile's window of offsets (about 2200
        # bags) is padded to the full 4096 LDS entries
        return wl.Spec("thin_bags", 2019, [4000, 1000], [8, 64], [0, 1], "bf16", 30000,
                       "list:0,5,0,0,7,1,0", "zipf:1.2", "i64", True)
    if name == "rows_21b":
        # 21 row bits: three 8-bit radix passes (an odd count) at a small size
        return wl.Spec("rows_21b", 2012, [(1 << 20) + 3, 50], [8, 16], [0, 1], "f16", 300,
                       "uniform:1:20", "uniform", "i32", True)
    if name == "rows_25b":
        # 25 row bits: three 10-bit radix passes
        return wl.Spec("rows_25b", 2013, [(1 << 24) + 5], [4], [1], "f32", 128,
                       "uniform:1:16", "uniform", "i64", False)
    raise KeyError(name)


MAIN = ["C1", "C2s", "C3s", "C4s", "C5s"]
EDGE = ["empty_bags", "all_empty", "one_bag", "one_row", "const31", "const32", "const255",
        "const256", "const257", "wide_f32", "wide_bf16", "many_tables", "many_bags",
        "heavy_chunks", "cut_bags", "dense_mean", "dense_wide", "rows_21b", "rows_25b",
        "sparse_bags", "thin_bags"]


def _announce(name, what):
    print(f"[gpu] {what} case={name}", flush=True)


@pytest.mark.parametrize("split", ["one_bag", "balanced"])
@pytest.mark.parametrize("name", MAIN + EDGE)
def test_forward_parity(name, split):
    _announce(name, f"forward {split}")
    case = S.Case(_spec(name))
    tb = case.tbe()
    import table_embedding_amd as te
    f = te.TBE_FWD_NO_BALANCE if split == "one_bag" else te.TBE_FWD_BALANCE
    out = tb.forward(case.spec.B, case.d_idx, case.d_off, case.d_psw,
                     flags=te.TBE_FWD_NO_HIST | f)
    torch.cuda.synchronize()
    S.check_forward(case, out)


@pytest.mark.parametrize("name", ["C2s", "C3s", "empty_bags", "many_tables", "wide_f32",
                                  "cut_bags"])
def test_forward_deterministic(name):
    """The order of every forward sum follows from the offsets alone: repeated
    calls give the same bits with either bag split, and the default is the
    equal-piece split."""
    _announce(name, "forward determinism")
    import table_embedding_amd as te
    case = S.Case(_spec(name))
    tb = case.tbe()

    def run(f):
        return tb.forward(case.spec.B, case.d_idx, case.d_off, case.d_psw,
                          flags=te.TBE_FWD_NO_HIST | f).cpu().numpy().tobytes()
    one, bal, dflt = run(te.TBE_FWD_NO_BALANCE), run(te.TBE_FWD_BALANCE), run(0)
    assert run(te.TBE_FWD_NO_BALANCE) == one
    assert run(te.TBE_FWD_BALANCE) == bal
    assert dflt == bal


@pytest.mark.parametrize("name", MAIN + EDGE)
def test_preprocess_bit_exact(name):
    _announce(name, "preprocess")
    case = S.Case(_spec(name))
    if case.N == 0:
        pytest.skip("no lookups: preprocessing enqueues nothing")
    tb = case.tbe()
    tb.preprocess(case.spec.B, case.d_idx, case.d_off, case.d_psw)
    torch.cuda.synchronize()
    S.check_preprocess(case, tb)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", MAIN + EDGE)
def test_backward_parity(name, fused):
    _announce(name, f"backward fused={fused}")
    import table_embedding_amd as te
    case = S.Case(_spec(name), m_nonzero=(name in ("C2s", "C3s", "wide_f32")))
    tb = case.tbe()
    flags = te.TBE_BWD_FUSED_LONG if fused else 0
    tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                case.spec.eps, flags=flags)
    torch.cuda.synchronize()
    S.check_backward(case, tb)


@pytest.mark.parametrize("name", ["C2s", "C3s", "C4s", "const257", "one_row"])
def test_fused_equals_two_launch_bitwise(name):
    _announce(name, "fused-vs-two-launch")
    import table_embedding_amd as te
    case = S.Case(_spec(name), m_nonzero=True)
    res = []
    for flags in (0, te.TBE_BWD_FUSED_LONG, te.TBE_BWD_FUSED_LONG, 0):
        case.reset_tables()
        tb = case.tbe()
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps, flags=flags)
        torch.cuda.synchronize()
        res.append([S.to_host_storage(w, case.spec.wdtype).tobytes() for w in tb.weights] +
                   [m.cpu().numpy().tobytes() for m in tb.momentum])
        tb.close()
    assert res[0] == res[1] == res[2] == res[3]


@pytest.mark.parametrize("name", ["C2s", "C3s", "C5s"])
def test_every_touched_row_updated_once(name):
    _announce(name, "debug-count")
    case = S.Case(_spec(name))
    tb = case.tbe()
    nkeys = sum(case.spec.rows)
    cnt = torch.zeros(nkeys, dtype=torch.uint32, device="cuda")
    tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                case.spec.eps, debug_row_updates=cnt)
    torch.cuda.synchronize()
    c = cnt.cpu().numpy()
    kb = tb.key_bases()
    for t in range(case.spec.T):
        seg = c[kb[t]:kb[t] + case.spec.rows[t]]
        want = np.zeros(case.spec.rows[t], np.int32)
        want[S.touched_rows(case, t)] = 1
        assert np.array_equal(seg, want), f"table {t}"


def test_preprocessed_flag_and_reuse():
    """tbe_preprocess then backward(PREPROCESSED) equals a self-preprocessing backward;
    the fused countdowns are re-armed, so a second fused backward on the same
    preprocessed workspace is still exact."""
    import table_embedding_amd as te
    case = S.Case(_spec("C2s"))
    tb = case.tbe()
    tb.preprocess(case.spec.B, case.d_idx, case.d_off)
    tb.backward(case.spec.B, case.d_idx, case.d_off, None, case.d_G, case.spec.lr,
                case.spec.eps, flags=te.TBE_BWD_PREPROCESSED | te.TBE_BWD_FUSED_LONG)
    torch.cuda.synchronize()
    S.check_backward(case, tb)
    a = [S.to_host_storage(w, "f16").tobytes() for w in tb.weights]
    case.reset_tables()
    tb2 = case.tbe()
    tb2._ws = tb._ws  # same preprocessed workspace, second fused use
    tb2.backward(case.spec.B, case.d_idx, case.d_off, None, case.d_G, case.spec.lr,
                 case.spec.eps, flags=te.TBE_BWD_PREPROCESSED | te.TBE_BWD_FUSED_LONG)
    torch.cuda.synchronize()
    assert [S.to_host_storage(w, "f16").tobytes() for w in tb2.weights] == a


def test_preprocessed_flag_with_weights_and_mean():
    """Per-sample weights and mean pooling are folded into the preprocessing."""
    import table_embedding_amd as te
    case = S.Case(_spec("C3s"))
    tb = case.tbe()
    tb.preprocess(case.spec.B, case.d_idx, case.d_off, case.d_psw)
    tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                case.spec.eps, flags=te.TBE_BWD_PREPROCESSED)
    torch.cuda.synchronize()
    S.check_backward(case, tb)


def test_histogram_path_forward():
    import table_embedding_amd as te
    for name in ("C4s",):
        _announce(name, "histogram forward")
        case = S.Case(_spec(name))
        tb = case.tbe()
        out = tb.forward(case.spec.B, case.d_idx, case.d_off, None,
                         flags=te.TBE_FWD_REQUIRE_HIST)
        torch.cuda.synchronize()
        S.check_forward(case, out)


def test_histogram_path_long_bags_and_mean():
    """Bags longer than the 256 counted lookups (scalar remainder), ragged B, mean pooling."""
    import table_embedding_amd as te
    spec = wl.Spec("hist_long", 2010, [50], [96], [1], "f16", 37, "uniform:64:700", "uniform",
                   "i64", False)
    case = S.Case(spec)
    tb = case.tbe()
    out = tb.forward(spec.B, case.d_idx, case.d_off, None, flags=te.TBE_FWD_REQUIRE_HIST)
    torch.cuda.synchronize()
    S.check_forward(case, out)


def test_repeat_runs_bitwise_identical():
    import table_embedding_amd as te
    case = S.Case(_spec("C3s"))
    outs, ws = [], []
    for _ in range(3):
        case.reset_tables()
        tb = case.tbe()
        o = tb.forward(case.spec.B, case.d_idx, case.d_off, case.d_psw)
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps)
        torch.cuda.synchronize()
        outs.append(o.cpu().numpy().tobytes())
        ws.append([S.to_host_storage(w, "bf16").tobytes() for w in tb.weights])
    assert outs[0] == outs[1] == outs[2]
    assert ws[0] == ws[1] == ws[2]


def _tables_bytes(tb, wdtype):
    return ([S.to_host_storage(w, wdtype).tobytes() for w in tb.weights] +
            [m.cpu().numpy().tobytes() for m in tb.momentum])


@pytest.mark.parametrize("name", ["C2s", "C3s", "C5s", "many_tables", "const257"])
@pytest.mark.parametrize("fused", [False, True])
def test_concurrent_backward_equals_one_stream(name, fused):
    """The run classes on three streams give the same bits as one stream: they
    own disjoint rows and every sum is in a data-determined order."""
    _announce(name, f"concurrent-vs-one-stream fused={fused}")
    import table_embedding_amd as te
    case = S.Case(_spec(name), m_nonzero=True)
    res = []
    base = te.TBE_BWD_FUSED_LONG if fused else 0
    for flags in (base, base | te.TBE_BWD_CONCURRENT, base | te.TBE_BWD_CONCURRENT_AUTO, base):
        case.reset_tables()
        tb = case.tbe()
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps, flags=flags)
        torch.cuda.synchronize()
        res.append(_tables_bytes(tb, case.spec.wdtype))
        tb.close()
    assert res[0] == res[1] == res[2] == res[3]


@pytest.mark.parametrize("name", ["C2s", "C3s", "empty_bags", "wide_f32"])
def test_forward_and_preprocess_schedule(name):
    """Forward with the preprocessing on a side stream (tbe_forward_preprocess),
    then backward on the preprocessed workspace: same output and tables as
    forward then a self-preprocessing backward on one stream, and within the
    oracle's bars.  Then two more steps of each, enqueued without waiting: the
    next step's preprocessing must wait for the backward that reads the
    workspace, so the bits still match step for step."""
    _announce(name, "forward||preprocess schedule")
    import table_embedding_amd as te
    case = S.Case(_spec(name), m_nonzero=True)
    if case.N == 0:
        pytest.skip("no lookups")
    B = case.spec.B
    tb = case.tbe()

    def overlapped():
        o = tb.forward_and_preprocess(B, case.d_idx, case.d_off, case.d_psw)
        tb.backward(B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps, flags=te.TBE_BWD_PREPROCESSED | te.TBE_BWD_CONCURRENT)
        return o
    out = overlapped()
    torch.cuda.synchronize()
    S.check_forward(case, out)
    S.check_backward(case, tb)
    got = [(out.cpu().numpy().tobytes(), _tables_bytes(tb, case.spec.wdtype))]
    outs = [overlapped() for _ in range(2)]
    torch.cuda.synchronize()
    got.append((outs[-1].cpu().numpy().tobytes(), _tables_bytes(tb, case.spec.wdtype)))
    case.reset_tables()
    tb2 = case.tbe()

    def serial():
        o = tb2.forward(B, case.d_idx, case.d_off, case.d_psw)
        tb2.backward(B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                     case.spec.eps)
        return o
    out2 = serial()
    torch.cuda.synchronize()
    assert got[0] == (out2.cpu().numpy().tobytes(), _tables_bytes(tb2, case.spec.wdtype))
    outs2 = [serial() for _ in range(2)]
    torch.cuda.synchronize()
    assert got[1] == (outs2[-1].cpu().numpy().tobytes(), _tables_bytes(tb2, case.spec.wdtype))


@pytest.mark.parametrize("name", ["C3s", "C5s", "many_tables", "const257"])
@pytest.mark.parametrize("fused", [False, True])
def test_chunk_order_changes_no_bit(name, fused):
    """Walking each table's chunks in bag order (forced; by default only when
    grad_out exceeds 256 MiB) gives the same bits as list order, within the
    oracle's bars; the walk order is a permutation of each (table, position
    mod 8) class, by non-decreasing bag of the chunk's first lookup."""
    _announce(name, f"chunk-order fused={fused}")
    import table_embedding_amd as te
    case = S.Case(_spec(name), m_nonzero=True)
    base = te.TBE_BWD_FUSED_LONG if fused else 0
    res = []
    for flags in (base | te.TBE_BWD_NO_ORDER_CHUNKS, base | te.TBE_BWD_ORDER_CHUNKS):
        case.reset_tables()
        tb = case.tbe()
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps, flags=flags)
        torch.cuda.synchronize()
        res.append(_tables_bytes(tb, case.spec.wdtype))
        if flags & te.TBE_BWD_ORDER_CHUNKS:
            S.check_backward(case, tb)
            g = S.gpu_preprocess_views(tb, case)
            v = te.tbe_workspace_views(tb.plan, case.spec.B, case.N)
            nc = g["n_chunks"]
            perm = S.read_u32(tb._ws, v["chunk_perm"], nc).astype(np.int64)
            ct = g["chunk_task"]
            B = case.spec.B
            for t in np.unique(ct[:, 2]) if nc else []:
                pos = np.nonzero(ct[:, 2] == t)[0]
                for x in range(8):
                    cls = pos[pos % 8 == x]
                    got = perm[cls]
                    assert np.array_equal(np.sort(got), cls), "not a permutation of the class"
                    bag = g["sorted_bag"][ct[got, 0]] - t * B
                    bins = bag * 256 // B
                    assert np.all(np.diff(bins) >= 0), "walk not in bag order"
        tb.close()
    assert res[0] == res[1]


def _hist_spec(name):
    # one small table: E rows, D a multiple of 16 up to 128
    if name == "hist_c4":
        return wl.config("C4", B=2048)
    if name == "hist_mean_psw":
        return wl.Spec("hist_mean_psw", 2011, [37], [48], [1], "bf16", 777, "uniform:0:150",
                       "uniform", "i64", True)
    if name == "hist_f32_d16":
        return wl.Spec("hist_f32_d16", 2012, [64], [16], [0], "f32", 300, "poisson:20:+1",
                       "zipf:1.2", "i32", False)
    if name == "hist_one_row":
        return wl.Spec("hist_one_row", 2013, [1], [128], [0], "f16", 129, "fixed:3", "uniform",
                       "i32", True)
    if name == "hist_many_bags":
        # more bags than 256 workgroups x 128: every workgroup takes several blocks
        return wl.Spec("hist_many_bags", 2014, [50], [32], [1], "f16", 40000, "uniform:0:6",
                       "zipf:1.05", "i32", False)
    raise KeyError(name)


HIST = ["hist_c4", "hist_mean_psw", "hist_f32_d16", "hist_one_row", "hist_many_bags"]


@pytest.mark.parametrize("name", HIST)
def test_backward_hist_parity(name):
    """Histogram-reuse backward (one contraction over the bags on the matrix
    cores) against the oracle: weights within 2 ulp (16-bit) / 1e-6 (fp32),
    momentum within 1e-5 relative, untouched rows bit-identical, every
    touched row updated once, repeated calls bit-identical."""
    _announce(name, "backward hist")
    import table_embedding_amd as te
    case = S.Case(_hist_spec(name), m_nonzero=True)
    res = []
    for rep in range(2):
        case.reset_tables()
        tb = case.tbe()
        dbg = torch.zeros(sum(case.spec.rows), dtype=torch.uint32, device="cuda")
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps, flags=te.TBE_BWD_HIST, debug_row_updates=dbg)
        torch.cuda.synchronize()
        if rep == 0:
            S.check_backward(case, tb)
            want = np.zeros(case.spec.rows[0], np.int32)
            want[S.touched_rows(case, 0)] = 1
            assert np.array_equal(dbg.cpu().numpy(), want), "each touched row once"
        res.append(_tables_bytes(tb, case.spec.wdtype))
        tb.close()
    assert res[0] == res[1]


def test_backward_hist_unsupported():
    """A plan the histogram backward does not serve is refused before any launch."""
    import table_embedding_amd as te
    case = S.Case(_spec("C2s"))
    tb = case.tbe()
    with pytest.raises(te.TBEError) as ei:
        tb.backward(case.spec.B, case.d_idx, case.d_off, case.d_psw, case.d_G, case.spec.lr,
                    case.spec.eps, flags=te.TBE_BWD_HIST)
    assert ei.value.code == te.TBE_E_UNSUPPORTED
    tb.close()


@pytest.mark.parametrize("name", ["C2s", "C3s", "const257"])
def test_graph_capture_replays_equal_eager(name):
    """A forward + backward step (preprocessing inside, one stream) captured in
    a HIP graph: the step launches kernels only (no allocation, copy or memset),
    so it can be captured.  Three replays, with eager steps of another plan and
    synchronizations between them, each give the bits of the same number of
    eager steps."""
    _announce(name, "graph capture")
    import table_embedding_amd as te
    case = S.Case(_spec(name))
    B = case.spec.B
    tb = case.tbe()
    ws = tb.workspace(B, case.N)
    out = torch.empty((B, case.spec.dtot), dtype=torch.float32, device="cuda")

    def step(t, w, o):
        te.tbe_forward(t.plan, B, case.d_idx, case.d_off, case.N, case.d_psw, o)
        te.tbe_backward_rowwise_adagrad(t.plan, B, case.d_idx, case.d_off, case.N, case.d_psw,
                                        case.d_G, case.spec.lr, case.spec.eps, w, 0)
    step(tb, ws, out)  # first calls outside the capture (per-kernel occupancy queries)
    torch.cuda.synchronize()
    case.reset_tables()
    tb = case.tbe()
    ws = tb.workspace(B, case.N)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(tb, ws, out)
    torch.cuda.synchronize()
    case.reset_tables()  # the eager plan gets its own copy of the initial tables
    tb2 = case.tbe()
    ws2 = tb2.workspace(B, case.N)
    out2 = torch.empty_like(out)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        step(tb2, ws2, out2)
        torch.cuda.synchronize()
        assert (out.cpu().numpy().tobytes(), _tables_bytes(tb, case.spec.wdtype)) == \
            (out2.cpu().numpy().tobytes(), _tables_bytes(tb2, case.spec.wdtype)), r
    del g


def test_forward_table_over_4gib():
    """A table of more than 4 GiB (2^25 + 1024 rows x 64 f16) beside a small one:
    the equal-piece forward reads rows with 32-bit byte offsets, so for this plan
    the host falls back to one bag per subgroup (64-bit addresses).  Lookups of
    rows near the end of the big table (byte offsets past 2^32) and near its
    start pool as the oracle pools the same rows renumbered into a compact
    table; the default and TBE_FWD_NO_BALANCE give the same bits."""
    import table_embedding_amd as te
    _announce("table_over_4gib", "forward")
    R0, D0, R1, D1, B = (1 << 25) + 1024, 64, 100, 32, 64
    assert R0 * D0 * 2 > (1 << 32)
    rng = np.random.default_rng(2012)
    hot = np.concatenate([R0 - 1 - 7919 * np.arange(40), np.arange(10)]).astype(np.int64)
    lengths = rng.integers(0, 9, size=2 * B)
    off = np.zeros(2 * B + 1, np.int64)
    np.cumsum(lengths, out=off[1:])
    n0 = int(off[B])
    idx = np.concatenate([hot[rng.integers(0, hot.size, size=n0)],
                          rng.integers(0, R1, size=int(off[-1]) - n0)]).astype(np.int64)
    vals = rng.uniform(-1, 1, size=(hot.size, D0)).astype(np.float16)
    small = rng.uniform(-1, 1, size=(R1, D1)).astype(np.float16)
    big = torch.empty((R0, D0), dtype=torch.float16, device="cuda")
    big[torch.from_numpy(hot).cuda()] = torch.from_numpy(vals).cuda()
    W = [big, torch.from_numpy(small).cuda()]
    M = [torch.zeros(R0, device="cuda"), torch.zeros(R1, device="cuda")]
    tb = te.TBE([R0, R1], [D0, D1], [0, 1], W, M)
    d_idx, d_off = torch.from_numpy(idx).cuda(), torch.from_numpy(off).cuda()
    got = tb.forward(B, d_idx, d_off, None, flags=te.TBE_FWD_NO_HIST)
    got1 = tb.forward(B, d_idx, d_off, None, flags=te.TBE_FWD_NO_HIST | te.TBE_FWD_NO_BALANCE)
    torch.cuda.synchronize()
    assert got.cpu().numpy().tobytes() == got1.cpu().numpy().tobytes()
    # the oracle on the touched rows, renumbered: row hot[k] of table 0 becomes row k
    renum = {int(r): k for k, r in enumerate(hot)}
    idx_c = idx.copy()
    idx_c[:n0] = [renum[int(r)] for r in idx[:n0]]
    ref = oracle.forward([hot.size, R1], [D0, D1], [0, 1], "f16",
                         [vals.view(np.uint16), small.view(np.uint16)], B, "i64", idx_c, off)
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() <= 1e-4, err.max()
    tb.close()
    del big, W, M
    torch.cuda.empty_cache()
