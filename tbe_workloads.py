"""Seeded synthetic TBE inputs shared by the tests, the bench and the smoke run.

This module only draws inputs: table shapes, bag lengths, indices, per-sample
weights, output gradients, weights and momentum.  It holds none of the TBE
arithmetic (no pooling, sorting or optimizer step), so both the CPU oracle and
the HIP path can consume its arrays without sharing any method code.

Workloads follow the five configurations of the TBE problem statement
("Modernizing Table Batched Embeddings with FBTriton", sections "Why redesign
a sparse operator?" and "Backward"): skewed access where most rows are hit
once and a few rows thousands of times.  The pages measured on production
shards that are not public; bounded Zipf draws stand in for them.

Seeding: every array comes from ``numpy.random.default_rng([S, stream, t])``
with S = 1000 + config number and a fixed stream id per array kind, so a table's
data does not change when other tables are added or removed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

# stream ids of the seed sequence [S, stream, t]
ST_LENGTHS, ST_INDICES, ST_PSW, ST_GRAD, ST_WEIGHTS, ST_PERM, ST_MOM = 1, 2, 3, 4, 5, 6, 7

WDTYPES = ("f32", "f16", "bf16")
POOL_SUM, POOL_MEAN = 0, 1
ZIPF_MULT = 2654435761  # odd multiplier of the rank -> row affine permutation


@dataclasses.dataclass
class Spec:
    """Shape and distributions of one TBE workload."""

    name: str
    seed: int                      # S of the seed sequence
    rows: List[int]                # R_t
    dims: List[int]                # D_t
    pooling: List[int]             # POOL_SUM / POOL_MEAN per table
    wdtype: str                    # "f32" | "f16" | "bf16"
    B: int                         # bags per table
    lengths: str                   # "fixed:L" | "uniform:lo:hi" | "poisson:lam:+c"
    index_dist: str                # "uniform" | "zipf:alpha"
    itype: str                     # "i32" | "i64"
    weighted: bool                 # per-sample weights present
    lr: float = 0.01
    eps: float = 1e-8

    @property
    def T(self) -> int:
        return len(self.rows)

    @property
    def dtot(self) -> int:
        return int(sum(self.dims))

    def col_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.dims)[:-1]]).astype(np.int64)

    # ------------------------------------------------------------------ draws
    def _rng(self, stream: int, t: int) -> np.random.Generator:
        return np.random.default_rng([self.seed, stream, t])

    def table_lengths(self, t: int) -> np.ndarray:
        rng = self._rng(ST_LENGTHS, t)
        kind, *args = self.lengths.split(":")
        if kind == "fixed":
            return np.full(self.B, int(args[0]), dtype=np.int64)
        if kind == "uniform":
            lo, hi = int(args[0]), int(args[1])
            return rng.integers(lo, hi + 1, size=self.B, dtype=np.int64)
        if kind == "poisson":
            lam, c = float(args[0]), int(args[1])
            return rng.poisson(lam, size=self.B).astype(np.int64) + c
        if kind == "list":  # explicit per-bag lengths, cycled (edge-case tests)
            vals = [int(v) for v in args[0].split(",")]
            return np.resize(np.array(vals, dtype=np.int64), self.B)
        raise ValueError(self.lengths)

    def lengths_all(self) -> np.ndarray:
        return np.concatenate([self.table_lengths(t) for t in range(self.T)])

    def offsets(self) -> np.ndarray:
        """Table-major CSR offsets, length T*B+1 (bag j = t*B + b)."""
        L = self.lengths_all()
        off = np.zeros(L.size + 1, dtype=np.int64)
        np.cumsum(L, out=off[1:])
        return off.astype(self.np_itype)

    @property
    def np_itype(self):
        return np.int32 if self.itype == "i32" else np.int64

    def table_indices(self, t: int, n: int) -> np.ndarray:
        R = self.rows[t]
        rng = self._rng(ST_INDICES, t)
        kind, *args = self.index_dist.split(":")
        if kind == "uniform":
            return rng.integers(0, R, size=n, dtype=np.int64)
        if kind == "zipf":
            alpha = float(args[0])
            rank0 = zipf_ranks(R, alpha, rng.random(n))
            off = int(self._rng(ST_PERM, t).integers(0, R))
            mult = ZIPF_MULT
            while math.gcd(mult, R) != 1:
                mult += 2
            return (rank0 * (mult % R) + off) % R
        if kind == "const":  # every lookup hits one row (edge-case tests)
            return np.full(n, int(args[0]) % R, dtype=np.int64)
        raise ValueError(self.index_dist)

    def indices(self) -> np.ndarray:
        parts = []
        for t in range(self.T):
            n = int(self.table_lengths(t).sum())
            parts.append(self.table_indices(t, n))
        out = np.concatenate(parts) if parts else np.zeros(0, np.int64)
        return out.astype(self.np_itype)

    def per_sample_weights(self) -> Optional[np.ndarray]:
        if not self.weighted:
            return None
        parts = []
        for t in range(self.T):
            n = int(self.table_lengths(t).sum())
            parts.append(self._rng(ST_PSW, t).random(n, dtype=np.float32))
        return np.concatenate(parts).astype(np.float32)

    def grad_out(self) -> np.ndarray:
        """FP32 [B, Dtot] ~ N(0,1), table t's column block drawn from stream (4, t)."""
        G = np.empty((self.B, self.dtot), dtype=np.float32)
        c = self.col_offsets()
        for t in range(self.T):
            G[:, c[t]:c[t] + self.dims[t]] = self._rng(ST_GRAD, t).standard_normal(
                (self.B, self.dims[t]), dtype=np.float32)
        return G

    def weights_f32(self, t: int) -> np.ndarray:
        """Table t's weights drawn in FP32 ~ U(-0.1, 0.1) before storage rounding."""
        u = self._rng(ST_WEIGHTS, t).random((self.rows[t], self.dims[t]), dtype=np.float32)
        return (u * np.float32(0.2) - np.float32(0.1)).astype(np.float32)

    def momentum(self, t: int, nonzero: bool = False) -> np.ndarray:
        if not nonzero:
            return np.zeros(self.rows[t], dtype=np.float32)
        return self._rng(ST_MOM, t).random(self.rows[t], dtype=np.float32)

    def num_lookups(self) -> int:
        return int(sum(int(self.table_lengths(t).sum()) for t in range(self.T)))


def zipf_ranks(R: int, alpha: float, u: np.ndarray) -> np.ndarray:
    """0-based ranks of a bounded Zipf law P(k) ~ k^-alpha, k = 1..R, by inverse CDF."""
    k = np.arange(1, R + 1, dtype=np.float64)
    cdf = np.cumsum(k ** -alpha)
    cdf /= cdf[-1]
    r = np.searchsorted(cdf, u, side="right")
    return np.minimum(r, R - 1).astype(np.int64)


# --------------------------------------------------------------------------
# The five workloads.  Scaled variants keep every distribution and shrink the
# table heights / bag counts so the oracle finishes in seconds.
# --------------------------------------------------------------------------

def _c3_dims(T):
    return [[32, 96, 128, 160, 256][t % 5] for t in range(T)]


def config(name: str, rows: Optional[int] = None, B: Optional[int] = None,
           T: Optional[int] = None) -> Spec:
    """Build a workload by name (C1..C5); rows/B/T override the sizes."""
    if name == "C1":  # tiny correctness workload
        T = T or 1
        R = rows or 1000
        return Spec("C1", 1001, [R] * T, [64] * T, [POOL_SUM] * T, "f32", B or 128,
                    "fixed:8", "uniform", "i64", False)
    if name == "C2":  # 8 x 1M rows, D 64/128 alternating, fp16, Zipf 1.05
        T = T or 8
        R = rows or 1_000_000
        return Spec("C2", 1002, [R] * T, [64 if t % 2 == 0 else 128 for t in range(T)],
                    [POOL_SUM] * T, "f16", B or 8192, "uniform:1:64", "zipf:1.05", "i64", False)
    if name == "C3":  # 16 x 2M rows, mixed D, bf16, Zipf 1.2, weighted, half mean
        T = T or 16
        R = rows or 2_000_000
        return Spec("C3", 1003, [R] * T, _c3_dims(T),
                    [POOL_SUM if t % 2 == 0 else POOL_MEAN for t in range(T)], "bf16",
                    B or 16384, "uniform:1:128", "zipf:1.2", "i64", True)
    if name == "C4":  # small-table histogram workload: 64 x 128 fp16, L=128
        R = rows or 64
        return Spec("C4", 1004, [R], [128], [POOL_SUM], "f16", B or 65536,
                    "fixed:128", "uniform", "i64", False)
    if name == "C5":  # 64 x 5M x 128 fp16, int32, Poisson(32)+1, Zipf 1.1
        T = T or 64
        R = rows or 5_000_000
        return Spec("C5", 1005, [R] * T, [128] * T, [POOL_SUM] * T, "f16", B or 65536,
                    "poisson:32:1", "zipf:1.1", "i32", False)
    raise KeyError(name)


CONFIG_NAMES = ("C1", "C2", "C3", "C4", "C5")

DESCRIPTIONS = {
    "C1": "1 table 1000x64 fp32, B=128, L=8 uniform, int64, sum",
    "C2": "8 tables x 1M rows, D 64/128, fp16, B=8192, L~U[1,64], Zipf 1.05, int64, sum",
    "C3": "16 tables x 2M rows, D in {32,96,128,160,256}, bf16, B=16384, L~U[1,128], "
          "Zipf 1.2, per-sample weights, half mean",
    "C4": "1 table 64x128 fp16, B=65536, L=128 uniform (histogram path)",
    "C5": "64 tables x 5M x 128 fp16, int32, B=65536, L~Poisson(32)+1, Zipf 1.1",
}


def random_tiny(seed: int, max_T=3, max_R=8, max_B=5, max_L=6, max_D=5) -> dict:
    """A random tiny problem for brute-force checks (all arrays host numpy)."""
    rng = np.random.default_rng([7, seed])
    T = int(rng.integers(1, max_T + 1))
    rows = [int(rng.integers(1, max_R + 1)) for _ in range(T)]
    dims = [int(rng.integers(1, max_D + 1)) for _ in range(T)]
    pooling = [int(rng.integers(0, 2)) for _ in range(T)]
    wdtype = WDTYPES[int(rng.integers(0, 3))]
    itype = "i32" if rng.integers(0, 2) else "i64"
    B = int(rng.integers(1, max_B + 1))
    L = rng.integers(0, max_L + 1, size=T * B)
    off = np.zeros(T * B + 1, np.int64)
    np.cumsum(L, out=off[1:])
    idx = np.concatenate([rng.integers(0, rows[j // B], size=int(L[j])) for j in range(T * B)]
                         ) if off[-1] else np.zeros(0, np.int64)
    weighted = bool(rng.integers(0, 2))
    psw = rng.random(int(off[-1])).astype(np.float32) if weighted else None
    W = [(rng.random((rows[t], dims[t]), dtype=np.float32) * 0.2 - 0.1) for t in range(T)]
    M = [(rng.random(rows[t], dtype=np.float32) * np.float32(rng.integers(0, 2))).astype(np.float32)
         for t in range(T)]
    G = rng.standard_normal((B, int(sum(dims))), dtype=np.float32)
    npi = np.int32 if itype == "i32" else np.int64
    return dict(T=T, rows=rows, dims=dims, pooling=pooling, wdtype=wdtype, itype=itype, B=B,
                offsets=off.astype(npi), indices=idx.astype(npi), psw=psw, W32=W, M=M, G=G,
                lr=float(rng.choice([0.01, 0.5])), eps=float(rng.choice([1e-8, 0.3])))


def to_storage(w32: np.ndarray, wdtype: str) -> np.ndarray:
    """Round FP32 draws to the storage type (RNE): float32, or raw uint16 bits."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    if wdtype == "f32":
        return w32.copy()
    if wdtype == "f16":
        return w32.astype(np.float16).view(np.uint16)
    import torch  # bfloat16 rounding of the draws
    return torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def storage_to_f64(stored: np.ndarray, wdtype: str) -> np.ndarray:
    """Exact widening of stored weights to float64 (for assertions)."""
    if wdtype == "f32":
        return stored.astype(np.float64)
    if wdtype == "f16":
        return stored.view(np.float16).astype(np.float64)
    return (stored.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
