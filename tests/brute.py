"""Brute-force TBE in pure Python for tiny inputs (test helper, no sorting).

Forward pools each bag by walking its lookups.  Backward gathers each row's
gradient in a dict keyed by (table, row) while walking the bags in their
natural order, then applies row-wise Adagrad once per key.  It shares nothing
with the C oracle: no sort, no run-length encoding, no chunking.  Definitions:
FBTriton TBE page ("Forward"; "Backward": every gradient of a row gathered and
applied exactly once; "Fusion boundaries": per-sample weights scale each
contribution), HugeCTR walkthrough (mean = sum scaled by 1/L, backward mean
scales by 1/L; Adagrad with eps outside the root).
"""
import math

import numpy as np


def forward(p):
    T, B = p["T"], p["B"]
    off, idx, psw = p["offsets"], p["indices"], p["psw"]
    W = p["Wf64"]
    out = [[0.0] * sum(p["dims"]) for _ in range(B)]
    col = 0
    for t in range(T):
        D = p["dims"][t]
        for b in range(B):
            j = t * B + b
            lo, hi = int(off[j]), int(off[j + 1])
            acc = [0.0] * D
            for q in range(lo, hi):
                s = 1.0 if psw is None else float(psw[q])
                row = W[t][int(idx[q])]
                for d in range(D):
                    acc[d] += s * float(row[d])
            if p["pooling"][t] == 1 and hi > lo:
                acc = [a / (hi - lo) for a in acc]
            for d in range(D):
                out[b][col + d] = acc[d]
        col += D
    return np.array(out, dtype=np.float64).reshape(B, sum(p["dims"]))


def row_gradients(p):
    """{(t, r): [g_0..g_{D-1}]} for every touched row."""
    T, B = p["T"], p["B"]
    off, idx, psw, G = p["offsets"], p["indices"], p["psw"], p["G"]
    grads = {}
    col = 0
    for t in range(T):
        D = p["dims"][t]
        for b in range(B):
            j = t * B + b
            lo, hi = int(off[j]), int(off[j + 1])
            for q in range(lo, hi):
                s = 1.0 if psw is None else float(psw[q])
                if p["pooling"][t] == 1:
                    s /= (hi - lo)
                key = (t, int(idx[q]))
                g = grads.setdefault(key, [0.0] * D)
                for d in range(D):
                    g[d] += s * float(G[b, col + d])
        col += D
    return grads


def adagrad(p):
    """Returns (W_new as float64 before storage rounding, M_new float64) per table."""
    grads = row_gradients(p)
    W = [w.copy() for w in p["Wf64"]]
    M = [m.astype(np.float64).copy() for m in p["M"]]
    lr = float(np.float32(p["lr"]))
    eps = float(np.float32(p["eps"]))
    for (t, r), g in grads.items():
        D = p["dims"][t]
        m = float(M[t][r]) + sum(x * x for x in g) / D
        m = float(np.float32(m))
        M[t][r] = m
        den = math.sqrt(m) + eps
        for d in range(D):
            W[t][r, d] = W[t][r, d] - lr * g[d] / den
    return W, M, set(grads)


def update(p, optimizer, state0=None):
    """SGD or element-wise Adagrad applied once per touched row (HugeCTR
    walkthrough, step 5: the element-wise accumulator A[r, d] += g[d]^2,
    stored as float32, eps outside the root).  Returns (W float64 before
    storage rounding, state float64 or None, touched keys)."""
    grads = row_gradients(p)
    W = [w.copy() for w in p["Wf64"]]
    A = None if optimizer == "sgd" else [a.astype(np.float64).copy() for a in state0]
    lr = float(np.float32(p["lr"]))
    eps = float(np.float32(p["eps"]))
    for (t, r), g in grads.items():
        D = p["dims"][t]
        for d in range(D):
            if optimizer == "sgd":
                W[t][r, d] = W[t][r, d] - lr * g[d]
            else:
                a = float(np.float32(A[t][r, d] + g[d] * g[d]))
                A[t][r, d] = a
                W[t][r, d] = W[t][r, d] - lr * g[d] / (math.sqrt(a) + eps)
    return W, A, set(grads)
