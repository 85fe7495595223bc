"""Pure-Python twin of the fp64 oracle, for tiny inputs (TEST INFRASTRUCTURE ONLY).

Written independently of ``oracle.cpp`` from the same definitions, with lists and
Python floats (IEEE fp64), so the two can be cross-checked element by element.

Pages cited: Page A = upppp.jp TwELL article of 2026-05-11.
"""
from __future__ import annotations


def up_relu(x, W_up, b):
    """ReLU(x W_up^T + b), ascending-i sum then bias (Page A, "What is the waste in LLM
    FFN layers")."""
    T, D, F = len(x), len(x[0]), len(W_up)
    h = [[0.0] * F for _ in range(T)]
    for t in range(T):
        for j in range(F):
            acc = 0.0
            for i in range(D):
                acc += x[t][i] * W_up[j][i]
            acc += b[j]
            h[t][j] = acc if acc > 0.0 else 0.0
    return h


def pack(h, K, W):
    """TwELL pack (Page A, "What TwELL and the custom CUDA kernels solve").

    Returns (counts[k][t], vals[k][t][s], cols[k][t][s], backup) where backup is a
    list of (k, t, slice) in ascending (k, t); slice holds the nonzeros of rank >= W.
    """
    T, F = len(h), len(h[0])
    nt = F // K
    counts = [[0] * T for _ in range(nt)]
    vals = [[[0.0] * W for _ in range(T)] for _ in range(nt)]
    cols = [[[0] * W for _ in range(T)] for _ in range(nt)]
    backup = []
    for k in range(nt):
        for t in range(T):
            nz = [(c, h[t][k * K + c]) for c in range(K) if h[t][k * K + c] != 0.0]
            counts[k][t] = len(nz)
            for s, (c, v) in enumerate(nz[:W]):
                vals[k][t][s] = v
                cols[k][t][s] = c
            if len(nz) > W:
                sl = [0.0] * K
                for c, v in nz[W:]:
                    sl[c] = v
                backup.append((k, t, sl))
    return counts, vals, cols, backup


def unpack(counts, vals, cols, backup, T, F, K, W):
    h = [[0.0] * F for _ in range(T)]
    for k in range(len(counts)):
        for t in range(T):
            for s in range(min(counts[k][t], W)):
                h[t][k * K + cols[k][t][s]] = vals[k][t][s]
    for k, t, sl in backup:
        for c in range(K):
            if sl[c] != 0.0:
                h[t][k * K + c] = sl[c]
    return h


def down_dense(h, W_down):
    T, F, D = len(h), len(h[0]), len(W_down[0])
    y = [[0.0] * D for _ in range(T)]
    for t in range(T):
        for j in range(F):
            for d in range(D):
                y[t][d] += h[t][j] * W_down[j][d]
    return y


def down_sparse(counts, vals, cols, backup, W_down, T, K, W):
    """Stored entries only; per tile: main slots, then backup remainder (ascending)."""
    D = len(W_down[0])
    bk = {(k, t): sl for k, t, sl in backup}
    y = [[0.0] * D for _ in range(T)]
    for t in range(T):
        for k in range(len(counts)):
            for s in range(min(counts[k][t], W)):
                j = k * K + cols[k][t][s]
                for d in range(D):
                    y[t][d] += vals[k][t][s] * W_down[j][d]
            sl = bk.get((k, t))
            if sl is not None:
                for c in range(K):
                    if sl[c] != 0.0:
                        for d in range(D):
                            y[t][d] += sl[c] * W_down[k * K + c][d]
    return y


def backward(x, h, g, W_up, W_down):
    """Gradients of sum(y * g) with the ReLU mask taken from the stored h (Page A,
    "What TwELL and the custom CUDA kernels solve": training from the hybrid form)."""
    T, D, F = len(x), len(x[0]), len(W_up)
    dh = [[0.0] * F for _ in range(T)]
    for t in range(T):
        for j in range(F):
            if h[t][j] != 0.0:
                dh[t][j] = sum(g[t][d] * W_down[j][d] for d in range(D))
    dWd = [[sum(h[t][j] * g[t][d] for t in range(T)) for d in range(D)] for j in range(F)]
    dWu = [[sum(dh[t][j] * x[t][d] for t in range(T)) for d in range(D)] for j in range(F)]
    db = [sum(dh[t][j] for t in range(T)) for j in range(F)]
    dx = [[sum(dh[t][j] * W_up[j][d] for j in range(F)) for d in range(D)] for t in range(T)]
    return dx, dWu, dWd, db, dh
