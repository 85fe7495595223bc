"""CPU fp64 oracle for the TwELL sparse FFN (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It shares no code with the HIP library: the arithmetic is in
``oracle.cpp`` (fp64 loops, OpenMP over rows), loaded here with ctypes, and a pure
Python twin for tiny cases is in ``tiny.py``.

Pin status: every function here is pinned by CPU tests (worked example, brute force
over all sparsity patterns of a small row, invariants, special cases that reduce to
classic ELLPACK / numpy matmul, exact identities, finite differences); none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SFFN_ORACLE_LIB names another build of the same source (the sanitizer test uses it)
_LIB_PATH = os.environ.get("SFFN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_up_relu.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P]
    lib.oracle_up_relu.restype = None
    lib.oracle_pack.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P]
    lib.oracle_pack.restype = ctypes.c_int
    lib.oracle_unpack.argtypes = [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _P]
    lib.oracle_unpack.restype = None
    lib.oracle_down_dense.argtypes = [_P, _P, _I, _I, _I, _P]
    lib.oracle_down_dense.restype = None
    lib.oracle_down_sparse.argtypes = [_P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]
    lib.oracle_down_sparse.restype = None
    lib.oracle_backward.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_int32, _P, _P, _P, _P, _P]
    lib.oracle_backward.restype = None
    lib.oracle_backward_from_dh.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P]
    lib.oracle_backward_from_dh.restype = None
    lib.oracle_dh_rows.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_int32, _P]
    lib.oracle_dh_rows.restype = None
    lib.oracle_dx_rows.argtypes = [_P, _P, _I, _I, _I, _P]
    lib.oracle_dx_rows.restype = None
    lib.oracle_dw.argtypes = [_P, _P, _I, _I, _I, _P, _P]
    lib.oracle_dw.restype = None
    lib.oracle_ffn_rows.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int32, _P, _P, _P]
    lib.oracle_ffn_rows.restype = None
    lib.oracle_round_bf16.argtypes = [_P, _I, _P]
    lib.oracle_round_bf16.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


@dataclass
class TwELL:
    """TwELL form of a [T, F] hidden tensor (tile-major), plus the ordered backup."""
    T: int
    F: int
    K: int
    W: int
    counts: np.ndarray   # uint16 [n_t, T]
    vals: np.ndarray     # float64 [n_t, T, W]
    cols: np.ndarray     # uint8 [n_t, T, W]
    bk_tile: np.ndarray  # int32 [R]
    bk_tok: np.ndarray   # int32 [R]
    bk_vals: np.ndarray  # float64 [R, K]
    n_backup: int        # entries needed (R == n_backup unless capacity ran out)

    @property
    def n_tiles(self) -> int:
        return self.F // self.K


def up_relu(x, W_up, b, return_z: bool = False):
    """O1 + O2: h = relu(x W_up^T + b) in fp64 (bias after the ascending sum)."""
    lib = _load()
    x = _c(x, np.float64); W_up = _c(W_up, np.float64); b = _c(b, np.float64)
    T, D = x.shape
    F = W_up.shape[0]
    h = np.empty((T, F), np.float64)
    z = np.empty((T, F), np.float64) if return_z else None
    lib.oracle_up_relu(_ptr(x), _ptr(W_up), _ptr(b), T, D, F,
                       _ptr(z) if z is not None else None, _ptr(h))
    return (h, z) if return_z else h


def pack(h, K: int, W: int, cap: int | None = None) -> TwELL:
    """O3: TwELL pack of a dense hidden tensor (nonzero iff h != 0)."""
    lib = _load()
    h = _c(h, np.float64)
    T, F = h.shape
    if F % K:
        raise ValueError("F must be a multiple of the tile width")
    nt = F // K
    if cap is None:
        cap = nt * T
    counts = np.zeros((nt, T), np.uint16)
    vals = np.zeros((nt, T, W), np.float64)
    cols = np.zeros((nt, T, W), np.uint8)
    bk_tile = np.zeros(max(cap, 1), np.int32)
    bk_tok = np.zeros(max(cap, 1), np.int32)
    bk_vals = np.zeros((max(cap, 1), K), np.float64)
    nb = ctypes.c_int64(0)
    lib.oracle_pack(_ptr(h), T, F, K, W, _ptr(counts), _ptr(vals), _ptr(cols), cap,
                    _ptr(bk_tile), _ptr(bk_tok), _ptr(bk_vals), ctypes.byref(nb))
    n = int(nb.value)
    r = min(n, cap)
    return TwELL(T, F, K, W, counts, vals, cols, bk_tile[:r].copy(), bk_tok[:r].copy(),
                 bk_vals[:r].copy(), n)


def unpack(tw: TwELL) -> np.ndarray:
    """O4: dense [T, F] from TwELL main + backup."""
    lib = _load()
    h = np.empty((tw.T, tw.F), np.float64)
    counts = _c(tw.counts, np.uint16); vals = _c(tw.vals, np.float64); cols = _c(tw.cols, np.uint8)
    bt = _c(tw.bk_tile, np.int32); bo = _c(tw.bk_tok, np.int32); bv = _c(tw.bk_vals, np.float64)
    lib.oracle_unpack(_ptr(counts), _ptr(vals), _ptr(cols), len(bt), _ptr(bt), _ptr(bo), _ptr(bv),
                      tw.T, tw.F, tw.K, tw.W, _ptr(h))
    return h


def down_dense(h, W_down) -> np.ndarray:
    """O5: y = h W_down (W_down stored [F, D]), fp64, j ascending."""
    lib = _load()
    h = _c(h, np.float64); W_down = _c(W_down, np.float64)
    T, F = h.shape
    D = W_down.shape[1]
    y = np.empty((T, D), np.float64)
    lib.oracle_down_dense(_ptr(h), _ptr(W_down), T, D, F, _ptr(y))
    return y


def down_sparse(tw: TwELL, W_down) -> np.ndarray:
    """O6: y from the stored TwELL entries only, in the same order as O5."""
    lib = _load()
    W_down = _c(W_down, np.float64)
    D = W_down.shape[1]
    y = np.empty((tw.T, D), np.float64)
    counts = _c(tw.counts, np.uint16); vals = _c(tw.vals, np.float64); cols = _c(tw.cols, np.uint8)
    bt = _c(tw.bk_tile, np.int32); bo = _c(tw.bk_tok, np.int32); bv = _c(tw.bk_vals, np.float64)
    lib.oracle_down_sparse(_ptr(counts), _ptr(vals), _ptr(cols), len(bt), _ptr(bt), _ptr(bo),
                           _ptr(bv), _ptr(W_down), tw.T, D, tw.F, tw.K, tw.W, _ptr(y))
    return y


def ffn_dense(x, W_up, b, W_down) -> np.ndarray:
    """O1, O2, O5: the plain ReLU FFN y = relu(x W_up^T + b) W_down in fp64."""
    return down_dense(up_relu(x, W_up, b), W_down)


def ffn_sparse(x, W_up, b, W_down, K: int, W: int):
    """O1, O2, O3, O6: the TwELL FFN; returns (y, twell)."""
    tw = pack(up_relu(x, W_up, b), K, W)
    return down_sparse(tw, W_down), tw


def ffn_rows(x, W_up, b, W_down, rows, K: int, W: int, return_z: bool = False,
             round_h: bool = False):
    """O1..O3 + O6 for selected token rows only (the FFN is per token).

    With ``round_h`` the activations are rounded to bf16 (O8) before the down-projection,
    the values a bf16 TwELL stores.  Returns (y_rows [R, D], counts_rows [R, n_t]) and
    optionally z_rows [R, F].
    """
    lib = _load()
    x = _c(x, np.float64); W_up = _c(W_up, np.float64); b = _c(b, np.float64)
    W_down = _c(W_down, np.float64)
    rows = _c(rows, np.int64)
    D = x.shape[1]
    F = W_up.shape[0]
    R = len(rows)
    y = np.empty((R, D), np.float64)
    counts = np.empty((R, F // K), np.uint16)
    z = np.empty((R, F), np.float64) if return_z else None
    lib.oracle_ffn_rows(_ptr(x), _ptr(W_up), _ptr(b), _ptr(W_down), _ptr(rows), R, D, F, K, W,
                        1 if round_h else 0, _ptr(y), _ptr(counts), _ptr(z) if z is not None else None)
    return (y, counts, z) if return_z else (y, counts)


def backward(x, h, g, W_up, W_down, round_dh=False):
    """O9: (dx, dW_up, dW_down, db, dh) of loss = sum(y * g), ReLU mask = stored h != 0.
    With round_dh, dh is stored in bf16 (O8) before dW_up, db and dx use it."""
    lib = _load()
    x = _c(x, np.float64); h = _c(h, np.float64); g = _c(g, np.float64)
    W_up = _c(W_up, np.float64); W_down = _c(W_down, np.float64)
    T, D = x.shape
    F = W_up.shape[0]
    dx = np.empty((T, D)); dWu = np.empty((F, D)); dWd = np.empty((F, D))
    db = np.empty(F); dh = np.empty((T, F))
    lib.oracle_backward(_ptr(x), _ptr(h), _ptr(g), _ptr(W_up), _ptr(W_down), T, D, F,
                        1 if round_dh else 0,
                        _ptr(dx), _ptr(dWu), _ptr(dWd), _ptr(db), _ptr(dh))
    return dx, dWu, dWd, db, dh


def backward_from_dh(x, dh, W_up):
    """(dx, dW_up, db) of O9 for a given dh [T, F] (e.g. the dh a layer stored)."""
    lib = _load()
    x = _c(x, np.float64); dh = _c(dh, np.float64); W_up = _c(W_up, np.float64)
    T, D = x.shape
    F = W_up.shape[0]
    dx = np.empty((T, D)); dWu = np.empty((F, D)); db = np.empty(F)
    lib.oracle_backward_from_dh(_ptr(x), _ptr(dh), _ptr(W_up), T, D, F, _ptr(dx), _ptr(dWu),
                                _ptr(db))
    return dx, dWu, db


def dh_rows(h, g, W_down, round_dh=False) -> np.ndarray:
    """O9's dh of given token rows: [h != 0] * (g W_down^T), bf16-rounded with round_dh.
    The same values oracle.backward returns as dh, without the weight gradients."""
    lib = _load()
    h = _c(h, np.float64); g = _c(g, np.float64); W_down = _c(W_down, np.float64)
    T, F = h.shape
    D = g.shape[1]
    dh = np.empty((T, F))
    lib.oracle_dh_rows(_ptr(h), _ptr(g), _ptr(W_down), T, D, F, 1 if round_dh else 0, _ptr(dh))
    return dh


def dx_rows(dh, W_up) -> np.ndarray:
    """O9's dx = dh W_up of given rows of dh [T, F] (zero dh entries skipped)."""
    lib = _load()
    dh = _c(dh, np.float64); W_up = _c(W_up, np.float64)
    T, F = dh.shape
    D = W_up.shape[1]
    dx = np.empty((T, D))
    lib.oracle_dx_rows(_ptr(dh), _ptr(W_up), T, D, F, _ptr(dx))
    return dx


def dw(a, b):
    """O9's weight-gradient sums over tokens: (a^T b [F, D], column sums of a [F]) for
    a [T, F] and b [T, D]: (h, g) gives dW_down, (dh, x) gives dW_up and db."""
    lib = _load()
    a = _c(a, np.float64); b = _c(b, np.float64)
    T, F = a.shape
    D = b.shape[1]
    out = np.empty((F, D)); cs = np.empty(F)
    lib.oracle_dw(_ptr(a), _ptr(b), T, D, F, _ptr(out), _ptr(cs))
    return out, cs


def round_bf16(a) -> np.ndarray:
    """O8: fp64 -> fp32 -> bf16 (nearest, ties to even), as uint16 bit patterns."""
    lib = _load()
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib.oracle_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_value(bits) -> np.ndarray:
    """Value of bf16 bit patterns as fp64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def stats(tw: TwELL) -> dict:
    """O7: counts-derived statistics of a TwELL (nnz, slots used, backup, fill)."""
    c = tw.counts.astype(np.int64)
    W = tw.W
    nnz = int(c.sum())
    slots = int(np.minimum(c, W).sum())
    over = int((c > W).sum())
    bk_nnz = int(np.maximum(c - W, 0).sum())
    nt, T = c.shape
    return {
        "nnz": nnz,
        "slots_used": slots,
        "overflow_tile_rows": over,
        "backup_nonzeros": bk_nnz,
        "max_count": int(c.max()) if c.size else 0,
        "density": nnz / float(T * tw.F) if T * tw.F else 0.0,
        "ell_fill": slots / float(nt * T * W) if nt * T * W else 0.0,
        "row_nnz": c.sum(axis=0),
    }


def count_histogram(tw: TwELL) -> np.ndarray:
    """hist[c] = number of tile-rows (k, t) of the TwELL with c stored nonzeros, c = 0..K
    (the per-tile nonzero counts the format is laid out from: upppp.jp TwELL article of
    2026-05-11, section "What TwELL and the custom CUDA kernels solve")."""
    return np.bincount(tw.counts.astype(np.int64).ravel(), minlength=tw.K + 1).astype(np.int64)


def twell_bytes(tw: TwELL, esz: int) -> int:
    """Bytes of a packed activation as stored: every tile-row's count (2 bytes) and its W
    value and column slots, plus each backup entry's dense K-value slice and its tile and
    token indices (4 bytes each) - the storage of the hybrid form's sparse main part and
    dense backups (same section)."""
    assert tw.n_backup == tw.bk_vals.shape[0], "measured on a TwELL whose backup fits"
    return (tw.counts.size * 2 + tw.vals.size * esz + tw.cols.size * 1
            + tw.bk_vals.size * esz + tw.bk_tile.size * 4 + tw.bk_tok.size * 4)


def choose_ell_width(hist, K: int, esz: int, candidates=None):
    """The ELL width with the fewest stored bytes for a count histogram: for each candidate
    W, every tile-row stores its count and W slots, and a row with more than W nonzeros
    also stores a backup entry; the smallest total wins, ties to the smaller W.  Returns
    (W, bytes)."""
    hist = np.asarray(hist, np.int64)
    rows = int(hist.sum())
    best = None
    for W in (range(1, K + 1) if candidates is None else candidates):
        n_over = int(hist[W + 1:].sum())
        total = rows * 2 + rows * W * (esz + 1) + n_over * (K * esz + 8)
        if best is None or total < best[1] or (total == best[1] and W < best[0]):
            best = (int(W), int(total))
    return best

