"""Pins for the CPU fp64 oracle: worked example, brute force, invariants, special cases,
exact identities and finite differences.  CPU only.

Each test fixes the oracle against something other than itself: a hand-derived example,
the IEEE definition of rounding, classic ELLPACK, numpy's matmul, exact algebraic
identities, central differences, or exhaustive enumeration.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import tiny
from gen import make_layer, make_hidden, CONFIGS


# ----------------------------------------------------------------------------- helpers
def _load_example(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


def _tw_backup_list(tw):
    return [(int(k), int(t), list(map(float, tw.bk_vals[i])))
            for i, (k, t) in enumerate(zip(tw.bk_tile, tw.bk_tok))]


def _check_invariants(h, tw):
    """Properties every TwELL of h must satisfy, whatever h is."""
    T, F = h.shape
    K, W = tw.K, tw.W
    nt = F // K
    nzmask = h != 0.0
    # per-tile counts sum to the row's nonzero count
    assert np.array_equal(tw.counts.astype(np.int64).sum(axis=0), nzmask.sum(axis=1))
    # each count is the tile-row's nonzero count and is at most K
    per_tile = nzmask.reshape(T, nt, K).sum(axis=2).T
    assert np.array_equal(tw.counts.astype(np.int64), per_tile)
    assert tw.counts.max(initial=0) <= K
    c = tw.counts.astype(np.int64)
    m = np.minimum(c, W)
    s_idx = np.arange(W)[None, None, :]
    used = s_idx < m[:, :, None]
    # padding is exactly (0, 0)
    assert np.all(tw.vals[~used] == 0.0) and np.all(tw.cols[~used] == 0)
    # stored columns strictly ascending within a tile-row; stored values nonzero
    cols = tw.cols.astype(np.int64)
    asc = (cols[:, :, 1:] > cols[:, :, :-1]) | ~used[:, :, 1:]
    assert np.all(asc)
    assert np.all(tw.vals[used] != 0.0)
    # backup: one entry per overflowing tile-row, ascending (k, t), disjoint from main
    over = np.argwhere(c > W)  # rows (k, t) in ascending order
    assert tw.n_backup == len(over) == len(tw.bk_tile)
    assert np.array_equal(np.stack([tw.bk_tile, tw.bk_tok], 1).reshape(-1, 2), over.reshape(-1, 2))
    for i, (k, t) in enumerate(over):
        sl = tw.bk_vals[i]
        main_cols = set(tw.cols[k, t, :W].tolist())
        nzc = np.nonzero(sl)[0]
        assert len(nzc) == c[k, t] - W
        assert not (set(nzc.tolist()) & main_cols)
        # remainder = nonzeros of rank >= W in ascending column order
        row_nz = np.nonzero(h[t, k * K:(k + 1) * K])[0]
        assert np.array_equal(nzc, row_nz[W:])
    # round trip (up to the sign of zero)
    hu = oracle.unpack(tw)
    assert np.array_equal(hu, np.where(nzmask, h, 0.0))


# ----------------------------------------------------------------------------- worked example
def test_worked_example_pack(golden_dir):
    ex = _load_example(golden_dir)
    h = np.array(ex["h"], np.float64)
    tw = oracle.pack(h, ex["K"], ex["W"])
    assert tw.counts.tolist() == ex["counts"]
    assert tw.vals.tolist() == ex["vals"]
    assert tw.cols.tolist() == ex["cols"]
    assert _tw_backup_list(tw) == [(b["tile"], b["tok"], b["slice"]) for b in ex["backup"]]
    _check_invariants(h, tw)


def test_worked_example_tiny_twin(golden_dir):
    ex = _load_example(golden_dir)
    counts, vals, cols, backup = tiny.pack(ex["h"], ex["K"], ex["W"])
    assert counts == ex["counts"] and vals == ex["vals"] and cols == ex["cols"]
    assert [(k, t, s) for k, t, s in backup] == [(b["tile"], b["tok"], b["slice"]) for b in ex["backup"]]
    y = tiny.down_sparse(counts, vals, cols, backup, ex["W_down"], ex["T"], ex["K"], ex["W"])
    assert y == ex["y"]


def test_worked_example_stats(golden_dir):
    ex = _load_example(golden_dir)
    tw = oracle.pack(np.array(ex["h"], np.float64), ex["K"], ex["W"])
    st = oracle.stats(tw)
    for key in ("nnz", "slots_used", "backup_nonzeros", "overflow_tile_rows", "max_count"):
        assert st[key] == ex["stats"][key], key
    assert st["row_nnz"].tolist() == ex["stats"]["row_nnz"]
    assert st["density"] == pytest.approx(ex["stats"]["density"], abs=0)
    assert st["ell_fill"] == pytest.approx(ex["stats"]["ell_fill"], abs=0)


def test_worked_example_forward(golden_dir):
    ex = _load_example(golden_dir)
    h = np.array(ex["h"], np.float64)
    Wd = np.array(ex["W_down"], np.float64)
    tw = oracle.pack(h, ex["K"], ex["W"])
    y_s = oracle.down_sparse(tw, Wd)
    y_d = oracle.down_dense(h, Wd)
    assert y_s.tolist() == ex["y"]
    assert y_d.tolist() == ex["y"]
    # row 2 splits into main and backup contributions
    tw_main = oracle.TwELL(**{**tw.__dict__, "bk_tile": tw.bk_tile[:0], "bk_tok": tw.bk_tok[:0],
                              "bk_vals": tw.bk_vals[:0], "n_backup": 0})
    y_main = oracle.down_sparse(tw_main, Wd)
    assert y_main[2].tolist() == ex["y_row2_main"]
    assert (y_s[2] - y_main[2]).tolist() == ex["y_row2_backup"]


def test_worked_example_backward(golden_dir):
    ex = _load_example(golden_dir)
    h = np.array(ex["h"], np.float64)
    Wd = np.array(ex["W_down"], np.float64)
    g = np.array(ex["g"], np.float64)
    # x and W_up do not enter dW_down and dh; use arbitrary ones
    x = np.ones((ex["T"], ex["D"]))
    Wu = np.ones((ex["F"], ex["D"]))
    dx, dWu, dWd, db, dh = oracle.backward(x, h, g, Wu, Wd)
    assert dWd.tolist() == ex["dW_down"]
    assert dh.tolist() == ex["dh"]
    y = oracle.down_dense(h, Wd)
    assert float((y * g).sum()) == ex["loss"]
    t0, j0 = ex["dh_stored_zero"]
    assert h[t0, j0] != 0 and dh[t0, j0] == 0.0
    # the twin agrees
    tdx, tdWu, tdWd, tdb, tdh = tiny.backward(x.tolist(), ex["h"], ex["g"], Wu.tolist(), ex["W_down"])
    assert tdWd == ex["dW_down"] and tdh == ex["dh"]


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_brute_force_all_patterns(W):
    """All 2^8 sparsity patterns of an 8-column row with K = 4."""
    K = 4
    rows = []
    for bits in range(256):
        rows.append([(c + 1) * 0.5 if (bits >> c) & 1 else 0.0 for c in range(8)])
    h = np.array(rows, np.float64)
    tw = oracle.pack(h, K, W)
    for t, bits in enumerate(range(256)):
        for k in range(2):
            nib = (bits >> (4 * k)) & 0xF
            cs = [c for c in range(4) if (nib >> c) & 1]
            assert tw.counts[k, t] == len(cs)
            kept = cs[:W]
            assert tw.cols[k, t, :len(kept)].tolist() == kept
            assert tw.vals[k, t, :len(kept)].tolist() == [(4 * k + c + 1) * 0.5 for c in kept]
    _check_invariants(h, tw)
    c2, v2, col2, b2 = tiny.pack(rows, K, W)
    assert c2 == tw.counts.tolist() and v2 == tw.vals.tolist() and col2 == tw.cols.tolist()
    assert [(k, t, s) for k, t, s in b2] == _tw_backup_list(tw)


# ----------------------------------------------------------------------------- special cases
def test_ellpack_special_case():
    """One tile spanning all columns is classic row-wise ELLPACK."""
    h = make_hidden(37, 64, 0.2, seed=3).astype(np.float64)
    W = 64
    tw = oracle.pack(h, 64, W)
    for t in range(h.shape[0]):
        nz = np.nonzero(h[t])[0]
        assert tw.counts[0, t] == len(nz)
        assert tw.cols[0, t, :len(nz)].tolist() == nz.tolist()
        assert tw.vals[0, t, :len(nz)].tolist() == h[t, nz].tolist()
    assert tw.n_backup == 0


def test_width_equal_tile_never_backs_up():
    h = make_hidden(50, 256, 0.9, seed=4).astype(np.float64)
    tw = oracle.pack(h, 64, 64)
    assert tw.n_backup == 0
    _check_invariants(h, tw)


def test_width_one_max_backup():
    h = make_hidden(40, 256, 0.3, seed=5).astype(np.float64)
    tw = oracle.pack(h, 64, 1)
    assert tw.n_backup == int((tw.counts > 1).sum())
    _check_invariants(h, tw)


def test_all_zero_and_all_positive():
    T, F, K, W = 9, 256, 128, 16
    z = np.zeros((T, F))
    tw = oracle.pack(z, K, W)
    assert tw.counts.max() == 0 and tw.n_backup == 0
    assert np.all(tw.vals == 0) and np.all(tw.cols == 0)
    p = np.full((T, F), 0.75)
    tw = oracle.pack(p, K, W)
    assert np.all(tw.counts == K)
    assert tw.n_backup == T * (F // K)
    _check_invariants(p, tw)


def test_negative_zero_is_zero():
    h = make_hidden(33, 256, 0.1, seed=6, signed_zero=True).astype(np.float64)
    assert np.any(np.signbit(h) & (h == 0))
    tw = oracle.pack(h, 128, 8)
    _check_invariants(h, tw)
    hu = oracle.unpack(tw)
    assert not np.any(np.signbit(hu))


def test_count_equal_width_boundary():
    K, W = 8, 3
    h = np.zeros((2, 8))
    h[0, [1, 4, 6]] = [1, 2, 3]          # count == W: no backup
    h[1, [0, 2, 5, 7]] = [1, 2, 3, 4]    # count == W + 1: one backup entry, one value
    tw = oracle.pack(h, K, W)
    assert tw.counts[0].tolist() == [3, 4]
    assert tw.n_backup == 1 and tw.bk_tok.tolist() == [1]
    assert tw.bk_vals[0].tolist() == [0, 0, 0, 0, 0, 0, 0, 4]


def test_capacity_short_reports_need():
    h = np.full((4, 16), 1.0)
    tw = oracle.pack(h, 8, 2, cap=3)
    assert tw.n_backup == 8 and len(tw.bk_tile) == 3


# ----------------------------------------------------------------------------- random invariants
@pytest.mark.parametrize("K,W,density", [(64, 8, 0.1), (128, 32, 0.05), (128, 16, 0.3),
                                         (256, 16, 0.03), (64, 64, 0.5), (128, 1, 0.02)])
def test_random_invariants(K, W, density):
    h = make_hidden(70, 4 * K, density, seed=K + W, heavy_rows=(0, 69), heavy_density=0.6)
    h = h.astype(np.float64)
    tw = oracle.pack(h, K, W)
    _check_invariants(h, tw)


# ----------------------------------------------------------------------------- rounding model
def test_round_bf16_definition():
    one = 1.0
    cases = [
        (1.0, 0x3F80),
        (-2.0, 0xC000),
        (one + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
        (one + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
        (one + 2.0 ** -8 - 2.0 ** -20, 0x3F80),    # just below the tie
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.0e38, 0x7F62),
    ]
    got = oracle.round_bf16(np.array([k for k, _ in cases]))
    for (k, want), g in zip(cases, got):
        assert int(g) == want, (k, hex(int(g)))
    # bf16 values are fixed points; value() widens exactly
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(oracle.round_bf16(oracle.bf16_value(bits)), bits)


# ----------------------------------------------------------------------------- dense FFN vs numpy
def test_dense_ffn_matches_numpy():
    L = make_layer(CONFIGS["C1"], seed=0, T=24)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    h = oracle.up_relu(x, Wu, b)
    z_np = x @ Wu.T + b
    assert np.allclose(h, np.maximum(z_np, 0.0), rtol=1e-12, atol=1e-12)
    y = oracle.down_dense(h, Wd)
    y_np = np.maximum(z_np, 0.0) @ Wd
    assert np.linalg.norm(y - y_np) <= 1e-12 * np.linalg.norm(y_np)


def test_sparse_equals_dense_bitwise():
    L = make_layer(CONFIGS["C1b"], seed=0, T=64)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    y_d = oracle.ffn_dense(x, Wu, b, Wd)
    y_s, tw = oracle.ffn_sparse(x, Wu, b, Wd, 128, 16)
    assert tw.n_backup > 0   # the backup path is exercised
    assert np.array_equal(y_s, y_d)
    rows = np.array([0, 5, 63, 17])
    y_r, c_r = oracle.ffn_rows(x, Wu, b, Wd, rows, 128, 16)
    assert np.array_equal(y_r, y_d[rows])
    assert np.array_equal(c_r, tw.counts[:, rows].T)


def test_rows_with_bf16_storage_model():
    """ffn_rows(round_h) == dense FFN of the O8-rounded activations (bf16 TwELL values)."""
    L = make_layer(CONFIGS["C3"], seed=0, T=24, rho=0.2)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    rows = np.array([0, 3, 23, 11])
    y_r, c_r = oracle.ffn_rows(x, Wu, b, Wd, rows, 128, 32, round_h=True)
    h = oracle.up_relu(x, Wu, b)
    hr = oracle.bf16_value(oracle.round_bf16(h))
    assert np.array_equal(y_r, oracle.down_dense(hr, Wd)[rows])
    # rounding never turns a positive activation into zero here (no underflow)
    assert np.array_equal(hr != 0, h != 0)
    y_e, _ = oracle.ffn_rows(x, Wu, b, Wd, rows, 128, 32)
    assert not np.array_equal(y_r, y_e)


def test_positive_homogeneity_bitwise():
    L = make_layer(CONFIGS["C1"], seed=1, T=16)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    y1, _ = oracle.ffn_sparse(x, Wu, b, Wd, 128, 32)
    y2, _ = oracle.ffn_sparse(2 * x, Wu, 2 * b, Wd, 128, 32)
    assert np.array_equal(y2, 2 * y1)


def test_token_permutation_equivariance():
    L = make_layer(CONFIGS["C1"], seed=2, T=40)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    perm = np.random.default_rng(0).permutation(40)
    y, _ = oracle.ffn_sparse(x, Wu, b, Wd, 128, 16)
    yp, _ = oracle.ffn_sparse(x[perm], Wu, b, Wd, 128, 16)
    assert np.array_equal(yp, y[perm])


def test_neuron_permutation_invariance():
    L = make_layer(CONFIGS["C1"], seed=3, T=20)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    perm = np.random.default_rng(1).permutation(Wu.shape[0])
    y, _ = oracle.ffn_sparse(x, Wu, b, Wd, 128, 32)
    yp, _ = oracle.ffn_sparse(x, Wu[perm], b[perm], Wd[perm], 128, 32)
    assert np.allclose(yp, y, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- C++ vs Python twin
def test_cpp_matches_python_twin():
    rng = np.random.default_rng(11)
    T, D, F, K, W = 5, 6, 16, 8, 2
    x = rng.standard_normal((T, D))
    Wu = rng.standard_normal((F, D)) / math.sqrt(D)
    b = rng.standard_normal(F) * 0.3
    Wd = rng.standard_normal((F, D))
    h = oracle.up_relu(x, Wu, b)
    ht = tiny.up_relu(x.tolist(), Wu.tolist(), b.tolist())
    assert h.tolist() == ht
    tw = oracle.pack(h, K, W)
    c, v, col, bk = tiny.pack(ht, K, W)
    assert tw.counts.tolist() == c and tw.vals.tolist() == v and tw.cols.tolist() == col
    assert _tw_backup_list(tw) == [(k, t, s) for k, t, s in bk]
    assert oracle.unpack(tw).tolist() == tiny.unpack(c, v, col, bk, T, F, K, W)
    assert oracle.down_sparse(tw, Wd).tolist() == tiny.down_sparse(c, v, col, bk, Wd.tolist(), T, K, W)
    assert oracle.down_dense(h, Wd).tolist() == tiny.down_dense(ht, Wd.tolist())
    g = rng.standard_normal((T, D))
    got = oracle.backward(x, h, g, Wu, Wd)
    ref = tiny.backward(x.tolist(), ht, g.tolist(), Wu.tolist(), Wd.tolist())
    for a, r in zip(got, ref):
        assert np.allclose(a, np.array(r), rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- backward pins
def _tiny_layer(seed, T=6, D=5, F=12):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    Wu = rng.standard_normal((F, D)) / math.sqrt(D)
    b = rng.standard_normal(F) * 0.2
    Wd = rng.standard_normal((F, D)) / math.sqrt(F)
    g = rng.standard_normal((T, D))
    return x, Wu, b, Wd, g


def _loss(x, Wu, b, Wd, g):
    return float((oracle.ffn_dense(x, Wu, b, Wd) * g).sum())


def test_backward_finite_differences():
    x, Wu, b, Wd, g = _tiny_layer(21)
    z = x @ Wu.T + b
    assert np.abs(z).min() >= 1e-3, "pick a seed with no pre-activation near the kink"
    h = oracle.up_relu(x, Wu, b)
    dx, dWu, dWd, db, dh = oracle.backward(x, h, g, Wu, Wd)
    eps = 1e-6

    def fd(arr, setter):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[idx] += eps
            a2 = arr.copy(); a2[idx] -= eps
            out[idx] = (setter(a1) - setter(a2)) / (2 * eps)
        return out

    num_dx = fd(x, lambda a: _loss(a, Wu, b, Wd, g))
    num_dWu = fd(Wu, lambda a: _loss(x, a, b, Wd, g))
    num_dWd = fd(Wd, lambda a: _loss(x, Wu, b, a, g))
    num_db = fd(b, lambda a: _loss(x, Wu, a, Wd, g))
    for an, nu in ((dx, num_dx), (dWu, num_dWu), (dWd, num_dWd), (db, num_db)):
        assert np.linalg.norm(an - nu) <= 1e-6 * max(1.0, np.linalg.norm(nu))


def test_backward_euler_identities():
    """For a ReLU layer: <dW_down,W_down> = <dh,h> = L and <dx,x> = <dW_up,W_up> = L - <db,b>."""
    L = make_layer(CONFIGS["C1b"], seed=0, T=32)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    g = np.random.default_rng(5).standard_normal((32, x.shape[1]))
    h = oracle.up_relu(x, Wu, b)
    dx, dWu, dWd, db, dh = oracle.backward(x, h, g, Wu, Wd)
    loss = float((oracle.down_dense(h, Wd) * g).sum())
    tol = 1e-10 * max(1.0, abs(loss))
    assert abs(float((dWd * Wd).sum()) - loss) <= tol
    assert abs(float((dh * h).sum()) - loss) <= tol
    rhs = loss - float((db * b).sum())
    assert abs(float((dx * x).sum()) - rhs) <= 1e-9 * max(1.0, abs(rhs))
    assert abs(float((dWu * Wu).sum()) - rhs) <= 1e-9 * max(1.0, abs(rhs))


def test_backward_bf16_storage_model():
    """round_dh: dh is the O8 rounding of the exact dh, dW_down does not depend on it, dx and
    dW_up stay consistent with each other for the rounded dh, and the change in dx is within
    the bf16 rounding bound of dh."""
    L = make_layer(CONFIGS["C1b"], seed=0, T=32)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    g = np.random.default_rng(6).standard_normal((32, x.shape[1]))
    h = oracle.up_relu(x, Wu, b)
    dx0, dWu0, dWd0, db0, dh0 = oracle.backward(x, h, g, Wu, Wd)
    dx1, dWu1, dWd1, db1, dh1 = oracle.backward(x, h, g, Wu, Wd, round_dh=True)
    assert np.array_equal(dh1, oracle.bf16_value(oracle.round_bf16(dh0)))
    assert np.array_equal(dWd1, dWd0)
    assert np.count_nonzero(dh1 != dh0) > 0
    # <dx, x> = <dW_up, W_up> = sum dh * (z - b), for whichever dh the layer stores
    z_b = x @ Wu.T
    ref = float((dh1 * z_b).sum())
    assert abs(float((dx1 * x).sum()) - ref) <= 1e-9 * max(1.0, abs(ref))
    assert abs(float((dWu1 * Wu).sum()) - ref) <= 1e-9 * max(1.0, abs(ref))
    assert abs(float(db1.sum()) - float(dh1.sum())) <= 1e-9 * max(1.0, float(np.abs(dh1).sum()))
    # the dh-consuming half on its own reproduces the full backward for its dh
    fx, fwu, fdb = oracle.backward_from_dh(x, dh1, Wu)
    assert np.array_equal(fx, dx1) and np.array_equal(fwu, dWu1) and np.array_equal(fdb, db1)
    # and the identity holds for an arbitrary dh
    dh_any = np.random.default_rng(8).standard_normal(dh1.shape) * (dh1 != 0)
    ax, awu, adb = oracle.backward_from_dh(x, dh_any, Wu)
    r2 = float((dh_any * z_b).sum())
    assert abs(float((ax * x).sum()) - r2) <= 1e-9 * max(1.0, abs(r2))
    assert abs(float((awu * Wu).sum()) - r2) <= 1e-9 * max(1.0, abs(r2))
    assert np.allclose(adb, dh_any.sum(axis=0), rtol=0, atol=1e-12)
    # |dx1 - dx0| <= sum_j |dh1 - dh0| |W_up| <= 2^-8 sum_j |dh0| |W_up|
    bound = 2.0 ** -8 * (np.abs(dh0) @ np.abs(Wu)) + 1e-12
    assert np.all(np.abs(dx1 - dx0) <= bound)


def test_backward_rows_match_backward_and_matmul():
    """dh_rows / dx_rows (the per-token half of O9 over many rows, zero products skipped):
    bit for bit the dh and dx of oracle.backward, with and without the bf16 storage of dh;
    against numpy's matmul, dh = mask * (g W_down^T) and dx = dh W_up within fp64 rounding;
    a row with no stored activation has dh = 0 and dx = 0."""
    L = make_layer(CONFIGS["C1b"], seed=0, T=32)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    g = np.random.default_rng(9).standard_normal((32, x.shape[1]))
    h = oracle.up_relu(x, Wu, b)
    h[3] = 0.0
    for rd in (False, True):
        dx, _, _, _, dh = oracle.backward(x, h, g, Wu, Wd, round_dh=rd)
        dh_r = oracle.dh_rows(h, g, Wd, round_dh=rd)
        dx_r = oracle.dx_rows(dh_r, Wu)
        assert np.array_equal(dh_r, dh) and np.array_equal(dx_r, dx)
        assert not np.any(dh_r[3]) and not np.any(dx_r[3])
    exact = (g @ Wd.T) * (h != 0)
    dh0 = oracle.dh_rows(h, g, Wd)
    assert np.allclose(dh0, exact, rtol=1e-12, atol=1e-12)
    assert np.array_equal(dh0 != 0, (h != 0) & (exact != 0))
    assert np.allclose(oracle.dx_rows(dh0, Wu), dh0 @ Wu, rtol=1e-12, atol=1e-12)
    # a row's result does not depend on the other rows
    assert np.array_equal(oracle.dh_rows(h[5:9], g[5:9], Wd), dh0[5:9])
    assert np.array_equal(oracle.dx_rows(dh0[5:9], Wu), oracle.dx_rows(dh0, Wu)[5:9])


def test_weight_gradients_match_backward_and_matmul():
    """oracle.dw (the token sums of O9 with zero products skipped): bit for bit the dW_down,
    dW_up and db of oracle.backward; against numpy, a^T b and the column sums within fp64
    rounding; a hidden column that never fires has zero gradients."""
    L = make_layer(CONFIGS["C1b"], seed=0, T=32)
    x, Wu, b, Wd = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    g = np.random.default_rng(10).standard_normal((32, x.shape[1]))
    h = oracle.up_relu(x, Wu, b)
    h[:, 7] = 0.0
    for rd in (False, True):
        _, dWu, dWd, db, dh = oracle.backward(x, h, g, Wu, Wd, round_dh=rd)
        wd, hs = oracle.dw(h, g)
        wu, cs = oracle.dw(dh, x)
        assert np.array_equal(wd, dWd) and np.array_equal(wu, dWu) and np.array_equal(cs, db)
        assert not np.any(wd[7]) and not np.any(wu[7]) and cs[7] == 0.0
    assert np.allclose(wd, h.T @ g, rtol=1e-12, atol=1e-12)
    assert np.allclose(hs, h.sum(axis=0), rtol=1e-12, atol=1e-12)
    assert np.allclose(wu, dh.T @ x, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(golden_dir, monkeypatch):
    """Plant plausible mistakes in the Python twin and check the pins reject them."""
    ex = _load_example(golden_dir)
    good = tiny.pack(ex["h"], ex["K"], ex["W"])

    def pack_descending(h, K, W):   # slots in descending column order
        c, v, col, bk = tiny.pack(h, K, W)
        for k in range(len(c)):
            for t in range(len(c[k])):
                m = min(c[k][t], W)
                v[k][t][:m] = v[k][t][:m][::-1]
                col[k][t][:m] = col[k][t][:m][::-1]
        return c, v, col, bk

    def pack_clipped_counts(h, K, W):  # counts clipped to W
        c, v, col, bk = tiny.pack(h, K, W)
        return [[min(n, W) for n in row] for row in c], v, col, bk

    def pack_no_backup(h, K, W):       # overflow dropped
        c, v, col, _ = tiny.pack(h, K, W)
        return c, v, col, []

    for bad in (pack_descending, pack_clipped_counts, pack_no_backup):
        got = bad(ex["h"], ex["K"], ex["W"])
        assert got != good
        ok = (got[0] == ex["counts"] and got[1] == ex["vals"] and got[2] == ex["cols"]
              and [(k, t, s) for k, t, s in got[3]] == [(b["tile"], b["tok"], b["slice"]) for b in ex["backup"]])
        assert not ok

    # a down-projection that drops the backup, or uses the transposed weight index
    c, v, col, bk = good
    y_nobk = tiny.down_sparse(c, v, col, [], ex["W_down"], ex["T"], ex["K"], ex["W"])
    assert y_nobk != ex["y"]
    WdT_like = [[row[1], row[0]] for row in ex["W_down"]]
    assert tiny.down_sparse(c, v, col, bk, WdT_like, ex["T"], ex["K"], ex["W"]) != ex["y"]


# ----------------------------------------------------------------------------- generator sanity
@pytest.mark.parametrize("rho", [0.01, 0.05, 0.10, 0.20])
def test_generator_density_c3_sample(rho):
    """Ordinary-token density of the synthetic 1.5B-like layer is close to rho (sampled rows)."""
    cfg = CONFIGS["C3"]
    L = make_layer(cfg, seed=0, rho=rho)
    heavy = set(L["heavy"].tolist())
    rows = np.array([t for t in range(0, cfg.T, 97) if t not in heavy][:48])
    x, Wu, b, Wd = (L[k] for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    _, counts = oracle.ffn_rows(x, Wu, b, Wd, rows, cfg.tile, cfg.ell_width)
    dens = counts.sum() / float(len(rows) * cfg.F)
    assert abs(dens - rho) < max(0.003, 0.15 * rho)


@pytest.mark.parametrize("T,F,K,density,heavy,esz", [
    (40, 256, 64, 0.05, (), 2), (40, 256, 64, 0.3, (3, 17), 2), (33, 512, 128, 0.02, (0,), 4),
    (20, 256, 128, 0.9, (), 2), (25, 512, 256, 0.1, (5,), 2)])
def test_choose_ell_width_is_the_smallest_packing(T, F, K, density, heavy, esz):
    """The width chosen from the count histogram is the one whose actual packing - the
    oracle's pack at every width, its arrays measured - takes the fewest bytes (ties to the
    smaller width), and the histogram counts every tile-row once."""
    h = make_hidden(T, F, density, seed=5, heavy_rows=heavy, heavy_density=0.7)
    tw1 = oracle.pack(h, K, 1)
    hist = oracle.count_histogram(tw1)
    assert hist.sum() == (F // K) * T and hist.size == K + 1
    assert np.array_equal(hist, np.bincount(((h != 0).reshape(T, F // K, K).sum(axis=2)).ravel(),
                                            minlength=K + 1))
    measured = [oracle.twell_bytes(oracle.pack(h, K, W), esz) for W in range(1, K + 1)]
    W_best = 1 + int(np.argmin(measured))  # argmin takes the first (smallest W) of ties
    assert oracle.choose_ell_width(hist, K, esz) == (W_best, measured[W_best - 1])
    cands = [16, 32, 48, 64]
    cands = [c for c in cands if c <= K]
    wc, bc = oracle.choose_ell_width(hist, K, esz, cands)
    assert bc == min(measured[c - 1] for c in cands) and wc == min(
        c for c in cands if measured[c - 1] == bc)


def test_choose_ell_width_special_cases():
    """Every tile-row with the same count c: the width c when ELL slots are cheaper than a
    dense backup slice (c (esz + 1) < esz K + 8), else width 1 with every row in the backup;
    all rows empty: width 1."""
    K, esz = 128, 2
    for c, expect in ((5, 5), (40, 40), (88, 88), (89, 1), (128, 1)):
        hist = np.zeros(K + 1, np.int64)
        hist[c] = 1000
        assert oracle.choose_ell_width(hist, K, esz)[0] == expect, c
    hist = np.zeros(K + 1, np.int64)
    hist[0] = 7
    assert oracle.choose_ell_width(hist, K, esz) == (1, 7 * (2 + 3))
