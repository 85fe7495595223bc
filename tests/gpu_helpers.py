"""Helpers shared by the GPU tests: decoding a device TwELL on the host, tolerances, and
the rounding-error band of an fp32 pre-activation.  Test code only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_transformer_amd as sffn
    sffn.lib()  # raises if the HIP library is not built: the tests must not pass without it
    return torch, sffn


def to_dev_bf16(torch, bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_f32(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def layer_to_dev(torch, L):
    cfg = L["cfg"]
    if cfg.dtype == "bf16":
        f = lambda k: to_dev_bf16(torch, L[k])
    else:
        f = lambda k: to_dev_f32(torch, L[k])
    return f("x"), f("W_up"), f("b_up"), f("W_down")


def y_to_host(torch, y) -> np.ndarray:
    if y.dtype == torch.bfloat16:
        bits = y.view(torch.int16).cpu().numpy().view(np.uint16)
        return oracle.bf16_value(bits)
    return y.cpu().numpy().astype(np.float64)


def vals_value(cfg, vals) -> np.ndarray:
    """Stored TwELL values as fp64."""
    if cfg.dtype == "bf16":
        return oracle.bf16_value(vals)
    return vals.astype(np.float64)


def decode_dense(cfg, host: dict, T: int) -> np.ndarray:
    """Dense [T, F] of a device TwELL (main + backup), decoded here in numpy."""
    K, W, nt = cfg.tile, cfg.ell_width, cfg.n_tiles
    h = np.zeros((T, cfg.d_ff), np.float64)
    vals = vals_value(cfg, host["vals"])
    cols = host["cols"].astype(np.int64)
    counts = host["counts"].astype(np.int64)
    m = np.minimum(counts, W)
    for k in range(nt):
        for s in range(W):
            sel = m[k] > s
            t = np.nonzero(sel)[0]
            h[t, k * K + cols[k, t, s]] = vals[k, t, s]
    bv = vals_value(cfg, host["bk_vals"])
    for e in range(len(host["bk_tile"])):
        k, t = int(host["bk_tile"][e]), int(host["bk_tok"][e])
        nz = np.nonzero(bv[e])[0]
        h[t, k * K + nz] = bv[e, nz]
    return h


def assert_y_close(y, ref, dtype: str, what=""):
    """The layer's output tolerance: bf16 max|d| <= 1e-2(1+|ref|), rel-Frobenius <= 5e-3;
    fp32 max|d| <= 1e-4(1+|ref|), rel-Frobenius <= 1e-5."""
    if dtype == "bf16":
        ea, ef = 1e-2, 5e-3
    else:
        ea, ef = 1e-4, 1e-5
    d = np.abs(y - ref)
    bad = d > ea * (1.0 + np.abs(ref))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond {ea}(1+|ref|); max {d.max():.3e}"
    nr = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / nr if nr > 0 else np.linalg.norm(y)
    assert rel <= ef, f"{what}: relative Frobenius error {rel:.3e} > {ef}"
    return rel


def fp32_sum_band(x64, W64, b64, rows=None):
    """Bound on |z_fp32 - z_exact| for z = sum_i x_i W_ji + b_j accumulated in fp32 in any
    order (Higham's recursive-summation bound gamma_{n} = n u / (1 - n u), u = 2^-24, with
    n = D + 1 terms; products of bf16 inputs are exact in fp32)."""
    D = x64.shape[1]
    u = 2.0 ** -24
    n = D + 1
    gamma = n * u / (1 - n * u)
    xa = np.abs(x64 if rows is None else x64[rows])
    return gamma * (xa @ np.abs(W64).T + np.abs(b64)[None, :])


def check_backup_structure(cfg, host: dict, T: int):
    """Invariants of the backup that hold at any size."""
    W = cfg.ell_width
    counts = host["counts"].astype(np.int64)
    over = np.argwhere(counts > W)  # ascending (k, t)
    assert host["bk_n"] == len(over)
    r = min(len(over), cfg.backup_capacity)
    assert np.array_equal(host["bk_tile"][:r], over[:r, 0])
    assert np.array_equal(host["bk_tok"][:r], over[:r, 1])
    ptr = host["bk_tile_ptr"]
    per_tile = (counts > W).sum(axis=1)
    assert np.array_equal(ptr, np.concatenate([[0], np.cumsum(per_tile)]))
    if r:
        bv = vals_value(cfg, host["bk_vals"][:r])
        nnz = (bv != 0).sum(axis=1)
        assert np.array_equal(nnz, counts[over[:r, 0], over[:r, 1]] - W)
