"""GPU parity of sparse_ffn_backward (through the C ABI) against the CPU fp64 oracle.

The oracle runs its backward (O9) from the activations the GPU stored (the forward's TwELL,
decoded), the same x, dy and weights, with dh stored in bf16 (the O8 model, as the GPU
stores dh).  Checked: dh only at h's stored positions and within the layer tolerance there;
dW_down within the layer tolerance and near fp32-exact; dW_up, db and dx within the layer
tolerance of the oracle's dh-consuming half run on the dh the GPU stored, and by relative
Frobenius error against the oracle's own dh and against unrounded dh; bit-identical
results on a second run.
"""
import numpy as np
import pytest

import oracle
from gen import CONFIGS, f32_to_bf16_bits, make_layer
from tests.gpu_helpers import (assert_y_close, decode_dense, layer_to_dev, need_gpu,
                               to_dev_bf16, y_to_host)

pytestmark = pytest.mark.gpu


def _cfg(sffn, T, c, cap=None):
    cap = c.n_tiles * T if cap is None else cap
    return sffn.Config(d_model=c.D, d_ff=c.F, tile=c.tile, ell_width=c.ell_width, max_tokens=T,
                       backup_capacity=cap, dtype=c.dtype)


def _rel(a, ref):
    n = np.linalg.norm(ref)
    return np.linalg.norm(a - ref) / n if n > 0 else np.linalg.norm(a)


def _backward_case(torch, sffn, L, seed=7):
    c = L["cfg"]
    T = c.T
    cfg = _cfg(sffn, T, c)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    y, act = layer.forward(x)
    assert sffn.check(act) == sffn.SFFN_OK
    g_bits = f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, c.D)).astype(np.float32))
    dy = to_dev_bf16(torch, g_bits)
    dx, dWu, dWd, db, dh_vals, dh_bk = layer.backward(x, dy, act)
    torch.cuda.synchronize()

    host = act.to_host()
    h_st = decode_dense(cfg, host, T)  # the activations exactly as stored
    dhost = dict(host)
    dhost["vals"] = dh_vals.view(torch.int16).cpu().numpy().view(np.uint16)
    r = min(host["bk_n"], cfg.backup_capacity)
    dhost["bk_vals"] = dh_bk.view(torch.int16).cpu().numpy().view(np.uint16)[:r]
    dh_gpu = decode_dense(cfg, dhost, T)

    x64, Wu64, Wd64 = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "W_down_f32"))
    g64 = oracle.bf16_value(g_bits)
    dx_r, dWu_r, dWd_r, db_r, dh_r = oracle.backward(x64, h_st, g64, Wu64, Wd64, round_dh=True)

    mask = h_st != 0
    assert not np.any(dh_gpu[~mask]), "dh written outside h's stored positions"
    assert_y_close(dh_gpu[mask], dh_r[mask], "bf16", f"dh {c.name}")
    dWd_h = dWd.cpu().numpy().astype(np.float64)
    assert_y_close(dWd_h, dWd_r, "bf16", f"dW_down {c.name}")
    assert _rel(dWd_h, dWd_r) <= 1e-4, "dW_down (no bf16 intermediate) should be near fp32 exact"
    dWu_h = dWu.cpu().numpy().astype(np.float64)
    db_h = db.cpu().numpy().astype(np.float64)
    dx_h = y_to_host(torch, dx)
    # dW_up, db and dx from the dh the GPU stored (its bf16 rounding of an fp32 sum can sit
    # one ulp away from the oracle's rounding of the exact sum), so that these compare the
    # kernels that consume dh
    fx, fwu, fdb = oracle.backward_from_dh(x64, dh_gpu, Wu64)
    assert_y_close(dWu_h, fwu, "bf16", f"dW_up {c.name}")
    assert_y_close(db_h, fdb, "bf16", f"db {c.name}")
    assert_y_close(dx_h, fx, "bf16", f"dx {c.name}")
    for name, got, want in (("dx", dx_h, dx_r), ("dW_up", dWu_h, dWu_r), ("db", db_h, db_r)):
        assert _rel(got, want) <= 5e-3, f"{name} vs oracle dh: {_rel(got, want):.3e}"
    # against exact (unrounded) dh, the relative Frobenius bound still holds
    ex = oracle.backward(x64, h_st, g64, Wu64, Wd64, round_dh=False)
    for name, got, want in (("dx", dx_h, ex[0]), ("dW_up", dWu_h, ex[1]), ("db", db_h, ex[3])):
        assert _rel(got, want) <= 5e-3, f"{name} vs exact dh: {_rel(got, want):.3e}"
    # deterministic: a second run gives the same bits
    dx2, dWu2, dWd2, db2, dh2, dhb2 = layer.backward(x, dy, act)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dWu, dWu2) and torch.equal(dWd, dWd2) and torch.equal(db, db2)
    assert torch.equal(dh_vals.view(torch.int16), dh2.view(torch.int16))
    return host


@pytest.mark.parametrize("name,T,rho", [
    ("C5", 300, None),      # 1.5B-like training layer (tile 128, W 32), ragged T
    ("C2", 200, None),      # 0.5B-like: W 48, 20% density
    ("C4", 260, None),      # 2B-like: tile 256 (two column halves per tile), W 16
    ("C5", 130, 0.20),      # dense enough that many rows overflow into the backup
    ("C5/w16", 200, None),  # tile 128 with 16 slots: half of the unit lanes idle
    ("C5/w64", 140, 0.50),  # tile 128 with 64 slots (two units per lane); rows overflow
])
def test_backward_parity(name, T, rho):
    torch, sffn = need_gpu()
    print(f"[backward] {name} T={T} rho={rho}", flush=True)
    base, _, w = name.partition("/w")
    cfg = CONFIGS[base] if not w else CONFIGS[base].replace(ell_width=int(w))
    L = make_layer(cfg, seed=0, T=T, rho=rho)
    host = _backward_case(torch, sffn, L)
    if rho is not None and rho >= 0.20:
        assert host["bk_n"] > 0, "the case should exercise backup rows"


def test_backward_heavy_rows():
    """2B-like layer at a reduced T with heavy rows: dh backup slices are in use."""
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C4"], seed=0, T=400)
    host = _backward_case(torch, sffn, L)
    assert host["bk_n"] > 0


def test_backward_arguments():
    torch, sffn = need_gpu()
    c = CONFIGS["C5"]
    T = 64
    cfg = sffn.Config(d_model=c.D, d_ff=c.F, tile=c.tile, ell_width=c.ell_width, max_tokens=T,
                      backup_capacity=16, dtype="bf16")
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    layer = sffn.SparseFFN(cfg, z(c.F, c.D), z(c.F), z(c.F, c.D))
    x = z(T, c.D)
    y, act = layer.forward(x)
    with pytest.raises(ValueError):
        layer.backward(x, z(T + 1, c.D), act)
    # an unsupported shape is refused before any launch
    cfg2 = sffn.Config(d_model=128, d_ff=256, tile=64, ell_width=16, max_tokens=T,
                       backup_capacity=16, dtype="bf16")
    layer2 = sffn.SparseFFN(cfg2, z(256, 128), z(256), z(256, 128))
    x2 = z(T, 128)
    _, act2 = layer2.forward(x2)
    with pytest.raises(sffn.SffnError) as ei:
        layer2.backward(x2, x2, act2)
    assert "SFFN_ERR_UNSUPPORTED" in str(ei.value)


def test_backward_full_size():
    """The 1.5B-like training layer at its full size (T=8192), in the launch configuration
    the benchmark times, compared with the oracle everywhere: dh and dx of every token (dh at
    the stored positions of the activation, dx from that dh), and every entry of dW_down,
    dW_up and db (sums over all tokens of the stored activations and of the stored dh)."""
    torch, sffn = need_gpu()
    print("[backward-full] C5", flush=True)
    L = make_layer(CONFIGS["C5"], seed=0)
    c = L["cfg"]
    T = c.T
    cfg = _cfg(sffn, T, c, cap=c.n_tiles * T // 8)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    y, act = layer.forward(x)
    assert sffn.check(act) == sffn.SFFN_OK
    g_bits = f32_to_bf16_bits(np.random.default_rng(3).standard_normal((T, c.D)).astype(np.float32))
    dy = to_dev_bf16(torch, g_bits)
    dx, dWu, dWd, db, dh_vals, dh_bk = layer.backward(x, dy, act)
    torch.cuda.synchronize()
    host = act.to_host()
    r = min(host["bk_n"], cfg.backup_capacity)
    dhost = dict(host)
    dhost["vals"] = dh_vals.view(torch.int16).cpu().numpy().view(np.uint16)
    dhost["bk_vals"] = dh_bk.view(torch.int16).cpu().numpy().view(np.uint16)[:r]
    rows = np.arange(T, dtype=np.int64)
    from tests.test_gpu_parity import _decode_rows
    h_rows = _decode_rows(cfg, host, rows)
    dh_rows = _decode_rows(cfg, dhost, rows)
    x64, Wu64, Wd64 = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "W_down_f32"))
    g64 = oracle.bf16_value(g_bits)
    dh_r = oracle.dh_rows(h_rows, g64, Wd64, round_dh=True)
    mask = h_rows != 0
    assert not np.any(dh_rows[~mask])
    assert_y_close(dh_rows[mask], dh_r[mask], "bf16", "full dh")
    dx_rows = y_to_host(torch, dx)
    assert_y_close(dx_rows, oracle.dx_rows(dh_rows, Wu64), "bf16", "full dx")
    assert _rel(dx_rows, oracle.dx_rows(dh_r, Wu64)) <= 5e-3
    del dh_r

    # every entry of the weight gradients: dW_down = H^T g over the stored activations,
    # dW_up = dH^T x and db = the column sums of dH over the stored dh
    dWd_h = dWd.cpu().numpy().astype(np.float64)
    dWu_h = dWu.cpu().numpy().astype(np.float64)
    dbh = db.cpu().numpy().astype(np.float64)
    wd_ref, _ = oracle.dw(h_rows, g64)
    del h_rows
    assert_y_close(dWd_h, wd_ref, "bf16", "full dW_down")
    assert _rel(dWd_h, wd_ref) <= 1e-4
    del wd_ref
    wu_ref, db_ref = oracle.dw(dh_rows, x64)
    assert_y_close(dWu_h, wu_ref, "bf16", "full dW_up")
    assert _rel(dWu_h, wu_ref) <= 1e-4
    assert_y_close(dbh, db_ref, "bf16", "full db")
