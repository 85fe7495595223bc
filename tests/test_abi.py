"""Host-only checks of the C ABI: the library loads, exports every function the header
declares, sizes buffers as documented, and rejects bad arguments before touching the GPU.
Runs without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_ffn.h")


@pytest.fixture(scope="module")
def sffn():
    import activation_sparse_transformer_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libsparse_ffn.so is not built (run __graft_entry__.build())")
    m.lib()
    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_header_symbols_exported(sffn):
    names = _declared_functions()
    assert "sparse_ffn_forward" in names and "twell_pack" in names and "twell_stats" in names
    L = ctypes.CDLL(sffn.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # the binding wraps exactly the declared functions
    from activation_sparse_transformer_amd import sparse_ffn as b
    assert sorted(b.exported_names()) == names


# The entry points the boundary is specified to export (the interface list the hot path
# is built behind): each must be declared, exported and documented.
BOUNDARY = ["twell_buffer_bytes", "sparse_ffn_create", "sparse_ffn_destroy", "twell_pack",
            "sparse_ffn_forward", "twell_stats", "sparse_ffn_check", "sparse_ffn_backward",
            "sffn_status_string", "sffn_last_error"]


def test_header_declares_boundary_with_comments(sffn):
    """Every boundary function is declared in the header, and every declaration in the
    header is preceded by its own comment block (meaning, layout, ownership, errors)."""
    text = open(HEADER).read()
    names = _declared_functions()
    for n in BOUNDARY:
        assert n in names, n
    for n in names:
        m = re.search(r"(\*/)\s*(?:const\s+)?[a-z_]+\s*\*?\s*" + n + r"\s*\(", text)
        assert m is not None, f"{n}: no comment block right before its declaration"


def test_buffer_bytes_matches_sizes(sffn):
    cfg = sffn.Config(d_model=2048, d_ff=8192, tile=128, ell_width=32, max_tokens=8192,
                      backup_capacity=4096, dtype="bf16")
    for T in (1, 100, 8192):
        s = sffn.buffer_sizes(cfg, T)
        b = sffn.buffer_bytes(cfg, T)
        assert b == [s[n] for n in sffn.BUFFER_FIELDS]
    with pytest.raises(sffn.SffnError):
        sffn.buffer_bytes(cfg, 0)
    from activation_sparse_transformer_amd.sparse_ffn import ConfigC, lib
    c = cfg.c()
    assert lib().twell_buffer_bytes(ctypes.byref(c), 8, None) == 1


def test_header_constants_match_binding(sffn):
    """The binding's down-policy codes, thresholds and token-count rules equal the header's
    #defines (the library reads the header's)."""
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(SFFN_DOWN_[A-Z_]+)\s+([0-9.]+)f?", text))
    want = {"SFFN_DOWN_AUTO": sffn.DOWN_AUTO, "SFFN_DOWN_GATHER": sffn.DOWN_GATHER,
            "SFFN_DOWN_MFMA": sffn.DOWN_MFMA, "SFFN_DOWN_TILES": sffn.DOWN_TILES,
            "SFFN_DOWN_UNION": sffn.DOWN_UNION, "SFFN_DOWN_SPARSE": sffn.DOWN_SPARSE,
            "SFFN_DOWN_GATHER_DENSITY_DEFAULT": sffn.DOWN_GATHER_DENSITY_DEFAULT,
            "SFFN_DOWN_MFMA_DENSITY_DEFAULT": sffn.DOWN_MFMA_DENSITY_DEFAULT,
            "SFFN_DOWN_TILES_MIN_T": sffn.DOWN_TILES_MIN_T,
            "SFFN_DOWN_MFMA_MIN_T": sffn.DOWN_MFMA_MIN_T}
    assert set(defs) == set(want), sorted(defs)
    for k, v in want.items():
        assert float(defs[k]) == pytest.approx(v, rel=1e-6), k
    assert sffn.DOWN_GATHER_DENSITY_DEFAULT <= sffn.DOWN_MFMA_DENSITY_DEFAULT
    mt = re.search(r"#define\s+SFFN_MAX_TILES\s+([0-9]+)", text)
    assert mt and int(mt.group(1)) == sffn.MAX_TILES
    nb = re.search(r"#define\s+SFFN_N_BUFFERS\s+([0-9]+)", text)
    assert nb and int(nb.group(1)) == len(sffn.BUFFER_FIELDS)


def test_status_strings(sffn):
    from activation_sparse_transformer_amd.sparse_ffn import status_string
    assert status_string(0) == "SFFN_OK"
    assert status_string(3) == "SFFN_ERR_BACKUP_OVERFLOW"
    assert status_string(99) == "SFFN_UNKNOWN_STATUS"


def test_buffer_sizes_formula(sffn):
    cfg = sffn.Config(d_model=2048, d_ff=8192, tile=128, ell_width=32, max_tokens=8192,
                      backup_capacity=4096, dtype="bf16")
    s = sffn.buffer_sizes(cfg, 8192)
    nt = 64
    assert s["counts"] == 2 * (nt * 8192 + 32)
    # [n_t, T, W] plus 32 tile-rows of padding read by whole-group loads
    assert s["vals"] == 2 * (nt * 8192 + 32) * 32
    assert s["cols"] == (nt * 8192 + 32) * 32
    assert s["bk_vals"] == 2 * 4096 * 128
    assert s["bk_tile"] == s["bk_tok"] == 4 * 4096
    assert s["bk_tile_ptr"] == 4 * (nt + 1)
    assert s["workspace"] > 0
    s32 = sffn.buffer_sizes(cfg.__class__(**{**cfg.__dict__, "dtype": "f32"}), 100)
    assert s32["vals"] == 4 * (nt * 100 + 32) * 32


@pytest.mark.parametrize("kw,code", [
    ({"tile": 100}, 2), ({"tile": 512}, 2), ({"ell_width": 0}, 1), ({"ell_width": 129}, 1),
    ({"d_ff": 1000}, 1), ({"d_model": 100}, 2), ({"max_tokens": 0}, 1),
    ({"backup_capacity": -1}, 1), ({"d_model": 0}, 1),
    ({"d_ff": 4097 * 64, "tile": 64, "backup_capacity": 0}, 2),  # more than SFFN_MAX_TILES tiles
])
def test_config_validation(sffn, kw, code):
    base = dict(d_model=256, d_ff=1024, tile=128, ell_width=32, max_tokens=64,
                backup_capacity=16, dtype="bf16")
    base.update(kw)
    with pytest.raises(sffn.SffnError) as ei:
        sffn.buffer_sizes(sffn.Config(**base), 8)
    assert ei.value.status == code


def test_T_range(sffn):
    cfg = sffn.Config(256, 1024, 128, 32, 64, 16, "bf16")
    for T in (0, 65, -1):
        with pytest.raises(sffn.SffnError) as ei:
            sffn.buffer_sizes(cfg, T)
        assert ei.value.status == sffn.SFFN_ERR_INVALID_ARGUMENT
    sffn.buffer_sizes(cfg, 64)


def test_layer_shape_constraints(sffn):
    from activation_sparse_transformer_amd.sparse_ffn import ConfigC, lib
    L = lib()
    dummy = ctypes.c_void_p(0x1000)
    h = ctypes.c_void_p()
    # bf16 layer with d_ff not a multiple of 256
    c = ConfigC(256, 1152, 128, 32, 64, 16, 1)
    assert L.sparse_ffn_create(ctypes.byref(c), dummy, dummy, dummy, ctypes.byref(h)) == 2
    # bf16 layer with d_model not a multiple of 128
    c = ConfigC(192, 1024, 128, 32, 64, 16, 1)
    assert L.sparse_ffn_create(ctypes.byref(c), dummy, dummy, dummy, ctypes.byref(h)) == 2
    # fp32 allows both
    c = ConfigC(192, 1152, 128, 32, 64, 16, 0)
    assert L.sparse_ffn_create(ctypes.byref(c), dummy, dummy, dummy, ctypes.byref(h)) == 0
    assert L.sparse_ffn_destroy(h) == 0
    # NULL weights
    assert L.sparse_ffn_create(ctypes.byref(c), None, dummy, dummy, ctypes.byref(h)) == 1
    assert L.sparse_ffn_destroy(None) == 0


def test_null_arguments_rejected_before_launch(sffn):
    """Every entry point validates pointers on the host; nothing reaches HIP."""
    from activation_sparse_transformer_amd.sparse_ffn import BuffersC, ConfigC, StatsC, lib
    L = lib()
    c = ConfigC(256, 1024, 128, 32, 64, 16, 0)
    empty = BuffersC()
    dummy = ctypes.c_void_p(0x1000)
    assert L.twell_pack(ctypes.byref(c), None, 8, ctypes.byref(empty), None) == 1
    assert L.twell_pack(ctypes.byref(c), dummy, 8, ctypes.byref(empty), None) == 1
    assert L.twell_pack(ctypes.byref(c), dummy, 8, None, None) == 1
    assert L.twell_pack(None, dummy, 8, ctypes.byref(empty), None) == 1
    assert L.sparse_ffn_forward(None, dummy, 8, dummy, ctypes.byref(empty), None) == 1
    h = ctypes.c_void_p()
    assert L.sparse_ffn_create(ctypes.byref(c), dummy, dummy, dummy, ctypes.byref(h)) == 0
    assert L.sparse_ffn_forward(h, None, 8, dummy, ctypes.byref(empty), None) == 1
    assert L.sparse_ffn_forward(h, dummy, 8, dummy, ctypes.byref(empty), None) == 1
    assert L.sparse_ffn_forward(h, dummy, 65, dummy, ctypes.byref(empty), None) == 1
    assert L.sparse_ffn_down(h, ctypes.byref(empty), 8, dummy, None) == 1
    assert L.sparse_ffn_forward_dump(h, dummy, 8, dummy, ctypes.byref(empty), None, None) == 1
    assert L.twell_stats(ctypes.byref(c), ctypes.byref(empty), 8, ctypes.byref(StatsC()), None) == 1
    assert L.sparse_ffn_check(None, None) == 1
    assert L.sffn_profile_read(None, None, None) == 1
    assert L.sparse_ffn_destroy(h) == 0
    assert b"NULL" in L.sffn_last_error()


def test_probe_arguments_rejected_before_launch(sffn):
    """The gather-multiply-add probe checks its pointers and sizes on the host."""
    from activation_sparse_transformer_amd.sparse_ffn import lib
    L = lib()
    d_ = ctypes.c_void_p(0x1000)
    assert L.sffn_probe_gather_fma(None, 16, 64, d_, d_, 4, 3, d_, None) == 1
    assert L.sffn_probe_gather_fma(d_, 16, 64, None, d_, 4, 3, d_, None) == 1
    assert L.sffn_probe_gather_fma(d_, 16, 64, d_, d_, 4, 3, None, None) == 1
    assert L.sffn_probe_gather_fma(d_, 16, 60, d_, d_, 4, 3, d_, None) == 1   # d % 8
    assert L.sffn_probe_gather_fma(d_, 0, 64, d_, d_, 4, 3, d_, None) == 1    # F
    assert L.sffn_probe_gather_fma(d_, 16, 64, d_, d_, 0, 3, d_, None) == 1   # T
    assert L.sffn_probe_gather_fma(d_, 16, 64, d_, d_, 4, -1, d_, None) == 1  # n
    assert b"probe" in L.sffn_last_error()
    assert L.sffn_probe_gather_fma(d_, 16, 64, d_, None, 4, 3, d_, None) == 1   # vals, n > 0


def test_profile_counters_host_only(sffn):
    sffn.profile_enable(True)
    sffn.profile_reset()
    ms, n = sffn.profile_read("up_pack")
    assert ms == 0.0 and n == 0
    sffn.profile_only(["up_pack", "down_mfma"])
    sffn.profile_only(None)
    sffn.profile_enable(False)


def test_product_path_does_not_import_oracle():
    """The HIP binding must never reach the CPU oracle."""
    pkg = os.path.join(ROOT, "activation_sparse_transformer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower().replace("oracle_", ""), f


@pytest.mark.parametrize("D,F,K,W,dtype", [
    (2048, 8192, 128, 32, "bf16"), (1024, 4096, 64, 16, "bf16"), (4096, 16384, 256, 64, "bf16"),
    (256, 1024, 128, 32, "f32")])
def test_buffer_sizes_monotone_in_T(sffn, D, F, K, W, dtype):
    """Every field grows with T, so buffers sized for T serve every call with fewer tokens
    (the split partial sums of the matrix-core down kernel and the small-batch up buffer
    included, which are not monotone per call)."""
    cfg = sffn.Config(d_model=D, d_ff=F, tile=K, ell_width=W, max_tokens=8192,
                      backup_capacity=1024, dtype=dtype)
    Ts = sorted(set(list(range(1, 300, 7)) + [128, 129, 255, 256, 257, 511, 512, 513, 1024,
                                              2048, 2049, 4096, 8191, 8192]))
    prev = None
    for T in Ts:
        s = sffn.buffer_sizes(cfg, T)
        if prev is not None:
            for k, v in s.items():
                assert v >= prev[k], (k, T, v, prev[k])
        prev = s


def test_choose_ell_width_matches_oracle(sffn):
    """The library's width choice (host code) equals the oracle's on random and edge
    histograms, with and without a candidate list; bad arguments are refused."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)
    for K, dtype in ((64, "bf16"), (128, "bf16"), (256, "f32"), (128, "f32")):
        cfg = sffn.Config(d_model=256, d_ff=4 * K, tile=K, ell_width=8, max_tokens=64,
                          backup_capacity=16, dtype=dtype)
        esz = 2 if dtype == "bf16" else 4
        for trial in range(25):
            lam = rng.uniform(0.5, K * 0.7)
            hist = np.bincount(np.minimum(rng.poisson(lam, 5000), K), minlength=K + 1).astype(np.int64)
            if trial % 5 == 0:
                hist[K] += rng.integers(0, 300)  # dense tile-rows
            assert sffn.choose_ell_width(cfg, hist) == oracle.choose_ell_width(hist, K, esz)
            cands = [w for w in (16, 32, 48, 64) if w <= K]
            assert sffn.choose_ell_width(cfg, hist, cands) == oracle.choose_ell_width(hist, K, esz, cands)
        zero = np.zeros(K + 1, np.int64)
        assert sffn.choose_ell_width(cfg, zero) == oracle.choose_ell_width(zero, K, esz)
        with pytest.raises(sffn.SffnError):
            sffn.choose_ell_width(cfg, zero, [0])
        with pytest.raises(sffn.SffnError):
            sffn.choose_ell_width(cfg, zero, [K + 1])
        bad = zero.copy()
        bad[3] = -1
        with pytest.raises(sffn.SffnError):
            sffn.choose_ell_width(cfg, bad)
