"""GPU parity of the HIP path (through the C ABI) against the CPU fp64 oracle.

* twell_pack: bit-exact TwELL (counts, values, columns, padding, ordered backup) for the
  same fp32 hidden tensor, fp32 and bf16 values, several tile/width settings, ragged T.
* sparse_ffn_down: y from a TwELL within the layer tolerance of the oracle's y.
* sparse_ffn_forward: y within tolerance; the fused TwELL pattern equals the oracle's
  wherever the fp32 sign of z is certain, and equals the standalone pack of the kernel's
  own fp32 z bit for bit.
"""
import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_hidden, make_layer
from tests.gpu_helpers import (assert_y_close, check_backup_structure, decode_dense,
                               fp32_sum_band, layer_to_dev, need_gpu, to_dev_f32, vals_value,
                               y_to_host)

pytestmark = pytest.mark.gpu


def _cfg(sffn, T, D, F, K, W, dtype, cap=None):
    nt = F // K
    cap = nt * T if cap is None else cap
    return sffn.Config(d_model=D, d_ff=F, tile=K, ell_width=W, max_tokens=T,
                       backup_capacity=cap, dtype=dtype)


def _compare_pack(cfg, host, tw, T, exact_values=True):
    K, W = cfg.tile, cfg.ell_width
    assert np.array_equal(host["counts"], tw.counts), "counts differ"
    assert np.array_equal(host["cols"], tw.cols), "cols differ"
    if cfg.dtype == "bf16":
        want_vals = oracle.round_bf16(tw.vals)
        want_bk = oracle.round_bf16(tw.bk_vals) if len(tw.bk_vals) else tw.bk_vals.astype(np.uint16)
    else:
        want_vals = tw.vals.astype(np.float32)
        want_bk = tw.bk_vals.astype(np.float32)
    assert np.array_equal(host["vals"].view(np.uint16 if cfg.dtype == "bf16" else np.uint32),
                          want_vals.view(np.uint16 if cfg.dtype == "bf16" else np.uint32)), "vals differ"
    assert host["bk_n"] == tw.n_backup
    r = min(tw.n_backup, cfg.backup_capacity)
    assert np.array_equal(host["bk_tile"][:r], tw.bk_tile[:r])
    assert np.array_equal(host["bk_tok"][:r], tw.bk_tok[:r])
    hb = host["bk_vals"][:r]
    assert np.array_equal(hb.view(np.uint16 if cfg.dtype == "bf16" else np.uint32),
                          want_bk[:r].view(np.uint16 if cfg.dtype == "bf16" else np.uint32)), "backup differs"


PACK_CASES = [
    # (T, F, K, W, dtype, density)
    (1, 256, 128, 32, "bf16", 0.1),
    (63, 512, 64, 8, "f32", 0.2),
    (65, 512, 128, 16, "bf16", 0.2),
    (300, 1024, 128, 32, "bf16", 0.05),
    (300, 1024, 128, 32, "f32", 0.3),
    (257, 1024, 256, 16, "bf16", 0.06),
    (200, 768, 256, 256, "f32", 0.5),
    (130, 512, 128, 1, "bf16", 0.02),
    (100, 512, 128, 128, "bf16", 0.9),
    (77, 384, 64, 63, "f32", 0.95),
    (333, 1152, 64, 5, "bf16", 0.1),
    # at least 2048 (tile, 32-token group) pairs: the one-wave-per-group pack kernel
    (4100, 4096, 64, 16, "bf16", 0.05),
    (2049, 4096, 128, 8, "f32", 0.1),
    # exactly 1024 pairs (the last size the one-launch backup order takes), and 2064 pairs
    (4096, 1024, 128, 16, "bf16", 0.1),
    (4097, 2048, 128, 16, "f32", 0.1),
]


@pytest.mark.parametrize("T,F,K,W,dtype,density", PACK_CASES)
def test_pack_bitexact(T, F, K, W, dtype, density):
    torch, sffn = need_gpu()
    print(f"[pack] T={T} F={F} K={K} W={W} {dtype} rho={density}", flush=True)
    h = make_hidden(T, F, density, seed=T + F + K + W, signed_zero=True,
                    heavy_rows=(0, T - 1), heavy_density=0.7)
    cfg = _cfg(sffn, T, 64, F, K, W, dtype)
    buf = sffn.twell_pack(cfg, to_dev_f32(torch, h))
    host = buf.to_host()
    assert host["status"] == 0
    tw = oracle.pack(h.astype(np.float64), K, W)
    _compare_pack(cfg, host, tw, T)
    check_backup_structure(cfg, host, T)
    st = sffn.twell_stats(cfg, buf)
    ost = oracle.stats(tw)
    for k in ("nnz", "slots_used", "overflow_tile_rows", "backup_nonzeros", "max_count"):
        assert st[k] == ost[k], k


def test_pack_edges():
    torch, sffn = need_gpu()
    T, F, K, W = 70, 512, 128, 16
    cfg = _cfg(sffn, T, 64, F, K, W, "bf16")
    for name, h in (("zeros", np.zeros((T, F), np.float32)),
                    ("ones", np.full((T, F), 0.75, np.float32)),
                    ("negzero", np.full((T, F), -0.0, np.float32))):
        print(f"[pack-edge] {name}", flush=True)
        buf = sffn.twell_pack(cfg, to_dev_f32(torch, h))
        host = buf.to_host()
        tw = oracle.pack(h.astype(np.float64), K, W)
        _compare_pack(cfg, host, tw, T)
    # count == W and W + 1 in the same tile
    h = np.zeros((T, F), np.float32)
    h[3, :W] = 1.0
    h[4, :W + 1] = 2.0
    buf = sffn.twell_pack(cfg, to_dev_f32(torch, h))
    host = buf.to_host()
    assert host["counts"][0, 3] == W and host["counts"][0, 4] == W + 1
    assert host["bk_n"] == 1 and host["bk_tok"].tolist() == [4]


def test_pack_capacity():
    torch, sffn = need_gpu()
    T, F, K, W = 96, 512, 128, 4
    h = make_hidden(T, F, 0.1, seed=9)
    need = oracle.pack(h.astype(np.float64), K, W).n_backup
    assert need > 2
    ok = _cfg(sffn, T, 64, F, K, W, "bf16", cap=need)
    buf = sffn.twell_pack(ok, to_dev_f32(torch, h))
    assert sffn.check(buf) == sffn.SFFN_OK
    short = _cfg(sffn, T, 64, F, K, W, "bf16", cap=need - 1)
    buf = sffn.twell_pack(short, to_dev_f32(torch, h))
    assert sffn.check(buf) == sffn.SFFN_ERR_BACKUP_OVERFLOW
    st = sffn.twell_stats(short, buf, raise_on_overflow=False)
    assert st["status"] == sffn.SFFN_ERR_BACKUP_OVERFLOW and st["backup_needed"] == need
    zero = _cfg(sffn, T, 64, F, K, W, "bf16", cap=0)
    buf = sffn.twell_pack(zero, to_dev_f32(torch, h))
    assert sffn.check(buf) == sffn.SFFN_ERR_BACKUP_OVERFLOW


DOWN_CASES = [
    (300, 256, 1024, 128, 32, "bf16", 0.05),
    (97, 512, 1024, 128, 8, "bf16", 0.2),
    (200, 256, 1024, 256, 16, "bf16", 0.08),
    (130, 384, 512, 64, 6, "bf16", 0.15),
    (150, 256, 1024, 128, 32, "f32", 0.1),
    (64, 128, 512, 128, 7, "bf16", 0.1),
    # shapes the matrix-core down-projection takes (bf16, W in 16/32/48/64): every width,
    # every tile size, ragged T, several token blocks
    (300, 256, 1024, 128, 48, "bf16", 0.2),
    (520, 384, 1024, 64, 64, "bf16", 0.3),
    (257, 128, 2048, 256, 48, "bf16", 0.1),
    (33, 256, 512, 64, 16, "bf16", 0.1),
    # 128-column tiles with 16 slots: two 8-slot units per row in the decode-once rebuild
    (200, 256, 1024, 128, 16, "bf16", 0.1),
    # fp32 layers of at most 128 tokens (the per-token row gather over 256-column chunks):
    # a partial last chunk, overflowing rows at every tile size, fewer tiles than waves
    (100, 320, 1024, 128, 32, "f32", 0.1),
    (17, 192, 512, 64, 8, "f32", 0.3),
    (3, 256, 768, 256, 40, "f32", 0.2),
]


@pytest.mark.parametrize("policy", ["gather", "tiles", "mfma", "union", "sparse"])
@pytest.mark.parametrize("T,D,F,K,W,dtype,density", DOWN_CASES)
def test_down_from_pack(T, D, F, K, W, dtype, density, policy):
    torch, sffn = need_gpu()
    print(f"[down] T={T} D={D} F={F} K={K} W={W} {dtype} {policy}", flush=True)
    rng = np.random.default_rng(T + D)
    h = make_hidden(T, F, density, seed=D + F, heavy_rows=(1, T // 2), heavy_density=0.6)
    Wd = (rng.standard_normal((F, D)) / np.sqrt(F)).astype(np.float32)
    cfg = _cfg(sffn, T, D, F, K, W, dtype)
    if dtype == "bf16":
        from gen import f32_to_bf16_bits, bf16_bits_to_f32
        Wd_bits = f32_to_bf16_bits(Wd)
        Wd64 = bf16_bits_to_f32(Wd_bits).astype(np.float64)
        h_ref = oracle.bf16_value(oracle.round_bf16(h.astype(np.float64)))
        Wd_dev = torch.from_numpy(Wd_bits.view(np.int16)).view(torch.bfloat16).cuda()
        Wu_dev = torch.zeros((F, D), dtype=torch.bfloat16, device="cuda")
        b_dev = torch.zeros(F, dtype=torch.bfloat16, device="cuda")
    else:
        Wd64 = Wd.astype(np.float64)
        h_ref = h.astype(np.float64)
        Wd_dev = to_dev_f32(torch, Wd)
        Wu_dev = torch.zeros((F, D), dtype=torch.float32, device="cuda")
        b_dev = torch.zeros(F, dtype=torch.float32, device="cuda")
    layer = sffn.SparseFFN(cfg, Wu_dev, b_dev, Wd_dev)
    layer.set_down_policy(policy)
    buf = sffn.twell_pack(cfg, to_dev_f32(torch, h))
    y = y_to_host(torch, layer.down(buf))
    tw = oracle.pack(h_ref, K, W)
    y_ref = oracle.down_sparse(tw, Wd64)
    assert_y_close(y, y_ref, dtype, f"down {policy}")
    # bit-identical on a second run
    y2 = y_to_host(torch, layer.down(buf))
    assert np.array_equal(y, y2)


def test_down_auto_policy_choice():
    """Token blocks with very different densities (0.1%, 4%, 0.3%, 2%; the last one ragged):
    the auto policy hands the whole layer to one kernel by its total stored density (about
    1.6% here), decided on the device.  Every row is written, the result matches the oracle,
    and it equals bit for bit the single-kernel result the thresholds select.  Below
    DOWN_TILES_MIN_T tokens the tiles range goes to the gather kernel."""
    torch, sffn = need_gpu()
    from gen import f32_to_bf16_bits, bf16_bits_to_f32
    T, D, F, K, W = 4200, 256, 2048, 128, 32
    assert T >= sffn.DOWN_TILES_MIN_T
    parts = [make_hidden(1024, F, 0.001, seed=11), make_hidden(1024, F, 0.04, seed=12),
             make_hidden(1024, F, 0.003, seed=13), make_hidden(1128, F, 0.02, seed=14)]
    h = np.concatenate(parts, axis=0)
    dens = np.count_nonzero(h) / h.size
    assert 0.01 < dens < 0.02
    rng = np.random.default_rng(5)
    Wd_bits = f32_to_bf16_bits((rng.standard_normal((F, D)) / np.sqrt(F)).astype(np.float32))
    Wd64 = bf16_bits_to_f32(Wd_bits).astype(np.float64)
    h_ref = oracle.bf16_value(oracle.round_bf16(h.astype(np.float64)))
    y_ref = oracle.down_sparse(oracle.pack(h_ref, K, W), Wd64)
    cfg = _cfg(sffn, T, D, F, K, W, "bf16")
    Wd_dev = torch.from_numpy(Wd_bits.view(np.int16)).view(torch.bfloat16).cuda()
    layer = sffn.SparseFFN(cfg, torch.zeros((F, D), dtype=torch.bfloat16, device="cuda"),
                           torch.zeros(F, dtype=torch.bfloat16, device="cuda"), Wd_dev)
    buf = sffn.twell_pack(cfg, to_dev_f32(torch, h))
    # (policy, gather_density, mfma_density) -> the kernel that must run
    cases = [("gather", 0.0, 0.0, "gather"), ("tiles", 0.0, 0.0, "tiles"),
             ("mfma", 0.0, 0.0, "mfma"), ("auto", 0.0, 0.0, "mfma"),
             ("auto", 1.0, 1.0, "gather"), ("auto", 0.0, 1.0, "tiles"),
             ("auto", 0.005, 0.03, "tiles"), ("auto", 0.02, 0.03, "gather"),
             ("auto", 0.002, 0.01, "mfma")]
    ys = {}
    for policy, tg, tm, expect in cases:
        layer.set_down_policy(policy, tg, tm)
        y = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        sffn.profile_reset()
        sffn.profile_enable(True)
        layer.down(buf, y=y)
        sffn.profile_enable(False)
        yh = y_to_host(torch, y)
        assert not np.isnan(yh).any(), f"{policy}/{tg}/{tm}: rows not written"
        assert_y_close(yh, y_ref, "bf16", f"{policy}/{tg}/{tm}")
        if policy != "auto":
            ys[expect] = yh
        else:
            assert np.array_equal(yh, ys[expect]), f"auto {tg}/{tm} should run {expect}"
        launched = {k: sffn.profile_read(n)[1] for k, n in
                    (("gather", "down"), ("tiles", "down_tiles"), ("mfma", "down_mfma"))}
        if policy == "auto":
            assert all(v == 1 for v in launched.values() if v) and launched[expect] == 1
        else:
            assert launched == {k: int(k == expect) for k in launched}, launched
    sffn.profile_reset()
    # a short activation (the first 48 tokens): the tiles range goes to the gather kernel,
    # and below DOWN_MFMA_MIN_T the matrix-core range too
    Ts = 48
    assert Ts < sffn.DOWN_MFMA_MIN_T
    cfg_s = _cfg(sffn, Ts, D, F, K, W, "bf16")
    layer_s = sffn.SparseFFN(cfg_s, torch.zeros((F, D), dtype=torch.bfloat16, device="cuda"),
                             torch.zeros(F, dtype=torch.bfloat16, device="cuda"), Wd_dev)
    buf_s = sffn.twell_pack(cfg_s, to_dev_f32(torch, h[:Ts]))
    y_refs = oracle.down_sparse(oracle.pack(h_ref[:Ts], K, W), Wd64)
    outs = {}
    for policy, tg, tm in (("gather", 0.0, 0.0), ("auto", 0.0, 1.0), ("auto", 0.0, 0.0)):
        layer_s.set_down_policy(policy, tg, tm)
        y = torch.full((Ts, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        layer_s.down(buf_s, y=y)
        outs[(policy, tm)] = y_to_host(torch, y)
        assert_y_close(outs[(policy, tm)], y_refs, "bf16", f"short {policy} {tm}")
    assert np.array_equal(outs[("auto", 1.0)], outs[("gather", 0.0)])
    assert np.array_equal(outs[("auto", 0.0)], outs[("gather", 0.0)])



@pytest.mark.parametrize("T", [64, 300])
def test_down_gather_candidate_runs(T):
    """Auto policy with every count in the gather's range, at token counts where the gather is
    launched as one candidate of the kernel choice: it runs, writes every row and matches the
    oracle; the matrix-core candidate returns."""
    torch, sffn = need_gpu()
    print(f"[down-candidate] T={T}", flush=True)
    D, F, K, W = 256, 1024, 128, 32
    h = make_hidden(T, F, 0.05, seed=T, heavy_rows=(1, T // 2), heavy_density=0.6)
    from gen import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(5)
    Wd_bits = f32_to_bf16_bits((rng.standard_normal((F, D)) / np.sqrt(F)).astype(np.float32))
    Wd_ref = bf16_bits_to_f32(Wd_bits).astype(np.float64)
    cfg = _cfg(sffn, T, D, F, K, W, "bf16")
    Wd_dev = torch.from_numpy(Wd_bits.view(np.int16)).view(torch.bfloat16).cuda()
    layer = sffn.SparseFFN(cfg, torch.zeros((F, D), dtype=torch.bfloat16, device="cuda"),
                           torch.zeros(F, dtype=torch.bfloat16, device="cuda"), Wd_dev)
    buf = sffn.twell_pack(cfg, to_dev_f32(torch, h))
    layer.set_down_policy("auto", 1.0, 1.0)
    y = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    try:
        sffn.profile_reset()
        sffn.profile_enable(True)
        layer.down(buf, y=y)
        sffn.profile_enable(False)
        assert sffn.profile_read("down")[1] == 1 and sffn.profile_read("down_mfma")[1] == 1
    finally:
        sffn.profile_enable(False)
        sffn.profile_reset()
    yh = y_to_host(torch, y)
    assert not np.isnan(yh).any(), "rows not written"
    # the bf16 TwELL stores the activations rounded to bf16
    h_ref = oracle.bf16_value(oracle.round_bf16(h.astype(np.float64)))
    y_ref = oracle.down_sparse(oracle.pack(h_ref, K, W), Wd_ref)
    assert_y_close(yh, y_ref, "bf16", f"gather candidate T={T}")
    layer.set_down_policy("gather")
    y2 = layer.down(buf)
    assert_y_close(y_to_host(torch, y2), y_ref, "bf16", f"gather alone T={T}")


def test_down_auto_policy_follows_the_last_count():
    """Auto policy over calls on one handle: the first call launches every candidate and the
    count decides on the device; the kernel that runs records its choice, and the next call
    launches that kernel alone.  When the density changes, the call after the change still
    runs the recorded kernel (a correct result at any density, equal to that kernel's forced
    result bit for bit) and records the new choice, which the call after it follows."""
    torch, sffn = need_gpu()
    from gen import f32_to_bf16_bits, bf16_bits_to_f32
    T, D, F, K, W = 300, 256, 1024, 128, 32
    rng = np.random.default_rng(8)
    Wd_bits = f32_to_bf16_bits((rng.standard_normal((F, D)) / np.sqrt(F)).astype(np.float32))
    Wd64 = bf16_bits_to_f32(Wd_bits).astype(np.float64)
    cfg = _cfg(sffn, T, D, F, K, W, "bf16")
    Wd_dev = torch.from_numpy(Wd_bits.view(np.int16)).view(torch.bfloat16).cuda()
    layer = sffn.SparseFFN(cfg, torch.zeros((F, D), dtype=torch.bfloat16, device="cuda"),
                           torch.zeros(F, dtype=torch.bfloat16, device="cuda"), Wd_dev)
    dense = make_hidden(T, F, 0.05, seed=21)
    sparse = make_hidden(T, F, 0.0003, seed=22)   # below the gather's 0.05% of T x F
    assert 0 < np.count_nonzero(sparse) <= 0.0005 * T * F < np.count_nonzero(dense)
    bufs = {k: sffn.twell_pack(cfg, to_dev_f32(torch, h)) for k, h in (("dense", dense), ("sparse", sparse))}
    refs = {}
    for k, h in (("dense", dense), ("sparse", sparse)):
        h_ref = oracle.bf16_value(oracle.round_bf16(h.astype(np.float64)))
        refs[k] = oracle.down_sparse(oracle.pack(h_ref, K, W), Wd64)
    forced = {}
    for pol in ("gather", "mfma"):
        layer.set_down_policy(pol)
        forced[pol] = {k: y_to_host(torch, layer.down(b)) for k, b in bufs.items()}
    layer.set_down_policy("auto")

    def call(which):
        sffn.profile_reset()
        sffn.profile_enable(True)
        try:
            yh = y_to_host(torch, layer.down(bufs[which]))
            launched = (sffn.profile_read("down")[1], sffn.profile_read("down_mfma")[1])
        finally:
            sffn.profile_enable(False)
            sffn.profile_reset()
        assert_y_close(yh, refs[which], "bf16", f"auto {which}")
        return yh, launched

    steps = [("dense", (1, 1), "mfma"),    # first call: both candidates, the count decides
             ("dense", (0, 1), "mfma"),    # recorded: the matrix cores alone
             ("sparse", (0, 1), "mfma"),   # density changed: the recorded kernel runs once more
             ("sparse", (1, 0), "gather"),  # and the new choice is followed
             ("dense", (1, 0), "gather"),
             ("dense", (0, 1), "mfma")]
    for which, launched_expect, kernel in steps:
        yh, launched = call(which)
        assert launched == launched_expect, (which, launched)
        assert np.array_equal(yh, forced[kernel][which]), (which, kernel)
    # a policy change forgets the recorded choice
    layer.set_down_policy("auto")
    yh, launched = call("sparse")
    assert launched == (1, 1) and np.array_equal(yh, forced["gather"]["sparse"])


def test_down_policy_arguments():
    torch, sffn = need_gpu()
    cfg = _cfg(sffn, 64, 128, 256, 128, 16, "bf16")
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    layer = sffn.SparseFFN(cfg, z(256, 128), z(256), z(256, 128))
    for g, m in ((-0.1, 0.5), (0.0, 1.5), (0.3, 0.2), (float("nan"), 0.5), (0.0, float("nan"))):
        with pytest.raises(sffn.SffnError):
            layer.set_down_policy("auto", g, m)
    with pytest.raises(ValueError):
        layer.set_down_policy("fastest")
    layer.set_down_policy("auto", 0.3, 0.3)  # equal thresholds: no tiles range


def _forward_case(torch, sffn, L, cap=None, check_pattern=True, policy="auto"):
    cfg0 = L["cfg"]
    T = cfg0.T
    cfg = _cfg(sffn, T, cfg0.D, cfg0.F, cfg0.tile, cfg0.ell_width, cfg0.dtype, cap)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    layer.set_down_policy(policy)
    y, act, z = layer.forward_dump(x)
    assert sffn.check(act) == sffn.SFFN_OK
    yh = y_to_host(torch, y)
    x64, Wu64, b64, Wd64 = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    h64, z64 = oracle.up_relu(x64, Wu64, b64, return_z=True)
    # a bf16 TwELL stores the activations in bf16 (nearest-even): the oracle applies the
    # same storage rounding (its O8 model) before the down-projection
    h_st = oracle.bf16_value(oracle.round_bf16(h64)) if cfg.dtype == "bf16" else h64
    tw = oracle.pack(h_st, cfg.tile, cfg.ell_width)
    y_ref = oracle.down_sparse(tw, Wd64)
    rel = assert_y_close(yh, y_ref, cfg.dtype, f"forward {cfg0.name}")
    # against the unrounded activations the relative Frobenius bound still holds
    y_exact = oracle.down_dense(h64, Wd64)
    nrm = np.linalg.norm(y_exact)
    if nrm == 0.0:
        assert not np.any(yh), "an all-zero hidden layer must give y == 0"
    else:
        rel_exact = np.linalg.norm(yh - y_exact) / nrm
        assert rel_exact <= (5e-3 if cfg.dtype == "bf16" else 1e-5), rel_exact
    host = act.to_host()
    check_backup_structure(cfg, host, T)
    if check_pattern:
        # fused pattern vs the oracle's, outside the fp32 rounding band of z
        band = fp32_sum_band(x64, Wu64, b64)
        gpu_h = decode_dense(cfg, host, T)
        certain = np.abs(z64) > band
        assert np.array_equal((gpu_h != 0)[certain], (z64 > 0)[certain]), "pattern differs"
        # stored values: bf16/fp32 rounding of a z within the band of z64
        nzc = certain & (z64 > 0)
        if cfg.dtype == "bf16":
            tol = np.abs(z64[nzc]) * 2.0 ** -8 + band[nzc]
        else:
            tol = np.abs(z64[nzc]) * 2.0 ** -23 + band[nzc]
        assert np.all(np.abs(gpu_h[nzc] - z64[nzc]) <= tol * 1.0001), "stored values off"
        # the fused epilogue equals the standalone pack of the kernel's own fp32 z
        hz = torch.relu(z).contiguous()
        ref_buf = sffn.twell_pack(cfg, hz)
        rh = ref_buf.to_host()
        for k in ("counts", "cols", "bk_tile", "bk_tok", "bk_tile_ptr"):
            assert np.array_equal(host[k], rh[k]), f"fused vs pack: {k}"
        assert np.array_equal(host["vals"].view(np.uint8), rh["vals"].view(np.uint8))
        assert np.array_equal(host["bk_vals"].view(np.uint8), rh["bk_vals"].view(np.uint8))
        assert host["bk_n"] == rh["bk_n"]
    return rel


@pytest.mark.parametrize("policy", ["gather", "tiles", "mfma", "union", "sparse"])
@pytest.mark.parametrize("name,T,rho", [
    ("C1", None, None), ("C1b", None, None), ("C1", 1, None), ("C1b", 100, None),
    ("C2", 300, None), ("C3", 300, 0.01), ("C3", 300, 0.05), ("C3", 300, 0.20),
    ("C4", 300, None),
    # decode-shaped batches (at most 128 tokens: the small-batch up-projection + pack path,
    # one to four 32-token blocks per workgroup, the last one ragged)
    ("C3", 1, 0.05), ("C3", 7, 0.01), ("C3", 32, 0.05), ("C2", 3, None), ("C4", 5, None),
    ("C3", 64, 0.05), ("C3", 100, 0.05), ("C2", 128, None), ("C4", 97, None),
    ("C3", 45, 0.05), ("C4", 33, None),
])
def test_forward_parity(name, T, rho, policy):
    torch, sffn = need_gpu()
    print(f"[forward] {name} T={T} rho={rho} {policy}", flush=True)
    L = make_layer(CONFIGS[name], seed=0, T=T, rho=rho)
    _forward_case(torch, sffn, L, policy=policy)


@pytest.mark.parametrize("policy", ["gather", "tiles", "mfma", "union", "sparse"])
def test_forward_heavy_rows_force_backup(policy):
    """2B-like layer at a reduced T with heavy rows: the backup is in use."""
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C4"], seed=0, T=400)
    assert len(L["heavy"]) >= 2
    _forward_case(torch, sffn, L, policy=policy)



@pytest.mark.parametrize("T", [32, 48])
@pytest.mark.parametrize("policy", ["auto", "gather", "union", "sparse"])
def test_forward_heavy_rows_short_batch(T, policy):
    """Decode-shaped batch of the 1.5B-like layer with two 3x-scaled token rows: most of their
    tile-rows overflow into the backup, and below 64 tokens the row gather (256-column chunks)
    is the only down kernel."""
    torch, sffn = need_gpu()
    print(f"[forward-heavy-short] T={T} {policy}", flush=True)
    L = make_layer(CONFIGS["C3"].replace(heavy_frac=2.0 / T), seed=0, T=T, rho=0.05)
    assert len(L["heavy"]) == 2
    _forward_case(torch, sffn, L, policy=policy)


@pytest.mark.parametrize("name,W,rho,T", [
    ("C3", 96, 0.7, 300), ("C3", 128, 0.9, 200), ("C4", 256, 0.9, 150), ("C4", 160, 0.6, 257)])
def test_forward_wide_ell(name, W, rho, T):
    """ELL widths far above the configured ones on the fused up-projection path (more than
    128 tokens): the pack epilogue stages a [32 tokens x W] block per tile and token half in
    LDS, which must hold W up to the tile width."""
    torch, sffn = need_gpu()
    print(f"[forward-wide] {name} W={W} rho={rho} T={T}", flush=True)
    L = make_layer(CONFIGS[name].replace(ell_width=W), seed=0, T=T, rho=rho)
    _forward_case(torch, sffn, L)


@pytest.mark.parametrize("policy", ["auto", "union", "sparse"])
def test_forward_edge_all_zero_all_positive(policy):
    torch, sffn = need_gpu()
    base = CONFIGS["C3"].replace(heavy_frac=0.0)
    for label, bias in (("all-zero", -1e4), ("all-positive", 1e4)):
        print(f"[forward-edge] {label} {policy}", flush=True)
        L = make_layer(base, seed=0, T=100)
        from gen import f32_to_bf16_bits, bf16_bits_to_f32
        L["b_up"] = f32_to_bf16_bits(np.full(base.F, bias, np.float32))
        L["b_up_f32"] = bf16_bits_to_f32(L["b_up"])
        _forward_case(torch, sffn, L, check_pattern=(label == "all-zero"), policy=policy)


def test_union_dense_steps_equal_dense_kernel():
    """Where every 64-column step of every 64-token block is contracted densely (20% density:
    unions of more than 48 columns), the union kernel sums the same products in the same
    order as the dense matrix-core kernel: y is identical bit for bit."""
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C3"].replace(heavy_frac=0.0), seed=0, T=520, rho=0.3)
    c = L["cfg"]
    cfg = _cfg(sffn, c.T, c.D, c.F, c.tile, c.ell_width, c.dtype)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    layer.set_down_policy("union")
    y_u, act = layer.forward(x)
    layer.set_down_policy("mfma")
    y_m = layer.down(act)
    torch.cuda.synchronize()
    assert torch.equal(y_u.view(torch.int16), y_m.view(torch.int16))


def test_forward_capacity_overflow_reported():
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C1b"], seed=0)
    c = L["cfg"]
    cfg = _cfg(sffn, c.T, c.D, c.F, c.tile, c.ell_width, c.dtype, cap=1)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    y, act = layer.forward(x)
    assert sffn.check(act) == sffn.SFFN_ERR_BACKUP_OVERFLOW


@pytest.mark.parametrize("T", [1, 32])
def test_forward_small_batch_capacity(T):
    """Decode-shaped batches (the small-batch up-projection, pack and one-launch ordering, the
    split row gather): with a 3x token in the batch, a backup capacity of exactly the rows it
    needs gives the same y and TwELL as a large one, one row fewer and none at all are
    reported as overflow."""
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C3"].replace(heavy_frac=1.0 / T), seed=0, T=T, rho=0.05)
    c = L["cfg"]
    x, Wu, b, Wd = layer_to_dev(torch, L)
    big = _cfg(sffn, T, c.D, c.F, c.tile, c.ell_width, c.dtype, c.n_tiles * T)
    y0, a0 = sffn.SparseFFN(big, Wu, b, Wd).forward(x)
    assert sffn.check(a0) == sffn.SFFN_OK
    h0 = a0.to_host()
    R = int(h0["bk_n"])
    assert R > 0, "the 3x token overflows some tile-rows"
    print(f"[small-capacity] T={T} R={R}", flush=True)
    exact = _cfg(sffn, T, c.D, c.F, c.tile, c.ell_width, c.dtype, R)
    y1, a1 = sffn.SparseFFN(exact, Wu, b, Wd).forward(x)
    assert sffn.check(a1) == sffn.SFFN_OK
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
    h1 = a1.to_host()
    for k in ("counts", "vals", "cols", "bk_tile", "bk_tok", "bk_vals", "bk_tile_ptr"):
        assert np.array_equal(h1[k].view(np.uint8), h0[k].view(np.uint8)), k
    for cap in (R - 1, 0):
        cfg = _cfg(sffn, T, c.D, c.F, c.tile, c.ell_width, c.dtype, cap)
        _, a = sffn.SparseFFN(cfg, Wu, b, Wd).forward(x)
        assert sffn.check(a) == sffn.SFFN_ERR_BACKUP_OVERFLOW, cap


@pytest.mark.parametrize("T", [32, 300])
def test_forward_graph_replay(T):
    """The forward records into a HIP graph (it allocates nothing and records no memset):
    three replays, each after an eager forward of other inputs into the same buffers, give the
    eager result bit for bit (y and the whole TwELL + backup)."""
    torch, sffn = need_gpu()
    print(f"[graph] T={T}", flush=True)
    L = make_layer(CONFIGS["C3"], seed=0, T=T, rho=0.05)
    c = L["cfg"]
    cfg = _cfg(sffn, T, c.D, c.F, c.tile, c.ell_width, c.dtype)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    act = sffn.TwellBuffers(cfg, T)
    y = torch.empty_like(x)
    layer.forward(x, act=act, y=y)
    torch.cuda.synchronize()
    y_ref, h_ref = y.clone(), act.to_host()
    keys = ("counts", "vals", "cols", "bk_tile", "bk_tok", "bk_vals", "bk_tile_ptr")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, act=act, y=y)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, act=act, y=y)
    x_other = torch.flip(x, dims=[0]).contiguous()
    for r in range(3):
        layer.forward(x_other, act=act, y=y)  # eager work on the same buffers in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert sffn.check(act) == sffn.SFFN_OK
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), r
        h = act.to_host()
        for k in keys:
            assert np.array_equal(h[k].view(np.uint8), h_ref[k].view(np.uint8)), (r, k)


def test_determinism_and_homogeneity():
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C3"], seed=0, T=257, rho=0.05)
    c = L["cfg"]
    cfg = _cfg(sffn, c.T, c.D, c.F, c.tile, c.ell_width, c.dtype)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    y1, a1 = layer.forward(x)
    y2, a2 = layer.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    h1, h2 = a1.to_host(), a2.to_host()
    for k in ("counts", "vals", "cols", "bk_tile", "bk_tok", "bk_vals"):
        assert np.array_equal(h1[k], h2[k]), k
    # y(2x, 2b) == 2 y(x, b) bit for bit (scaling by 2 is exact)
    layer2 = sffn.SparseFFN(cfg, Wu, (b.float() * 2).to(torch.bfloat16), Wd)
    y3, _ = layer2.forward((x.float() * 2).to(torch.bfloat16))
    assert torch.equal((y1.float() * 2).to(torch.bfloat16).view(torch.int16), y3.view(torch.int16))
    # token permutation: each token's output is computed the same way wherever it sits
    perm = torch.randperm(c.T, generator=torch.Generator().manual_seed(0)).cuda()
    yp, _ = layer.forward(x[perm].contiguous())
    assert torch.equal(yp.view(torch.int16), y1[perm].view(torch.int16))



def test_forward_buffers_reused_for_fewer_tokens():
    """One set of buffers sized for 300 tokens serves calls of 300, 100, 32, 257 and 1
    tokens in a row (the fused and the small-batch up paths, split and unsplit down
    kernels): each call's y and TwELL equal those of fresh buffers bit for bit, so no kernel
    depends on what an earlier, larger call left in the buffers or the workspace."""
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C3"], seed=0, T=300, rho=0.05)
    c = L["cfg"]
    cfg = _cfg(sffn, 300, c.D, c.F, c.tile, c.ell_width, c.dtype)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    act = sffn.TwellBuffers(cfg, 300)
    keys = ("counts", "vals", "cols", "bk_tile", "bk_tok", "bk_vals", "bk_tile_ptr")
    for T in (300, 100, 32, 257, 1):
        print(f"[reuse] T={T}", flush=True)
        xs = x[:T].contiguous()
        y, a = layer.forward(xs, act=act)
        assert a is act and act.T == T and act.capacity == 300
        y_ref, a_ref = layer.forward(xs)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), T
        h, hr = act.to_host(), a_ref.to_host()
        for k in keys:
            assert np.array_equal(h[k].view(np.uint8), hr[k].view(np.uint8)), (T, k)
        assert h["bk_n"] == hr["bk_n"] and h["status"] == hr["status"] == 0
        assert sffn.twell_stats(cfg, act)["nnz"] == sffn.twell_stats(cfg, a_ref)["nnz"]
        yd = layer.down(act)
        assert torch.equal(yd.view(torch.int16), y_ref.view(torch.int16)), T
    with pytest.raises(ValueError):
        layer.forward(x[:1].repeat(301, 1).contiguous(), act=act)


def _decode_rows(cfg, host, rows):
    """Dense [len(rows), F] of selected tokens of a device TwELL."""
    K, W, nt = cfg.tile, cfg.ell_width, cfg.n_tiles
    out = np.zeros((len(rows), cfg.d_ff), np.float64)
    vals = vals_value(cfg, host["vals"][:, rows, :])
    cols = host["cols"][:, rows, :].astype(np.int64)
    counts = host["counts"][:, rows].astype(np.int64)
    for i in range(len(rows)):
        for k in range(nt):
            m = min(counts[k, i], W)
            out[i, k * K + cols[k, i, :m]] = vals[k, i, :m]
    bt, bo = host["bk_tile"], host["bk_tok"]
    bv = vals_value(cfg, host["bk_vals"])
    pos = {int(t): i for i, t in enumerate(rows)}
    for e in range(len(bt)):
        i = pos.get(int(bo[e]))
        if i is not None:
            nz = np.nonzero(bv[e])[0]
            out[i, int(bt[e]) * K + nz] = bv[e, nz]
    return out


def _plain_bound_report(yh, y_plain, heavy, what):
    """Cost of the storage rounding of the activations (bf16 TwELL values), measured against
    the plain fp64 FFN with unrounded activations: elements beyond the elementwise bound
    1e-2 (1 + |ref|) and their largest ratio to it.  Every element of a row that is not a
    heavy token must still meet the bound against the plain FFN."""
    ratio = np.abs(yh - y_plain) / (1e-2 * (1.0 + np.abs(y_plain)))
    over = ratio > 1.0
    rows_over = np.unique(np.nonzero(over)[0])
    print(f"[plain-ffn] {what}: {int(over.sum())} of {over.size} elements beyond the bound, "
          f"max ratio {ratio.max():.3f}, rows {rows_over.tolist()[:20]}", flush=True)
    light = np.setdiff1d(np.arange(yh.shape[0]), np.asarray(heavy, np.int64))
    assert not over[light].any(), \
        f"{what}: non-heavy rows beyond the bound against the plain FFN: {rows_over.tolist()[:10]}"
    nr = np.linalg.norm(y_plain)
    assert np.linalg.norm(yh - y_plain) / nr <= 5e-3
    return int(over.sum()), float(ratio.max())


@pytest.mark.parametrize("name,rho,policy", [
    ("C2", None, "auto"), ("C3", 0.01, "auto"), ("C3", 0.05, "auto"), ("C3", 0.05, "gather"),
    ("C3", 0.05, "tiles"), ("C3", 0.05, "mfma"), ("C3", 0.05, "union"), ("C3", 0.01, "union"),
    ("C3", 0.002, "union"), ("C3", 0.10, "auto"), ("C3", 0.20, "auto"), ("C3", 0.20, "union"),
    ("C2", None, "union"), ("C4", None, "auto"), ("C4", None, "gather"), ("C4", None, "tiles"),
    ("C4", None, "union"), ("C3", 0.05, "sparse"), ("C3", 0.01, "sparse"), ("C3", 0.002, "sparse"),
    ("C3", 0.20, "sparse"), ("C2", None, "sparse"), ("C4", None, "sparse")])
def test_forward_full_size(name, rho, policy):
    """Full layer sizes, in the launch configuration the benchmark times: every token row
    against the oracle (activations stored in bf16 as the TwELL holds them), every row
    against the plain fp64 FFN (non-heavy rows within the elementwise bound, the whole
    output within the relative-Frobenius bound), the counts of every tile-row, the decoded
    activations of sampled rows, and size-independent invariants on the whole TwELL."""
    torch, sffn = need_gpu()
    print(f"[forward-full] {name} rho={rho} {policy}", flush=True)
    L = make_layer(CONFIGS[name], seed=0, rho=rho)
    c = L["cfg"]
    T = c.T
    cap = max(4096, c.n_tiles * T // 8)
    cfg = _cfg(sffn, T, c.D, c.F, c.tile, c.ell_width, c.dtype, cap)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    layer.set_down_policy(policy)
    y, act = layer.forward(x)
    assert sffn.check(act) == sffn.SFFN_OK
    st = sffn.twell_stats(cfg, act)
    host = act.to_host()
    check_backup_structure(cfg, host, T)
    assert st["nnz"] == int(host["counts"].astype(np.int64).sum())
    yh = y_to_host(torch, y)
    rows = np.arange(T, dtype=np.int64)
    x64, Wu64, b64, Wd64 = (L[k].astype(np.float64) for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
    y_r, c_r, z_r = oracle.ffn_rows(x64, Wu64, b64, Wd64, rows, c.tile, c.ell_width,
                                    return_z=True, round_h=True)
    assert_y_close(yh, y_r, c.dtype, f"full {name} {rho} {policy}")
    y_plain, _ = oracle.ffn_rows(x64, Wu64, b64, Wd64, rows, c.tile, c.ell_width, round_h=False)
    _plain_bound_report(yh, y_plain, L["heavy"], f"{name} {rho} {policy}")
    del y_plain
    # counts of every tile-row may differ only by pre-activations whose fp32 sign is uncertain
    band = fp32_sum_band(x64, Wu64, b64)
    unc = (np.abs(z_r) <= band).reshape(T, c.n_tiles, c.tile).sum(axis=2)
    gpu_c = host["counts"].T.astype(np.int64)
    assert np.all(np.abs(gpu_c - c_r.astype(np.int64)) <= unc)
    # decoded activations of sampled rows (first, last, heavy, random): same pattern where
    # certain, values within bf16 rounding of the fp32 sum
    rng = np.random.default_rng(1)
    heavy = L["heavy"][:8].tolist()
    srows = np.array(sorted(set([0, 1, T - 1, T - 2] + heavy +
                                rng.choice(T, 24, replace=False).tolist())), np.int64)
    hg = _decode_rows(cfg, host, srows)
    zs, bs = z_r[srows], band[srows]
    certain = np.abs(zs) > bs
    assert np.array_equal((hg != 0)[certain], (zs > 0)[certain])
    nzc = certain & (zs > 0)
    assert np.all(np.abs(hg[nzc] - zs[nzc]) <= (np.abs(zs[nzc]) * 2.0 ** -8 + bs[nzc]) * 1.0001)


@pytest.mark.parametrize("F,d,T,n", [(300, 520, 7, 37), (64, 8, 3, 1), (1024, 2048, 5, 0),
                                     (8192, 2048, 33, 430)])
def test_probe_gather_fma(F, d, T, n):
    """The measurement probe computes y[t] = sum_j vals[t, j] W[rows[t, j]] (rows outside
    [0, F) read the first or last row), against an fp64 numpy sum of the same bf16 values."""
    torch, sffn = need_gpu()
    from gen import f32_to_bf16_bits, bf16_bits_to_f32
    print(f"[probe] F={F} d={d} T={T} n={n}", flush=True)
    rng = np.random.default_rng(3)
    W_bits = f32_to_bf16_bits(rng.standard_normal((F, d)).astype(np.float32))
    v_bits = f32_to_bf16_bits(rng.standard_normal((T, n)).astype(np.float32))
    rows = rng.integers(0, F, (T, n)).astype(np.int32)
    if n >= 2:
        rows[0, 0], rows[-1, -1] = -5, F + 3
    W = torch.from_numpy(W_bits.view(np.int16)).view(torch.bfloat16).cuda()
    vals = torch.from_numpy(v_bits.view(np.int16)).view(torch.bfloat16).cuda()
    y = sffn.probe_gather_fma(W, torch.from_numpy(rows).cuda(), vals)
    torch.cuda.synchronize()
    yh = bf16_bits_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    Wf = bf16_bits_to_f32(W_bits).astype(np.float64)
    vf = bf16_bits_to_f32(v_bits).astype(np.float64)
    ref = np.einsum("tj,tjd->td", vf, Wf[np.clip(rows, 0, F - 1)]) if n else np.zeros((T, d))
    assert np.all(np.abs(yh - ref) <= 1e-2 * (1.0 + np.abs(ref)))


@pytest.mark.parametrize("T,F,K,W,dtype,density", [(300, 1024, 128, 16, "bf16", 0.08),
                                                     (8192, 8192, 128, 32, "bf16", 0.05),
                                                     (77, 512, 64, 8, "f32", 0.3),
                                                     (130, 1024, 256, 16, "bf16", 0.03)])
def test_count_histogram_and_width(T, F, K, W, dtype, density):
    """The device count histogram of a packed activation equals the oracle's, bit for bit,
    and the width chosen from it is the oracle's."""
    torch, sffn = need_gpu()
    print(f"[hist] T={T} F={F} K={K} W={W} {dtype} {density}", flush=True)
    h = make_hidden(T, F, density, seed=2, heavy_rows=(0, T - 1), heavy_density=0.6)
    cap = (F // K) * T
    cfg = _cfg(sffn, T, 256, F, K, W, dtype, cap)
    act = sffn.TwellBuffers(cfg, T)
    sffn.twell_pack(cfg, torch.from_numpy(h).cuda(), act)
    hist = sffn.count_histogram(cfg, act)
    tw = oracle.pack(h.astype(np.float64), K, W)
    ref = oracle.count_histogram(tw)
    assert np.array_equal(hist, ref)
    esz = 2 if dtype == "bf16" else 4
    assert sffn.choose_ell_width(cfg, hist) == oracle.choose_ell_width(ref, K, esz)


def test_profile_only_times_named_kernels():
    """With a name list only those launches are timed and counted; without, all are."""
    torch, sffn = need_gpu()
    L = make_layer(CONFIGS["C3"], seed=0, T=300, rho=0.05)
    c = L["cfg"]
    cfg = _cfg(sffn, 300, c.D, c.F, c.tile, c.ell_width, c.dtype)
    x, Wu, b, Wd = layer_to_dev(torch, L)
    layer = sffn.SparseFFN(cfg, Wu, b, Wd)
    # auto at 300 tokens: the gather and matrix-core kernels (one returns); the one-launch
    # ordering of its 640 (tile, group) pairs also writes the per-block counts the choice
    # reads, so block_nnz does not run
    names = ("up_pack", "order", "down", "down_mfma")
    try:
        sffn.profile_reset()
        sffn.profile_enable(True)
        sffn.profile_only(["up_pack", "down_mfma"])
        layer.forward(x)
        got = {n: sffn.profile_read(n) for n in names}
        assert got["up_pack"][1] == 1 and got["down_mfma"][1] == 1, got
        assert got["up_pack"][0] > 0 and got["down_mfma"][0] > 0, got
        assert got["order"][1] == got["down"][1] == 0, got
        sffn.profile_only(None)
        sffn.profile_reset()
        # the first call's count selected the matrix cores: this call launches only them
        layer.forward(x)
        assert all(sffn.profile_read(n)[1] == 1 for n in ("up_pack", "order", "down_mfma"))
        assert sffn.profile_read("down")[1] == 0 and sffn.profile_read("block_nnz")[1] == 0
        # a policy change forgets the recorded choice: every candidate again
        layer.set_down_policy("auto")
        sffn.profile_reset()
        layer.forward(x)
        assert all(sffn.profile_read(n)[1] == 1 for n in names)
    finally:
        sffn.profile_enable(False)
        sffn.profile_only(None)
        sffn.profile_reset()
