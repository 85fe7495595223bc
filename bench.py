"""Benchmark: FFN-layer tokens/s of the fused TwELL sparse FFN vs a dense bf16 FFN.

One "step" is one pass of the whole forward hot path over one batch: the fused MFMA
up-projection with its bias + ReLU + TwELL-pack epilogue, the canonical backup
ordering, and the down-projection over the packed activations (per 256-token block the
vector gather kernel or the matrix-core kernel, by the block's stored density), i.e. the
library call sparse_ffn_forward.

Workload: the 1.5B-like ReLU FFN layer, bf16, T = 8192 tokens (16 x 512), d_model 2048,
d_ff 8192, tile 128, ELL width 32, density 5%, 1% of tokens with inputs x3; seeded
synthetic inputs (gen/layers.py), resident in device memory before timing starts.
The other densities of the sweep (1/10/20%) and the dense bf16 FFN (torch -> hipBLASLt)
are reported next to it.  Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import subprocess
import json
import os
import sys
import glob
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FFN-layer tokens/s, fused TwELL vs dense bf16 FFN, at 1-20% density"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_VALU_TFLOPS = 157.3      # MI355X vector: 256 CU x 4 SIMD x 16 lanes x 2 MAC (dot2) x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# launches of one forward, by the names the library's event timing uses
KERNELS = ("up_pack", "up_small", "pack", "order", "block_nnz", "down", "down_tiles", "down_mfma",
           "down_union", "down_sparse")
TRAIN_KERNELS = KERNELS + ("bwd_dh", "bwd_dw_down", "bwd_dw_up", "bwd_dx")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# the sources each kernel with stored traffic counters is built from (its own file and the
# shared header): its counters stay valid while these files are unchanged
KERNEL_SOURCES = {
    "up_pack": ("k_up_pack.hip", "sffn_common.hpp"),
    "down_mfma": ("k_down_mfma.hip", "sffn_common.hpp"),
    "down_tiles": ("k_down_lds.hip", "sffn_common.hpp"),
    "down": ("k_down_rows.hip", "sffn_common.hpp"),
    "down_union": ("k_down_union.hip", "sffn_common.hpp"),
    "down_sparse": ("k_down_sparse.hip", "sffn_common.hpp"),
}


def kernel_source_hash(files=None) -> str:
    """sha256 prefix of the named csrc files (all of them when files is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "activation_sparse_transformer_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def power_sensor():
    """Path of the GPU's board power reading (hwmon power1_input, microwatts), or None."""
    for p in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")):
        try:
            dev_dir = p.split("/hwmon/")[0]
            with open(os.path.join(dev_dir, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
            with open(p) as f:
                int(f.read())
            return p
        except (OSError, ValueError):
            continue
    return None


def average_power(path, run, seconds):
    """Mean board power (W) while `run()` is called repeatedly for about `seconds` (the first
    fifth of the samples, the ramp, is dropped); returns (watts, calls, elapsed_s)."""
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            with open(path) as f:
                samples.append(int(f.read()) * 1e-6)
            time.sleep(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    calls, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            run()
        calls += 20
        run.sync()
    elapsed = time.perf_counter() - t0
    stop.set()
    th.join()
    keep = samples[len(samples) // 5:] or samples
    return (sum(keep) / len(keep) if keep else float("nan")), calls, elapsed


def down_roofline(st, T, D, F, K, esz, ms, kernel):
    """Roofline of a down-projection launch on the method's own work: flops = one
    multiply-add per stored main slot and output column plus the dense [1 x K] x [K x D]
    product of every backup entry (2 slots_used D + 2 K D R); HBM bytes = the TwELL main
    part and backup read once, W_down read once, y written once.  `kernel` is "mfma" (a
    matrix-core kernel: flops against the bf16 MFMA peak) or "alu" (vector kernel: against
    the vector peak).  The binding roofline is the one with the larger floor time."""
    R = int(st["overflow_tile_rows"])
    flops = 2.0 * float(st["slots_used"]) * D + 2.0 * K * D * R
    hbm_bytes = float(st["bytes_main"] + st["bytes_backup"]) + F * D * esz + T * D * esz
    sec = ms * 1e-3
    peak_c = PEAK_BF16_TFLOPS if kernel == "mfma" else PEAK_VALU_TFLOPS
    tflops = flops / sec / 1e12 if sec > 0 else 0.0
    gbs = hbm_bytes / sec / 1e9 if sec > 0 else 0.0
    floor_c = flops / (peak_c * 1e12)
    floor_m = hbm_bytes / (PEAK_HBM_GBS * 1e9)
    out = {"algorithmic_flops": flops, "algorithmic_bytes": hbm_bytes,
           "tflops": round(tflops, 3), f"{kernel}_frac": round(tflops / peak_c, 5),
           "hbm_gbs": round(gbs, 2), "hbm_frac": round(gbs / PEAK_HBM_GBS, 5),
           "dense_equiv_tflops": round(2.0 * T * F * D / sec / 1e12, 2) if sec > 0 else 0.0,
           "floor_us": {kernel: round(floor_c * 1e6, 3), "hbm": round(floor_m * 1e6, 3)}}
    out["bound"] = "hbm" if floor_m >= floor_c else kernel
    return out


def parity_metrics(y, ref):
    """max |y - ref| / (1 + |ref|) and the relative Frobenius error (fp64)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(y - ref)
    nr = float(np.linalg.norm(ref))
    return {"max_rel_elem": float((d / (1.0 + np.abs(ref))).max()) if d.size else 0.0,
            "rel_frobenius": float(np.linalg.norm(y - ref) / nr) if nr > 0 else float(np.linalg.norm(y))}


def spread(ms_list):
    """median, p10 and p90 of per-step times (ms)."""
    a = np.sort(np.asarray(ms_list, np.float64))
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rho", type=float, default=0.05, help="density of the headline point")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--sweep-policies", default="auto",
                    help="comma-separated down policies the density sweep runs, each at every "
                         "density (auto, gather, tiles, mfma, union, sparse)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the per-point oracle checks")
    ap.add_argument("--no-train", action="store_true", help="skip the forward+backward timing")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy / GEMM ceilings")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times): the reference "
                         "kernel that scales hardware byte counters to bytes")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="target seconds of one CPU oracle run (each path is run 3 times)")
    ap.add_argument("--energy-seconds", type=float, default=2.0,
                    help="seconds of repeated forwards per energy measurement (0: skip)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-shaped points")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the 0.5B-like (20%%) and 2B-like (3%%) layer points")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the layer shards by tokens with no exchange, "
              "so a multi-GPU figure is the one-GPU figure times N; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import torch.nn.functional as Fn
    import activation_sparse_transformer_amd as sffn
    from gen import CONFIGS, make_layer, bias_for_density

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    base = CONFIGS["C3"]
    log("generating the 1.5B-like layer")
    L0 = make_layer(base, seed=0, rho=args.rho)
    c = L0["cfg"]
    T, D, F = c.T, c.D, c.F

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def bf16_host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    x = bf16_dev(L0["x"])
    Wu = bf16_dev(L0["W_up"])
    Wd = bf16_dev(L0["W_down"])
    cap = c.n_tiles * T // 8
    cfg = sffn.Config(d_model=D, d_ff=F, tile=c.tile, ell_width=c.ell_width, max_tokens=T,
                      backup_capacity=cap, dtype="bf16")
    act = sffn.TwellBuffers(cfg, T, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def time_steps(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    def per_step(fn, steps, warmup):
        """Per-step times (ms) from events around each step: median, p10, p90."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return spread([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])

    rng_rows = np.random.default_rng(7)

    def sample_rows(Tn, heavy, n):
        """First, last, up to 16 heavy and random token rows (sorted, unique)."""
        r = set([0, Tn - 1]) | set(np.asarray(heavy, np.int64)[:16].tolist())
        r |= set(rng_rows.choice(Tn, min(n, Tn), replace=False).tolist())
        return np.array(sorted(r), np.int64)

    # Per-point parity: the GPU's y of sampled rows is kept here (host copy); the CPU leg at
    # the end runs the oracle on the same rows and fills in each point's "parity" entry.
    pending = []

    def point_parity(target, Lp, yt, rows, K, W):
        if args.no_parity or args.no_cpu:
            target["parity"] = None
            return
        yb = bf16_host(yt[torch.from_numpy(rows).to(dev)]).copy()
        pending.append((target, Lp, yb, rows, K, W))

    down_names = sffn_down_names()
    timed_names = ("up_pack",) + down_names

    def sparse_point(rho, steps, warmup, profile=False, only=None, policy="auto"):
        L = bias_for_density(L0, rho)
        b = bf16_dev(L["b_up"])
        layer = sffn.SparseFFN(cfg, Wu, b, Wd)
        layer.set_down_policy(policy)
        fn = lambda: layer.forward(x, act=act, y=y)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if profile:
            sffn.profile_reset()
            sffn.profile_only(only)
            sffn.profile_enable(True)
        ms, wall = time_steps(fn, steps, 0)
        kt = {}
        if profile:
            sffn.profile_enable(False)
            for k in (only or KERNELS):
                tot, n = sffn.profile_read(k)
                kt[k] = tot / max(n, 1)
            sffn.profile_reset()
            sffn.profile_only(None)
        assert sffn.check(act) == sffn.SFFN_OK, "backup overflow in a timed point"
        st = sffn.twell_stats(cfg, act)
        return ms, wall, kt, st, b, L, layer

    def down_of(kt):
        name = max(down_names, key=lambda k: kt.get(k, 0.0))
        return name, ("alu" if name in ("down", "down_tiles") else "mfma")

    # ---- headline point: the timed region brackets the up kernel and the down kernels (the
    # roofline's candidates) with HIP events on the launch stream; the small kernels' times
    # come from a separate pass that times every launch
    log(f"sparse forward, rho={args.rho}, {args.warmup} warmup + {args.steps} timed steps")
    ms, wall, kt, st, b0, Lh, layer_h = sparse_point(args.rho, args.steps, args.warmup, profile=True,
                                                    only=timed_names)
    ms_plain, _, _, _, _, _, _ = sparse_point(args.rho, args.steps, 2, profile=False)
    _, _, kt_all, _, _, _, _ = sparse_point(args.rho, max(10, args.steps // 5), 2, profile=True)
    kt = {**kt_all, **kt}
    sp_steps = per_step(lambda: layer_h.forward(x, act=act, y=y), max(20, args.steps), 3)
    log(f"  {ms:.4f} ms/step (profiled), {ms_plain:.4f} ms/step (no events), per step {sp_steps}; "
        f"kernels {kt}")
    down_ran, down_kind = down_of(kt)
    nnz = st["nnz"]
    head = {}
    point_parity(head, Lh, y, sample_rows(T, Lh["heavy"], 512), c.tile, c.ell_width)
    # the headline activation's tile-row count histogram and the ELL width with the fewest
    # stored bytes for it (any width, and among the widths the matrix-core kernels take)
    hist = sffn.count_histogram(cfg, act)
    w_any, b_any = sffn.choose_ell_width(cfg, hist)
    w_k, b_k = sffn.choose_ell_width(cfg, hist, [16, 32, 48, 64])
    _, b_cfg = sffn.choose_ell_width(cfg, hist, [c.ell_width])
    cum = np.cumsum(hist) / max(int(hist.sum()), 1)
    width_choice = {"configured_w": c.ell_width, "bytes_at_configured_w": b_cfg,
                    "best_w": w_any, "bytes_at_best_w": b_any,
                    "best_kernel_w": w_k, "bytes_at_best_kernel_w": b_k,
                    "count_quantiles": {q: int(np.searchsorted(cum, q)) for q in (0.5, 0.9, 0.99, 0.999)},
                    "max_count": int(np.nonzero(hist)[0].max()) if hist.any() else 0,
                    "rule": "bytes(W) = rows (2 + W (esz + 1)) + rows_over_W (esz K + 8)"}
    log(f"  ELL width from the count histogram: {width_choice}")

    # ---- dense bf16 FFN baseline (hipBLASLt through torch), same inputs and stream
    def dense():
        h = Fn.relu(Fn.linear(x, Wu, b0))
        return torch.matmul(h, Wd)
    log("dense bf16 FFN baseline")
    ms_dense, _ = time_steps(dense, args.steps, args.warmup)
    dn_steps = per_step(dense, max(20, args.steps), 3)
    log(f"  {ms_dense:.4f} ms/step, per step {dn_steps}")

    # ---- measured ceilings on this GPU: a plain device copy (HBM) and hipBLASLt GEMMs of the
    # layer's two shapes (dense bf16 MFMA)
    ceilings = None
    if not args.no_ceilings:
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        cp_ms, _ = time_steps(lambda: dst.copy_(src), 20, 3)
        h_b = torch.randn((T, F), device=dev).to(torch.bfloat16)
        g_up, _ = time_steps(lambda: torch.matmul(x, Wu.t()), 20, 3)
        g_dn, _ = time_steps(lambda: torch.matmul(h_b, Wd), 20, 3)
        fl = 2.0 * T * D * F
        ceilings = {"copy_gbs": round(2 * nb / (cp_ms * 1e-3) / 1e9, 1),
                    "copy_bytes": 2 * nb,
                    "gemm_up_shape_tflops": round(fl / (g_up * 1e-3) / 1e12, 1),
                    "gemm_down_shape_tflops": round(fl / (g_dn * 1e-3) / 1e12, 1),
                    "gemm_up_ms": round(g_up, 5), "gemm_down_ms": round(g_dn, 5),
                    "shapes": f"[{T},{D}]x[{D},{F}] and [{T},{F}]x[{F},{D}] bf16 (torch.matmul)"}
        del src, dst, h_b
        # the gather-multiply-add of a vector down-projection alone (the library's probe): per
        # token n random rows of this layer's W_down with bf16 weights, n = the stored nonzeros
        # per token at 0.37% (where the vector tile kernel runs) and at the headline density
        rng_p = np.random.default_rng(11)
        gf = []
        for npt in (max(1, int(round(0.0037 * F))), max(1, int(round(nnz / T)))):
            rows_p = torch.from_numpy(rng_p.integers(0, F, (T, npt)).astype(np.int32)).to(dev)
            vals_p = torch.randn((T, npt), device=dev).to(torch.bfloat16)
            y_p = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
            pm, _ = time_steps(lambda: sffn.probe_gather_fma(Wd, rows_p, vals_p, y_p), 20, 3)
            fl_p = 2.0 * T * npt * D
            gf.append({"rows_per_token": npt, "ms": round(pm, 5),
                       "tflops": round(fl_p / (pm * 1e-3) / 1e12, 2),
                       "gathered_gbs": round(T * npt * D * 2 / (pm * 1e-3) / 1e9, 1)})
            del rows_p, vals_p, y_p
        ceilings["gather_fma"] = gf
        ceilings["gather_fma_note"] = ("y[t] = sum_j v[t,j] W_down[r[t,j]] with random rows, fp32 FMA "
                                       "on the vector units, one 16-byte load per lane and row")
        torch.cuda.empty_cache()
        log(f"  ceilings {ceilings}")

    # ---- training step of the same layer (1.5B-like training layer): forward + backward over
    # TwELL, against the dense bf16 FFN forward + its backward matmuls
    train = None
    if not args.no_train:
        g = torch.from_numpy(np.random.default_rng(11).standard_normal((T, D)).astype(np.float32))
        dy = g.to(dev).to(torch.bfloat16)
        layer_t = sffn.SparseFFN(cfg, Wu, b0, Wd)
        bout = layer_t.backward(x, dy, layer_t.forward(x, act=act, y=y)[1])

        def sparse_train():
            layer_t.forward(x, act=act, y=y)
            layer_t.backward(x, dy, act, out=bout)

        def sparse_bwd():
            layer_t.backward(x, dy, act, out=bout)

        def dense_train():
            h = Fn.relu(Fn.linear(x, Wu, b0))
            torch.matmul(h, Wd)
            dWd_d = torch.matmul(h.t(), dy)
            dh = torch.matmul(dy, Wd.t()) * (h > 0)
            dWu_d = torch.matmul(dh.t(), x)
            dh.sum(dim=0)
            torch.matmul(dh, Wu)
            return dWd_d, dWu_d

        log("training step: sparse forward + backward, dense bf16 forward + backward")
        for _ in range(3):
            sparse_train()
        torch.cuda.synchronize()
        sffn.profile_reset()
        sffn.profile_enable(True)
        ms_tr, _ = time_steps(sparse_train, max(10, args.steps // 2), 0)
        sffn.profile_enable(False)
        ktr = {}
        for k in TRAIN_KERNELS:
            tot, n = sffn.profile_read(k)
            ktr[k] = round(tot / max(n, 1), 5)
        sffn.profile_reset()
        ms_bwd, _ = time_steps(sparse_bwd, max(10, args.steps // 2), 3)
        ms_dtr, _ = time_steps(dense_train, max(10, args.steps // 2), 3)
        train = {"workload": "1.5B-like training layer (same shapes and density as the forward), "
                             "dL/dy ~ N(0,1) in bf16; backward = dh at the stored positions, "
                             "dW_down, dW_up, db (fp32) and dx",
                 "ms_forward_backward": round(ms_tr, 5), "ms_backward": round(ms_bwd, 5),
                 "tokens_per_s": round(T / (ms_tr * 1e-3), 1),
                 "dense_ms_forward_backward": round(ms_dtr, 5),
                 "dense_tokens_per_s": round(T / (ms_dtr * 1e-3), 1),
                 "speedup_vs_dense": round(ms_dtr / ms_tr, 4),
                 "kernel_ms": ktr,
                 "saved_activation_bytes": int(st["bytes_main"] + st["bytes_backup"]),
                 "dense_activation_bytes": int(st["bytes_dense_equiv"])}
        log(f"  sparse {ms_tr:.4f} ms (backward {ms_bwd:.4f}), dense {ms_dtr:.4f} ms; {ktr}")
        del bout

    # ---- density sweep: per point the kernel times, the down kernel's roofline on the
    # method's work, and the oracle check of sampled rows
    sweep = []
    if not args.no_sweep:
        for rho, pol in [(r, p) for p in args.sweep_policies.split(",")
                         for r in (0.002, 0.005, 0.01, 0.05, 0.10, 0.20)]:
            m, _, k2, s2, _, Lr, layer_r = sparse_point(rho, max(10, args.steps // 2), 3,
                                                        profile=True, policy=pol)
            dn, kind = down_of(k2)
            pt = {"rho_target": rho, "policy": pol, "density": round(s2["density"], 5),
                  "nnz": int(s2["nnz"]), "slots_used": int(s2["slots_used"]),
                  "overflow_tile_rows": int(s2["overflow_tile_rows"]),
                  "ms_per_step": round(m, 4), "tokens_per_s": round(T / (m * 1e-3), 1),
                  "dense_tokens_per_s": round(T / (ms_dense * 1e-3), 1),
                  "speedup_vs_dense": round(ms_dense / m, 4),
                  "kernel_ms": {k: round(v, 4) for k, v in k2.items()},
                  "down_kernel": dn,
                  "down_roofline": down_roofline(s2, T, D, F, c.tile, 2, k2[dn], kind)}
            point_parity(pt, Lr, y, sample_rows(T, Lr["heavy"], 96), c.tile, c.ell_width)
            sweep.append(pt)
            log(f"  sweep rho={rho} {pol}: {m:.4f} ms, density {s2['density']:.4f}, {k2}")
            del layer_r

    # ---- per-kernel rates and the roofline of the dominant kernel
    src_hash = kernel_source_hash()
    tc = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}

    def traffic_of(name):
        ent = tc.get(name)
        if ent and name in KERNEL_SOURCES and \
                ent.get("source_hash") == kernel_source_hash(KERNEL_SOURCES[name]) and \
                ent.get("workload") == f"C3-{args.rho:.0%}":
            return ent["bytes_per_launch"]
        return None

    up_ms, dn_ms = kt["up_pack"], kt[down_ran]
    up_flops = 2.0 * T * D * F
    rate = lambda fl, ms_: fl / (ms_ * 1e-3) / 1e12 if ms_ > 0 else 0.0
    dn_roof = down_roofline(st, T, D, F, c.tile, 2, dn_ms, down_kind)
    kernels = {
        "up_pack": {"ms": round(up_ms, 5), "tflops": round(rate(up_flops, up_ms), 2),
                    "frac_mfma_peak": round(rate(up_flops, up_ms) / PEAK_BF16_TFLOPS, 4)},
        "order": {"ms": round(kt.get("order", 0.0), 5)},
        "block_nnz": {"ms": round(kt.get("block_nnz", 0.0), 5)},
        "down_launches_ms": {k: round(kt.get(k, 0.0), 5) for k in down_names},
        "down": {"kernel": down_ran, "ms": round(dn_ms, 5), **dn_roof},
    }
    if up_ms >= dn_ms:
        roofline = {"bound": "mfma", "achieved": round(rate(up_flops, up_ms), 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(rate(up_flops, up_ms) / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_of("up_pack"),
                    "kernel": "up_pack_bf16_kernel (fused up-projection + bias + ReLU + TwELL pack)",
                    "avg_launch_ms": round(up_ms, 5), "algorithmic_flops_per_launch": up_flops}
    else:
        kname = {"down": "down_rows_kernel (per-token W_down row gather)",
                 "down_tiles": "down_lds_kernel (W_down tiles in LDS, bf16 dot products)",
                 "down_mfma": "down_mfma_kernel (TwELL tiles rebuilt in LDS, MFMA down-projection)",
                 "down_union": "down_union_kernel (column-union compacted MFMA down-projection)",
                 "down_sparse": "down_sparse_kernel (2:4 structured-sparse MFMA down-projection)"}.get(
            down_ran, down_ran)
        if dn_roof["bound"] == "hbm":
            roofline = {"bound": "hbm", "achieved": dn_roof["hbm_gbs"], "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": dn_roof["hbm_frac"]}
        else:
            pk = PEAK_BF16_TFLOPS if down_kind == "mfma" else PEAK_VALU_TFLOPS
            roofline = {"bound": down_kind, "achieved": dn_roof["tflops"], "peak": pk,
                        "unit": "TFLOP/s", "frac": dn_roof[f"{down_kind}_frac"]}
        roofline.update({"traffic": traffic_of(down_ran), "kernel": kname,
                         "avg_launch_ms": round(dn_ms, 5),
                         "algorithmic_flops_per_launch": dn_roof["algorithmic_flops"],
                         "algorithmic_bytes_per_launch": dn_roof["algorithmic_bytes"],
                         f"{down_kind}_frac": dn_roof[f"{down_kind}_frac"],
                         "hbm_frac": dn_roof["hbm_frac"],
                         "dense_equiv_tflops": dn_roof["dense_equiv_tflops"]})

    # ---- energy per token of the headline forward, sparse and dense (board power sampled
    # every 10 ms while the forward runs back to back)
    energy = None
    sensor = power_sensor() if args.energy_seconds > 0 else None
    if sensor:
        class Runner:
            def __init__(self, f):
                self.f = f

            def __call__(self):
                self.f()

            def sync(self):
                torch.cuda.synchronize()
        layer_e = sffn.SparseFFN(cfg, Wu, b0, Wd)
        run_s = Runner(lambda: layer_e.forward(x, act=act, y=y))
        run_d = Runner(dense)
        time.sleep(0.5)
        with open(sensor) as f:
            idle_w = int(f.read()) * 1e-6
        res = {}
        for name, run in (("sparse", run_s), ("dense_bf16", run_d)):
            for _ in range(10):
                run()
            run.sync()
            w, calls, el = average_power(sensor, run, args.energy_seconds)
            tps = calls * T / el
            res[name] = {"avg_power_w": round(w, 1), "tokens_per_s": round(tps, 1),
                         "joules_per_token": w / tps, "microjoules_per_token": round(w / tps * 1e6, 4)}
            log(f"  energy {name}: {w:.1f} W, {tps:.3e} tokens/s, {w / tps * 1e6:.4f} uJ/token")
        energy = {"sensor": sensor, "idle_power_w": round(idle_w, 1),
                  "seconds_per_point": args.energy_seconds, **res,
                  "sparse_vs_dense_energy_per_token": round(
                      res["sparse"]["joules_per_token"] / res["dense_bf16"]["joules_per_token"], 4)}
        del layer_e

    # ---- the other layer shapes at their own densities: 0.5B-like (T=4096, d_model 1536,
    # d_ff 6144, tile 128, W 48, 20%) and 2B-like (T=16384, d_model 2304, d_ff 9216, tile 256,
    # W 16, 3% with 0.5% heavy tokens); the auto down policy, against the dense bf16 FFN
    layers = []
    if not args.no_layers:
        for name in ("C2", "C4"):
            Lc = make_layer(CONFIGS[name], seed=0)
            cc = Lc["cfg"]
            cfg_c = sffn.Config(d_model=cc.D, d_ff=cc.F, tile=cc.tile, ell_width=cc.ell_width,
                                max_tokens=cc.T, backup_capacity=cc.n_tiles * cc.T // 8,
                                dtype="bf16")
            xc, Wuc, bc, Wdc = (bf16_dev(Lc[k]) for k in ("x", "W_up", "b_up", "W_down"))
            layer_c = sffn.SparseFFN(cfg_c, Wuc, bc, Wdc)
            act_c = sffn.TwellBuffers(cfg_c, cc.T)
            yc = torch.empty_like(xc)
            for _ in range(3):  # warm-ups outside the per-launch timing (a first launch of a
                layer_c.forward(xc, act=act_c, y=yc)  # kernel variant sets up its resources)
            torch.cuda.synchronize()
            sffn.profile_reset()
            sffn.profile_enable(True)
            ms_c, _ = time_steps(lambda: layer_c.forward(xc, act=act_c, y=yc), max(10, args.steps // 2), 0)
            sffn.profile_enable(False)
            kc = {k: sffn.profile_read(k)[0] / max(sffn.profile_read(k)[1], 1) for k in KERNELS}
            sffn.profile_reset()
            ms_cd, _ = time_steps(lambda: torch.matmul(Fn.relu(Fn.linear(xc, Wuc, bc)), Wdc),
                                  max(10, args.steps // 2), 3)
            assert sffn.check(act_c) == sffn.SFFN_OK
            gemm_c = None
            if not args.no_ceilings:
                h_c = torch.randn((cc.T, cc.F), device=dev).to(torch.bfloat16)
                g_u, _ = time_steps(lambda: torch.matmul(xc, Wuc.t()), 10, 2)
                g_d, _ = time_steps(lambda: torch.matmul(h_c, Wdc), 10, 2)
                fl_c = 2.0 * cc.T * cc.D * cc.F
                gemm_c = {"up_shape_tflops": round(fl_c / (g_u * 1e-3) / 1e12, 1),
                          "down_shape_tflops": round(fl_c / (g_d * 1e-3) / 1e12, 1),
                          "up_ms": round(g_u, 5), "down_ms": round(g_d, 5)}
                del h_c
            stc = sffn.twell_stats(cfg_c, act_c)
            dn_c, kind_c = down_of(kc)
            lp = {"layer": cc.name, "T": cc.T, "d_model": cc.D, "d_ff": cc.F,
                  "tile": cc.tile, "ell_width": cc.ell_width,
                  "density": round(stc["density"], 5),
                  "overflow_tile_rows": int(stc["overflow_tile_rows"]),
                  "ms_sparse": round(ms_c, 5), "ms_dense": round(ms_cd, 5),
                  "tokens_per_s": round(cc.T / (ms_c * 1e-3), 1),
                  "speedup_vs_dense": round(ms_cd / ms_c, 4),
                  "kernel_ms": {k: round(v, 4) for k, v in kc.items()},
                  "down_kernel": dn_c,
                  "gemm_ceiling": gemm_c,
                  "down_roofline": down_roofline(stc, cc.T, cc.D, cc.F, cc.tile, 2, kc[dn_c], kind_c)}
            point_parity(lp, Lc, yc, sample_rows(cc.T, Lc["heavy"], 96), cc.tile, cc.ell_width)
            layers.append(lp)
            log(f"  layer {cc.name}: sparse {ms_c:.4f} ms, dense {ms_cd:.4f} ms, "
                f"density {stc['density']:.4f}")
            del layer_c, act_c, xc, Wuc, bc, Wdc, yc
            torch.cuda.empty_cache()

    # ---- decode-shaped points: few tokens, the layer reads all of W_up but only the W_down
    # rows the stored nonzeros select; sparse (auto policy and each down kernel) vs dense
    decode = []
    if not args.no_decode:
        for Td in (1, 8, 32, 64, 128, 256):
            cfg_d = sffn.Config(d_model=D, d_ff=F, tile=c.tile, ell_width=c.ell_width,
                                max_tokens=Td, backup_capacity=max(64, c.n_tiles * Td // 8),
                                dtype="bf16")
            act_d = sffn.TwellBuffers(cfg_d, Td, device=dev)
            xd = x[:Td].contiguous()
            yd = torch.empty_like(xd)
            layer_d = sffn.SparseFFN(cfg_d, Wu, b0, Wd)
            pt = {"T": Td}
            for pol in decode_policies():
                layer_d.set_down_policy(pol)
                ms_d, _ = time_steps(lambda: layer_d.forward(xd, act=act_d, y=yd), 50, 10)
                assert sffn.check(act_d) == sffn.SFFN_OK
                pt[f"ms_{pol}"] = round(ms_d, 5)
            layer_d.set_down_policy("auto")
            layer_d.forward(xd, act=act_d, y=yd)
            assert sffn.check(act_d) == sffn.SFFN_OK
            ms_dd, _ = time_steps(lambda: torch.matmul(Fn.relu(Fn.linear(xd, Wu, b0)), Wd), 50, 10)
            hs = act_d.to_host()
            used = np.zeros(F, bool)
            K = c.tile
            for k in range(c.n_tiles):
                m = np.minimum(hs["counts"][k].astype(np.int64), c.ell_width)
                for t in range(Td):
                    used[k * K + hs["cols"][k, t, :m[t]].astype(np.int64)] = True
            for e in range(len(hs["bk_tile"])):
                used[int(hs["bk_tile"][e]) * K + np.nonzero(hs["bk_vals"][e])[0]] = True
            rows = int(used.sum())
            sp_bytes = F * D * 2 + F * 2 + rows * D * 2 + 2 * Td * D * 2
            dn_bytes = 2 * F * D * 2 + F * 2 + 2 * Td * D * 2
            pt.update({"ms_dense": round(ms_dd, 5), "speedup_vs_dense": round(ms_dd / pt["ms_auto"], 4),
                       "tokens_per_s": round(Td / (pt["ms_auto"] * 1e-3), 1),
                       "w_down_rows_used": rows, "w_down_rows": F,
                       "weight_bytes_sparse": sp_bytes, "weight_bytes_dense": dn_bytes,
                       "hbm_gbs_sparse": round(sp_bytes / (pt["ms_auto"] * 1e-3) / 1e9, 1),
                       "hbm_gbs_dense": round(dn_bytes / (ms_dd * 1e-3) / 1e9, 1)})
            Ld = {k: (v[:Td] if k in ("x", "x_f32") else v) for k, v in Lh.items()}
            point_parity(pt, Ld, yd, np.arange(Td, dtype=np.int64), c.tile, c.ell_width)
            decode.append(pt)
            log(f"  decode T={Td}: {pt}")
            del layer_d, act_d

    # ---- the tiny fp32 layer (T=64, d_model 256, d_ff 1024, tile 128, W 32, 10%) is launch-bound,
    # so it is reported as latency: each forward timed on its own (events around it), median and
    # spread of 200 calls, against the dense fp32 FFN; the oracle's time for the same 64 tokens
    latency_tiny, tiny_case = None, None
    if not args.no_layers:
        Lt = make_layer(CONFIGS["C1"], seed=0)
        ct = Lt["cfg"]
        f32d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        xt, Wut, bt, Wdt = (f32d(Lt[k]) for k in ("x", "W_up", "b_up", "W_down"))
        cfg_t = sffn.Config(d_model=ct.D, d_ff=ct.F, tile=ct.tile, ell_width=ct.ell_width,
                            max_tokens=ct.T, backup_capacity=ct.n_tiles * ct.T, dtype="f32")
        layer_t = sffn.SparseFFN(cfg_t, Wut, bt, Wdt)
        act_t = sffn.TwellBuffers(cfg_t, ct.T)
        yt = torch.empty_like(xt)
        lt = per_step(lambda: layer_t.forward(xt, act=act_t, y=yt), 200, 10)
        ld = per_step(lambda: torch.matmul(Fn.relu(Fn.linear(xt, Wut, bt)), Wdt), 200, 10)
        assert sffn.check(act_t) == sffn.SFFN_OK
        stt = sffn.twell_stats(cfg_t, act_t)
        us = lambda d_: {k: (round(v * 1e3, 2) if k != "n" else v) for k, v in d_.items()}
        latency_tiny = {"layer": ct.name, "T": ct.T, "d_model": ct.D, "d_ff": ct.F,
                        "tile": ct.tile, "ell_width": ct.ell_width, "dtype": "f32",
                        "density": round(stt["density"], 5), "sparse_us": us(lt),
                        "dense_fp32_us": us(ld),
                        "speedup_vs_dense_median": round(ld["median"] / lt["median"], 4)}
        torch.cuda.synchronize()
        tiny_case = (latency_tiny, Lt, yt.cpu().numpy().astype(np.float64))
        log(f"  tiny fp32 layer latency: sparse {latency_tiny['sparse_us']} us, "
            f"dense {latency_tiny['dense_fp32_us']} us")
        del layer_t, act_t

    # ---- CPU fp64 oracle on bounded samples of the same workload, the sparse path (up-projection,
    # ReLU, TwELL pack, sparse down-projection, per token) and the dense FFN; median of 3 runs each
    cpu = None
    if not args.no_cpu:
        import oracle as orc  # the CPU fp64 oracle: this leg only
        for target, Lp, yb, rows, K, W in pending:
            x64, Wu64, b64, Wd64 = (Lp[k].astype(np.float64)
                                    for k in ("x_f32", "W_up_f32", "b_up_f32", "W_down_f32"))
            y_st, _ = orc.ffn_rows(x64, Wu64, b64, Wd64, rows, K, W, round_h=True)
            y_pl, _ = orc.ffn_rows(x64, Wu64, b64, Wd64, rows, K, W, round_h=False)
            yh = orc.bf16_value(yb)
            a = parity_metrics(yh, y_st)
            target["parity"] = {"rows": int(len(rows)), "vs_oracle_bf16_activations": a,
                                "vs_plain_fp64_ffn": parity_metrics(yh, y_pl),
                                "within_tolerance": bool(a["max_rel_elem"] <= 1e-2 and
                                                         a["rel_frobenius"] <= 5e-3)}
        log(f"parity of {len(pending)} points checked against the oracle; headline {head.get('parity')}")
        if tiny_case is not None:
            lat, Lt, yt_h = tiny_case
            xt64, Wut64, bt64, Wdt64 = (Lt[k].astype(np.float64) for k in ("x", "W_up", "b_up", "W_down"))
            rows_t = np.arange(lat["T"], dtype=np.int64)
            tt = []
            for _ in range(20):
                t0 = time.perf_counter()
                y_t, _ = orc.ffn_rows(xt64, Wut64, bt64, Wdt64, rows_t, lat["tile"], lat["ell_width"])
                tt.append(time.perf_counter() - t0)
            a = parity_metrics(yt_h, y_t)
            lat["parity"] = {"rows": int(lat["T"]), "vs_oracle": a,
                             "within_tolerance": bool(a["max_rel_elem"] <= 1e-4 and
                                                      a["rel_frobenius"] <= 1e-5)}
            lat["cpu_oracle_us"] = {"median": round(float(np.median(tt)) * 1e6, 1), "runs": 20,
                                    "threads": orc.num_threads()}
        x64 = Lh["x_f32"].astype(np.float64)
        Wu64 = Lh["W_up_f32"].astype(np.float64)
        b64 = Lh["b_up_f32"].astype(np.float64)
        Wd64 = Lh["W_down_f32"].astype(np.float64)
        threads = orc.num_threads()
        n = max(threads, 16)
        t0 = time.perf_counter()
        orc.ffn_rows(x64, Wu64, b64, Wd64, np.arange(n, dtype=np.int64), c.tile, c.ell_width, round_h=True)
        t1 = time.perf_counter() - t0
        n2 = int(min(T, max(n, n * args.cpu_seconds / max(t1, 1e-3))))
        rows = np.linspace(0, T - 1, n2).astype(np.int64)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            orc.ffn_rows(x64, Wu64, b64, Wd64, rows, c.tile, c.ell_width, round_h=True)
            ts.append(time.perf_counter() - t0)
        t_sp = float(np.median(ts))
        nd = max(threads, n2 // 2)
        rows_d = np.linspace(0, T - 1, nd).astype(np.int64)
        td = []
        for _ in range(3):
            t0 = time.perf_counter()
            orc.ffn_dense(x64[rows_d], Wu64, b64, Wd64)
            td.append(time.perf_counter() - t0)
        t_dn = float(np.median(td))
        log(f"CPU oracle: sparse path {n2} tokens {t_sp:.2f} s, dense FFN {nd} tokens {t_dn:.2f} s, "
            f"{threads} threads")
        cpu = {"value": round(n2 / t_sp, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n2} of {T} tokens of the same layer through the oracle's sparse path "
                         f"(per-token fp64 up-projection, ReLU, TwELL pack, sparse down-projection), "
                         f"median of 3 runs ({', '.join(f'{v:.2f}' for v in ts)} s)",
               "dense_ffn_tokens_per_s": round(nd / t_dn, 2),
               "dense_sample": f"{nd} tokens through the oracle's dense FFN, median of 3 runs "
                               f"({', '.join(f'{v:.2f}' for v in td)} s)",
               "label": f"CPU fp64 oracle, {threads} threads - reference baseline, not the target"}

    tok_s = T / (ms * 1e-3)
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random N(0,1/fan_in) weights, bias-tuned density)",
        "config": {"workload": "1.5B-like ReLU FFN layer forward: T=8192 (16x512), d_model=2048, "
                               f"d_ff=8192, tile=128, ELL width=32, density {args.rho:.0%}, "
                               "1% heavy tokens (inputs x3)",
                   "global_batch": T, "seq_len": 512, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_bf16": {"ms_per_step": round(ms_dense, 5), "tokens_per_s": round(T / (ms_dense * 1e-3), 1),
                       "speedup_sparse_vs_dense": round(ms_dense / ms, 4), "per_step_ms": dn_steps},
        "per_step_ms": sp_steps,
        "ms_per_step_without_kernel_events": round(ms_plain, 5),
        "parity": head.get("parity"),
        "measured": {"density": round(st["density"], 5), "nnz": int(nnz),
                     "slots_used": int(st["slots_used"]),
                     "overflow_tile_rows": int(st["overflow_tile_rows"]),
                     "ell_fill": round(st["ell_fill"], 4)},
        "kernels": kernels,
        "ceilings": ceilings,
        "ell_width_choice": width_choice,
        "effective_tflops_dense_equiv": round(4.0 * T * D * F / (ms * 1e-3) / 1e12, 2),
        "train": train,
        "energy": energy,
        "decode": decode,
        "layers": layers,
        "device": {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                   "torch": torch.__version__, **machine_info()},
        "latency_tiny": latency_tiny,
        "sweep": sweep,
        "kernel_source_hash": src_hash,
    }
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n
    print(json.dumps(out), flush=True)


def machine_info():
    """Host CPU model and thread counts, and the GPU's current clocks as amd-smi reports them
    (best effort: absent tools or fields give None)."""
    info = {"cpu_model": None, "host_threads_affinity": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "gpu_clocks": None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "-g", "0"], capture_output=True, text=True,
                           timeout=20)
        if r.returncode == 0:
            info["gpu_clocks"] = " ".join(r.stdout.split())[:600]
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def sffn_down_names():
    """Event names of the library's down-projection launches."""
    return ("down", "down_tiles", "down_mfma", "down_union", "down_sparse")


def decode_policies():
    return ("auto", "gather", "mfma")


if __name__ == "__main__":
    main()
