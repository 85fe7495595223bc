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
KERNELS = ("zero", "up_pack", "order", "block_nnz", "down", "down_tiles", "down_mfma")
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rho", type=float, default=0.05, help="density of the headline point")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the forward+backward timing")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times): the reference "
                         "kernel that scales hardware byte counters to bytes")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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

    def sparse_point(rho, steps, warmup, profile=False, only=None):
        L = bias_for_density(L0, rho)
        b = bf16_dev(L["b_up"])
        layer = sffn.SparseFFN(cfg, Wu, b, Wd)
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
        st = sffn.twell_stats(cfg, act)
        return ms, wall, kt, st, b

    # ---- headline point: the timed region brackets the up kernel and the down kernels (the
    # roofline's candidates) with HIP events on the launch stream; the small kernels' times
    # come from a separate pass that times every launch
    log(f"sparse forward, rho={args.rho}, {args.warmup} warmup + {args.steps} timed steps")
    down_names = ("down", "down_tiles", "down_mfma")
    timed_names = ("up_pack",) + down_names
    ms, wall, kt, st, b0 = sparse_point(args.rho, args.steps, args.warmup, profile=True,
                                        only=timed_names)
    ms_plain, _, _, _, _ = sparse_point(args.rho, args.steps, 2, profile=False)
    _, _, kt_all, _, _ = sparse_point(args.rho, max(10, args.steps // 5), 2, profile=True)
    kt = {**kt_all, **kt}
    log(f"  {ms:.4f} ms/step (profiled), {ms_plain:.4f} ms/step (no events); kernels {kt}")

    # ---- which down-projection kernel took the layer: under the auto policy all candidates
    # are launched and all but one return at once (a few microseconds)
    down_ran = max(down_names, key=lambda k: kt.get(k, 0.0))
    nnz = st["nnz"]

    # ---- dense bf16 FFN baseline (hipBLASLt through torch), same inputs and stream
    def dense():
        h = Fn.relu(Fn.linear(x, Wu, b0))
        return torch.matmul(h, Wd)
    log("dense bf16 FFN baseline")
    ms_dense, _ = time_steps(dense, args.steps, args.warmup)
    log(f"  {ms_dense:.4f} ms/step")

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

    # ---- density sweep
    sweep = []
    if not args.no_sweep:
        for rho in (0.002, 0.005, 0.01, 0.05, 0.10, 0.20):
            m, _, k2, s2, _ = sparse_point(rho, max(10, args.steps // 2), 3, profile=True)
            sweep.append({"rho_target": rho, "density": round(s2["density"], 5),
                          "overflow_tile_rows": int(s2["overflow_tile_rows"]),
                          "ms_per_step": round(m, 4), "tokens_per_s": round(T / (m * 1e-3), 1),
                          "dense_tokens_per_s": round(T / (ms_dense * 1e-3), 1),
                          "speedup_vs_dense": round(ms_dense / m, 4),
                          "kernel_ms": {k: round(v, 4) for k, v in k2.items()}})
            log(f"  sweep rho={rho}: {m:.4f} ms, density {s2['density']:.4f}, {k2}")

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
    dense_flops = 2.0 * T * F * D              # the matrix-core kernel's dense-equivalent work
    sparse_flops = 2.0 * nnz * D               # one MAC per stored nonzero per output column
    rate = lambda fl, ms: fl / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    kernels = {
        "up_pack": {"ms": round(up_ms, 5), "tflops": round(rate(up_flops, up_ms), 2),
                    "frac_mfma_peak": round(rate(up_flops, up_ms) / PEAK_BF16_TFLOPS, 4)},
        "order": {"ms": round(kt["order"], 5)}, "zero": {"ms": round(kt["zero"], 5)},
        "block_nnz": {"ms": round(kt["block_nnz"], 5)},
        "down_launches_ms": {k: round(kt[k], 5) for k in down_names},
    }
    if down_ran == "down_mfma":
        kernels["down"] = {"kernel": "down_mfma", "ms": round(dn_ms, 5),
                           "dense_equiv_tflops": round(rate(dense_flops, dn_ms), 2),
                           "frac_mfma_peak": round(rate(dense_flops, dn_ms) / PEAK_BF16_TFLOPS, 4)}
    else:
        kernels["down"] = {"kernel": down_ran, "ms": round(dn_ms, 5), "nnz": int(nnz),
                           "tflops": round(rate(sparse_flops, dn_ms), 2),
                           "frac_valu_peak": round(rate(sparse_flops, dn_ms) / PEAK_VALU_TFLOPS, 4)}
    if up_ms >= dn_ms:
        roofline = {"bound": "mfma", "achieved": round(rate(up_flops, up_ms), 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(rate(up_flops, up_ms) / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_of("up_pack"),
                    "kernel": "up_pack_bf16_kernel (fused up-projection + bias + ReLU + TwELL pack)",
                    "avg_launch_ms": round(up_ms, 5), "algorithmic_flops_per_launch": up_flops}
    elif down_ran == "down_mfma":
        roofline = {"bound": "mfma", "achieved": round(rate(dense_flops, dn_ms), 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(rate(dense_flops, dn_ms) / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_of("down_mfma"),
                    "kernel": "down_mfma_kernel (TwELL tiles rebuilt in LDS, MFMA down-projection)",
                    "avg_launch_ms": round(dn_ms, 5), "algorithmic_flops_per_launch": dense_flops}
    else:
        kname = {"down": "down_rows_kernel (per-token W_down row gather)",
                 "down_tiles": "down_lds_kernel (W_down tiles in LDS, bf16 dot products)"}[down_ran]
        roofline = {"bound": "alu", "achieved": round(rate(sparse_flops, dn_ms), 2),
                    "peak": PEAK_VALU_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(rate(sparse_flops, dn_ms) / PEAK_VALU_TFLOPS, 4),
                    "traffic": traffic_of(down_ran), "kernel": kname,
                    "avg_launch_ms": round(dn_ms, 5), "algorithmic_flops_per_launch": sparse_flops}

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
            ms_c, _ = time_steps(lambda: layer_c.forward(xc, act=act_c, y=yc), max(10, args.steps // 2), 3)
            ms_cd, _ = time_steps(lambda: torch.matmul(Fn.relu(Fn.linear(xc, Wuc, bc)), Wdc),
                                  max(10, args.steps // 2), 3)
            stc = sffn.twell_stats(cfg_c, act_c)
            layers.append({"layer": cc.name, "T": cc.T, "d_model": cc.D, "d_ff": cc.F,
                           "tile": cc.tile, "ell_width": cc.ell_width,
                           "density": round(stc["density"], 5),
                           "overflow_tile_rows": int(stc["overflow_tile_rows"]),
                           "ms_sparse": round(ms_c, 5), "ms_dense": round(ms_cd, 5),
                           "tokens_per_s": round(cc.T / (ms_c * 1e-3), 1),
                           "speedup_vs_dense": round(ms_cd / ms_c, 4)})
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
            for pol in ("auto", "gather", "mfma"):
                layer_d.set_down_policy(pol)
                ms_d, _ = time_steps(lambda: layer_d.forward(xd, act=act_d, y=yd), 50, 10)
                pt[f"ms_{pol}"] = round(ms_d, 5)
            layer_d.set_down_policy("auto")
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
            decode.append(pt)
            log(f"  decode T={Td}: {pt}")
            del layer_d, act_d

    # ---- CPU fp64 oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        import oracle
        x64 = L0["x_f32"].astype(np.float64)
        Wu64 = L0["W_up_f32"].astype(np.float64)
        b64 = oracle.bf16_value(b0.view(torch.int16).cpu().numpy().view(np.uint16))
        Wd64 = L0["W_down_f32"].astype(np.float64)
        threads = oracle.num_threads()
        n = max(threads, 16)
        rows = np.arange(n, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.ffn_rows(x64, Wu64, b64, Wd64, rows, c.tile, c.ell_width, round_h=True)
        t1 = time.perf_counter() - t0
        n2 = int(min(T, max(n, n * args.cpu_seconds / max(t1, 1e-3))))
        rows = np.linspace(0, T - 1, n2).astype(np.int64)
        log(f"CPU oracle: {n2} tokens on {threads} threads")
        t0 = time.perf_counter()
        oracle.ffn_rows(x64, Wu64, b64, Wd64, rows, c.tile, c.ell_width, round_h=True)
        t2 = time.perf_counter() - t0
        cpu = {"value": round(n2 / t2, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{n2} of {T} tokens of the same layer (per-token fp64 up-projection, "
                         f"ReLU, TwELL-order sparse down-projection), {t2:.1f} s"}

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
                       "speedup_sparse_vs_dense": round(ms_dense / ms, 4)},
        "ms_per_step_without_kernel_events": round(ms_plain, 5),
        "measured": {"density": round(st["density"], 5), "nnz": int(nnz),
                     "overflow_tile_rows": int(st["overflow_tile_rows"]),
                     "ell_fill": round(st["ell_fill"], 4)},
        "kernels": kernels,
        "effective_tflops_dense_equiv": round(4.0 * T * D * F / (ms * 1e-3) / 1e12, 2),
        "train": train,
        "energy": energy,
        "decode": decode,
        "layers": layers,
        "device": {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                   "torch": torch.__version__},
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


if __name__ == "__main__":
    main()
