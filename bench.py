#!/usr/bin/env python3
"""Benchmark of the MOSS-Image DiT denoising step on one MI355X.

Workload (default): the full 42-block DiT at 1024^2 -- a [1, 32, 128, 128] fp32 latent patched to
4,096 image tokens plus 256 synthetic text tokens (dim 3072), random-init bf16 weights ~N(0, 0.02),
batch 2 per step (the conditional row and the unconditional row, which skips block 22 inside the
skip-layer-guidance window), followed by the FP32 CFG (scale 3) + Euler (shift 5) update. One
timed step = one moss_sample_step call = two DiT forward passes ("each step runs the transformer
twice", MOSS-Image: specs, settings, VRAM and text rendering tested -- "Recommended settings").

Prints ONE JSON line on stdout. Progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--image-steps 50] [--cpu-baseline-blocks 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "DiT forwards/sec at 1024² (4096 img tok, 1 MI355X); s/image 50 steps CFG3"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def block_linear_flops(M, D, F):
    return 2.0 * M * (4 * D * D + 3 * D * F)


def attention_flops(nb, S, D):
    return 4.0 * nb * S * S * D


def class_work(cls, L, D, F, S, N, T, B, skipped, lat_elems, mod_rows, P):
    """Algorithmic work of one profiled class over ONE sampling step: (flops, bytes)."""
    runs = [B] * L
    for l in skipped:
        runs[l] -= 1
    rows = [r * S for r in runs]
    if cls == "gemm_qkv_rope":
        return sum(2.0 * M * 3 * D * D for M in rows), 0
    if cls == "gemm_out_residual":
        return sum(2.0 * M * D * D for M in rows), 0
    if cls == "gemm_gate_up_swiglu":
        return sum(2.0 * M * 2 * F * D for M in rows), 0
    if cls == "gemm_down_residual":
        return sum(2.0 * M * D * F for M in rows), 0
    if cls == "attention":
        return sum(attention_flops(r, S, D) for r in runs), 0
    if cls == "ln_mod":
        return 0, sum(2 * (2.0 * M * D * 2) for M in rows)          # read x, write a; twice per block
    if cls == "modulation":
        return 2.0 * B * mod_rows * 256, mod_rows * 256 * 2.0
    if cls == "embed":
        return 2.0 * B * N * P * D, B * (T * D * 4.0 + T * D * 2 + lat_elems * 4 + N * P * 2 * 2 + N * D * 2)
    if cls == "final_layer":
        return 2.0 * B * N * D * P, B * (N * D * 2 * 2 + N * D * 2 + lat_elems * 4)
    if cls == "cfg_euler":
        return 0, 16.0 * lat_elems
    return 0, 0


def measured_traffic(kernel_class):
    """HBM bytes per launch of `kernel_class` from the committed FETCH_SIZE / WRITE_SIZE passes, or None
    when there is no such record or the kernel sources changed since it was taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "gemm_gate_up_traffic.json")
    try:
        rec = json.load(open(path))
        if rec.get("kernel") != kernel_class:
            return None
        src = b"".join(open(os.path.join(here, f), "rb").read() for f in rec["sources"])
        if hashlib.sha256(src).hexdigest() != rec["sources_sha256"]:
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class ClockSampler:
    """Shader clock of the GPU while it works: a thread reads the current frequency from the amdgpu
    kernel driver's DPM table (sysfs pp_dpm_sclk of the card whose PCI address is torch's device 0; the
    line marked '*') every `period` seconds between start() and stop(). Nothing is read from the GPU
    itself."""

    def __init__(self, period=0.05):
        self.period = period
        self.path = None
        self.error = None
        try:
            import glob
            import torch
            pr = torch.cuda.get_device_properties(0)
            bus = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}"
            for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
                if bus in os.path.realpath(os.path.dirname(f)):
                    self.path = f
                    break
            if self.path is None:
                self.error = f"no pp_dpm_sclk for PCI {bus}"
        except Exception as e:          # the record then says why there is no clock
            self.error = repr(e)
        self.samples = []

    def read(self):
        if not self.path:
            return None
        try:
            for line in open(self.path):
                if "*" in line:
                    return float(line.split(":")[1].strip().lower().split("mhz")[0])
        except Exception as e:
            self.error = repr(e)
        return None

    def start(self):
        import threading
        self.samples = []
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                v = self.read()
                if v is not None:
                    self.samples.append(v)
                self._stop.wait(self.period)
        self._t = threading.Thread(target=run, daemon=True)
        self._t.start()

    def stop(self):
        self._stop.set()
        self._t.join()
        if not self.samples:
            return {"median_mhz": None, "n": 0, "error": self.error}
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "n": len(v)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def _host_f64(t):
    import numpy as np
    import torch
    import oracle as O
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return O.from_bf16_bits(bits)


def run_cpu_baseline(weights, nblocks, S, T, gw):
    """The oracle as it stands, on a bounded sample of the same workload: `nblocks` joint blocks of
    one sample at the 1024^2 sequence length, float64 numpy with the bf16 storage points mirrored."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = O.Config()
    W = {"t_w1": _host_f64(weights["t_w1"]), "t_w2": _host_f64(weights["t_w2"]),
         "final_mod_w": _host_f64(weights["final_mod_w"])}
    for k in ("mod_w", "qkv_w", "out_w", "gate_up_w", "down_w"):
        W[k] = [_host_f64(weights[k][l]) if l < nblocks else None for l in range(cfg.num_layers)]
    rng = np.random.default_rng(0)
    x = O.from_bf16_bits(synth.bf16_normal_bits(rng, (S, cfg.hidden)))
    Wm = dict(W)
    Wm["mod_w"] = [W["mod_w"][l] if l < nblocks else np.zeros((6 * cfg.hidden, 256)) for l in range(cfg.num_layers)]
    t0 = time.perf_counter()
    m, _ = O.modulation(0.5, Wm, cfg, mirror=True)
    for l in range(nblocks):
        x = O.block(x, m[l], W, l, cfg, T, gw, mirror=True)
    el = time.perf_counter() - t0
    per_block = el / nblocks
    fwd_s = cfg.num_layers * per_block
    return {"value": 1.0 / fwd_s, "unit": "DiT forwards/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": (f"{nblocks} of 42 joint blocks (+ the modulation MLP) of one sample at 1024^2 "
                       f"(S = {S}: {T} text + {S - T} image tokens), float64 numpy with bf16 storage points "
                       f"mirrored; {el:.1f} s wall; forwards/s = 1 / (42 x {per_block:.2f} s per block)")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--image-steps", type=int, default=50, help="steps of the full-image timing (0 = skip)")
    ap.add_argument("--cpu-baseline-blocks", type=int, default=3,
                    help="oracle blocks of one sample for cpu_baseline, about 4 s each on 16 threads (0 = skip)")
    ap.add_argument("--profile-steps", type=int, default=3, help="steps of the per-kernel event pass")
    ap.add_argument("--text-len", type=int, default=256)
    ap.add_argument("--latent", type=int, default=128, help="latent side (1024 px / 8)")
    ap.add_argument("--variant-steps", type=int, default=3,
                    help="steps timed for each guidance variant (three-pass SLG, CFG truncation; 0 = skip)")
    ap.add_argument("--steps-2048", type=int, default=2,
                    help="window steps timed at 2048^2 with 4096 text tokens (0 = skip everything at 2048^2)")
    ap.add_argument("--image-steps-2048", type=int, default=50,
                    help="steps of the full-image wall time at 2048^2 (seed 42; 0 = skip)")
    ap.add_argument("--step-cache-threshold", type=float, default=0.02,
                    help="a 50-step image with the step cache at this threshold (0 = skip)")
    ap.add_argument("--refiner-reps", type=int, default=3,
                    help="timed text-refiner calls per prompt length (256 and 4096 tokens; 0 = skip)")
    ap.add_argument("--fp8-steps", type=int, default=5,
                    help="steps timed with the FP8 tier (MXFP8 block projections, a second handle; 0 = skip)")
    ap.add_argument("--library-gemm-reps", type=int, default=10,
                    help="timed vendor calls for reference: torch.matmul (hipBLASLt) and torch._scaled_mm (FP8) "
                         "on the gate/up shape, torch SDPA (flash backend) on the attention shape (0 = skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="MiB of a plain device-to-device copy run once before the steps (scales the "
                         "FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU: the denoising step runs on one MI355X and the library has no multi-GPU "
            "path (CFG-parallel / Ulysses sharding is a design note only). Run it with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch
    import diffusion_transformer_text_amd as dt
    import synth

    torch.cuda.set_device(0)
    L, D, F, H = 42, 3072, 8192, 24
    lat_side, T = args.latent, args.text_len
    gw = lat_side // 2
    N = gw * gw
    S = T + N
    P = 128
    lat_elems = 32 * lat_side * lat_side
    mod_rows = L * 6 * D + 2 * D

    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calibrate_copy} MiB done")
        del src, dst

    t0 = time.time()
    log(f"[bench] drawing random bf16 weights (42 blocks, hidden 3072, FFN 8192) on the GPU")
    weights = synth.torch_weights(synth.FULL, seed=0, device="cuda")
    weights.update(synth.torch_refiner_weights(synth.FULL, seed=100, device="cuda"))
    cfg = dt.moss_dit_config_init()
    model = dt.MossDiT(cfg, weights)
    log(f"[bench] model created in {time.time() - t0:.1f} s")
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    text_cond = torch.randn((1, T, D), generator=g, device="cuda", dtype=torch.float32)
    text_uncond = torch.zeros_like(text_cond)
    x0 = torch.randn((1, 32, lat_side, lat_side), generator=g, device="cuda", dtype=torch.float32)
    sig = dt.moss_sigmas(50, 5.0)
    x = x0.clone()

    def step(k):
        # steps 1..49 lie inside the 0.01..1.0 window: the unconditional row skips block 22
        model.moss_sample_step(x, text_cond, text_uncond, sig, 1 + (k % 49), cfg_scale=3.0,
                               uncond_skip_layers=[22], slg_start=0.01, slg_stop=1.0)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    clock = ClockSampler()
    clocks = {"idle_before_mhz": clock.read()}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clock.start()
    start.record()
    for k in range(args.steps):
        step(k)
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    clocks["timed_steps"] = clock.stop()
    clocks["idle_after_mhz"] = clock.read()
    ms_step = start.elapsed_time(end) / args.steps
    fwd_per_s = 2.0 * 1000.0 / ms_step
    def flops_of_step(block_samples, rows, S_, N_):
        # blocks run per (sample, block) pair; patch embedding + final projection and the modulation
        # GEMV per row
        return block_samples * (block_linear_flops(S_, D, F) + attention_flops(1, S_, D)) + \
            rows * (2.0 * N_ * P * D) * 2 + 2.0 * rows * mod_rows * 256

    step_flops = flops_of_step(2 * L - 1, 2, S, N)
    mfma_frac = step_flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    log(f"[bench] {ms_step:.2f} ms/step, {fwd_per_s:.2f} forwards/s, whole-step MFMA fraction {mfma_frac:.3f}")

    # ---- per-kernel-class event timing (separate pass over the same steps) ----
    model.moss_dit_profile_enable(True)
    for k in range(args.profile_steps):
        step(k)
    prof = model.moss_dit_profile_read()
    model.moss_dit_profile_enable(False)
    kernels = {}
    for cls, (ms, n) in prof.items():
        if n == 0:
            continue
        fl, by = class_work(cls, L, D, F, S, N, T, 2, [22], lat_elems, mod_rows, P)
        ms_s = ms / args.profile_steps
        e = {"ms_per_step": round(ms_s, 4), "launches_per_step": n // args.profile_steps}
        if fl and (cls.startswith("gemm") or cls == "attention"):
            e["tflops"] = round(fl / (ms_s * 1e-3) / 1e12, 1)
            e["frac_mfma_peak"] = round(e["tflops"] / PEAK_BF16_TFLOPS, 4)
        elif by:
            e["gbs"] = round(by / (ms_s * 1e-3) / 1e9, 1)
            e["frac_hbm_peak"] = round(e["gbs"] / PEAK_HBM_GBS, 4)
        kernels[cls] = e
    dom = max(kernels, key=lambda c: kernels[c]["ms_per_step"])
    fl, by = class_work(dom, L, D, F, S, N, T, 2, [22], lat_elems, mod_rows, P)
    launches = kernels[dom]["launches_per_step"]
    if dom.startswith("gemm") or dom == "attention":
        roof = {"bound": "mfma", "achieved": kernels[dom]["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": kernels[dom]["frac_mfma_peak"], "traffic": measured_traffic(dom), "kernel": dom,
                "sclk_mhz_timed_steps": clocks["timed_steps"].get("median_mhz"),
                "peak_note": "published 2.5 PFLOP/s = 2.4 GHz x 1024 flop/clk per SIMD; see sclk for the clock held",
                "flops_per_launch": fl / launches, "avg_launch_ms": kernels[dom]["ms_per_step"] / launches}
    else:
        roof = {"bound": "hbm", "achieved": kernels[dom]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": kernels[dom]["frac_hbm_peak"], "traffic": measured_traffic(dom), "kernel": dom,
                "bytes_per_launch": by / launches, "avg_launch_ms": kernels[dom]["ms_per_step"] / launches}
    log(f"[bench] per-kernel: {json.dumps(kernels)}")

    # ---- the vendor GEMM (torch.matmul -> hipBLASLt) on the gate/up shape, for reference: the same
    # M x N x K bf16 product without the SwiGLU epilogue, both operands contiguous ----
    library_gemm = None
    if args.library_gemm_reps > 0:
        M_gu = 2 * S
        glib = torch.Generator(device="cuda")
        glib.manual_seed(7)
        ga = torch.randn((M_gu, D), generator=glib, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        gb = (0.02 * torch.randn((D, 2 * F), generator=glib, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
        gc = torch.matmul(ga, gb)
        for _ in range(3):
            torch.matmul(ga, gb, out=gc)
        lg0, lg1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        lg0.record()
        for _ in range(args.library_gemm_reps):
            torch.matmul(ga, gb, out=gc)
        lg1.record()
        lg1.synchronize()
        ms_lib = lg0.elapsed_time(lg1) / args.library_gemm_reps
        fl_lib = 2.0 * M_gu * (2 * F) * D
        library_gemm = {"shape": f"{M_gu} x {2 * F} x {D}", "ms": round(ms_lib, 4),
                        "tflops": round(fl_lib / (ms_lib * 1e-3) / 1e12, 1),
                        "frac_mfma_peak": round(fl_lib / (ms_lib * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "ours_gate_up_tflops": kernels.get("gemm_gate_up_swiglu", {}).get("tflops")}
        log(f"[bench] vendor GEMM on the gate/up shape: {json.dumps(library_gemm)}")
        del ga, gb, gc

    # ---- the vendor attention (torch SDPA restricted to its flash backend, which raises rather than
    # fall back to the math path) on the step's attention shape, for reference ----
    library_attention = None
    if args.library_gemm_reps > 0:
        Hh = D // 128
        glib = torch.Generator(device="cuda")
        glib.manual_seed(8)
        qa, ka, va = (torch.randn((2, Hh, S, 128), generator=glib, device="cuda", dtype=torch.float32)
                      .to(torch.bfloat16) for _ in range(3))
        try:
            from torch.nn.attention import SDPBackend, sdpa_kernel
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                for _ in range(3):
                    torch.nn.functional.scaled_dot_product_attention(qa, ka, va)
                la0, la1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                la0.record()
                for _ in range(args.library_gemm_reps):
                    torch.nn.functional.scaled_dot_product_attention(qa, ka, va)
                la1.record()
                la1.synchronize()
            ms_la = la0.elapsed_time(la1) / args.library_gemm_reps
            fl_la = attention_flops(2, S, D)
            library_attention = {"shape": f"B 2, {Hh} heads x 128, S {S}", "backend": "flash", "ms": round(ms_la, 4),
                                 "tflops": round(fl_la / (ms_la * 1e-3) / 1e12, 1),
                                 "frac_mfma_peak": round(fl_la / (ms_la * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                 "ours_attention_tflops": kernels.get("attention", {}).get("tflops")}
        except (RuntimeError, ImportError) as e:
            library_attention = {"backend": "flash", "unavailable": str(e)[:200]}
        log(f"[bench] vendor attention on the step's shape: {json.dumps(library_attention)}")
        del qa, ka, va

    # ---- the vendor FP8 GEMM (torch._scaled_mm -> hipBLASLt, E4M3 with one scale per tensor, bf16 out) on
    # the gate/up shape, for reference next to the FP8 tier's MXFP8 GEMM (block scales, fused epilogue) ----
    library_fp8_gemm = None
    if args.library_gemm_reps > 0:
        M_gu = 2 * S
        glib = torch.Generator(device="cuda")
        glib.manual_seed(9)
        try:
            fa = torch.randn((M_gu, D), generator=glib, device="cuda").to(torch.float8_e4m3fn)
            fb = (0.05 * torch.randn((2 * F, D), generator=glib, device="cuda")).to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda", dtype=torch.float32)
            for _ in range(3):
                torch._scaled_mm(fa, fb.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            lf0, lf1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            lf0.record()
            for _ in range(args.library_gemm_reps):
                torch._scaled_mm(fa, fb.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
            lf1.record()
            lf1.synchronize()
            ms_lf = lf0.elapsed_time(lf1) / args.library_gemm_reps
            fl_lf = 2.0 * M_gu * (2 * F) * D
            library_fp8_gemm = {"shape": f"{M_gu} x {2 * F} x {D}", "format": "E4M3, one scale per tensor",
                                "ms": round(ms_lf, 4), "tflops": round(fl_lf / (ms_lf * 1e-3) / 1e12, 1),
                                "frac_fp8_peak": round(fl_lf / (ms_lf * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
            del fa, fb
        except (RuntimeError, TypeError, AttributeError) as e:
            library_fp8_gemm = {"unavailable": str(e)[:200]}
        log(f"[bench] vendor FP8 GEMM on the gate/up shape: {json.dumps(library_fp8_gemm)}")

    # ---- one full 50-step image (step 0 runs full CFG, steps 1..49 skip block 22 in the negative pass) ----
    s_image = None
    if args.image_steps > 0:
        x.copy_(x0)
        sig_i = dt.moss_sigmas(args.image_steps, 5.0)
        torch.cuda.synchronize()
        clock.start()
        start.record()
        for i in range(args.image_steps):
            model.moss_sample_step(x, text_cond, text_uncond, sig_i, i, cfg_scale=3.0, uncond_skip_layers=[22])
        end.record()
        end.synchronize()
        clocks["image_1024"] = clock.stop()
        s_image = start.elapsed_time(end) / 1000.0
        assert torch.isfinite(x).all().item()
        log(f"[bench] {args.image_steps}-step image: {s_image:.2f} s (DiT + guidance only)")

    def timed(fn, n):
        fn(0)                                     # untimed: grows the workspace for a new shape
        torch.cuda.synchronize()
        start.record()
        for k in range(n):
            fn(k)
        end.record()
        end.synchronize()
        return start.elapsed_time(end) / n

    # ---- the same 50-step image with the step cache (First-Block Cache; lossy, opt-in): at the given
    # threshold, and at an unreachable one (every call after the cache's first full call of a row plan
    # reuses), which times the reused calls themselves ----
    cached = None
    if args.step_cache_threshold > 0 and args.image_steps > 0:
        cached = []
        for thr in (args.step_cache_threshold, 1.0e30):
            x.copy_(x0)
            sig_i = dt.moss_sigmas(args.image_steps, 5.0)
            torch.cuda.synchronize()
            start.record()
            for i in range(args.image_steps):
                model.moss_sample_step(x, text_cond, text_uncond, sig_i, i, cfg_scale=3.0, uncond_skip_layers=[22],
                                       step_cache=True, step_cache_threshold=thr)
            end.record()
            end.synchronize()
            full_c, reused_c, _ = model.moss_step_cache_stats()
            assert torch.isfinite(x).all().item()
            cached.append({"threshold": thr, "s_per_image": round(start.elapsed_time(end) / 1000.0, 3),
                           "full_calls": full_c, "reused_calls": reused_c})
        log(f"[bench] step cache (random N(0, 0.02) weights: the reuse rate says nothing about a trained model's): "
            f"{json.dumps(cached)}")

    # ---- guidance variants at the same size: three-pass skip-layer guidance inside the window (rows
    # cond, uncond skipping 22, cond skipping 22) and a CFG-truncated step (the conditional row only) ----
    variants = None
    if args.variant_steps > 0:
        x.copy_(x0)
        ms3 = timed(lambda k: model.moss_sample_step(x, text_cond, text_uncond, sig, 1 + (k % 49), cfg_scale=3.0,
                                                     uncond_skip_layers=[22], slg_scale=2.5), args.variant_steps)
        ms1 = timed(lambda k: model.moss_sample_step(x, text_cond, text_uncond, sig, 25 + (k % 25), cfg_scale=3.0,
                                                     uncond_skip_layers=[22], cfg_truncation=0.5), args.variant_steps)
        f3, f1 = flops_of_step(3 * L - 2, 3, S, N), flops_of_step(L, 1, S, N)
        variants = {
            "three_pass_slg": {"ms_per_step": round(ms3, 3), "rows": 3, "slg_scale": 2.5,
                               "tflops": round(f3 / (ms3 * 1e-3) / 1e12, 1),
                               "mfma_fraction": round(f3 / (ms3 * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)},
            "cfg_truncated": {"ms_per_step": round(ms1, 3), "rows": 1, "cfg_truncation": 0.5,
                              "tflops": round(f1 / (ms1 * 1e-3) / 1e12, 1),
                              "mfma_fraction": round(f1 / (ms1 * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)},
        }
        log(f"[bench] guidance variants: {json.dumps(variants)}")

    # ---- 2048^2 with a 4096-token prompt (16384 image tokens, S = 20480), seed 42: its own random
    # weights and inputs; one full 50-step image timed as one wall time (step 0 full CFG, steps 1..49
    # with the negative pass skipping block 22), plus the step-0 + 49 x window-step estimate as a
    # cross-check ----
    big = None
    if args.steps_2048 > 0:
        T2, side2, seed2 = 4096, 256, 42
        N2 = (side2 // 2) ** 2
        S2 = T2 + N2
        t0 = time.time()
        w42 = synth.torch_weights(synth.FULL, seed=seed2, device="cuda")
        model42 = dt.MossDiT(cfg, w42)
        del w42
        g42 = torch.Generator(device="cuda")
        g42.manual_seed(seed2)
        tc2 = torch.randn((1, T2, D), generator=g42, device="cuda", dtype=torch.float32)
        tu2 = torch.zeros_like(tc2)
        x2_0 = torch.randn((1, 32, side2, side2), generator=g42, device="cuda", dtype=torch.float32)
        x2 = x2_0.clone()
        sig2 = dt.moss_sigmas(50, 5.0)
        log(f"[bench] 2048^2 model (seed {seed2}) created in {time.time() - t0:.1f} s")
        ms0 = timed(lambda k: model42.moss_sample_step(x2, tc2, tu2, sig2, 0, cfg_scale=3.0,
                                                       uncond_skip_layers=[22]), 1)
        msw = timed(lambda k: model42.moss_sample_step(x2, tc2, tu2, sig2, 1 + k, cfg_scale=3.0,
                                                       uncond_skip_layers=[22]), args.steps_2048)
        s_img2 = None
        if args.image_steps_2048 > 0:
            x2.copy_(x2_0)
            sig_i2 = dt.moss_sigmas(args.image_steps_2048, 5.0)
            torch.cuda.synchronize()
            clock.start()
            start.record()
            for i in range(args.image_steps_2048):
                model42.moss_sample_step(x2, tc2, tu2, sig_i2, i, cfg_scale=3.0, uncond_skip_layers=[22],
                                         slg_start=0.01, slg_stop=1.0)
                if i % 10 == 9:
                    log(f"[bench] 2048^2 image: step {i + 1} of {args.image_steps_2048} enqueued")
            end.record()
            end.synchronize()
            clocks["image_2048"] = clock.stop()
            s_img2 = start.elapsed_time(end) / 1000.0
        assert torch.isfinite(x2).all().item()
        fw = flops_of_step(2 * L - 1, 2, S2, N2)
        fw0 = flops_of_step(2 * L, 2, S2, N2)
        big = {"s_per_image": round(s_img2, 3) if s_img2 else None, "image_steps": args.image_steps_2048,
               "seed": seed2, "method": "wall time of the 50 moss_sample_step calls between two events",
               "s_per_image_estimate": round((ms0 + 49 * msw) / 1000.0, 3),
               "estimate_method": "step 0 (full CFG) + 49 x the mean of the timed window steps",
               "ms_step0": round(ms0, 2), "ms_per_window_step": round(msw, 2), "seq_len": S2, "text_len": T2,
               "image_tokens": N2, "tflops": round(fw / (msw * 1e-3) / 1e12, 1),
               "mfma_fraction": round(fw / (msw * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)}
        if s_img2:
            img_flops = fw0 + (args.image_steps_2048 - 1) * fw
            big["image_mfma_fraction"] = round(img_flops / s_img2 / (PEAK_BF16_TFLOPS * 1e12), 4)
        log(f"[bench] 2048^2: {json.dumps(big)}")
        model42.close()
        del model42, tc2, tu2, x2, x2_0

    # ---- text refiner (projection 4096 -> 3072 + two text-only blocks), once per prompt ----
    refiner = None
    if args.refiner_reps > 0:
        refiner = {}
        E = synth.FULL.text_dim
        for Tr in (256, 4096):
            enc = torch.randn((1, Tr, E), generator=g, device="cuda", dtype=torch.float32)
            outr = torch.empty((1, Tr, D), device="cuda", dtype=torch.float32)
            msr = timed(lambda k: model.moss_text_refine(enc, outr), args.refiner_reps)
            fr = 2.0 * Tr * E * D + synth.FULL.refiner_layers * (block_linear_flops(Tr, D, F) + attention_flops(1, Tr, D))
            refiner[f"prompt_{Tr}"] = {"ms": round(msr, 3), "tflops": round(fr / (msr * 1e-3) / 1e12, 1)}
            del enc, outr
        log(f"[bench] text refiner: {json.dumps(refiner)}")

    # ---- the FP8 tier (lossy, opt-in): second handles on the same weights, with the MXFP8 block
    # projections, then also with 8-bit attention; the same window steps, the per-class split, and one
    # step's drift from the bf16 tier ----
    fp8 = None
    if args.fp8_steps > 0:
        fp8 = {}
        for name, kw in (("mxfp8_gemm", {"gemm_precision": 1}),
                         ("mxfp8_gemm_q8_attention", {"gemm_precision": 1, "attention_mode": 1})):
            t0 = time.time()
            model8 = dt.MossDiT(dt.moss_dit_config_init(**kw), weights)
            log(f"[bench] {name} handle created (weights quantized) in {time.time() - t0:.1f} s")

            def step8(k):
                model8.moss_sample_step(x, text_cond, text_uncond, sig, 1 + (k % 49), cfg_scale=3.0,
                                        uncond_skip_layers=[22], slg_start=0.01, slg_stop=1.0)

            x.copy_(x0)
            ms8 = timed(step8, args.fp8_steps)
            model8.moss_dit_profile_enable(True)
            for k in range(args.profile_steps):
                step8(k)
            prof8 = model8.moss_dit_profile_read()
            model8.moss_dit_profile_enable(False)
            k8 = {}
            for cls, (ms, n) in prof8.items():
                if n == 0 or not (cls.startswith("gemm") or cls == "attention"):
                    continue
                fl, _ = class_work(cls, L, D, F, S, N, T, 2, [22], lat_elems, mod_rows, P)
                ms_s = ms / args.profile_steps
                k8[cls] = {"ms_per_step": round(ms_s, 4), "tflops": round(fl / (ms_s * 1e-3) / 1e12, 1),
                           "frac_fp8_peak": round(fl / (ms_s * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
            # one step from the same state with each tier: the tier's drift on this (random-weight) model
            xa, xb = x0.clone(), x0.clone()
            model.moss_sample_step(xa, text_cond, text_uncond, sig, 1, cfg_scale=3.0, uncond_skip_layers=[22])
            model8.moss_sample_step(xb, text_cond, text_uncond, sig, 1, cfg_scale=3.0, uncond_skip_layers=[22])
            torch.cuda.synchronize()
            dv = ((xb - x0) - (xa - x0)).double().norm() / (xa - x0).double().norm()
            fp8[name] = {"ms_per_step": round(ms8, 3), "forwards_per_s": round(2000.0 / ms8, 3),
                         "speedup_vs_bf16": round(ms_step / ms8, 3), "classes": k8,
                         "step_update_rel_l2_vs_bf16": round(float(dv), 5)}
            log(f"[bench] FP8 tier {name}: {json.dumps(fp8[name])}")
            model8.close()
            del model8
        fp8["format"] = ("OCP MXFP8 GEMMs (E4M3, E8M0 scale per 32 along K; weights quantized at creation, "
                         "activations written as MXFP8 by the kernels that produce them); 8-bit attention: INT8 Q "
                         "(per token) and "
                         "K (per 64-key block), E4M3 P and V (per channel)")

    cpu = None
    if args.cpu_baseline_blocks > 0:
        log(f"[bench] cpu_baseline: oracle on {args.cpu_baseline_blocks} block(s) of one sample")
        cpu = run_cpu_baseline(weights, args.cpu_baseline_blocks, S, T, gw)
        log(f"[bench] cpu_baseline {cpu['value']:.5f} forwards/s ({cpu['cores']} threads)")

    out = {
        "metric": METRIC, "value": round(fwd_per_s, 3), "unit": "DiT forwards/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"MOSS-Image DiT sampling step at {lat_side * 8}^2: 42 blocks, hidden 3072, 24x128 "
                               f"heads, FFN 8192, {N} image + {T} text tokens, batch 2 (cond + uncond skipping block "
                               f"22), CFG 3, Euler shift 5",
                   "global_batch": 2, "seq_len": S, "parallelism": "none (1 GPU)"},
        "s_per_image": round(s_image, 3) if s_image else None,
        "image_steps": args.image_steps,
        "mfma_fraction_step": round(mfma_frac, 4),
        "step_tflop": round(step_flops / 1e12, 2),
        "roofline": roof,
        "kernels": kernels,
        "library_gemm": library_gemm,
        "library_attention": library_attention,
        "library_fp8_gemm": library_fp8_gemm,
        "step_cache": cached,
        "guidance_variants": variants,
        "sampling_2048": big,
        "text_refiner": refiner,
        "fp8_tier": fp8,
        "cpu_baseline": cpu,
        "clocks": clocks,
    }
    print(json.dumps(out), flush=True)
    model.close()


if __name__ == "__main__":
    main()
