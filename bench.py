#!/usr/bin/env python3
"""Benchmark of the BEAM masked-MoE layer forward on one MI355X.

Workload (default): the DeepSeek-V2-Lite-shaped decode layer -- D=2048, 64
routed experts, top-6, expert intermediate 1408, 2 shared experts of 1408,
bf16, mask bias for Avg-K ~3 -- at a decode batch of T=64 tokens.  One step
is one beam_moe_forward call (router, top-K/mask, compaction, grouped SwiGLU
gate/up, grouped down, combine) on a fresh batch x from a pool of seeded
synthetic batches, with the layer's weights taken round-robin from enough
copies that more than 1 GB is read between two uses of the same copy (so the
256 MB last-level cache cannot serve them).

Prints one JSON line.  `value` is layer tokens/s = T / (time per step).  The
`roofline` object covers the dominant kernel (grouped gate/up): algorithmic
bytes per launch (the gate and up weights of the experts that received at
least one pair, plus the shared experts' gate and up weights) divided by its
mean launch time from hipEvents recorded around each launch on the call's
stream during a second timed pass.  `cpu_baseline` times the float64 oracle
on the host on a bounded sample of the same workload.  `fp8_weights` reports
the same decode layer with its expert weights stored as OCP FP8 E4M3 codes
with fp32 row scales (same batch size, same timing method); `prefill` the
same layer shapes at T=4096 with its MFMA fraction of the bf16 peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
DOMINANT = "gate_up_swiglu"    # prefix of the dominant kernel's names
KERNEL_SOURCES = ("dynamic_expert_masking_amd/csrc/experts.hip",
                  "dynamic_expert_masking_amd/csrc/stream_engine.h",
                  "dynamic_expert_masking_amd/csrc/gemm_engines.h",
                  "dynamic_expert_masking_amd/csrc/device_common.h")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="dsv2lite_decode")
    p.add_argument("--tokens", type=int, default=None, help="batch size (default: 64 for decode)")
    p.add_argument("--copies", type=int, default=0, help="weight copies rotated (0 = auto)")
    p.add_argument("--pool", type=int, default=16, help="distinct input batches")
    p.add_argument("--no-sweep", action="store_true", help="skip the other batch sizes")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--segment", type=int, default=0,
                   help="segment routing: tokens route as their S-token segment's first token")
    p.add_argument("--gating", type=int, default=None, help="gate option bits (default: the config's)")
    p.add_argument("--zero-mask", action="store_true",
                   help="zero mask router (every top-K candidate kept: plain top-K routing)")
    p.add_argument("--mask-backward", action="store_true",
                   help="time the mask-router training step (beam_moe_mask_backward) instead of the forward")
    p.add_argument("--no-next", action="store_true",
                   help="skip the gate-option and mask-backward timings of the decode layer")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the prefill figure (DeepSeek-V2-Lite-shaped layer, T=4096)")
    p.add_argument("--no-fp8", action="store_true",
                   help="skip the FP8 (E4M3) expert-weight variant of the decode layer")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calibrate-copy", type=int, default=0,
                   help="only run the plain copy kernel on this many MiB (counter calibration)")
    return p.parse_args()


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str = DOMINANT):
    """HBM bytes per launch of a kernel from the committed counter summary,
    or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != kernel_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_expert_masking_amd as dm
    from dynamic_expert_masking_amd.device import DeviceLayer, to_device
    import synth

    dev = "cuda"
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dm.beam_copy_kernel(b, a, n, sh)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 5}))
        return

    cfg = synth.CONFIGS[args.config]
    from dataclasses import replace
    if args.segment or args.gating is not None:
        cfg = replace(cfg, segment=args.segment,
                      gating=cfg.gating if args.gating is None else args.gating)
    T = args.tokens or (64 if args.config.startswith("dsv2lite_decode") else cfg.tokens[-1])

    def setup(c):
        t0 = time.time()
        host = synth.make_layer(c)
        if args.zero_mask:
            host = replace(host, w_mask=np.zeros_like(host.w_mask), b_mask=None)
        dl = DeviceLayer(host, dev)
        per_copy = sum(v.numel() * v.element_size() for k, v in dl.t.items() if v is not None)
        copies = args.copies or max(2, min(16, int(np.ceil(1.5e9 / max(1, per_copy))) + 1))
        reps = [(dl.t, dl.desc)] + dl.replicas(copies - 1)
        print(f"[bench] {c.name}: layer {per_copy / 1e9:.2f} GB x {copies} copies "
              f"(setup {time.time() - t0:.1f}s)", file=sys.stderr, flush=True)
        return host, dl, reps, copies

    def gate_up_bytes(c, active):
        """Algorithmic bytes of one gate/up launch: gate and up weights (and
        FP8 row scales) of the active routed experts and of the shared ones."""
        if c.expert_format == synth.FP8:
            return (2 * c.D * c.I + 8 * c.I) * active + (2 * c.D * c.I_s + 8 * c.I_s) * c.S
        elt = 4 if c.dtype == "f32" else 2
        return 2 * c.D * c.I * elt * active + 2 * c.D * c.I_s * elt * c.S

    def run_T(c, dl, reps, Tb: int, steps: int, warmup: int, profile: bool, backward: bool = False):
        xs = [to_device(synth.make_x(c, Tb, f"bench{i}"), dev) for i in range(args.pool)]
        y = torch.empty(Tb, c.D, dtype=dl.torch_dtype, device=dev)
        ws = dl.workspace(Tb)
        # per-batch work accounting (outside any timed region)
        stats, cand = [], []
        for i in range(args.pool):
            bufs, out = dl.route_buffers(Tb)
            dm.beam_moe_route(dl.desc, xs[i], Tb, out, ws, ws.numel(), sh)
            stats.append(dm.beam_moe_stats(dl.desc, bufs["expert_count"], Tb, sh))
            cand.append(int(torch.unique(bufs["topk_idx"]).numel()))   # experts with a candidate

        if backward:
            # dL/dy of the task loss: a seeded batch of the same shape as y
            dys = [to_device(synth.make_x(c, Tb, f"dy{i}"), dev) for i in range(args.pool)]
            dwm = torch.empty(c.E, c.D, dtype=torch.float32, device=dev)
            dbm = torch.empty(c.E, dtype=torch.float32, device=dev)
            lreg = torch.empty(1, dtype=torch.float32, device=dev)

        def step(i):
            _, desc = reps[i % len(reps)]
            if backward:
                dm.beam_moe_mask_backward(desc, xs[i % args.pool], dys[i % args.pool], Tb, 0.1, dwm,
                                          dbm, lreg, ws, ws.numel(), sh)
            else:
                dm.beam_moe_forward(desc, xs[i % args.pool], Tb, y, None, ws, ws.numel(), sh)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            step(warmup + i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        res = {"T": Tb, "ms_per_step": elapsed * 1e3 / steps}
        used = [stats[(warmup + i) % args.pool] for i in range(steps)]
        res["bytes_per_step"] = float(np.mean([s["bytes_total_min"] for s in used]))
        res["weight_bytes_per_step"] = float(np.mean([s["bytes_active_expert_weights"] for s in used]))
        res["flops_per_step"] = float(np.mean([s["flops_routed"] + s["flops_shared"] + s["flops_router"]
                                               for s in used]))
        res["avg_k"] = float(np.mean([s["avg_k"] for s in used]))
        res["active_experts"] = float(np.mean([s["active_experts"] for s in used]))
        if backward:
            # every top-K candidate runs its expert (the shared experts do not enter)
            elt = 4 if c.dtype == "f32" else 2
            ce = [cand[(warmup + i) % args.pool] for i in range(steps)]
            res["candidate_experts"] = float(np.mean(ce))
            res["bytes_per_step"] = float(np.mean([3 * c.D * c.I * elt * n for n in ce])
                                          + 2 * c.E * c.D * elt + 2 * Tb * c.D * elt)
            res["flops_per_step"] = 6.0 * c.D * c.I * Tb * c.K + 4.0 * c.E * c.D * Tb
        if profile:
            # second timed pass with a hipEvent pair around every launch
            dm.beam_profile_begin(steps * 16)
            torch.cuda.synchronize()
            for i in range(steps):
                step(warmup + i)
            torch.cuda.synchronize()
            prof = dm.beam_profile_end(64)
            res["kernels"] = {k: {"launches": n, "mean_us": ms * 1e3 / max(n, 1)}
                              for k, (n, ms) in prof.items()}
            if backward:
                elt = 4 if c.dtype == "f32" else 2
                res["gate_up_alg_bytes"] = float(np.mean(
                    [2 * c.D * c.I * elt * cand[(warmup + i) % args.pool] for i in range(steps)]))
            else:
                res["gate_up_alg_bytes"] = float(np.mean([gate_up_bytes(c, s["active_experts"])
                                                          for s in used]))
        return res

    host, dl, reps, copies = setup(cfg)
    main_res = run_T(cfg, dl, reps, T, args.steps, args.warmup, profile=True,
                     backward=args.mask_backward)
    ms = main_res["ms_per_step"]
    value = T / (ms / 1e3)

    dom = [k for k in main_res["kernels"] if k.startswith(DOMINANT)]
    roofline = None
    if dom:
        kname = dom[0]
        mean_us = main_res["kernels"][kname]["mean_us"]
        achieved = main_res["gate_up_alg_bytes"] / (mean_us * 1e-6) / 1e9
        workload = f"{cfg.name}_T{T}" + ("_mask_backward" if args.mask_backward else "")
        traffic = read_traffic(workload)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "kernel": kname, "mean_launch_us": round(mean_us, 2),
                    "alg_bytes_per_launch": main_res["gate_up_alg_bytes"]}

    sweep = []
    if not args.no_sweep:
        for Tb in cfg.tokens:
            if Tb == T:
                continue
            r = run_T(cfg, dl, reps, Tb, max(10, args.steps // 2), args.warmup, profile=False)
            sweep.append({"T": Tb, "tokens_per_s": round(Tb / (r["ms_per_step"] / 1e3), 1),
                          "ms_per_step": round(r["ms_per_step"], 4),
                          "layer_hbm_gbs": round(r["bytes_per_step"] / (r["ms_per_step"] / 1e3) / 1e9, 1),
                          "avg_k": round(r["avg_k"], 3)})

    # the gate options and the mask-router training step on the same layer and batch
    nxt = None
    plain = not (args.segment or args.gating is not None or args.zero_mask or args.mask_backward)
    if args.config == "dsv2lite_decode" and plain and not args.no_next:
        nsteps = max(10, args.steps // 2)
        nxt = {"gate_options_ms_per_step": {}}
        for g in (dm.GATE_SOFTMAX_ALL, dm.GATE_RENORM, dm.GATE_BINARY, dm.GATE_BINARY | dm.GATE_RENORM):
            for _, d in reps:
                d.gating = g
            r = run_T(cfg, dl, reps, T, nsteps, args.warmup, profile=False)
            nxt["gate_options_ms_per_step"][str(g)] = round(r["ms_per_step"], 4)
        for _, d in reps:
            d.gating = cfg.gating
        r = run_T(cfg, dl, reps, T, nsteps, args.warmup, profile=True, backward=True)
        sec = r["ms_per_step"] / 1e3
        nxt["mask_backward"] = {
            "what": "beam_moe_mask_backward: L_reg and straight-through dL/dWm, dL/db_m; "
                    "every top-K candidate runs its expert",
            "tokens_per_s": round(T / sec, 1), "ms_per_step": round(r["ms_per_step"], 4),
            "candidate_experts": round(r["candidate_experts"], 2),
            "hbm_gbs": round(r["bytes_per_step"] / sec / 1e9, 1),
            "kernels_mean_us": {k: round(v["mean_us"], 2) for k, v in r["kernels"].items()}}

    # the same decode layer with FP8 (E4M3) expert weights, same batch size
    fp8 = None
    if args.config == "dsv2lite_decode" and not args.no_fp8 and plain:
        del reps
        dl = None
        torch.cuda.empty_cache()
        c8 = synth.CONFIGS["dsv2lite_decode_fp8"]
        _, dl8, reps8, copies8 = setup(c8)
        r = run_T(c8, dl8, reps8, T, args.steps, args.warmup, profile=True)
        k8 = [k for k in r["kernels"] if k.startswith(DOMINANT)]
        fp8 = {"workload": f"{c8.name}: expert weights OCP E4M3 with fp32 row scales, T={T}",
               "tokens_per_s": round(T / (r["ms_per_step"] / 1e3), 1),
               "ms_per_step": round(r["ms_per_step"], 4),
               "speedup_vs_bf16": round(ms / r["ms_per_step"], 3),
               "avg_k": round(r["avg_k"], 3),
               "layer_hbm_gbs": round(r["bytes_per_step"] / (r["ms_per_step"] / 1e3) / 1e9, 1),
               "weight_copies": copies8,
               "kernels_mean_us": {k: round(v["mean_us"], 2) for k, v in r["kernels"].items()}}
        if k8:
            mu = r["kernels"][k8[0]]["mean_us"]
            a8 = r["gate_up_alg_bytes"] / (mu * 1e-6) / 1e9
            fp8["gate_up"] = {"kernel": k8[0], "mean_launch_us": round(mu, 2),
                              "alg_bytes_per_launch": r["gate_up_alg_bytes"],
                              "achieved_gbs": round(a8, 1), "frac": round(a8 / HBM_PEAK_GBS, 4),
                              "traffic": read_traffic(f"{c8.name}_T{T}", f"{DOMINANT}_stream_fp8")}
        del reps8, dl8
        torch.cuda.empty_cache()

    # prefill: the same layer shapes at T=4096 (high sparsity, router-bias skew)
    prefill = None
    if args.config == "dsv2lite_decode" and not args.no_prefill and plain:
        reps = dl = None
        torch.cuda.empty_cache()
        cp = synth.CONFIGS["dsv2lite_prefill"]
        Tp = cp.tokens[-1]
        _, dlp, repsp, _ = setup(cp)
        # warm-up touches every weight copy before the timed steps, as for the
        # decode layer; 30 timed steps, since the first steps after an idle
        # moment run slower (10 steps: 537 us per step, 30 steps: 479 us)
        r = run_T(cp, dlp, repsp, Tp, max(30, args.steps // 2), len(repsp) + 3, profile=False)
        sec = r["ms_per_step"] / 1e3
        prefill = {"workload": f"{cp.name}: D={cp.D} E={cp.E} K={cp.K} I={cp.I} shared={cp.S}x{cp.I_s} "
                               f"T={Tp}, router bias N(0,1)",
                   "tokens_per_s": round(Tp / sec, 1), "ms_per_step": round(r["ms_per_step"], 4),
                   "avg_k": round(r["avg_k"], 3),
                   "mfma_frac_peak": round(r["flops_per_step"] / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                   "hbm_gbs": round(r["bytes_per_step"] / sec / 1e9, 1),
                   "flops_per_step": r["flops_per_step"]}
        del repsp, dlp
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, host, T, args)

    layer_gbs = main_res["bytes_per_step"] / (ms / 1e3) / 1e9
    out = {
        "metric": "masked-MoE layer tokens/s; decode HBM GB/s, prefill MFMA % of peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; x~N(0,1), weights~N(0,1/D))",
        "config": {"workload": f"{cfg.name}: D={cfg.D} E={cfg.E} K={cfg.K} I={cfg.I} "
                               f"shared={cfg.S}x{cfg.I_s} T={T}"
                               + (" expert weights E4M3" if cfg.expert_format == synth.FP8 else "")
                               + (f" segment={cfg.segment}" if cfg.segment > 1 else "")
                               + (f" gating={cfg.gating}" if cfg.gating else "")
                               + (" mask router zero" if args.zero_mask else "")
                               + (" mask-router backward step" if args.mask_backward else ""),
                   "tokens": T, "weight_copies": copies, "input_pool": args.pool},
        "layer": {"avg_k": round(main_res["avg_k"], 3),
                  "active_experts": round(main_res["active_experts"], 2),
                  "alg_bytes_per_step": main_res["bytes_per_step"],
                  "hbm_gbs": round(layer_gbs, 1),
                  "frac_hbm_peak": round(layer_gbs / HBM_PEAK_GBS, 4),
                  "mfma_frac_peak": round(main_res["flops_per_step"] / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 5),
                  "kernels_mean_us": {k: round(v["mean_us"], 2) for k, v in main_res["kernels"].items()}},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "next_rows": nxt,
        "fp8_weights": fp8,
        "prefill": prefill,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, host, T, args):
    """The oracle, as it stands, on the host: whole-layer forward over
    successive batches of the same workload until cpu-seconds have passed."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    done = 0
    t0 = time.perf_counter()
    batches = 0
    while time.perf_counter() - t0 < args.cpu_seconds:
        x = synth.make_x(cfg, T, f"bench{batches % args.pool}")
        if args.mask_backward:
            dy = oracle.widen(synth.make_x(cfg, T, f"dy{batches % args.pool}"), cfg.dtype)
            oracle.mask_router_backward(host, x, dy, 0.1)
        else:
            oracle.forward(host, x)
        done += T
        batches += 1
    el = time.perf_counter() - t0
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{batches} whole batches of T={T} ({done} tokens) of the same workload, "
                      f"{'mask-router backward, ' if args.mask_backward else ''}float64 numpy, {el:.1f}s"}


if __name__ == "__main__":
    main()
