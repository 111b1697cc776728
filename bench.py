#!/usr/bin/env python3
"""Benchmark of the BEAM masked-MoE layer forward on one MI355X.

One step is one beam_moe_forward call -- router, top-K and mask, compaction,
grouped SwiGLU gate/up, grouped down, combine -- on a fresh batch x from a
pool of seeded synthetic batches, with the layer's weights taken round-robin
from enough copies that more than 1.5 GB is read between two uses of a copy
(so the 256 MB last-level cache cannot serve them).

Rows: every workload at every batch size it is specified for --
  tiny fp32 layer T=64; DeepSeek-V2-Lite-shaped decode T=1/8/64/256 and
  prefill T=4096; Mixtral-shaped T=1/32/2048; fine-grained T=16/512/8192.
Each row is timed over --windows windows of --steps steps (after --warmup
steps and a pass over every weight copy), each window bracketed by device
synchronisations; the row's time per step is the median window.  `value` is
the headline row, the largest workload (Mixtral-shaped, T=2048), in tokens/s.

Each row reports its algorithmic work (the weights of the experts that got a
pair plus the shared experts, the router weights, x and y; the FLOPs of the
surviving pairs, the shared experts and the router), its fraction of the HBM
and bf16 MFMA peaks, and the binding roofline max(t_HBM, t_MFMA) / t_step.
Per-kernel mean durations come from hipEvent pairs recorded on the call's
stream around every launch in a separate pass; the dominant kernel's
`roofline` object divides its algorithmic bytes (decode) or FLOPs and bytes
(prefill) per launch by that mean.  `traffic` is read from the committed
rocprofv3 counter summary of the same launch configuration, when it was taken
on the current kernel sources.  `peaks` holds the copy-kernel bandwidth and
MFMA-loop rate measured in the same run.  `cpu_baseline` times the oracle on
the host on a bounded sample of the headline workload.

`--only NAME:T` runs a single row (for profilers); `--mask-backward`,
`--segment`, `--gating`, `--zero-mask` alter that row's call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
KERNEL_SOURCES = ("dynamic_expert_masking_amd/csrc/experts.hip",
                  "dynamic_expert_masking_amd/csrc/stream_engine.h",
                  "dynamic_expert_masking_amd/csrc/gemm_engines.h",
                  "dynamic_expert_masking_amd/csrc/prefill_engine.h",
                  "dynamic_expert_masking_amd/csrc/device_common.h")

# (workload, T, shape, target): every batch size of every workload.
ROWS = [("tiny_f32", 64, "parity", None),
        ("dsv2lite_decode", 1, "decode", 0.60), ("dsv2lite_decode", 8, "decode", 0.60),
        ("dsv2lite_decode", 64, "decode", 0.60), ("dsv2lite_decode", 256, "decode", 0.60),
        ("dsv2lite_prefill", 4096, "prefill", 0.50),
        ("mixtral", 1, "decode", 0.60), ("mixtral", 32, "decode", 0.60),
        ("mixtral", 2048, "prefill", 0.50),
        ("finegrained", 16, "decode", 0.60), ("finegrained", 512, "decode", 0.60),
        ("finegrained", 8192, "prefill", 0.50)]
HEADLINE = ("mixtral", 2048)
CONFIG_LABEL = {"tiny_f32": "c1", "dsv2lite_decode": "c2", "dsv2lite_prefill": "c3",
                "mixtral": "c4", "finegrained": "c5", "dsv2lite_decode_fp8": "c2-fp8"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50, help="timed steps per window")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--windows", type=int, default=5, help="timed windows per row (median taken)")
    p.add_argument("--only", default=None, help="one row, NAME:T (e.g. mixtral:2048)")
    p.add_argument("--copies", type=int, default=0, help="weight copies rotated (0 = auto)")
    p.add_argument("--pool", type=int, default=8, help="distinct input batches per row")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the FP8, gate-option and mask-backward rows")
    p.add_argument("--no-peaks", action="store_true", help="skip the copy and MFMA-loop probes")
    p.add_argument("--no-profile", action="store_true", help="skip the per-kernel event pass")
    p.add_argument("--segment", type=int, default=0,
                   help="segment routing: tokens route as their S-token segment's first token")
    p.add_argument("--gating", type=int, default=None, help="gate option bits (default: the config's)")
    p.add_argument("--zero-mask", action="store_true",
                   help="zero mask router (every top-K candidate kept: plain top-K routing)")
    p.add_argument("--mask-backward", action="store_true",
                   help="time the mask-router training step (beam_moe_mask_backward) instead")
    p.add_argument("--pack", choices=("prefill", "all", "none"), default="prefill",
                   help="give the layer packed copies of its expert weights (beam_moe_pack_weights, "
                        "done once at load): for the prefill rows (default), every row, or none")
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


def read_traffic(kernel: str, workload: str):
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (the layer is a "
                                   "single-GPU path); --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_expert_masking_amd as dm
    from dynamic_expert_masking_amd.device import DeviceLayer, to_device
    import synth
    from dataclasses import replace

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

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------------
    # layers (built once per workload, with their weight copies)
    # ------------------------------------------------------------------
    cache = {}

    def layer_for(name, pack=False):
        key = (name, pack)
        if key in cache:
            return cache[key]
        for k in list(cache):   # one workload resident at a time
            del cache[k]
        torch.cuda.empty_cache()
        c = synth.CONFIGS[name]
        if args.segment or args.gating is not None:
            c = replace(c, segment=args.segment, gating=c.gating if args.gating is None else args.gating)
        t0 = time.time()
        host = synth.make_layer(c)
        if args.zero_mask:
            host = replace(host, w_mask=np.zeros_like(host.w_mask), b_mask=None)
        # the workload's Avg-K (K times its keep probability) as the kernel-choice hint
        dl = DeviceLayer(host, dev, pack=pack, avg_k_hint=c.avg_k_target)
        per_copy = sum(v.numel() * v.element_size() for v in dl.t.values() if v is not None)
        copies = args.copies or max(2, min(16, int(np.ceil(1.5e9 / max(1, per_copy))) + 1))
        reps = [(dl.t, dl.desc)] + dl.replicas(copies - 1)
        log(f"{c.name}: layer {per_copy / 1e9:.2f} GB x {copies} copies"
            f"{' (with packed expert weights)' if dl.packed else ''} (setup {time.time() - t0:.1f}s)")
        cache[key] = (c, host, dl, reps, copies)
        return cache[key]

    def gate_up_work(c, active, T):
        """Algorithmic bytes and FLOPs of one gate/up launch: the gate and up
        weights (and FP8 row scales) of the active routed experts and the
        shared ones, read once; 2 products of 2*D flops per intermediate
        element of every surviving pair and every token of the shared ones."""
        if c.expert_format == synth.FP8:
            b = (2 * c.D * c.I + 8 * c.I) * active + (2 * c.D * c.I_s + 8 * c.I_s) * c.S
        else:
            elt = 4 if c.dtype == "f32" else 2
            b = 2 * c.D * c.I * elt * active + 2 * c.D * c.I_s * elt * c.S
        return float(b)

    def run_row(name, T, shape, backward=False, gating=None, profile=True):
        pack = args.pack == "all" or (args.pack == "prefill" and shape == "prefill")
        c, host, dl, reps, copies = layer_for(name, pack)
        descs = [d for _, d in reps]
        if gating is not None:
            for d in descs:
                d.gating = gating
        xs = [to_device(synth.make_x(c, T, f"bench{i}"), dev) for i in range(args.pool)]
        y = torch.empty(T, c.D, dtype=dl.torch_dtype, device=dev)
        ws = dl.workspace(T)
        stats, cand = [], []
        for i in range(args.pool):   # work accounting, outside any timed region
            bufs, out = dl.route_buffers(T)
            dm.beam_moe_route(descs[0], xs[i], T, out, ws, ws.numel(), sh)
            stats.append(dm.beam_moe_stats(descs[0], bufs["expert_count"], T, sh))
            cand.append(int(torch.unique(bufs["topk_idx"]).numel()))
        if backward:
            dys = [to_device(synth.make_x(c, T, f"dy{i}"), dev) for i in range(args.pool)]
            dwm = torch.empty(c.E, c.D, dtype=torch.float32, device=dev)
            dbm = torch.empty(c.E, dtype=torch.float32, device=dev)
            lreg = torch.empty(1, dtype=torch.float32, device=dev)

        def step(i):
            desc = descs[i % len(descs)]
            if backward:
                dm.beam_moe_mask_backward(desc, xs[i % args.pool], dys[i % args.pool], T, 0.1, dwm,
                                          dbm, lreg, ws, ws.numel(), sh)
            else:
                dm.beam_moe_forward(desc, xs[i % args.pool], T, y, None, ws, ws.numel(), sh)

        n_warm = max(args.warmup, len(descs) + 3)   # every weight copy touched first
        for i in range(n_warm):
            step(i)
        torch.cuda.synchronize()
        win_ms = []
        i0 = n_warm
        for _ in range(args.windows):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                step(i0 + i)
            torch.cuda.synchronize()
            win_ms.append((time.perf_counter() - t0) * 1e3 / args.steps)
            i0 += args.steps
        ms = statistics.median(win_ms)
        used = [stats[i % args.pool] for i in range(args.pool)]
        elt = 4 if c.dtype == "f32" else 2
        r = {"workload": name, "config": CONFIG_LABEL.get(name, name), "T": T, "shape": shape,
             "expert_weights": "row-major + packed copy" if dl.packed else "row-major",
             "ms_per_step": round(ms, 5), "window_ms": [round(w, 5) for w in win_ms],
             "tokens_per_s": round(T / (ms / 1e3), 1)}
        bytes_step = float(np.mean([s["bytes_total_min"] for s in used]))
        flops_step = float(np.mean([s["flops_routed"] + s["flops_shared"] + s["flops_router"]
                                    for s in used]))
        if backward:
            ce = float(np.mean(cand))
            bytes_step = 3 * c.D * c.I * elt * ce + 2 * c.E * c.D * elt + 2 * T * c.D * elt
            flops_step = 6.0 * c.D * c.I * T * c.K + 4.0 * c.E * c.D * T
            r["candidate_experts"] = round(ce, 2)
        sec = ms / 1e3
        t_hbm = bytes_step / (HBM_PEAK_GBS * 1e9)
        t_mfma = flops_step / (BF16_PEAK_TFLOPS * 1e12)
        r.update({"avg_k": round(float(np.mean([s["avg_k"] for s in used])), 3),
                  "active_experts": round(float(np.mean([s["active_experts"] for s in used])), 2),
                  "alg_bytes_per_step": bytes_step, "alg_flops_per_step": flops_step,
                  "hbm_gbs": round(bytes_step / sec / 1e9, 1),
                  "frac_hbm_peak": round(t_hbm / sec, 4),
                  "frac_mfma_peak": round(t_mfma / sec, 4),
                  "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                  "frac_binding_roofline": round(max(t_hbm, t_mfma) / sec, 4)})
        if profile and not args.no_profile:
            dm.beam_profile_begin(args.steps * 16)
            torch.cuda.synchronize()
            for i in range(args.steps):
                step(i0 + i)
            torch.cuda.synchronize()
            prof = dm.beam_profile_end(64)
            r["kernels_mean_us"] = {k: round(ms_ * 1e3 / max(n, 1), 2) for k, (n, ms_) in prof.items()}
            gu = [k for k in prof if k.startswith("gate_up")]
            if gu:
                k = gu[0]
                n, tot = prof[k]
                mean_us = tot * 1e3 / max(n, 1)
                act = float(np.mean([s["active_experts"] for s in used])) if not backward \
                    else float(np.mean(cand))
                b = gate_up_work(c, act, T) if not backward else 2 * c.D * c.I * elt * act
                pairs = float(np.mean([s["active_pairs"] for s in used])) if not backward else T * c.K
                f = 4.0 * c.D * (pairs * c.I + T * c.S * c.I_s)
                sec_k = mean_us * 1e-6
                kb, kf = b / (HBM_PEAK_GBS * 1e9), f / (BF16_PEAK_TFLOPS * 1e12)
                wl = f"{name}_T{T}"
                if kb >= kf:
                    roof = {"bound": "hbm", "achieved": round(b / sec_k / 1e9, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(kb / sec_k, 4)}
                else:
                    roof = {"bound": "mfma", "achieved": round(f / sec_k / 1e12, 1),
                            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(kf / sec_k, 4)}
                roof.update({"traffic": read_traffic(k, wl), "kernel": k,
                             "mean_launch_us": round(mean_us, 2), "alg_bytes_per_launch": b,
                             "alg_flops_per_launch": f,
                             "frac_hbm": round(kb / sec_k, 4), "frac_mfma": round(kf / sec_k, 4)})
                r["roofline"] = roof
        if gating is not None:
            for d in descs:
                d.gating = c.gating
        return r

    rows = []
    if args.only:
        name, t = args.only.split(":")
        shape = next((s for n, tt, s, _ in ROWS if n == name and tt == int(t)), "decode")
        rows.append(run_row(name, int(t), shape, backward=args.mask_backward))
        head = rows[0]
    else:
        for name, T, shape, target in ROWS:
            r = run_row(name, T, shape)
            if target is not None:
                key = "frac_hbm_peak" if shape == "decode" else "frac_mfma_peak"
                r["target"] = f">= {int(target * 100)}% of {'HBM' if shape == 'decode' else 'bf16 MFMA'} peak"
                r["target_met"] = bool(r[key] >= target)
            rows.append(r)
            log(f"{name} T={T}: {r['ms_per_step'] * 1e3:.1f} us/step, "
                f"HBM {r['frac_hbm_peak']:.3f}, MFMA {r['frac_mfma_peak']:.3f}")
        head = next(r for r in rows if (r["workload"], r["T"]) == HEADLINE)

    extra = {}
    if not args.only and not args.no_extra:
        # the same DeepSeek-V2-Lite decode batch with each gate option, the
        # mask-router training step, and FP8 expert weights
        g = {}
        for bits in (dm.GATE_SOFTMAX_ALL, dm.GATE_RENORM, dm.GATE_BINARY, dm.GATE_BINARY | dm.GATE_RENORM):
            g[str(bits)] = run_row("dsv2lite_decode", 64, "decode", gating=bits, profile=False)["ms_per_step"]
        extra["gate_options_ms_per_step"] = g
        mb = run_row("dsv2lite_decode", 64, "decode", backward=True)
        extra["mask_backward"] = {
            "what": "beam_moe_mask_backward: L_reg and straight-through dL/dWm, dL/db_m; "
                    "every top-K candidate runs its expert",
            **{k: mb[k] for k in ("T", "ms_per_step", "tokens_per_s", "candidate_experts", "hbm_gbs",
                                  "kernels_mean_us") if k in mb}}
        f8 = [run_row("dsv2lite_decode_fp8", T, "decode") for T in (1, 64, 256)]
        extra["fp8_weights"] = {
            "what": "DeepSeek-V2-Lite-shaped decode layer, expert weights OCP E4M3 with fp32 row scales",
            "rows": f8}

    peaks = None
    if not args.no_peaks and not args.only:
        cache.clear()
        torch.cuda.empty_cache()
        peaks = measure_peaks(dm, torch, sh)

    cpu = None
    if not args.no_cpu:
        cache.clear()
        torch.cuda.empty_cache()
        cpu = cpu_baseline(head["workload"], head["T"], args)

    c = synth.CONFIGS[head["workload"]]
    out = {
        "metric": "masked-MoE layer tokens/s; decode HBM GB/s, prefill MFMA % of peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "windows": args.windows,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; x~N(0,1), weights~N(0,1/D), mask-router bias set per workload)",
        "config": {"workload": f"{c.name}: D={c.D} E={c.E} K={c.K} I={c.I} "
                               f"shared={c.S}x{c.I_s} T={head['T']}"
                               + (f" segment={args.segment}" if args.segment > 1 else "")
                               + (f" gating={args.gating}" if args.gating else "")
                               + (" mask router zero" if args.zero_mask else "")
                               + (" mask-router backward step" if args.mask_backward else ""),
                   "tokens": head["T"], "input_pool": args.pool},
        "roofline": head.get("roofline"),
        "cpu_baseline": cpu,
        "peaks": peaks,
        "rows": rows,
        **extra,
    }
    print(json.dumps(out), flush=True)


def measure_peaks(dm, torch, sh):
    """Copy-kernel bandwidth (2 GiB read + 2 GiB written) and MFMA-loop rate,
    each the best of 5 event-timed launches."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    best = 1e30
    for _ in range(6):
        e0, e1 = ev(), ev()
        e0.record()
        dm.beam_copy_kernel(b, a, n, sh)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    copy_gbs = 2 * n / (best / 1e3) / 1e9
    del a, b
    blocks, iters = 256 * 8, 4096
    o = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    bm = 1e30
    for _ in range(6):
        e0, e1 = ev(), ev()
        e0.record()
        dm.beam_mfma_loop(o, blocks, iters, sh)
        e1.record()
        torch.cuda.synchronize()
        bm = min(bm, e0.elapsed_time(e1))
    flops = blocks * 4.0 * iters * 4 * 2 * 32 * 32 * 16
    return {"copy_gbs": round(copy_gbs, 1), "copy_frac_of_published": round(copy_gbs / HBM_PEAK_GBS, 4),
            "mfma_bf16_tflops": round(flops / (bm / 1e3) / 1e12, 1),
            "mfma_frac_of_published": round(flops / (bm / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "what": "beam_copy_kernel over 2 GiB (bytes read + written); beam_mfma_loop "
                    f"({blocks} workgroups x 4 waves x {iters} rounds of 4 bf16 32x32x16 MFMA chains); "
                    "best of 6"}


def cpu_baseline(name, T, args):
    """The oracle, as it stands, on the host: its forward over a sample of
    tokens of the headline workload's batches, repeated until cpu-seconds
    have passed."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    cfg = synth.CONFIGS[name]
    layer = synth.make_layer(cfg)
    n_tok = min(T, 256)
    done = 0
    batches = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.cpu_seconds:
        x = synth.make_x(cfg, T, f"bench{batches % args.pool}")
        toks = np.arange(n_tok)
        if args.mask_backward:
            dy = oracle.widen(synth.make_x(cfg, T, f"dy{batches % args.pool}"), cfg.dtype)
            oracle.mask_router_backward(layer, x[:n_tok], dy[:n_tok], 0.1)
        else:
            oracle.forward(layer, x, tokens=toks)
        done += n_tok
        batches += 1
    el = time.perf_counter() - t0
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"the first {n_tok} tokens of {batches} batches of {name} T={T} "
                      f"({done} tokens), {'mask-router backward, ' if args.mask_backward else ''}"
                      f"float64 numpy with {threads} BLAS threads, {el:.1f}s"}


if __name__ == "__main__":
    main()
