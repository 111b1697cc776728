"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle."""
from __future__ import annotations

import sys
from dataclasses import replace

import numpy as np
import torch

import dynamic_expert_masking_amd as dm
from dynamic_expert_masking_amd.device import DeviceLayer, to_device, to_host_bits

import oracle

# Output tolerances, relative to the largest |y_ref| over the compared tokens.
TOL = {"bf16": 2e-2, "f32": 1e-5}
GATE_TOL = 1e-5

_dev_cache = {}


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_layer(layer, key=None) -> DeviceLayer:
    if key is None:
        return DeviceLayer(layer)
    if key not in _dev_cache:
        _dev_cache.clear()
        torch.cuda.empty_cache()
        _dev_cache[key] = DeviceLayer(layer)
    return _dev_cache[key]


def widen_host(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def run_forward(dl: DeviceLayer, x: np.ndarray, with_route: bool = True, reps: int = 1):
    """Forward through the C ABI; returns (y as float64, routing dict or None, ys of all reps)."""
    T = x.shape[0]
    xd = to_device(x)
    y = torch.empty(T, dl.cfg.D, dtype=dl.torch_dtype, device="cuda")
    ws = dl.workspace(T)
    bufs, out = dl.route_buffers(T) if with_route else (None, None)
    stream = torch.cuda.current_stream().cuda_stream
    ys = []
    for _ in range(reps):
        dm.beam_moe_forward(dl.desc, xd, T, y, out, ws, ws.numel(), stream)
        torch.cuda.synchronize()
        ys.append(to_host_bits(y).copy())
    rt = None
    if with_route:
        rt = {k: v.cpu().numpy() for k, v in bufs.items()}
        rt["mask"] = rt["mask"].view(np.uint32)
    return widen_host(ys[-1], dl.cfg.dtype), rt, ys


def run_route(dl: DeviceLayer, x: np.ndarray):
    T = x.shape[0]
    xd = to_device(x)
    ws = dl.workspace(T)
    bufs, out = dl.route_buffers(T)
    dm.beam_moe_route(dl.desc, xd, T, out, ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rt = {k: v.cpu().numpy() for k, v in bufs.items()}
    rt["mask"] = rt["mask"].view(np.uint32)
    return rt


def check_routing(rt_gpu: dict, rt_ref, E: int, tokens=None) -> None:
    """Indices, mask bits and counts bit-exact; gates within GATE_TOL."""
    idx = rt_gpu["topk_idx"] if tokens is None else rt_gpu["topk_idx"][tokens]
    mask = rt_gpu["mask"] if tokens is None else rt_gpu["mask"][tokens]
    gates = rt_gpu["gates"] if tokens is None else rt_gpu["gates"][tokens]
    bad = np.nonzero((idx != rt_ref.idx).any(axis=1))[0]
    assert bad.size == 0, f"top-K indices differ at tokens {bad[:10]}: {idx[bad[:3]]} vs {rt_ref.idx[bad[:3]]}"
    badm = np.nonzero(mask != rt_ref.mask_bits)[0]
    assert badm.size == 0, f"mask bits differ at tokens {badm[:10]}"
    gerr = np.abs(gates.astype(np.float64) - rt_ref.ghat).max()
    assert gerr <= GATE_TOL, f"gate error {gerr}"
    if tokens is None:
        ref_counts = oracle.expert_counts(rt_ref, E)
        assert np.array_equal(rt_gpu["expert_count"].astype(np.int64), ref_counts), "expert counts differ"


# Every compared output's max|err| / max|y_ref|, by dtype (reported at the end
# of the session by conftest.py).
REL_ERRORS = {"bf16": [], "f32": []}


def check_output(y_gpu: np.ndarray, y_ref: np.ndarray, dtype: str) -> float:
    scale = np.abs(y_ref).max()
    err = np.abs(y_gpu - y_ref).max()
    rel = err / scale if scale > 0 else err
    REL_ERRORS[dtype].append(float(rel))
    assert err <= TOL[dtype] * max(scale, 1e-30) or (scale == 0 and err == 0), \
        f"max|err| {err:.3e} > {TOL[dtype]} * max|y_ref| {scale:.3e}"
    return rel


def sample_tokens(T: int, n: int = 64, seed: int = 5) -> np.ndarray:
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    head = np.arange(8)
    tail = np.arange(T - 8, T)
    mid = rng.choice(np.arange(8, T - 8), size=n - 16, replace=False)
    return np.unique(np.concatenate([head, mid, tail]))


def padded_layer(layer, D: int, I: int, I_s: int = 0):
    """Embed a small layer into larger D / I with zero weights (exactly the
    same layer on the first D inputs / outputs)."""
    c = layer.cfg

    def pad(a, shape):
        out = np.zeros(shape, dtype=a.dtype)
        out[tuple(slice(0, s) for s in a.shape)] = a
        return out

    cfg = replace(c, D=D, I=I, I_s=I_s if c.S else 0)
    return replace(layer, cfg=cfg,
                   w_router=pad(layer.w_router, (c.E, D)), w_mask=pad(layer.w_mask, (c.E, D)),
                   w_gate=pad(layer.w_gate, (c.E, I, D)), w_up=pad(layer.w_up, (c.E, I, D)),
                   w_down=pad(layer.w_down, (c.E, D, I)),
                   ws_gate=None if layer.ws_gate is None else pad(layer.ws_gate, (c.S, I_s, D)),
                   ws_up=None if layer.ws_up is None else pad(layer.ws_up, (c.S, I_s, D)),
                   ws_down=None if layer.ws_down is None else pad(layer.ws_down, (c.S, D, I_s)))
