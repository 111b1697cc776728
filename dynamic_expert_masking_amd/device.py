"""Device-memory plumbing for the binding: uploads host parameter arrays to
torch device tensors, fills the layer descriptor and sizes workspaces.

Host arrays follow one convention: bf16 values are uint16 bit patterns,
fp32 values are float32.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (BEAM_BF16, BEAM_F32, WEIGHTS_DTYPE, WEIGHTS_FP8_E4M3, beam_moe_pack_weights,
               beam_moe_workspace_size, make_layer, make_route_out)

SCALES = ("s_gate", "s_up", "s_down", "ss_gate", "ss_up", "ss_down")
PACKED = ("wp_gate", "wp_up", "wp_down", "wsp_gate", "wsp_up", "wsp_down")


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a host array: uint16 -> torch.bfloat16 (same bits), float32 ->
    float32, uint8 (E4M3 codes) -> torch.uint8."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(device)
    raise TypeError(f"unsupported host dtype {a.dtype}")


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Download: bfloat16 -> uint16 bit patterns, float32 -> float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceLayer:
    """Device copy of a layer's parameters plus its C descriptor.

    `host` is any object with the attributes of the parameter set: cfg (with
    D, E, K, I, S, I_s, dtype and optionally gating, expert_format, segment), w_router,
    w_mask, b_router, b_mask, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
    and for FP8 expert weights the row scales s_gate, s_up, s_down, ss_gate,
    ss_up, ss_down.  pack=True adds packed copies of bf16 expert weights
    (beam_moe_pack_weights); avg_k_hint fills the descriptor's
    expected_avg_k (0: unknown).
    """

    def __init__(self, host, device="cuda", pack=False, avg_k_hint=0.0):
        c = host.cfg
        self.cfg = c
        self.device = device
        self.avg_k_hint = float(avg_k_hint)   # expected_avg_k of the descriptor (0: unknown)
        up = lambda a: None if a is None else to_device(a, device)  # noqa: E731
        self.t = {name: up(getattr(host, name)) for name in
                  ("w_router", "w_mask", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
        self.t["b_router"] = up(host.b_router)
        self.t["b_mask"] = up(host.b_mask)
        self.fp8 = getattr(c, "expert_format", "") == "fp8"
        for name in SCALES:
            self.t[name] = up(getattr(host, name, None)) if self.fp8 else None
        self.dtype_code = BEAM_F32 if c.dtype == "f32" else BEAM_BF16
        self.torch_dtype = torch.float32 if c.dtype == "f32" else torch.bfloat16
        # optional second copies of the expert weights in the packed operand layout
        self.packed = bool(pack) and c.dtype == "bf16" and not self.fp8
        for name in PACKED:
            self.t[name] = None
        if self.packed:
            self._pack()
        self.desc = self._desc(self.t)

    def _pack(self):
        """Packed copies of the bf16 expert weights (beam_moe_pack_weights)."""
        c = self.cfg
        plan = [("wp_gate", "w_gate", c.E, c.I, c.D), ("wp_up", "w_up", c.E, c.I, c.D),
                ("wp_down", "w_down", c.E, c.D, c.I)]
        if c.S:
            plan += [("wsp_gate", "ws_gate", 1, c.S * c.I_s, c.D), ("wsp_up", "ws_up", 1, c.S * c.I_s, c.D),
                     ("wsp_down", "ws_down", c.S, c.D, c.I_s)]
        stream = torch.cuda.current_stream().cuda_stream
        for dst, src, mats, rows, cols in plan:
            w = self.t[src]
            out = torch.empty_like(w)
            beam_moe_pack_weights(w, mats, rows, cols, out, stream)
            self.t[dst] = out

    def _desc(self, t):
        c = self.cfg
        return make_layer(c.D, c.E, c.K, c.I, self.dtype_code, t["w_router"], t["w_mask"],
                          t["w_gate"], t["w_up"], t["w_down"], b_router=t["b_router"],
                          b_mask=t["b_mask"], n_shared=c.S, I_shared=c.I_s if c.S else 0,
                          ws_gate=t["ws_gate"], ws_up=t["ws_up"], ws_down=t["ws_down"],
                          gating=getattr(c, "gating", 0),
                          expert_format=WEIGHTS_FP8_E4M3 if self.fp8 else WEIGHTS_DTYPE,
                          scale_gate=t["s_gate"], scale_up=t["s_up"], scale_down=t["s_down"],
                          scale_shared_gate=t["ss_gate"], scale_shared_up=t["ss_up"],
                          scale_shared_down=t["ss_down"], segment_len=getattr(c, "segment", 0),
                          expected_avg_k=self.avg_k_hint, **{k: t[k] for k in PACKED})

    def replicas(self, n: int):
        """n extra copies of the expert weights at distinct addresses (same
        values); returns their descriptors.  Used to keep repeated calls from
        being served by the last-level cache."""
        out = []
        for _ in range(n):
            t = {k: (None if v is None else v.clone()) for k, v in self.t.items()}
            out.append((t, self._desc(t)))
        return out

    def workspace(self, T_max: int) -> torch.Tensor:
        n = beam_moe_workspace_size(self.desc, T_max)
        if n == 0 and T_max > 0:
            raise ValueError("invalid layer for workspace sizing")
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def route_buffers(self, T: int):
        c = self.cfg
        d = self.device
        bufs = dict(topk_idx=torch.empty(T, c.K, dtype=torch.int32, device=d),
                    gates=torch.empty(T, c.K, dtype=torch.float32, device=d),
                    mask=torch.empty(T, dtype=torch.int32, device=d),
                    expert_count=torch.empty(c.E, dtype=torch.int32, device=d))
        return bufs, make_route_out(**bufs)
