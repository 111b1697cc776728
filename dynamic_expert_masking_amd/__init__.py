"""Python binding of the BEAM masked-MoE C ABI (include/beam_moe.h).

Argument marshalling only: every step of the layer runs in the HIP library
libbeam_moe.so built from csrc/ (python -m dynamic_expert_masking_amd.build).
Tensors are passed as device pointers (torch tensors' data_ptr()); streams as
hipStream_t handles.  There is no fallback: if the library is missing,
importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbeam_moe.so")

BEAM_OK = 0
BEAM_ERR_INVALID_ARG = -1
BEAM_ERR_UNSUPPORTED = -2
BEAM_ERR_WORKSPACE = -3
BEAM_ERR_HIP = -4

BEAM_F32 = 0
BEAM_BF16 = 1


class BeamError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {beam_status_str(status)} ({status})")


class beam_moe_layer(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("I", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("I_shared", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("w_router", ctypes.c_void_p), ("w_mask", ctypes.c_void_p),
                ("b_router", ctypes.c_void_p), ("b_mask", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
                ("gating", ctypes.c_int32), ("expert_format", ctypes.c_int32),
                ("scale_gate", ctypes.c_void_p), ("scale_up", ctypes.c_void_p),
                ("scale_down", ctypes.c_void_p), ("scale_shared_gate", ctypes.c_void_p),
                ("scale_shared_up", ctypes.c_void_p), ("scale_shared_down", ctypes.c_void_p),
                ("segment_len", ctypes.c_int32),
                ("wp_gate", ctypes.c_void_p), ("wp_up", ctypes.c_void_p), ("wp_down", ctypes.c_void_p),
                ("wsp_gate", ctypes.c_void_p), ("wsp_up", ctypes.c_void_p), ("wsp_down", ctypes.c_void_p),
                ("expected_avg_k", ctypes.c_float)]


# beam_gate_flag bits of beam_moe_layer.gating
GATE_SOFTMAX_ALL = 1
GATE_RENORM = 2
GATE_BINARY = 4
# beam_weight_format values of beam_moe_layer.expert_format
WEIGHTS_DTYPE = 0
WEIGHTS_FP8_E4M3 = 1


class beam_route_out(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("gates", ctypes.c_void_p),
                ("mask", ctypes.c_void_p), ("expert_count", ctypes.c_void_p)]


class beam_stats(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("active_experts", ctypes.c_int32), ("active_pairs", ctypes.c_int64),
                ("avg_k", ctypes.c_double), ("flops_routed", ctypes.c_double),
                ("flops_topk_routed", ctypes.c_double), ("flops_shared", ctypes.c_double),
                ("flops_router", ctypes.c_double), ("flops_reduction", ctypes.c_double),
                ("bytes_active_expert_weights", ctypes.c_double),
                ("bytes_total_min", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m dynamic_expert_masking_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, I32, SZ = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.beam_moe_workspace_size.argtypes = [P(beam_moe_layer), I32]
        L.beam_moe_workspace_size.restype = SZ
        L.beam_moe_route.argtypes = [P(beam_moe_layer), VP, I32, P(beam_route_out), VP, SZ, VP]
        L.beam_moe_route.restype = ctypes.c_int
        L.beam_moe_forward.argtypes = [P(beam_moe_layer), VP, I32, VP, P(beam_route_out), VP, SZ, VP]
        L.beam_moe_forward.restype = ctypes.c_int
        L.beam_moe_forward_static.argtypes = [P(beam_moe_layer), VP, I32, VP, P(beam_route_out), VP]
        L.beam_moe_forward_static.restype = ctypes.c_int
        L.beam_moe_mask_backward.argtypes = [P(beam_moe_layer), VP, VP, I32, ctypes.c_float, VP, VP,
                                             VP, VP, SZ, VP]
        L.beam_moe_mask_backward.restype = ctypes.c_int
        L.beam_moe_stats.argtypes = [P(beam_moe_layer), VP, I32, P(beam_stats), VP]
        L.beam_moe_stats.restype = ctypes.c_int
        L.beam_moe_stats_host.argtypes = [P(beam_moe_layer), P(ctypes.c_int32), I32, P(beam_stats)]
        L.beam_moe_stats_host.restype = ctypes.c_int
        L.beam_status_str.argtypes = [ctypes.c_int]
        L.beam_status_str.restype = ctypes.c_char_p
        L.beam_profile_begin.argtypes = [I32]
        L.beam_profile_begin.restype = ctypes.c_int
        L.beam_profile_end.argtypes = [P(ctypes.c_char_p), P(I32), P(ctypes.c_double), I32]
        L.beam_profile_end.restype = ctypes.c_int
        L.beam_moe_pack_weights.argtypes = [VP, I32, I32, I32, VP, VP]
        L.beam_moe_pack_weights.restype = ctypes.c_int
        L.beam_mfma_loop.argtypes = [VP, I32, I32, VP]
        L.beam_mfma_loop.restype = ctypes.c_int
        L.beam_copy_kernel.argtypes = [VP, VP, SZ, VP]
        L.beam_copy_kernel.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(status: int, where: str) -> None:
    if status != BEAM_OK:
        raise BeamError(status, where)


def make_layer(D, E, K, I, dtype, w_router, w_mask, w_gate, w_up, w_down, b_router=None,
               b_mask=None, n_shared=0, I_shared=0, ws_gate=None, ws_up=None,
               ws_down=None, gating=0, expert_format=WEIGHTS_DTYPE, scale_gate=None,
               scale_up=None, scale_down=None, scale_shared_gate=None, scale_shared_up=None,
               scale_shared_down=None, segment_len=0, wp_gate=None, wp_up=None, wp_down=None,
               wsp_gate=None, wsp_up=None, wsp_down=None, expected_avg_k=0.0) -> beam_moe_layer:
    """Fill a beam_moe_layer descriptor from tensors (or raw addresses).  The
    caller keeps the tensors alive while the descriptor is in use."""
    return beam_moe_layer(D, E, K, I, n_shared, I_shared, dtype, _ptr(w_router), _ptr(w_mask),
                          _ptr(b_router), _ptr(b_mask), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                          _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), int(gating),
                          int(expert_format), _ptr(scale_gate), _ptr(scale_up), _ptr(scale_down),
                          _ptr(scale_shared_gate), _ptr(scale_shared_up), _ptr(scale_shared_down),
                          int(segment_len), _ptr(wp_gate), _ptr(wp_up), _ptr(wp_down),
                          _ptr(wsp_gate), _ptr(wsp_up), _ptr(wsp_down), float(expected_avg_k))


def make_route_out(topk_idx, gates, mask, expert_count) -> beam_route_out:
    return beam_route_out(_ptr(topk_idx), _ptr(gates), _ptr(mask), _ptr(expert_count))


def beam_moe_workspace_size(layer: beam_moe_layer, T_max: int) -> int:
    return int(lib().beam_moe_workspace_size(ctypes.byref(layer), int(T_max)))


def beam_moe_route(layer: beam_moe_layer, x, T: int, out: beam_route_out, ws, ws_bytes: int,
                   stream: int = 0) -> None:
    _check(lib().beam_moe_route(ctypes.byref(layer), _ptr(x), int(T), ctypes.byref(out), _ptr(ws),
                                int(ws_bytes), stream), "beam_moe_route")


def beam_moe_mask_backward(layer: beam_moe_layer, x, dy, T: int, beta: float, dwm, dbm, lreg, ws,
                           ws_bytes: int, stream: int = 0) -> None:
    """Mask-router loss value and straight-through gradient (see the header)."""
    _check(lib().beam_moe_mask_backward(ctypes.byref(layer), _ptr(x), _ptr(dy), int(T), float(beta),
                                        _ptr(dwm), _ptr(dbm), _ptr(lreg), _ptr(ws), int(ws_bytes),
                                        stream), "beam_moe_mask_backward")


def beam_moe_forward(layer: beam_moe_layer, x, T: int, y, out: Optional[beam_route_out], ws,
                     ws_bytes: int, stream: int = 0) -> None:
    outp = ctypes.byref(out) if out is not None else None
    _check(lib().beam_moe_forward(ctypes.byref(layer), _ptr(x), int(T), _ptr(y), outp, _ptr(ws),
                                  int(ws_bytes), stream), "beam_moe_forward")


# Size of the static device workspace of beam_moe_forward_static (bytes).
STATIC_WORKSPACE_BYTES = 128 << 20


def beam_moe_forward_static(layer: beam_moe_layer, x, T: int, y, out: Optional[beam_route_out],
                            stream: int = 0) -> None:
    """beam_moe_forward without a caller workspace (the library's static
    device array; allocates nothing)."""
    outp = ctypes.byref(out) if out is not None else None
    _check(lib().beam_moe_forward_static(ctypes.byref(layer), _ptr(x), int(T), _ptr(y), outp, stream),
           "beam_moe_forward_static")


def beam_moe_stats(layer: beam_moe_layer, expert_count, T: int, stream: int = 0) -> dict:
    st = beam_stats()
    _check(lib().beam_moe_stats(ctypes.byref(layer), _ptr(expert_count), int(T),
                                ctypes.byref(st), stream), "beam_moe_stats")
    return st.as_dict()


def beam_moe_stats_host(layer: beam_moe_layer, counts, T: int) -> dict:
    """counts: a sequence of E host integers."""
    arr = (ctypes.c_int32 * len(counts))(*[int(c) for c in counts])
    st = beam_stats()
    _check(lib().beam_moe_stats_host(ctypes.byref(layer), arr, int(T), ctypes.byref(st)),
           "beam_moe_stats_host")
    return st.as_dict()


def beam_status_str(status: int) -> str:
    return lib().beam_status_str(int(status)).decode()


def beam_profile_begin(max_launches: int) -> None:
    _check(lib().beam_profile_begin(int(max_launches)), "beam_profile_begin")


def beam_profile_end(max_out: int = 64) -> dict:
    """{kernel name: (launches, total ms)} for the launches timed since begin."""
    names = (ctypes.c_char_p * max_out)()
    launches = (ctypes.c_int32 * max_out)()
    ms = (ctypes.c_double * max_out)()
    n = lib().beam_profile_end(names, launches, ms, max_out)
    if n < 0:
        raise BeamError(n, "beam_profile_end")
    return {names[i].decode(): (int(launches[i]), float(ms[i])) for i in range(n)}


def beam_copy_kernel(dst, src, nbytes: int, stream: int = 0) -> None:
    _check(lib().beam_copy_kernel(_ptr(dst), _ptr(src), int(nbytes), stream), "beam_copy_kernel")


def beam_mfma_loop(out, blocks: int, iters: int, stream: int = 0) -> None:
    """MFMA throughput probe (see the header); out holds blocks * 256 floats."""
    _check(lib().beam_mfma_loop(_ptr(out), int(blocks), int(iters), stream), "beam_mfma_loop")


def beam_moe_pack_weights(w, mats: int, rows: int, cols: int, packed, stream: int = 0) -> None:
    """Packed operand layout of `mats` bf16 matrices [rows][cols] (see the header)."""
    _check(lib().beam_moe_pack_weights(_ptr(w), int(mats), int(rows), int(cols), _ptr(packed), stream),
           "beam_moe_pack_weights")
