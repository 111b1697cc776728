"""Seeded synthetic inputs for the BEAM masked-MoE layer.

This module is shared by the tests, the bench and the oracle's callers.  It
holds workload shapes and random-number generation only: no routing, no
expert arithmetic, nothing the layer itself computes.

Random numbers come from Philox-4x64 (Salmon et al., "Parallel random numbers:
as easy as 1, 2, 3", SC'11), a counter-based generator, through numpy's
implementation; normals are drawn with numpy's `standard_normal` on top of it.
Every tensor has its own key, derived from (base seed, workload, tensor name,
sub-stream ids) with BLAKE2b, so any tensor -- or any redrawn token row -- can
be regenerated on its own.  bf16 values are produced once, on the host, by
round-to-nearest-even from float32 and stored as their raw uint16 bit patterns.

Distributions follow the workload descriptions of the masked-MoE layer:
x ~ N(0, 1); router, expert and shared-expert weights ~ N(0, 1/D); mask-router
weights ~ N(0, 0.5/D) so that a mask logit has standard deviation sqrt(0.5);
a scalar mask bias sqrt(0.5) * Phi^-1(keep) sets the expected keep rate of a
top-K candidate; the skewed prefill workload adds a per-expert router bias
~ N(0, 1).

FP8 workloads store the routed and shared expert weights as OCP FP8 E4M3
codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
value 448; no infinities) with one float32 scale per output row: the
float32 draws of a row are divided by max|row| / 448 and rounded to the
nearest code, ties to the even code.  This is how the inputs are prepared,
like the bf16 rounding above; the layer only ever reads the codes and scales.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

BASE_SEED = 20260514

F32 = "f32"
BF16 = "bf16"
FP8 = "fp8"     # expert_format: OCP E4M3 expert weights with per-row float32 scales


@dataclass(frozen=True)
class LayerConfig:
    """Shapes of one masked-MoE layer workload."""
    name: str
    dtype: str          # "f32" or "bf16"
    D: int              # hidden size
    E: int              # routed experts
    K: int              # top-K
    I: int              # routed expert intermediate size
    S: int              # shared experts (0 = none)
    I_s: int            # shared expert intermediate size
    tokens: Tuple[int, ...]   # batch sizes this workload is run at
    keep: float         # expected keep probability of a top-K candidate
    router_bias: bool   # per-expert router bias ~ N(0, 1)
    gating: int = 0     # gate option bits: 1 softmax over all E, 2 renormalise after masking
    expert_format: str = ""   # "" = expert weights in dtype; FP8 = E4M3 codes + row scales
    segment: int = 0    # > 1: every token routes as the first token of its S-token segment

    @property
    def avg_k_target(self) -> float:
        return self.K * self.keep

    @property
    def mask_bias(self) -> float:
        """Scalar mask-router bias giving P(z >= 0) = keep for z ~ N(b, 0.5)."""
        return math.sqrt(0.5) * _norm_ppf(self.keep)


CONFIGS: Dict[str, LayerConfig] = {
    # Tiny fp32 layer, ~50% of top-K candidates kept.
    "tiny_f32": LayerConfig("tiny_f32", F32, D=128, E=8, K=2, I=256, S=0, I_s=0,
                            tokens=(64,), keep=0.5, router_bias=False),
    # DeepSeek-V2-Lite-shaped decode batches, mid sparsity (Avg-K ~3 of 6).
    "dsv2lite_decode": LayerConfig("dsv2lite_decode", BF16, D=2048, E=64, K=6, I=1408,
                                   S=2, I_s=1408, tokens=(1, 8, 64, 256), keep=0.5,
                                   router_bias=False),
    # Same shapes, prefill, high sparsity (Avg-K ~0.5 of 6) with router-bias skew.
    "dsv2lite_prefill": LayerConfig("dsv2lite_prefill", BF16, D=2048, E=64, K=6, I=1408,
                                    S=2, I_s=1408, tokens=(4096,), keep=1.0 / 12.0,
                                    router_bias=True),
    # Mixtral-shaped layer, Avg-K ~1.0 of 2.
    "mixtral": LayerConfig("mixtral", BF16, D=4096, E=8, K=2, I=14336, S=0, I_s=0,
                           tokens=(1, 32, 2048), keep=0.5, router_bias=False),
    # Fine-grained layer, extreme sparsity (Avg-K ~0.15 K).
    "finegrained": LayerConfig("finegrained", BF16, D=1536, E=212, K=16, I=256, S=0, I_s=0,
                               tokens=(16, 512, 8192), keep=0.15, router_bias=False),
    # The DeepSeek-V2-Lite-shaped decode layer with FP8 (E4M3) expert weights.
    "dsv2lite_decode_fp8": LayerConfig("dsv2lite_decode_fp8", BF16, D=2048, E=64, K=6, I=1408,
                                       S=2, I_s=1408, tokens=(1, 8, 64, 256), keep=0.5,
                                       router_bias=False, expert_format=FP8),
}

CONFIG_ORDER = ("tiny_f32", "dsv2lite_decode", "dsv2lite_prefill", "mixtral", "finegrained",
                "dsv2lite_decode_fp8")


def _norm_ppf(p: float) -> float:
    """Inverse standard-normal CDF by bisection on math.erf (inputs only)."""
    if p == 0.5:
        return 0.0
    lo, hi = -12.0, 12.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 0.5 * (1.0 + math.erf(mid / math.sqrt(2.0))) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# --------------------------------------------------------------------------
# Counter-based streams
# --------------------------------------------------------------------------

def stream_key(*parts) -> int:
    """128-bit Philox key for a named sub-stream."""
    text = "/".join(str(p) for p in (BASE_SEED,) + parts).encode()
    return int.from_bytes(hashlib.blake2b(text, digest_size=16).digest(), "little")


def normal_f32(key: int, n: int, std: float) -> np.ndarray:
    """n float32 samples of N(0, std^2) from the stream with this key."""
    g = np.random.Generator(np.random.Philox(key=key))
    a = g.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    return a if dtype == F32 else f32_to_bf16_bits(a)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# Non-negative E4M3 values in code order (codes 0x00 .. 0x7E; 0x7F is NaN):
# exponent field 0 holds the subnormals m * 2^-9, field e > 0 the values
# (1 + m/8) * 2^(e-7).  Strictly increasing, so a code is found by bisection.
_E4M3_POS = np.array([(m * 2.0 ** -9) if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
                      for e in range(16) for m in range(8)][:127], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_encode(a: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (ties to the even code) of each float32 value in
    [-448, 448]; returns uint8 codes.  -0.0 keeps its sign bit."""
    a = np.asarray(a, dtype=np.float32)
    if not np.all(np.abs(a) <= E4M3_MAX):
        raise ValueError("values outside the E4M3 range")
    mag = np.abs(a).astype(np.float64).ravel()
    hi = np.searchsorted(_E4M3_POS, mag, side="left")      # first value >= mag
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3_POS[hi] - mag
    d_lo = mag - _E4M3_POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(d_hi == 0.0, hi, np.where(pick_lo, lo, hi)).astype(np.uint8)
    code |= (np.signbit(a.ravel()).astype(np.uint8) << np.uint8(7))
    return code.reshape(a.shape)


def quantize_rows_e4m3(w: np.ndarray):
    """Per-row scaled E4M3 codes of a float32 matrix [R][C]: scale = max|row|
    / 448 (1 for an all-zero row), code = nearest E4M3 to w / scale."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = w / scale[..., None]
    np.clip(q, -E4M3_MAX, E4M3_MAX, out=q)
    return e4m3_encode(q), scale


def _gen_fp8(cfg: LayerConfig, name: str, shape: Tuple[int, ...], std: float):
    """E4M3 codes [n][R][C] and row scales [n][R] of N(0, std^2) draws, one
    stream per leading index (the same streams as an unquantised tensor)."""
    codes = np.empty(shape, dtype=np.uint8)
    scales = np.empty(shape[:2], dtype=np.float32)
    inner = int(np.prod(shape[1:]))

    def fill(i):
        a = normal_f32(stream_key(cfg.name, name, i), inner, std).reshape(shape[1:])
        codes[i], scales[i] = quantize_rows_e4m3(a)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(shape[0])))
    return codes, scales


def _gen_tensor(cfg: LayerConfig, name: str, shape: Tuple[int, ...], std: float,
                split_leading: bool) -> np.ndarray:
    """Tensor of N(0, std^2) values; with split_leading, one stream per leading index."""
    out_dtype = np.float32 if cfg.dtype == F32 else np.uint16
    out = np.empty(shape, dtype=out_dtype)
    if not split_leading:
        out[...] = _encode(normal_f32(stream_key(cfg.name, name), out.size, std),
                           cfg.dtype).reshape(shape)
        return out
    inner = int(np.prod(shape[1:]))

    def fill(i):
        out[i] = _encode(normal_f32(stream_key(cfg.name, name, i), inner, std),
                         cfg.dtype).reshape(shape[1:])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(shape[0])))
    return out


@dataclass
class Layer:
    """Host copy of one layer's parameters (bf16 as uint16 bits, f32 as float32,
    FP8 expert weights as uint8 E4M3 codes with float32 row scales)."""
    cfg: LayerConfig
    w_router: np.ndarray              # [E][D]
    w_mask: np.ndarray                # [E][D]
    b_router: Optional[np.ndarray]    # [E] float32 or None
    b_mask: Optional[np.ndarray]      # [E] float32 or None
    w_gate: np.ndarray                # [E][I][D]
    w_up: np.ndarray                  # [E][I][D]
    w_down: np.ndarray                # [E][D][I]
    ws_gate: Optional[np.ndarray] = None   # [S][I_s][D]
    ws_up: Optional[np.ndarray] = None     # [S][I_s][D]
    ws_down: Optional[np.ndarray] = None   # [S][D][I_s]
    extra: dict = field(default_factory=dict)
    # FP8 expert weights only: float32 scale of each output row
    s_gate: Optional[np.ndarray] = None    # [E][I]
    s_up: Optional[np.ndarray] = None      # [E][I]
    s_down: Optional[np.ndarray] = None    # [E][D]
    ss_gate: Optional[np.ndarray] = None   # [S][I_s]
    ss_up: Optional[np.ndarray] = None     # [S][I_s]
    ss_down: Optional[np.ndarray] = None   # [S][D]


def make_layer(cfg: LayerConfig, experts: bool = True) -> Layer:
    """Generate a layer's parameters.  experts=False leaves expert tensors empty
    (shape [E][0][0]) for routing-only use."""
    D, E, I = cfg.D, cfg.E, cfg.I
    sd = 1.0 / math.sqrt(D)
    w_router = _gen_tensor(cfg, "w_router", (E, D), sd, False)
    w_mask = _gen_tensor(cfg, "w_mask", (E, D), math.sqrt(0.5 / D), False)
    b_router = normal_f32(stream_key(cfg.name, "b_router"), E, 1.0) if cfg.router_bias else None
    bm = cfg.mask_bias
    b_mask = np.full(E, bm, dtype=np.float32) if bm != 0.0 else None
    if cfg.expert_format == FP8:
        if cfg.dtype != BF16:
            raise ValueError("FP8 expert weights go with bf16 activations")
        return _make_fp8_experts(cfg, w_router, w_mask, b_router, b_mask, experts)
    if experts:
        w_gate = _gen_tensor(cfg, "w_gate", (E, I, D), sd, True)
        w_up = _gen_tensor(cfg, "w_up", (E, I, D), sd, True)
        w_down = _gen_tensor(cfg, "w_down", (E, D, I), sd, True)
    else:
        z = np.empty((E, 0, 0), dtype=np.float32 if cfg.dtype == F32 else np.uint16)
        w_gate = w_up = w_down = z
    ws_gate = ws_up = ws_down = None
    if cfg.S > 0 and experts:
        ws_gate = _gen_tensor(cfg, "ws_gate", (cfg.S, cfg.I_s, D), sd, True)
        ws_up = _gen_tensor(cfg, "ws_up", (cfg.S, cfg.I_s, D), sd, True)
        ws_down = _gen_tensor(cfg, "ws_down", (cfg.S, D, cfg.I_s), sd, True)
    return Layer(cfg, w_router, w_mask, b_router, b_mask, w_gate, w_up, w_down,
                 ws_gate, ws_up, ws_down)


def _make_fp8_experts(cfg, w_router, w_mask, b_router, b_mask, experts):
    D, E, I = cfg.D, cfg.E, cfg.I
    sd = 1.0 / math.sqrt(D)
    if not experts:
        z = np.empty((E, 0, 0), dtype=np.uint8)
        return Layer(cfg, w_router, w_mask, b_router, b_mask, z, z, z)
    w_gate, s_gate = _gen_fp8(cfg, "w_gate", (E, I, D), sd)
    w_up, s_up = _gen_fp8(cfg, "w_up", (E, I, D), sd)
    w_down, s_down = _gen_fp8(cfg, "w_down", (E, D, I), sd)
    sh = {}
    if cfg.S > 0:
        sh["ws_gate"], sh["ss_gate"] = _gen_fp8(cfg, "ws_gate", (cfg.S, cfg.I_s, D), sd)
        sh["ws_up"], sh["ss_up"] = _gen_fp8(cfg, "ws_up", (cfg.S, cfg.I_s, D), sd)
        sh["ws_down"], sh["ss_down"] = _gen_fp8(cfg, "ws_down", (cfg.S, D, cfg.I_s), sd)
    return Layer(cfg, w_router, w_mask, b_router, b_mask, w_gate, w_up, w_down,
                 s_gate=s_gate, s_up=s_up, s_down=s_down, **sh)


def make_x(cfg: LayerConfig, T: int, stream: str = "x") -> np.ndarray:
    """Token activations [T][D], x ~ N(0, 1)."""
    a = normal_f32(stream_key(cfg.name, stream, T), T * cfg.D, 1.0)
    return _encode(a, cfg.dtype).reshape(T, cfg.D)


def redraw_row(cfg: LayerConfig, T: int, token: int, attempt: int,
               stream: str = "x") -> np.ndarray:
    """Replacement row for one token, from its own sub-stream (attempt >= 1)."""
    a = normal_f32(stream_key(cfg.name, stream, T, token, attempt), cfg.D, 1.0)
    return _encode(a, cfg.dtype)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (input decoding only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
