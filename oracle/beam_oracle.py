"""Oracle for the BEAM masked-MoE layer forward pass.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  It is a plain, slow, float64 numpy
implementation of what the layer computes, written from the method's
description and sharing nothing with the HIP library: no kernels, headers,
helpers or tables.

Sources (cited below by the short names on the left):

  [P3]  "BEAM: Dynamic MoE 라우팅을 위한 Binary Expert Activation Masking"
        (aitrends.kr).  Its method paragraph gives the four steps: Step 1
        Standard Top-K Routing, Step 2 Raw Mask Generation, Step 3 Binary
        Masking, Step 4 Masked Aggregation; its architecture paragraph restates
        them and adds the zero-initialised mask router; its limitations list,
        item C, mentions shared experts.
  [P1]  "BEAM: 用于 MoE 动态路由的二进制专家激活掩码" (ai-feeds.com), section
        方法 / 输出与推理加速: at inference only experts whose mask is 1 run.
  [P2]  "BEAM: Binäre Expertenaktivierungsmaskierung für dynamisches Routing in
        MoE" (chatpaper.ai), the English abstract: MoE-layer FLOPs fall with
        the number of active experts.
  [P5]  "Stepped MoE: Segment-Level Routing with Configurable Inference
        Complexity" (paper.rainbus.top), sections 核心方法 (core method) and
        方法步骤详情 (method steps): the tokens are cut into segments of S
        tokens, the representation at each segment's first position picks
        the segment's top-k experts as a {0,1} mask, and the choice is
        refreshed every S tokens.

Readings where the pages leave a step open (each is also listed with the
design notes of the repository):

  * Router R(x) is linear, r = x.Wr^T (+ optional per-expert bias b_r).
  * The mask router has one logit per expert, z = x.Wm^T (+ optional bias b_m),
    gathered at the top-K experts; m_hat = sigmoid(z).
  * "m = 1 if m_hat >= 0.5" is decided as z >= 0, which is the same set in
    exact arithmetic and avoids a rounded sigmoid landing on 0.5.
  * Softmax runs over the K kept logits only; masked gates are NOT
    renormalised (g_hat = g * m, so sum(g_hat) <= 1).
  * Top-K order: descending logit, equal logits ordered by lower expert index.
  * Experts are SwiGLU FFNs: E(x) = Wd (silu(Wg x) * (Wu x)), silu(a) = a/(1+e^-a).
  * Shared experts are always on, with gate 1, and are added to y.
  * Gate options (off by default; not part of the method as the pages
    describe it): [P1]'s section on the input and overall flow applies the
    mask to the router's scores without fixing where the softmax sits, so
    select_experts also offers g = softmax over all E logits read at the
    top-K experts (gating bit 1), and renormalising g_hat over the kept
    slots after masking (gating bit 2; all zero when no slot is kept).
  * Segment routing (off by default; [P5]): with cfg.segment = S > 1, token t
    uses the routing (top-K set, g, m) computed from token t - t mod S, the
    first token of its segment of the batch.  Gate bit 4 (GATE_BINARY)
    gives every top-K slot g = 1, so g_hat = m: [P5]'s {0,1} expert mask
    with unweighted expert outputs.  It cannot be combined with bit 1.
  * Router and mask decisions (which experts, which bits) are taken on
    float32 logits, the precision the GPU kernels decide in: the logits are
    computed in float64 and rounded once to float32.  Everything else is
    float64.

mask_router_backward follows [P3]'s training strategy (L_reg and the
straight-through estimator); see its docstring.

FP8 expert weights ([P1], section on interfaces with existing products and
workflows, item 3: the masking combines with model quantisation): a layer
whose config has expert_format "fp8" stores every routed and shared expert
matrix as OCP FP8 E4M3 codes with one float32 scale per output row.  Its
weights are decode_e4m3(code) * scale[row], exactly, in float64; everything
after that is the same computation.  decode_e4m3 is written from the format's
definition (OCP 8-bit floating point specification, E4M3: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent field 0,
S.1111.111 is NaN, no infinities).

Parity status: every function here is pinned by tests in tests/test_oracle.py
(closed forms, a hand-derived worked example under tests/golden/, library
special cases and brute-force sums); none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "widen", "router_logits", "select_experts", "Routing", "route", "silu",
    "GATE_SOFTMAX_ALL", "GATE_RENORM", "GATE_BINARY", "segment_heads",
    "mask_router_backward",
    "expert_ffn", "forward", "expert_counts", "layer_stats", "decode_e4m3",
    "expert_matrices",
]


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs: bf16 bit patterns (uint16) are
    moved to the top half of a float32 word; float32 is widened directly."""
    a = np.asarray(a)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are stored as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 inputs are stored as float32")
        return a.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def router_logits(layer, x: np.ndarray):
    """Router logits r and mask-router logits z, float64, shape [T][E].

    [P3] Step 1: r = R(x); Step 2: the raw mask is sigmoid(x Wm), so z = x Wm
    is its argument.  Optional biases are added when the layer has them.
    """
    dt = layer.cfg.dtype
    X = widen(x, dt)
    r = X @ widen(layer.w_router, dt).T
    z = X @ widen(layer.w_mask, dt).T
    if layer.b_router is not None:
        r = r + np.asarray(layer.b_router, dtype=np.float64)
    if layer.b_mask is not None:
        z = z + np.asarray(layer.b_mask, dtype=np.float64)
    return r, z


@dataclass
class Routing:
    idx: np.ndarray        # [T][K] int32, top-K experts by descending logit
    g: np.ndarray          # [T][K] float64, softmax over the K kept logits (over all E with GATE_SOFTMAX_ALL)
    keep: np.ndarray       # [T][K] bool, binary mask m on the top-K candidates
    ghat: np.ndarray       # [T][K] float64, g * m
    mask_bits: np.ndarray  # [T] uint32, bit k = keep[t][k]


GATE_SOFTMAX_ALL = 1
GATE_RENORM = 2
GATE_BINARY = 4


def select_experts(r: np.ndarray, z: np.ndarray, K: int, gating: int = 0) -> Routing:
    """Top-K, softmax, binary mask and masked gates for each token.

    [P3] Step 1: keep the K largest router logits and apply a softmax to them
    (g).  Step 2/3: m_i = 1 when sigmoid(z_i) >= 0.5, for i in the top-K set.
    Step 4: g_hat = g * m.  Decisions are taken on float32-rounded logits.
    Gate options (see the module notes): GATE_SOFTMAX_ALL takes g from a
    softmax over all E logits; GATE_RENORM divides g_hat by its sum over the
    token's slots when that sum is positive; GATE_BINARY sets g = 1 on every
    top-K slot ([P5]'s {0,1} mask).
    """
    r32 = np.asarray(r, dtype=np.float64).astype(np.float32)
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32)
    T, E = r32.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    if (gating & GATE_BINARY) and (gating & GATE_SOFTMAX_ALL):
        raise ValueError("binary gates exclude the all-expert softmax")
    idx = np.empty((T, K), dtype=np.int32)
    g = np.empty((T, K), dtype=np.float64)
    keep = np.empty((T, K), dtype=bool)
    for t in range(T):
        # Stable sort of the negated logits: equal logits keep index order,
        # so the lower expert index comes first.
        order = np.argsort(-r32[t], kind="stable")[:K]
        idx[t] = order
        if gating & GATE_BINARY:
            g[t] = 1.0
        elif gating & GATE_SOFTMAX_ALL:
            v = r32[t].astype(np.float64)
            w = np.exp(v - v.max())
            g[t] = w[order] / w.sum()
        else:
            v = r32[t, order].astype(np.float64)
            w = np.exp(v - v.max())
            g[t] = w / w.sum()
        keep[t] = z32[t, order] >= np.float32(0.0)
    ghat = np.where(keep, g, 0.0)
    if gating & GATE_RENORM:
        s = ghat.sum(axis=1, keepdims=True)
        ghat = np.where(s > 0.0, ghat / np.where(s > 0.0, s, 1.0), 0.0)
    weights = (np.uint64(1) << np.arange(K, dtype=np.uint64))
    mask_bits = (keep.astype(np.uint64) * weights).sum(axis=1).astype(np.uint32)
    return Routing(idx, g, keep, ghat, mask_bits)


def segment_heads(tokens: np.ndarray, S: int) -> np.ndarray:
    """[P5]: the first token of each token's S-token segment (t - t mod S);
    S <= 1 leaves every token its own head."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return tokens - tokens % S if S > 1 else tokens


def route(layer, x: np.ndarray, tokens: Optional[Sequence[int]] = None) -> Routing:
    """[P3] Steps 1-3 (and the gate product of Step 4) for the given tokens
    of x (all by default).  With segment routing ([P5]) each token takes the
    decisions computed on its segment's first token."""
    cfg = layer.cfg
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    src = segment_heads(tok, getattr(cfg, "segment", 0))
    r, z = router_logits(layer, x[src])
    return select_experts(r, z, cfg.K, getattr(cfg, "gating", 0))


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a * sigmoid(a) = a / (1 + exp(-a))."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def expert_ffn(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, X: np.ndarray) -> np.ndarray:
    """SwiGLU expert applied to rows of X (float64): Wd (silu(Wg x) * (Wu x)).

    wg, wu: [I][D]; wd: [D][I]; X: [n][D]  ->  [n][D].
    """
    h = silu(X @ wg.T) * (X @ wu.T)
    return h @ wd.T


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Value of OCP FP8 E4M3 codes (uint8) as float64.

    Bit 7 is the sign, bits 6..3 the exponent field e, bits 2..0 the
    mantissa field m.  e = 0: (-1)^s m 2^-9 (subnormal, 2^(1-7) m/8);
    0 < e: (-1)^s (1 + m/8) 2^(e-7); e = 15 with m = 7 is NaN (the format
    has no infinities, so e = 15, m < 7 are ordinary values up to 448).
    """
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("E4M3 codes are stored as uint8")
    c = c.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def _matrix(layer, name: str, i: int) -> np.ndarray:
    """float64 value of expert matrix `name` ("w_gate", "ws_down", ...) number i."""
    cfg = layer.cfg
    a = getattr(layer, name)[i]
    if getattr(cfg, "expert_format", "") == "fp8":
        scale = getattr(layer, "s" + name[1:] if name.startswith("ws_") else "s_" + name[2:])[i]
        return decode_e4m3(a) * np.asarray(scale, dtype=np.float64)[:, None]
    return widen(a, cfg.dtype)


def expert_matrices(layer, i: int, shared: bool = False):
    """(Wg, Wu, Wd) of routed expert i, or of shared expert i, in float64."""
    p = "ws_" if shared else "w_"
    return tuple(_matrix(layer, p + n, i) for n in ("gate", "up", "down"))


def _expert_weights(layer, e: int):
    return expert_matrices(layer, e)


def _shared_weights(layer, s: int):
    return expert_matrices(layer, s, shared=True)


def forward(layer, x: np.ndarray, tokens: Optional[Sequence[int]] = None,
            routing: Optional[Routing] = None):
    """Layer output y (float64) for the given tokens (all by default).

    [P3] Step 4: y = sum_i g_hat_i E_i(x) over the top-K candidates; [P1]
    only candidates with m = 1 are evaluated (g_hat = 0 for the others, so
    skipping them leaves y unchanged).  Shared experts ([P3] limitations C)
    are added with gate 1.  Terms are added token by token in slot order
    k = 0..K-1, then shared expert 0..S-1; tokens that use the same expert in
    the same slot are evaluated together.

    Returns (routing of the selected tokens, y [n][D]).
    """
    cfg = layer.cfg
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, dtype=np.int64)
    rt = route(layer, x, tok) if routing is None else routing
    X = widen(x[tok], cfg.dtype)
    y = np.zeros((len(tok), cfg.D), dtype=np.float64)
    cache = {}
    for k in range(cfg.K):
        for e in np.unique(rt.idx[:, k]):
            rows = np.nonzero((rt.idx[:, k] == e) & rt.keep[:, k])[0]
            if rows.size == 0:
                continue
            if e not in cache:
                cache[e] = _expert_weights(layer, int(e))
            out = expert_ffn(*cache[e], X[rows])
            y[rows] += rt.ghat[rows, k][:, None] * out
    for s in range(cfg.S):
        y += expert_ffn(*_shared_weights(layer, s), X)
    return rt, y


def mask_router_backward(layer, x: np.ndarray, dy: np.ndarray, beta: float):
    """Gradient of L = L_task + beta * L_reg with respect to the mask router.

    [P3] training strategy (method paragraph): L = L_lm + alpha L_bal + beta
    L_reg with L_reg = (1/K) sum_{i in TK} |m_hat_i|, and the straight-through
    estimator passes m_hat's gradient through the binarisation (dm/dm_hat :=
    1); [P1] method section, binarisation and STE.  Over a batch, L_reg is the
    mean over tokens.  dy = dL_task/dy (float64 [T][D]) is given; with
    y = sum_k g_k m_k E_k(x):

      dL/dm_hat_k = g_k <dy, E_k(x)> + beta / (T K)       (m_hat > 0)
      dL/dz_k     = dL/dm_hat_k * m_hat_k (1 - m_hat_k)
      dL/dWm[e]   = sum over (t, k) with TK_k = e of dL/dz_k * x_t
      dL/db_m[e]  = sum over the same (t, k) of dL/dz_k

    E_k(x) is evaluated for every top-K candidate, masked or not.  m_hat is
    taken from the float32-rounded mask logit, like the decisions.  Only the
    method's own gate (gating 0) is covered.

    Returns (L_reg, dWm [E][D], db_m [E], dz [T][K]) in float64.
    """
    cfg = layer.cfg
    if getattr(cfg, "gating", 0) or getattr(cfg, "segment", 0) > 1:
        raise ValueError("the mask-router backward covers the method's own per-token gate only")
    T = x.shape[0]
    r, z = router_logits(layer, x)
    rt = select_experts(r, z, cfg.K)
    z32 = np.asarray(z, dtype=np.float64).astype(np.float32).astype(np.float64)
    zk = np.take_along_axis(z32, rt.idx.astype(np.int64), axis=1)
    mhat = 1.0 / (1.0 + np.exp(-zk))
    X = widen(x, cfg.dtype)
    DY = np.asarray(dy, dtype=np.float64)
    dot = np.zeros((T, cfg.K))
    for e in np.unique(rt.idx):
        wg, wu, wd = _expert_weights(layer, int(e))
        for k in range(cfg.K):
            rows = np.nonzero(rt.idx[:, k] == e)[0]
            if rows.size:
                dot[rows, k] = np.sum(DY[rows] * expert_ffn(wg, wu, wd, X[rows]), axis=1)
    dmhat = rt.g * dot + beta / (T * cfg.K)
    dz = dmhat * mhat * (1.0 - mhat)
    dwm = np.zeros((cfg.E, cfg.D))
    dbm = np.zeros(cfg.E)
    for t in range(T):
        for k in range(cfg.K):
            e = int(rt.idx[t, k])
            dwm[e] += dz[t, k] * X[t]
            dbm[e] += dz[t, k]
    lreg = float(mhat.sum() / (T * cfg.K))
    return lreg, dwm, dbm, dz


def expert_counts(rt: Routing, E: int) -> np.ndarray:
    """Surviving (token, expert) pairs per expert: c_e = #{(t,k): idx=e, m=1}."""
    return np.bincount(rt.idx[rt.keep].astype(np.int64), minlength=E).astype(np.int64)


def layer_stats(cfg, counts: np.ndarray, T: int) -> dict:
    """Work accounting from the per-expert counts.

    Avg-K = surviving pairs / T ([P3] results: average active experts per
    token).  MoE-layer FLOPs scale with the surviving pairs ([P2] abstract):
    a SwiGLU expert costs 6*D*I flops per token (three D x I products, two
    flops per multiply-add); the router costs 4*E*D per token (two E x D
    products).  Active-expert bytes: every expert with at least one pair is
    read once, plus the shared experts.
    """
    counts = np.asarray(counts, dtype=np.int64)
    P = int(counts.sum())
    active = int((counts > 0).sum())
    elt = 4 if cfg.dtype == "f32" else 2
    D, I = cfg.D, cfg.I
    fp8 = getattr(cfg, "expert_format", "") == "fp8"
    # bytes of one expert's three matrices (FP8: codes plus a float32 per row)
    per_routed = 3 * D * I + 4 * (2 * I + D) if fp8 else 3 * D * I * elt
    per_shared = 3 * D * cfg.I_s + 4 * (2 * cfg.I_s + D) if fp8 else 3 * D * cfg.I_s * elt
    out = {
        "T": T, "E": cfg.E, "K": cfg.K,
        "active_pairs": P,
        "active_experts": active,
        "avg_k": (P / T) if T > 0 else 0.0,
        "flops_routed": 6.0 * D * I * P,
        "flops_topk_routed": 6.0 * D * I * T * cfg.K,
        "flops_shared": 6.0 * D * cfg.I_s * cfg.S * T,
        "flops_router": 4.0 * cfg.E * D * T,
        "bytes_active_expert_weights": float(per_routed * active + per_shared * cfg.S),
    }
    out["flops_reduction"] = (1.0 - out["flops_routed"] / out["flops_topk_routed"]) if T > 0 else 0.0
    out["bytes_total_min"] = (out["bytes_active_expert_weights"]
                              + 2.0 * cfg.E * D * elt          # router + mask-router weights
                              + 2.0 * T * D * elt)             # x in, y out
    return out
