"""Shared test helpers: layers from fixtures, margin-checked inputs, caching."""
from __future__ import annotations

import json
import math
import os
from dataclasses import replace
from functools import lru_cache

import numpy as np

import synth
from synth import Layer, LayerConfig

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Decision margins for generated inputs: consecutive sorted router logits among
# the top K+1 differ by at least GAP, and every top-K candidate has
# |sigmoid(z) - 0.5| >= MASK_MARGIN.  Both are far above the float32
# accumulation error of a D-term dot product at these sizes, so the top-K set,
# its order and the mask bits cannot depend on summation order.
GAP = 1e-4
MASK_MARGIN = 1e-3


def small_config(name: str, dtype: str, D: int, E: int, K: int, I: int, S: int = 0,
                 I_s: int = 0, keep: float = 0.5, router_bias: bool = False) -> LayerConfig:
    return LayerConfig(name, dtype, D=D, E=E, K=K, I=I, S=S, I_s=I_s, tokens=(),
                       keep=keep, router_bias=router_bias)


def layer_from_json(name: str):
    """Layer and x from a hand-written fixture under tests/golden/."""
    with open(os.path.join(GOLDEN, name)) as f:
        j = json.load(f)
    assert j["dtype"] == "f32"
    cfg = small_config("golden:" + name, "f32", j["D"], j["E"], j["K"], j["I"], j["S"], j["I_s"])
    a = lambda k: np.asarray(j[k], dtype=np.float32)  # noqa: E731
    layer = Layer(cfg, a("w_router"), a("w_mask"), None, None, a("w_gate"), a("w_up"), a("w_down"),
                  a("ws_gate") if j["S"] else None, a("ws_up") if j["S"] else None,
                  a("ws_down") if j["S"] else None)
    return j, layer, a("x")


def eval_closed_form(expr) -> float:
    """Evaluate a closed-form string from a fixture (only e, exp are defined)."""
    return float(eval(str(expr), {"__builtins__": {}}, {"e": math.e, "exp": math.exp}))


def margins_ok(r: np.ndarray, z: np.ndarray, K: int, mask_margin: bool = True) -> np.ndarray:
    """Per-token check of the decision margins (float64 logits).  mask_margin=False
    skips the mask check (for layers whose mask logits are exactly constant)."""
    T, E = r.shape
    srt = -np.sort(-r, axis=1)
    upto = min(K + 1, E)
    gaps = srt[:, : upto - 1] - srt[:, 1:upto]
    ok = (gaps >= GAP).all(axis=1) if upto > 1 else np.ones(T, bool)
    if not mask_margin:
        return ok
    top = np.argsort(-r, axis=1, kind="stable")[:, :K]
    zt = np.take_along_axis(z, top, axis=1)
    sig = 1.0 / (1.0 + np.exp(-zt))
    ok &= (np.abs(sig - 0.5) >= MASK_MARGIN).all(axis=1)
    return ok


def enforce_margins(layer: Layer, x: np.ndarray, T: int, stream: str = "x",
                    max_attempts: int = 64) -> np.ndarray:
    """Redraw (from each token's own sub-stream) every row whose decisions are
    closer than the margins; returns a new x."""
    x = x.copy()
    cfg = layer.cfg
    bad = np.arange(T)
    attempt = 0
    while True:
        r, z = oracle.router_logits(layer, x[bad])
        fail = bad[~margins_ok(r, z, cfg.K, mask_margin=bool(np.any(layer.w_mask)))]
        if fail.size == 0:
            return x
        attempt += 1
        if attempt > max_attempts:
            raise RuntimeError(f"could not satisfy margins for {fail.size} tokens")
        for t in fail:
            x[t] = synth.redraw_row(cfg, T, int(t), attempt, stream)
        bad = fail


@lru_cache(maxsize=4)
def cached_layer(name: str, experts: bool = True) -> Layer:
    return synth.make_layer(synth.CONFIGS[name], experts=experts)


def inputs(cfg: LayerConfig, T: int, layer: Layer, stream: str = "x") -> np.ndarray:
    """Margin-checked x for a layer."""
    return enforce_margins(layer, synth.make_x(cfg, T, stream), T, stream)


def with_mask(layer: Layer, w_mask_zero: bool = False, b_mask=None) -> Layer:
    """Copy of a layer with the mask router zeroed and/or its bias replaced."""
    wm = np.zeros_like(layer.w_mask) if w_mask_zero else layer.w_mask
    bm = layer.b_mask if b_mask is None else np.full(layer.cfg.E, b_mask, dtype=np.float32)
    return replace(layer, w_mask=wm, b_mask=bm)
