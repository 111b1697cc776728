"""Every plausible mistake planted in a copy of the oracle fails some pin.

Mistakes are planted only in fresh copies of the oracle module, on the CPU.
"""
import os
import types

import numpy as np
import pytest

import oracle.beam_oracle as real
from oracle_pins import ALL_PINS

SRC = open(real.__file__).read()


def _copy():
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = real.__file__
    exec(compile(SRC, real.__file__, "exec"), mod.__dict__)
    return mod


def _src_mutant(*edits):
    src = SRC
    for old, new in edits:
        assert src.count(old) == 1, old
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, real.__file__, "exec"), mod.__dict__)
    return mod


MUTANTS = {
    # gates renormalised after masking
    "renormalise": ("ghat = np.where(keep, g, 0.0)",
                    "ghat = np.where(keep, g, 0.0); ghat = ghat / np.maximum(ghat.sum(1, keepdims=True), 1e-300)"),
    # softmax over all experts, then top-K
    "softmax_all_E": ("v = r32[t, order].astype(np.float64)\n            w = np.exp(v - v.max())\n            g[t] = w / w.sum()",
                      "v = r32[t, order].astype(np.float64)\n            w = np.exp(v - r32[t].max())\n            g[t] = w / np.exp(r32[t].astype(np.float64) - r32[t].max()).sum()"),
    # gate option 1 taken over the top-K logits only
    "softmax_all_ignored": ("g[t] = w[order] / w.sum()", "g[t] = w[order] / w[order].sum()"),
    # gate option 2 ignored
    "renorm_ignored": ("if gating & GATE_RENORM:", "if False:"),
    # backward: sigmoid derivative dropped
    "bwd_no_sigmoid_grad": ("dz = dmhat * mhat * (1.0 - mhat)", "dz = dmhat"),
    # backward: masked gates used (masked candidates get no task gradient)
    "bwd_masked_gate": ("dmhat = rt.g * dot + beta / (T * cfg.K)", "dmhat = rt.ghat * dot + beta / (T * cfg.K)"),
    # backward: L_reg summed over tokens instead of averaged
    "bwd_lreg_sum": ("lreg = float(mhat.sum() / (T * cfg.K))", "lreg = float(mhat.sum() / cfg.K)"),
    # gate option 2 normalising by the unmasked gates
    "renorm_unmasked_sum": ("s = ghat.sum(axis=1, keepdims=True)", "s = g.sum(axis=1, keepdims=True)"),
    # strict threshold
    "strict_threshold": ("keep[t] = z32[t, order] >= np.float32(0.0)", "keep[t] = z32[t, order] > np.float32(0.0)"),
    # mask read by slot instead of by expert
    "mask_by_slot": ("keep[t] = z32[t, order] >= np.float32(0.0)", "keep[t] = z32[t, :K] >= np.float32(0.0)"),
    # mask ignored: masked candidates evaluated with their unmasked gate
    "mask_ignored": [("rows = np.nonzero((rt.idx[:, k] == e) & rt.keep[:, k])[0]",
                      "rows = np.nonzero(rt.idx[:, k] == e)[0]"),
                     ("y[rows] += rt.ghat[rows, k][:, None] * out", "y[rows] += rt.g[rows, k][:, None] * out")],
    # ties broken toward the higher index
    "ties_high": ('order = np.argsort(-r32[t], kind="stable")[:K]',
                  'order = (E - 1 - np.argsort(-r32[t][::-1], kind="stable"))[:K]'),
    # ascending instead of descending
    "ascending": ('order = np.argsort(-r32[t], kind="stable")[:K]', 'order = np.argsort(r32[t], kind="stable")[:K]'),
    # silu replaced by sigmoid
    "sigmoid_not_silu": ("return a / (1.0 + np.exp(-a))", "return 1.0 / (1.0 + np.exp(-a))"),
    # gate and up swapped inside silu
    "gate_up_swapped": ("h = silu(X @ wg.T) * (X @ wu.T)", "h = silu(X @ wu.T) * (X @ wg.T)"),
    # shared experts dropped
    "no_shared": ("for s in range(cfg.S):\n        y +=", "for s in range(0):\n        y +="),
    # router bias dropped
    "no_router_bias": ("r = r + np.asarray(layer.b_router, dtype=np.float64)", "r = r"),
    # mask bias sign flipped
    "mask_bias_sign": ("z = z + np.asarray(layer.b_mask, dtype=np.float64)", "z = z - np.asarray(layer.b_mask, dtype=np.float64)"),
    # down projection not transposed (wrong operand orientation)
    "down_no_transpose": ("return h @ wd.T", "return (h @ wd.reshape(wd.shape[1], wd.shape[0]))"),
    # mask applied to the router logit instead of the mask logit
    "mask_from_router": ("keep[t] = z32[t, order] >= np.float32(0.0)", "keep[t] = r32[t, order] >= np.float32(0.0)"),
    # bf16 widening drops the shift
    "widen_wrong": ("(a.astype(np.uint32) << np.uint32(16))", "(a.astype(np.uint32) << np.uint32(15))"),
    # E4M3 exponent bias 8 instead of 7
    "e4m3_bias8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    # E4M3 exponent field 0 decoded as a normal number
    "e4m3_no_subnormals": ("np.where(e == 0, m * 2.0 ** -9,", "np.where(e < 0, m * 2.0 ** -9,"),
    # every code with exponent field 15 taken as NaN (as in formats with infinities)
    "e4m3_top_binade_nan": ("np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)",
                            "np.where(e == 15, np.nan, mag)"),
    # FP8 row scales not applied
    "fp8_no_scale": ("return decode_e4m3(a) * np.asarray(scale, dtype=np.float64)[:, None]",
                     "return decode_e4m3(a)"),
    # FP8 scale applied per input column (broadcast over the other axis)
    "fp8_scale_columns": ("return decode_e4m3(a) * np.asarray(scale, dtype=np.float64)[:, None]",
                          "return decode_e4m3(a) * np.resize(np.asarray(scale, dtype=np.float64), a.shape[1])[None, :]"),
    # shared experts read the routed experts' scales
    "fp8_shared_uses_routed_scales": ('"s" + name[1:] if name.startswith("ws_")', '"s_" + name[3:] if name.startswith("ws_")'),
    # segment routing ignored
    "segment_ignored": ("return tokens - tokens % S if S > 1 else tokens", "return tokens"),
    # segment decided by its second token
    "segment_second_token": ("return tokens - tokens % S if S > 1 else tokens",
                             "return np.minimum(tokens - tokens % S + 1, tokens) if S > 1 else tokens"),
    # heads computed on positions within a token sample instead of token indices
    "segment_sample_positions": ("src = segment_heads(tok, getattr(cfg, \"segment\", 0))",
                                 "src = tok[segment_heads(np.arange(len(tok)), getattr(cfg, \"segment\", 0))]"),
    # binary gates normalised over K
    "binary_over_k": ("            g[t] = 1.0\n", "            g[t] = 1.0 / K\n"),
    # Avg-K counts all top-K slots
    "avgk_topk": ('"avg_k": (P / T) if T > 0 else 0.0', '"avg_k": (cfg.K if T > 0 else 0.0)'),
    # bytes: every routed expert counted, active or not
    "bytes_all_experts": ('"bytes_active_expert_weights": float(per_routed * active + per_shared * cfg.S)',
                          '"bytes_active_expert_weights": float(per_routed * cfg.E + per_shared * cfg.S)'),
    # bytes: one router matrix instead of two
    "bytes_one_router": ("+ 2.0 * cfg.E * D * elt          # router + mask-router weights",
                         "+ 1.0 * cfg.E * D * elt          # router + mask-router weights"),
    # bytes: FP8 row scales left out
    "bytes_fp8_no_scales": ("per_routed = 3 * D * I + 4 * (2 * I + D) if fp8 else 3 * D * I * elt",
                            "per_routed = 3 * D * I if fp8 else 3 * D * I * elt"),
}


def test_real_copy_passes_all_pins():
    mod = _copy()
    for pin in ALL_PINS[:2]:
        pin(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    edits = MUTANTS[name]
    mod = _src_mutant(*(edits if isinstance(edits, list) else [edits]))
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"mutant {name} passed every pin"
