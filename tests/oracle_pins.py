"""Pins for the oracle: checks against facts fixed by the method's definition,
not by the oracle's own code.

Each pin takes the oracle module as an argument so that the same checks can be
run against deliberately broken copies of it (tests/test_oracle_mutants.py):
every plausible mistake must make at least one pin fail.

Independent computations used here are written with torch (float64, CPU):
torch.topk + torch.softmax + torch.sigmoid + torch.nn.functional.silu, i.e.
library routines, never the oracle's functions.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import json
import os

from common import (GOLDEN, eval_closed_form, layer_from_json, small_config, with_mask)
import synth


# --------------------------------------------------------------------------
# Independent torch computations (library special cases)
# --------------------------------------------------------------------------

def _t(a, dtype):
    """float64 torch tensor of stored inputs (bf16 bits or float32)."""
    a = np.asarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(a.astype(np.float32)).to(torch.float64)


def torch_logits(layer, x):
    dt = layer.cfg.dtype
    X = _t(x, dt)
    r = torch.matmul(X, _t(layer.w_router, dt).t())
    z = torch.matmul(X, _t(layer.w_mask, dt).t())
    if layer.b_router is not None:
        r = r + torch.from_numpy(np.asarray(layer.b_router, np.float64))
    if layer.b_mask is not None:
        z = z + torch.from_numpy(np.asarray(layer.b_mask, np.float64))
    # decisions on float32 logits
    return r.to(torch.float32).to(torch.float64), z.to(torch.float32).to(torch.float64)


def torch_dense_gates(layer, x, use_mask=True):
    """G[t][e]: masked top-K softmax gate of expert e for token t (0 elsewhere).
    Gate options of layer.cfg.gating: bit 1 takes the softmax over all E and
    reads it at the top-K experts; bit 2 renormalises the masked gates; bit 4
    gives every top-K expert gate 1.  With layer.cfg.segment = S > 1 every
    token takes the gates and experts of token t - t % S."""
    r, z = torch_logits(layer, x)
    S = getattr(layer.cfg, "segment", 0)
    if S > 1:
        head = torch.arange(r.shape[0]) // S * S
        r, z = r[head], z[head]
    K = layer.cfg.K
    gating = getattr(layer.cfg, "gating", 0)
    vals, idx = torch.topk(r, K, dim=1)
    if gating & 4:
        g = torch.ones_like(vals)
    elif gating & 1:
        g = torch.gather(torch.softmax(r, dim=1), 1, idx)
    else:
        g = torch.softmax(vals, dim=1)
    if use_mask:
        m = (torch.sigmoid(torch.gather(z, 1, idx)) >= 0.5).to(torch.float64)
        g = g * m
    if gating & 2:
        s = g.sum(dim=1, keepdim=True)
        g = torch.where(s > 0, g / torch.where(s > 0, s, torch.ones_like(s)), torch.zeros_like(g))
    G = torch.zeros_like(r)
    G.scatter_(1, idx, g)
    return G, idx


def with_gating(layer, gating):
    """The same layer with other gate options."""
    from dataclasses import replace
    return replace(layer, cfg=replace(layer.cfg, gating=gating))


def with_segment(layer, S, gating=None):
    """The same layer with segment routing of S tokens (and other gate options)."""
    from dataclasses import replace
    kw = {"segment": S}
    if gating is not None:
        kw["gating"] = gating
    return replace(layer, cfg=replace(layer.cfg, **kw))


def torch_e4m3(codes):
    """float64 values of E4M3 codes by torch's own float8_e4m3fn type."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64)


def torch_weights(layer, e, shared=False):
    """(Wg, Wu, Wd) in float64: stored values, or E4M3 codes times row scales."""
    dt = layer.cfg.dtype
    names = ("ws_gate", "ws_up", "ws_down") if shared else ("w_gate", "w_up", "w_down")
    out = []
    for n in names:
        a = getattr(layer, n)[e]
        if getattr(layer.cfg, "expert_format", "") == "fp8":
            sc = getattr(layer, ("ss_" if shared else "s_") + n.split("_")[1])[e]
            out.append(torch_e4m3(a) * torch.from_numpy(np.asarray(sc, np.float64)).unsqueeze(1))
        else:
            out.append(_t(a, dt))
    return out


def torch_expert(layer, e, X, shared=False):
    wg, wu, wd = torch_weights(layer, e, shared)
    h = F.silu(X @ wg.t()) * (X @ wu.t())
    return h @ wd.t()


def torch_dense_forward(layer, x, use_mask=True):
    """Brute force: y = sum over ALL experts of G[:, e] * E_e(x) + shared."""
    X = _t(x, layer.cfg.dtype)
    G, _ = torch_dense_gates(layer, x, use_mask)
    y = torch.zeros(X.shape[0], layer.cfg.D, dtype=torch.float64)
    for e in range(layer.cfg.E):
        y += G[:, e:e + 1] * torch_expert(layer, e, X)
    for s in range(layer.cfg.S):
        y += torch_expert(layer, s, X, shared=True)
    return y.numpy()


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


# --------------------------------------------------------------------------
# Small random layers (drawn with the shared seeded generator)
# --------------------------------------------------------------------------

def small_layer(tag, dtype="bf16", D=96, E=10, K=3, I=40, S=0, I_s=0, keep=0.5, router_bias=False):
    cfg = small_config("pin:" + tag, dtype, D, E, K, I, S, I_s, keep, router_bias)
    return synth.make_layer(cfg)


def small_x(layer, T, tag="x"):
    from common import enforce_margins
    return enforce_margins(layer, synth.make_x(layer.cfg, T, tag), T, tag)


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_golden_routed(O):
    """Hand-derived worked example: idx, mask bits, g, g_hat, counts, Avg-K, y."""
    j, layer, x = layer_from_json("worked_example_routed.json")
    rt, y = O.forward(layer, x)
    ex = j["expect"]
    assert np.array_equal(rt.idx, np.array(ex["idx"])), rt.idx
    assert np.array_equal(rt.mask_bits, np.array(ex["mask_bits"], np.uint32)), rt.mask_bits
    g = np.vectorize(eval_closed_form)(np.array(ex["g"], dtype=object)).astype(float)
    gh = np.vectorize(eval_closed_form)(np.array(ex["ghat"], dtype=object)).astype(float)
    assert np.allclose(rt.g, g, rtol=0, atol=1e-7), rt.g
    assert np.allclose(rt.ghat, gh, rtol=0, atol=1e-7), rt.ghat
    assert np.array_equal(O.expert_counts(rt, layer.cfg.E), np.array(ex["counts"]))
    st = O.layer_stats(layer.cfg, O.expert_counts(rt, layer.cfg.E), x.shape[0])
    assert abs(st["avg_k"] - eval_closed_form(ex["avg_k"])) < 1e-15
    yy = np.vectorize(eval_closed_form)(np.array(ex["y"], dtype=object)).astype(float)
    assert np.allclose(y, yy, rtol=0, atol=1e-6), (y, yy)
    assert np.all(y[2] == 0.0)   # all candidates masked: exact zero


def pin_golden_shared(O):
    """Worked example with an always-on shared expert."""
    j, layer, x = layer_from_json("worked_example_shared.json")
    rt, y = O.forward(layer, x)
    ex = j["expect"]
    assert np.array_equal(rt.idx, np.array(ex["idx"]))
    assert np.array_equal(rt.mask_bits, np.array(ex["mask_bits"], np.uint32))
    assert np.array_equal(O.expert_counts(rt, layer.cfg.E), np.array(ex["counts"]))
    yy = np.vectorize(eval_closed_form)(np.array(ex["y"], dtype=object)).astype(float)
    assert np.allclose(y, yy, rtol=0, atol=1e-6), (y, yy)


def pin_golden_gating(O):
    """Hand-derived worked example of the gate options (softmax over all E;
    renormalised masked gates; both), on the routed example's inputs."""
    j, layer0, x = layer_from_json("worked_example_routed.json")
    with open(os.path.join(GOLDEN, "worked_example_gating.json")) as f:
        jg = json.load(f)
    ev = lambda a: np.vectorize(eval_closed_form)(np.array(a, dtype=object)).astype(float)  # noqa: E731
    for flags, ex in jg["expect"].items():
        layer = with_gating(layer0, int(flags))
        rt, y = O.forward(layer, x)
        assert np.array_equal(rt.idx, np.array(j["expect"]["idx"])), (flags, rt.idx)
        assert np.array_equal(rt.mask_bits, np.array(j["expect"]["mask_bits"], np.uint32))
        assert np.allclose(rt.g, ev(ex["g"]), rtol=0, atol=1e-7), (flags, rt.g)
        assert np.allclose(rt.ghat, ev(ex["ghat"]), rtol=0, atol=1e-7), (flags, rt.ghat)
        assert np.allclose(y, ev(ex["y"]), rtol=0, atol=1e-6), (flags, y)
        assert np.all(y[2] == 0.0)


def pin_gate_options_vs_torch(O):
    """Gate options against torch (softmax over all E gathered at torch.topk;
    renormalisation of the masked gates), gates and the dense brute-force y."""
    base = small_layer("gating", D=64, E=9, K=4, I=24, S=1, I_s=16, keep=0.45, router_bias=True)
    x = small_x(base, 12, "gating")
    for flags in (1, 2, 3, 4, 6):
        layer = with_gating(base, flags)
        G, idx = torch_dense_gates(layer, x)
        rt = O.route(layer, x)
        assert np.array_equal(rt.idx, idx.numpy())
        assert _rel(rt.ghat, torch.gather(G, 1, idx).numpy()) < 1e-12, flags
        _, y = O.forward(layer, x)
        assert _rel(y, torch_dense_forward(layer, x)) < 1e-9, flags
        if flags & 2:
            s = rt.ghat.sum(axis=1)
            kept = rt.keep.any(axis=1)
            assert np.allclose(s[kept], 1.0, atol=1e-12) and np.all(s[~kept] == 0.0)


def pin_golden_segment(O):
    """Hand-derived worked example of segment routing (S = 2), with the
    method's own gate and with binary gates."""
    j, layer0, x = layer_from_json("worked_example_routed.json")
    with open(os.path.join(GOLDEN, "worked_example_segment.json")) as f:
        js = json.load(f)
    ev = lambda a: np.vectorize(eval_closed_form)(np.array(a, dtype=object)).astype(float)  # noqa: E731
    ex = js["expect"]
    layer = with_segment(layer0, js["segment"])
    rt, y = O.forward(layer, x)
    assert np.array_equal(rt.idx, np.array(ex["idx"])), rt.idx
    assert np.array_equal(rt.mask_bits, np.array(ex["mask_bits"], np.uint32))
    assert np.allclose(rt.ghat, ev(ex["ghat"]), rtol=0, atol=1e-7)
    assert np.array_equal(O.expert_counts(rt, 3), np.array(ex["counts"]))
    assert np.allclose(y, ev(ex["y"]), rtol=0, atol=1e-6), y
    _, yb = O.forward(with_segment(layer0, js["segment"], 4), x)
    assert np.allclose(yb, ev(ex["y_binary"]), rtol=0, atol=1e-6), yb


def pin_segment_vs_torch(O):
    """Segment routing (S = 4 and 16 over ragged batches; with the method's
    gate, binary gates, and binary + renormalised) against torch: top-K,
    softmax and mask of each segment's first token, dense brute-force y."""
    base = small_layer("segment", D=64, E=10, K=3, I=24, S=1, I_s=16, keep=0.5, router_bias=True)
    x = small_x(base, 23, "segment")
    for S, flags in ((4, 0), (4, 4), (16, 6), (5, 2)):
        layer = with_segment(base, S, flags)
        G, idx = torch_dense_gates(layer, x)
        rt = O.route(layer, x)
        assert np.array_equal(rt.idx, idx.numpy()), (S, flags)
        assert _rel(rt.ghat, torch.gather(G, 1, idx).numpy()) < 1e-12, (S, flags)
        _, y = O.forward(layer, x)
        assert _rel(y, torch_dense_forward(layer, x)) < 1e-9, (S, flags)


def pin_segment_properties(O):
    """S <= 1 is per-token routing; S >= T gives every token token 0's
    experts and mask; routing a sample of tokens equals routing them within
    the whole batch; a batch whose segments repeat one token routes exactly
    as per-token routing."""
    base = small_layer("segprop", D=48, E=8, K=2, I=16, keep=0.5)
    x = small_x(base, 13, "segprop")
    rt0 = O.route(base, x)
    for S in (0, 1):
        rt = O.route(with_segment(base, S), x)
        assert np.array_equal(rt.idx, rt0.idx) and np.array_equal(rt.ghat, rt0.ghat)
    rt = O.route(with_segment(base, 64), x)
    assert np.all(rt.idx == rt0.idx[0]) and np.all(rt.mask_bits == rt0.mask_bits[0])
    lay3 = with_segment(base, 3)
    _, yall = O.forward(lay3, x)
    toks = np.array([12, 4, 7, 1])
    rts, ys = O.forward(lay3, x, tokens=toks)
    assert np.array_equal(rts.idx, O.route(lay3, x).idx[toks])
    assert np.allclose(ys, yall[toks], rtol=0, atol=1e-12)
    rep = x[np.arange(12) // 3 * 3]           # every segment of 3 repeats its first token
    rt_seg, y_seg = O.forward(lay3, rep)
    rt_tok, y_tok = O.forward(base, rep)
    assert np.array_equal(rt_seg.idx, rt_tok.idx) and np.array_equal(y_seg, y_tok)


def pin_gate_options_identity(O):
    """With every candidate kept (Wm = 0), softmax over all E read at the top K
    and then renormalised over the K equals the softmax over the K logits."""
    base = with_mask(small_layer("gate_id", D=48, E=7, K=3, I=16), True, 0.0)
    x = small_x(base, 10, "gate_id")
    rt0, y0 = O.forward(base, x)
    rt3, y3 = O.forward(with_gating(base, 3), x)
    assert np.array_equal(rt0.idx, rt3.idx)
    assert _rel(rt3.ghat, rt0.ghat) < 1e-12 and _rel(y3, y0) < 1e-12
    rt1 = O.route(with_gating(base, 1), x)
    assert np.all(rt1.g.sum(axis=1) < 1.0)   # K < E: part of the mass is outside the top K


def pin_mask_backward_autograd(O):
    """Mask-router gradient against torch autograd of the straight-through
    surrogate (m replaced by m_hat in y, so dm/dm_hat = 1) plus beta * L_reg,
    L_reg = mean over tokens of (1/K) sum_{i in TK} m_hat_i."""
    layer = small_layer("mbwd", D=48, E=7, K=3, I=20, S=1, I_s=12, keep=0.5, router_bias=True)
    T, beta = 9, 0.37
    x = small_x(layer, T, "mbwd")
    dy = np.random.default_rng(11).standard_normal((T, layer.cfg.D))
    lreg, dwm, dbm, _ = O.mask_router_backward(layer, x, dy, beta)
    dt = layer.cfg.dtype
    X = _t(x, dt)
    r, _ = torch_logits(layer, x)
    _, idx = torch.topk(r, layer.cfg.K, dim=1)
    g = torch.softmax(torch.gather(r, 1, idx), dim=1)
    Wm = _t(layer.w_mask, dt).clone().requires_grad_(True)
    bm0 = np.zeros(layer.cfg.E) if layer.b_mask is None else np.asarray(layer.b_mask, np.float64)
    bm = torch.from_numpy(bm0).clone().requires_grad_(True)
    z = X @ Wm.t() + bm
    mh = torch.sigmoid(torch.gather(z, 1, idx))
    y = torch.zeros(T, layer.cfg.D, dtype=torch.float64)
    for t in range(T):
        for k in range(layer.cfg.K):
            y[t] += g[t, k] * mh[t, k] * torch_expert(layer, int(idx[t, k]), X[t:t + 1])[0]
    L_reg = mh.sum() / (T * layer.cfg.K)
    L = (torch.from_numpy(dy) * y).sum() + beta * L_reg
    L.backward()
    assert abs(lreg - float(L_reg.detach())) < 1e-7
    assert _rel(dwm, Wm.grad.numpy()) < 1e-6, _rel(dwm, Wm.grad.numpy())
    assert _rel(dbm, bm.grad.numpy()) < 1e-6


def pin_mask_backward_zero_router(O):
    """Zero-initialised mask router (Wm = 0, b_m = 0): m_hat = 1/2 exactly, so
    L_reg = 1/2, and with dL/dy = 0 every candidate gets dL/dz = beta/(T K) / 4."""
    layer = with_mask(small_layer("mbwd0", D=32, E=6, K=2, I=16), True, 0.0)
    T, beta = 5, 0.8
    x = small_x(layer, T, "mbwd0")
    lreg, dwm, dbm, dz = O.mask_router_backward(layer, x, np.zeros((T, layer.cfg.D)), beta)
    assert lreg == 0.5
    c = beta / (T * layer.cfg.K) * 0.25
    assert np.all(dz == c)
    r, _ = torch_logits(layer, x)
    _, idx = torch.topk(r, layer.cfg.K, dim=1)
    X = _t(x, layer.cfg.dtype).numpy()
    ref = np.zeros((layer.cfg.E, layer.cfg.D))
    cnt = np.zeros(layer.cfg.E)
    for t in range(T):
        for e in idx[t].numpy():
            ref[e] += c * X[t]
            cnt[e] += 1
    assert np.allclose(dwm, ref, rtol=0, atol=1e-15) and np.allclose(dbm, c * cnt, rtol=0, atol=1e-15)


def pin_zero_mask_router_is_topk(O):
    """Wm = 0 (zero-initialised mask router): m_hat = 0.5 everywhere, every
    top-K expert is kept, and the layer equals plain top-K MoE (torch)."""
    for tag, kw in (("zm_bf16", dict(dtype="bf16", D=64, E=12, K=3, I=48)),
                    ("zm_f32", dict(dtype="f32", D=40, E=6, K=2, I=24, S=1, I_s=16)),
                    ("zm_k1", dict(dtype="bf16", D=32, E=5, K=1, I=20))):
        layer = with_mask(small_layer(tag, **kw), w_mask_zero=True)
        layer = with_mask(layer, b_mask=0.0)
        x = small_x(layer, 17)
        rt, y = O.forward(layer, x)
        assert rt.keep.all()
        assert np.all(rt.mask_bits == (1 << layer.cfg.K) - 1)
        ref = torch_dense_forward(layer, x, use_mask=False)
        assert _rel(y, ref) < 1e-12, (tag, _rel(y, ref))
        G, idx = torch_dense_gates(layer, x, use_mask=False)
        assert np.array_equal(rt.idx, idx.numpy()), tag


def pin_dense_bruteforce(O):
    """Brute-force dense sum over all E experts with masked gates (zeros for
    non-candidates and masked candidates) equals the oracle's sparse forward."""
    for tag, kw in (("bf_bf16", dict(dtype="bf16", D=64, E=9, K=4, I=32, S=2, I_s=16, keep=0.4)),
                    ("bf_f32", dict(dtype="f32", D=48, E=7, K=3, I=24, keep=0.6)),
                    ("bf_bias", dict(dtype="bf16", D=64, E=16, K=5, I=16, keep=0.2, router_bias=True))):
        layer = small_layer(tag, **kw)
        x = small_x(layer, 23)
        rt, y = O.forward(layer, x)
        ref = torch_dense_forward(layer, x, use_mask=True)
        assert _rel(y, ref) < 1e-12, (tag, _rel(y, ref))
        G, idx = torch_dense_gates(layer, x, use_mask=True)
        assert np.array_equal(rt.idx, idx.numpy()), tag
        Gs = np.zeros((x.shape[0], layer.cfg.E))
        np.put_along_axis(Gs, rt.idx.astype(np.int64), rt.ghat, axis=1)
        assert np.abs(Gs - G.numpy()).max() < 1e-12, tag


def pin_avgk_popcount(O):
    """Avg-K = popcount(mask)/T = sum_e c_e / T (exact integers)."""
    layer = small_layer("avgk", D=64, E=20, K=6, I=8, keep=0.3)
    x = small_x(layer, 50)
    rt = O.route(layer, x)
    pop = sum(bin(int(b)).count("1") for b in rt.mask_bits)
    c = O.expert_counts(rt, layer.cfg.E)
    assert int(c.sum()) == pop == int(rt.keep.sum())
    st = O.layer_stats(layer.cfg, c, 50)
    assert st["avg_k"] == pop / 50
    assert st["active_pairs"] == pop
    # FLOPs(BEAM) / FLOPs(top-K) = Avg-K / K, compared as exact integer products
    assert st["flops_routed"] * 50 * layer.cfg.K == st["flops_topk_routed"] * pop


def pin_mask_bias_extremes(O):
    """b_m = -1e4: every candidate masked, y = shared part only (0 without shared).
    b_m = +1e4: every candidate kept, y equals the Wm = 0 layer."""
    for tag, kw in (("ext_noshared", dict(D=64, E=8, K=2, I=32)),
                    ("ext_shared", dict(D=64, E=8, K=3, I=32, S=2, I_s=24))):
        base = small_layer(tag, **kw)
        x = small_x(base, 11)
        lo = with_mask(base, b_mask=-1e4)
        rt, y = O.forward(lo, x)
        assert not rt.keep.any() and np.all(rt.mask_bits == 0)
        if base.cfg.S == 0:
            assert np.all(y == 0.0)
        else:
            X = _t(x, "bf16")
            sh = sum(torch_expert(base, s, X, shared=True) for s in range(base.cfg.S)).numpy()
            assert _rel(y, sh) < 1e-12
        hi = with_mask(base, b_mask=1e4)
        zero = with_mask(with_mask(base, w_mask_zero=True), b_mask=0.0)
        _, y_hi = O.forward(hi, x)
        _, y_zero = O.forward(zero, x)
        assert _rel(y_hi, y_zero) < 1e-15


def pin_k1(O):
    """K = 1: the softmax of one logit is exactly 1, so y = m * E_argmax(x)."""
    layer = small_layer("k1", D=64, E=7, K=1, I=24, keep=0.5)
    x = small_x(layer, 19)
    rt, y = O.forward(layer, x)
    assert np.all(rt.g == 1.0)
    r, _ = torch_logits(layer, x)
    am = torch.argmax(r, dim=1).numpy()
    assert np.array_equal(rt.idx[:, 0], am)
    X = _t(x, "bf16")
    for t in range(x.shape[0]):
        ref = torch_expert(layer, int(am[t]), X[t:t + 1]).numpy()[0] * float(rt.keep[t, 0])
        assert np.abs(y[t] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def pin_k_equals_e(O):
    """K = E: the top-K is a full descending sort of the logits."""
    layer = small_layer("kfull", dtype="f32", D=32, E=8, K=8, I=8)
    x = small_x(layer, 13)
    rt = O.route(layer, x)
    r, _ = torch_logits(layer, x)
    srt = torch.sort(r, dim=1, descending=True, stable=True).indices.numpy()
    assert np.array_equal(rt.idx, srt)


def pin_gate_properties(O):
    """sum_k g_k = 1 and g is non-increasing in k; g_hat = g on kept slots, 0 elsewhere."""
    layer = small_layer("gates", D=64, E=30, K=8, I=8, keep=0.5, router_bias=True)
    x = small_x(layer, 40)
    rt = O.route(layer, x)
    assert np.abs(rt.g.sum(axis=1) - 1.0).max() < 1e-12
    assert np.all(np.diff(rt.g, axis=1) <= 0.0)
    assert np.array_equal(rt.ghat, np.where(rt.keep, rt.g, 0.0))
    assert np.all(rt.ghat.sum(axis=1) <= 1.0 + 1e-12)


def pin_threshold_is_sigmoid_half(O):
    """m = [sigmoid(z) >= 0.5] on the candidates, checked with torch.sigmoid."""
    layer = small_layer("thr", D=64, E=16, K=6, I=8, keep=0.35)
    x = small_x(layer, 64)
    rt = O.route(layer, x)
    _, z = torch_logits(layer, x)
    zc = torch.gather(z, 1, torch.from_numpy(rt.idx.astype(np.int64)))
    assert np.array_equal(rt.keep, (torch.sigmoid(zc) >= 0.5).numpy())


def pin_batch_invariance(O):
    """Routing and output of each token computed alone equal the batched ones."""
    layer = small_layer("batch", D=48, E=9, K=3, I=16, S=1, I_s=8, keep=0.5)
    x = small_x(layer, 9)
    rt, y = O.forward(layer, x)
    for t in range(9):
        rt1, y1 = O.forward(layer, x[t:t + 1])
        assert np.array_equal(rt1.idx[0], rt.idx[t])
        assert rt1.mask_bits[0] == rt.mask_bits[t]
        assert np.abs(y1[0] - y[t]).max() <= 1e-12 * max(1.0, np.abs(y[t]).max())


def pin_expert_permutation(O):
    """Permuting every per-expert tensor consistently permutes the indices and
    leaves g, m and y unchanged."""
    layer = small_layer("perm", D=48, E=11, K=4, I=16, keep=0.5, router_bias=True)
    x = small_x(layer, 15)
    rt, y = O.forward(layer, x)
    p = np.random.default_rng(7).permutation(layer.cfg.E)   # new expert j = old p[j]
    inv = np.argsort(p)
    from dataclasses import replace
    lp = replace(layer, w_router=layer.w_router[p], w_mask=layer.w_mask[p],
                 b_router=layer.b_router[p], b_mask=None if layer.b_mask is None else layer.b_mask[p],
                 w_gate=layer.w_gate[p], w_up=layer.w_up[p], w_down=layer.w_down[p])
    rtp, yp = O.forward(lp, x)
    assert np.array_equal(p[rtp.idx], rt.idx)
    assert np.array_equal(inv[rt.idx], rtp.idx)
    assert np.array_equal(rtp.mask_bits, rt.mask_bits)
    assert np.abs(rtp.g - rt.g).max() == 0.0
    assert _rel(yp, y) < 1e-13


def pin_silu_closed_forms(O):
    """silu(0) = 0; silu(a) - silu(-a) = a; silu(1) = e/(1+e); large-|a| limits."""
    a = np.linspace(-30, 30, 601)
    s = O.silu(a)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.abs((s - O.silu(-a)) - a).max() < 1e-12
    assert abs(O.silu(np.array([1.0]))[0] - np.e / (1 + np.e)) < 1e-15
    assert abs(O.silu(np.array([-800.0]))[0]) == 0.0
    assert O.silu(np.array([800.0]))[0] == 800.0


def pin_widen_bf16(O):
    """bf16 bit patterns widen exactly: 0x3F80 = 1, 0xC000 = -2, 0x3EAB = 0.333984375."""
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    v = O.widen(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.333984375 and v[3] == 0.0
    assert v[5] == float.fromhex("0x1.fep+127")


def pin_e4m3_known_values(O):
    """E4M3 values fixed by the format (OCP 8-bit floating point, E4M3):
    1.0 = 0 0111 000, the largest finite 448 = S 1111 110, the smallest
    subnormal 2^-9 = 0 0000 001, the smallest normal 2^-6 = 0 0001 000,
    S 1111 111 is NaN, and exponent field 15 with m < 7 is finite."""
    codes = np.array([0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x07, 0x08, 0x3C, 0x77, 0x78,
                      0x00, 0x80, 0x7F, 0xFF, 0x3B, 0x30], dtype=np.uint8)
    v = O.decode_e4m3(codes)
    want = [1.0, -1.0, 448.0, -448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.5, 240.0, 256.0,
            0.0, -0.0]
    assert np.array_equal(v[:12], want)
    assert np.signbit(v[11]) and not np.signbit(v[10])
    assert np.isnan(v[12]) and np.isnan(v[13])
    assert v[14] == 1.375 and v[15] == 0.5


def pin_e4m3_vs_torch(O):
    """All 256 codes against torch's float8_e4m3fn conversion (NaN codes as NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    v = O.decode_e4m3(codes)
    ref = torch_e4m3(codes).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(v), nan)
    assert np.array_equal(v[~nan], ref[~nan])
    assert np.array_equal(np.signbit(v[~nan]), np.signbit(ref[~nan]))


def fp8_layer(tag, D=64, E=9, K=3, I=32, S=1, I_s=32, keep=0.5, router_bias=False):
    from dataclasses import replace
    cfg = replace(small_config("pin:" + tag, "bf16", D, E, K, I, S, I_s, keep, router_bias),
                  expert_format="fp8")
    return synth.make_layer(cfg)


def pin_fp8_layer_vs_torch(O):
    """A layer with E4M3 expert weights and row scales (routed and shared):
    the oracle's forward equals the torch brute-force dense sum whose weights
    are torch's float8_e4m3fn values times the row scales."""
    for tag, kw in (("fp8_a", dict(D=64, E=9, K=3, I=32, S=2, I_s=32, keep=0.5)),
                    ("fp8_b", dict(D=32, E=6, K=2, I=48, S=0, I_s=0, keep=0.7, router_bias=True))):
        layer = fp8_layer(tag, **kw)
        assert layer.w_gate.dtype == np.uint8
        x = small_x(layer, 19)
        rt, y = O.forward(layer, x)
        ref = torch_dense_forward(layer, x, use_mask=True)
        assert _rel(y, ref) < 1e-12, (tag, _rel(y, ref))
        st = O.layer_stats(layer.cfg, O.expert_counts(rt, layer.cfg.E), x.shape[0])
        c = layer.cfg
        act = int((O.expert_counts(rt, c.E) > 0).sum())
        assert st["bytes_active_expert_weights"] == act * (3 * c.D * c.I + 4 * (2 * c.I + c.D)) + \
            c.S * (3 * c.D * c.I_s + 4 * (2 * c.I_s + c.D))


def pin_stats_formulas(O):
    """FLOPs and bytes: FLOPs(BEAM)/FLOPs(top-K) = AvgK/K; per-expert SwiGLU
    cost 6*D*I per pair; bytes count each active expert once."""
    cfg = small_config("stats", "bf16", D=10, E=4, K=2, I=3, S=1, I_s=5)
    st = O.layer_stats(cfg, np.array([3, 0, 1, 0]), 4)
    assert st["active_pairs"] == 4 and st["active_experts"] == 2 and st["avg_k"] == 1.0
    assert st["flops_routed"] == 6 * 10 * 3 * 4
    assert st["flops_topk_routed"] == 6 * 10 * 3 * 4 * 2
    assert st["flops_reduction"] == 0.5
    assert st["flops_shared"] == 6 * 10 * 5 * 1 * 4
    assert st["flops_router"] == 4 * 4 * 10 * 4
    assert st["bytes_active_expert_weights"] == 3 * 10 * 3 * 2 * 2 + 3 * 10 * 5 * 2


def pin_stats_bytes_from_arrays(O):
    """The byte counts against the parameter arrays themselves: every expert
    with at least one surviving pair contributes the nbytes of its three
    matrices (FP8: codes and row scales), the shared experts theirs, and the
    total adds both router matrices, x and y -- for bf16, fp32 and FP8
    layers, with the counts taken from the oracle's own routing."""
    cases = [small_layer("bytes_bf16", "bf16", D=64, E=12, K=3, I=40, S=1, I_s=24, keep=0.3),
             small_layer("bytes_f32", "f32", D=32, E=6, K=2, I=16, keep=0.6),
             fp8_layer("bytes_fp8", D=64, E=9, K=3, I=32, S=2, I_s=32, keep=0.4)]
    for layer in cases:
        x = small_x(layer, 7)
        rt = O.route(layer, x)
        counts = O.expert_counts(rt, layer.cfg.E)
        st = O.layer_stats(layer.cfg, counts, x.shape[0])
        scales = [layer.s_gate, layer.s_up, layer.s_down]
        routed = 0
        for e in np.nonzero(counts > 0)[0]:
            routed += layer.w_gate[e].nbytes + layer.w_up[e].nbytes + layer.w_down[e].nbytes
            routed += sum(a[e].nbytes for a in scales if a is not None)
        shared = sum(a.nbytes for a in (layer.ws_gate, layer.ws_up, layer.ws_down,
                                        layer.ss_gate, layer.ss_up, layer.ss_down)
                     if a is not None and a.size)
        assert st["bytes_active_expert_weights"] == routed + shared, layer.cfg.name
        total = routed + shared + layer.w_router.nbytes + layer.w_mask.nbytes + 2 * x.nbytes
        assert st["bytes_total_min"] == total, layer.cfg.name
        assert 0 < (counts > 0).sum() < layer.cfg.E or layer.cfg.E <= 6, "some experts idle"


ALL_PINS = [
    pin_golden_routed, pin_golden_shared, pin_golden_gating, pin_gate_options_vs_torch,
    pin_gate_options_identity, pin_mask_backward_autograd, pin_mask_backward_zero_router,
    pin_zero_mask_router_is_topk, pin_dense_bruteforce,
    pin_avgk_popcount, pin_mask_bias_extremes, pin_k1, pin_k_equals_e, pin_gate_properties,
    pin_threshold_is_sigmoid_half, pin_batch_invariance, pin_expert_permutation,
    pin_silu_closed_forms, pin_widen_bf16, pin_stats_formulas, pin_stats_bytes_from_arrays,
    pin_e4m3_known_values, pin_e4m3_vs_torch, pin_fp8_layer_vs_torch,
    pin_golden_segment, pin_segment_vs_torch, pin_segment_properties,
]
