"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Routing (top-K indices, mask bits, per-expert counts) must match bit for bit;
gates within 1e-5; the layer output within max|err| <= 2e-2 max|y_ref| (bf16)
or 1e-5 max|y_ref| (fp32).  Full-size workloads compare routing on every
token and y on a sample of tokens (the oracle computes those one by one).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from common import (GOLDEN, cached_layer, inputs, layer_from_json, small_config, with_mask)
from gpu_helpers import (check_output, check_routing, device_layer, note, padded_layer,
                         run_forward, run_route, sample_tokens)
from gpu_helpers import _dev_cache as _gpu_dev_cache
from dynamic_expert_masking_amd.device import to_device, to_host_bits
import dynamic_expert_masking_amd as dm


def _dev_cache_clear():
    """Frees the cached device layer (the packed tests hold a second copy)."""
    _gpu_dev_cache.clear()
    torch.cuda.empty_cache()
from oracle_pins import small_layer, small_x

pytestmark = pytest.mark.gpu

CASES = [(n, T) for n in synth.CONFIG_ORDER for T in synth.CONFIGS[n].tokens]
# Largest batch for which every token's output is compared with the oracle
# (the oracle's per-expert products make these seconds).  Beyond it (the
# Mixtral-shaped layer at T=2048, 1.4 TFLOP in float64) the compared tokens
# include at least one row of every 32-row block of every expert's rows in
# the expert-major pair order, so that every tile and MFMA block of the
# expert kernels produces at least one compared output.
FULL_Y_MAX = {"tiny_f32": 64, "dsv2lite_decode": 256, "dsv2lite_prefill": 4096, "mixtral": 32,
              "finegrained": 8192, "dsv2lite_decode_fp8": 256}


def tile_cover_tokens(rt_ref, E: int, T: int, block: int = 32, seed: int = 5) -> np.ndarray:
    """Tokens that cover every `block`-row block of every expert's rows in
    the expert-major pair order (the expert kernels' row order: experts
    ascending, tokens ascending within an expert), one random row of each
    block, plus the batch's first and last 8 tokens."""
    rng = np.random.default_rng(seed)
    toks = set(range(min(8, T))) | set(range(max(0, T - 8), T))
    keep = rt_ref.keep
    for e in range(E):
        rows = np.nonzero(((rt_ref.idx == e) & keep).any(axis=1))[0]   # ascending tokens
        for b0 in range(0, rows.size, block):
            blk = rows[b0:b0 + block]
            toks.add(int(blk[rng.integers(blk.size)]))
    return np.array(sorted(toks))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name,T", CASES, ids=[f"{n}-T{T}" for n, T in CASES])
def test_workload_parity(name, T):
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, T, layer)
    dl = device_layer(layer, key=name)
    note(f"[parity] {name} T={T} beam_moe_forward")
    y, rt, ys = run_forward(dl, x, reps=2)
    rt_ref = oracle.route(layer, x)
    check_routing(rt, rt_ref, cfg.E)
    assert np.array_equal(ys[0], ys[1]), "two identical calls gave different y"
    toks = np.arange(T) if T <= FULL_Y_MAX[name] else tile_cover_tokens(rt_ref, cfg.E, T)
    _, y_ref = oracle.forward(layer, x, tokens=toks)
    rel = check_output(y[toks], y_ref, cfg.dtype)
    note(f"[parity] {name} T={T}: avg_k={rt_ref.keep.sum() / T:.3f} rel_err={rel:.2e} "
         f"tokens_compared={len(toks)}")


@pytest.mark.parametrize("fname", ["worked_example_routed.json", "worked_example_shared.json"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_golden_examples(fname, dtype):
    """The hand-derived worked examples, zero-padded to D = 64, I = 64 (every
    value in them is exact in bf16 too)."""
    j, layer, x = layer_from_json(fname)
    big = padded_layer(layer, 64, 64, 64)
    xp = np.zeros((x.shape[0], 64), np.float32)
    xp[:, :2] = x
    if dtype == "bf16":
        conv = lambda a: None if a is None else synth.f32_to_bf16_bits(a)  # noqa: E731
        from dataclasses import replace
        big = replace(big, cfg=replace(big.cfg, dtype="bf16"),
                      **{k: conv(getattr(big, k)) for k in
                         ("w_router", "w_mask", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")})
        xp = synth.f32_to_bf16_bits(xp)
    note(f"[golden] {fname} {dtype}")
    y, rt, _ = run_forward(device_layer(big), xp)
    ex = j["expect"]
    assert np.array_equal(rt["topk_idx"], np.array(ex["idx"]))
    assert np.array_equal(rt["mask"], np.array(ex["mask_bits"], np.uint32))
    assert np.array_equal(rt["expert_count"], np.array(ex["counts"]))
    from common import eval_closed_form
    yy = np.vectorize(eval_closed_form)(np.array(ex["y"], dtype=object)).astype(float)
    tol = 1e-6 if dtype == "f32" else 1e-2
    assert np.abs(y[:, :2] - yy).max() <= tol * np.abs(yy).max()
    assert np.all(y[:, 2:] == 0.0)
    if fname == "worked_example_routed.json":
        assert np.all(y[2] == 0.0)


@pytest.mark.parametrize("T", [1, 37, 100, 129, 1638, 1639])
def test_ragged_batches(T):
    """Batch sizes that are not multiples of the 16/64-token blocks.  With
    K = 5, 1638 tokens (8190 selections) is the largest batch whose plan comes
    from per-expert token bitmaps in one workgroup (at most 8192 selections),
    1639 the smallest that takes the block ranks, scan and scatter kernels."""
    layer = small_layer("ragged", D=192, E=24, K=5, I=128, S=1, I_s=64, keep=0.45, router_bias=True)
    x = small_x(layer, T, "ragged")
    note(f"[ragged] T={T}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("T", [60, 150])
def test_shared_cooperative_tiles(T):
    """Shared experts taken as cooperative items (one shared tile per wave of
    a workgroup, the weight block streamed once): D = I = 1024 gives a 4-way
    k split in both expert kernels; 60 tokens are 4 shared tiles (gate/up
    cooperative, the last tile partial), 150 tokens 10 tiles (gate/up and
    down cooperative; the last group has two tiles, so two waves hold none)."""
    layer = small_layer("coop", D=1024, E=32, K=2, I=1024, S=2, I_s=256, keep=0.5)
    x = small_x(layer, T, "coop")
    note(f"[cooperative shared tiles] T={T}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("D", [128, 192])
def test_wide_tiles(D):
    """256-row tiles (the prefill kernels' tallest): 2100 tokens, 8 experts, top-2
    (525 candidates per expert); D = 128 and 192 give an even and an odd number
    of 64-wide k slices; I = 192 leaves the second 128-row block of
    intermediate rows half empty; the shared expert's last token tile is
    partial."""
    layer = small_layer(f"wide{D}", D=D, E=8, K=2, I=192, S=1, I_s=128, keep=0.8)
    x = small_x(layer, 2100, "wide")
    note(f"[wide tiles] D={D}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("T,S", [(1200, 2), (700, 0), (3000, 1)])
def test_split_down(T, S):
    """The prefill down product split over k (fp32 partials added by the
    combine): few tiles against the resident workgroups make every split
    count from 2 to 4 occur; two shared experts put a segment boundary inside
    a split's k range, and splits of fewer chunks than the split count get
    empty ranges (zero partials)."""
    layer = small_layer(f"split{S}", D=256, E=8, K=2, I=256, S=S, I_s=128 if S else 0, keep=0.7,
                        router_bias=True)
    x = small_x(layer, T, "split")
    note(f"[split down] T={T} S={S}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


def _packed_reference(w: np.ndarray) -> np.ndarray:
    """The packed operand layout of matrices w [mats][rows][cols] (bf16 bits),
    written out from its definition in the header: block (rb, kb) of 32 rows
    x 64 columns, then k-step s, lane l, element j."""
    mats, rows, cols = w.shape
    out = np.empty(w.size, dtype=w.dtype)
    kbs = cols // 64
    q = 0
    for m in range(mats):
        for rb in range(rows // 32):
            for kb in range(kbs):
                for s in range(4):
                    for l in range(64):
                        r = 32 * rb + l % 32
                        c = 64 * kb + 16 * s + 8 * (l // 32)
                        out[q:q + 8] = w[m, r, c:c + 8]
                        q += 8
    return out


def test_pack_weights_layout():
    """beam_moe_pack_weights against the layout's definition, element by element."""
    rng = np.random.default_rng(3)
    w = rng.integers(0, 1 << 16, size=(3, 64, 192), dtype=np.uint16)
    wd = to_device(w)
    out = torch.empty_like(wd)
    dm.beam_moe_pack_weights(wd, 3, 64, 192, out, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = to_host_bits(out).reshape(-1)
    assert np.array_equal(got, _packed_reference(w))


PACKED_CASES = [("mixtral", 2048), ("dsv2lite_prefill", 4096), ("finegrained", 8192), ("mixtral", 32),
                ("dsv2lite_decode", 256)]


@pytest.mark.parametrize("name,T", PACKED_CASES, ids=[f"{n}-T{T}" for n, T in PACKED_CASES])
def test_packed_weights_workloads(name, T):
    """The layer with packed copies of its expert weights: prefill-sized
    batches run the packed kernels (tiles of 128 rows; the Mixtral down
    product splits its k range), decode batches the streaming kernels on the
    row-major weights.  Routing exact; y on every token up to 8192 (Mixtral
    T=2048: a sample covering every 32-row block of every expert)."""
    from dynamic_expert_masking_amd.device import DeviceLayer
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, T, layer)
    _dev_cache_clear()
    dl = DeviceLayer(layer, pack=True)
    note(f"[packed weights] {name} T={T}")
    y, rt, ys = run_forward(dl, x, reps=2)
    rt_ref = oracle.route(layer, x)
    check_routing(rt, rt_ref, cfg.E)
    assert np.array_equal(ys[0], ys[1]), "two identical calls gave different y"
    toks = np.arange(T) if T <= FULL_Y_MAX[name] or name != "mixtral" else tile_cover_tokens(rt_ref, cfg.E, T)
    _, y_ref = oracle.forward(layer, x, tokens=toks)
    rel = check_output(y[toks], y_ref, cfg.dtype)
    note(f"[packed weights] {name} T={T}: rel_err={rel:.2e} tokens_compared={len(toks)}")
    del dl
    torch.cuda.empty_cache()


# The benchmark's launch configuration for the layers without shared
# experts, where the descriptor's Avg-K hint can change the kernels: it gives
# every layer its workload's Avg-K as expected_avg_k and the prefill-sized
# batches packed weight copies (fine-grained T = 512: 16-row streaming tiles
# instead of 64-row ones; T = 8192: the 128-row packed kernels instead of the
# expert-stationary ones).  Layers with shared experts choose the same kernels
# with or without the hint and are covered by the workload tests above.
HINT_CASES = [("finegrained", 16, False), ("finegrained", 512, False), ("finegrained", 8192, True),
              ("mixtral", 1, False), ("mixtral", 32, False), ("mixtral", 2048, True)]


@pytest.mark.parametrize("name,T,pack", HINT_CASES, ids=[f"{n}-T{T}" for n, T, _ in HINT_CASES])
def test_bench_configuration(name, T, pack):
    """Routing exact on every token, y on every token (Mixtral T = 2048: every
    32-row block of every expert), with the benchmark's Avg-K hint and packing."""
    from dynamic_expert_masking_amd.device import DeviceLayer
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, T, layer)
    _dev_cache_clear()
    dl = DeviceLayer(layer, pack=pack, avg_k_hint=cfg.avg_k_target)
    note(f"[bench configuration] {name} T={T} pack={pack} expected_avg_k={cfg.avg_k_target:.3f}")
    y, rt, ys = run_forward(dl, x, reps=2)
    rt_ref = oracle.route(layer, x)
    check_routing(rt, rt_ref, cfg.E)
    assert np.array_equal(ys[0], ys[1]), "two identical calls gave different y"
    toks = np.arange(T) if T <= FULL_Y_MAX[name] or name != "mixtral" else tile_cover_tokens(rt_ref, cfg.E, T)
    _, y_ref = oracle.forward(layer, x, tokens=toks)
    rel = check_output(y[toks], y_ref, cfg.dtype)
    note(f"[bench configuration] {name} T={T}: rel_err={rel:.2e} tokens_compared={len(toks)}")
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T,S", [(1200, 2), (700, 0), (3000, 1), (2100, 2), (1100, 0), (3000, 0), (130, 1)])
def test_packed_small_layers(T, S):
    """Packed weights on small layers: two shared experts (one packed down
    matrix per shared expert, a segment boundary inside a split k range), no
    shared expert, ragged tiles, and a batch small enough for the streaming
    kernels.  Without shared experts and with at least 256 candidates per
    expert (T = 1100, 3000) the expert-stationary kernels run, on tiles of up
    to 384 rows (T = 3000: two tiles for most experts); with shared experts
    and at least 2048 tokens (T = 2100, 3000) the shared experts run on them
    beside the routed 128-row tiles (one packed down matrix per shared
    expert, the last tile partly filled)."""
    from dynamic_expert_masking_amd.device import DeviceLayer
    layer = small_layer(f"packed{S}", D=256, E=8, K=2, I=256, S=S, I_s=128 if S else 0, keep=0.7,
                        router_bias=True)
    x = small_x(layer, T, "packed")
    note(f"[packed weights] small layer T={T} S={S}")
    y, rt, _ = run_forward(DeviceLayer(layer, pack=True), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("fp8", [False, True])
def test_max_hidden_size(fp8):
    """The largest supported hidden size, D = 16384 (router k split, 256-chunk
    weight rows, shared expert), bf16 and FP8 expert weights."""
    from oracle_pins import fp8_layer
    kw = dict(D=16384, E=6, K=2, I=128, S=1, I_s=128, keep=0.6)
    layer = fp8_layer("maxd", **kw) if fp8 else small_layer("maxd", **kw)
    x = small_x(layer, 40, "maxd")
    note(f"[max D] fp8={fp8}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


def test_empty_batch_is_noop():
    layer = small_layer("empty", D=64, E=8, K=2, I=64)
    dl = device_layer(layer)
    y = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    import dynamic_expert_masking_amd as dm
    dm.beam_moe_forward(dl.desc, x, 0, y, None, None, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_zero_mask_router_is_plain_topk():
    """Wm = 0: every top-K candidate kept; GPU equals the oracle's plain top-K."""
    base = small_layer("gpu_zm", D=128, E=16, K=4, I=64, S=1, I_s=64)
    layer = with_mask(with_mask(base, w_mask_zero=True), b_mask=0.0)
    x = small_x(layer, 48, "zm")
    note("[zero mask router]")
    y, rt, _ = run_forward(device_layer(layer), x)
    assert np.all(rt["mask"] == (1 << 4) - 1)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, 16)
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("shared", [0, 1])
def test_all_masked(shared):
    """b_m = -1e4: nothing survives; y is the shared part, or exactly 0."""
    base = small_layer(f"gpu_allmask{shared}", D=128, E=8, K=2, I=64, S=shared, I_s=64 if shared else 0)
    layer = with_mask(base, b_mask=-1e4)
    x = small_x(base, 20, "am")
    note(f"[all masked] shared={shared}")
    y, rt, _ = run_forward(device_layer(layer), x)
    assert np.all(rt["mask"] == 0) and np.all(rt["expert_count"] == 0)
    assert np.all(rt["gates"] == 0.0)
    if shared:
        _, y_ref = oracle.forward(layer, x)
        check_output(y, y_ref, "bf16")
    else:
        assert np.all(y == 0.0)


# Single-token batches of bf16 layers with intermediate sizes up to 2048 take
# the fused down+combine kernel: row counts of 64 (one chunk in a quarter of
# the lanes) to 2048 (four chunks in every lane), 0-8 shared experts, K up to
# 32, and tokens with every slot masked.
T1_CASES = [dict(D=256, E=16, K=4, I=64, S=0, I_s=0), dict(D=512, E=12, K=3, I=2048, S=1, I_s=2048),
            dict(D=128, E=40, K=32, I=192, S=2, I_s=64), dict(D=1024, E=64, K=6, I=1408, S=8, I_s=128),
            dict(D=64, E=5, K=5, I=320, S=3, I_s=1984)]


T1_FP8_CASES = [dict(D=256, E=16, K=4, I=128, S=0, I_s=0), dict(D=512, E=12, K=3, I=4096, S=1, I_s=4096),
                dict(D=128, E=40, K=8, I=384, S=2, I_s=128)]


@pytest.mark.parametrize("case", range(len(T1_FP8_CASES)))
def test_single_token_fused_down_fp8(case):
    """T = 1 with E4M3 expert weights and row scales perturbed by 2^+-6: the
    fused kernel widens the codes and applies each row's scale."""
    from oracle_pins import fp8_layer
    kw = T1_FP8_CASES[case]
    layer = _fp8_scaled(fp8_layer(f"t1fp8{case}", **kw, keep=0.5, router_bias=True), 11 + case)
    dl = device_layer(layer)
    note(f"[single token fp8] case={case} {kw}")
    for i in range(6):
        x = small_x(layer, 1, f"t1f_{i}")
        y, rt, _ = run_forward(dl, x)
        check_routing(rt, oracle.route(layer, x), kw["E"])
        _, y_ref = oracle.forward(layer, x)
        check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("case", range(len(T1_CASES)))
@pytest.mark.parametrize("masked", [False, True])
def test_single_token_fused_down(case, masked):
    """T = 1: routing exact, y against the oracle on many single tokens
    (each its own batch), including batches where nothing survives."""
    kw = T1_CASES[case]
    base = small_layer(f"t1fused{case}", **kw, keep=0.5, router_bias=True)
    layer = with_mask(base, b_mask=-1e4) if masked else base
    dl = device_layer(layer)
    note(f"[single token] case={case} masked={masked} {kw}")
    for i in range(6):
        x = small_x(base, 1, f"t1_{i}")
        y, rt, ys = run_forward(dl, x, reps=2)
        assert np.array_equal(ys[0], ys[1]), "two identical calls gave different y"
        rt_ref = oracle.route(layer, x)
        check_routing(rt, rt_ref, kw["E"])
        if masked and kw["S"] == 0:
            assert np.all(y == 0.0)
            continue
        _, y_ref = oracle.forward(layer, x)
        check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("E,K", [(7, 1), (8, 8), (64, 32), (300, 12), (1024, 3)])
def test_k_extremes(E, K):
    layer = small_layer(f"gpu_k{E}_{K}", D=128, E=E, K=K, I=64, keep=0.5)
    x = small_x(layer, 33, "kx")
    note(f"[K extremes] E={E} K={K}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, E)
    check_output(y, y_ref, "bf16")


def _tied_layer(E, K):
    """Router logits from a handful of exact values, so that most tokens have
    equal logits inside their top-K and across the K-th / (K+1)-th boundary:
    r_e = x[t, e % 16] * w_e + b_e with x in {-1, 0, 1, 2}, w_e in {0, 0.25, 0.5}
    and b_e in {-0.5, -0.0, 0, 0.5} (every product and sum exact in fp32, -0
    and +0 both present).  Mask logits are b_m = +-1 (fixed keep pattern)."""
    from dataclasses import replace
    layer = small_layer(f"gpu_tie{E}_{K}", D=128, E=E, K=K, I=64, keep=0.5)
    rng = np.random.default_rng(1000 + E + K)
    wr = np.zeros((E, 128), np.float32)
    wr[np.arange(E), np.arange(E) % 16] = rng.choice([0.0, 0.25, 0.5], size=E)
    b_r = rng.choice(np.array([-0.5, -0.0, 0.0, 0.5], np.float32), size=E).astype(np.float32)
    b_m = rng.choice(np.array([-1.0, 1.0], np.float32), size=E).astype(np.float32)
    return replace(layer, w_router=synth.f32_to_bf16_bits(wr),
                   w_mask=synth.f32_to_bf16_bits(np.zeros((E, 128), np.float32)),
                   b_router=b_r, b_mask=b_m)


@pytest.mark.parametrize("E,K", [(40, 7), (100, 32), (212, 16), (700, 5)])
@pytest.mark.parametrize("T", [2, 9, 70, 1200])
def test_topk_ties(E, K, T):
    """Top-K with many exactly equal logits (equal logits go to the lower
    expert index, also at the boundary of the K kept), for every register
    width of the selection (E <= 64, 128, 256, 1024) and each selection form:
    2 tokens (one 4-wave workgroup selects and plans), 9 (the same with 16
    waves), 70 (one wave per token, then the bitmap plan) and 1200 (64-token
    blocks, scan, scatter)."""
    layer = _tied_layer(E, K)
    rng = np.random.default_rng(7 + T)
    x = synth.f32_to_bf16_bits(rng.choice(np.array([-1.0, 0.0, 1.0, 2.0], np.float32),
                                          size=(T, 128)).astype(np.float32))
    note(f"[top-K ties] E={E} K={K} T={T}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, E)
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("E,K", [(7, 1), (40, 7), (212, 16), (700, 5), (1024, 3)])
def test_single_token_ties(E, K):
    """One token per batch on the tied-logit layer: the single-token router's
    fixed-order sums keep the exact ties, and the single-token gate/up and
    down kernels consume what the selection kept."""
    layer = _tied_layer(E, K)
    dl = device_layer(layer)
    rng = np.random.default_rng(50 + E + K)
    note(f"[single token ties] E={E} K={K}")
    for i in range(4):
        x = synth.f32_to_bf16_bits(rng.choice(np.array([-1.0, 0.0, 1.0, 2.0], np.float32),
                                              size=(1, 128)).astype(np.float32))
        y, rt, _ = run_forward(dl, x)
        rt_ref, y_ref = oracle.forward(layer, x)
        check_routing(rt, rt_ref, E)
        check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("T", [1, 37, 4200])
def test_gate_options(flags, T):
    """Gate options (softmax over all E; renormalised masked gates), for one
    token (the single-token kernels), in the one-wave-per-token selection (37
    tokens) and the 64-token-block one (4200)."""
    from oracle_pins import with_gating
    base = small_layer("gates", D=128, E=40, K=6, I=64, S=1, I_s=64, keep=0.4, router_bias=True)
    layer = with_gating(base, flags)
    x = small_x(base, T, "gates")
    note(f"[gate options] flags={flags} T={T}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


def test_gate_options_on_workload():
    """Both gate options on the DeepSeek-V2-Lite-shaped decode layer, T=64."""
    from oracle_pins import with_gating
    name, T = "dsv2lite_decode", 64
    cfg = synth.CONFIGS[name]
    layer = with_gating(cached_layer(name), 3)
    x = inputs(cfg, T, layer)
    note("[gate options] dsv2lite_decode T=64 flags=3")
    y, rt, _ = run_forward(device_layer(layer, key=name + ":gating3"), x)
    rt_ref = oracle.route(layer, x)
    check_routing(rt, rt_ref, cfg.E)
    toks = sample_tokens(T)
    _, y_ref = oracle.forward(layer, x, tokens=toks)
    check_output(y[toks], y_ref, cfg.dtype)


@pytest.mark.parametrize("seg,flags", [(16, 0), (32, 4), (16, 6), (7, 2)])
@pytest.mark.parametrize("T", [13, 37, 4200])
def test_segment_routing(seg, flags, T):
    """Segment routing (every token routes as its segment's first token), with
    the method's gate, binary gates, binary + renormalised and renormalised
    gates; selection and plan in one workgroup (13 tokens), one-wave-per-token
    selection (37) and 64-token blocks (4200)."""
    from oracle_pins import with_segment
    base = small_layer("segment", D=128, E=40, K=6, I=64, S=1, I_s=64, keep=0.4, router_bias=True)
    layer = with_segment(base, seg, flags)
    x = small_x(base, T, "segment")
    note(f"[segment routing] S={seg} flags={flags} T={T}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


def test_segment_routing_stepped_form():
    """The Stepped MoE form on the fine-grained layer (212 experts of 256,
    top-16): 16-token segments, binary gates, zero-initialised mask router
    (every top-K expert kept), T = 512."""
    from oracle_pins import with_segment
    name, T = "finegrained", 512
    cfg = synth.CONFIGS[name]
    layer = with_segment(with_mask(cached_layer(name), True, 0.0), 16, 4)
    x = inputs(cfg, T, cached_layer(name))
    note("[segment routing] finegrained T=512 S=16 binary")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref = oracle.route(layer, x)
    check_routing(rt, rt_ref, cfg.E)
    assert np.all(rt["mask"] == (1 << cfg.K) - 1)
    for s0 in range(0, T, 16):
        assert np.all(rt["topk_idx"][s0:s0 + 16] == rt["topk_idx"][s0])
    toks = sample_tokens(T)
    _, y_ref = oracle.forward(layer, x, tokens=toks)
    check_output(y[toks], y_ref, cfg.dtype)


def _mask_backward_case(layer, x, beta, seed, dev=None):
    import dynamic_expert_masking_amd as dm
    from dynamic_expert_masking_amd.device import to_device
    cfg = layer.cfg
    T = x.shape[0]
    dy32 = np.random.default_rng(seed).standard_normal((T, cfg.D)).astype(np.float32)
    dy_store = synth.f32_to_bf16_bits(dy32) if cfg.dtype == "bf16" else dy32
    dl = dev or device_layer(layer)
    ws = dl.workspace(T)
    dwm = torch.empty(cfg.E, cfg.D, dtype=torch.float32, device="cuda")
    dbm = torch.empty(cfg.E, dtype=torch.float32, device="cuda")
    lreg = torch.empty(1, dtype=torch.float32, device="cuda")
    dm.beam_moe_mask_backward(dl.desc, to_device(x), to_device(dy_store), T, beta, dwm, dbm, lreg,
                              ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    dy64 = oracle.widen(dy_store, cfg.dtype)
    lreg_ref, dwm_ref, dbm_ref, _ = oracle.mask_router_backward(layer, x, dy64, beta)
    tol = 3e-2 if cfg.dtype == "bf16" else 1e-4
    assert abs(float(lreg.item()) - lreg_ref) <= 2e-6, (float(lreg.item()), lreg_ref)
    for got, ref, name in ((dwm.cpu().numpy(), dwm_ref, "dWm"), (dbm.cpu().numpy(), dbm_ref, "db_m")):
        err = np.abs(got - ref).max()
        assert err <= tol * np.abs(ref).max(), f"{name}: max|err| {err:.3e} vs max|ref| {np.abs(ref).max():.3e}"
    return dwm, dbm


@pytest.mark.parametrize("T", [5, 37, 4200])
def test_mask_backward_small(T):
    """Mask-router loss value and straight-through gradient: selection and
    plan in one workgroup (5 tokens), one-wave-per-token selection (37) and
    the 64-token-block one (4200)."""
    layer = small_layer("mbwd", D=128, E=40, K=6, I=64, S=1, I_s=64, keep=0.4, router_bias=True)
    x = small_x(layer, T, "mbwd")
    note(f"[mask backward] small T={T}")
    _mask_backward_case(layer, x, 0.25, 3)


def test_mask_backward_f32_and_zero():
    """fp32 layer (tiny workload); with dL/dy = 0 and beta = 0 the gradient is exactly 0."""
    import dynamic_expert_masking_amd as dm
    from dynamic_expert_masking_amd.device import to_device
    name = "tiny_f32"
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, 64, layer)
    note("[mask backward] tiny_f32 T=64")
    dl = device_layer(layer, key=name)
    _mask_backward_case(layer, x, 0.5, 4, dl)
    ws = dl.workspace(64)
    dwm = torch.full((cfg.E, cfg.D), 7.0, device="cuda")
    lreg = torch.empty(1, device="cuda")
    dm.beam_moe_mask_backward(dl.desc, to_device(x), torch.zeros(64, cfg.D, device="cuda"), 64, 0.0,
                              dwm, None, lreg, ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dwm).item() == 0


def test_mask_backward_workload():
    name, T = "dsv2lite_decode", 64
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, T, layer)
    note("[mask backward] dsv2lite_decode T=64")
    _mask_backward_case(layer, x, 0.1, 5, device_layer(layer, key=name))


def _fp8_scaled(layer, seed):
    """The same FP8 layer with every row scale multiplied by its own power of
    two in 2^-6 .. 2^6, so that a scale applied to the wrong row shows."""
    from dataclasses import replace
    rng = np.random.default_rng(seed)
    kw = {}
    for n in ("s_gate", "s_up", "s_down", "ss_gate", "ss_up", "ss_down"):
        a = getattr(layer, n)
        if a is not None:
            kw[n] = (a * np.exp2(rng.integers(-6, 7, size=a.shape))).astype(np.float32)
    return replace(layer, **kw)


@pytest.mark.parametrize("S", [0, 1, 2])
@pytest.mark.parametrize("T", [1, 37, 129, 700])
def test_fp8_small(S, T):
    """FP8 (E4M3) expert weights with widely varying row scales: 1 to 700
    tokens (700 x 3 / 12 = 175 pairs per expert, which FP8 still runs in
    64-row streaming tiles), with 0, 1 or 2 shared experts (2: the fused
    shared down projection has one scaled k segment per shared expert)."""
    from oracle_pins import fp8_layer
    base = fp8_layer(f"gpu_fp8_{S}", D=256, E=12, K=3, I=128, S=S, I_s=128 if S else 0, keep=0.6,
                     router_bias=True)
    layer = _fp8_scaled(base, 10 + S)
    x = small_x(layer, T, "fp8")
    note(f"[fp8] S={S} T={T}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, layer.cfg.E)
    check_output(y, y_ref, "bf16")


def test_fp8_ksplit_and_wide_rows():
    """FP8 layer with D = 4096 and I = 1024: 3 tokens (16-row tiles, gate/up
    k split four ways, down two ways), 100 (32-row tiles, both split two
    ways) and 200 (64-row tiles, no split)."""
    from oracle_pins import fp8_layer
    layer = _fp8_scaled(fp8_layer("gpu_fp8_wide", D=4096, E=8, K=2, I=1024, S=1, I_s=256,
                                  keep=0.7), 21)
    for T in (3, 100, 200):
        x = small_x(layer, T, "fp8w")
        note(f"[fp8 wide] T={T}")
        y, rt, _ = run_forward(device_layer(layer), x)
        rt_ref, y_ref = oracle.forward(layer, x)
        check_routing(rt, rt_ref, layer.cfg.E)
        check_output(y, y_ref, "bf16")


def test_fp8_mask_backward():
    """Mask-router gradient of an FP8 layer (every candidate's expert runs on
    the E4M3 weights)."""
    from oracle_pins import fp8_layer
    layer = _fp8_scaled(fp8_layer("gpu_fp8_bwd", D=256, E=16, K=4, I=128, S=1, I_s=128, keep=0.5),
                        31)
    x = small_x(layer, 45, "fp8bwd")
    note("[fp8 mask backward] T=45")
    _mask_backward_case(layer, x, 0.3, 6)


def test_route_entry_matches_forward():
    name, T = "finegrained", 512
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, T, layer)
    dl = device_layer(layer, key=name)
    note("[route vs forward]")
    rt_r = run_route(dl, x)
    _, rt_f, _ = run_forward(dl, x)
    for k in rt_r:
        assert np.array_equal(rt_r[k], rt_f[k]), k
    check_routing(rt_r, oracle.route(layer, x), cfg.E)


def test_stats_on_device_counts():
    import dynamic_expert_masking_amd as dm
    name, T = "dsv2lite_decode", 64
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    x = inputs(cfg, T, layer)
    dl = device_layer(layer, key=name)
    _, rt, _ = run_forward(dl, x)
    counts_dev = torch.from_numpy(rt["expert_count"]).cuda()
    st = dm.beam_moe_stats(dl.desc, counts_dev, T, torch.cuda.current_stream().cuda_stream)
    ref = oracle.layer_stats(cfg, oracle.expert_counts(oracle.route(layer, x), cfg.E), T)
    for k, v in ref.items():
        assert st[k] == pytest.approx(v, rel=1e-12), k


@pytest.mark.parametrize("T", [1, 64, 1400])
def test_graph_capture_replays(T):
    """beam_moe_forward captured once in a HIP graph and replayed on three
    different batches copied into the captured input buffer (eager copies and
    synchronisations between the replays): every replay's y and routing
    outputs equal an eager call's bit for bit.  The forward path enqueues
    kernels only (no memsets, allocations or host synchronisation), so it can
    be captured; 1, 64 and 1400 tokens take the one-workgroup, bitmap-plan and
    block-rank routing forms."""
    import dynamic_expert_masking_amd as dm
    from dynamic_expert_masking_amd.device import to_device, to_host_bits
    name = "dsv2lite_decode"
    cfg = synth.CONFIGS[name]
    layer = cached_layer(name)
    dl = device_layer(layer, key=name)
    xs = [to_device(inputs(cfg, T, layer, f"graph{i}")) for i in range(3)]
    ws = dl.workspace(T)
    y_ref = []
    route_ref = []
    for i in range(3):
        yi = torch.empty(T, cfg.D, dtype=dl.torch_dtype, device="cuda")
        bufs, out = dl.route_buffers(T)
        dm.beam_moe_forward(dl.desc, xs[i], T, yi, out, ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        y_ref.append(to_host_bits(yi).copy())
        route_ref.append({k: v.cpu().numpy().copy() for k, v in bufs.items()})
    x_static = xs[0].clone()
    y_static = torch.empty(T, cfg.D, dtype=dl.torch_dtype, device="cuda")
    bufs, out = dl.route_buffers(T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a side stream before capture
        dm.beam_moe_forward(dl.desc, x_static, T, y_static, out, ws, ws.numel(), side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note(f"[graph] capture T={T}")
    with torch.cuda.graph(graph):
        dm.beam_moe_forward(dl.desc, x_static, T, y_static, out, ws, ws.numel(),
                            torch.cuda.current_stream().cuda_stream)
    for rep in range(2):
        for i in (2, 0, 1):
            x_static.copy_(xs[i])
            y_static.fill_(0)
            torch.cuda.synchronize()
            note(f"[graph] replay {rep} batch {i} T={T}")
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(to_host_bits(y_static), y_ref[i]), f"replay {rep} batch {i}: y differs"
            for k, v in bufs.items():
                assert np.array_equal(v.cpu().numpy(), route_ref[i][k]), f"replay {rep} batch {i}: {k} differs"


def _random_case(i: int):
    """Seeded random small layer configuration number i."""
    rng = np.random.default_rng(4242 + i)
    E = int(rng.choice([3, 7, 16, 40, 64, 65, 100, 128, 129, 212, 256, 257, 300]))
    K = int(rng.integers(1, min(E, 32) + 1))
    D = int(rng.choice([64, 128, 192, 256, 512]))
    I = int(rng.choice([64, 128, 192, 320]))
    S = int(rng.choice([0, 0, 1, 2]))
    I_s = int(rng.choice([64, 128])) if S else 0
    keep = float(rng.uniform(0.1, 0.9))
    router_bias = bool(rng.random() < 0.5)
    T = int(rng.choice([1, 2, 5, 16, 17, 33, 64, 65, 200, 513, 700]))
    gating = int(rng.choice([0, 0, 1, 2, 3, 4, 6]))
    segment = int(rng.choice([0, 0, 0, 2, 5]))
    dtype = "f32" if rng.random() < 0.15 else "bf16"
    return dict(E=E, K=K, D=D, I=I, S=S, I_s=I_s, keep=keep, router_bias=router_bias, T=T,
                gating=gating, segment=segment, dtype=dtype)


@pytest.mark.parametrize("case", range(24))
def test_random_configs(case):
    """Seeded random small configurations across the parameter space: 3 to 300
    experts (every register width of the selection), K up to min(E, 32),
    hidden and intermediate sizes from 64 to 512, no, one or two shared
    experts, every gate option, segment routing, 1 to 700 tokens (every tile
    height and routing form), bf16 and fp32.  Routing bit-exact against the
    oracle, y within the dtype's tolerance."""
    from oracle_pins import with_segment
    c = _random_case(case)
    note(f"[random config {case}] {c}")
    base = small_layer(f"rand{case}", dtype=c["dtype"], D=c["D"], E=c["E"], K=c["K"], I=c["I"],
                       S=c["S"], I_s=c["I_s"], keep=c["keep"], router_bias=c["router_bias"])
    layer = with_segment(base, c["segment"], c["gating"])
    x = small_x(base, c["T"], f"rand{case}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, c["E"])
    check_output(y, y_ref, c["dtype"])


def _random_fp8_case(i: int):
    """Seeded random small FP8 layer configuration number i (hidden and
    intermediate sizes multiples of 128, as the format requires)."""
    rng = np.random.default_rng(5151 + i)
    E = int(rng.choice([4, 12, 40, 64, 130]))
    K = int(rng.integers(1, min(E, 8) + 1))
    D = int(rng.choice([128, 256, 384, 512]))
    I = int(rng.choice([128, 256, 384]))
    S = int(rng.choice([0, 1, 2]))
    I_s = int(rng.choice([128, 256])) if S else 0
    T = int(rng.choice([1, 3, 16, 40, 129, 300, 600]))
    return dict(E=E, K=K, D=D, I=I, S=S, I_s=I_s, keep=float(rng.uniform(0.2, 0.9)),
                router_bias=bool(rng.random() < 0.5), T=T)


@pytest.mark.parametrize("case", range(8))
def test_random_fp8_configs(case):
    """Seeded random small FP8 (E4M3) layers with widely varying row scales,
    1 to 600 tokens (16-, 32- and 64-row tiles): routing bit-exact, y within
    the bf16 tolerance."""
    from oracle_pins import fp8_layer
    c = _random_fp8_case(case)
    note(f"[random fp8 config {case}] {c}")
    layer = _fp8_scaled(fp8_layer(f"rfp8_{case}", D=c["D"], E=c["E"], K=c["K"], I=c["I"], S=c["S"],
                                  I_s=c["I_s"], keep=c["keep"], router_bias=c["router_bias"]),
                        900 + case)
    x = small_x(layer, c["T"], f"rfp8_{case}")
    y, rt, _ = run_forward(device_layer(layer), x)
    rt_ref, y_ref = oracle.forward(layer, x)
    check_routing(rt, rt_ref, c["E"])
    check_output(y, y_ref, "bf16")


@pytest.mark.parametrize("case", range(6))
def test_random_mask_backward(case):
    """The mask-router loss and straight-through gradient on seeded random
    small layers (the random forward configurations' shapes, method's gate,
    no segment routing)."""
    c = _random_case(100 + case)
    note(f"[random mask backward {case}] {c}")
    layer = small_layer(f"rbwd{case}", dtype=c["dtype"], D=c["D"], E=c["E"], K=c["K"], I=c["I"],
                        S=c["S"], I_s=c["I_s"], keep=c["keep"], router_bias=c["router_bias"])
    x = small_x(layer, c["T"], f"rbwd{case}")
    _mask_backward_case(layer, x, 0.2, 40 + case)
