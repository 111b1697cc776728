"""Seeded input generator: determinism, bf16 rounding, workload statistics."""
import math

import numpy as np
import torch

import synth
import oracle
from common import enforce_margins, margins_ok


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        # exact halfway cases between two bf16 values
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, 1.0, -2.5, 3.4e38], np.float32)])
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(ours, ref)


def test_streams_deterministic_and_distinct():
    a = synth.normal_f32(synth.stream_key("c", "t", 1), 1000, 1.0)
    b = synth.normal_f32(synth.stream_key("c", "t", 1), 1000, 1.0)
    c = synth.normal_f32(synth.stream_key("c", "t", 2), 1000, 1.0)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    big = synth.normal_f32(synth.stream_key("c", "big"), 400000, 2.0)
    assert abs(big.mean()) < 0.02 and abs(big.std() - 2.0) < 0.02


def test_mask_bias_gives_keep_rate():
    for cfg in synth.CONFIGS.values():
        b = cfg.mask_bias
        keep = 1.0 - 0.5 * (1.0 + math.erf((0.0 - b) / math.sqrt(0.5) / math.sqrt(2.0)))
        assert abs(keep - cfg.keep) < 1e-9, cfg.name


def test_make_layer_shapes_and_determinism():
    cfg = synth.CONFIGS["tiny_f32"]
    l1 = synth.make_layer(cfg)
    l2 = synth.make_layer(cfg)
    assert l1.w_gate.shape == (8, 256, 128) and l1.w_down.shape == (8, 128, 256)
    assert l1.w_gate.dtype == np.float32
    for n in ("w_router", "w_mask", "w_gate", "w_up", "w_down"):
        assert np.array_equal(getattr(l1, n), getattr(l2, n))
    # weights ~ N(0, 1/D), mask router ~ N(0, 0.5/D)
    assert abs(l1.w_gate.std() * math.sqrt(cfg.D) - 1.0) < 0.01
    assert abs(l1.w_mask.std() * math.sqrt(cfg.D / 0.5) - 1.0) < 0.05


def test_realised_avg_k_near_targets():
    """Routing-only statistics of the generated workloads (mask bias sets Avg-K)."""
    for name, T, lo, hi in (("tiny_f32", 64, 0.6, 1.4), ("dsv2lite_decode", 256, 2.6, 3.4),
                            ("dsv2lite_prefill", 1024, 0.35, 0.65), ("mixtral", 512, 0.85, 1.15),
                            ("finegrained", 512, 2.0, 2.8)):
        cfg = synth.CONFIGS[name]
        layer = synth.make_layer(cfg, experts=False)
        x = synth.make_x(cfg, T)
        rt = oracle.route(layer, x)
        avgk = rt.keep.sum() / T
        assert lo <= avgk <= hi, (name, avgk)


def test_margin_enforcement():
    cfg = synth.CONFIGS["finegrained"]
    layer = synth.make_layer(cfg, experts=False)
    x0 = synth.make_x(cfg, 256)
    x = enforce_margins(layer, x0, 256)
    r, z = oracle.router_logits(layer, x)
    assert margins_ok(r, z, cfg.K).all()
    changed = (x != x0).any(axis=1).sum()
    assert 0 < changed < 64   # a few percent of tokens are redrawn


def test_e4m3_encode_matches_torch():
    """Nearest-even E4M3 encoding of in-range float32 values equals torch's
    float8_e4m3fn conversion, including exact halfway cases and subnormals."""
    rng = np.random.default_rng(7)
    vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    finite = vals.to(torch.float64).numpy()
    finite = np.sort(np.unique(finite[np.isfinite(finite)]))
    mids = 0.5 * (finite[1:] + finite[:-1])        # every halfway point
    a = np.concatenate([rng.standard_normal(200000) * 40.0, rng.standard_normal(20000) * 0.01,
                        finite, mids, -mids, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10]])
    a = np.clip(a, -448.0, 448.0).astype(np.float32)
    ours = synth.e4m3_encode(a)
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # ties go to the even code: 1.0625 -> 1.0 (0x38), 1.1875 -> 1.25 (0x3A)
    assert list(synth.e4m3_encode(np.array([1.0625, 1.1875, 3 * 2.0 ** -10], np.float32))) == [0x38, 0x3A, 0x02]


def test_row_quantisation_error_bound():
    """Per-row scales: every row reaches 448 in magnitude, and each value is
    within half a step of its code (relative 2^-4 for normal codes, 2^-10
    times the scale below the normal range)."""
    w = synth.normal_f32(synth.stream_key("q", "w"), 64 * 300, 0.05).reshape(64, 300)
    w[3] = 0.0
    codes, scale = synth.quantize_rows_e4m3(w)
    dec = oracle.decode_e4m3(codes)
    assert np.array_equal(np.abs(dec).max(axis=1)[np.arange(64) != 3], np.full(63, 448.0))
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    q = w.astype(np.float64) / scale[:, None].astype(np.float64)
    err = np.abs(dec - q)
    normal = np.abs(q) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(q[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 1e-6))


def test_fp8_workload_layer_shapes():
    cfg = synth.CONFIGS["dsv2lite_decode_fp8"]
    assert cfg.expert_format == synth.FP8 and cfg.dtype == synth.BF16
    small = synth.LayerConfig("fp8shape", "bf16", D=128, E=4, K=2, I=64, S=1, I_s=128, tokens=(),
                              keep=0.5, router_bias=False, expert_format=synth.FP8)
    lay = synth.make_layer(small)
    assert lay.w_gate.dtype == np.uint8 and lay.w_gate.shape == (4, 64, 128)
    assert lay.s_gate.shape == (4, 64) and lay.s_down.shape == (4, 128)
    assert lay.ws_up.shape == (1, 128, 128) and lay.ss_down.shape == (1, 128)
    assert lay.w_router.dtype == np.uint16
