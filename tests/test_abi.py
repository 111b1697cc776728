"""The C-ABI library on the host: it loads, exports every declared symbol,
sizes workspaces, validates arguments before touching any GPU, and its
host-side work accounting matches the oracle's."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import dynamic_expert_masking_amd as dm
import oracle
import synth
from common import small_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(dm.LIB_PATH), reason="library not built")


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(beam_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "beam_moe_forward" in names and "beam_moe_route" in names and "beam_moe_stats" in names
    lib = ctypes.CDLL(dm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


FAKE = 0x10000   # aligned, never dereferenced: validation fails before any use


def fake_layer(**kw):
    p = dict(D=128, E=8, K=2, I=256, dtype=dm.BEAM_BF16, w_router=FAKE, w_mask=FAKE,
             w_gate=FAKE, w_up=FAKE, w_down=FAKE)
    p.update(kw)
    return dm.make_layer(**p)


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert dm.beam_status_str(s).startswith("BEAM_")
    assert "unknown" in dm.beam_status_str(7)


def test_workspace_size_monotone_and_invalid():
    L = fake_layer()
    sizes = [dm.beam_moe_workspace_size(L, T) for T in (0, 1, 64, 65, 4096)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:])) and sizes[-1] > sizes[1] > 0
    assert dm.beam_moe_workspace_size(fake_layer(K=9), 16) == 0          # K > E
    assert dm.beam_moe_workspace_size(fake_layer(gating=16), 16) == 0    # unknown gate bit
    assert dm.beam_moe_workspace_size(fake_layer(gating=dm.GATE_SOFTMAX_ALL | dm.GATE_RENORM), 16) > 0
    assert dm.beam_moe_workspace_size(fake_layer(D=100), 16) == 0        # D % 64
    assert dm.beam_moe_workspace_size(fake_layer(gating=dm.GATE_BINARY | dm.GATE_RENORM), 16) > 0
    assert dm.beam_moe_workspace_size(fake_layer(gating=dm.GATE_BINARY | dm.GATE_SOFTMAX_ALL), 16) == 0
    assert dm.beam_moe_workspace_size(fake_layer(gating=8), 16) == 0
    assert dm.beam_moe_workspace_size(fake_layer(segment_len=16), 16) > 0
    assert dm.beam_moe_workspace_size(fake_layer(segment_len=-1), 16) == 0
    assert dm.beam_moe_workspace_size(L, -1) == 0
    f8 = dict(expert_format=dm.WEIGHTS_FP8_E4M3, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE)
    assert dm.beam_moe_workspace_size(fake_layer(**f8), 64) == sizes[2]


def test_shared_expert_stationary_workspace():
    """Packed layers with shared experts run the shared experts on the
    expert-stationary kernels from 2048 tokens: the workspace then also holds
    their packed tokens and h (ceil(T / 384) tiles of 384 x (D + S Is) bf16),
    and it stays non-decreasing in T across the switch.  Below it, the packed
    and the unpacked layer need the same workspace."""
    cfg = synth.CONFIGS["dsv2lite_prefill"]
    kw = dict(D=cfg.D, E=cfg.E, K=cfg.K, I=cfg.I, n_shared=cfg.S, I_shared=cfg.I_s, ws_gate=FAKE,
              ws_up=FAKE, ws_down=FAKE)
    packed = dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE, wsp_gate=FAKE, wsp_up=FAKE, wsp_down=FAKE)
    Lp, Lu = fake_layer(**kw, **packed), fake_layer(**kw)
    Ts = [1, 64, 1024, 2000, 2047, 2048, 2049, 3000, 4096]
    sizes = [dm.beam_moe_workspace_size(Lp, T) for T in Ts]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    for T in (64, 1024, 2047):
        assert dm.beam_moe_workspace_size(Lp, T) == dm.beam_moe_workspace_size(Lu, T)
    es_bytes = -(-2048 // 384) * 384 * (cfg.D + cfg.S * cfg.I_s) * 2
    assert (dm.beam_moe_workspace_size(Lp, 2048) - dm.beam_moe_workspace_size(Lu, 2048)) >= es_bytes


def config_layer(cfg):
    """A descriptor with a workload's shapes and fake (never dereferenced) pointers."""
    kw = dict(D=cfg.D, E=cfg.E, K=cfg.K, I=cfg.I,
              dtype=dm.BEAM_F32 if cfg.dtype == "f32" else dm.BEAM_BF16)
    if cfg.S:
        kw.update(n_shared=cfg.S, I_shared=cfg.I_s, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE)
    if cfg.expert_format == synth.FP8:
        kw.update(expert_format=dm.WEIGHTS_FP8_E4M3, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE,
                  scale_shared_gate=FAKE, scale_shared_up=FAKE, scale_shared_down=FAKE)
    return fake_layer(**kw)


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_workspace_serves_every_smaller_batch(name):
    """A workspace sized for T_max serves every batch T <= T_max: the size is
    non-decreasing in T (the router's k split, and so its partial-logit rows,
    rises as T falls; the workspace reserves a bound that does not), so
    ws(T) <= ws(T_max) for every T <= T_max; and a workspace one byte short
    of ws(T) is rejected before any launch.  (No call here is given enough
    workspace to pass validation: it would launch kernels on fake pointers.)"""
    L = config_layer(synth.CONFIGS[name])
    Ts = list(range(0, 1100)) + list(range(1100, 17000, 7)) + [4080, 5440, 5441, 8128, 8129,
                                                               8192, 8193, 10880, 10881,
                                                               16383, 16384, 16385]
    Ts = sorted(set(Ts))
    sizes = [dm.beam_moe_workspace_size(L, T) for T in Ts]
    for (t0, a), (t1, b) in zip(zip(Ts, sizes), zip(Ts[1:], sizes[1:])):
        assert a <= b, f"workspace size drops from T={t0} ({a}) to T={t1} ({b})"
    f = dm.lib().beam_moe_forward
    for T_max in (161, 497, 1360, 4080):
        need = dm.beam_moe_workspace_size(L, T_max)
        for T in sorted({1, 2, 48, 64, 144, 160, 496, T_max - 1, T_max}):
            if T > T_max:
                continue
            # a workspace one byte short of ws(T) is rejected; ws(T_max) is not
            assert f(ctypes.byref(L), FAKE, T, FAKE * 2, None, FAKE * 3,
                     dm.beam_moe_workspace_size(L, T) - 1, None) == dm.BEAM_ERR_WORKSPACE
            assert dm.beam_moe_workspace_size(L, T) <= need


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), dm.BEAM_ERR_INVALID_ARG),
    (dict(K=9), dm.BEAM_ERR_INVALID_ARG),
    (dict(E=40, K=33), dm.BEAM_ERR_UNSUPPORTED),
    (dict(E=2000, K=4), dm.BEAM_ERR_UNSUPPORTED),
    (dict(D=96), dm.BEAM_ERR_UNSUPPORTED),
    (dict(I=100), dm.BEAM_ERR_UNSUPPORTED),
    (dict(dtype=5), dm.BEAM_ERR_INVALID_ARG),
    (dict(w_gate=None), dm.BEAM_ERR_INVALID_ARG),
    (dict(w_up=FAKE + 8), dm.BEAM_ERR_INVALID_ARG),
    (dict(n_shared=2, I_shared=0), dm.BEAM_ERR_INVALID_ARG),
    (dict(n_shared=1, I_shared=64), dm.BEAM_ERR_INVALID_ARG),       # shared pointers missing
    (dict(n_shared=1, I_shared=96, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE), dm.BEAM_ERR_UNSUPPORTED),
    (dict(D=16384, I=131072), dm.BEAM_ERR_UNSUPPORTED),               # I * D = 2^31 elements
    (dict(D=8192, n_shared=2, I_shared=131072, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE),
     dm.BEAM_ERR_UNSUPPORTED),                                          # shared rows * D = 2^31
    # FP8 (E4M3) expert weights
    (dict(expert_format=2), dm.BEAM_ERR_INVALID_ARG),
    (dict(expert_format=1), dm.BEAM_ERR_INVALID_ARG),                  # scales missing
    (dict(expert_format=1, scale_gate=FAKE, scale_up=FAKE + 4, scale_down=FAKE), dm.BEAM_ERR_INVALID_ARG),
    (dict(expert_format=1, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE, dtype=dm.BEAM_F32),
     dm.BEAM_ERR_UNSUPPORTED),
    (dict(expert_format=1, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE, D=192),
     dm.BEAM_ERR_UNSUPPORTED),                                          # D % 128
    (dict(expert_format=1, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE, I=320),
     dm.BEAM_ERR_UNSUPPORTED),                                          # I % 128
    (dict(expert_format=1, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE, n_shared=1,
          I_shared=128, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE), dm.BEAM_ERR_INVALID_ARG),  # shared scales
    (dict(expert_format=1, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE, n_shared=1,
          I_shared=192, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE, scale_shared_gate=FAKE,
          scale_shared_up=FAKE, scale_shared_down=FAKE), dm.BEAM_ERR_UNSUPPORTED),  # I_shared % 128
])
def test_forward_rejects_bad_layers(kw, status):
    L = fake_layer(**kw)
    rc = dm.lib().beam_moe_forward(ctypes.byref(L), FAKE, 4, FAKE * 2, None, FAKE * 3, 1 << 40, None)
    assert rc == status


def test_forward_rejects_bad_calls():
    L = fake_layer()
    f = dm.lib().beam_moe_forward
    big = 1 << 40
    assert f(ctypes.byref(L), FAKE, -1, FAKE, None, FAKE, big, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(ctypes.byref(L), None, 4, FAKE, None, FAKE, big, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(ctypes.byref(L), FAKE + 4, 4, FAKE * 2, None, FAKE, big, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(ctypes.byref(L), FAKE, 4, None, None, FAKE, big, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(ctypes.byref(L), FAKE, 4, FAKE, None, FAKE * 3, big, None) == dm.BEAM_ERR_INVALID_ARG  # y == x
    assert f(ctypes.byref(L), FAKE, 4, FAKE * 2, None, None, big, None) == dm.BEAM_ERR_WORKSPACE
    need = dm.beam_moe_workspace_size(L, 4)
    assert f(ctypes.byref(L), FAKE, 4, FAKE * 2, None, FAKE * 3, need - 1, None) == dm.BEAM_ERR_WORKSPACE
    bad_out = dm.beam_route_out(FAKE, None, FAKE, FAKE)
    assert f(ctypes.byref(L), FAKE, 4, FAKE * 2, ctypes.byref(bad_out), FAKE * 3, big, None) \
        == dm.BEAM_ERR_INVALID_ARG
    # x [T][D] of 2^31 elements or more is outside the kernels' 32-bit offsets
    L2 = fake_layer(D=16384)
    assert f(ctypes.byref(L2), FAKE, 131072, FAKE * 2, None, FAKE * 3, big, None) == dm.BEAM_ERR_UNSUPPORTED
    assert dm.beam_moe_workspace_size(L2, 131072) == 0
    assert dm.beam_moe_workspace_size(L2, 131071) > 0
    assert dm.beam_moe_workspace_size(fake_layer(D=16384, I=131008), 1) > 0   # I * D just below 2^31
    # T = 0 is a no-op, even with no workspace
    assert f(ctypes.byref(L), FAKE, 0, FAKE * 2, None, None, 0, None) == dm.BEAM_OK


def test_forward_static_argument_checks():
    """The allocation-free forward validates (layer, T, and the batch's
    workspace against the static array's size) before any HIP call."""
    L = fake_layer()
    f = dm.lib().beam_moe_forward_static
    assert f(ctypes.byref(fake_layer(K=9)), FAKE, 4, FAKE * 2, None, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(ctypes.byref(L), FAKE, -1, FAKE * 2, None, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(ctypes.byref(L), FAKE, 0, FAKE * 2, None, None) == dm.BEAM_OK
    big = 1
    while dm.beam_moe_workspace_size(L, big) <= dm.STATIC_WORKSPACE_BYTES:
        big *= 2
    assert f(ctypes.byref(L), FAKE, big, FAKE * 2, None, None) == dm.BEAM_ERR_WORKSPACE
    # every decode batch of the DeepSeek-V2-Lite-, Mixtral- and fine-grained-shaped layers fits
    for name in ("dsv2lite_decode", "mixtral", "finegrained", "dsv2lite_decode_fp8"):
        assert dm.beam_moe_workspace_size(config_layer(synth.CONFIGS[name]), 512) \
            <= dm.STATIC_WORKSPACE_BYTES, name


def test_pack_weights_argument_checks():
    """beam_moe_pack_weights validates before launching: rows a multiple of 32,
    columns of 64, aligned non-null pointers, no overlap."""
    f = dm.lib().beam_moe_pack_weights
    assert f(FAKE, 2, 48, 64, FAKE * 64, None) == dm.BEAM_ERR_INVALID_ARG      # rows % 32
    assert f(FAKE, 2, 64, 96, FAKE * 64, None) == dm.BEAM_ERR_INVALID_ARG      # cols % 64
    assert f(None, 2, 64, 64, FAKE * 64, None) == dm.BEAM_ERR_INVALID_ARG
    assert f(FAKE, 2, 64, 64, FAKE + 8, None) == dm.BEAM_ERR_INVALID_ARG        # misaligned
    assert f(FAKE, 2, 64, 64, FAKE + 4096, None) == dm.BEAM_ERR_INVALID_ARG     # overlaps the input
    assert f(FAKE, 0, 64, 64, FAKE * 64, None) == dm.BEAM_OK                    # nothing to do


@pytest.mark.parametrize("kw,status", [
    (dict(wp_gate=FAKE), dm.BEAM_ERR_INVALID_ARG),                               # partial set
    (dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE + 8), dm.BEAM_ERR_INVALID_ARG),  # misaligned
    (dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE, dtype=dm.BEAM_F32), dm.BEAM_ERR_INVALID_ARG),
    (dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE, wsp_gate=FAKE, wsp_up=FAKE, wsp_down=FAKE),
     dm.BEAM_ERR_INVALID_ARG),                                                   # shared copies, no shared experts
    (dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE, n_shared=1, I_shared=64, ws_gate=FAKE, ws_up=FAKE,
          ws_down=FAKE), dm.BEAM_ERR_INVALID_ARG),                               # shared copies missing
    (dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE, expert_format=1, scale_gate=FAKE, scale_up=FAKE,
          scale_down=FAKE), dm.BEAM_ERR_INVALID_ARG),                            # FP8 weights
])
def test_packed_weight_fields(kw, status):
    L = fake_layer(**kw)
    assert dm.beam_moe_workspace_size(L, 16) == 0
    rc = dm.lib().beam_moe_forward(ctypes.byref(L), FAKE, 4, FAKE * 2, None, FAKE * 3, 1 << 40, None)
    assert rc == status
    ok = fake_layer(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE)
    assert dm.beam_moe_workspace_size(ok, 16) > 0


def test_mask_backward_argument_checks():
    L = fake_layer()
    ws = 0x20000
    n = dm.beam_moe_workspace_size(L, 4)
    lib = dm.lib()
    def call(layer, dwm=FAKE, lreg=FAKE, dy=FAKE, T=4, ws_bytes=n):
        return lib.beam_moe_mask_backward(ctypes.byref(layer), FAKE, dy, T, 0.1, dwm, None, lreg,
                                          ws, ws_bytes, None)
    assert call(fake_layer(gating=1)) == dm.BEAM_ERR_UNSUPPORTED
    assert call(fake_layer(segment_len=4)) == dm.BEAM_ERR_UNSUPPORTED
    assert call(L, dwm=None) == dm.BEAM_ERR_INVALID_ARG
    assert call(L, dwm=FAKE + 4) == dm.BEAM_ERR_INVALID_ARG     # dWm must be 16-byte aligned
    assert call(L, lreg=None) == dm.BEAM_ERR_INVALID_ARG
    assert call(L, dy=None) == dm.BEAM_ERR_INVALID_ARG
    assert call(L, ws_bytes=n - 1) == dm.BEAM_ERR_WORKSPACE
    assert call(L, T=0) == dm.BEAM_OK


def test_route_requires_all_outputs():
    L = fake_layer()
    r = dm.lib().beam_moe_route
    assert r(ctypes.byref(L), FAKE, 4, None, FAKE, 1 << 40, None) == dm.BEAM_ERR_INVALID_ARG
    out = dm.beam_route_out(FAKE, FAKE, None, FAKE)
    assert r(ctypes.byref(L), FAKE, 4, ctypes.byref(out), FAKE, 1 << 40, None) == dm.BEAM_ERR_INVALID_ARG


def test_profile_and_copy_argument_checks():
    assert dm.lib().beam_profile_begin(0) == dm.BEAM_ERR_INVALID_ARG
    assert dm.lib().beam_profile_end(None, None, None, 0) == dm.BEAM_ERR_INVALID_ARG
    assert dm.lib().beam_copy_kernel(FAKE, FAKE, 15, None) == dm.BEAM_ERR_INVALID_ARG
    assert dm.lib().beam_copy_kernel(FAKE, FAKE, 0, None) == dm.BEAM_OK


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_stats_host_matches_oracle(name):
    cfg = synth.CONFIGS[name]
    rng = np.random.default_rng(11)
    T = cfg.tokens[-1]
    counts = rng.integers(0, 5, size=cfg.E)
    counts[rng.random(cfg.E) < 0.3] = 0
    kw = dict(D=cfg.D, E=cfg.E, K=cfg.K, I=cfg.I,
              dtype=dm.BEAM_F32 if cfg.dtype == "f32" else dm.BEAM_BF16)
    if cfg.S:
        kw.update(n_shared=cfg.S, I_shared=cfg.I_s, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE)
    if cfg.expert_format == synth.FP8:
        kw.update(expert_format=dm.WEIGHTS_FP8_E4M3, scale_gate=FAKE, scale_up=FAKE, scale_down=FAKE,
                  scale_shared_gate=FAKE, scale_shared_up=FAKE, scale_shared_down=FAKE)
    L = fake_layer(**kw)
    got = dm.beam_moe_stats_host(L, list(counts), T)
    ref = oracle.layer_stats(cfg, counts, T)
    for k, v in ref.items():
        assert got[k] == pytest.approx(v, rel=1e-12, abs=0), k


def test_stats_host_rejects_negative_counts():
    L = fake_layer()
    with pytest.raises(dm.BeamError):
        dm.beam_moe_stats_host(L, [1, -1, 0, 0, 0, 0, 0, 0], 4)


def test_expected_avg_k_hint():
    """expected_avg_k must lie in [0, K]; it only steers the kernel choice:
    for a packed layer without shared experts, the expert-stationary
    kernels (and their workspace) are chosen from T x Avg-K / E >= 256."""
    for bad in (-0.5, 2.5, float("nan"), float("inf")):
        assert dm.beam_moe_workspace_size(fake_layer(expected_avg_k=bad), 16) == 0
    packed = dict(wp_gate=FAKE, wp_up=FAKE, wp_down=FAKE)
    T = 1024   # T x K / E = 256: expert-stationary without a hint
    full = dm.beam_moe_workspace_size(fake_layer(**packed), T)
    thin = dm.beam_moe_workspace_size(fake_layer(expected_avg_k=0.5, **packed), T)
    same = dm.beam_moe_workspace_size(fake_layer(expected_avg_k=2.0, **packed), T)
    assert full == same > thin > 0
    # without packed copies the hint changes nothing
    assert (dm.beam_moe_workspace_size(fake_layer(), T) ==
            dm.beam_moe_workspace_size(fake_layer(expected_avg_k=0.5), T))
    # sizes stay non-decreasing in T with the hint as well
    L = fake_layer(expected_avg_k=1.0, **packed)
    sizes = [dm.beam_moe_workspace_size(L, t) for t in (1, 512, 1024, 2047, 2048, 4096)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
