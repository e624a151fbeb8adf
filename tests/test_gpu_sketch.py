"""Ternary sketch codes and channel statistics built on the device, checked bit
for bit against the CPU oracle and against the host preparation (sketch
switched to the host threads with MOE_SEL_SKETCH=host): the codes, both scales
and the down-column norm of every channel.

The weights span what the exact statistics must survive: magnitudes from
subnormal to 1e36 in one row, all-zero and constant rows, signed zeros, a row
with a single non-zero, other threshold ratios, and the smallest and largest
hidden sizes (64 and 16384)."""
import os

import numpy as np
import pytest

import oracle
from activation_sparse_expert_amd import synth
from gpu_common import torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    torch_cuda()
    from activation_sparse_expert_amd import binding
    return binding


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _export_all(b, cfg, wg, wu, wd, where):
    old = os.environ.get("MOE_SEL_SKETCH")
    os.environ["MOE_SEL_SKETCH"] = where
    try:
        ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    finally:
        if old is None:
            del os.environ["MOE_SEL_SKETCH"]
        else:
            os.environ["MOE_SEL_SKETCH"] = old
    try:
        return [b.moe_sel_export_expert(ctx, e, cfg) for e in range(cfg.n_experts)]
    finally:
        b.moe_sel_destroy(ctx)


def _same(dev, ref, keys=(("tern_gate", "tern_gate"), ("tern_up", "tern_up"), ("alpha_gate", "alpha_gate"),
                          ("alpha_up", "alpha_up"), ("down_norm", "down_norm"))):
    for kd, kr in keys:
        a, r = dev[kd], ref[kr]
        if a.dtype == np.float32:
            a, r = a.view(np.uint32), np.asarray(r, np.float32).view(np.uint32)
        bad = np.argwhere(a != r)
        assert bad.size == 0, (kd, bad[:5])


ORACLE_KEYS = (("tern_gate", "tern_g"), ("tern_up", "tern_u"), ("alpha_gate", "alpha_g"), ("alpha_up", "alpha_u"),
               ("down_norm", "c"))


def _extreme_layer(seed, d, m):
    rng = np.random.default_rng(seed)
    mags = 10.0 ** rng.uniform(-40, 36, size=(m, d))   # below 1e-38 the bf16 values are subnormal
    wg = _bits(rng.standard_normal((m, d)) * mags)
    wu = _bits(rng.standard_normal((m, d)) * 0.02)
    wu[3] = 0                                          # all-zero channel
    wu[4] = _bits(np.full(d, 0.25))                    # constant magnitude: every element is kept
    wu[5] = 0x8000                                     # negative zeros only
    wu[6] = 0
    wu[6, d // 3] = _bits([-3.0])[0]                    # a single non-zero
    wg[7] = _bits(rng.standard_normal(d) * 1e-39)      # subnormal row
    wg[8] = _bits(np.where(rng.random(d) < 0.5, 3e38, 1e-40) * np.sign(rng.standard_normal(d)))
    wd = _bits(rng.standard_normal((d, m)) * 10.0 ** rng.uniform(-30, 30, size=(d, m)))
    return wg, wu, wd


def test_device_sketch_matches_oracle_extreme_magnitudes(b):
    d, m, E = 128, 64, 2
    layers = [_extreme_layer(31 + e, d, m) for e in range(E)]
    wg = np.stack([x[0] for x in layers])
    wu = np.stack([x[1] for x in layers])
    wd = np.stack([x[2] for x in layers])
    cfg = b.make_config(d, E, m, 0, 1)
    dev = _export_all(b, cfg, wg, wu, wd, "device")
    host = _export_all(b, cfg, wg, wu, wd, "host")
    for e in range(E):
        prep = oracle.prepare_expert(wg[e], wu[e], wd[e], 0)
        _same(dev[e], prep, ORACLE_KEYS)
        _same(dev[e], host[e])
        assert dev[e]["alpha_up"][3] == 0 and not dev[e]["tern_up"][3].any()
        assert dev[e]["alpha_up"][5] == 0 and not dev[e]["tern_up"][5].any()
        assert dev[e]["alpha_up"][6] == 3.0 and dev[e]["tern_up"][6, d // 3] == -1


@pytest.mark.parametrize("ratio", [0.3, 1.5, 4.0])
def test_device_sketch_other_ratios_smallest_d(b, ratio):
    rng = np.random.default_rng(41)
    d, m, E = 64, 128, 3
    wg = _bits(rng.laplace(size=(E, m, d)) * 0.02)
    wu = _bits(rng.standard_normal((E, m, d)) * 0.02)
    wd = _bits(rng.standard_normal((E, d, m)) * 0.02)
    cfg = b.make_config(d, E, m, 0, 1, tern_ratio=ratio)
    dev = _export_all(b, cfg, wg, wu, wd, "device")
    for e in range(E):
        _same(dev[e], oracle.prepare_expert(wg[e], wu[e], wd[e], 0, tern_ratio=ratio), ORACLE_KEYS)


def test_device_sketch_largest_hidden_size(b):
    rng = np.random.default_rng(43)
    d, m, E = 16384, 64, 1
    wg = _bits(rng.standard_normal((E, m, d)) * 10.0 ** rng.uniform(-5, 5, size=(E, m, d)))
    wu = _bits(rng.standard_normal((E, m, d)) * 0.02)
    wd = _bits(rng.standard_normal((E, d, m)) * 10.0 ** rng.uniform(-5, 5, size=(E, d, m)))
    cfg = b.make_config(d, E, m, 0, 1)
    dev = _export_all(b, cfg, wg, wu, wd, "device")
    host = _export_all(b, cfg, wg, wu, wd, "host")
    _same(dev[0], host[0])


def test_device_sketch_matches_host_qwen3_layer(b):
    w = synth.WORKLOADS["qwen3"]
    d, m, E = w["d"], w["m"], 8
    wg, wu, wd = synth.layer_weights(w["wid"], 0, E, d, m, w["channel_scale"])
    cfg = b.make_config(d, E, m, 0, min(w["top_e"], E))
    dev = _export_all(b, cfg, wg, wu, wd, "device")
    host = _export_all(b, cfg, wg, wu, wd, "host")
    for e in range(E):
        _same(dev[e], host[e])
