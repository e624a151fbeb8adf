"""Rank-r maps built on the device (fp64 Gram matrix, tridiagonalisation and
projection on the GPU) against the host-built maps and against the Eckart-Young
bound from NumPy's singular values."""
import os

import numpy as np
import pytest

from activation_sparse_expert_amd import synth
from gpu_common import torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    torch_cuda()
    from activation_sparse_expert_amd import binding
    return binding


def _maps(b, name, n_experts, where, experts):
    w = synth.WORKLOADS[name]
    d, m, r = w["d"], w["m"], w["rank"]
    wg, wu, wd = synth.layer_weights(w["wid"], 0, n_experts, d, m, w["channel_scale"])
    cfg = b.make_config(d, n_experts, m, r, min(w["top_e"], n_experts), 1)
    old = os.environ.get("MOE_SEL_LOWRANK")
    os.environ["MOE_SEL_LOWRANK"] = where
    try:
        ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    finally:
        if old is None:
            del os.environ["MOE_SEL_LOWRANK"]
        else:
            os.environ["MOE_SEL_LOWRANK"] = old
    try:
        out = []
        for e in experts:
            ex = b.moe_sel_export_expert(ctx, e, cfg)
            p = synth.bf16_bits_to_f32(ex["p_bf16"]).astype(np.float64).reshape(r, d)
            q = synth.bf16_bits_to_f32(ex["q_bf16"]).astype(np.float64).reshape(m, r)
            out.append((p, q, wd[e]))
        return out
    finally:
        b.moe_sel_destroy(ctx)


def test_device_maps_match_host_maps_qwen3_shape(b):
    dev = _maps(b, "qwen3", 3, "device", [0, 2])
    host = _maps(b, "qwen3", 3, "host", [0, 2])
    for (pd, qd, _), (ph, qh, _) in zip(dev, host):
        ad, ah = pd.T @ qd.T, ph.T @ qh.T  # d x m rank-r approximations
        rel = np.linalg.norm(ad - ah) / np.linalg.norm(ah)
        print(f"device vs host rank-r map: relative difference {rel:.2e}")
        assert rel <= 1e-2


def test_device_map_meets_eckart_young_mixtral_shape(b):
    r = synth.WORKLOADS["mixtral"]["rank"]
    (p, q, wd_bits), = _maps(b, "mixtral", 1, "device", [0])
    wd = synth.bf16_bits_to_f32(wd_bits).astype(np.float64)
    approx = p.T @ q.T
    err2 = np.linalg.norm(wd - approx) ** 2
    s = np.linalg.svd(wd, compute_uv=False)
    tail = float((s[r:] ** 2).sum())
    print(f"||W - PQ^T||^2 / optimum = {err2 / tail:.6f}")
    assert err2 <= (1 + 1e-2) * tail
