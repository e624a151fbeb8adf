"""Shared helpers of the GPU parity tests (imported only by tests marked gpu)."""
import numpy as np

import oracle
from activation_sparse_expert_amd import synth

TOL = 2e-2  # max over tokens of ||out - y_oracle||_inf / ||y_oracle||_inf


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch


def to_dev_u16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def to_dev_f32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def out_to_f64(torch, out):
    bits = out.cpu().numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(bits)


def rel_err(got, ref):
    got = np.atleast_2d(got)
    ref = np.atleast_2d(ref)
    errs = []
    for t in range(ref.shape[0]):
        den = np.abs(ref[t]).max()
        errs.append(np.abs(got[t] - ref[t]).max() / den if den > 0 else np.abs(got[t]).max())
    return max(errs)


class Layer:
    """Weights of one synthetic layer plus the library context and the oracle."""

    def __init__(self, b, name, max_batch=8, layer=0, n_experts=None, rank=None):
        w = synth.WORKLOADS[name]
        self.w = w
        self.d, self.m = w["d"], w["m"]
        self.E = n_experts or w["n_experts"]
        self.top_e = w["top_e"]
        self.r = w["rank"] if rank is None else rank
        self.wg, self.wu, self.wd = synth.layer_weights(w["wid"], layer, self.E, self.d, self.m, w["channel_scale"])
        self.cfg = b.make_config(self.d, self.E, self.m, self.r, self.top_e, max_batch)
        self.ctx = b.moe_sel_prepare(self.cfg, self.wg, self.wu, self.wd)
        self.oracle = oracle.OracleLayer(lambda e: (self.wg[e], self.wu[e], self.wd[e]), self.E, self.d, self.m,
                                         self.r)
        self.b = b

    def close(self):
        self.b.moe_sel_destroy(self.ctx)
