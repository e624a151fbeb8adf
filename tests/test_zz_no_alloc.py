"""moe_sel_forward_noalloc against moe_sel_forward, through the C ABI.

The no-allocation entry point runs the same single-launch kernel with its
per-call scratch in the library's static per-GPU array instead of the
context's workspace, so its outputs must equal moe_sel_forward's bit for bit
(and the oracle's to the usual 2e-2). Two calls in a row, the second with a
smaller input, on the small layer and on the Qwen3-30B-A3B-shaped layer; and
calls the entry point cannot take are refused before anything is enqueued.
"""
import numpy as np
import pytest

from activation_sparse_expert_amd import synth
from gpu_common import TOL, Layer, out_to_f64, rel_err, to_dev_f32, to_dev_u16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from activation_sparse_expert_amd import binding
    return binding


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _both(b, torch, lay, bsz, k, index):
    xb = synth.tokens(lay.w["wid"], 0, bsz, lay.d, index=index)
    lgb = synth.router_logits(lay.w["wid"], 0, bsz, lay.E, index=index)
    x, lg = to_dev_u16(torch, xb), to_dev_f32(torch, lgb)
    ref_out = torch.zeros((bsz, lay.d), dtype=torch.int16, device="cuda")
    na_out = torch.full((bsz, lay.d), 0x7FC0, dtype=torch.int16, device="cuda")
    print(f"[noalloc] {lay.w['wid']} B={bsz} k={k}", flush=True)
    b.moe_sel_forward(lay.ctx, x, lg, bsz, lay.top_e, k, ref_out)
    assert b.moe_sel_last_path(lay.ctx) == b.MOE_SEL_PATH_SINGLE_LAUNCH
    b.moe_sel_forward_noalloc(lay.ctx, x, lg, bsz, lay.top_e, k, na_out)
    torch.cuda.synchronize()
    b.moe_sel_check_device(lay.ctx)
    assert np.array_equal(na_out.cpu().numpy(), ref_out.cpu().numpy())
    ref = lay.oracle.forward(xb, lgb, lay.top_e, k)
    assert rel_err(out_to_f64(torch, na_out), ref["y"]) <= TOL


def test_noalloc_equals_forward_tiny(b, torch):
    lay = Layer(b, "tiny", max_batch=4)
    try:
        _both(b, torch, lay, 4, 92, 11)
        _both(b, torch, lay, 1, 40, 12)  # smaller input second
    finally:
        lay.close()


def test_noalloc_equals_forward_qwen3(b, torch):
    lay = Layer(b, "qwen3", max_batch=1)
    try:
        _both(b, torch, lay, 1, 138, 13)
        _both(b, torch, lay, 1, 100, 14)  # fewer channels second
    finally:
        lay.close()


def test_noalloc_refuses_what_it_cannot_run(b, torch):
    # m above the single launch's limit: refused before anything is enqueued
    d, E, m, r = 64, 2, 8192, 8
    rng = np.random.default_rng(0)
    wg = synth.f32_to_bf16_bits(rng.normal(0, 0.02, (E, m, d)).astype(np.float32))
    wd = synth.f32_to_bf16_bits(rng.normal(0, 0.02, (E, d, m)).astype(np.float32))
    ctx = b.moe_sel_prepare(b.make_config(d, E, m, r, 1, 1), wg, wg, wd)
    try:
        x = torch.zeros((1, d), dtype=torch.int16, device="cuda")
        lg = torch.zeros((1, E), dtype=torch.float32, device="cuda")
        out = torch.full((1, d), 0x1234, dtype=torch.int16, device="cuda")
        with pytest.raises(b.MoeSelError) as ei:
            b.moe_sel_forward_noalloc(ctx, x, lg, 1, 1, 100, out)
        assert ei.value.status == b.MOE_SEL_EUNSUPPORTED
        torch.cuda.synchronize()
        assert (out.cpu().numpy() == 0x1234).all()
    finally:
        b.moe_sel_destroy(ctx)
