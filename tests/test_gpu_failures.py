"""Failure handling on the GPU, forced from the host so that every kernel still
finishes normally.

* A cross-workgroup wait of the single-launch kernel that gives up (the host
  sets a wait limit of 0 polls, so every wait gives up at once) turns the
  outputs of the call into NaN and sets the error that moe_sel_check_device
  reports; while that error is set, later single-launch calls write NaN too;
  after moe_sel_check_device the context computes correct outputs again.
* Allocation failures injected at every allocation of moe_sel_prepare and
  moe_sel_load return MOE_SEL_ENOMEM and leave no device memory behind.
* moe_sel_export_expert returns the sketch's kept-entry counts, equal to the
  oracle's.
"""
import numpy as np
import pytest

from activation_sparse_expert_amd import synth
from gpu_common import TOL, Layer, rel_err, to_dev_f32, to_dev_u16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from activation_sparse_expert_amd import binding
    return binding


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _is_nan_bf16(bits):
    bits = np.asarray(bits).view(np.uint16)
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def _forward(b, torch, lay, x, lg, k):
    out = torch.zeros((x.shape[0], lay.d), dtype=torch.int16, device="cuda")
    b.moe_sel_forward(lay.ctx, x, lg, x.shape[0], lay.top_e, k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name,bsz", [("tiny", 2), ("qwen3", 1)])
def test_wait_that_gives_up_poisons_until_checked(b, torch, name, bsz):
    lay = Layer(b, name, max_batch=bsz)
    try:
        k = synth.WORKLOADS[name]["ks"][0]
        xb = synth.tokens(lay.w["wid"], 0, bsz, lay.d, index=5)
        lgb = synth.router_logits(lay.w["wid"], 0, bsz, lay.E, index=5)
        x, lg = to_dev_u16(torch, xb), to_dev_f32(torch, lgb)
        ref = lay.oracle.forward(xb, lgb, lay.top_e, k)
        print(f"[failures] {name}: normal call", flush=True)
        ok = _forward(b, torch, lay, x, lg, k)
        assert b.moe_sel_last_path(lay.ctx) == b.MOE_SEL_PATH_SINGLE_LAUNCH
        b.moe_sel_check_device(lay.ctx)
        assert rel_err(oracle_f64(ok), ref["y"]) <= TOL
        print(f"[failures] {name}: every wait gives up", flush=True)
        b.moe_sel_set_wait_limit(lay.ctx, 0)
        bad = _forward(b, torch, lay, x, lg, k)
        assert _is_nan_bf16(bad).all()
        b.moe_sel_set_wait_limit(lay.ctx, 1 << 21)
        print(f"[failures] {name}: sticky error", flush=True)
        still = _forward(b, torch, lay, x, lg, k)
        assert _is_nan_bf16(still).all()
        with pytest.raises(b.MoeSelError) as ei:
            b.moe_sel_check_device(lay.ctx)
        assert ei.value.status == b.MOE_SEL_EDEVICE
        print(f"[failures] {name}: after the reset", flush=True)
        again = _forward(b, torch, lay, x, lg, k)
        b.moe_sel_check_device(lay.ctx)
        assert rel_err(oracle_f64(again), ref["y"]) <= TOL
    finally:
        lay.close()


def oracle_f64(bits):
    import oracle
    return oracle.bf16_bits_to_f64(np.asarray(bits).view(np.uint16))


def test_export_returns_kept_counts(b, torch):
    lay = Layer(b, "tiny", max_batch=1)
    try:
        for e in (0, lay.E - 1):
            dev = b.moe_sel_export_expert(lay.ctx, e, lay.cfg)
            prep = lay.oracle.expert(e)
            assert np.array_equal(dev["nnz_gate"], prep["nnz_g"])
            assert np.array_equal(dev["nnz_up"], prep["nnz_u"])
            assert np.array_equal(dev["nnz_gate"], (dev["tern_gate"] != 0).sum(axis=1))
    finally:
        lay.close()


def _free_bytes(torch):
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_injected_allocation_failures_leave_nothing_behind(b, torch, tmp_path):
    w = synth.WORKLOADS["tiny"]
    d, m, E, r = w["d"], w["m"], w["n_experts"], w["rank"]
    wg, wu, wd = synth.layer_weights(w["wid"], 0, E, d, m, w["channel_scale"])
    cfg = b.make_config(d, E, m, r, w["top_e"], 4)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)  # warm up the runtime before measuring
    path = str(tmp_path / "layer.moesel")
    b.moe_sel_save(ctx, path)
    b.moe_sel_destroy(ctx)
    free0 = _free_bytes(torch)
    for what in ("prepare", "load"):
        hit = 0
        for n in range(1, 200):
            b.moe_sel_debug_fail_alloc(n)
            try:
                c = b.moe_sel_prepare(cfg, wg, wu, wd) if what == "prepare" else b.moe_sel_load(path)
            except b.MoeSelError as e:
                assert e.status == b.MOE_SEL_ENOMEM, (what, n, str(e))
                hit += 1
                continue
            b.moe_sel_debug_fail_alloc(0)
            b.moe_sel_destroy(c)
            break
        else:
            pytest.fail(f"{what}: still failing after 200 allocations")
        print(f"[failures] {what}: {hit} injected failures, all ENOMEM", flush=True)
        assert hit >= 20
    free1 = _free_bytes(torch)
    assert free1 >= free0 - (2 << 20), (free0, free1)
