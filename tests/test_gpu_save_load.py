"""A prepared layer written with moe_sel_save and read back with moe_sel_load
gives bit-identical forwards (sparse on both paths, dense) and exports, and the
file written again from the loaded context is byte-identical. Damaged files
(one flipped byte, truncation, trailing bytes) are refused with EIO and leave
nothing behind."""
import numpy as np
import pytest

from activation_sparse_expert_amd import synth
from gpu_common import Layer, to_dev_f32, to_dev_u16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    torch_cuda()
    from activation_sparse_expert_amd import binding
    return binding


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _forwards(b, torch, ctx, d, E, top_e, k, batch):
    x = to_dev_u16(torch, synth.tokens(4, 0, batch, d))
    lg = to_dev_f32(torch, synth.router_logits(4, 0, batch, E))
    outs = []
    for path in (b.MOE_SEL_PATH_AUTO, b.MOE_SEL_PATH_MULTI_KERNEL):
        b.moe_sel_set_path(ctx, path)
        out = torch.zeros((batch, d), dtype=torch.int16, device="cuda")
        b.moe_sel_forward(ctx, x, lg, batch, top_e, k, out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy().copy())
        dense = torch.zeros((batch, d), dtype=torch.int16, device="cuda")
        b.moe_sel_forward_dense(ctx, x, lg, batch, top_e, dense)
        torch.cuda.synchronize()
        outs.append(dense.cpu().numpy().copy())
    b.moe_sel_set_path(ctx, b.MOE_SEL_PATH_AUTO)
    b.moe_sel_check_device(ctx)
    return outs


@pytest.mark.parametrize("name,n_experts", [("tiny", None), ("qwen3", 16)])
def test_save_load_round_trip_is_bit_identical(b, torch, tmp_path, name, n_experts):
    lay = Layer(b, name, max_batch=4, n_experts=n_experts)
    k = synth.WORKLOADS[name]["ks"][0]
    path = tmp_path / "layer.moesel"
    try:
        print(f"[save/load] {name} E={lay.E} k={k}", flush=True)
        before = _forwards(b, torch, lay.ctx, lay.d, lay.E, lay.top_e, k, 3)
        exp_before = [b.moe_sel_export_expert(lay.ctx, e, lay.cfg) for e in (0, lay.E - 1)]
        b.moe_sel_save(lay.ctx, path)
    finally:
        lay.close()
    ctx = b.moe_sel_load(path)
    try:
        cfg = b.moe_sel_get_config(ctx)
        assert (cfg.d, cfg.n_experts, cfg.m, cfg.rank, cfg.max_top_e, cfg.max_batch) == \
            (lay.d, lay.E, lay.m, lay.r, lay.top_e, 4)
        after = _forwards(b, torch, ctx, lay.d, lay.E, lay.top_e, k, 3)
        for u, v in zip(before, after):
            assert np.array_equal(u, v)
        for e, ref in zip((0, lay.E - 1), exp_before):
            got = b.moe_sel_export_expert(ctx, e, lay.cfg)
            for key in ref:
                assert np.array_equal(got[key], ref[key]), (e, key)
        again = tmp_path / "again.moesel"
        b.moe_sel_save(ctx, again)
        assert again.read_bytes() == path.read_bytes()
    finally:
        b.moe_sel_destroy(ctx)


def test_load_refuses_damaged_files(b, tmp_path):
    lay = Layer(b, "tiny", max_batch=2)
    good = tmp_path / "good.moesel"
    try:
        b.moe_sel_save(lay.ctx, good)
    finally:
        lay.close()
    data = bytearray(good.read_bytes())
    flipped = bytearray(data)
    flipped[len(data) // 2] ^= 0x10
    cases = {"checksum": bytes(flipped), "truncated data": bytes(data[:-100]),
             "trailing": bytes(data) + b"\0"}
    for what, blob in cases.items():
        bad = tmp_path / f"bad_{what.replace(' ', '_')}.moesel"
        bad.write_bytes(blob)
        with pytest.raises(b.MoeSelError) as ei:
            b.moe_sel_load(bad)
        assert ei.value.status == b.MOE_SEL_EIO, what
        assert what in str(ei.value), (what, str(ei.value))
    ctx = b.moe_sel_load(good)  # the good file still loads after the failures
    b.moe_sel_destroy(ctx)
