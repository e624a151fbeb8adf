"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Selections (routed experts, channel indices, counts) and the channel scores are
compared bit for bit; outputs to max_t ||out - y||_inf / ||y||_inf <= 2e-2
(bf16 output of an fp32 accumulation against the float64 oracle).
"""
import numpy as np
import pytest

import oracle
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


PATHS = ["single_launch", "multi_kernel"]


@pytest.fixture(scope="module")
def tiny_layer(b, torch):
    lay = Layer(b, "tiny", max_batch=16)
    yield lay
    lay.close()


@pytest.fixture(params=PATHS)
def tiny(request, b, tiny_layer):
    tiny_layer.path = request.param
    b.moe_sel_set_path(tiny_layer.ctx, b.MOE_SEL_PATH_AUTO if request.param == "single_launch"
                       else b.MOE_SEL_PATH_MULTI_KERNEL)
    return tiny_layer


def _run(b, torch, lay, x_bits, logits, k, top_e=None, dense=False):
    top_e = top_e or lay.top_e
    bsz = x_bits.shape[0]
    x = to_dev_u16(torch, x_bits)
    lg = to_dev_f32(torch, logits)
    out = torch.zeros((bsz, lay.d), dtype=torch.int16, device="cuda")
    print(f"[run] {lay.w['wid']} path={getattr(lay, 'path', '?')} B={bsz} top_e={top_e} k={k} dense={dense}",
          flush=True)
    if dense:
        b.moe_sel_forward_dense(lay.ctx, x, lg, bsz, top_e, out)
    else:
        b.moe_sel_forward(lay.ctx, x, lg, bsz, top_e, k, out)
    torch.cuda.synchronize()
    b.moe_sel_check_device(lay.ctx)
    expect = getattr(lay, "path", None)
    if expect == "multi_kernel" or (expect == "single_launch" and bsz <= 8):
        want = b.MOE_SEL_PATH_MULTI_KERNEL if expect == "multi_kernel" else b.MOE_SEL_PATH_SINGLE_LAUNCH
        assert b.moe_sel_last_path(lay.ctx) == want
    return out


def _check_selection(b, lay, ref, bsz, top_e, k, scores=True):
    dbg = b.moe_sel_debug_selection(lay.ctx, bsz, top_e, k, lay.m, with_scores=scores)
    assert np.array_equal(dbg["expert_ids"], ref["expert_ids"])
    assert np.all(dbg["chan_count"] == k)
    for t in range(bsz):
        for s in range(top_e):
            assert np.array_equal(dbg["chan_idx"][t, s], ref["sel"][t][s]), (t, s)
            if scores:
                assert np.array_equal(dbg["score"][t, s].view(np.uint32), ref["score"][t][s].view(np.uint32)), (t, s)
                assert np.array_equal(dbg["h_hat"][t, s].view(np.uint32), ref["h_hat"][t][s].view(np.uint32)), (t, s)
    assert np.allclose(dbg["gate_w"], ref["gate_w"], rtol=1e-5, atol=1e-7)
    return dbg


def test_device_layout_round_trip(b, tiny):
    for e in (0, 7):
        dev = b.moe_sel_export_expert(tiny.ctx, e, tiny.cfg)
        prep = tiny.oracle.expert(e)
        assert np.array_equal(dev["tern_gate"], prep["tern_g"])
        assert np.array_equal(dev["tern_up"], prep["tern_u"])
        assert np.array_equal(dev["alpha_gate"].view(np.uint32), prep["alpha_g"].view(np.uint32))
        assert np.array_equal(dev["down_norm"].view(np.uint32), prep["c"].view(np.uint32))


def test_routing_ties_and_signed_zeros(b, torch, tiny):
    """Equal logits go to the lower expert index, and -0 equals +0 (so a -0 at a
    lower index comes first); each row also runs alone (batch 1)."""
    k = synth.WORKLOADS["tiny"]["ks"][0]
    E = tiny.E
    rows = np.full((4, E), -1.0, np.float32)
    rows[0, :] = np.where(np.arange(E) % 2 == 0, -0.0, 0.0)          # all zero, mixed signs
    rows[1, [5, 2, 7]] = 1.5                                          # a three-way tie
    rows[2, 1], rows[2, 3] = -0.0, 0.0                                # -0 before +0
    rows[3, 3], rows[3, 1] = 0.0, -0.0
    rows[3, 6] = 2.0
    x = synth.tokens(0, 0, 4, tiny.d)
    for lg, xx in [(rows, x)] + [(rows[i:i + 1], x[i:i + 1]) for i in range(4)]:
        bsz = lg.shape[0]
        out = _run(b, torch, tiny, xx, lg, k)
        ref = tiny.oracle.forward(xx, lg, tiny.top_e, k)
        _check_selection(b, tiny, ref, bsz, tiny.top_e, k)
        err = rel_err(out_to_f64(torch, out), ref["y"])
        assert err <= TOL, err
    ids = tiny.oracle.forward(x, rows, tiny.top_e, k)["expert_ids"]
    assert ids[0].tolist() == [0, 1] and ids[1].tolist() == [2, 5] and ids[2].tolist() == [1, 3]
    assert ids[3].tolist() == [6, 1]


def test_tiny_workload_parity(b, torch, tiny):
    k = synth.WORKLOADS["tiny"]["ks"][0]
    x = synth.tokens(0, 0, 1, tiny.d)
    logits = synth.router_logits(0, 0, 1, tiny.E)
    out = _run(b, torch, tiny, x, logits, k)
    ref = tiny.oracle.forward(x, logits, tiny.top_e, k)
    _check_selection(b, tiny, ref, 1, tiny.top_e, k)
    err = rel_err(out_to_f64(torch, out), ref["y"])
    print(f"tiny k={k}: max-rel-err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("k", [0, 1, 3, 91, 255, 511, 512])
def test_budgets_including_edges(b, torch, tiny, k):
    rng = np.random.default_rng(100 + k)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((2, tiny.E)).astype(np.float32)
    out = _run(b, torch, tiny, x, logits, k)
    ref = tiny.oracle.forward(x, logits, tiny.top_e, k)
    _check_selection(b, tiny, ref, 2, tiny.top_e, k)
    assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL


def test_k_equals_m_equals_dense(b, torch, tiny):
    rng = np.random.default_rng(7)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((3, tiny.E)).astype(np.float32)
    full = out_to_f64(torch, _run(b, torch, tiny, x, logits, tiny.m))
    dense = out_to_f64(torch, _run(b, torch, tiny, x, logits, 0, dense=True))
    ref = tiny.oracle.forward_dense(x, logits, tiny.top_e)
    assert rel_err(dense, ref) <= TOL and rel_err(full, ref) <= TOL
    assert rel_err(full, dense) <= 1e-2


@pytest.mark.parametrize("bsz", [8, 16])
def test_batch_rows_match_single_token_calls(b, torch, tiny, bsz):
    rng = np.random.default_rng(8)
    k = 92
    x = synth.f32_to_bf16_bits(rng.standard_normal((bsz, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((bsz, tiny.E)).astype(np.float32)
    outb = _run(b, torch, tiny, x, logits, k).cpu().numpy()
    path_b = b.moe_sel_last_path(tiny.ctx)
    selb = b.moe_sel_debug_selection(tiny.ctx, bsz, tiny.top_e, k, tiny.m, with_scores=False)
    ref = tiny.oracle.forward(x, logits, tiny.top_e, k)
    _check_selection(b, tiny, ref, bsz, tiny.top_e, k)
    assert rel_err(oracle.bf16_bits_to_f64(outb.view(np.uint16)), ref["y"]) <= TOL
    for t in (0, 5):
        out1 = _run(b, torch, tiny, x[t:t + 1], logits[t:t + 1], k).cpu().numpy()
        sel1 = b.moe_sel_debug_selection(tiny.ctx, 1, tiny.top_e, k, tiny.m, with_scores=False)
        assert np.array_equal(sel1["chan_idx"][0], selb["chan_idx"][t])
        if b.moe_sel_last_path(tiny.ctx) == path_b == b.MOE_SEL_PATH_SINGLE_LAUNCH:
            # one block sums a token's terms in the same order at every batch size
            assert np.array_equal(out1[0], outb[t])
        else:
            o1 = oracle.bf16_bits_to_f64(out1[0].view(np.uint16))
            ob = oracle.bf16_bits_to_f64(outb[t].view(np.uint16))
            assert rel_err(o1, ob) <= 1e-2


def test_fewer_experts_than_trained(b, torch, tiny):
    rng = np.random.default_rng(9)
    x = synth.f32_to_bf16_bits(rng.standard_normal((1, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((1, tiny.E)).astype(np.float32)
    out = _run(b, torch, tiny, x, logits, 40, top_e=1)
    ref = tiny.oracle.forward(x, logits, 1, 40)
    _check_selection(b, tiny, ref, 1, 1, 40)
    assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL


def test_degenerate_inputs(b, torch, tiny):
    x = np.zeros((1, tiny.d), np.uint16)
    logits = np.zeros((1, tiny.E), np.float32)
    out = _run(b, torch, tiny, x, logits, 92).cpu().numpy()
    assert not out.any()
    dbg = b.moe_sel_debug_selection(tiny.ctx, 1, tiny.top_e, 92, tiny.m, with_scores=False)
    assert dbg["expert_ids"][0].tolist() == [0, 1]
    assert np.allclose(dbg["gate_w"], 0.5)
    # all-zero scores: the k lowest channel indices
    assert dbg["chan_idx"][0, 0].tolist() == list(range(92))


def test_repeatable_bitwise(b, torch, tiny):
    rng = np.random.default_rng(10)
    x = synth.f32_to_bf16_bits(rng.standard_normal((4, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((4, tiny.E)).astype(np.float32)
    o1 = _run(b, torch, tiny, x, logits, 92).cpu().numpy()
    o2 = _run(b, torch, tiny, x, logits, 92).cpu().numpy()
    assert np.array_equal(o1, o2)


def test_forward_argument_errors(b, torch, tiny):
    x = torch.zeros((1, tiny.d), dtype=torch.int16, device="cuda")
    lg = torch.zeros((1, tiny.E), dtype=torch.float32, device="cuda")
    out = torch.zeros((1, tiny.d), dtype=torch.int16, device="cuda")
    before = out.clone()
    cases = [dict(batch=0), dict(batch=17), dict(top_e=0), dict(top_e=3), dict(k=-1), dict(k=513)]
    for c in cases:
        args = dict(batch=1, top_e=2, k=10)
        args.update(c)
        with pytest.raises(b.MoeSelError) as ei:
            b.moe_sel_forward(tiny.ctx, x, lg, args["batch"], args["top_e"], args["k"], out)
        assert ei.value.status == b.MOE_SEL_EINVAL
    with pytest.raises(b.MoeSelError):
        b.moe_sel_forward(tiny.ctx, x, lg, 1, 2, 10, 0)
    with pytest.raises(b.MoeSelError):
        b.moe_sel_forward(tiny.ctx, x.data_ptr() + 2, lg, 1, 2, 10, out)
    torch.cuda.synchronize()
    assert torch.equal(out, before)


@pytest.fixture(scope="module")
def qwen_layer(b, torch):
    lay = Layer(b, "qwen3", max_batch=4)
    yield lay
    lay.close()


@pytest.fixture(params=PATHS)
def qwen(request, b, qwen_layer):
    qwen_layer.path = request.param
    b.moe_sel_set_path(qwen_layer.ctx, b.MOE_SEL_PATH_AUTO if request.param == "single_launch"
                       else b.MOE_SEL_PATH_MULTI_KERNEL)
    return qwen_layer


@pytest.mark.parametrize("k", [100, 138])
def test_qwen3_shape_parity(b, torch, qwen, k):
    w = synth.WORKLOADS["qwen3"]
    x = synth.tokens(w["wid"], 0, 1, qwen.d)
    logits = synth.router_logits(w["wid"], 0, 1, qwen.E)
    out = _run(b, torch, qwen, x, logits, k)
    ref = qwen.oracle.forward(x, logits, qwen.top_e, k)
    _check_selection(b, qwen, ref, 1, qwen.top_e, k)
    err = rel_err(out_to_f64(torch, out), ref["y"])
    print(f"qwen3 k={k}: max-rel-err {err:.2e}")
    assert err <= TOL
    # the read budget is exactly k of m channels per routed expert
    assert abs(k / qwen.m - {100: 0.13, 138: 0.18}[k]) <= 1 / (2 * qwen.m)


@pytest.mark.parametrize("k", [100, 138])
def test_qwen3_batch2_single_launch(b, torch, qwen_layer, k):
    """Two tokens of the Qwen3 shape fit the single launch at three blocks per
    CU (64-channel score blocks at k = 138: 192 + 288 + 16 + 128 = 624 of 768);
    selections bit-exact and outputs within tolerance. Three tokens do not fit:
    a forced single launch is refused before anything runs."""
    lay = qwen_layer
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_SINGLE_LAUNCH)
    lay.path = "single_launch"
    try:
        w = synth.WORKLOADS["qwen3"]
        x = synth.tokens(w["wid"], 0, 3, lay.d, index=60)
        logits = synth.router_logits(w["wid"], 0, 3, lay.E, index=60)
        out = _run(b, torch, lay, x[:2], logits[:2], k)
        assert b.moe_sel_last_path(lay.ctx) == b.MOE_SEL_PATH_SINGLE_LAUNCH
        ref = lay.oracle.forward(x[:2], logits[:2], lay.top_e, k)
        _check_selection(b, lay, ref, 2, lay.top_e, k)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
        xd, lgd = to_dev_u16(torch, x), to_dev_f32(torch, logits)
        out3 = torch.zeros((3, lay.d), dtype=torch.int16, device="cuda")
        with pytest.raises(b.MoeSelError) as ei:
            b.moe_sel_forward(lay.ctx, xd, lgd, 3, lay.top_e, k, out3)
        assert ei.value.status == b.MOE_SEL_EUNSUPPORTED
    finally:
        b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_AUTO)
        lay.path = None


@pytest.mark.parametrize("top_e,k", [(8, 138), (6, 100)])
def test_qwen3_small_batch_parity(b, torch, qwen_layer, top_e, k):
    """Four tokens on the expert-grouped path: 32 or 24 routed pairs over 128
    experts, so every pair gets a tile of its own (the row kernels, no plan or
    union launch); selections and outputs match the oracle token by token, and
    the dense block of the same tokens stays on expert tiles."""
    lay = qwen_layer
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_MULTI_KERNEL)
    lay.path = "multi_kernel"
    try:
        w = synth.WORKLOADS["qwen3"]
        x = synth.tokens(w["wid"], 0, 4, lay.d, index=40)
        logits = synth.router_logits(w["wid"], 0, 4, lay.E, index=40)
        out = _run(b, torch, lay, x, logits, k, top_e=top_e)
        ref = lay.oracle.forward(x, logits, top_e, k)
        _check_selection(b, lay, ref, 4, top_e, k)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
        dense = _run(b, torch, lay, x, logits, 0, top_e=top_e, dense=True)
        assert rel_err(out_to_f64(torch, dense), lay.oracle.forward_dense(x, logits, top_e)) <= TOL
    finally:
        b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_AUTO)
        lay.path = None


@pytest.mark.parametrize("bsz", [1, 4])
def test_many_experts_parity(b, torch, bsz):
    """320 experts (more than the score blocks route themselves): one pair per
    tile with the routing kernel writing the plan, on the grouped path, at batch
    1 and 4; selections bit-exact, outputs within tolerance."""
    lay = Layer(b, "wide", max_batch=4)
    try:
        b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_MULTI_KERNEL)
        lay.path = "multi_kernel"
        w = synth.WORKLOADS["wide"]
        k = w["ks"][0]
        x = synth.tokens(w["wid"], 0, bsz, lay.d, index=3)
        logits = synth.router_logits(w["wid"], 0, bsz, lay.E, index=3)
        out = _run(b, torch, lay, x, logits, k)
        ref = lay.oracle.forward(x, logits, lay.top_e, k)
        _check_selection(b, lay, ref, bsz, lay.top_e, k)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        lay.close()


def test_qwen3_shape_dense_parity(b, torch, qwen):
    w = synth.WORKLOADS["qwen3"]
    x = synth.tokens(w["wid"], 0, 1, qwen.d, index=1)
    logits = synth.router_logits(w["wid"], 0, 1, qwen.E, index=1)
    out = _run(b, torch, qwen, x, logits, 0, dense=True)
    ref = qwen.oracle.forward_dense(x, logits, qwen.top_e)
    assert rel_err(out_to_f64(torch, out), ref) <= TOL


def test_qwen3_paths_agree_bitwise_on_selection(b, torch, qwen_layer):
    """Both execution paths select the same channels; outputs agree to fp32 summation order."""
    w = synth.WORKLOADS["qwen3"]
    x = synth.tokens(w["wid"], 0, 1, qwen_layer.d, index=2)
    logits = synth.router_logits(w["wid"], 0, 1, qwen_layer.E, index=2)
    outs, sels = [], []
    for path in (b.MOE_SEL_PATH_SINGLE_LAUNCH, b.MOE_SEL_PATH_MULTI_KERNEL):
        b.moe_sel_set_path(qwen_layer.ctx, path)
        qwen_layer.path = None
        outs.append(out_to_f64(torch, _run(b, torch, qwen_layer, x, logits, 138)))
        assert b.moe_sel_last_path(qwen_layer.ctx) == path
        sels.append(b.moe_sel_debug_selection(qwen_layer.ctx, 1, 8, 138, qwen_layer.m, with_scores=True))
    b.moe_sel_set_path(qwen_layer.ctx, b.MOE_SEL_PATH_AUTO)
    for key in ("expert_ids", "chan_idx", "chan_count"):
        assert np.array_equal(sels[0][key], sels[1][key])
    assert np.array_equal(sels[0]["score"].view(np.uint32), sels[1]["score"].view(np.uint32))
    assert rel_err(outs[0], outs[1]) <= 1e-2


def test_graph_replay_matches_eager(b, torch, tiny_layer):
    """A captured sequence of calls replayed several times, with eager work and
    synchronisation in between, reproduces the eager outputs every time."""
    lay = tiny_layer
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_AUTO)
    lay.path = None
    rng = np.random.default_rng(11)
    n = 3
    xs = [to_dev_u16(torch, synth.f32_to_bf16_bits(rng.standard_normal((1, lay.d)).astype(np.float32)))
          for _ in range(n)]
    lgs = [to_dev_f32(torch, rng.standard_normal((1, lay.E)).astype(np.float32)) for _ in range(n)]
    outs = [torch.zeros((1, lay.d), dtype=torch.int16, device="cuda") for _ in range(n)]
    stream = torch.cuda.Stream()
    def calls():
        for i in range(n):
            if i == 1:
                b.moe_sel_forward_dense(lay.ctx, xs[i], lgs[i], 1, lay.top_e, outs[i], stream.cuda_stream)
            else:
                b.moe_sel_forward(lay.ctx, xs[i], lgs[i], 1, lay.top_e, 50 + i, outs[i], stream.cuda_stream)
    with torch.cuda.stream(stream):
        calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert b.moe_sel_last_path(lay.ctx) == b.MOE_SEL_PATH_SINGLE_LAUNCH
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    for rep in range(4):
        for o in outs:
            o.zero_()
        # unrelated eager work on the context between replays
        junk = torch.zeros((1, lay.d), dtype=torch.int16, device="cuda")
        b.moe_sel_forward(lay.ctx, xs[0], lgs[1], 1, lay.top_e, 7, junk)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        b.moe_sel_check_device(lay.ctx)
        for i in range(n):
            assert torch.equal(outs[i], eager[i]), (rep, i)


def test_graph_replay_matches_eager_multi_kernel(b, torch, tiny_layer):
    """The expert-grouped path under graph capture: per-tile arrival counters and
    all workspace state are left clean by every call, so replays reproduce the
    eager outputs."""
    lay = tiny_layer
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_MULTI_KERNEL)
    lay.path = None
    rng = np.random.default_rng(12)
    bsz = 12
    x = to_dev_u16(torch, synth.f32_to_bf16_bits(rng.standard_normal((bsz, lay.d)).astype(np.float32)))
    lg = to_dev_f32(torch, rng.standard_normal((bsz, lay.E)).astype(np.float32))
    outs = [torch.zeros((bsz, lay.d), dtype=torch.int16, device="cuda") for _ in range(2)]
    stream = torch.cuda.Stream()
    def calls():
        b.moe_sel_forward(lay.ctx, x, lg, bsz, lay.top_e, 60, outs[0], stream.cuda_stream)
        b.moe_sel_forward_dense(lay.ctx, x, lg, bsz, lay.top_e, outs[1], stream.cuda_stream)
    with torch.cuda.stream(stream):
        calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    for rep in range(3):
        for o in outs:
            o.zero_()
        junk = torch.zeros((bsz, lay.d), dtype=torch.int16, device="cuda")
        b.moe_sel_forward(lay.ctx, x, lg, bsz, lay.top_e, 5, junk)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], eager[i]), (rep, i)
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_AUTO)


def test_graph_replay_matches_eager_batch1_rows(b, torch, qwen_layer):
    """The batch-1 grouped kernels (the score blocks route and write the plan,
    row-streaming gate/up and down) under graph capture: sparse, fewer experts,
    dense and threshold calls replayed several times, with batch-4 calls that
    rewrite the plan and unions in between, reproduce the eager outputs."""
    lay = qwen_layer
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_MULTI_KERNEL)
    lay.path = None
    w = synth.WORKLOADS["qwen3"]
    n = 4
    xh = [synth.tokens(w["wid"], 0, 1, lay.d, index=20 + i) for i in range(n)]
    lh = [synth.router_logits(w["wid"], 0, 1, lay.E, index=20 + i) for i in range(n)]
    xs = [to_dev_u16(torch, v) for v in xh]
    lgs = [to_dev_f32(torch, v) for v in lh]
    outs = [torch.zeros((1, lay.d), dtype=torch.int16, device="cuda") for _ in range(n)]
    stream = torch.cuda.Stream()
    s = stream.cuda_stream

    def calls():
        b.moe_sel_forward(lay.ctx, xs[0], lgs[0], 1, lay.top_e, 138, outs[0], s)
        b.moe_sel_forward(lay.ctx, xs[1], lgs[1], 1, 6, 100, outs[1], s)
        b.moe_sel_forward_dense(lay.ctx, xs[2], lgs[2], 1, lay.top_e, outs[2], s)
        b.moe_sel_forward_threshold(lay.ctx, xs[3], lgs[3], 1, lay.top_e, 0.3, outs[3], s)

    with torch.cuda.stream(stream):
        calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    # the eager outputs are the oracle's to the usual tolerance
    ref = lay.oracle.forward(xh[0], lh[0], lay.top_e, 138)
    assert rel_err(out_to_f64(torch, eager[0]), ref["y"]) <= TOL
    xb = to_dev_u16(torch, synth.tokens(w["wid"], 0, 4, lay.d, index=30))
    lb = to_dev_f32(torch, synth.router_logits(w["wid"], 0, 4, lay.E, index=30))
    junk = torch.zeros((4, lay.d), dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        calls()
    for rep in range(3):
        for o in outs:
            o.zero_()
        b.moe_sel_forward(lay.ctx, xb, lb, 4, lay.top_e, 77 + rep, junk)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        b.moe_sel_check_device(lay.ctx)
        for i in range(n):
            assert torch.equal(outs[i], eager[i]), (rep, i)
    b.moe_sel_set_path(lay.ctx, b.MOE_SEL_PATH_AUTO)


def test_tiles_split_across_many_tokens_per_expert(b, torch):
    """200 tokens over 8 experts (top-2): experts receive more tokens than one
    expert tile holds, so their pairs span several tiles; every token still
    matches the oracle."""
    lay = Layer(b, "tiny", max_batch=200)
    try:
        rng = np.random.default_rng(13)
        bsz, k = 200, 92
        x = synth.f32_to_bf16_bits(rng.standard_normal((bsz, lay.d)).astype(np.float32))
        logits = rng.standard_normal((bsz, lay.E)).astype(np.float32)
        logits[:, 3] += 2.0  # expert 3 takes most tokens
        lay.path = "multi_kernel"
        out = _run(b, torch, lay, x, logits, k)
        ref = lay.oracle.forward(x, logits, lay.top_e, k)
        assert (ref["expert_ids"] == 3).sum() > 128
        _check_selection(b, lay, ref, bsz, lay.top_e, k)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
        dense = _run(b, torch, lay, x, logits, 0, dense=True)
        assert rel_err(out_to_f64(torch, dense), lay.oracle.forward_dense(x, logits, lay.top_e)) <= TOL
    finally:
        lay.close()


@pytest.mark.parametrize("k", [1, 5, 40])
def test_expert_tile_work_items_small_budgets(b, torch, k):
    """Expert tiles of 1 to 32 tokens with budgets that leave most of each
    tile's m/16 channel chunks empty: the gate/up work items are laid out for
    at most n k union channels per tile (n tokens), so small budgets give tiles
    fewer items than chunks, and a tile of many tokens more items than its union
    fills. Selections and outputs match the oracle."""
    lay = Layer(b, "tiny", max_batch=96)
    try:
        rng = np.random.default_rng(29 + k)
        bsz = 96
        x = synth.f32_to_bf16_bits(rng.standard_normal((bsz, lay.d)).astype(np.float32))
        logits = rng.standard_normal((bsz, lay.E)).astype(np.float32)
        logits[:, 5] += 1.5  # one expert takes about three tiles of tokens, another few
        logits[:, 6] -= 2.0
        lay.path = "multi_kernel"
        out = _run(b, torch, lay, x, logits, k)
        ref = lay.oracle.forward(x, logits, lay.top_e, k)
        assert (ref["expert_ids"] == 5).sum() > 64
        _check_selection(b, lay, ref, bsz, lay.top_e, k)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        lay.close()


def test_qwen3_batch64_zipf_parity(b, torch):
    """Qwen3-shaped block at 64 decode tokens with Zipf(1.1)-skewed routing: the
    per-expert union path selects each token's own channels bit for bit and every
    token's output is within tolerance."""
    w = synth.WORKLOADS["qwen3_b64"]
    lay = Layer(b, "qwen3_b64", max_batch=64)
    try:
        bsz, k = 64, w["ks"][0]
        x = synth.tokens(w["wid"], 0, bsz, lay.d)
        logits = synth.router_logits(w["wid"], 0, bsz, lay.E, "zipf")
        lay.path = None
        out = _run(b, torch, lay, x, logits, k)
        assert b.moe_sel_last_path(lay.ctx) == b.MOE_SEL_PATH_MULTI_KERNEL
        ref = lay.oracle.forward(x, logits, lay.top_e, k)
        counts = np.bincount(ref["expert_ids"].ravel(), minlength=lay.E)
        print(f"experts used {np.count_nonzero(counts)}, hottest {counts.max()} tokens")
        _check_selection(b, lay, ref, bsz, lay.top_e, k)
        err = rel_err(out_to_f64(torch, out), ref["y"])
        print(f"qwen3 batch 64 zipf k={k}: max-rel-err {err:.2e}")
        assert err <= TOL
    finally:
        lay.close()


@pytest.fixture(scope="module")
def mixtral(b, torch):
    """Two Mixtral-8x7B-shaped experts (d=4096, m=14336, r=64, per-channel
    LogNormal scales); with top-2 routing both are routed for every token."""
    lay = Layer(b, "mixtral", max_batch=1, n_experts=2)
    yield lay
    lay.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("k", [1864, 2580])
def test_mixtral_shape_parity(b, torch, mixtral, k):
    w = synth.WORKLOADS["mixtral"]
    x = synth.tokens(w["wid"], 0, 1, mixtral.d)
    logits = synth.router_logits(w["wid"], 0, 1, mixtral.E)
    mixtral.path = None
    out = _run(b, torch, mixtral, x, logits, k)
    assert b.moe_sel_last_path(mixtral.ctx) == b.MOE_SEL_PATH_MULTI_KERNEL
    ref = mixtral.oracle.forward(x, logits, mixtral.top_e, k)
    _check_selection(b, mixtral, ref, 1, mixtral.top_e, k)
    err = rel_err(out_to_f64(torch, out), ref["y"])
    print(f"mixtral k={k}: max-rel-err {err:.2e}")
    assert err <= TOL
    assert abs(k / mixtral.m - {1864: 0.13, 2580: 0.18}[k]) <= 1 / (2 * mixtral.m)


@pytest.mark.parametrize("top_e", [4, 2])
def test_qwen3_fewer_routed_experts_than_trained(b, torch, qwen, top_e):
    """Routing to fewer experts than the trained top-8, composed with the budget."""
    w = synth.WORKLOADS["qwen3"]
    x = synth.tokens(w["wid"], 0, 1, qwen.d, index=3)
    logits = synth.router_logits(w["wid"], 0, 1, qwen.E, index=3)
    out = _run(b, torch, qwen, x, logits, 138, top_e=top_e)
    ref = qwen.oracle.forward(x, logits, top_e, 138)
    _check_selection(b, qwen, ref, 1, top_e, 138)
    assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL


@pytest.mark.parametrize("kind", ["gate_only", "no_down_norm"])
def test_score_ablation_kinds_match_oracle(b, torch, tiny, kind):
    code = {"gate_only": b.MOE_SEL_SCORE_GATE_ONLY, "no_down_norm": b.MOE_SEL_SCORE_NO_DOWN_NORM}[kind]
    rng = np.random.default_rng(30)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((3, tiny.E)).astype(np.float32)
    b.moe_sel_set_score(tiny.ctx, code)
    try:
        out = _run(b, torch, tiny, x, logits, 92)
        ref = tiny.oracle.forward(x, logits, tiny.top_e, 92, score_kind=kind)
        _check_selection(b, tiny, ref, 3, tiny.top_e, 92)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        b.moe_sel_set_score(tiny.ctx, b.MOE_SEL_SCORE_FULL)
    with pytest.raises(b.MoeSelError):
        b.moe_sel_set_score(tiny.ctx, 7)


def test_int16_activation_score_single_launch_and_unsupported_paths(b, torch, tiny):
    """The int16-activation score ablation: bit-exact selections and scores on the
    single launch; multi-kernel calls whose score blocks do not quantise x
    themselves refuse it with EUNSUPPORTED."""
    rng = np.random.default_rng(31)
    x = synth.f32_to_bf16_bits(rng.standard_normal((3, tiny.d)).astype(np.float32))
    logits = rng.standard_normal((3, tiny.E)).astype(np.float32)
    b.moe_sel_set_score(tiny.ctx, b.MOE_SEL_SCORE_X_INT16)
    try:
        if tiny.path == "single_launch":
            out = _run(b, torch, tiny, x, logits, 92)
            ref = tiny.oracle.forward(x, logits, tiny.top_e, 92, score_kind="x_int16")
            _check_selection(b, tiny, ref, 3, tiny.top_e, 92)
            assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
            ref8 = tiny.oracle.forward(x, logits, tiny.top_e, 92)
            assert any(not np.array_equal(u, v) for u, v in zip(ref["h_hat"][0], ref8["h_hat"][0]))
        else:
            for bsz in (3, 1):
                with pytest.raises(b.MoeSelError) as ei:
                    _run(b, torch, tiny, x[:bsz], logits[:bsz], 92)
                assert ei.value.status == b.MOE_SEL_EUNSUPPORTED
    finally:
        b.moe_sel_set_score(tiny.ctx, b.MOE_SEL_SCORE_FULL)


def test_int16_activation_score_batch1_rows(b, torch, qwen):
    """Batch-1 calls on both paths: the single launch and the multi-kernel path
    with one pair per tile (its score blocks route and quantise x themselves)."""
    w = synth.WORKLOADS["qwen3"]
    x = synth.tokens(w["wid"], 0, 1, qwen.d, index=5)
    logits = synth.router_logits(w["wid"], 0, 1, qwen.E, index=5)
    b.moe_sel_set_score(qwen.ctx, b.MOE_SEL_SCORE_X_INT16)
    try:
        out = _run(b, torch, qwen, x, logits, 138)
        ref = qwen.oracle.forward(x, logits, qwen.top_e, 138, score_kind="x_int16")
        _check_selection(b, qwen, ref, 1, qwen.top_e, 138)
        assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        b.moe_sel_set_score(qwen.ctx, b.MOE_SEL_SCORE_FULL)


@pytest.mark.parametrize("d", [64, 192])
@pytest.mark.parametrize("path", PATHS)
def test_small_and_uneven_hidden_sizes(b, torch, d, path):
    """Hidden sizes below four 64-element blocks (some score-block quarters of d are
    empty) and an odd block count, on both paths, batch 1 and 3."""
    E, m, top_e, r, k = 4, 128, 2, 8, 24
    wg, wu, wd = synth.layer_weights(0, 9, E, d, m)
    cfg = b.make_config(d, E, m, r, top_e, 4)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    try:
        b.moe_sel_set_path(ctx, b.MOE_SEL_PATH_AUTO if path == "single_launch" else b.MOE_SEL_PATH_MULTI_KERNEL)
        ref_layer = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), E, d, m, r)
        for bsz in (1, 3):
            x = synth.tokens(0, 9, bsz, d, index=d)
            logits = synth.router_logits(0, 9, bsz, E, index=d)
            print(f"[run] d={d} path={path} B={bsz}", flush=True)
            out = torch.zeros((bsz, d), dtype=torch.int16, device="cuda")
            b.moe_sel_forward(ctx, to_dev_u16(torch, x), to_dev_f32(torch, logits), bsz, top_e, k, out)
            torch.cuda.synchronize()
            b.moe_sel_check_device(ctx)
            want = b.MOE_SEL_PATH_SINGLE_LAUNCH if path == "single_launch" else b.MOE_SEL_PATH_MULTI_KERNEL
            assert b.moe_sel_last_path(ctx) == want
            ref = ref_layer.forward(x, logits, top_e, k)
            dbg = b.moe_sel_debug_selection(ctx, bsz, top_e, k, m, with_scores=True)
            assert np.array_equal(dbg["expert_ids"], ref["expert_ids"])
            for t in range(bsz):
                for s in range(top_e):
                    assert np.array_equal(dbg["chan_idx"][t, s], ref["sel"][t][s]), (t, s)
                    assert np.array_equal(dbg["score"][t, s].view(np.uint32), ref["score"][t][s].view(np.uint32))
            assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        b.moe_sel_destroy(ctx)


@pytest.mark.parametrize("path", PATHS)
def test_wide_rank_score_blocks_of_64_channels(b, torch, path):
    """Rank 64 with 1024 channels: 32-channel score blocks would leave the
    rank-r partial sums more slots than a z block holds, so the single launch
    scores 64 channels per block (the multi-kernel path is the control).
    Selections and scores bit-exact, outputs within tolerance, batch 1 and 2."""
    E, d, m, r, top_e, k = 8, 512, 1024, 64, 4, 133
    wg, wu, wd = synth.layer_weights(0, 11, E, d, m)
    cfg = b.make_config(d, E, m, r, top_e, 2)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    try:
        want = b.MOE_SEL_PATH_SINGLE_LAUNCH if path == "single_launch" else b.MOE_SEL_PATH_MULTI_KERNEL
        b.moe_sel_set_path(ctx, want)
        ref_layer = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), E, d, m, r)
        for bsz in (1, 2):
            x = synth.tokens(0, 11, bsz, d, index=bsz)
            logits = synth.router_logits(0, 11, bsz, E, index=bsz)
            print(f"[run] m={m} r={r} path={path} B={bsz}", flush=True)
            out = torch.zeros((bsz, d), dtype=torch.int16, device="cuda")
            b.moe_sel_forward(ctx, to_dev_u16(torch, x), to_dev_f32(torch, logits), bsz, top_e, k, out)
            torch.cuda.synchronize()
            b.moe_sel_check_device(ctx)
            assert b.moe_sel_last_path(ctx) == want
            ref = ref_layer.forward(x, logits, top_e, k)
            dbg = b.moe_sel_debug_selection(ctx, bsz, top_e, k, m, with_scores=True)
            assert np.array_equal(dbg["expert_ids"], ref["expert_ids"])
            for t in range(bsz):
                for s in range(top_e):
                    assert np.array_equal(dbg["chan_idx"][t, s], ref["sel"][t][s]), (t, s)
                    assert np.array_equal(dbg["score"][t, s].view(np.uint32), ref["score"][t][s].view(np.uint32))
            assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        b.moe_sel_destroy(ctx)


@pytest.mark.parametrize("m", [2048, 4096])
@pytest.mark.parametrize("path", PATHS)
def test_many_channels_single_launch_select(b, torch, m, path):
    """More than 1024 channels per expert, up to the single launch's largest
    (4096): the gather and z blocks select with sixteen key slots per thread
    (the multi-kernel path is the control). Selections and scores bit-exact,
    outputs within tolerance, batch 1 and 2 (batch 1 only at 4096 channels,
    where the grid of two tokens no longer fits on the chip at once)."""
    E, d, r, top_e = 4, 256, 8, 2
    k = (m * 3) // 20  # 15% of the channels
    wg, wu, wd = synth.layer_weights(0, 13, E, d, m)
    cfg = b.make_config(d, E, m, r, top_e, 2)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    try:
        want = b.MOE_SEL_PATH_SINGLE_LAUNCH if path == "single_launch" else b.MOE_SEL_PATH_MULTI_KERNEL
        b.moe_sel_set_path(ctx, want)
        ref_layer = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), E, d, m, r)
        for bsz in ((1, 2) if m < 4096 else (1,)):
            x = synth.tokens(0, 13, bsz, d, index=m + bsz)
            logits = synth.router_logits(0, 13, bsz, E, index=m + bsz)
            print(f"[run] m={m} k={k} path={path} B={bsz}", flush=True)
            out = torch.zeros((bsz, d), dtype=torch.int16, device="cuda")
            b.moe_sel_forward(ctx, to_dev_u16(torch, x), to_dev_f32(torch, logits), bsz, top_e, k, out)
            torch.cuda.synchronize()
            b.moe_sel_check_device(ctx)
            assert b.moe_sel_last_path(ctx) == want
            ref = ref_layer.forward(x, logits, top_e, k)
            dbg = b.moe_sel_debug_selection(ctx, bsz, top_e, k, m, with_scores=True)
            assert np.array_equal(dbg["expert_ids"], ref["expert_ids"])
            for t in range(bsz):
                for s in range(top_e):
                    assert np.array_equal(dbg["chan_idx"][t, s], ref["sel"][t][s]), (t, s)
                    assert np.array_equal(dbg["score"][t, s].view(np.uint32), ref["score"][t][s].view(np.uint32))
            assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        b.moe_sel_destroy(ctx)


@pytest.mark.parametrize("E", [192, 256])
@pytest.mark.parametrize("path", PATHS)
def test_routing_up_to_256_experts_with_ties(b, torch, E, path):
    """Routing ranks for 129 to 256 experts (four keys per lane, a padded last
    lane block at 192) with heavy ties among the logits and signed zeros: the
    routed experts, selections and scores bit-exact against the oracle, outputs
    within tolerance, batch 1 and 2."""
    d, m, r, top_e, k = 128, 256, 8, 8, 40
    wg, wu, wd = synth.layer_weights(0, 17, E, d, m)
    cfg = b.make_config(d, E, m, r, top_e, 2)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    try:
        want = b.MOE_SEL_PATH_SINGLE_LAUNCH if path == "single_launch" else b.MOE_SEL_PATH_MULTI_KERNEL
        b.moe_sel_set_path(ctx, want)
        ref_layer = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), E, d, m, r)
        rng = np.random.default_rng(E)
        for bsz in (1, 2):
            x = synth.tokens(0, 17, bsz, d, index=E + bsz)
            logits = (rng.integers(-3, 4, size=(bsz, E)) * 0.5).astype(np.float32)  # few distinct values
            logits[logits == 0] = np.where(rng.random(int((logits == 0).sum())) < 0.5, -0.0, 0.0)
            print(f"[run] E={E} path={path} B={bsz}", flush=True)
            out = torch.zeros((bsz, d), dtype=torch.int16, device="cuda")
            b.moe_sel_forward(ctx, to_dev_u16(torch, x), to_dev_f32(torch, logits), bsz, top_e, k, out)
            torch.cuda.synchronize()
            b.moe_sel_check_device(ctx)
            assert b.moe_sel_last_path(ctx) == want
            ref = ref_layer.forward(x, logits, top_e, k)
            dbg = b.moe_sel_debug_selection(ctx, bsz, top_e, k, m, with_scores=True)
            assert np.array_equal(dbg["expert_ids"], ref["expert_ids"])
            for t in range(bsz):
                for s in range(top_e):
                    assert np.array_equal(dbg["chan_idx"][t, s], ref["sel"][t][s]), (t, s)
                    assert np.array_equal(dbg["score"][t, s].view(np.uint32), ref["score"][t][s].view(np.uint32))
            assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL
    finally:
        b.moe_sel_destroy(ctx)
