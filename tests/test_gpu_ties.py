"""Exact score ties at the k-th position, on both execution paths.

"Top-k instead of a threshold" (page "KAIST drops calibration from MoE
decoding, speeds up blocks by up to 2.69x over vLLM"): each token keeps its k
highest-scoring channels; equal scores go to the lower channel index (the
reading the oracle's select_topk implements, itself pinned by brute force).

Random weights essentially never give two channels the same binary32 score, so
these tests make ties on purpose: a channel's score depends only on its own
gate row, up row and down column (and the token), so copying one channel's
three vectors into other channel slots gives those slots exactly its score.
The source channel is taken at a chosen rank of the oracle's scores and copied
over channels that score lower, so the plateau of equal scores covers ranks
[above, above + size), around the k-th position. Cases: a pair, a plateau of 40,
a plateau of 300 (more than the 256 candidates the selects rank directly, so
their radix fallback runs), a plateau entirely above the boundary together
with one across it, and x = 0 (every score 0). Shapes: m = 768 on the single launch and
on the multi-kernel path, and m = 14336 on the multi-kernel path (the
sixteen-key-per-thread select). Selections are compared with the oracle bit for
bit; outputs to the usual 2e-2.
"""
import numpy as np
import pytest

import oracle
from activation_sparse_expert_amd import synth
from gpu_common import TOL, out_to_f64, rel_err, to_dev_f32, to_dev_u16, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    from activation_sparse_expert_amd import binding
    return binding


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _weights(seed, E, d, m):
    rng = np.random.default_rng(seed)
    wg = synth.f32_to_bf16_bits(rng.normal(0.0, 0.02, (E, m, d)).astype(np.float32))
    wu = synth.f32_to_bf16_bits(rng.normal(0.0, 0.02, (E, m, d)).astype(np.float32))
    wd = synth.f32_to_bf16_bits(rng.normal(0.0, 0.02, (E, d, m)).astype(np.float32))
    return wg, wu, wd


def _oracle(wg, wu, wd, r):
    E, m, d = wg.shape
    return oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), E, d, m, r)


def _make_plateaus(wg, wu, wd, e, score, k, plateaus, rng):
    """Plateaus of equal scores in expert e. Each (start, size) asks for `size`
    channels of one score whose first rank is `start` (k + start when negative)
    once all plateaus are made: the channel at the matching rank of `score` is
    copied over size - 1 channels drawn from the lower half of the ranking
    (disjoint between plateaus, so copies sit both below and above the source's
    index). Plateaus come in descending rank order; the copies of an earlier one
    rank above every later source. Returns the final first rank of the last."""
    m = score.size
    order = np.lexsort((np.arange(m), -score.astype(np.float64)))
    pool = rng.permutation(order[m // 2:])
    extra = 0
    final = None
    for start, size in plateaus:
        final = start if start >= 0 else k + start
        src = int(order[final - extra])
        dst, pool = pool[:size - 1], pool[size - 1:]
        wg[e, dst] = wg[e, src]
        wu[e, dst] = wu[e, src]
        wd[e][:, dst] = wd[e][:, [src]]
        extra += size - 1
    return final


def _run(b, torch, ctx, d, x_bits, logits, top_e, k, path):
    b.moe_sel_set_path(ctx, path)
    x = to_dev_u16(torch, x_bits)
    lg = to_dev_f32(torch, logits)
    out = torch.zeros((x_bits.shape[0], d), dtype=torch.int16, device="cuda")
    print(f"[ties] path={path} d={d} k={k} B={x_bits.shape[0]}", flush=True)
    b.moe_sel_forward(ctx, x, lg, x_bits.shape[0], top_e, k, out)
    torch.cuda.synchronize()
    b.moe_sel_check_device(ctx)
    return out


def _check(b, torch, ctx, ref, out, bsz, top_e, k, m, path_expected):
    assert b.moe_sel_last_path(ctx) == path_expected
    dbg = b.moe_sel_debug_selection(ctx, bsz, top_e, k, m, with_scores=True)
    assert np.array_equal(dbg["expert_ids"], ref["expert_ids"])
    assert np.all(dbg["chan_count"] == k)
    for t in range(bsz):
        for s in range(top_e):
            assert np.array_equal(dbg["score"][t, s].view(np.uint32), ref["score"][t][s].view(np.uint32)), (t, s)
            assert np.array_equal(dbg["chan_idx"][t, s], ref["sel"][t][s]), (t, s)
    assert rel_err(out_to_f64(torch, out), ref["y"]) <= TOL


# (name, plateaus as (rank of the first tied key, size))
CASES = [
    ("pair", [(-1, 2)]),
    ("plateau40", [(-20, 40)]),
    ("plateau300", [(-120, 300)]),
    ("above_and_across", [(10, 5), (-3, 7)]),
]


def _tie_case(b, torch, d, m, E, top_e, r, k, plateaus, seed, paths):
    wg, wu, wd = _weights(seed, E, d, m)
    rng = np.random.default_rng(seed + 1)
    x = synth.f32_to_bf16_bits(rng.standard_normal((1, d)).astype(np.float32))
    logits = rng.standard_normal((1, E)).astype(np.float32)
    ref0 = _oracle(wg, wu, wd, r).forward(x, logits, top_e, k)
    for s, e in enumerate(ref0["expert_ids"][0]):
        above = _make_plateaus(wg, wu, wd, int(e), ref0["score"][0][s], k, plateaus, rng)
    lay = _oracle(wg, wu, wd, r)
    ref = lay.forward(x, logits, top_e, k)
    assert np.array_equal(ref["expert_ids"], ref0["expert_ids"])
    # the last plateau straddles the k-th position in every routed pair
    size = plateaus[-1][1]
    for s in range(top_e):
        sc = ref["score"][0][s]
        kth = np.sort(sc)[::-1][k - 1]
        assert (sc > kth).sum() == above and (sc == kth).sum() == size
        assert above < k < above + size
    cfg = b.make_config(d, E, m, r, top_e, 2)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    try:
        for path, expect in paths:
            out = _run(b, torch, ctx, d, x, logits, top_e, k, path)
            _check(b, torch, ctx, ref, out, 1, top_e, k, m, expect)
    finally:
        b.moe_sel_destroy(ctx)


@pytest.mark.parametrize("name,plateaus", CASES, ids=[c[0] for c in CASES])
def test_ties_m768_both_paths(b, torch, name, plateaus):
    paths = [(b.MOE_SEL_PATH_SINGLE_LAUNCH, b.MOE_SEL_PATH_SINGLE_LAUNCH),
             (b.MOE_SEL_PATH_MULTI_KERNEL, b.MOE_SEL_PATH_MULTI_KERNEL)]
    _tie_case(b, torch, d=256, m=768, E=8, top_e=2, r=8, k=138, plateaus=plateaus, seed=300, paths=paths)


@pytest.mark.parametrize("name,plateaus", CASES, ids=[c[0] for c in CASES])
def test_ties_m14336_multi_kernel(b, torch, name, plateaus):
    paths = [(b.MOE_SEL_PATH_AUTO, b.MOE_SEL_PATH_MULTI_KERNEL)]
    _tie_case(b, torch, d=128, m=14336, E=2, top_e=1, r=8, k=2580, plateaus=plateaus, seed=400, paths=paths)


@pytest.mark.parametrize("m,k", [(768, 138), (14336, 2580)])
def test_zero_token_takes_lowest_indices(b, torch, m, k):
    """x = 0: every score is 0, so the k lowest channel indices are kept (and the
    output is 0)."""
    d, E, top_e, r = 128, 4, 2, 8
    wg, wu, wd = _weights(500 + m, E, d, m)
    x = np.zeros((1, d), np.uint16)
    logits = np.random.default_rng(m).standard_normal((1, E)).astype(np.float32)
    ref = _oracle(wg, wu, wd, r).forward(x, logits, top_e, k)
    assert all(np.array_equal(ref["sel"][0][s], np.arange(k)) for s in range(top_e))
    cfg = b.make_config(d, E, m, r, top_e, 1)
    ctx = b.moe_sel_prepare(cfg, wg, wu, wd)
    paths = [(b.MOE_SEL_PATH_MULTI_KERNEL, b.MOE_SEL_PATH_MULTI_KERNEL)]
    if m <= 4096:
        paths.append((b.MOE_SEL_PATH_SINGLE_LAUNCH, b.MOE_SEL_PATH_SINGLE_LAUNCH))
    try:
        for path, expect in paths:
            out = _run(b, torch, ctx, d, x, logits, top_e, k, path)
            assert not out.cpu().numpy().any()
            _check(b, torch, ctx, ref, out, 1, top_e, k, m, expect)
    finally:
        b.moe_sel_destroy(ctx)
