"""The pinned binary32 silu and channel score on the GPU against the oracle, bit for bit.

The score that decides the selection uses a silu written out from its
definition (Cody & Waite reduction, degree-7 Taylor series, no fused
multiply-add) so that the GPU and the CPU oracle give the same bits and hence
the same top-k ("Top-k instead of a threshold"; channels are filtered by a
ternary sketch, "A reader built from weights alone", page "KAIST drops
calibration from MoE decoding, speeds up blocks by up to 2.69x over vLLM").
These tests evaluate the device function through moe_sel_debug_silu and
moe_sel_debug_score and compare every output bit with oracle.silu_pinned and
oracle.score_from_preacts on:

* a sweep of binary32 bit patterns over [-87, 87] (stride 251, so every low-bit
  residue occurs) on both signs;
* the values next to the cuts at +-87;
* the arguments at which t * L2E lands within a few ulp of a half-integer,
  where the rounding of n = rint(t * L2E) changes;
* zeros, subnormals and the smallest normals;
* channel scores over random integer dots, exponents and statistics, for every
  score kind.

MOE_SEL_EXHAUSTIVE=1 also runs the exhaustive sweep over every binary32 value in
[-87, 87] (about 2.2e9 values, a few minutes).
"""
import os

import numpy as np
import pytest

import oracle
from gpu_common import torch_cuda

pytestmark = pytest.mark.gpu

CUT = 0x42AE0000  # bits of 87.0


@pytest.fixture(scope="module")
def b():
    from activation_sparse_expert_amd import binding
    return binding


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _gpu_silu(b, torch, z):
    zd = torch.from_numpy(np.ascontiguousarray(z, np.float32)).to("cuda")
    out = torch.empty_like(zd)
    b.moe_sel_debug_silu(zd, out, zd.numel())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _compare_silu(b, torch, z):
    got = _gpu_silu(b, torch, z).view(np.uint32)
    ref = oracle.silu_pinned(z).view(np.uint32)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(hex(z.view(np.uint32)[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


def _half_integer_arguments():
    """Arguments z whose t * L2E (t = -z) is within a few ulp of n + 1/2."""
    l2e = float(oracle.ORACLE_CONSTANTS["L2E"])
    out = []
    for n in range(-126, 126):
        z0 = np.float32(-(n + 0.5) / l2e)
        base = np.int64(z0.view(np.uint32))
        for d in range(-6, 7):
            out.append(np.uint32(base + d))
    z = np.array(out, np.uint32).view(np.float32)
    return z[np.abs(z) <= 87.0]


def test_silu_bit_pattern_sweep(b, torch):
    pos = np.arange(0, CUT + 1, 251, dtype=np.uint32)
    z = np.concatenate([pos, pos | np.uint32(0x80000000)]).view(np.float32)
    _compare_silu(b, torch, z)


def test_silu_near_cuts_half_integers_and_subnormals(b, torch):
    near = np.arange(CUT - 512, CUT + 513, dtype=np.uint32)
    small = np.concatenate([np.arange(0, 4096, dtype=np.uint32),                  # zeros, subnormals
                            np.arange(0x00800000 - 64, 0x00800000 + 64, dtype=np.uint32),
                            np.array([0x3F800000, 0x3F000000, 0x33800000], np.uint32)])
    bits = np.concatenate([near, small])
    z = np.concatenate([bits, bits | np.uint32(0x80000000)]).view(np.float32)
    z = np.concatenate([z, _half_integer_arguments()])
    _compare_silu(b, torch, z)
    # beyond the cuts: z itself above +87, +0 below -87
    assert np.array_equal(_gpu_silu(b, torch, np.float32([87.00001, 100.0])), np.float32([87.00001, 100.0]))
    assert not _gpu_silu(b, torch, np.float32([-87.00001, -1e30])).view(np.uint32).any()


@pytest.mark.skipif(os.environ.get("MOE_SEL_EXHAUSTIVE") != "1", reason="set MOE_SEL_EXHAUSTIVE=1")
def test_silu_exhaustive(b, torch):
    chunk = 1 << 26
    for sign in (0, 0x80000000):
        for start in range(0, CUT + 1, chunk):
            bits = np.arange(start, min(start + chunk, CUT + 1), dtype=np.uint32) | np.uint32(sign)
            _compare_silu(b, torch, bits.view(np.float32))
        print(f"sign {sign:#x}: {CUT + 1} values", flush=True)


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_score_from_integer_dots(b, torch, kind):
    rng = np.random.default_rng(20 + kind)
    n = 1 << 20
    lim = 127 * 2048
    dg = rng.integers(-lim, lim + 1, n, dtype=np.int32)
    du = rng.integers(-lim, lim + 1, n, dtype=np.int32)
    dg[:4096] = rng.integers(-64, 65, 4096)  # small dots (|G| near 0, where silu is steep)
    du[4096:8192] = 0
    xexp = rng.integers(-24, 4, n, dtype=np.int32)
    stats = np.zeros((n, 4), np.float32)
    stats[:, 0] = rng.lognormal(np.log(0.03), 0.5, n)
    stats[:, 1] = rng.lognormal(np.log(0.03), 0.5, n)
    stats[:, 2] = rng.lognormal(np.log(0.9), 0.3, n)
    stats[8192:8200, 0] = 0.0  # alpha = 0 (a channel with nothing kept)
    dev = [torch.from_numpy(a).to("cuda") for a in (dg, du, xexp, stats)]
    h = torch.empty(n, dtype=torch.float32, device="cuda")
    sc = torch.empty_like(h)
    b.moe_sel_debug_score(dev[0], dev[1], dev[2], dev[3], kind, h, sc, n)
    torch.cuda.synchronize()
    g, u = oracle.preacts_from_dots(dg, du, xexp, stats[:, 0], stats[:, 1])
    kname = oracle.SCORE_KINDS[kind]
    ref_h, ref_s = oracle.score_from_preacts(g, u, stats[:, 2], kname)
    assert np.array_equal(h.cpu().numpy().view(np.uint32), ref_h.view(np.uint32))
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
