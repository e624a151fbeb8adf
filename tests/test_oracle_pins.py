"""Pins of the CPU oracle against things other than itself.

Closed forms, brute force on tiny inputs, exact rational arithmetic, hand-derived
fixtures under tests/golden/ and textbook special cases. A plausible slip in the
oracle (a dropped term, a wrong sign, a transposed operand, a wrong tie rule)
fails at least one of these.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import moe_oracle as om
from activation_sparse_expert_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _bits(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ---------------------------------------------------------------- silu_pinned
def _ulp_err(got: np.ndarray, exact: np.ndarray) -> np.ndarray:
    ex32 = exact.astype(F32)
    ulp = np.spacing(np.abs(ex32)).astype(np.float64)
    ulp = np.maximum(ulp, np.spacing(F32(0)).astype(np.float64))
    return np.abs(got.astype(np.float64) - exact) / ulp


def test_silu_pinned_within_4_ulp_of_float64_silu():
    z = np.concatenate([
        np.linspace(-87, 87, 1_000_003, dtype=np.float64),
        np.linspace(-1, 1, 200_001),
        np.geomspace(1e-30, 87, 20_000), -np.geomspace(1e-30, 87, 20_000),
        [0.0, 87.0, -87.0, 0.5 * math.log(2), -0.5 * math.log(2)],
    ]).astype(F32)
    got = oracle.silu_pinned(z)
    zz = z.astype(np.float64)
    exact = zz / (1.0 + np.exp(-zz))
    err = _ulp_err(got, exact)
    assert err.max() <= 4.0, (err.max(), z[np.argmax(err)])


def test_silu_pinned_cutoffs_and_sign():
    z = np.array([87.00001, 100, 3e38, -87.00001, -100, -3e38], dtype=F32)
    got = oracle.silu_pinned(z)
    assert np.array_equal(got[:3], z[:3])
    assert np.all(got[3:] == 0) and not np.any(np.signbit(got[3:]))
    # silu is negative on (-87, 0) and positive on (0, 87)
    s = oracle.silu_pinned(np.array([-50, -1, -1e-3, 1e-3, 1, 50], dtype=F32))
    assert np.all(s[:3] < 0) and np.all(s[3:] > 0)


def test_silu_pinned_constants_from_their_definitions():
    c = oracle.ORACLE_CONSTANTS
    # LN2_HI has 12 fractional bits and the split sums to ln 2 far below binary32 precision
    assert float(c["LN2_HI"]) * 4096 == int(float(c["LN2_HI"]) * 4096)
    assert abs(float(c["LN2_HI"]) + float(c["LN2_LO"]) - math.log(2)) < 2.0 ** -36
    assert abs(float(c["L2E"]) * math.log(2) - 1) < 2.0 ** -24
    for k, v in enumerate(c["INV_FACT"]):
        assert abs(float(v) * math.factorial(k) - 1) <= 2.0 ** -24


# ---------------------------------------------------------------- top-k select
def _brute_topk(score, k):
    """The unique k-subset whose members all precede all non-members in the order
    (higher score first, lower index first on equal scores): enumerated, no sort."""
    m = len(score)
    found = []
    for sub in itertools.combinations(range(m), k):
        inside = set(sub)
        ok = all((score[i] > score[j]) or (score[i] == score[j] and i < j)
                 for i in inside for j in range(m) if j not in inside)
        if ok:
            found.append(sub)
    assert len(found) == 1
    return list(found[0])


def test_topk_hand_cases():
    with open(os.path.join(GOLDEN, "topk_hand_cases.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 8
    for ln in rows:
        sc, k, exp = (p.strip() for p in ln.split("|"))
        score = np.array([float(v) for v in sc.split()], dtype=F32)
        expected = [int(v) for v in exp.split()]
        assert oracle.select_topk(score, int(k)).tolist() == expected, ln


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(300):
        m = int(rng.integers(1, 9))
        levels = rng.choice([1, 2, 3, 8], p=[0.2, 0.3, 0.3, 0.2])
        score = rng.integers(0, levels, size=m).astype(F32) * F32(0.25)
        for k in range(m + 1):
            got = oracle.select_topk(score, k).tolist()
            assert got == _brute_topk(score.tolist(), k), (score, k)


def test_topk_exact_count_and_separation():
    rng = np.random.default_rng(2)
    for m, k in [(512, 92), (768, 100), (768, 138), (14336, 2580)]:
        score = np.abs(rng.standard_normal(m)).astype(F32)
        score[rng.integers(0, m, size=m // 4)] = score[0]        # plateaus
        sel = oracle.select_topk(score, k)
        assert len(sel) == k and len(set(sel.tolist())) == k
        assert np.all(np.diff(sel) > 0)
        mask = np.zeros(m, bool)
        mask[sel] = True
        if 0 < k < m:
            lo = score[mask].min()
            hi = score[~mask].max()
            assert lo >= hi
            # ties straddling the boundary go to the lower indices
            if lo == hi:
                assert np.where(mask & (score == lo))[0].max() < np.where(~mask & (score == lo))[0].min()


# ---------------------------------------------------------------- routing
def test_route_brute_force_and_weights():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n_exp = int(rng.integers(2, 9))
        top_e = int(rng.integers(1, n_exp + 1))
        logits = (rng.integers(0, 4, size=n_exp) * 0.5).astype(F32)
        ids, w = oracle.route(logits, top_e)
        order_key = sorted(range(n_exp), key=lambda i: (-float(logits[i]), i))
        assert ids.tolist() == order_key[:top_e]
        assert abs(w.sum() - 1) < 1e-12 and np.all(w > 0)
        # softmax over the chosen logits: ratios are exp of logit differences
        for a in range(top_e):
            for b in range(top_e):
                assert math.isclose(w[a] / w[b], math.exp(float(logits[ids[a]]) - float(logits[ids[b]])),
                                    rel_tol=1e-12)


def test_route_equal_logits_pick_lowest_ids():
    ids, w = oracle.route(np.zeros(128, F32), 8)
    assert ids.tolist() == list(range(8)) and np.allclose(w, 1 / 8)


# ---------------------------------------------------------------- quantisation
def test_quantize_matches_brute_force_exponent_search():
    rng = np.random.default_rng(4)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-30, 30)
        x = _bits(rng.standard_normal(int(rng.integers(1, 300))) * scale)
        q, e = oracle.quantize_token(x)
        xv = om.bf16_bits_to_f64(x)
        a = np.abs(xv).max()
        if a == 0:
            assert e == 0 and not q.any()
            continue
        # smallest e with a * 2^-e <= 127, found by scanning
        e_bf = -300
        while a * 2.0 ** (-e_bf) > 127:
            e_bf += 1
        assert e == e_bf
        assert 64 <= np.abs(q).max() <= 127
        assert np.all(np.abs(xv - q * 2.0 ** e) <= 2.0 ** (e - 1))
        # half-way cases go to even
        half = np.abs(xv * 2.0 ** (-e) - np.floor(xv * 2.0 ** (-e))) == 0.5
        assert np.all(q[half] % 2 == 0)


def test_quantize_int16_matches_brute_force_exponent_search():
    """The int16 activations of the score ablation: the smallest exponent with
    max|x| * 2^-e <= 32767, found by scanning, and round-half-even."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-30, 30)
        x = _bits(rng.standard_normal(int(rng.integers(1, 300))) * scale)
        q, e = oracle.quantize_token(x, 16)
        xv = om.bf16_bits_to_f64(x)
        a = np.abs(xv).max()
        if a == 0:
            assert e == 0 and not q.any()
            continue
        e_bf = -300
        while a * 2.0 ** (-e_bf) > 32767:
            e_bf += 1
        assert e == e_bf
        assert 16384 <= np.abs(q).max() <= 32767
        assert np.all(np.abs(xv - q * 2.0 ** e) <= 2.0 ** (e - 1))
        # bf16 x has 8 significant bits, so int16 keeps every value of the
        # largest binades exactly
        big = np.abs(xv) >= a / 2 ** 7
        assert np.array_equal(q[big] * 2.0 ** e, xv[big])


def test_int16_score_is_the_full_score_on_finer_activations():
    """x_int16 ranks by the full score of the int16 sketch: its pre-activations
    sit within alpha * nnz * 2^(e - 1) of the sketch's exact value alpha * (t . x),
    about 256 times closer than with int8 activations."""
    d, m = 256, 64
    wg, wu, wd = synth.expert_weights(0, 7, 0, d, m)
    prep = oracle.prepare_expert(wg, wu, wd, 0)
    x = synth.tokens(0, 7, 1, d)[0]
    xv = om.bf16_bits_to_f64(x)
    exact = prep["alpha_g"].astype(np.float64) * (prep["tern_g"].astype(np.float64) @ xv)
    errs = {}
    for bits in (8, 16):
        q, e = oracle.quantize_token(x, bits)
        g, _ = oracle.sketch_preacts(prep, q, e)
        bound = prep["alpha_g"].astype(np.float64) * prep["nnz_g"] * 2.0 ** (e - 1)
        err = np.abs(g.astype(np.float64) - exact)
        assert np.all(err <= bound + np.abs(exact) * 2.0 ** -23), bits
        errs[bits] = err.max()
    assert errs[16] < errs[8] / 64
    q16, e16 = oracle.quantize_token(x, 16)
    h, sc = oracle.score_channels(prep, q16, e16, "x_int16")
    h_full, sc_full = oracle.score_channels(prep, q16, e16, "full")
    assert np.array_equal(sc.view(np.uint32), sc_full.view(np.uint32))
    assert np.array_equal(h.view(np.uint32), h_full.view(np.uint32))


def test_quantize_zero_token():
    q, e = oracle.quantize_token(np.zeros(64, np.uint16))
    assert e == 0 and not q.any()


# ---------------------------------------------------------------- sketch
def test_sketch_hand_rows():
    with open(os.path.join(GOLDEN, "sketch_hand_rows.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 6
    for ln in rows:
        name, w, t, nnz, alpha = (p.strip() for p in ln.split("|"))
        wv = np.array([float(v) for v in w.split()])
        got_t, got_a, got_n = oracle.ternary_sketch_row(wv)
        assert got_t.tolist() == [int(v) for v in t.split()], name
        assert got_n == int(nnz) and float(got_a) == float(alpha), name


def _fraction_sketch(wv, ratio=0.7):
    """Same statistics by exact rational arithmetic (correctly rounded conversions)."""
    a = [abs(Fraction(float(v))) for v in wv]
    total = float(sum(a, Fraction(0)))        # exact sum, rounded once
    delta = ratio * (total / len(a))
    keep = [float(v) > delta for v in a]
    nnz = sum(keep)
    kept = float(sum((v for v, kf in zip(a, keep) if kf), Fraction(0)))
    alpha = F32(kept / nnz) if nnz else F32(0)
    return keep, alpha, nnz


def test_sketch_statistics_are_exactly_rounded():
    rng = np.random.default_rng(5)
    for trial in range(60):
        d = int(rng.integers(1, 200))
        mags = 10.0 ** rng.uniform(-35, 35, size=d) if trial % 3 == 0 else np.full(d, 0.02)
        w = om.bf16_bits_to_f64(_bits(rng.standard_normal(d) * mags))
        t, alpha, nnz = oracle.ternary_sketch_row(w)
        keep, a_ref, n_ref = _fraction_sketch(w)
        assert nnz == n_ref and alpha.view(np.uint32) == a_ref.view(np.uint32)
        assert np.array_equal(t != 0, np.array(keep))
        assert np.all(t[t != 0] == np.sign(w[t != 0]))
        col = w
        exact = math.sqrt(float(sum((Fraction(float(v)) ** 2 for v in col), Fraction(0))))
        assert om.down_column_norm(col) == F32(exact)


def _phi(x):
    return math.exp(-x * x / 2) / math.sqrt(2 * math.pi)


def test_sketch_gaussian_closed_forms():
    """Ternary Weight Networks closed forms for Gaussian rows: threshold
    delta/sigma = 0.7 sqrt(2/pi), kept fraction erfc(delta/(sigma sqrt 2)),
    alpha/sigma = phi(delta)/(1 - Phi(delta))."""
    delta = 0.7 * math.sqrt(2 / math.pi)
    p_keep = math.erfc(delta / math.sqrt(2))
    alpha_over_sigma = _phi(delta) / (0.5 * math.erfc(delta / math.sqrt(2)))
    assert abs(delta - 0.558519) < 1e-6 and abs(p_keep - 0.576490) < 1e-6
    assert abs(alpha_over_sigma - 1.184161) < 1e-6
    d = 1 << 16
    rng = np.random.default_rng(6)
    for sigma, scale in [(0.02, 1.0), (0.02, 7.3)]:
        w = om.bf16_bits_to_f64(_bits(rng.standard_normal(d) * sigma * scale))
        t, alpha, nnz = oracle.ternary_sketch_row(w)
        sd = math.sqrt(p_keep * (1 - p_keep) / d)
        assert abs(nnz / d - p_keep) < 5 * sd
        assert abs(float(alpha) / (sigma * scale) - alpha_over_sigma) < 0.01


# ---------------------------------------------------------------- integer dot / score
def test_sketch_preacts_integer_dot_brute_force():
    rng = np.random.default_rng(7)
    m, d = 12, 40
    prep = dict(tern_g=rng.integers(-1, 2, size=(m, d)).astype(np.int8),
                tern_u=rng.integers(-1, 2, size=(m, d)).astype(np.int8),
                alpha_g=rng.uniform(0.001, 0.1, m).astype(F32),
                alpha_u=rng.uniform(0.001, 0.1, m).astype(F32),
                c=rng.uniform(0.1, 1, m).astype(F32))
    q = rng.integers(-127, 128, size=d)
    for e in (-9, 0, 3):
        g, u = oracle.sketch_preacts(prep, q, e)
        for j in range(m):
            dg = sum(int(prep["tern_g"][j, i]) * int(q[i]) for i in range(d))
            du = sum(int(prep["tern_u"][j, i]) * int(q[i]) for i in range(d))
            # one binary32 rounding of alpha * D, then an exact power of two
            assert g[j] == F32(float(prep["alpha_g"][j]) * dg) * F32(2.0 ** e)
            assert u[j] == F32(float(prep["alpha_u"][j]) * du) * F32(2.0 ** e)
        h, sc = oracle.score_channels(prep, q, e)
        assert np.array_equal(sc, np.abs(h) * prep["c"])
        assert np.all(sc >= 0)


# ---------------------------------------------------------------- low-rank map
def test_lowrank_recovers_constructed_svd():
    rng = np.random.default_rng(8)
    d, m, r = 96, 40, 7
    u, _ = np.linalg.qr(rng.standard_normal((d, m)))
    v, _ = np.linalg.qr(rng.standard_normal((m, m)))
    s = np.linspace(3.0, 0.5, m)
    w = (u * s) @ v.T
    p, q, _ = om.lowrank_factors(w, r)
    target = (u[:, :r] * s[:r]) @ v[:, :r].T
    assert np.abs(p @ q.T - target).max() < 1e-10
    # Eckart-Young: residual energy equals the discarded singular values
    assert math.isclose(np.sum((w - p @ q.T) ** 2), np.sum(s[r:] ** 2), rel_tol=1e-10)
    assert np.allclose(q.T @ q, np.eye(r), atol=1e-12)


# ---------------------------------------------------------------- block level
def _small_layer(rank, d=64, m=128, n_exp=4, seed=9, scale=0.02):
    rng = np.random.default_rng(seed)
    wg = _bits(rng.standard_normal((n_exp, m, d)) * scale)
    wu = _bits(rng.standard_normal((n_exp, m, d)) * scale)
    wd = _bits(rng.standard_normal((n_exp, d, m)) * scale)
    layer = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), n_exp, d, m, rank)
    return layer, (wg, wu, wd)


def _einsum_dense(wg, wu, wd, x_bits, logits, top_e):
    """Textbook dense SwiGLU MoE block, written independently of the oracle."""
    g_all = om.bf16_bits_to_f64(wg)
    u_all = om.bf16_bits_to_f64(wu)
    d_all = om.bf16_bits_to_f64(wd)
    x = om.bf16_bits_to_f64(x_bits)
    y = np.zeros((x.shape[0], d_all.shape[1]))
    for t in range(x.shape[0]):
        lg = logits[t].astype(np.float64)
        ids = sorted(range(len(lg)), key=lambda i: (-lg[i], i))[:top_e]
        w = np.exp(lg[ids] - lg[ids].max())
        w /= w.sum()
        g = np.einsum("emd,d->em", g_all[ids], x[t])
        u = np.einsum("emd,d->em", u_all[ids], x[t])
        h = g * (1 / (1 + np.exp(-g))) * u
        y[t] = np.einsum("e,edm,em->d", w, d_all[ids], h)
    return y


def test_k_equals_m_is_the_dense_block():
    layer, (wg, wu, wd) = _small_layer(rank=5)
    rng = np.random.default_rng(10)
    x = _bits(rng.standard_normal((3, 64)))
    logits = rng.standard_normal((3, 4)).astype(F32)
    out = layer.forward(x, logits, top_e=2, k=128)
    ref = _einsum_dense(wg, wu, wd, x, logits, 2)
    assert np.abs(out["y"] - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.allclose(layer.forward_dense(x, logits, 2), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_rank_zero_has_no_compensation():
    layer, _ = _small_layer(rank=0)
    rng = np.random.default_rng(11)
    x = _bits(rng.standard_normal((2, 64)))
    logits = rng.standard_normal((2, 4)).astype(F32)
    a = layer.forward(x, logits, 2, 20, compensate=True)["y"]
    b = layer.forward(x, logits, 2, 20, compensate=False)["y"]
    assert np.array_equal(a, b)


def test_exact_sketch_with_full_rank_map_is_dense_for_every_k():
    """When the weights are exactly alpha_j * t_j and x is exactly q * 2^e, the
    sketch pre-activations are the true ones (to binary32 rounding), and with a
    full-rank map the compensation reproduces the skipped channels exactly: the
    block equals the dense block for every k. A sign, index or transpose slip in
    the score, the selection bookkeeping or the compensation breaks this."""
    rng = np.random.default_rng(12)
    d, m, n_exp, top_e = 64, 48, 3, 2
    alpha = (2.0 ** rng.integers(-7, -4, size=(n_exp, m)) * (1 + rng.integers(0, 8, size=(n_exp, m)) / 8))
    tg = rng.integers(-1, 2, size=(n_exp, m, d))
    tu = rng.integers(-1, 2, size=(n_exp, m, d))
    tg[:, :, 0] = 1
    tu[:, :, 0] = -1                                         # no all-zero rows
    wg = _bits(alpha[:, :, None] * tg)
    wu = _bits(alpha[:, :, None] * tu)
    wd = _bits(rng.standard_normal((n_exp, d, m)) * 0.05)
    layer = oracle.OracleLayer(lambda e: (wg[e], wu[e], wd[e]), n_exp, d, m, rank=min(d, m))
    q = rng.integers(-127, 128, size=(1, d))
    q[0, 5] = 127
    x = _bits(q / 128.0)
    logits = rng.standard_normal((1, n_exp)).astype(F32)
    ref = _einsum_dense(wg, wu, wd, x, logits, top_e)
    for k in (0, 1, 7, 24, 47, 48):
        y = layer.forward(x, logits, top_e, k)["y"]
        assert np.abs(y - ref).max() <= 2e-6 * np.abs(ref).max(), k
    # the same block with the compensation dropped is not dense (so the test has teeth)
    y0 = layer.forward(x, logits, top_e, 7, compensate=False)["y"]
    assert np.abs(y0 - ref).max() > 1e-2 * np.abs(ref).max()


def test_channel_and_expert_permutation_equivariance():
    layer, (wg, wu, wd) = _small_layer(rank=6, seed=13)
    rng = np.random.default_rng(14)
    x = _bits(rng.standard_normal((2, 64)))
    logits = rng.standard_normal((2, 4)).astype(F32)
    base = layer.forward(x, logits, 2, 30)
    perm = rng.permutation(128)
    inv = np.argsort(perm)
    wg2, wu2, wd2 = wg[:, perm], wu[:, perm], wd[:, :, perm]
    lay2 = oracle.OracleLayer(lambda e: (wg2[e], wu2[e], wd2[e]), 4, 64, 128, 6)
    out2 = lay2.forward(x, logits, 2, 30)
    for t in range(2):
        for s in range(2):
            sc = base["score"][t][s]
            assert len(np.unique(sc)) == len(sc)                  # no ties, selection is unique
            assert np.array_equal(np.sort(perm[out2["sel"][t][s]]), base["sel"][t][s])
            assert np.array_equal(out2["score"][t][s], sc[perm])
    assert np.allclose(out2["y"], base["y"], rtol=0, atol=1e-12 * np.abs(base["y"]).max())
    ep = rng.permutation(4)
    wg3, wu3, wd3 = wg[ep], wu[ep], wd[ep]
    lay3 = oracle.OracleLayer(lambda e: (wg3[e], wu3[e], wd3[e]), 4, 64, 128, 6)
    out3 = lay3.forward(x, logits[:, ep], 2, 30)
    assert np.allclose(out3["y"], base["y"], rtol=0, atol=1e-12 * np.abs(base["y"]).max())
    assert inv is not None


def test_budget_is_exact_per_token():
    layer, _ = _small_layer(rank=4, seed=15)
    rng = np.random.default_rng(16)
    x = _bits(rng.standard_normal((4, 64)))
    logits = rng.standard_normal((4, 4)).astype(F32)
    for k in (0, 1, 23, 128):
        out = layer.forward(x, logits, 3, k)
        assert all(len(s) == k for row in out["sel"] for s in row)
    for budget, m, k in [(0.18, 512, 92), (0.13, 768, 100), (0.18, 768, 138), (0.178, 768, 137),
                         (0.13, 14336, 1864), (0.18, 14336, 2580)]:
        assert synth.budget_to_k(budget, m) == k
        assert abs(k / m - budget) <= 1 / (2 * m)


def test_degenerate_inputs():
    layer, _ = _small_layer(rank=4, seed=17)
    out = layer.forward(np.zeros((1, 64), np.uint16), np.zeros((1, 4), F32), 2, 10)
    assert not out["y"].any()
    assert out["expert_ids"][0].tolist() == [0, 1]
    assert np.allclose(out["gate_w"][0], 0.5)


def test_batch_rows_are_independent():
    layer, _ = _small_layer(rank=4, seed=18)
    rng = np.random.default_rng(19)
    x = _bits(rng.standard_normal((5, 64)))
    logits = rng.standard_normal((5, 4)).astype(F32)
    full = layer.forward(x, logits, 2, 17)
    for t in (0, 3):
        one = layer.forward(x[t:t + 1], logits[t:t + 1], 2, 17)
        assert np.array_equal(one["y"][0], full["y"][t])
        for s in range(2):
            assert np.array_equal(one["sel"][0][s], full["sel"][t][s])


# ---------------------------------------------------------------------------
# Decode-step glue: router logits and the renormalised residual stream
# ---------------------------------------------------------------------------
def test_f64_to_bf16_ties_to_even_and_carry():
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 255.9, -1.2, 1.6, 0.0])
    got = oracle.f64_to_bf16_bits(vals)
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour 1 wins;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: 1 + 2^-6 is even.
    assert got.tolist() == [0x3F80, 0x3F82, 0x4380, 0xBF9A, 0x3FCD, 0x0000]


def test_f64_to_bf16_agrees_with_float32_bit_rounding():
    # values exactly representable in binary32: a one-step rounding from float64
    # and the binary32 bit trick of the input generator must agree
    rng = np.random.default_rng(3)
    v = rng.standard_normal(4000).astype(np.float32)
    assert np.array_equal(oracle.f64_to_bf16_bits(v.astype(np.float64)), synth.f32_to_bf16_bits(v))


def test_router_logits_one_hot_reads_a_column():
    rng = np.random.default_rng(4)
    d, E = 64, 9
    w = synth.f32_to_bf16_bits(rng.standard_normal((E, d)).astype(np.float32))
    x = np.zeros((2, d), np.uint16)
    x[0, 5] = 0x3F80          # 1.0
    x[1, 17] = 0x4000         # 2.0
    lg = oracle.router_logits(x, w)
    assert np.array_equal(lg[0], synth.bf16_bits_to_f32(w[:, 5]))
    assert np.array_equal(lg[1], 2 * synth.bf16_bits_to_f32(w[:, 17]))


def test_residual_rmsnorm_hand_cases():
    d = 4
    x = np.zeros((3, d), np.uint16)
    y = np.zeros((3, d), np.uint16)
    x[0] = [0x4040, 0x4080, 0, 0]          # (3, 4, 0, 0): rms 2.5 -> (1.2, 1.6, 0, 0)
    x[1] = [0x3F80] * 4                    # constant 1 + (-3) = -2 everywhere -> -1
    y[1] = [0xC040] * 4
    x[2] = [0x4120, 0xC0A0, 0x3F00, 0x4000]
    y[2] = x[2] ^ 0x8000                   # y = -x: the sum is zero, so is the output
    out = oracle.residual_rmsnorm(x, y)
    assert out[0].tolist() == [0x3F9A, 0x3FCD, 0, 0]
    assert out[1].tolist() == [0xBF80] * 4
    assert not (out[2] & 0x7FFF).any()


# ---------------------------------------------------------------------------
# Threshold selector (the baseline the pages contrast with top-k)
# ---------------------------------------------------------------------------
def test_threshold_just_below_the_kth_score_is_topk():
    rng = np.random.default_rng(21)
    for k in (1, 7, 40, 99):
        sc = rng.random(100).astype(np.float32)   # distinct with probability one
        kth = np.sort(sc)[::-1][k - 1]
        thr = np.nextafter(kth, np.float32(-1.0))
        assert np.array_equal(oracle.select_threshold(sc, thr), oracle.select_topk(sc, k))


def test_threshold_edges_and_ties():
    sc = np.array([0.0, 0.5, 0.5, 1.0, 0.25], np.float32)
    assert oracle.select_threshold(sc, 1.0).tolist() == []           # strict: the maximum itself is not above
    assert oracle.select_threshold(sc, 0.5).tolist() == [3]
    assert oracle.select_threshold(sc, 0.25).tolist() == [1, 2, 3]   # equal scores move together
    assert oracle.select_threshold(sc, 0.0).tolist() == [1, 2, 3, 4]


def test_threshold_calibration_keeps_the_budget_on_its_own_sample():
    from activation_sparse_expert_amd import threshold as th
    rng = np.random.default_rng(22)
    sc = rng.random((64, 8, 768)).astype(np.float32)
    thr = th.calibrate(sc, 0.18)
    assert abs((sc > np.float32(thr)).mean() - 0.18) <= 1.0 / sc.size


# ---------------------------------------------------------------------------
# Score ablations: which weights each kind depends on
# ---------------------------------------------------------------------------
def _kind_scores(wg, wu, wd, x_bits, kind):
    prep = oracle.prepare_expert(wg, wu, wd, 0)
    q, e = oracle.quantize_token(x_bits)
    return oracle.score_channels(prep, q, e, kind)


def test_score_kinds_depend_on_the_right_weights():
    d, m = 128, 64
    wg, wu, wd = synth.expert_weights(0, 5, 0, d, m)
    _, wu2, wd2 = synth.expert_weights(0, 6, 0, d, m)
    x = synth.tokens(0, 5, 1, d)[0]
    full = _kind_scores(wg, wu, wd, x, "full")[1]
    gate = _kind_scores(wg, wu, wd, x, "gate_only")[1]
    nodn = _kind_scores(wg, wu, wd, x, "no_down_norm")[1]
    # gate-only ignores the up weights; no-down-norm ignores the down weights
    assert np.array_equal(gate, _kind_scores(wg, wu2, wd, x, "gate_only")[1])
    assert not np.array_equal(full, _kind_scores(wg, wu2, wd, x, "full")[1])
    assert np.array_equal(nodn, _kind_scores(wg, wu, wd2, x, "no_down_norm")[1])
    assert not np.array_equal(full, _kind_scores(wg, wu, wd2, x, "full")[1])
    # the full score is the no-down-norm score scaled by the column norm (one rounding)
    c = oracle.prepare_expert(wg, wu, wd, 0)["c"].astype(np.float32)
    assert np.array_equal(full, (nodn * c).astype(np.float32))
    # and h_hat does not depend on the kind
    assert np.array_equal(_kind_scores(wg, wu, wd, x, "gate_only")[0], _kind_scores(wg, wu, wd, x, "full")[0])
