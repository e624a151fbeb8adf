"""CPU oracle: calibration-free top-k channel selection inside routed MoE experts.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain NumPy, float64
everywhere except the channel score, which is pinned to IEEE binary32 so that a
second, independent implementation can reproduce its bits.

Sources, cited by page title and section:

* [KAIST] "KAIST drops calibration from MoE decoding, speeds up blocks by up to
  2.69x over vLLM" (its French twin, "KAIST supprime la calibration du decodage
  MoE ...", carries the same content). Sections: opening paragraph; "The
  threshold promises a budget but does not keep it"; "Top-k instead of a
  threshold"; "A reader built from weights alone".
* [GHOST] "Calibration-free top-k MoE selector saves tuning" (paragraphs quoting
  the paper "Channel Selection for Mixture-of-Experts Decoding Needs No
  Calibration Data").
* [MLX] "MoE top_k override (--moe-top-k)", section "Ce que ca fait" (routing
  of a Qwen3-30B-A3B-class layer: 8 of 128 experts per token).

What the pages fix: decoding reads the routed experts' weights for every token
([KAIST] opening paragraph); a selector scores the *intermediate channels* of an
expert and only those channels' weights are read ([KAIST] "The threshold
promises..."); each token keeps its k highest-scoring channels, so the read
budget is known in advance ([KAIST] "Top-k instead of a threshold"; [GHOST]);
channels are filtered with a *ternary sketch of the weights* and the skipped
channels are compensated by a *low-rank map built from the weights*
([KAIST] "A reader built from weights alone"); weights are bf16 ([GHOST]).

What the pages leave open is closed by readings, each stated where it is used:
SwiGLU experts without biases; routing = top experts by logit, lowest index on
ties, softmax over the chosen logits; ternary threshold 0.7 * mean|w| per
channel with the Ternary-Weight-Networks scale (mean |w| over the kept
entries); int8 activations with a power-of-two scale inside the score;
score = |silu(G_hat) * U_hat| * ||down column||_2; ties in the top-k broken by
the lowest channel index; compensation = truncated SVD of the down matrix
applied to the sketch activations of the skipped channels; each token of a
batch uses only its own channels.

Parity status: every function below is pinned by tests against closed forms,
brute force, exact rational arithmetic or textbook special cases. Fidelity to
the authors' own (unpublished) score and compensation formulas is not something
any test can check; the pins cover the readings above.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# binary32 constants of silu_pinned (written out from their definitions).
# L2E: nearest binary32 to 1/ln 2.  LN2_HI: ln 2 truncated to 12 fractional
# bits (n * LN2_HI is exact for |n| <= 2^12); LN2_LO: nearest binary32 to the
# remainder ln 2 - LN2_HI (two-part argument reduction of Cody & Waite, 1980).
# INV_FACT[k]: nearest binary32 to 1/k!, k = 0..7 (Taylor series of e^r).
# ---------------------------------------------------------------------------
_LN2 = math.log(2.0)
L2E = F32(1.0 / _LN2)
LN2_HI = F32(math.floor(_LN2 * 4096.0) / 4096.0)
LN2_LO = F32(_LN2 - float(LN2_HI))
INV_FACT = [F32(1.0 / math.factorial(k)) for k in range(8)]
SILU_CUT = F32(87.0)

ORACLE_CONSTANTS = dict(L2E=L2E, LN2_HI=LN2_HI, LN2_LO=LN2_LO, INV_FACT=INV_FACT, SILU_CUT=SILU_CUT)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of raw bfloat16 bits, as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Offline preparation: ternary sketch, channel statistics, low-rank map.
# ---------------------------------------------------------------------------
def ternary_sketch_row(w: np.ndarray, tern_ratio: float = 0.7):
    """Ternary sketch of one intermediate channel (one gate or up row).

    [KAIST] "A reader built from weights alone": channels are first filtered
    with a ternary sketch of the weights. Reading: the threshold is
    delta = 0.7 * mean|w| over the channel's d weights and the scale is the mean
    |w| over the entries kept (the closed-form scale of Ternary Weight Networks,
    Li et al. 2016, whose threshold 0.7 * E|w| is this one).

    Arithmetic: both sums are exact sums rounded once to float64 (math.fsum);
    mean and delta are float64 operations in that order; the comparison is
    strict and in float64; alpha is the float64 quotient rounded to binary32.

    Returns (t int8 [d] in {-1, 0, 1}, alpha float32, nnz int).
    """
    w = np.asarray(w, dtype=np.float64)
    d = w.shape[0]
    a = np.abs(w)
    total = math.fsum(a.tolist())
    mean = total / d
    delta = tern_ratio * mean
    keep = a > delta
    t = (np.sign(w) * keep).astype(np.int8)
    nnz = int(keep.sum())
    if nnz == 0:
        return t, F32(0.0), 0
    kept = math.fsum(a[keep].tolist())
    alpha = F32(kept / nnz)
    return t, alpha, nnz


def down_column_norm(col: np.ndarray) -> np.float32:
    """||W_down[:, j]||_2: exact sum of squares rounded once, float64 sqrt, rounded to binary32."""
    c = np.asarray(col, dtype=np.float64)
    return F32(math.sqrt(math.fsum((c * c).tolist())))


def lowrank_factors(w_down: np.ndarray, rank: int):
    """Rank-r map built from the down matrix alone.

    [KAIST] "A reader built from weights alone": skipped channels are
    compensated by a low-rank mapping built from the model's weights. Reading:
    the best rank-r approximation (truncated SVD) W_down ~= P Q^T with
    P = U_r diag(s_r) [d][r] and Q = V_r [m][r].
    """
    wd = np.asarray(w_down, dtype=np.float64)
    d, m = wd.shape
    if rank == 0:
        return np.zeros((d, 0)), np.zeros((m, 0)), np.zeros(0)
    u, s, vt = np.linalg.svd(wd, full_matrices=False)
    p = u[:, :rank] * s[None, :rank]
    q = vt[:rank].T.copy()
    return p, q, s


def prepare_expert(wg_bits, wu_bits, wd_bits, rank: int, tern_ratio: float = 0.7):
    """Everything the selector needs for one expert, computed from its weights only.

    wg_bits, wu_bits: bf16 bits [m][d]; wd_bits: bf16 bits [d][m].
    """
    wg = bf16_bits_to_f64(wg_bits)
    wu = bf16_bits_to_f64(wu_bits)
    wd = bf16_bits_to_f64(wd_bits)
    m, d = wg.shape
    tg = np.zeros((m, d), np.int8)
    tu = np.zeros((m, d), np.int8)
    ag = np.zeros(m, F32)
    au = np.zeros(m, F32)
    ng = np.zeros(m, np.int64)
    nu = np.zeros(m, np.int64)
    c = np.zeros(m, F32)
    for j in range(m):
        tg[j], ag[j], ng[j] = ternary_sketch_row(wg[j], tern_ratio)
        tu[j], au[j], nu[j] = ternary_sketch_row(wu[j], tern_ratio)
        c[j] = down_column_norm(wd[:, j])
    p, q, s = lowrank_factors(wd, rank)
    return dict(wg=wg, wu=wu, wd=wd, tern_g=tg, tern_u=tu, alpha_g=ag, alpha_u=au,
                nnz_g=ng, nnz_u=nu, c=c, P=p, Q=q, sing=s, d=d, m=m, rank=rank)


# ---------------------------------------------------------------------------
# Per-token steps.
# ---------------------------------------------------------------------------
def route(logits_row: np.ndarray, top_e: int):
    """Routed experts of one token and their gate weights.

    [KAIST] opening paragraph: each token loads the weights of its routed
    experts; [MLX] "Ce que ca fait": a Qwen3-30B-A3B-class layer routes each
    token to 8 of 128 experts. Reading: the top_e largest float32 logits,
    lowest expert index first on equal logits, listed best first; gate weights
    are the softmax over the chosen logits (float64).
    """
    lg = np.asarray(logits_row, dtype=np.float32).astype(np.float64)
    order = np.lexsort((np.arange(lg.shape[0]), -lg))
    ids = order[:top_e]
    sel = lg[ids]
    ex = np.exp(sel - sel.max())
    return ids.astype(np.int64), ex / ex.sum()


def quantize_token(x_bits: np.ndarray, bits: int = 8):
    """Integer activations with a power-of-two scale, used only inside the score.

    Reading (pages silent on the precision of x in the score): with
    a = max|x| and qmax = 2^(bits-1) - 1, e = ilogb(a) - (bits - 2), raised by
    one if a * 2^-e > qmax; q = round-half-even(x * 2^-e). Then max|q| <= qmax
    and x ~= q * 2^e. bits = 8 is the method's score; bits = 16 is the int16
    ablation of the score.
    Returns (q int64 [d], e int).
    """
    qmax = float(2 ** (bits - 1) - 1)
    x = bf16_bits_to_f64(x_bits)
    a = float(np.max(np.abs(x))) if x.size else 0.0
    if a == 0.0:
        return np.zeros(x.shape, np.int64), 0
    _, ex = math.frexp(a)          # a = f * 2^ex, f in [0.5, 1)
    e = (ex - 1) - (bits - 2)
    if a * 2.0 ** (-e) > qmax:
        e += 1
    q = np.rint(x * 2.0 ** (-e)).astype(np.int64)
    return q, e


def silu_pinned(z) -> np.ndarray:
    """silu(z) = z / (1 + e^-z) in binary32, every operation separately rounded.

    Definition (pinned so that any IEEE binary32 implementation without fused
    multiply-add reproduces it bit for bit):
      z > 87 -> z;  z < -87 -> +0;  otherwise with t = -z:
      n = rint(t * L2E);  r = (t - n*LN2_HI) - n*LN2_LO      (Cody & Waite)
      p = Horner(r; 1/7!, ..., 1/1!, 1/0!)                   (Taylor, degree 7)
      e^t ~= ldexp(p, n);  result = z / (1 + e^t).
    """
    z = np.asarray(z, dtype=F32)
    t = np.clip(-z, -SILU_CUT, SILU_CUT).astype(F32)
    n = np.rint(t * L2E).astype(F32)
    r = (t - n * LN2_HI) - n * LN2_LO
    p = INV_FACT[7]
    for k in range(6, -1, -1):
        p = p * r + INV_FACT[k]
    p = np.asarray(p, dtype=F32)
    et = np.ldexp(p, n.astype(np.int32)).astype(F32)
    out = (z / (F32(1.0) + et)).astype(F32)
    out = np.where(z > SILU_CUT, z, out)
    out = np.where(z < -SILU_CUT, F32(0.0), out)
    return out.astype(F32)


def sketch_preacts(prep: dict, q: np.ndarray, e: int):
    """Sketch estimates of the gate and up pre-activations of every channel.

    G_hat_j = binary32(alpha_g_j * binary32(t_g[j] . q)) * 2^e, likewise U_hat_j.
    The integer dot is exact; its binary32 value is exact for int8 activations
    (|t . q| <= 127 d < 2^24) and rounded to nearest even for int16 ones.
    """
    dg = prep["tern_g"].astype(np.int64) @ q
    du = prep["tern_u"].astype(np.int64) @ q
    return preacts_from_dots(dg, du, e, prep["alpha_g"], prep["alpha_u"])


def preacts_from_dots(dg, du, e, alpha_g, alpha_u):
    """G_hat = binary32(alpha_g * binary32(dg)) * 2^e and likewise U_hat, from the
    exact integer sketch dots (the second half of ``sketch_preacts``); ``e`` may be
    a scalar or one exponent per entry."""
    g = np.ldexp(np.asarray(alpha_g, F32) * np.asarray(dg).astype(F32), e).astype(F32)
    u = np.ldexp(np.asarray(alpha_u, F32) * np.asarray(du).astype(F32), e).astype(F32)
    return g, u


SCORE_KINDS = ("full", "gate_only", "no_down_norm", "x_int16")


def score_channels(prep: dict, q: np.ndarray, e: int, kind: str = "full"):
    """Sketch activations and channel scores for one (token, expert) pair.

    [KAIST] "The threshold promises a budget...": a channel matters when it
    changes the token's output; "A reader built from weights alone": the sketch
    filters channels. Reading: G_hat = alpha_g * (t_g . q) * 2^e and
    U_hat = alpha_u * (t_u . q) * 2^e (integer dots are exact, each product
    rounded once to binary32, the power of two applied exactly);
    h_hat = silu_pinned(G_hat) * U_hat; score = |h_hat| * ||down_j||_2.
    Ablations of the score (the pages leave it open; h_hat is unchanged):
    ``gate_only``: |silu_pinned(G_hat)| * ||down_j||_2; ``no_down_norm``: |h_hat|.
    ``x_int16`` is the full score on int16 activations: the caller passes the
    int16 q and e of quantize_token(x, 16).
    Returns (h_hat float32 [m], score float32 [m]).
    """
    g, u = sketch_preacts(prep, q, e)
    return score_from_preacts(g, u, prep["c"], kind)


def score_from_preacts(g: np.ndarray, u: np.ndarray, c: np.ndarray, kind: str = "full"):
    """The score's binary32 arithmetic after the sketch pre-activations (the
    second half of ``score_channels``): h_hat = silu_pinned(G_hat) * U_hat and the
    score of the given kind from h_hat and the down-column norms c.
    Returns (h_hat float32, score float32)."""
    sg = silu_pinned(g)
    h = (sg * np.asarray(u, F32)).astype(F32)
    c = np.asarray(c, F32)
    if kind in ("full", "x_int16"):
        score = (np.abs(h) * c).astype(F32)
    elif kind == "gate_only":
        score = (np.abs(sg) * c).astype(F32)
    elif kind == "no_down_norm":
        score = np.abs(h).astype(F32)
    else:
        raise ValueError(f"unknown score kind {kind!r}")
    return h, score


def select_topk(score: np.ndarray, k: int) -> np.ndarray:
    """Each token keeps its k highest-scoring channels ([KAIST] "Top-k instead of a
    threshold"; [GHOST]). Equal scores: lower channel index first. Returned ascending."""
    s = np.asarray(score, dtype=np.float32).astype(np.float64)
    order = np.lexsort((np.arange(s.shape[0]), -s))
    return np.sort(order[:k]).astype(np.int64)


def select_threshold(score: np.ndarray, threshold: float) -> np.ndarray:
    """The threshold selector the pages contrast with top-k ([KAIST] "The threshold
    promises a budget but does not keep it": channels whose score exceeds a
    threshold tuned offline): indices with score > threshold, compared in binary32,
    ascending. The number kept varies from token to token."""
    return np.flatnonzero(np.asarray(score, np.float32) > np.float32(threshold))


def expert_swiglu_selected(prep: dict, x: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Expert output from the selected channels only: sum_{j in S} silu(g_j) u_j down_j.

    [KAIST] "The threshold promises...": only the selected channels' weights are
    read. Reading: SwiGLU expert, no biases; float64.
    """
    g = prep["wg"][sel] @ x
    u = prep["wu"][sel] @ x
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * u
    return prep["wd"][:, sel] @ h


def compensation(prep: dict, h_hat: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Low-rank stand-in for the skipped channels: P (Q^T h_hat restricted to j not in S).

    [KAIST] "A reader built from weights alone". Reading: the skipped channels'
    true contribution W_down[:, skipped] h[skipped] is approximated with the
    sketch activations h_hat in place of h and the rank-r map in place of W_down.
    """
    if prep["rank"] == 0:
        return np.zeros(prep["d"])
    mask = np.ones(prep["m"], bool)
    mask[sel] = False
    z = prep["Q"][mask].T @ h_hat[mask].astype(np.float64)
    return prep["P"] @ z


# ---------------------------------------------------------------------------
# Block level.
# ---------------------------------------------------------------------------
class OracleLayer:
    """One MoE layer; experts are prepared lazily on first use.

    ``weights(e)`` returns expert e's (w_gate [m][d], w_up [m][d], w_down [d][m])
    as bf16 bits.
    """

    def __init__(self, weights, n_experts: int, d: int, m: int, rank: int, tern_ratio: float = 0.7):
        self.weights = weights
        self.n_experts, self.d, self.m, self.rank = n_experts, d, m, rank
        self.tern_ratio = tern_ratio
        self._prep = {}

    def expert(self, e: int) -> dict:
        e = int(e)
        if e not in self._prep:
            wg, wu, wd = self.weights(e)
            self._prep[e] = prepare_expert(wg, wu, wd, self.rank, self.tern_ratio)
        return self._prep[e]

    def forward(self, x_bits: np.ndarray, logits: np.ndarray, top_e: int, k: int, compensate: bool = True,
                threshold: float | None = None, score_kind: str = "full"):
        """Selected-channel block for a batch; every token uses only its own channels.

        With ``threshold`` given, each pair keeps the channels whose score exceeds
        it instead of its top k (``k`` is then ignored).

        Returns a dict with y float64 [B][d] and, per token, the routed experts,
        gate weights, selected channels (ascending), h_hat and scores.
        """
        x_bits = np.atleast_2d(x_bits)
        logits = np.atleast_2d(logits)
        b = x_bits.shape[0]
        y = np.zeros((b, self.d))
        ids = np.zeros((b, top_e), np.int64)
        gw = np.zeros((b, top_e))
        sels, hs, scores = [], [], []
        for t in range(b):
            x = bf16_bits_to_f64(x_bits[t])
            q, e_t = quantize_token(x_bits[t], 16 if score_kind == "x_int16" else 8)
            ids[t], gw[t] = route(logits[t], top_e)
            row_s, row_h, row_sc = [], [], []
            for slot, ex in enumerate(ids[t]):
                prep = self.expert(ex)
                h_hat, sc = score_channels(prep, q, e_t, score_kind)
                sel = select_topk(sc, k) if threshold is None else select_threshold(sc, threshold)
                part = expert_swiglu_selected(prep, x, sel)
                if compensate:
                    part = part + compensation(prep, h_hat, sel)
                y[t] += gw[t, slot] * part
                row_s.append(sel)
                row_h.append(h_hat)
                row_sc.append(sc)
            sels.append(row_s)
            hs.append(row_h)
            scores.append(row_sc)
        return dict(y=y, expert_ids=ids, gate_w=gw, sel=sels, h_hat=hs, score=scores)

    def forward_dense(self, x_bits: np.ndarray, logits: np.ndarray, top_e: int) -> np.ndarray:
        """Dense routed block (every channel read): the k = m case of ``forward``."""
        x_bits = np.atleast_2d(x_bits)
        logits = np.atleast_2d(logits)
        y = np.zeros((x_bits.shape[0], self.d))
        for t in range(x_bits.shape[0]):
            x = bf16_bits_to_f64(x_bits[t])
            ids, gw = route(logits[t], top_e)
            for slot, ex in enumerate(ids):
                y[t] += gw[slot] * expert_swiglu_selected(self.expert(ex), x, np.arange(self.m))
        return y


# ---------------------------------------------------------------------------
# Stacked decode step (glue between blocks). The pages measure MoE blocks inside
# decoding ([KAIST] opening paragraph); chaining blocks over layers needs a
# router per layer and a residual stream between layers. Readings: the router is
# a plain linear map of the hidden state to one logit per expert; the residual
# adds the block output and renormalises to unit root-mean-square.
# ---------------------------------------------------------------------------
def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray) -> np.ndarray:
    """logits[t][e] = sum_i x[t][i] * W[e][i] in float64, rounded once to binary32."""
    x = bf16_bits_to_f64(np.atleast_2d(x_bits))
    w = bf16_bits_to_f64(w_router_bits)
    return (x @ w.T).astype(np.float32)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16, nearest with ties to even, returning raw bits.

    Exact: the value is split into sign, exponent and a 53-bit significand with
    math.frexp, and the significand is rounded to 8 bits by integer arithmetic.
    Subnormal bfloat16 results are not needed here (|v| >= 2^-126 or v == 0)."""
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.empty(flat.shape, np.uint16)
    for i, val in enumerate(flat):
        if val == 0.0:
            out[i] = 0x8000 if math.copysign(1.0, val) < 0 else 0
            continue
        sign = 0x8000 if val < 0 else 0
        mant, exp = math.frexp(abs(val))          # abs(val) = mant * 2^exp, mant in [0.5, 1)
        sig = int(mant * (1 << 53))               # exact 53-bit integer significand
        keep, rest = divmod(sig, 1 << 45)         # 8 significant bits kept, 45 dropped
        half = 1 << 44
        if rest > half or (rest == half and (keep & 1)):
            keep += 1
        if keep == (1 << 8):                      # rounding carried into the next binade
            keep >>= 1
            exp += 1
        biased = exp - 1 + 127                    # value = (keep / 2^7) * 2^(exp - 1)
        assert 1 <= biased <= 254, "outside the normal bfloat16 range"
        out[i] = sign | (biased << 7) | (keep & 0x7F)
    return out.reshape(np.shape(v))


def residual_rmsnorm(x_bits: np.ndarray, y_bits: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x_next = bf16(v / sqrt(mean(v^2) + eps)) with v = x + y, all in float64."""
    v = bf16_bits_to_f64(np.atleast_2d(x_bits)) + bf16_bits_to_f64(np.atleast_2d(y_bits))
    scale = 1.0 / np.sqrt((v * v).mean(axis=1, keepdims=True) + eps)
    return f64_to_bf16_bits(v * scale)
