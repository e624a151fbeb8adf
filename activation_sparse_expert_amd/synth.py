"""Seeded synthetic inputs for the routed-MoE channel-selection block.

This module holds no arithmetic of the method itself: only random draws, the
round-to-nearest-even conversion of those draws to bfloat16, and the shapes of
the workloads. Both the library's tests/benchmark and the CPU oracle's tests
draw their inputs from here, so they always see identical bytes.

Every stream is a NumPy PCG64 generator keyed by
``SeedSequence(0, spawn_key=(workload, layer, tensor, index))``, so any single
expert of any layer can be regenerated on its own without drawing the rest.

Workload shapes (hidden size d, experts E, routed experts per token top_e,
intermediate channels per expert m, channel budgets k, compensation rank r):

* ``tiny``     d=256,  E=8,   top_e=2, m=512,   k=92,          r=8,  B=1
* ``qwen3``    d=2048, E=128, top_e=8, m=768,   k=100 / 138,   r=32, B=1
* ``mixtral``  d=4096, E=8,   top_e=2, m=14336, k=1864 / 2580, r=64, B=1,
  each intermediate channel scaled by a LogNormal(0, 0.5) draw
* ``qwen3_b64``  qwen3 shape at 64 decode tokens, Zipf(1.1)-skewed routing, k=138
* ``qwen3_48l``  48 stacked qwen3-shaped layers, B in {1, 8, 32}, k=137
"""
from __future__ import annotations

import os

import numpy as np

# tensor ids inside a spawn key
T_GATE, T_UP, T_DOWN, T_CHSCALE, T_X, T_LOGITS, T_ROUTER, T_PERM = range(8)

WORKLOADS = {
    "tiny": dict(wid=0, d=256, n_experts=8, top_e=2, m=512, ks=(92,), rank=8,
                 batch=1, routing="normal", channel_scale=False, layers=1),
    "qwen3": dict(wid=1, d=2048, n_experts=128, top_e=8, m=768, ks=(100, 138),
                  rank=32, batch=1, routing="normal", channel_scale=False, layers=1),
    "mixtral": dict(wid=2, d=4096, n_experts=8, top_e=2, m=14336, ks=(1864, 2580),
                    rank=64, batch=1, routing="normal", channel_scale=True, layers=1),
    "qwen3_b64": dict(wid=3, d=2048, n_experts=128, top_e=8, m=768, ks=(138,),
                      rank=32, batch=64, routing="zipf", channel_scale=False, layers=1),
    "qwen3_48l": dict(wid=4, d=2048, n_experts=128, top_e=8, m=768, ks=(137,),
                      rank=32, batch=1, routing="router", channel_scale=False, layers=48),
    # many small experts (a parity case, not a benchmark): more experts than one
    # block of the one-pair-tile score kernel routes itself
    "wide": dict(wid=5, d=512, n_experts=320, top_e=4, m=256, ks=(46,), rank=8,
                 batch=1, routing="normal", channel_scale=False, layers=1),
}

WEIGHT_STD = 0.02
ZIPF_S = 1.1


def _rng(wid: int, layer: int, tensor: int, index: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(0, spawn_key=(int(wid), int(layer), int(tensor), int(index)))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def expert_weights(wid: int, layer: int, expert: int, d: int, m: int,
                   channel_scale: bool = False, std: float = WEIGHT_STD):
    """One expert's weights as raw bf16 bits.

    Returns ``(w_gate [m][d], w_up [m][d], w_down [d][m])``: gate/up rows are
    intermediate channels, the down matrix maps the m channels back to d.
    With ``channel_scale`` every intermediate channel j gets one LogNormal(0, 0.5)
    factor applied to gate row j, up row j and down column j before rounding.
    """
    g = _rng(wid, layer, T_GATE, expert).standard_normal((m, d), dtype=np.float32) * np.float32(std)
    u = _rng(wid, layer, T_UP, expert).standard_normal((m, d), dtype=np.float32) * np.float32(std)
    dn = _rng(wid, layer, T_DOWN, expert).standard_normal((d, m), dtype=np.float32) * np.float32(std)
    if channel_scale:
        s = _rng(wid, layer, T_CHSCALE, expert).lognormal(0.0, 0.5, size=m).astype(np.float32)
        g *= s[:, None]
        u *= s[:, None]
        dn *= s[None, :]
    return f32_to_bf16_bits(g), f32_to_bf16_bits(u), f32_to_bf16_bits(dn)


def layer_weights(wid: int, layer: int, n_experts: int, d: int, m: int,
                  channel_scale: bool = False, experts=None):
    """Stacked weights ``[E][m][d], [E][m][d], [E][d][m]`` (bf16 bits).

    With ``experts`` given, only those experts are drawn; the others stay zero
    (useful when only the routed experts of a token are needed on the CPU).
    """
    wg = np.zeros((n_experts, m, d), np.uint16)
    wu = np.zeros((n_experts, m, d), np.uint16)
    wd = np.zeros((n_experts, d, m), np.uint16)

    def one(e):
        wg[e], wu[e], wd[e] = expert_weights(wid, layer, e, d, m, channel_scale)

    todo = list(range(n_experts) if experts is None else experts)
    if len(todo) > 1:
        # every expert has its own seeded stream, so threads change no value
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, len(todo), os.cpu_count() or 1)) as pool:
            list(pool.map(one, todo))
    else:
        for e in todo:
            one(e)
    return wg, wu, wd


def tokens(wid: int, layer: int, batch: int, d: int, index: int = 0) -> np.ndarray:
    """Decode-token activations x ~ N(0, 1), as bf16 bits ``[B][d]``."""
    return f32_to_bf16_bits(_rng(wid, layer, T_X, index).standard_normal((batch, d), dtype=np.float32))


def router_logits(wid: int, layer: int, batch: int, n_experts: int,
                  kind: str = "normal", index: int = 0, group: int = 0, group_size: int = 0) -> np.ndarray:
    """Router logits, float32 ``[B][E]``.

    ``normal``: iid N(0, 1).
    ``zipf``: expert popularity p_e proportional to rank^-1.1 over a seeded random
    ranking of the experts; logit = log p_e + Gumbel(0, 1) noise, so taking the
    top experts of a row samples experts without replacement in proportion to p.
    ``disjoint``: iid N(0, 1), then the experts of group ``group`` (members
    group * group_size .. + group_size - 1 of a seeded permutation of the
    experts) are lifted by a common shift that puts them above every other
    expert. Calls with different groups route to disjoint expert sets; the gate
    weights (a softmax over the chosen logits) are those of N(0, 1) logits.
    """
    rng = _rng(wid, layer, T_LOGITS, index)
    if kind == "normal":
        return rng.standard_normal((batch, n_experts), dtype=np.float32)
    if kind == "disjoint":
        lg = rng.standard_normal((batch, n_experts), dtype=np.float32)
        perm = _rng(wid, layer, T_PERM, 0).permutation(n_experts)
        chosen = perm[group * group_size:(group + 1) * group_size]
        assert chosen.size == group_size > 0, "group out of range"
        rest = np.setdiff1d(np.arange(n_experts), chosen)
        for t in range(batch):
            lift = (lg[t, rest].max() if rest.size else np.float32(0)) - lg[t, chosen].min() + np.float32(1)
            lg[t, chosen] += np.float32(max(lift, 0))
        return lg
    if kind == "zipf":
        perm = _rng(wid, layer, T_PERM, 0).permutation(n_experts)
        rank = np.empty(n_experts, np.int64)
        rank[perm] = np.arange(1, n_experts + 1)
        logp = -ZIPF_S * np.log(rank.astype(np.float64))
        logp -= np.log(np.exp(logp).sum())
        gumbel = rng.gumbel(0.0, 1.0, size=(batch, n_experts))
        return (logp[None, :] + gumbel).astype(np.float32)
    raise ValueError(f"unknown routing kind {kind!r}")


def router_weights(wid: int, layer: int, n_experts: int, d: int) -> np.ndarray:
    """Synthetic router matrix ``[E][d]`` ~ N(0, 0.02) as bf16 bits (stacked-layer workload)."""
    return f32_to_bf16_bits(_rng(wid, layer, T_ROUTER, 0).standard_normal((n_experts, d), dtype=np.float32)
                            * np.float32(WEIGHT_STD))


def budget_to_k(budget: float, m: int) -> int:
    """Channel count for a read budget given as a fraction of m (nearest integer)."""
    return int(np.floor(budget * m + 0.5))
