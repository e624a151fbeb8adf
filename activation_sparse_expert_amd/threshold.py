"""Offline calibration of the threshold selector.

The pages contrast top-k with the usual selector, which keeps the channels whose
score exceeds a threshold tuned on an offline sample ("KAIST drops calibration
from MoE decoding, speeds up blocks by up to 2.69x over vLLM", section "The
threshold promises a budget but does not keep it"). These helpers set such a
threshold from channel scores the library produced on calibration tokens (read
back with moe_sel_debug_selection) and summarise the read fractions a selector
achieves, so the two selectors can be compared on identical scores.
"""
from __future__ import annotations

import numpy as np


def calibrate(scores: np.ndarray, budget: float) -> float:
    """Threshold over a set of channel scores (any shape, one entry per (token,
    routed expert, channel)) that keeps the `budget` fraction of them: the
    round(budget * N)-th largest score's successor in sorted order, so that (ties
    aside) exactly that many scores are strictly above it."""
    flat = np.sort(np.asarray(scores, np.float32).ravel())[::-1]
    keep = int(np.floor(budget * flat.size + 0.5))
    if keep >= flat.size:
        return 0.0
    return float(flat[keep])


def read_fractions(chan_count: np.ndarray, m: int) -> np.ndarray:
    """Per-token fraction of the routed experts' channels read: the mean over the
    token's routed experts of count / m. chan_count: [tokens][top_e]."""
    return np.asarray(chan_count, np.float64).mean(axis=1) / m


def summary(fractions: np.ndarray) -> dict:
    f = np.asarray(fractions, np.float64)
    return {"mean": round(float(f.mean()), 5), "std": round(float(f.std()), 5), "min": round(float(f.min()), 5),
            "p5": round(float(np.percentile(f, 5)), 5), "p95": round(float(np.percentile(f, 95)), 5),
            "max": round(float(f.max()), 5)}
