"""Target distribution over the vocabulary (oracle; test infrastructure only).

At temperature T > 0 the target's next-token distribution after node i is the
softmax of its logits divided by T; at T = 0 decoding always takes the most
probable token (EAGLE-2 overview blog, §1: temperature 0 always picks the
highest-probability candidate; EAGLE-p2 §2 Preliminaries covers greedy and
non-greedy decoding).  Ties in the argmax go to the lowest token id.
"""
from __future__ import annotations

import numpy as np


def argmax_lowest(logits_row) -> int:
    row = np.asarray(logits_row)
    best = 0
    for v in range(1, row.shape[0]):
        if row[v] > row[best]:
            best = v
    return best


def target_distribution(logits_row, T: float) -> np.ndarray:
    """fp64 [V]: softmax(logits / T) for T > 0, one-hot of the argmax for T = 0."""
    row = np.asarray(logits_row, dtype=np.float64)
    if not np.all(np.isfinite(row)):
        raise ValueError("non-finite logits")
    if T < 0 or not np.isfinite(T):
        raise ValueError("temperature must be finite and >= 0")
    if T == 0:
        out = np.zeros(row.shape[0])
        out[argmax_lowest(row)] = 1.0
        return out
    z = (row - row.max()) / T
    e = np.exp(z)
    return e / e.sum()
