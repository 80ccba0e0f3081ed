"""Skip set as a knapsack (test infrastructure only).

MLX layer-skip blog, "Paper -> the idea": choosing the skipped layers is a
constrained optimisation, keeping the draft accurate within a compute budget
with per-layer costs measured on the hardware, and the cosine similarity
between hidden states serving as the acceptance proxy.  Reading: a layer's
value is 1 - cos(its input, its output) averaged over rows (how much it turns
the residual), the kept set maximises the summed value of kept layers with
their summed cost within the budget; written here by brute force.
"""
from __future__ import annotations

import itertools

import numpy as np


def layer_cosines(embedded: np.ndarray, residuals: list[np.ndarray]) -> np.ndarray:
    """Mean over rows of cos(input of layer l, output of layer l); the input of
    layer 0 is the embedding, of layer l > 0 the output of layer l - 1."""
    out, prev = [], np.asarray(embedded, dtype=np.float64)
    for x in residuals:
        x = np.asarray(x, dtype=np.float64)
        c = np.sum(prev * x, axis=-1) / np.sqrt(np.sum(prev * prev, axis=-1) * np.sum(x * x, axis=-1))
        out.append(float(np.mean(c)))
        prev = x
    return np.array(out)


def knapsack_skip_brute(cost, value, budget) -> tuple[float, list[tuple[int, ...]]]:
    """Best summed value of a kept set within the budget, and every kept set
    (as a tuple of layer indices) that reaches it."""
    n = len(cost)
    best, sets = -1.0, []
    for r in range(n + 1):
        for keep in itertools.combinations(range(n), r):
            if sum(cost[i] for i in keep) > budget:
                continue
            v = sum(value[i] for i in keep)
            if v > best + 1e-12:
                best, sets = v, [keep]
            elif abs(v - best) <= 1e-12:
                sets.append(keep)
    return best, sets
