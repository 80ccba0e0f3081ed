"""Skip set of the naive layer-skip draft.

Source: MLX layer-skip blog ("I built self-speculative decoding for MLX"),
section "Code -> the implementation": the draft drops a contiguous block of
max(1, round(n * skip_frac)) layers centred in the stack, starting at
(n - n_skip) // 2, and keeps every other layer in its original order.
``round`` is Python's (half to even); layers are 0-indexed.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations


def skip_layers(n_layers: int, frac: float) -> list[int]:
    """0-indexed layers the draft skips."""
    if n_layers <= 0:
        return []
    n_skip = max(1, round(n_layers * frac))
    n_skip = min(n_skip, n_layers)
    start = (n_layers - n_skip) // 2
    return list(range(start, start + n_skip))


def skip_mask(n_layers: int, frac: float) -> list[int]:
    """u8-style mask: 1 where the draft skips the layer."""
    s = set(skip_layers(n_layers, frac))
    return [1 if l in s else 0 for l in range(n_layers)]
