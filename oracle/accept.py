"""Greedy accept of a verified draft block.

Sources: mlx-dflash README, "Architecture" (accept = greedy cumulative-product
match of draft against target prediction, then advance by the accepted length
plus one); LayerSkip summary page, 4.3.2 "Self-Verification" (consecutive
accepted drafts from the start are kept, the verifier's own prediction replaces
the first rejected draft, and the next cycle starts after it).

Inputs: drafts d[0..k) (the drafted tokens d_1..d_k) and the verifier's greedy
predictions p[0..k] (p[i] is the target's argmax after block position i).
Draft d[i] is correct when it equals p[i].

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations


def accept(drafts, posterior) -> tuple[int, list[int]]:
    """Return (a, emitted): a = length of the longest matching prefix,
    emitted = d[0..a) followed by the correction/bonus token p[a]."""
    k = len(drafts)
    if len(posterior) != k + 1:
        raise ValueError("posterior must hold k+1 predictions")
    a = 0
    while a < k and int(drafts[a]) == int(posterior[a]):
        a += 1
    return a, [int(t) for t in drafts[:a]] + [int(posterior[a])]


def accept_brute(drafts, posterior) -> int:
    """Accepted length as the cumulative product of the match indicators:
    a = sum_i prod_{j <= i} [d_j == p_j]."""
    a, run = 0, 1
    for i in range(len(drafts)):
        run *= 1 if int(drafts[i]) == int(posterior[i]) else 0
        a += run
    return a
