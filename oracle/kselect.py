"""Draft-length choice from step times (test infrastructure only).

Speculative decoding for MoE models (abstract): the time of a step is its
bytes over the effective bandwidth plus a fixed time, and that cost model is
what decides how many tokens to speculate.  With the method's greedy accept
(mlx-dflash README, "Architecture": cumulative-product match), a draft that
agrees with the target with independent probability alpha per token makes a
cycle of k drafts emit 1 + alpha + ... + alpha^k tokens in expectation
(accepted prefix + the verifier's token).  Reading: the acceptance is taken
as geometric (independent per position), the plainest model the pages'
cumulative-product accept admits.
"""
from __future__ import annotations


def expected_tokens(alpha: float, k: int) -> float:
    """E_k = sum_{i=0..k} alpha^i, summed term by term."""
    return sum(alpha ** i for i in range(k + 1))


def select_k(t_verify, t_draft: float, t_cycle: float, alpha: float) -> tuple[int, float]:
    """Smallest k in 0..len(t_verify)-1 maximising E_k / (k t_draft + t_verify[k] + t_cycle)."""
    best_k, best = 0, -1.0
    for k in range(len(t_verify)):
        r = expected_tokens(alpha, k) / (k * t_draft + t_verify[k] + t_cycle)
        if r > best:
            best_k, best = k, r
    return best_k, best
