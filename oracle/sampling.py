"""Speculative sampling: the non-greedy accept (test infrastructure only).

LayerSkip summary 4.3.2 (self-verification): under sampling, rejection
sampling makes the output distribution equal to the full model's, following
the standard speculative decoding protocol.  Written here from that protocol:
draft d_i ~ q_i; accept d_i with probability min(1, p_{i-1}(d_i) / q_i(d_i))
in order; at the first rejection emit a token drawn from max(0, p - q)
normalised and stop; if all k drafts pass, emit a token drawn from p_k.
p and q are softmax(logits / T).

Random numbers: Philox4x64-10 (Salmon et al., "Parallel random numbers: as
easy as 1, 2, 3", SC 2011), key (seed, 0), counter (cycle, slot, purpose, 0);
the first output word's top 24 bits make u in [0, 1).  Purposes: 0 the
draft of slot j, 1 the accept test of draft i, 2 the final token of a cycle
whose accepted count is a (slot a).  Draws from a distribution take the
smallest index whose running sum exceeds u times the total.
"""
from __future__ import annotations

import numpy as np

M64 = (1 << 64) - 1


def philox4x64_10(ctr, key) -> list[int]:
    """Ten Philox rounds on a 4x64-bit counter with a 2x64-bit key."""
    c, k = [int(x) & M64 for x in ctr], [int(x) & M64 for x in key]
    for _ in range(10):
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & M64, (p0 >> 64) ^ c[3] ^ k[1], p0 & M64]
        k = [(k[0] + 0x9E3779B97F4A7C15) & M64, (k[1] + 0xBB67AE8584CAA73B) & M64]
    return c


def uniform24(seed: int, cycle: int, slot: int, purpose: int) -> float:
    w = philox4x64_10([cycle, slot, purpose, 0], [seed, 0])[0]
    return (w >> 40) / float(1 << 24)


def probs(logits, T: float) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / T
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def draw(weights, u: float) -> tuple[int, float]:
    """Smallest j with cumsum(w)[j] > u * sum(w); also the distance of u * sum
    to the nearest running-sum boundary relative to the sum (a near tie is
    decided by rounding)."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    tot = c[-1]
    t = u * tot
    j = int(np.searchsorted(c, t, side="right"))
    if j >= len(w):
        j = int(np.nonzero(w > 0)[0][-1])
    lo = c[j - 1] if j > 0 else 0.0
    margin = min(abs(t - lo), abs(c[j] - t)) / tot
    return j, margin


def spec_cycle(target_logits, draft_logits, T: float, seed: int, cycle: int, drafts=None):
    """One draft/verify/accept cycle.  target_logits [k+1, V] (rows p_0..p_k),
    draft_logits [k, V] (row i-1 is q for draft i).  drafts: the k draft
    tokens, or None to draw them from q.  Returns (a, emitted, margin) where
    emitted = d_1..d_a + the final token and margin the smallest relative
    distance of any decision to its threshold."""
    tl = np.asarray(target_logits, dtype=np.float64)
    dl = np.asarray(draft_logits, dtype=np.float64).reshape(-1, tl.shape[1])
    k = dl.shape[0]
    margin = np.inf
    if drafts is None:
        drafts = []
        for i in range(k):
            j, m = draw(probs(dl[i], T), uniform24(seed, cycle, i, 0))
            drafts.append(j)
            margin = min(margin, m)
    out = []
    for i in range(1, k + 1):
        p, q = probs(tl[i - 1], T), probs(dl[i - 1], T)
        d = int(drafts[i - 1])
        u = uniform24(seed, cycle, i, 1)
        margin = min(margin, abs(u * q[d] - p[d]) / max(q[d], 1e-300))
        if u * q[d] < p[d]:
            out.append(d)
            continue
        r = np.maximum(p - q, 0.0)
        if not np.any(r > 0):
            r = p
        j, m = draw(r, uniform24(seed, cycle, i - 1, 2))
        return i - 1, out + [j], min(margin, m)
    j, m = draw(probs(tl[k], T), uniform24(seed, cycle, k, 2))
    return k, out + [j], min(margin, m)
