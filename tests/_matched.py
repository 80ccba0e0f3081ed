"""The oracle run with its bf16 rounding decisions checked against the GPU's.

A bf16 workload stores bf16(v) at fixed points (the GEMM inputs, q after the
rotary embedding, the K/V entries, the attention output, the SwiGLU
activation).  The GPU computes v in float32 and the oracle in float64; where
v lies within the float32 error of a rounding midpoint, both bf16 neighbours
are correct results, and one such decision that differs moves every later
value by a bf16 step.  Those decisions compound through the layers, which is
why two correct implementations drift apart at the 8B widths.

MatchedModel compares, at every storage point of a pass, the GPU's stored
value g with the oracle's own value v:

- g == bf16(v): an exact match;
- otherwise g is accepted as an ambiguous decision when it is the bf16
  rounding of some value within delta = WINDOW * rms(row) of v, i.e.
  bf16(v - delta) <= g <= bf16(v + delta) (rounding is monotone): for a value
  well away from zero that is the other neighbour of v when v lies within
  delta of their midpoint; for a value within delta of zero, any bf16 value
  within delta of it;
- anything else: a mismatch, recorded as a failure.

The oracle then continues with g, so the next operations see the same
operands on both sides and only float32-level differences remain.  WINDOW =
2^-14 bounds the float32 error of the computed values relative to the row's
magnitude: a float32 dot product of K <= 14336 random-sign terms has a
relative error of about 2^-24 * sqrt(K) (the rounding errors add like a
random walk); 8 standard deviations of that is 5.7e-5, below 2^-14 = 6.1e-5.
The other steps between storage points (the norm factor, the rotary
rotation, the softmax with bf16-pair probabilities (16 significant bits)
and the SwiGLU) add less than 2^-16 relative.

Test infrastructure: the oracle's arithmetic is unchanged (this subclasses
the storage rounding only), and nothing here is used by the HIP path.
"""
from __future__ import annotations

import numpy as np

from oracle import Model
from oracle.model import bf16_round

WINDOW = 2.0 ** -14


def bits_to_f64(a) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Point:
    """Counts of one storage point over a pass."""

    def __init__(self, name):
        self.name, self.n, self.exact, self.ambiguous, self.bad, self.worst = name, 0, 0, 0, 0, 0.0

    def __repr__(self):
        return f"{self.name}: {self.n} values, {self.exact} exact, {self.ambiguous} ambiguous, {self.bad} mismatched"


class MatchedModel(Model):
    """Oracle whose storage roundings check (and then follow) the GPU's stored
    values.  ``expect`` is the list of (name, GPU values as float64) in the
    order the oracle stores them during the pass."""

    def __init__(self, cfg, weights, **kw):
        super().__init__(cfg, weights, **kw)
        assert self.bf16, "storage points exist in bf16 workloads only"
        self.expect = []
        self.points, self.h_after, self.x_after = {}, {}, {}
        self.moe_act = {}

    def rn(self, x):
        r = bf16_round(x)
        if not self.expect:
            return r
        name, g = self.expect.pop(0)
        g = np.asarray(g, dtype=np.float64).reshape(r.shape)
        p = self.points.setdefault(name, Point(name))
        rows = x.reshape(x.shape[0], -1)
        rms = np.sqrt(np.mean(rows * rows, axis=1)).reshape((-1,) + (1,) * (x.ndim - 1))
        exact = g == r
        delta = WINDOW * rms
        ok = (g >= bf16_round(x - delta)) & (g <= bf16_round(x + delta))
        amb = ~exact & ok
        bad = ~ok
        p.n += x.size
        p.exact += int(exact.sum())
        p.ambiguous += int(amb.sum())
        p.bad += int(bad.sum())
        if bad.any():
            p.worst = max(p.worst, float(np.max((np.abs(g - r) / rms)[bad])))
        return g

    # MoE layers: each expert evaluation's activation is checked against the
    # GPU's act buffer [token][slot][expert_ffn] (routed slots, then shared)
    def expert(self, l, e, rows, rstd, shared=False):
        act = self.moe_act.get(l)
        if act is None:
            return super().expert(l, e, rows, rstd, shared)
        xg = self._xg
        t = np.array([int(np.nonzero(np.all(xg == r, axis=1))[0][0]) for r in rows])
        if shared:
            j = np.full(len(t), self.cfg["top_k"] + e)
        else:
            ids = np.asarray(self.routing[l])[:xg.shape[0]]
            j = np.array([int(np.nonzero(ids[ti] == e)[0][0]) for ti in t])
        self.expect.insert(0, ("moe_act", act[t, j]))
        return super().expert(l, e, rows, rstd, shared)

    def moe_ffn(self, l, xg, rstd=None, dedup=False):
        self._xg = xg
        return super().moe_ffn(l, xg, rstd, dedup)

    # the residual after each block, for comparison with the GPU's trace
    def attention_block(self, l, x, pos0, cache):
        h = super().attention_block(l, x, pos0, cache)
        self.h_after[l] = h
        return h

    def layer(self, l, x, pos0, cache, dedup=False):
        y = super().layer(l, x, pos0, cache, dedup)
        self.x_after[l] = y
        return y

    def run(self, tokens, pos0, cache, expect, layers=None, moe_act=None, dedup=False):
        """One pass with the GPU's stored values ``expect`` (and, for MoE
        layers, their activations ``moe_act``: layer -> [M, slots, fe]);
        returns logits."""
        self.expect = list(expect)
        self.moe_act = dict(moe_act or {})
        self.points, self.h_after, self.x_after = {}, {}, {}
        logits = self.forward(tokens, pos0, cache, layers=layers, dedup=dedup)
        assert not self.expect, f"{len(self.expect)} stored values left unused"
        return logits


def expected_points(eng, cfg, layers, rows, n, kv_rows):
    """The GPU's stored values of the last traced pass, in the oracle's order:
    per run layer the QKV input, q, the new K and V entries, the attention
    output, the gate/up input (bf16(x * ffn_norm), also in MoE layers) and, for dense layers, the
    activation; then, for a full pass of a feature-tap model, the concat of
    the tapped residuals and the fc output; then the LM head input.  Returns
    (expect, moe_act), moe_act: layer -> [rows, slots, fe] of the MoE layers.
    kv_rows: (K, V) bf16 arrays per layer, [heads, n + rows, hd]."""
    c = eng.cfg
    hq, hd = c.n_q_heads, c.head_dim
    out, moe_act = [], {}
    for l in layers:
        k, v = kv_rows[l]
        out += [("xg_attn", bits_to_f64(eng.read_trace_point(l, 0, rows))),
                ("q", bits_to_f64(eng.read_trace_point(l, 1, rows)).reshape(rows, hq, hd)),
                ("k", bits_to_f64(k[:, n:n + rows]).transpose(1, 0, 2)),
                ("v", bits_to_f64(v[:, n:n + rows]).transpose(1, 0, 2)),
                ("att", bits_to_f64(eng.read_trace_point(l, 2, rows))),
                ("xg_ffn", bits_to_f64(eng.read_trace_point(l, 4, rows)))]
        act = bits_to_f64(eng.read_trace_point(l, 5, rows))
        if c.n_experts > 0 and l >= c.n_dense_layers:
            moe_act[l] = act.reshape(rows, c.top_k + c.n_shared, c.expert_ffn)
        else:
            out.append(("act", act))
    if cfg["feat_layers"] and list(layers) == list(range(c.n_layers)):
        x = eng.read_trace(rows)
        cat = np.concatenate([x[l] for l in cfg["feat_layers"]], axis=-1).astype(np.float64)
        out += [("cat", bf16_round(cat)),            # the tap stores bf16 of the float32 residual
                ("features", bits_to_f64(eng.read_features(rows)))]
    out.append(("xg_head", bits_to_f64(eng.read_trace_point(c.n_layers, 0, rows))))
    return out, moe_act


def _prefix_cache(cfg, kv, n):
    """Oracle cache holding the GPU's entries of positions [0, n) of every layer."""
    from oracle.model import Cache
    cache = Cache(cfg)
    for l, (k, v) in enumerate(kv):
        cache.K[l][:, :n] = bits_to_f64(k[:, :n])
        cache.V[l][:, :n] = bits_to_f64(v[:, :n])
    return cache


def check_matched(tag, cfg, w, eng, tokens, n, layers, gpu_logits, routing=None, dedup=False):
    """The oracle runs the GPU's last traced pass (tokens at positions n.., the
    layers in `layers`, the GPU's cache entries before n) with every bf16
    storage decision checked against the GPU's stored value (MatchedModel).

    Bounds, all derived rather than fitted:
    - stored values: the oracle's own rounding, or the rounding of a value
      within 2^-14 of the row's rms of the oracle's value (the float32 error
      of the computed value, WINDOW above);
    - residuals: after the attention block and after the layer, within the
      sum over the layers so far of 2^-14 x (rms of the attention update +
      rms of the FFN update), plus one float32 rounding of the residual;
    - logits: |dlogit| <= 3e-2, tokens equal wherever the oracle's top-1 /
      top-2 gap exceeds 6e-2.
    Also runs the plain oracle (its own rounding decisions) on the same
    prefix: its logits move by the rounding flips compounding through the
    layers, which the matched run shows to be the whole of the difference."""
    M = len(tokens)
    kv = [eng.read_kv(l, 0, n + M) for l in range(cfg["n_layers"])]
    x_gpu = eng.read_trace(M).astype(np.float64)
    h_gpu = {l: eng.read_trace_point(l, 3, M).astype(np.float64) for l in layers}
    expect, moe_act = expected_points(eng, cfg, layers, M, n, kv)
    mm = MatchedModel(cfg, w)
    if routing is not None:
        mm.routing = {l: routing[l] for l in range(cfg["n_layers"])}
    run_layers = None if list(layers) == list(range(cfg["n_layers"])) else layers
    lg = mm.run(tokens, n, _prefix_cache(cfg, kv, n), expect, layers=run_layers, moe_act=moe_act, dedup=dedup)
    for name, p in mm.points.items():
        print(f"[{tag}] {p} (worst mismatch {p.worst:.2e} of the row rms)", flush=True)
        assert p.bad == 0, (name, p.bad)
    drift, prev, worst = 0.0, None, 0.0
    for l in layers:
        x_in = mm.x_after[prev] if prev is not None else mm.embed(tokens)
        u_att = mm.h_after[l] - x_in
        u_ffn = mm.x_after[l] - mm.h_after[l]
        rms = lambda a: float(np.sqrt(np.mean(a * a)))
        drift_h = drift + 2.0 ** -14 * rms(u_att)
        drift += 2.0 ** -14 * (rms(u_att) + rms(u_ffn))
        for got, ref, lim in ((h_gpu[l], mm.h_after[l], drift_h), (x_gpu[l], mm.x_after[l], drift)):
            err = np.abs(got - ref) - 2.0 ** -23 * np.abs(ref)
            worst = max(worst, float(np.max(err)) / lim)
            assert np.max(err) <= lim, (l, float(np.max(err)), lim)
        prev = l
    err = float(np.max(np.abs(lg - gpu_logits)))
    print(f"[{tag}] matched: residual drift <= {worst:.2e} of its bound; max |dlogit| {err:.2e}", flush=True)
    assert err <= 3e-2
    for r, g in zip(lg, gpu_logits):
        top = np.sort(r)[-2:]
        if top[1] - top[0] > 6e-2:
            assert int(np.argmax(r)) == int(np.argmax(g))
    mm.expect = []                      # the oracle's own rounding decisions from here on
    mm.moe_act = {}
    plain = mm.forward(tokens, n, _prefix_cache(cfg, kv, n), layers=run_layers, dedup=dedup)
    print(f"[{tag}] plain oracle (own rounding decisions) on the same prefix: max |dlogit| "
          f"{float(np.max(np.abs(plain - gpu_logits))):.2e}", flush=True)
    return err
