"""Oracle decoder, greedy decode and shared-cache greedy self-speculation.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 throughout.

Model (LayerSkip summary page, "Notation and Baseline Architecture"): a
decoder-only stack of L residual layers x_{l+1} = x_l + f_l(x_l), then the
shared head g = final norm + LM head.  The layer is the Llama family the
summary names in its limitations section: pre-norm RMSNorm, rotary position
embedding, grouped-query attention, SwiGLU feed-forward; no biases; untied
head.  Readings the pages leave open: RoPE base 10000 with the rotate-half
pairing (i, i + hd/2); RMSNorm epsilon 1e-5; query head h reads KV head
floor(h * Hkv / Hq).

Self-speculation (LayerSkip summary 4.3.1-4.3.3; MLX layer-skip blog "Code";
mlx-dflash README "Architecture"): the draft runs k tokens autoregressively
through the kept layers only, reading and writing one KV cache shared with the
full model; one verify pass runs [t_last, d_1..d_k] through all layers and
overwrites those cache positions; the longest matching prefix is accepted plus
the verifier's next token, and the cache is cut back to the committed length.

MoE feed-forward (speculative decoding for MoE models, abstract): the router
softmax picks top_k experts per token; the per-slot form evaluates each
(token, slot) expert separately, the deduplicated form evaluates every expert
of the pass's union once over all rows that chose it.  Both sum
sum_j w_j E_{e_j}(x) + sum_s S_s(x) in slot order.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# numerics
# ---------------------------------------------------------------------------


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits,
    ties to even), returned as float64.  Normal range only (the path never
    produces bf16 subnormals or overflows)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def decode_weight(a: np.ndarray) -> np.ndarray:
    """Stored weight -> float64: float32 as is; uint16 read as bf16 bits."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing.  x [M, H, hd], pos [M].

    Dimension pair (i, i + hd/2) of a row at position p is rotated by the
    angle p * theta**(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [M, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(z: np.ndarray) -> np.ndarray:
    z = z - np.max(z, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# KV cache
# ---------------------------------------------------------------------------


class Cache:
    """One KV cache shared by draft and verify: K, V [L][Hkv, max_ctx, hd]."""

    def __init__(self, cfg: dict):
        L, hkv, hd, n = cfg["n_layers"], cfg["n_kv_heads"], cfg["head_dim"], cfg["max_ctx"]
        self.K = [np.zeros((hkv, n, hd)) for _ in range(L)]
        self.V = [np.zeros((hkv, n, hd)) for _ in range(L)]


# ---------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------


class Model:
    """Decoder of ``cfg`` with weights ``weights`` (name -> stored array)."""

    def __init__(self, cfg: dict, weights: dict[str, np.ndarray], keep_f32: bool | None = None):
        self.cfg = cfg
        self.bf16 = cfg["dtype"] == "bf16"
        n_el = sum(int(np.prod(a.shape)) for a in weights.values())
        # Large models keep weights as float32 (exact for bf16 values) and widen per product.
        if keep_f32 is None:
            keep_f32 = n_el > 300_000_000
        self.w = {}
        for k, a in weights.items():
            v = decode_weight(a)
            self.w[k] = v.astype(np.float32) if keep_f32 else v
        self.L = cfg["n_layers"]
        self.hq, self.hkv, self.hd = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        self.eps, self.theta = cfg["rms_eps"], cfg["rope_theta"]
        self.routing = None          # optional injected expert ids {layer: [M, top_k]}
        self.union = {}              # layer -> size of the last pass's expert union
        self.features = None         # last pass's fc output (feature tap)

    # storage rounding: identity for float32 workloads
    def rn(self, x):
        return bf16_round(x) if self.bf16 else x

    def lin(self, x: np.ndarray, W: np.ndarray) -> np.ndarray:
        """x [M, in] times W [out, in] transposed."""
        return x @ W.astype(np.float64, copy=False).T

    def norm_input(self, x: np.ndarray, g: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
        """RMSNorm with gain g, as it feeds a product: the stored operand is
        the gain-scaled input x * g (rounded like every stored matrix input)
        and the per-row 1/rms factor [M, 1] multiplies each product of it.
        The normalisation is a per-row scalar, so it commutes with the
        product: in exact arithmetic lin(x * g, W) * rstd = lin(rmsnorm(x, g), W)."""
        rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + self.eps)
        return self.rn(x * g), rstd

    def normed_lin(self, x: np.ndarray, g: np.ndarray, Ws) -> list[np.ndarray]:
        """RMSNorm with gain g followed by products with each W of Ws (norm_input)."""
        xg, rstd = self.norm_input(x, g)
        return [self.lin(xg, W) * rstd for W in Ws]

    # -- blocks --------------------------------------------------------------

    def embed(self, tokens) -> np.ndarray:
        return self.w["embed"][np.asarray(tokens, dtype=np.int64)].astype(np.float64)

    def attention_block(self, l: int, x: np.ndarray, pos0: int, cache: Cache) -> np.ndarray:
        w, p = self.w, f"l{l}."
        M = x.shape[0]
        pos = np.arange(pos0, pos0 + M)
        q, k, v = self.normed_lin(x, w[p + "attn_norm"], [w[p + "wq"], w[p + "wk"], w[p + "wv"]])
        q = q.reshape(M, self.hq, self.hd)
        k = k.reshape(M, self.hkv, self.hd)
        v = v.reshape(M, self.hkv, self.hd)
        q = self.rn(rope(q, pos, self.theta))
        k = self.rn(rope(k, pos, self.theta))
        v = self.rn(v)
        cache.K[l][:, pos0:pos0 + M] = k.transpose(1, 0, 2)
        cache.V[l][:, pos0:pos0 + M] = v.transpose(1, 0, 2)
        out = self.attend(q, cache.K[l][:, :pos0 + M], cache.V[l][:, :pos0 + M], pos)
        att = self.rn(out.reshape(M, self.hq * self.hd))
        return x + self.lin(att, w[p + "wo"])

    def attend(self, q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """Causal grouped-query attention of queries q [M, Hq, hd] at positions
        pos over the cache entries Kc, Vc [Hkv, ctx, hd]: softmax(q.k / sqrt(hd))
        over the keys at positions <= the query's own."""
        M, ctx = q.shape[0], Kc.shape[1]
        out = np.zeros((M, self.hq, self.hd))
        scale = 1.0 / np.sqrt(self.hd)
        for h in range(self.hq):
            g = (h * self.hkv) // self.hq
            s = (q[:, h, :] @ Kc[g].T) * scale                     # [M, ctx]
            s = np.where(np.arange(ctx)[None, :] <= pos[:, None], s, -np.inf)
            out[:, h, :] = softmax(s) @ Vc[g]
        return out

    def dense_ffn(self, l: int, h: np.ndarray) -> np.ndarray:
        """SwiGLU feed-forward of the normed residual h (ffn_norm folded in)."""
        w, p = self.w, f"l{l}."
        gate, up = self.normed_lin(h, w[p + "ffn_norm"], [w[p + "w_gate"], w[p + "w_up"]])
        act = self.rn(silu(gate) * up)
        return self.lin(act, w[p + "w_down"])

    def expert(self, l: int, e: int, rows: np.ndarray, rstd: np.ndarray, shared: bool = False) -> np.ndarray:
        """SwiGLU expert e of layer l on stored input rows [n, d] whose gate
        and up products take their rows' 1/rms factors rstd [n, 1]."""
        w, p = self.w, f"l{l}." + ("sh_" if shared else "exp_")
        gate = self.lin(rows, w[p + "gate"][e]) * rstd
        up = self.lin(rows, w[p + "up"][e]) * rstd
        act = self.rn(silu(gate) * up)
        return self.lin(act, w[p + "down"][e])

    def route(self, l: int, xg: np.ndarray, rstd: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
        """Router probabilities [M, E] and top_k ids [M, top_k] (ties -> lower
        id) of stored input rows xg with 1/rms factors rstd (None: 1)."""
        z = self.lin(xg, self.w[f"l{l}.router"])
        if rstd is not None:
            z = z * rstd
        probs = softmax(z)
        ids = np.argsort(-probs, axis=-1, kind="stable")[:, :self.cfg["top_k"]]
        return probs, ids

    def moe_ffn(self, l: int, xg: np.ndarray, rstd: np.ndarray | None = None, dedup: bool = False) -> np.ndarray:
        """Routed and shared experts of layer l over stored input rows xg
        [M, d]; rstd [M, 1]: the rows' 1/rms factors of the folded ffn norm
        (norm_input), which multiply the router's and the experts' gate and
        up products (None: 1, the block applied to xg itself)."""
        M = xg.shape[0]
        r = np.ones((M, 1)) if rstd is None else rstd
        probs, ids = self.route(l, xg, r)
        if self.routing is not None:
            ids = np.asarray(self.routing[l], dtype=np.int64)[:M]
        gate = np.take_along_axis(probs, ids, axis=-1)             # not renormalised
        self.union[l] = len(set(int(e) for e in ids.reshape(-1)))
        y = np.zeros(xg.shape)
        if dedup:
            # every expert of the union evaluated once over the rows that chose it
            per = np.zeros((M, ids.shape[1], xg.shape[1]))
            for e in sorted(set(int(e) for e in ids.reshape(-1))):
                t, j = np.nonzero(ids == e)
                per[t, j] = self.expert(l, e, xg[t], r[t])
            for j in range(ids.shape[1]):
                y = y + gate[:, j:j + 1] * per[:, j]
        else:
            for j in range(ids.shape[1]):
                outj = np.stack([self.expert(l, int(ids[t, j]), xg[t:t + 1], r[t:t + 1])[0] for t in range(M)])
                y = y + gate[:, j:j + 1] * outj
        for s in range(self.cfg["n_shared"]):
            y = y + self.expert(l, s, xg, r, shared=True)
        return y

    def layer(self, l: int, x: np.ndarray, pos0: int, cache: Cache, dedup: bool = False) -> np.ndarray:
        h = self.attention_block(l, x, pos0, cache)
        if self.cfg["n_experts"] > 0 and l >= self.cfg["n_dense_layers"]:
            # router and experts share one stored input, the ffn norm folded in
            xg, rstd = self.norm_input(h, self.w[f"l{l}.ffn_norm"])
            return h + self.moe_ffn(l, xg, rstd, dedup)
        return h + self.dense_ffn(l, h)

    def head(self, x: np.ndarray) -> np.ndarray:
        return self.normed_lin(x, self.w["final_norm"], [self.w["lm_head"]])[0]

    def forward(self, tokens, pos0: int, cache: Cache, layers=None, dedup: bool = False) -> np.ndarray:
        """Logits [M, V] for tokens at positions pos0..pos0+M-1, writing the
        cache of every layer run.  ``layers``: the layers to run, in order
        (default all); skipped layers leave the residual unchanged."""
        x = self.embed(tokens)
        feat = {}
        for l in (range(self.L) if layers is None else layers):
            x = self.layer(l, x, pos0, cache, dedup)
            feat[l] = x
        fl = self.cfg["feat_layers"]
        if fl and layers is None:
            cat = self.rn(np.concatenate([feat[l] for l in fl], axis=-1))
            self.features = self.rn(self.lin(cat, self.w["fc"]))
        return self.head(x)

    # -- decoding ----------------------------------------------------------------

    def prefill(self, prompt) -> tuple[Cache, int, np.ndarray]:
        cache = Cache(self.cfg)
        logits = self.forward(prompt, 0, cache)
        return cache, len(prompt), logits[-1]

    def greedy(self, prompt, n_new: int) -> tuple[list[int], np.ndarray]:
        """Plain greedy decode: n_new tokens (the first from the prefill).
        Returns the tokens and the logits row that produced each."""
        cache, n, last = self.prefill(prompt)
        out, rows = [int(np.argmax(last))], [last]
        while len(out) < n_new:
            lg = self.forward([out[-1]], n, cache)[0]
            n += 1
            out.append(int(np.argmax(lg)))
            rows.append(lg)
        return out, np.stack(rows)

    def teacher_forced(self, prompt, generated) -> np.ndarray:
        """Logits rows that predict generated[0..N) in one causal pass over
        prompt + generated[:-1]."""
        seq = list(prompt) + list(generated[:-1])
        cache = Cache(self.cfg)
        return self.forward(seq, 0, cache)[len(prompt) - 1:]

    def self_spec(self, prompt, n_new: int, skip, k: int, draft_fn=None) -> tuple[list[int], dict]:
        """Greedy self-speculative decode with one shared KV cache.

        ``skip``: iterable of 0-indexed layers the draft skips.  ``draft_fn``
        (tests only) may replace each drafted token: draft_fn(j, token) -> token.
        Returns the tokens (truncated to n_new) and cycle statistics."""
        from .accept import accept
        skip = set(int(s) for s in skip)
        kept = [l for l in range(self.L) if l not in skip]
        cache, n, last = self.prefill(prompt)
        out = [int(np.argmax(last))]
        t_last = out[0]
        stats = dict(cycles=0, drafted=0, accepted=0, a_hist=[])
        while len(out) < n_new:
            if n + k + 1 > self.cfg["max_ctx"]:
                raise ValueError("context capacity exceeded")
            drafts, tok = [], t_last
            for j in range(k):
                lg = self.forward([tok], n + j, cache, layers=kept)[0]
                tok = int(np.argmax(lg))
                if draft_fn is not None:
                    tok = int(draft_fn(j, tok))
                drafts.append(tok)
            lg = self.forward([t_last] + drafts, n, cache)
            post = [int(np.argmax(r)) for r in lg]
            a, emitted = accept(drafts, post)
            out += emitted
            n += a + 1
            t_last = emitted[-1]
            stats["cycles"] += 1
            stats["drafted"] += k
            stats["accepted"] += a
            stats["a_hist"].append(a)
        return out[:n_new], stats
