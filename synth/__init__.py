"""Seeded synthetic inputs shared by the HIP path's harness and by the oracle.

This module holds the workload shapes and the random draws only: model
weights, prompts, the synthetic MoE routing trace and the random parts of the
geometric-prefix verify blocks.  It contains none of the decoding method's
arithmetic, and it imports neither the oracle nor the HIP binding.

Weight matrices are normal N(0, 0.02), drawn per tensor chunk from
``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id, chunk])))``
(norm gains are 1).  bf16 configurations draw float32 and store the
round-to-nearest-even bf16 bit pattern (uint16); float32 configurations
store float32.  Prompts are uniform over the vocabulary.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

_DENSE_DEFAULTS = dict(rms_eps=1e-5, rope_theta=10000.0, n_experts=0, top_k=0,
                       n_shared=0, expert_ffn=0, n_dense_layers=0, dense_ffn=0,
                       feat_layers=(), out_scale={})

CONFIGS = {
    # tiny fp32 decoder: parity workload (fits in cache)
    "tiny": dict(_DENSE_DEFAULTS, name="tiny", cid=0, n_layers=4, d_model=256,
                 n_q_heads=4, n_kv_heads=4, head_dim=64, ffn_dim=1024,
                 vocab=4096, dtype="f32", prompt_len=32, n_new=64,
                 skip_layers=(1, 2), k=3, max_ctx=128,
                 out_scale={1: 0.1, 2: 0.1}),
    # Qwen3-4B-shaped bf16
    "qwen3-4b": dict(_DENSE_DEFAULTS, name="qwen3-4b", cid=1, n_layers=36,
                     d_model=2560, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     ffn_dim=9728, vocab=151936, dtype="bf16", prompt_len=512,
                     n_new=256, skip_frac=0.2, k=3, max_ctx=2048 + 17),
    # Llama-3.1-8B-shaped bf16 (the headline decode workload)
    "llama-8b": dict(_DENSE_DEFAULTS, name="llama-8b", cid=2, n_layers=32,
                     d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     ffn_dim=14336, vocab=128256, dtype="bf16", prompt_len=1024,
                     n_new=512, skip_fracs=(0.1, 0.2, 0.3, 0.4, 0.5),
                     ks=(2, 3, 5), skip_frac=0.2, k=3, max_ctx=2048 + 17),
    # Qwen3-8B-shaped bf16 target verifying 16-token blocks at context 2048
    "qwen3-8b": dict(_DENSE_DEFAULTS, name="qwen3-8b", cid=3, n_layers=36,
                     d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     ffn_dim=12288, vocab=151936, dtype="bf16", prompt_len=2048,
                     block=16, geo_p=(0.5, 0.7, 0.9),
                     feat_layers=(1, 9, 17, 25, 33), max_ctx=2048 + 448),
    # DeepSeek-V2-Lite-shaped MoE bf16
    "dsv2-lite": dict(_DENSE_DEFAULTS, name="dsv2-lite", cid=4, n_layers=27,
                      d_model=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                      ffn_dim=0, vocab=102400, dtype="bf16", prompt_len=256,
                      n_experts=64, top_k=6, n_shared=2, expert_ffn=1408,
                      n_dense_layers=1, dense_ffn=10944, pass_sizes=tuple(range(1, 9)),
                      max_ctx=512),
}


def config(name: str, **overrides) -> dict:
    """A copy of a named workload with optional overrides (for smaller test models)."""
    c = dict(CONFIGS[name])
    c.update(overrides)
    return c


def micro_config(n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                 ffn_dim=128, vocab=64, max_ctx=96, **kw) -> dict:
    """A very small fp32 dense model for exhaustive CPU checks."""
    c = dict(_DENSE_DEFAULTS, name="micro", cid=100, n_layers=n_layers, d_model=d_model,
             n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
             ffn_dim=ffn_dim, vocab=vocab, dtype="f32", prompt_len=8, n_new=24,
             max_ctx=max_ctx)
    c.update(kw)
    return c


def is_moe_layer(cfg: dict, layer: int) -> bool:
    return cfg["n_experts"] > 0 and layer >= cfg["n_dense_layers"]


# ---------------------------------------------------------------------------
# weight table: canonical order and shapes
# ---------------------------------------------------------------------------

def weight_specs(cfg: dict) -> list[tuple[str, tuple[int, ...], str]]:
    """(name, shape, kind) in the canonical order the C ABI expects.

    kind is "gain" (filled with ones) or "mat" (random, standard deviation 0.02).
    Matrices are row-major [out_features, in_features].
    """
    d, hd = cfg["d_model"], cfg["head_dim"]
    hq, hkv = cfg["n_q_heads"], cfg["n_kv_heads"]
    s = [("embed", (cfg["vocab"], d), "mat")]
    for l in range(cfg["n_layers"]):
        p = f"l{l}."
        s += [(p + "attn_norm", (d,), "gain"),
              (p + "wq", (hq * hd, d), "mat"),
              (p + "wk", (hkv * hd, d), "mat"),
              (p + "wv", (hkv * hd, d), "mat"),
              (p + "wo", (d, hq * hd), "mat"),
              (p + "ffn_norm", (d,), "gain")]
        if is_moe_layer(cfg, l):
            e, fe, ns = cfg["n_experts"], cfg["expert_ffn"], cfg["n_shared"]
            s += [(p + "router", (e, d), "mat"),
                  (p + "exp_gate", (e, fe, d), "mat"),
                  (p + "exp_up", (e, fe, d), "mat"),
                  (p + "exp_down", (e, d, fe), "mat"),
                  (p + "sh_gate", (ns, fe, d), "mat"),
                  (p + "sh_up", (ns, fe, d), "mat"),
                  (p + "sh_down", (ns, d, fe), "mat")]
        else:
            f = cfg["dense_ffn"] if cfg["n_experts"] > 0 else cfg["ffn_dim"]
            s += [(p + "w_gate", (f, d), "mat"),
                  (p + "w_up", (f, d), "mat"),
                  (p + "w_down", (d, f), "mat")]
    s += [("final_norm", (d,), "gain"), ("lm_head", (cfg["vocab"], d), "mat")]
    if cfg["feat_layers"]:
        s += [("fc", (d, len(cfg["feat_layers"]) * d), "mat")]
    return s


def weight_bytes(cfg: dict) -> int:
    eb = 4 if cfg["dtype"] == "f32" else 2
    return sum(int(np.prod(sh)) * eb for _, sh, _ in weight_specs(cfg))


# ---------------------------------------------------------------------------
# random draws
# ---------------------------------------------------------------------------

_CHUNK = 1 << 24  # elements per independently seeded chunk


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns uint16 bits."""
    u = a.view(np.uint32)
    r = u >> 16
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


_STD = 0.02


def _fill_chunk(flat: np.ndarray, seed: int, tid: int, chunk: int, bf16: bool, scale: float) -> None:
    c0 = chunk * _CHUNK
    c1 = min(flat.size, c0 + _CHUNK)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, chunk])))
    v = g.standard_normal(c1 - c0, dtype=np.float32)
    v *= np.float32(_STD * scale)
    flat[c0:c1] = _f32_to_bf16_bits(v) if bf16 else v


def make_weights(cfg: dict, seed: int = 0, threads: int | None = None, progress=None) -> dict[str, np.ndarray]:
    """All weights of ``cfg``: name -> float32 array (f32 configs) or uint16 bf16 bits.

    Matrices are normal with mean 0 and standard deviation 0.02, drawn in
    independently seeded chunks of 2^24 elements; norm gains are 1.  Layers
    listed in cfg["out_scale"] have both residual-writing matrices (wo and
    w_down) scaled by the given factor.  ``progress``, if
    given, is called with the finished fraction about every tenth of the work.
    """
    bf16 = cfg["dtype"] == "bf16"
    one = np.uint16(0x3F80) if bf16 else np.float32(1.0)
    out, jobs = {}, []
    for tid, (name, shape, kind) in enumerate(weight_specs(cfg)):
        if kind == "gain":
            out[name] = np.full(shape, one, dtype=np.uint16 if bf16 else np.float32)
            continue
        scale = 1.0
        if name.endswith(".wo") or name.endswith(".w_down"):
            layer = int(name[1:name.index(".")])
            scale = float(cfg["out_scale"].get(layer, 1.0))
        arr = np.empty(shape, dtype=np.uint16 if bf16 else np.float32)
        out[name] = arr
        flat = arr.reshape(-1)
        for chunk in range((flat.size + _CHUNK - 1) // _CHUNK):
            jobs.append((flat, tid, chunk, scale))
    threads = threads or min(16, os.cpu_count() or 1)
    step = max(1, len(jobs) // 10)
    with ThreadPoolExecutor(threads) as ex:
        for i, _ in enumerate(ex.map(lambda j: _fill_chunk(j[0], seed, j[1], j[2], bf16, j[3]), jobs), 1):
            if progress is not None and (i % step == 0 or i == len(jobs)):
                progress(i / len(jobs))
    return out


def make_prompt(cfg: dict, seed: int = 0, length: int | None = None) -> np.ndarray:
    """Uniform token ids over [0, vocab), int32."""
    n = cfg["prompt_len"] if length is None else length
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 10_000 + cfg["cid"]])))
    return g.integers(0, cfg["vocab"], size=n, dtype=np.int64).astype(np.int32)


def make_tokens(vocab: int, n: int, seed: int, stream: int) -> np.ndarray:
    """Uniform int32 tokens from an independent stream (test inputs)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 20_000 + stream])))
    return g.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def make_routing_trace(n_layers: int, n: int, n_experts: int, top_k: int, seed: int,
                       stream: int = 0, reuse_p: float = 0.5) -> np.ndarray:
    """Synthetic expert ids [n_layers, n, top_k] (int32) for one pass of n tokens.

    Token 0 draws top_k distinct experts uniformly.  For token t >= 1, slot j
    copies token t-1's slot-j expert with probability reuse_p (if that expert
    is not already chosen for token t); otherwise it draws uniformly from the
    experts not yet chosen for token t.  Layers are independent.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 30_000 + stream, n])))
    ids = np.zeros((n_layers, n, top_k), dtype=np.int32)
    for l in range(n_layers):
        for t in range(n):
            chosen: list[int] = []
            for j in range(top_k):
                coin = g.random()
                if t > 0 and coin < reuse_p and int(ids[l, t - 1, j]) not in chosen:
                    e = int(ids[l, t - 1, j])
                else:
                    free = [x for x in range(n_experts) if x not in chosen]
                    e = free[int(g.integers(0, len(free)))]
                chosen.append(e)
            ids[l, t] = chosen
    return ids


def make_geometric_block(true_tokens: np.ndarray, vocab: int, p: float, block: int,
                         seed: int, stream: int) -> tuple[np.ndarray, int]:
    """Draft tokens [block-1] whose correct prefix length m ~ geometric(p).

    P(m >= j) = p**j, capped at block-1.  d[0..m) = true_tokens[0..m);
    d[m] is uniform but differs from true_tokens[m]; the rest are uniform.
    Returns (drafts, m).
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 40_000 + stream])))
    k = block - 1
    m = 0
    while m < k and g.random() < p:
        m += 1
    d = g.integers(0, vocab, size=k, dtype=np.int64).astype(np.int32)
    d[:m] = true_tokens[:m]
    if m < k:
        r = int(g.integers(0, vocab - 1))
        d[m] = r if r < true_tokens[m] else r + 1
    return d, m
