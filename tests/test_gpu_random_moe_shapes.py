"""Seeded random small MoE shapes through the C ABI (needs an MI355X).

Each case draws routed experts (16-64), top-k (1-8), shared experts (0-2,
none as in MoE models without them), the expert FFN width (one to 22 K
chunks), dense first layers or none, the head grouping and the verify-block
limit.  With an injected routing trace (speculative decoding for MoE models,
abstract: the per-slot and deduplicated expert reads of one pass) the
per-slot and dedup passes agree bit for bit, their logits are within 3e-2
of the oracle's on the same trace and the reported union is the
brute-force one; with the router's own choice a verify block reproduces the
decode rows bit for bit on both engines and self-speculation emits greedy.
"""

import numpy as np
import pytest

import synth
from oracle import Model
from oracle.model import Cache
from _common import engine

pytestmark = pytest.mark.gpu


def _shape(seed):
    r = np.random.default_rng(7000 + seed)
    hkv = int(r.choice([1, 2, 4, 8]))
    hq = hkv * int(r.choice([1, 2, 4]))
    E = int(r.choice([16, 32, 64]))
    top_k = int(r.choice([1, 2, 4, 6, 8]))
    top_k = min(top_k, E)
    P = int(r.integers(8, 120))
    cfg = synth.config("dsv2-lite", n_layers=int(r.choice([2, 3])), d_model=int(r.choice([256, 512, 1024, 2048])),
                       n_q_heads=hq, n_kv_heads=hkv, head_dim=int(r.choice([64, 128])), vocab=int(r.choice([1024, 4096])),
                       n_experts=E, top_k=top_k, n_shared=int(r.choice([0, 1, 2])),
                       expert_ffn=int(r.choice([64, 128, 192, 1408])), n_dense_layers=int(r.choice([0, 1])),
                       dense_ffn=int(r.choice([512, 768])), max_ctx=P + 64, prompt_len=P, cid=400 + seed)
    return cfg, int(r.choice([4, 9, 17])), r


@pytest.mark.parametrize("seed", range(12))
def test_random_moe_shape(seed):
    cfg, mb, r = _shape(seed)
    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k", "n_shared",
            "expert_ffn", "n_dense_layers", "vocab", "prompt_len")
    print(f"[moe {seed}] " + " ".join(f"{k}={cfg[k]}" for k in keys) + f" max_block={mb}", flush=True)
    w = synth.make_weights(cfg, seed=seed)
    ps = engine(cfg, w, max_block=mb, prefill_chunk=64, moe_dedup=0)
    dd = engine(cfg, w, max_block=mb, prefill_chunk=64, moe_dedup=1)
    try:
        L, n = cfg["n_layers"], mb
        prompt = synth.make_prompt(cfg)
        block = list(synth.make_tokens(cfg["vocab"], n, seed=seed, stream=3))
        trace = synth.make_routing_trace(L, n, cfg["n_experts"], cfg["top_k"], seed=seed)
        res = []
        for eng in (ps, dd):
            eng.set_routing(None)
            eng.reset()
            eng.prefill(prompt)
            eng.set_routing(trace)
            eng.verify(block)
            res.append((eng.read_logits(n), eng.read_union()))
            eng.accept()
            eng.set_routing(None)
        assert np.array_equal(res[0][0], res[1][0])
        ora = Model(cfg, w)
        cache = Cache(cfg)
        ora.forward(prompt, 0, cache)          # prompt on the router's own choice
        ora.routing = {l: trace[l] for l in range(L)}
        ref = ora.forward(block, len(prompt), cache)
        err = float(np.max(np.abs(res[0][0] - ref)))
        print(f"[moe {seed}] injected: max |dlogit| = {err:.3e}", flush=True)
        assert err <= 3e-2
        for l in range(cfg["n_dense_layers"], L):
            assert res[1][1][l] == len(set(trace[l, :n].reshape(-1).tolist()))
        # router choice: verify rows == decode rows, per-slot == dedup, lossless
        toks, rows = None, None
        for eng in (ps, dd):
            eng.reset()
            t = eng.prefill(prompt)
            tk, rw = [t], [eng.read_logits(1)[0]]
            while len(tk) < n + 1:
                eng.verify([tk[-1]])
                rw.append(eng.read_logits(1)[0])
                tk.append(eng.accept()[1][0])
            if toks is None:
                toks, rows = tk, np.stack(rw)
            else:
                assert tk == toks and np.array_equal(np.stack(rw), rows)
            eng.reset()
            eng.prefill(prompt)
            post = eng.verify(toks[:n])
            assert np.array_equal(eng.read_logits(n), rows[1:n + 1]) and post == toks[1:n + 1]
            eng.accept()
            mask = (r.random(L) < 0.5).astype(np.uint8)
            k = int(r.integers(1, mb))
            base, _ = eng.generate(prompt, 12)
            spec, _ = eng.generate(prompt, 12, mask, k)
            assert spec == base, (mask.tolist(), k)
    finally:
        ps.close()
        dd.close()
