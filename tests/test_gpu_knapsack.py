"""Knapsack skip-set search inputs through the C ABI (needs an MI355X): the
per-layer cosine proxy computed by the library from a full pass's residual
trace, against the oracle's definition on the same trace and against the
oracle decoder's own residuals; and a knapsack-chosen mask stays lossless."""
import numpy as np
import pytest

import synth
from oracle import Model, layer_cosines
from oracle.model import Cache
from _common import engine, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def test_layer_cosines_match_oracle_and_knapsack_mask_is_lossless():
    from self_speculative_decoding_amd import knapsack_skip
    cfg = synth.config("llama-8b", n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2, ffn_dim=1024,
                       vocab=2048, max_ctx=320, prompt_len=150, cid=80)
    w = synth.make_weights(cfg, seed=9)
    eng = engine(cfg, w, max_block=17, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        toks, _ = eng.generate(prompt, 10)
        eng.set_trace(True)
        eng.reset()
        eng.prefill(prompt)
        block = toks[:8]
        eng.verify(block)
        cos = eng.layer_cosines(8)
        trace = eng.read_trace(8).reshape(cfg["n_layers"], 8, cfg["d_model"])
        emb = bf16_bits_to_f32(w["embed"][np.array(block)]).astype(np.float64)
        # the library's arithmetic on its own trace
        np.testing.assert_allclose(cos, layer_cosines(emb, list(trace)), rtol=0, atol=1e-9)
        # against the oracle decoder's residuals
        ora = Model(cfg, w)
        cache, n, _ = ora.prefill(prompt)
        x = ora.embed(block)
        res = []
        for l in range(cfg["n_layers"]):
            x = ora.layer(l, x, n, cache)
            res.append(x)
        ref = layer_cosines(ora.embed(block), res)
        print(f"[knapsack] cos gpu {np.round(cos, 5)} oracle {np.round(ref, 5)}")
        assert np.max(np.abs(cos - ref)) <= 2e-3
        # a knapsack mask (uniform costs, keep 3 of 4) drives a lossless decode
        mask, _ = knapsack_skip(np.ones(4, np.int32), 1.0 - cos, 3)
        assert int(mask.sum()) == 1
        eng.set_trace(False)
        base, _ = eng.generate(prompt, 40)
        spec, _ = eng.generate(prompt, 40, mask, 3)
        assert spec == base
    finally:
        eng.close()
