"""Seeded random feature-tap models through the C ABI (needs an MI355X).

Each case draws 1-5 tapped layers (mlx-dflash README, "Architecture": the
verifier's hidden states of chosen layers, concatenated, through one fc),
the width (including 8- and 10-row residual tiles), head grouping and head
dim, the FFN width, the vocabulary (including a grouped-tile LM head), the
verify-block limit and the prefill chunk.  One verify block after the
prompt is checked against the oracle decision by decision at every bf16
storage point, the tap concat and the fc features included
(tests/_matched.py: the same checker and derived bounds as the full-size
tests, since several layers at these widths compound ambiguous rounding
decisions beyond the plain 3e-2 bound); the same tokens run as one-row
passes reproduce the block's features and logits bit for bit.
"""
import numpy as np
import pytest

import synth
from _common import engine
from _matched import check_matched

pytestmark = pytest.mark.gpu


def _shape(seed):
    r = np.random.default_rng(11000 + seed)
    hkv = int(r.choice([1, 2, 4, 8]))
    hq = hkv * int(r.choice([1, 2, 4]))
    L = int(r.choice([2, 3, 4, 6]))
    nf = int(r.integers(1, min(L, 5) + 1))
    feats = tuple(sorted(r.choice(L, size=nf, replace=False).tolist()))
    P = int(r.integers(1, 250))
    cfg = synth.config("qwen3-8b", n_layers=L, d_model=int(r.choice([256, 512, 1280, 2560])),
                       n_q_heads=hq, n_kv_heads=hkv, head_dim=int(r.choice([64, 128])),
                       ffn_dim=int(r.choice([512, 1792, 3584])), vocab=int(r.choice([2048, 16384])),
                       prompt_len=P, max_ctx=P + 64, cid=600 + seed, feat_layers=feats)
    return cfg, int(r.choice([1, 4, 9, 17])), int(r.choice([16, 64, 256])), r


@pytest.mark.parametrize("seed", range(12))
def test_random_feature_tap_shape(seed):
    cfg, mb, chunk, r = _shape(seed)
    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "prompt_len", "feat_layers")
    print(f"[feat {seed}] " + " ".join(f"{k}={cfg[k]}" for k in keys) + f" max_block={mb} chunk={chunk}", flush=True)
    w = synth.make_weights(cfg, seed=seed)
    eng = engine(cfg, w, max_block=mb, prefill_chunk=chunk)
    try:
        prompt = synth.make_prompt(cfg)
        eng.reset()
        eng.set_trace(True)
        t = eng.prefill(prompt)
        block = [t] + list(synth.make_tokens(cfg["vocab"], mb - 1, seed=seed, stream=9))
        eng.verify(block)
        raw = eng.read_features(mb).copy()
        logits = eng.read_logits(mb)
        check_matched(f"feat {seed}", cfg, w, eng, block, len(prompt), list(range(cfg["n_layers"])), logits)
        eng.accept()
        eng.set_trace(False)
        # the same tokens as one-row passes (each verify places its token at the
        # next position, as the block did): features and logits bit for bit
        eng.reset()
        eng.prefill(prompt)
        fr, lr = [], []
        for j in range(mb):
            eng.verify([block[j]])
            fr.append(eng.read_features(1)[0].copy())
            lr.append(eng.read_logits(1)[0].copy())
            eng.accept()
        assert np.array_equal(np.stack(fr), raw)
        assert np.array_equal(np.stack(lr), logits)
    finally:
        eng.close()
