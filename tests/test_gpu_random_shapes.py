"""Seeded random small bf16 shapes through the C ABI (needs an MI355X).

Each case draws a model shape (layers, width, head dim 64 or 128, 1/2/4
query heads per KV head, FFN widths that take 16- or 14-row gate/up tiles,
QKV widths that take 16- or 12-row tiles), a prompt length, a verify-block
limit and a prefill chunk.  The wide cases add 8 KV heads (the XCD-aware
attention grids), widths with 8- and 10-row residual tiles, FFN widths whose
14-row tiles do not split evenly over the compute units, a vocabulary whose
LM head groups column tiles above 8 rows, and verify blocks of up to 16 rows.
The float32 cases draw ragged widths the float32 kernels take (d_model 4-260,
FFN widths 1-513, vocabularies of 2-1000, verify blocks of 1-17 rows) and use
the float32 bound of 1e-3.  Bars as in test_gpu_parity: greedy logits within
|dlogit| <= 3e-2 of the oracle's teacher-forced logits, tokens equal wherever
the oracle's top-2 gap exceeds twice that; a verify block's rows equal to the
decode rows bit for bit; self-speculation equal to greedy for random skip
masks and draft lengths.
"""
import numpy as np
import pytest

import synth
from oracle import Model
from _common import engine
from test_gpu_parity import _gap_ok, _stepwise

pytestmark = pytest.mark.gpu

BOUND = 3e-2


def _shape(seed):
    r = np.random.default_rng(1000 + seed)
    hd = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 4]))
    hq = hkv * int(r.choice([1, 2, 4]))
    P = int(r.integers(1, 300))
    cfg = synth.config("llama-8b", n_layers=int(r.choice([2, 3, 5])), d_model=int(r.choice([256, 512, 768])),
                       n_q_heads=hq, n_kv_heads=hkv, head_dim=hd,
                       ffn_dim=int(r.choice([512, 1024, 1792, 3584])), vocab=int(r.choice([1024, 2048, 4096])),
                       prompt_len=P, max_ctx=P + 80, cid=90 + seed)
    return cfg, int(r.choice([4, 8, 17])), int(r.choice([16, 64, 256])), r


def _wide_shape(seed):
    r = np.random.default_rng(5000 + seed)
    hd = int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 4, 8]))
    hq = hkv * int(r.choice([1, 2, 4]))
    P = int(r.integers(1, 300))
    cfg = synth.config("llama-8b", n_layers=int(r.choice([2, 3])),
                       d_model=int(r.choice([256, 512, 768, 1280, 2048, 2560])),
                       n_q_heads=hq, n_kv_heads=hkv, head_dim=hd,
                       ffn_dim=int(r.choice([512, 1792, 3584, 8960, 4480])),
                       vocab=int(r.choice([2048, 4096, 16384])), prompt_len=P, max_ctx=P + 80, cid=300 + seed)
    return cfg, int(r.choice([4, 8, 12, 17])), int(r.choice([16, 64, 256])), r


def _run_shape(tag, seed, cfg, max_block, chunk, r, n_tok, max_m, bound=BOUND):
    keys = ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "prompt_len")
    print(f"[{tag} {seed}] " + " ".join(f"{k}={cfg[k]}" for k in keys) + f" max_block={max_block} chunk={chunk}",
          flush=True)
    w = synth.make_weights(cfg, seed=seed)
    eng = engine(cfg, w, max_block=max_block, prefill_chunk=chunk)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, n_tok)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = float(np.max(np.abs(rows - ref)))
        print(f"[{tag} {seed}] max |dlogit| = {err:.3e}", flush=True)
        assert err <= bound
        assert _gap_ok(toks, ref, bound) == []
        m = min(max_block, max_m)
        assert m + 1 <= len(rows)
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:m])
        assert np.array_equal(eng.read_logits(m), rows[1:m + 1])
        assert post == toks[1:m + 1]
        eng.accept()
        L = cfg["n_layers"]
        for _ in range(2):
            mask = (r.random(L) < 0.5).astype(np.uint8)
            k = int(r.integers(0 if max_block == 1 else 1, max_block))
            spec, _ = eng.generate(prompt, n_tok, mask, k)
            assert spec == toks, (mask.tolist(), k)
    finally:
        eng.close()


def _f32_shape(seed):
    r = np.random.default_rng(9000 + seed)
    hkv = int(r.choice([1, 2, 4]))
    hq = hkv * int(r.choice([1, 2, 4]))
    P = int(r.integers(1, 200))
    cfg = synth.micro_config(n_layers=int(r.choice([1, 2, 3])), d_model=int(r.choice([4, 12, 36, 100, 132, 260])),
                             n_q_heads=hq, n_kv_heads=hkv, head_dim=int(r.choice([64, 128])),
                             ffn_dim=int(r.choice([1, 3, 17, 100, 513])), vocab=int(r.choice([2, 10, 34, 258, 1000])),
                             max_ctx=P + 80, prompt_len=P, cid=500 + seed)
    return cfg, int(r.choice([1, 4, 8, 17, 32])), int(r.choice([16, 48, 256])), r


@pytest.mark.parametrize("seed", range(6))
def test_random_shape(seed):
    cfg, max_block, chunk, r = _shape(seed)
    _run_shape("shape", seed, cfg, max_block, chunk, r, 16, 8)


@pytest.mark.parametrize("seed", range(16))
def test_random_wide_shape(seed):
    cfg, max_block, chunk, r = _wide_shape(seed)
    _run_shape("wide", seed, cfg, max_block, chunk, r, 18, 16)


@pytest.mark.parametrize("seed", range(12))
def test_random_f32_shape(seed):
    """float32 models with ragged widths (d_model 4-260, FFN widths 1-513,
    vocabularies of 2-1000) at the float32 bound of 1e-3."""
    cfg, max_block, chunk, r = _f32_shape(seed)
    _run_shape("f32", seed, cfg, max_block, chunk, r, 18, 17, bound=1e-3)
