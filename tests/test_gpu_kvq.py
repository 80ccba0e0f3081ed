"""Exit-state reuse of an early-exit draft (SSD_OPT_KVQ) through the C ABI
(needs an MI355X).

LayerSkip summary 4.3.3: with a draft that runs the first E layers, the
verify reuses the draft's KV entries of layers < E and the state at the exit
layer, so it starts at layer E for the drafted rows.  Every row's arithmetic
is independent of the pass width, so the reused verify must give the full
verify's posterior and logits bit for bit, and self-speculation stays the
greedy sequence.  Models: bf16 dense (4 layers), bf16 MoE (dense layer 0,
MoE layers 1-2), float32 tiny.
"""
import numpy as np
import pytest

import synth
from _common import engine
from test_gpu_moe import _cfg as _moe_cfg

pytestmark = pytest.mark.gpu


def _tail(L, E):
    m = np.zeros(L, np.uint8)
    m[E:] = 1
    return m


def _cycle(eng, prompt, mask, k, kvq):
    eng.set_kvq(kvq)
    eng.reset()
    eng.prefill(prompt)
    d = eng.draft(mask, k)
    post = eng.verify(None, k + 1)
    logits = eng.read_logits(k + 1)
    a, em = eng.accept()
    return d, post, logits, a, em


def _check_model(cfg, eng, Es, ks, N=40):
    prompt = synth.make_prompt(cfg)
    L = cfg["n_layers"]
    eng.set_kvq(False)
    base, _ = eng.generate(prompt, N)
    for E in Es:
        mask = _tail(L, E)
        for k in ks:
            full = _cycle(eng, prompt, mask, k, False)
            reuse = _cycle(eng, prompt, mask, k, True)
            assert full[0] == reuse[0] and full[1] == reuse[1], (E, k)
            assert np.array_equal(full[2], reuse[2]), (E, k)
            assert full[3:] == reuse[3:], (E, k)
            eng.set_kvq(True)
            out, st_on = eng.generate(prompt, N, mask, k)
            eng.set_kvq(False)
            out_off, st_off = eng.generate(prompt, N, mask, k)
            assert out == out_off == base, (E, k)
            assert st_on["accepted"] == st_off["accepted"], (E, k)
    eng.set_kvq(False)


def test_kvq_bf16_dense_bitwise_equal_full_verify():
    cfg = synth.config("llama-8b", n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2, ffn_dim=1024,
                       vocab=2048, max_ctx=320, prompt_len=150, cid=80)
    w = synth.make_weights(cfg, seed=9)
    print("[kvq] bf16 dense", flush=True)
    eng = engine(cfg, w, max_block=17, prefill_chunk=64)
    try:
        _check_model(cfg, eng, Es=(1, 2, 3), ks=(1, 3, 5, 16))
    finally:
        eng.close()


def test_kvq_bf16_moe_bitwise_equal_full_verify():
    cfg = _moe_cfg()
    w = synth.make_weights(cfg, seed=6)
    print("[kvq] bf16 MoE", flush=True)
    eng = engine(cfg, w, max_block=9, prefill_chunk=64, moe_dedup=1)
    try:
        _check_model(cfg, eng, Es=(1, 2), ks=(2, 4))
    finally:
        eng.close()


def test_kvq_f32_tiny_bitwise_equal_full_verify():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    print("[kvq] f32 tiny", flush=True)
    eng = engine(cfg, w)
    try:
        _check_model(cfg, eng, Es=(1, 3), ks=(1, 3))
    finally:
        eng.close()


def test_kvq_other_masks_and_host_blocks_verify_in_full():
    """A middle-skip mask is not an early exit: with the option on, drafting and
    verifying give the plain results.  A host block after a draft replaces the
    drafted tokens, so its verify must not reuse their exit states."""
    cfg = synth.config("llama-8b", n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2, ffn_dim=1024,
                       vocab=2048, max_ctx=320, prompt_len=150, cid=80)
    w = synth.make_weights(cfg, seed=9)
    eng = engine(cfg, w, max_block=17, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        mid = np.array([0, 1, 1, 0], np.uint8)
        full = _cycle(eng, prompt, mid, 3, False)
        reuse = _cycle(eng, prompt, mid, 3, True)
        assert full[1] == reuse[1] and np.array_equal(full[2], reuse[2])
        # host block after an early-exit draft
        toks, _ = eng.generate(prompt, 6)
        out = []
        for kvq in (False, True):
            eng.set_kvq(kvq)
            eng.reset()
            eng.prefill(prompt)
            eng.draft(_tail(4, 2), 3)
            post = eng.verify(toks[:4])
            out.append((post, eng.read_logits(4)))
            eng.accept()
        assert out[0][0] == out[1][0] == toks[1:5]
        assert np.array_equal(out[0][1], out[1][1])
    finally:
        eng.set_kvq(False)
        eng.close()


def _random_shape(kind, seed):
    from test_gpu_random_moe_shapes import _shape as moe_shape
    from test_gpu_random_shapes import _f32_shape, _wide_shape
    if kind == "moe":
        cfg, mb, _ = moe_shape(seed)
        return cfg, mb, dict(prefill_chunk=64, moe_dedup=seed % 2)
    cfg, mb, chunk, _ = (_wide_shape if kind == "wide" else _f32_shape)(seed)
    return cfg, mb, dict(prefill_chunk=chunk)


@pytest.mark.parametrize("kind,seed", [("wide", s) for s in range(6)] + [("f32", s) for s in (1, 5, 7, 8)] +
                         [("moe", s) for s in (0, 2, 3, 4)])
def test_kvq_random_shapes_bitwise_equal_full_verify(kind, seed):
    """Exit-state reuse on the random shapes of the other GPU tests (bf16
    wide, float32 ragged, MoE per-slot and dedup): every exit layer E and
    draft lengths 1 to max_block-1, bitwise equal to the full verify."""
    cfg, mb, kw = _random_shape(kind, seed)
    if cfg["n_layers"] < 2 or mb < 2:
        pytest.skip("needs two layers and room for a draft")
    w = synth.make_weights(cfg, seed=seed)
    eng = engine(cfg, w, max_block=mb, **kw)
    try:
        _check_model(cfg, eng, range(1, cfg["n_layers"]), sorted({1, min(3, mb - 1), mb - 1}), N=20)
    finally:
        eng.close()
