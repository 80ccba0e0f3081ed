"""The other workloads at full size (needs an MI355X): Qwen3-4B-shaped (10-row
residual tiles), Qwen3-8B-shaped (16-token verify blocks with the feature tap
and fc) and DeepSeek-V2-Lite-shaped (MoE, per-slot and deduplicated expert
reads) bf16 models with every layer and the full vocabulary.

Properties at the full size: self-speculation emits exactly plain greedy; a
verify block reproduces the decode rows bit for bit (per-slot and dedup MoE
verify blocks agree bit for bit).  Oracle parity: one verify block after the
workload's full prompt (512, 2048 and 256 tokens), every layer, checked
against the oracle decision by decision at every bf16 storage point (with the
fc features of the tap and the MoE expert activations), end to end from the
embedding to the logits (tests/_matched.py).
"""
import numpy as np
import pytest

import synth
from _common import engine

pytestmark = pytest.mark.gpu


def _matched_verify(tag, cfg, w, eng, prompt, block, routing=None, dedup=False):
    """A verify block after the workload's full prompt, all layers, checked
    against the oracle decision by decision (tests/_matched.py)."""
    from _matched import check_matched
    eng.reset()
    eng.set_trace(True)
    try:
        eng.prefill(prompt)
        if routing is not None:
            eng.set_routing(routing)
        eng.verify(block)
        logits = eng.read_logits(len(block))
        check_matched(tag, cfg, w, eng, block, len(prompt), list(range(cfg["n_layers"])), logits,
                      routing=routing, dedup=dedup)
        eng.accept()
    finally:
        if routing is not None:
            eng.set_routing(None)
        eng.set_trace(False)


def _verify_rows_equal_decode_rows(eng, prompt, m):
    eng.reset()
    t = eng.prefill(prompt)
    toks, rows = [t], []
    for _ in range(m):
        eng.verify([toks[-1]])
        rows.append(eng.read_logits(1)[0])
        toks.append(eng.accept()[1][0])
    eng.reset()
    eng.prefill(prompt)
    post = eng.verify(toks[:m])
    assert post == toks[1:m + 1]
    assert np.array_equal(eng.read_logits(m), np.stack(rows))
    eng.accept()


def _lossless(cfg, eng, prompt, n_new, frac, k):
    from self_speculative_decoding_amd import skip_mask
    base, _ = eng.generate(prompt, n_new)
    out, st = eng.generate(prompt, n_new, skip_mask(cfg["n_layers"], frac), k)
    print(f"[{cfg['name']}] skip {frac} k {k}: {st['cycles']} cycles, {st['accepted']} accepted", flush=True)
    assert out == base


@pytest.fixture(scope="module")
def qwen4b():
    cfg = synth.config("qwen3-4b")
    print("[qwen3-4b] generating weights", flush=True)
    w = synth.make_weights(cfg)
    eng = engine(cfg, w, max_block=8, prefill_chunk=256)
    print("[qwen3-4b] engine ready", flush=True)
    yield cfg, w, eng
    eng.close()


def test_qwen3_4b_fullsize(qwen4b):
    cfg, w, eng = qwen4b
    prompt = synth.make_prompt(cfg)
    _lossless(cfg, eng, prompt, 40, cfg["skip_frac"], cfg["k"])
    _verify_rows_equal_decode_rows(eng, prompt, 6)
    block = [int(t) for t in synth.make_tokens(cfg["vocab"], 4, seed=2, stream=78)]
    _matched_verify("qwen3-4b verify", cfg, w, eng, prompt, block)


@pytest.fixture(scope="module")
def qwen8b():
    cfg = synth.config("qwen3-8b")
    print("[qwen3-8b] generating weights", flush=True)
    w = synth.make_weights(cfg)
    eng = engine(cfg, w, max_block=17, prefill_chunk=256)
    print("[qwen3-8b] engine ready", flush=True)
    yield cfg, w, eng
    eng.close()


def test_qwen3_8b_fullsize_feature_tap(qwen8b):
    cfg, w, eng = qwen8b
    prompt = synth.make_prompt(cfg)
    _lossless(cfg, eng, prompt[:600], 32, 0.2, 3)
    _verify_rows_equal_decode_rows(eng, prompt[:600], 16)
    block = [int(t) for t in synth.make_tokens(cfg["vocab"], cfg["block"], seed=3, stream=79)]
    _matched_verify("qwen3-8b 16-row verify", cfg, w, eng, prompt, block)


@pytest.fixture(scope="module")
def dsv2():
    cfg = synth.config("dsv2-lite")
    print("[dsv2-lite] generating weights", flush=True)
    w = synth.make_weights(cfg)
    engs = [engine(cfg, w, max_block=9, prefill_chunk=256, moe_dedup=d) for d in (0, 1)]
    print("[dsv2-lite] engines ready (per-slot, dedup)", flush=True)
    yield cfg, w, engs
    for e in engs:
        e.close()


def test_dsv2_lite_fullsize_moe(dsv2):
    cfg, w, (ps, dd) = dsv2
    prompt = synth.make_prompt(cfg)
    _lossless(cfg, dd, prompt, 24, 0.2, 3)
    _verify_rows_equal_decode_rows(dd, prompt, 5)
    # per-slot and dedup verify blocks with the model's own router: bit for bit
    block = [int(t) for t in synth.make_tokens(cfg["vocab"], 8, seed=4, stream=80)]
    res = []
    for eng in (ps, dd):
        eng.reset()
        eng.prefill(prompt)
        eng.verify(block)
        res.append(eng.read_logits(8))
        eng.accept()
    assert np.array_equal(res[0], res[1])
    # oracle parity of an 8-row verify with an injected routing trace (dense
    # layer 0 and the 26 MoE layers, expert activations included)
    L = cfg["n_layers"]
    trace = synth.make_routing_trace(L, 8, cfg["n_experts"], cfg["top_k"], seed=4, stream=81)
    _matched_verify("dsv2-lite verify", cfg, w, dd, prompt, block, routing=trace, dedup=True)
