"""The headline Llama-3.1-8B-shaped bf16 workload at full size (needs an MI355X).

Properties at the full size: self-speculation emits exactly plain greedy over
the 1024-token prompt and 512 generated tokens; a verify block at context
1024+ reproduces the decode rows bitwise.  Oracle parity at context 1024 for
4- and 6-row verify passes and a draft step, all layers end to end, with every bf16
storage decision checked against the oracle's (tests/_matched.py); and the
whole greedy run's tokens against the plain oracle teacher-forced on them.
"""
import numpy as np
import pytest

import synth
from _common import engine
from _matched import check_matched

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def big():
    cfg = synth.config("llama-8b")
    print("[llama-8b] generating weights", flush=True)
    w = synth.make_weights(cfg)
    eng = engine(cfg, w, max_block=6, prefill_chunk=256)
    print("[llama-8b] engine ready", flush=True)
    yield cfg, w, eng
    eng.close()


def test_fullsize_self_spec_is_lossless(big):
    cfg, w, eng = big
    from self_speculative_decoding_amd import skip_mask
    prompt = synth.make_prompt(cfg)
    base, st = eng.generate(prompt, cfg["n_new"])
    print(f"[llama-8b] greedy {st['t_decode_ms']:.0f} ms", flush=True)
    for frac, k in ((0.2, 3), (0.5, 5)):
        out, st = eng.generate(prompt, cfg["n_new"], skip_mask(cfg["n_layers"], frac), k)
        print(f"[llama-8b] skip {frac} k {k}: {st['cycles']} cycles, {st['accepted']} accepted", flush=True)
        assert out == base


def test_fullsize_verify_rows_equal_decode_rows(big):
    cfg, w, eng = big
    prompt = synth.make_prompt(cfg)
    eng.reset()
    t = eng.prefill(prompt)
    toks, rows = [t], []
    for _ in range(5):
        eng.verify([toks[-1]])
        rows.append(eng.read_logits(1)[0])
        toks.append(eng.accept()[1][0])
    eng.reset()
    eng.prefill(prompt)
    post = eng.verify(toks[:5])
    assert post == toks[1:6]
    assert np.array_equal(eng.read_logits(5), np.stack(rows))
    eng.accept()


@pytest.mark.parametrize("rows", [4, 6])
def test_fullsize_verify_pass_matches_oracle_decision_by_decision(big, rows):
    """Verify pass at context 1024 (the workload's prompt), all 32 layers,
    checked end to end from the embedding against the oracle: 4 rows (k = 3)
    and 6 rows (k = 5: GEMM inputs in fragment order, two 16-query tiles per
    attention wave)."""
    cfg, w, eng = big
    prompt = synth.make_prompt(cfg)
    eng.reset()
    eng.set_trace(True)
    try:
        t = eng.prefill(prompt)
        block = [t] + [int(x) for x in synth.make_tokens(cfg["vocab"], rows - 1, seed=1, stream=77)]
        eng.verify(block)
        logits = eng.read_logits(rows)
        check_matched(f"llama-8b {rows}-row verify", cfg, w, eng, block, len(prompt), list(range(cfg["n_layers"])),
                      logits)
        eng.accept()
    finally:
        eng.set_trace(False)


def test_fullsize_draft_step_matches_oracle_decision_by_decision(big):
    """One draft step (20 % middle skip: layers 13-18 skipped) at context
    1025, checked the same way through the kept layers."""
    from self_speculative_decoding_amd import skip_mask
    cfg, w, eng = big
    prompt = synth.make_prompt(cfg)
    mask = skip_mask(cfg["n_layers"], 0.2)
    kept = [l for l in range(cfg["n_layers"]) if not mask[l]]
    eng.reset()
    eng.set_trace(True)
    try:
        t = eng.prefill(prompt)
        eng.verify([t])
        t2 = eng.accept()[1][0]
        n = eng.context_length
        d = eng.draft(mask, 1)
        logits = eng.read_logits(1)
        check_matched("llama-8b draft", cfg, w, eng, [t2], n, kept, logits)
        assert d[0] == int(np.argmax(logits[0]))
        eng.verify(None, 2)
        eng.accept()
    finally:
        eng.set_trace(False)


def test_fullsize_greedy_tokens_match_teacher_forced_oracle(big):
    """The workload end to end: GPU greedy over the 1024-token prompt and 512
    tokens against the plain oracle teacher-forced on the GPU's tokens.  The
    tokens must equal the oracle's argmax wherever its top-1/top-2 gap exceeds
    6e-2.  The logits themselves drift by the compounding of float32-vs-float64
    rounding decisions at the bf16 storage points (about 0.1 over 32 layers);
    the decision-matched tests above show that this is the whole of the
    difference (1e-6 once the decisions agree)."""
    from oracle import Model
    cfg, w, eng = big
    prompt, N = synth.make_prompt(cfg), cfg["n_new"]
    eng.reset()
    t = eng.prefill(prompt)
    toks, rows = [t], [eng.read_logits(1)[0]]
    while len(toks) < N:
        eng.verify([toks[-1]])
        rows.append(eng.read_logits(1)[0])
        toks.append(eng.accept()[1][0])
    assert eng.generate(prompt, N)[0] == toks
    print("[llama-8b] oracle teacher-forced over 1536 positions", flush=True)
    ref = Model(cfg, w).teacher_forced(prompt, toks)
    per = np.max(np.abs(np.stack(rows) - ref), axis=1)
    gaps = np.array([float(np.diff(np.sort(r)[-2:])[0]) for r in ref])
    wrong = np.array([int(np.argmax(r)) != tk for r, tk in zip(ref, toks)])
    print(f"[llama-8b] teacher-forced: max |dlogit| {per.max():.4f} (median per position {np.median(per):.4f}); "
          f"{int((gaps > 6e-2).sum())} of {N} positions with gap > 6e-2, token differs at "
          f"{int((wrong & (gaps > 6e-2)).sum())} of them; largest gap where a token differs "
          f"{float(gaps[wrong].max()) if wrong.any() else 0.0:.4f}", flush=True)
    assert not (wrong & (gaps > 6e-2)).any()
