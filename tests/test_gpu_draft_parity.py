"""Draft passes and exit-state reuse vs the oracle, cycle by cycle (needs an MI355X).

LayerSkip summary 4.3.1 (self-drafting): each draft step runs one token
through the kept layers only, reading the verified cache entries and this
cycle's own draft entries of those layers, and writing its own.  The output
tokens of self-speculation do not depend on what the draft computes (the
method is lossless), so the draft is checked here on its own: the GPU and the
oracle run the same cycles in lockstep on one shared cache each, and every
draft step's logits, every verify row and every accept decision is compared.
The oracle drafts from the GPU's tokens, so a near-tie decided differently on
the two sides (top-1/top-2 gap within twice the bound) does not make them
drift apart; tokens are compared wherever the gap exceeds twice the bound.

LayerSkip summary 4.3.3 (reusing the cache): with an early-exit draft and
exit-state reuse on, the verify starts at the exit layer for the drafted
rows; its logits must follow the oracle's full verify on the same cache.

Bounds: |dlogit| <= 1e-3 for float32 models, 3e-2 for bf16 models.
"""
import numpy as np
import pytest

import synth
from oracle import Model, accept as oracle_accept
from _common import engine

pytestmark = pytest.mark.gpu


def _gap(row):
    top = np.sort(row)[-2:]
    return float(top[1] - top[0])


def _mask(L, layers):
    m = np.zeros(L, np.uint8)
    m[list(layers)] = 1
    return m


def lockstep(eng, ora, cfg, prompt, mask, ks, bound, kvq=False):
    """Runs cycles with draft lengths ks on the GPU and the oracle side by
    side.  Returns per-cycle records (k, GPU a, oracle a, near-tie flag) and
    the largest draft / verify |dlogit|.  Only the last draft step's logits
    are readable from the GPU, so varying k covers every draft position."""
    L = cfg["n_layers"]
    kept = [l for l in range(L) if not mask[l]]
    eng.set_kvq(kvq)
    eng.reset()
    t = eng.prefill(prompt)
    cache, n, last = ora.prefill(prompt)
    err_p = float(np.max(np.abs(eng.read_logits(1)[0] - last)))
    assert err_p <= bound, ("prefill", err_p)
    assert t == int(np.argmax(last)) or _gap(last) <= 2 * bound
    t_last = t
    recs, worst_d, worst_v = [], 0.0, 0.0
    try:
        for c, k in enumerate(ks):
            d = eng.draft(mask, k)
            gd = eng.read_logits(1)[0]
            tie = False
            tok, ora_d = t_last, []
            for j in range(k):
                lg = ora.forward([tok], n + j, cache, layers=kept)[0]
                ora_d.append(int(np.argmax(lg)))
                if _gap(lg) <= 2 * bound:
                    tie = True
                else:
                    assert d[j] == ora_d[-1], ("draft token", c, j)
                tok = d[j]                        # follow the GPU's draft
            err = float(np.max(np.abs(gd - lg)))
            worst_d = max(worst_d, err)
            assert err <= bound, ("draft logits", c, k, err)
            post = eng.verify(None, k + 1)
            gv = eng.read_logits(k + 1)
            ref = ora.forward([t_last] + d, n, cache)
            err = float(np.max(np.abs(gv - ref)))
            worst_v = max(worst_v, err)
            assert err <= bound, ("verify logits", c, k, err)
            ora_p = [int(np.argmax(r)) for r in ref]
            for i, r in enumerate(ref):
                if _gap(r) <= 2 * bound:
                    tie = True
                else:
                    assert post[i] == ora_p[i], ("posterior", c, i)
            a, em = eng.accept()
            assert (a, em) == oracle_accept(d, post)          # the GPU kernel on the GPU's tokens
            a_ora = oracle_accept(ora_d, ora_p)[0]             # the oracle's own decision
            if not tie:
                assert a == a_ora, ("accepted", c, a, a_ora)
            recs.append((k, a, a_ora, tie))
            n += a + 1
            t_last = em[-1]
            assert eng.context_length == n
    finally:
        eng.set_kvq(False)
    return recs, worst_d, worst_v


# ---------------------------------------------------------------------------
# float32 tiny workload
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    print("[draft-tiny] building engine", flush=True)
    eng = engine(cfg, w)
    yield cfg, w, eng, Model(cfg, w)
    eng.close()


KS = (1, 2, 3, 4, 5, 3, 2, 1, 5, 4)


@pytest.mark.parametrize("layers", [(1, 2), (3,), (0,), (2, 3), (0, 3)],
                         ids=["middle", "last", "first", "tail2", "ends"])
def test_tiny_draft_steps_match_oracle(tiny, layers):
    cfg, w, eng, ora = tiny
    prompt = synth.make_prompt(cfg)
    recs, ed, ev = lockstep(eng, ora, cfg, prompt, _mask(cfg["n_layers"], layers), KS, 1e-3)
    print(f"[draft-tiny] skip {layers}: draft |dlogit| {ed:.2e}, verify {ev:.2e}, "
          f"a {[r[1] for r in recs]}, near-tie cycles {sum(r[3] for r in recs)}", flush=True)


def test_tiny_cycle_history_equals_oracle_self_spec(tiny):
    """Fixed k: the GPU's accepted count in every cycle equals the oracle's
    free-running self-speculation, up to the first cycle with a near-tie."""
    cfg, w, eng, ora = tiny
    prompt, N, k = synth.make_prompt(cfg), cfg["n_new"], cfg["k"]
    mask = _mask(cfg["n_layers"], cfg["skip_layers"])
    out_ora, st = ora.self_spec(prompt, N, cfg["skip_layers"], k)
    n_cycles = len(st["a_hist"])
    recs, _, _ = lockstep(eng, ora, cfg, prompt, mask, [k] * n_cycles, 1e-3)
    first_tie = next((i for i, r in enumerate(recs) if r[3]), len(recs))
    got = [r[1] for r in recs]
    print(f"[draft-tiny] a_hist gpu {got}\n[draft-tiny] a_hist ora {st['a_hist']} (first near-tie: {first_tie})",
          flush=True)
    assert got[:first_tie] == st["a_hist"][:first_tie]
    assert sum(st["a_hist"]) > 0
    # and the decode loop runs the same cycles when no near-tie intervenes
    out, gst = eng.generate(prompt, N, mask, k)
    assert out == out_ora
    if first_tie == len(recs):
        assert gst["cycles"] == st["cycles"] and gst["accepted"] == st["accepted"]


def test_tiny_exit_state_reuse_matches_oracle(tiny):
    """Early-exit drafts (tail masks) with exit-state reuse on: the verify that
    starts at the exit layer gives the oracle's full-verify logits."""
    cfg, w, eng, ora = tiny
    prompt = synth.make_prompt(cfg)
    for E in (1, 2, 3):
        mask = _mask(cfg["n_layers"], range(E, cfg["n_layers"]))
        recs, ed, ev = lockstep(eng, ora, cfg, prompt, mask, KS, 1e-3, kvq=True)
        print(f"[kvq-tiny] E={E}: draft |dlogit| {ed:.2e}, verify {ev:.2e}", flush=True)


# ---------------------------------------------------------------------------
# small bf16 workload (head dim 128, 4 query heads per KV head)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small():
    cfg = synth.config("llama-8b", n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2,
                       ffn_dim=1024, vocab=2048, max_ctx=320, prompt_len=150, cid=50)
    w = synth.make_weights(cfg, seed=3)
    print("[draft-bf16] building engine", flush=True)
    eng = engine(cfg, w, max_block=17, prefill_chunk=64)
    yield cfg, w, eng, Model(cfg, w)
    eng.close()


@pytest.mark.parametrize("layers", [(1, 2), (3,), (0,)], ids=["middle", "last", "first"])
def test_small_bf16_draft_steps_match_oracle(small, layers):
    cfg, w, eng, ora = small
    prompt = synth.make_prompt(cfg)
    recs, ed, ev = lockstep(eng, ora, cfg, prompt, _mask(cfg["n_layers"], layers), KS, 3e-2)
    print(f"[draft-bf16] skip {layers}: draft |dlogit| {ed:.2e}, verify {ev:.2e}, "
          f"near-tie cycles {sum(r[3] for r in recs)}", flush=True)


def test_small_bf16_exit_state_reuse_matches_oracle(small):
    cfg, w, eng, ora = small
    prompt = synth.make_prompt(cfg)
    for E in (1, 3):
        mask = _mask(cfg["n_layers"], range(E, cfg["n_layers"]))
        recs, ed, ev = lockstep(eng, ora, cfg, prompt, mask, (1, 3, 5, 16, 2), 3e-2, kvq=True)
        print(f"[kvq-bf16] E={E}: draft |dlogit| {ed:.2e}, verify {ev:.2e}", flush=True)
