"""HIP path vs the oracle, through the C ABI (needs an MI355X).

Bars: float32 workloads |dlogit| <= 1e-3, bf16 workloads <= 3e-2; tokens equal
wherever the oracle's top-1/top-2 gap exceeds twice that bound; GPU
self-speculation bitwise equal to GPU plain greedy at every mask and k.
"""
import itertools

import numpy as np
import pytest

import synth
from oracle import Model, accept as oracle_accept
from _common import engine

pytestmark = pytest.mark.gpu


def _gap_ok(gpu_tokens, ora_rows, bound):
    """Tokens must equal the oracle argmax where its top-1/top-2 gap > 2*bound."""
    bad = []
    for t, row in enumerate(ora_rows):
        top = np.sort(row)[-2:]
        if top[1] - top[0] > 2 * bound and int(np.argmax(row)) != gpu_tokens[t]:
            bad.append(t)
    return bad


def _stepwise(eng, prompt, n_new):
    """Plain greedy through prefill + verify([t]) + accept, with each step's logits."""
    eng.reset()
    t = eng.prefill(prompt)
    toks, rows = [t], [eng.read_logits(1)[0]]
    while len(toks) < n_new:
        eng.verify([toks[-1]])
        rows.append(eng.read_logits(1)[0])
        a, em = eng.accept()
        assert a == 0 and len(em) == 1
        toks.append(em[0])
    return toks, np.stack(rows)


# ---------------------------------------------------------------------------
# tiny float32 workload
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    print(f"[tiny] building engine", flush=True)
    eng = engine(cfg, w)
    yield cfg, w, eng, Model(cfg, w)
    eng.close()


def test_accept_kernel_exhaustive_v3(tiny):
    eng = tiny[2]
    for k in range(0, 5):
        for d in itertools.product(range(3), repeat=k):
            for p in itertools.product(range(3), repeat=k + 1):
                assert eng.test_accept(d, p) == oracle_accept(d, p)[0], (d, p)


def test_accept_kernel_long_blocks(tiny):
    eng = tiny[2]
    g = np.random.default_rng(0)
    for k in (8, 15, 16, 31):
        for a in range(k + 1):
            p = g.integers(0, 100, k + 1)
            d = p[:k].copy()
            if a < k:
                d[a] = (d[a] + 1) % 100
            assert eng.test_accept(d, p) == a


def test_tiny_prefill_logits(tiny):
    cfg, w, eng, ora = tiny
    prompt = synth.make_prompt(cfg)
    eng.reset()
    eng.prefill(prompt)
    gl = eng.read_logits(1)[0]
    _, _, last = ora.prefill(prompt)
    assert np.max(np.abs(gl - last)) <= 1e-3


def test_tiny_greedy_matches_oracle(tiny):
    cfg, w, eng, ora = tiny
    prompt, N = synth.make_prompt(cfg), cfg["n_new"]
    toks, rows = _stepwise(eng, prompt, N)
    ref = ora.teacher_forced(prompt, toks)
    err = np.max(np.abs(rows - ref))
    print(f"[tiny] max |dlogit| = {err:.3e}")
    assert err <= 1e-3
    assert _gap_ok(toks, ref, 1e-3) == []
    # the oracle's own free-running greedy gives the same tokens outright
    assert ora.greedy(prompt, N)[0] == toks
    # the sync-free decode loop emits the same tokens
    out, st = eng.generate(prompt, N)
    assert out == toks and st["cycles"] == N - 1


def test_tiny_self_spec_matches_greedy_and_oracle(tiny):
    cfg, w, eng, ora = tiny
    prompt, N = synth.make_prompt(cfg), cfg["n_new"]
    mask = np.zeros(cfg["n_layers"], np.uint8)
    mask[list(cfg["skip_layers"])] = 1
    base, _ = eng.generate(prompt, N)
    out, st = eng.generate(prompt, N, mask, cfg["k"])
    assert out == base
    ref, ost = ora.self_spec(prompt, N, cfg["skip_layers"], cfg["k"])
    assert out == ref
    print(f"[tiny] cycles gpu {st['cycles']} oracle {ost['cycles']}, accepted {st['accepted']} / {ost['accepted']}")
    assert st["accepted"] > 0
    # the cycle-by-cycle history against the oracle: test_gpu_draft_parity.py


def test_tiny_every_mask_and_k_is_lossless(tiny):
    cfg, w, eng, _ = tiny
    prompt, N = synth.make_prompt(cfg), 40
    base, _ = eng.generate(prompt, N)
    for bits in itertools.product([0, 1], repeat=cfg["n_layers"]):
        for k in (1, 2, 3, 5, 8):
            out, _ = eng.generate(prompt, N, np.array(bits, np.uint8), k)
            assert out == base, (bits, k)


def test_tiny_stepwise_cycle_matches_oracle_cycle(tiny):
    cfg, w, eng, ora = tiny
    prompt = synth.make_prompt(cfg)
    mask = np.zeros(cfg["n_layers"], np.uint8)
    mask[[1, 2]] = 1
    eng.reset()
    t = eng.prefill(prompt)
    d = eng.draft(mask, 3)
    p = eng.verify(None, 4)
    a, em = eng.accept()
    assert (a, em) == oracle_accept(d, p)
    assert eng.context_length == len(prompt) + a + 1
    # the verify rows are the full model's greedy predictions: compare with the oracle
    ref = ora.forward(list(prompt) + [t] + d, 0, __import__("oracle").model.Cache(cfg))[len(prompt):]
    assert np.max(np.abs(eng.read_logits(4) - ref)) <= 1e-3


def test_state_errors_on_gpu(tiny):
    from self_speculative_decoding_amd import SSDError
    cfg, w, eng, _ = tiny
    eng.reset()
    with pytest.raises(SSDError) as e:
        eng.draft(None, 2)                       # before prefill
    assert e.value.status == -2
    eng.prefill(synth.make_prompt(cfg))
    with pytest.raises(SSDError) as e:
        eng.accept()                             # nothing verified
    assert e.value.status == -2
    with pytest.raises(SSDError) as e:
        eng.verify([cfg["vocab"]])               # token out of range
    assert e.value.status == -1
    with pytest.raises(SSDError) as e:
        eng.generate(synth.make_prompt(cfg), 8, greedy=0)     # sampling never configured
    assert e.value.status == -2
    with pytest.raises(SSDError) as e:
        eng.generate(synth.make_prompt(cfg), 8, greedy=2)
    assert e.value.status == -5
    with pytest.raises(SSDError) as e:
        eng.generate(synth.make_prompt(cfg), cfg["max_ctx"])
    assert e.value.status == -3


def test_smallest_requests_on_gpu(tiny):
    """The degenerate request sizes: an empty prompt and zero new tokens are
    argument errors; one new token is the prefill's token alone, with or
    without a draft; two tokens with k = 3 stop inside the first cycle and
    the output is the greedy prefix (the last cycle's overshoot is cut)."""
    from self_speculative_decoding_amd import SSDError, skip_mask
    cfg, w, eng, _ = tiny
    prompt = synth.make_prompt(cfg)
    eng.reset()
    with pytest.raises(SSDError) as e:
        eng.prefill([])
    assert e.value.status == -1
    with pytest.raises(SSDError) as e:
        eng.generate(prompt, 0)
    assert e.value.status == -1
    base, _ = eng.generate(prompt, 8)
    mask = skip_mask(cfg["n_layers"], 0.5)
    assert eng.generate(prompt, 1)[0] == base[:1]
    assert eng.generate(prompt, 1, mask, 3)[0] == base[:1]
    assert eng.generate(prompt, 2, mask, 3)[0] == base[:2]
    assert eng.generate(prompt, 8, mask, 3)[0] == base


# ---------------------------------------------------------------------------
# small bf16 workload with the real head geometry (hd 128, 4 q heads per KV head)
# ---------------------------------------------------------------------------

def _small_bf16():
    return synth.config("llama-8b", n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2,
                        ffn_dim=1024, vocab=2048, max_ctx=320, prompt_len=150, cid=50)


@pytest.fixture(scope="module")
def small():
    cfg = _small_bf16()
    w = synth.make_weights(cfg, seed=3)
    # make layers 1-2 weak so the skip draft is often right
    print(f"[small-bf16] building engine", flush=True)
    eng = engine(cfg, w, max_block=17, prefill_chunk=64)
    yield cfg, w, eng, Model(cfg, w)
    eng.close()


def test_small_bf16_greedy_matches_oracle(small):
    cfg, w, eng, ora = small
    prompt, N = synth.make_prompt(cfg), 48
    toks, rows = _stepwise(eng, prompt, N)
    ref = ora.teacher_forced(prompt, toks)
    err = np.max(np.abs(rows - ref))
    print(f"[small-bf16] max |dlogit| = {err:.3e}")
    assert err <= 3e-2
    assert _gap_ok(toks, ref, 3e-2) == []
    out, _ = eng.generate(prompt, N)
    assert out == toks


def test_small_bf16_self_spec_lossless(small):
    cfg, w, eng, _ = small
    prompt, N = synth.make_prompt(cfg), 64
    base, _ = eng.generate(prompt, N)
    for frac in (0.25, 0.5):
        from self_speculative_decoding_amd import skip_mask
        mask = skip_mask(cfg["n_layers"], frac)
        for k in (1, 2, 3, 5, 7, 16):
            out, st = eng.generate(prompt, N, mask, k)
            assert out == base, (frac, k)


def test_small_bf16_verify_rows_bitwise_equal_decode_rows(small):
    """A block verified in one pass gives the exact logits of decoding it row by row."""
    cfg, w, eng, _ = small
    prompt = synth.make_prompt(cfg)
    toks, rows = _stepwise(eng, prompt, 18)
    for m in (2, 5, 16, 17):
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:m])
        got = eng.read_logits(m)
        assert np.array_equal(got, rows[1:m + 1]), m
        assert post == toks[1:m + 1]
        eng.accept()


def test_small_bf16_prefill_chunking_invariant(small):
    cfg, w, eng, ora = small
    prompt = synth.make_prompt(cfg)
    eng.reset()
    t = eng.prefill(prompt)
    gl = eng.read_logits(1)[0]
    _, _, last = ora.prefill(prompt)
    assert np.max(np.abs(gl - last)) <= 3e-2
    assert t == int(np.argmax(gl))


def test_small_bf16_graph_replays_match_eager(small):
    """Captured passes replayed many times (with eager prefill work and host
    synchronisation between replays) give exactly the eager results."""
    from self_speculative_decoding_amd import skip_mask
    cfg, w, eng, _ = small
    prompt, N = synth.make_prompt(cfg), 40
    mask = skip_mask(cfg["n_layers"], 0.5)
    try:
        eng.set_graphs(False)
        base_e, _ = eng.generate(prompt, N)
        spec_e, _ = eng.generate(prompt, N, mask, 3)
        toks_e, rows_e = _stepwise(eng, prompt, 12)
        eng.set_graphs(True)
        for rep in range(3):
            base_g, _ = eng.generate(prompt, N)
            spec_g, _ = eng.generate(prompt, N, mask, 3)
            toks_g, rows_g = _stepwise(eng, prompt, 12)
            assert base_g == base_e and spec_g == spec_e, rep
            assert toks_g == toks_e and np.array_equal(rows_g, rows_e), rep
    finally:
        eng.set_graphs(True)


def test_tiny_graph_and_eager_agree(tiny):
    cfg, w, eng, _ = tiny
    prompt = synth.make_prompt(cfg)
    mask = np.zeros(cfg["n_layers"], np.uint8)
    mask[[1, 2]] = 1
    try:
        eng.set_graphs(False)
        e1, s1 = eng.generate(prompt, 48, mask, 3)
        eng.set_graphs(True)
        g1, s2 = eng.generate(prompt, 48, mask, 3)
        g2, _ = eng.generate(prompt, 48, mask, 3)
        assert e1 == g1 == g2 and s1["accepted"] == s2["accepted"]
    finally:
        eng.set_graphs(True)


# ---------------------------------------------------------------------------
# feature tap + fc, and geometric-prefix verify blocks
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def feat():
    cfg = synth.config("qwen3-8b", n_layers=4, d_model=512, n_q_heads=8, n_kv_heads=2,
                       ffn_dim=1024, vocab=2048, max_ctx=400, prompt_len=200, cid=51,
                       feat_layers=(1, 3))
    w = synth.make_weights(cfg, seed=4)
    print("[feat] building engine", flush=True)
    eng = engine(cfg, w, max_block=17, prefill_chunk=128)
    yield cfg, w, eng, Model(cfg, w)
    eng.close()


def test_feature_tap_matches_oracle(feat):
    from _common import bf16_bits_to_f32
    from oracle.model import Cache
    cfg, w, eng, ora = feat
    prompt = synth.make_prompt(cfg)
    eng.reset()
    t = eng.prefill(prompt)
    block = [t] + list(synth.make_tokens(cfg["vocab"], 15, seed=4, stream=9))
    eng.verify(block)
    got = bf16_bits_to_f32(eng.read_features(16))
    cache = Cache(cfg)
    ora.forward(prompt, 0, cache)
    lg = ora.forward(block, len(prompt), cache)
    ref = ora.features
    err = np.max(np.abs(got - ref))
    print(f"[feat] max |dfeature| = {err:.3e} (scale {np.max(np.abs(ref)):.2f})")
    assert err <= 3e-2 * max(1.0, float(np.max(np.abs(ref))))
    assert np.max(np.abs(eng.read_logits(16) - lg)) <= 3e-2
    eng.accept()


def test_geometric_blocks_accept_exactly_the_correct_prefix(feat):
    cfg, w, eng, _ = feat
    prompt = synth.make_prompt(cfg)
    true, _ = eng.generate(prompt, 120)          # the target's own greedy continuation
    eng.reset()
    t = eng.prefill(prompt)
    assert t == true[0]
    pos = 0
    for s in range(12):
        rest = np.array(true[pos + 1:pos + 16], dtype=np.int32)
        if len(rest) < 15:
            break
        d, m = synth.make_geometric_block(rest, cfg["vocab"], 0.7, 16, seed=4, stream=s)
        post = eng.verify([true[pos]] + list(d))
        a, em = eng.accept()
        assert a == m, (s, a, m)
        assert em == list(true[pos + 1:pos + a + 2])
        pos += a + 1
        assert eng.context_length == len(prompt) + pos
