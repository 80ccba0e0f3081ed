"""Edge cases of the HIP path through the C ABI (needs an MI355X).

A bf16 model whose KV capacity is not a whole number of 64-key attention
partitions, filled to the last position; one-token prompts; the largest
verify block (32 rows); the degenerate skip masks (nothing skipped: the draft
is the full model, so every draft is accepted; everything skipped: the draft
is embedding + head); query-head groups of 1 and 2 per KV head; the largest
KV capacity the boundary accepts (8192 keys, 128 attention partitions).
Bars as in test_gpu_parity: bf16 |dlogit| <= 3e-2, GPU self-speculation
bitwise equal to GPU greedy.
"""
import numpy as np
import pytest

import synth
from oracle import Model
from _common import engine
from test_gpu_parity import _gap_ok, _stepwise

pytestmark = pytest.mark.gpu

BOUND = 3e-2


def _edge_cfg(**kw):
    base = dict(n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=2, ffn_dim=1024, vocab=2048,
                max_ctx=330, prompt_len=100, cid=70)
    base.update(kw)
    return synth.config("llama-8b", **base)


@pytest.fixture(scope="module")
def edge():
    cfg = _edge_cfg()
    w = synth.make_weights(cfg, seed=5)
    print("[edge] building engine (max_ctx 330, max_block 32)", flush=True)
    eng = engine(cfg, w, max_block=32, prefill_chunk=64)
    yield cfg, w, eng, Model(cfg, w)
    eng.close()


def test_fill_to_the_last_position(edge):
    """Greedy up to the last position a verify can reach (ragged last partition)
    matches the oracle; self-speculation filling max_ctx exactly is lossless;
    one more token is a capacity error."""
    from self_speculative_decoding_amd import SSDError, skip_mask
    cfg, w, eng, ora = edge
    prompt = synth.make_prompt(cfg)
    P, cap = len(prompt), cfg["max_ctx"]
    n = cap - P                                       # last verify row at position cap - 2
    toks, rows = _stepwise(eng, prompt, n)
    ref = ora.teacher_forced(prompt, toks)
    err = np.max(np.abs(rows - ref))
    tail = np.max(np.abs(rows[-8:] - ref[-8:]))
    print(f"[edge] max |dlogit| = {err:.3e} (last 8 rows {tail:.3e})")
    assert err <= BOUND
    assert _gap_ok(toks, ref, BOUND) == []
    k = 3
    n_full = cap - P - (k + 1)
    base, _ = eng.generate(prompt, n_full)
    spec, _ = eng.generate(prompt, n_full, skip_mask(cfg["n_layers"], 0.34), k)
    assert spec == base == toks[:n_full]
    with pytest.raises(SSDError) as e:
        eng.generate(prompt, n_full + 1, skip_mask(cfg["n_layers"], 0.34), k)
    assert e.value.status == -3


def test_one_token_prompt(edge):
    cfg, w, eng, ora = edge
    prompt = synth.make_prompt(cfg)[:1]
    toks, rows = _stepwise(eng, prompt, 24)
    ref = ora.teacher_forced(prompt, toks)
    assert np.max(np.abs(rows - ref)) <= BOUND
    assert _gap_ok(toks, ref, BOUND) == []
    mask = np.zeros(cfg["n_layers"], np.uint8)
    mask[1] = 1
    spec, _ = eng.generate(prompt, 24, mask, 4)
    assert spec == toks


def test_largest_verify_block_rows_equal_decode_rows(edge):
    """A 32-row verify (two 16-row MFMA tiles, the block limit) gives the
    logits of decoding its rows one at a time, bit for bit."""
    cfg, w, eng, _ = edge
    prompt = synth.make_prompt(cfg)
    toks, rows = _stepwise(eng, prompt, 33)
    eng.reset()
    eng.prefill(prompt)
    post = eng.verify(toks[:32])
    got = eng.read_logits(32)
    assert np.array_equal(got, rows[1:33])
    assert post == toks[1:33]
    a, em = eng.accept()
    assert a == 31 and em == toks[1:33]


def test_degenerate_masks(edge):
    """No layer skipped: the draft is the full model with the same arithmetic,
    so every draft is accepted.  Every layer skipped: the draft is embedding +
    final norm + head; the output is still the greedy sequence."""
    cfg, w, eng, _ = edge
    prompt = synth.make_prompt(cfg)
    base, _ = eng.generate(prompt, 40)
    for k in (1, 3, 8):
        out, st = eng.generate(prompt, 40, np.zeros(cfg["n_layers"], np.uint8), k)
        assert out == base, k
        assert st["accepted"] == st["drafted"] > 0, (k, st)
        out, st = eng.generate(prompt, 40, np.ones(cfg["n_layers"], np.uint8), k)
        assert out == base, k


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 8), (32, 16)])
def test_query_groups_of_one_and_two(hq, hkv):
    """The attention kernel's other head groupings (G = 1, 2) against the
    oracle; with 8 and 16 kv heads the XCD-aware grids (one and two kv heads
    per XCD slot).  A 12-row verify (two 16-query tiles per wave at G = 2)
    reproduces the decode rows bit for bit."""
    cfg = _edge_cfg(n_q_heads=hq, n_kv_heads=hkv, max_ctx=200, prompt_len=90, cid=71 + hq // hkv)
    w = synth.make_weights(cfg, seed=7)
    print(f"[edge] G = {hq // hkv}, {hkv} kv heads", flush=True)
    eng = engine(cfg, w, max_block=12, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, 32)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] G = {hq // hkv}: max |dlogit| = {err:.3e}")
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        mask = np.zeros(cfg["n_layers"], np.uint8)
        mask[1] = 1
        spec, _ = eng.generate(prompt, 32, mask, 3)
        assert spec == toks
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:12])
        assert np.array_equal(eng.read_logits(12), rows[1:13]) and post == toks[1:13]
        eng.accept()
    finally:
        eng.close()


def test_grouped_lm_head_tiles():
    """A vocabulary of 16384 (1024 column tiles): passes wider than 8 rows run
    the LM head with four column tiles per workgroup, the others one.  Greedy
    against the oracle, and a 16-row verify reproduces the one-tile decode
    rows bit for bit."""
    cfg = _edge_cfg(vocab=16384, max_ctx=200, prompt_len=90, cid=76)
    w = synth.make_weights(cfg, seed=9)
    print("[edge] vocab 16384 (grouped LM head tiles)", flush=True)
    eng = engine(cfg, w, max_block=16, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, 32)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] vocab 16384: max |dlogit| = {err:.3e}")
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:16])
        assert np.array_equal(eng.read_logits(16), rows[1:17]) and post == toks[1:17]
        eng.accept()
    finally:
        eng.close()


@pytest.mark.parametrize("ffn", [3584, 8960])
def test_narrow_gate_up_tiles(ffn):
    """FFN widths whose gate/up weight is packed in 14-row tiles against the
    oracle: 3584 = 256 tiles of 14 columns, one per compute unit (two-chunk
    load batches), and 8960 = 640 tiles, which do not split evenly over the
    compute units (one-chunk load batches); the narrow tiles keep verify rows
    bitwise equal to decode rows and self-speculation lossless."""
    cfg = _edge_cfg(ffn_dim=ffn, max_ctx=200, prompt_len=90, cid=74)
    w = synth.make_weights(cfg, seed=8)
    print(f"[edge] ffn {ffn} (14-row gate/up tiles)", flush=True)
    eng = engine(cfg, w, max_block=8, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, 33)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] ffn {ffn}: max |dlogit| = {err:.3e}")
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:8])
        assert np.array_equal(eng.read_logits(8), rows[1:9])
        assert post == toks[1:9]
        eng.accept()
        mask = np.zeros(cfg["n_layers"], np.uint8)
        mask[1] = 1
        spec, _ = eng.generate(prompt, 32, mask, 3)
        assert spec == toks[:32]
    finally:
        eng.close()


def test_narrow_residual_tiles():
    """d = 2560 (the Qwen3-4B width): the o-projection and down weights are
    packed in 10-row tiles (256 tiles, one per compute unit) and the folded
    norm's sums of squares come one per 10 columns from every producer
    (embedding, both residual GEMMs).  Against the oracle, verify rows bitwise
    equal to decode rows, self-speculation lossless."""
    cfg = _edge_cfg(n_layers=2, d_model=2560, n_q_heads=16, n_kv_heads=4, max_ctx=200, prompt_len=70, cid=75)
    w = synth.make_weights(cfg, seed=12)
    print("[edge] d 2560 (10-row residual tiles)", flush=True)
    eng = engine(cfg, w, max_block=8, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, 25)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] d 2560: max |dlogit| = {err:.3e}")
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:8])
        assert np.array_equal(eng.read_logits(8), rows[1:9])
        assert post == toks[1:9]
        eng.accept()
        mask = np.array([0, 1], np.uint8)
        spec, _ = eng.generate(prompt, 24, mask, 3)
        assert spec == toks[:24]
    finally:
        eng.close()


def test_prefill_widest_column_groups_bitwise():
    """SSD_OPT_TILE_GROUPS = 1 forces the widest grouping of the prefill tile
    kernel (four column tiles per wave for QKV, o and down, two for gate/up),
    which the default threshold only picks at very long chunks; the last-row
    logits and the KV cache equal the default grouping's bit for bit."""
    cfg = _edge_cfg(n_layers=2, d_model=1024, n_q_heads=16, n_kv_heads=4, ffn_dim=14336,
                    max_ctx=400, prompt_len=300, cid=78)
    w = synth.make_weights(cfg, seed=14)
    prompt = synth.make_prompt(cfg)
    out = []
    for groups in (0, 1):
        print(f"[edge] prefill tile groups threshold {groups}", flush=True)
        eng = engine(cfg, w, max_block=4, prefill_chunk=256)
        try:
            eng.set_tile_groups(groups)
            t = eng.prefill(prompt)
            out.append((t, eng.read_logits(1)[0], [eng.read_kv(l, 0, len(prompt)) for l in range(cfg["n_layers"])]))
        finally:
            eng.close()
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])
    for (k0, v0), (k1, v1) in zip(out[0][2], out[1][2]):
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    _, _, last = Model(cfg, w).prefill(prompt)
    assert np.max(np.abs(out[1][1] - last)) <= BOUND


def test_prefill_fallback_kernel_for_odd_k():
    """d = 576 and FFN 1600 give 9 and 25 K chunks, not a multiple of the
    tile kernel's ring unroll, so the long prefill chunks run the layer
    GEMMs on the multi-row-tile kernel instead; against the oracle, and
    self-speculation still equals greedy."""
    cfg = _edge_cfg(n_layers=2, d_model=576, n_q_heads=9, n_kv_heads=9, head_dim=64, ffn_dim=1600,
                    max_ctx=240, prompt_len=150, cid=77)
    w = synth.make_weights(cfg, seed=13)
    print("[edge] d 576, ffn 1600 (prefill fallback kernel)", flush=True)
    eng = engine(cfg, w, max_block=8, prefill_chunk=64)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, 25)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] d 576: max |dlogit| = {err:.3e}")
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        spec, _ = eng.generate(prompt, 24, np.array([1, 0], np.uint8), 3)
        assert spec == toks[:24]
    finally:
        eng.close()


def test_long_context_combine_batches():
    """A 3300-token context: 52 key partitions, so the combine loads its
    partials in two batches and the passes replay from a high context
    bucket.  Logits against the oracle; verify rows equal decode rows bit
    for bit; self-speculation lossless."""
    cfg = _edge_cfg(n_layers=2, max_ctx=3400, prompt_len=3300, cid=75)
    w = synth.make_weights(cfg, seed=10)
    print("[edge] context 3300 (52 partitions)", flush=True)
    eng = engine(cfg, w, max_block=8, prefill_chunk=256)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, 12)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] context 3300: max |dlogit| = {err:.3e}")
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:8])
        assert np.array_equal(eng.read_logits(8), rows[1:9])
        assert post == toks[1:9]
        eng.accept()
        mask = np.zeros(cfg["n_layers"], np.uint8)
        mask[1] = 1
        spec, _ = eng.generate(prompt, 12, mask, 3)
        assert spec == toks
    finally:
        eng.close()


def test_maximum_context():
    """The largest KV capacity the boundary accepts, 8192 keys = 128 attention
    partitions: every lane of the combine holds a partition and its partials
    load in three batches.  Greedy filled to the last position a verify can
    reach against the oracle; an 8-row verify block ending there equals the
    decode rows bit for bit; self-speculation filling the cache is lossless."""
    from self_speculative_decoding_amd import skip_mask
    cap = 128 * 64
    cfg = _edge_cfg(n_layers=2, max_ctx=cap, prompt_len=cap - 16, cid=79)
    w = synth.make_weights(cfg, seed=11)
    print("[edge] context 8192 (128 partitions)", flush=True)
    eng = engine(cfg, w, max_block=8, prefill_chunk=256)
    try:
        prompt = synth.make_prompt(cfg)
        P = len(prompt)
        toks, rows = _stepwise(eng, prompt, cap - P)      # last row at position cap - 2
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = np.max(np.abs(rows - ref))
        print(f"[edge] context 8192: max |dlogit| = {err:.3e}", flush=True)
        assert err <= BOUND
        assert _gap_ok(toks, ref, BOUND) == []
        eng.reset()
        eng.prefill(prompt)
        for t in toks[:7]:                                 # one-row steps to position P + 6
            eng.verify([t])
            eng.accept()
        post = eng.verify(toks[7:15])                      # rows at P + 7 .. cap - 2
        assert np.array_equal(eng.read_logits(8), rows[8:16])
        assert post == toks[8:16]
        eng.accept()
        k = 3
        n_full = cap - P - (k + 1)
        spec, _ = eng.generate(prompt, n_full, skip_mask(cfg["n_layers"], 0.5), k)
        assert spec == toks[:n_full]
    finally:
        eng.close()


def test_prefill_column_groups_bitwise_across_chunkings():
    """Long prefill chunks group column tiles per workgroup; 64-row chunks do
    not (256-row chunks here: QKV tiles in pairs in the multi-row-tile kernel,
    and the gate/up tile kernel, 14-row tiles of FFN 14336, takes two column
    tiles per wave).  The per-row arithmetic of both kernels depends neither
    on the grouping nor on the chunk, so the last-row logits and the KV cache
    agree bit for bit; the logits match the oracle."""
    cfg = _edge_cfg(n_layers=2, d_model=1024, n_q_heads=16, n_kv_heads=4, ffn_dim=14336,
                    max_ctx=700, prompt_len=640, cid=76)
    w = synth.make_weights(cfg, seed=12)
    prompt = synth.make_prompt(cfg)
    out = []
    for chunk in (256, 64):
        print(f"[edge] prefill chunk {chunk}", flush=True)
        eng = engine(cfg, w, max_block=4, prefill_chunk=chunk)
        try:
            t = eng.prefill(prompt)
            out.append((t, eng.read_logits(1)[0], [eng.read_kv(l, 0, len(prompt)) for l in range(cfg["n_layers"])]))
        finally:
            eng.close()
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])
    for (k0, v0), (k1, v1) in zip(out[0][2], out[1][2]):
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    _, _, last = Model(cfg, w).prefill(prompt)
    err = np.max(np.abs(out[0][1] - last))
    print(f"[edge] prefill 640 rows: max |dlogit| = {err:.3e}")
    assert err <= BOUND


def _bucket_shape(seed):
    r = np.random.default_rng(13000 + seed)
    hkv = int(r.choice([1, 2, 4, 8]))
    hq = hkv * int(r.choice([1, 2, 4]))
    b = int(r.choice([512, 1024]))
    P = b - int(r.integers(3, 40))              # cross the bucket boundary while decoding
    cfg = synth.config("llama-8b", n_layers=2, d_model=int(r.choice([256, 512, 1280])),
                       n_q_heads=hq, n_kv_heads=hkv, head_dim=int(r.choice([64, 128])),
                       ffn_dim=int(r.choice([512, 1792])), vocab=int(r.choice([2048, 16384])),
                       prompt_len=P, max_ctx=P + 96, cid=700 + seed, dtype=str(r.choice(["bf16", "f32"])))
    return cfg, int(r.choice([4, 9, 17])), int(r.choice([64, 256])), r


def _decode_rows(eng, prompt, n):
    eng.reset()
    t = eng.prefill(prompt)
    toks, rows = [t], [eng.read_logits(1)[0].copy()]
    while len(toks) < n:
        eng.verify([toks[-1]])
        rows.append(eng.read_logits(1)[0].copy())
        toks.append(eng.accept()[1][0])
    return toks, np.stack(rows)


@pytest.mark.parametrize("seed", range(12))
def test_graphs_across_context_buckets(seed):
    """Passes replay as HIP graphs keyed by the 512-position context bucket
    of their last row: decoding from just below a bucket boundary (512 or
    1024) across it, captured graphs, their later replays and eager
    launches give the same tokens and logits bit for bit (bf16 and float32,
    random head groupings), and so does self-speculation."""
    cfg, mb, chunk, r = _bucket_shape(seed)
    print(f"[graph {seed}] dtype={cfg['dtype']} d={cfg['d_model']} hq={cfg['n_q_heads']} hkv={cfg['n_kv_heads']} "
          f"hd={cfg['head_dim']} P={cfg['prompt_len']} max_block={mb}", flush=True)
    w = synth.make_weights(cfg, seed=seed)
    eng = engine(cfg, w, max_block=mb, prefill_chunk=chunk)
    try:
        prompt = synth.make_prompt(cfg)
        eng.set_graphs(True)
        g = _decode_rows(eng, prompt, 60)
        g2 = _decode_rows(eng, prompt, 60)          # replays of graphs captured in the first run
        eng.set_graphs(False)
        e = _decode_rows(eng, prompt, 60)
        assert g[0] == e[0] == g2[0]
        assert np.array_equal(g[1], e[1]) and np.array_equal(g2[1], e[1])
        mask = (r.random(cfg["n_layers"]) < 0.5).astype(np.uint8)
        k = int(r.integers(1, mb))
        eng.set_graphs(True)
        sg, _ = eng.generate(prompt, 60, mask, k)
        eng.set_graphs(False)
        se, _ = eng.generate(prompt, 60, mask, k)
        assert sg == se == g[0]
    finally:
        eng.close()


def _prefill_shape(seed):
    r = np.random.default_rng(15000 + seed)
    hkv = int(r.choice([1, 2, 4, 8]))
    hq = hkv * int(r.choice([1, 2, 4]))
    P = int(r.integers(33, 900))
    cfg = synth.config("llama-8b", n_layers=2, d_model=int(r.choice([256, 512, 1024, 1280, 2560])),
                       n_q_heads=hq, n_kv_heads=hkv, head_dim=int(r.choice([64, 128])),
                       ffn_dim=int(r.choice([512, 1792, 3584, 4480, 8960])), vocab=int(r.choice([2048, 16384])),
                       prompt_len=P, max_ctx=P + 16, cid=800 + seed)
    chunks = sorted(set(int(c) for c in r.choice([48, 64, 96, 128, 160, 256], size=2, replace=False)))
    return cfg, chunks


@pytest.mark.parametrize("seed", range(16))
def test_prefill_random_shapes_and_chunkings(seed):
    """Prompts of 33-900 tokens prefilled in chunks of 48-256 rows over random
    widths, head groupings, FFN widths and vocabularies: the last row's
    logits against the oracle; where every chunk of both chunkings is wider
    than 32 rows (the multi-row-tile and prefill tile kernels, whose per-row
    arithmetic depends on neither the chunk nor the tile grouping), the KV
    cache and the logits bit for bit across the chunkings.  A tail of 32
    rows or fewer runs the decode kernels, equal to rounding only."""
    cfg, chunks = _prefill_shape(seed)
    print(f"[prefill {seed}] d={cfg['d_model']} hq={cfg['n_q_heads']} hkv={cfg['n_kv_heads']} hd={cfg['head_dim']} "
          f"F={cfg['ffn_dim']} V={cfg['vocab']} P={cfg['prompt_len']} chunks={chunks}", flush=True)
    w = synth.make_weights(cfg, seed=seed)
    prompt = synth.make_prompt(cfg)
    out = []
    for chunk in chunks:
        eng = engine(cfg, w, max_block=4, prefill_chunk=chunk)
        try:
            t = eng.prefill(prompt)
            out.append((t, eng.read_logits(1)[0].copy(),
                        [eng.read_kv(l, 0, len(prompt)) for l in range(cfg["n_layers"])]))
        finally:
            eng.close()
    P = len(prompt)
    wide = [(P - 1) % c + 1 > 32 for c in chunks]    # every chunk of the chunking wider than 32 rows
    print(f"[prefill {seed}] tails {[(P - 1) % c + 1 for c in chunks]}", flush=True)
    _, _, last = Model(cfg, w).prefill(prompt)
    for o in out:
        err = float(np.max(np.abs(o[1] - last)))
        print(f"[prefill {seed}] max |dlogit| = {err:.3e}", flush=True)
        assert err <= 3e-2
    if not all(wide):
        return
    for o in out[1:]:
        assert o[0] == out[0][0]
        assert np.array_equal(o[1], out[0][1])
        for (k0, v0), (k1, v1) in zip(out[0][2], o[2]):
            assert np.array_equal(k0, k1) and np.array_equal(v0, v1)


def _long_shape(seed):
    r = np.random.default_rng(17000 + seed)
    hkv = int(r.choice([1, 2, 4, 8]))
    hq = min(16, hkv * int(r.choice([1, 2, 4])))
    P = int(r.integers(2000, 8100))
    cfg = synth.config("llama-8b", n_layers=2, d_model=int(r.choice([256, 512])), n_q_heads=hq, n_kv_heads=hkv,
                       head_dim=int(r.choice([64, 128])), ffn_dim=512, vocab=2048,
                       prompt_len=P, max_ctx=min(8192, P + 40), cid=900 + seed)
    return cfg, int(r.choice([4, 9, 17])), r


@pytest.mark.parametrize("seed", range(10))
def test_long_context_random_shapes(seed):
    """Contexts of 2000-8100 positions (up to 127 attention partitions, the
    combine's second load batch, the XCD-aware grids with 8 kv heads) over
    random head groupings: greedy against the oracle, and a verify block
    equal to the decode rows bit for bit."""
    cfg, mb, r = _long_shape(seed)
    n = min(18, cfg["max_ctx"] - cfg["prompt_len"] - 1)
    print(f"[edge long {seed}] hq={cfg['n_q_heads']} hkv={cfg['n_kv_heads']} hd={cfg['head_dim']} d={cfg['d_model']} "
          f"P={cfg['prompt_len']} max_ctx={cfg['max_ctx']} max_block={mb} n={n}", flush=True)
    w = synth.make_weights(cfg, seed=seed)
    eng = engine(cfg, w, max_block=mb, prefill_chunk=256)
    try:
        prompt = synth.make_prompt(cfg)
        toks, rows = _stepwise(eng, prompt, n)
        ref = Model(cfg, w).teacher_forced(prompt, toks)
        err = float(np.max(np.abs(rows - ref)))
        print(f"[edge long {seed}] max |dlogit| = {err:.3e}", flush=True)
        assert err <= 3e-2
        assert _gap_ok(toks, ref, 3e-2) == []
        m = min(mb, n - 1)
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(toks[:m])
        assert np.array_equal(eng.read_logits(m), rows[1:m + 1]) and post == toks[1:m + 1]
        eng.accept()
    finally:
        eng.close()


@pytest.mark.parametrize("kind,seed", [("tiny", 0), ("tiny", 1), ("bf16", 0), ("bf16", 1)])
def test_random_call_sequences_follow_the_state_machine(kind, seed):
    """400 random calls (prefill, draft, verify of the drafts, verify of a host
    block, accept, reset) on a float32 and a bf16 model: each call succeeds
    exactly when ssd_check_transition allows it and leaves the documented
    state; a refused call returns SSD_E_STATE and changes neither the state
    nor the context length; an accept of a drafts advances the committed
    length by a + 1."""
    import self_speculative_decoding_amd as S
    from self_speculative_decoding_amd import SSDError
    if kind == "tiny":
        cfg = synth.config("tiny", max_ctx=400)
    else:
        cfg = synth.config("llama-8b", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=2, ffn_dim=1024,
                           vocab=2048, max_ctx=400, prompt_len=60, cid=950)
    mb = 6
    w = synth.make_weights(cfg, seed=seed)
    eng = engine(cfg, w, max_block=mb, prefill_chunk=64)
    r = np.random.default_rng(seed)
    L, V = cfg["n_layers"], cfg["vocab"]
    try:
        eng.reset()
        n_drafted = 0
        counts = {}
        for step in range(400):
            st, n = eng.state, eng.context_length
            op = str(r.choice(["prefill", "draft", "verify", "block", "accept", "reset"],
                              p=[0.12, 0.22, 0.18, 0.18, 0.22, 0.08]))
            code = {"prefill": S.OP_PREFILL, "draft": S.OP_DRAFT, "verify": S.OP_VERIFY,
                    "block": S.OP_VERIFY_BLOCK, "accept": S.OP_ACCEPT, "reset": S.OP_RESET}[op]
            want = S.check_transition(st, code)
            try:
                if op == "prefill":
                    P = int(r.integers(1, 80))
                    eng.prefill(list(synth.make_tokens(V, P, seed=seed, stream=step)))
                    got_n = P
                elif op == "draft":
                    k = int(r.integers(1, mb))
                    mask = (r.random(L) < 0.5).astype(np.uint8)
                    d = eng.draft(mask, k)
                    assert len(d) == k and all(0 <= x < V for x in d)
                    n_drafted = k
                    got_n = n
                elif op == "verify":
                    post = eng.verify(None, n_drafted + 1)
                    assert len(post) == n_drafted + 1
                    got_n = n
                elif op == "block":
                    m = int(r.integers(1, mb + 1))
                    post = eng.verify(list(synth.make_tokens(V, m, seed=seed, stream=1000 + step)))
                    assert len(post) == m
                    n_drafted = m - 1
                    got_n = n
                elif op == "accept":
                    a, em = eng.accept()
                    assert 0 <= a <= n_drafted and len(em) == a + 1
                    got_n = n + a + 1
                else:
                    eng.reset()
                    got_n = 0
                ok = True
            except SSDError as e:
                ok = False
                status = e.status
            if want >= 0:
                if not ok and status == -3:      # capacity: the state stays
                    assert eng.state == st and eng.context_length == n
                    counts["capacity"] = counts.get("capacity", 0) + 1
                    continue
                assert ok, (step, op, st, want, status)
                assert eng.state == want, (step, op, st, want, eng.state)
                if op != "reset":
                    assert eng.context_length == got_n, (step, op, n, got_n, eng.context_length)
                counts[op] = counts.get(op, 0) + 1
            else:
                assert not ok and status == want, (step, op, st, want, ok)
                assert eng.state == st and eng.context_length == n, (step, op)
                counts["refused"] = counts.get("refused", 0) + 1
        print(f"[edge fsm {kind} {seed}] {counts}", flush=True)
    finally:
        eng.close()
