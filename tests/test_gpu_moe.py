"""MoE verify pass through the C ABI vs the oracle (needs an MI355X).

Per-slot and deduplicated expert reads must agree bitwise; the union the
dedup path reports must equal the brute-force union of the routed ids; the
logits follow the oracle within the bf16 bound; self-speculation stays
lossless on an MoE model.
"""
import numpy as np
import pytest

import synth
from oracle import Model
from oracle.model import Cache
from _common import engine

pytestmark = pytest.mark.gpu


def _cfg():
    return synth.config("dsv2-lite", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        vocab=2048, n_experts=16, top_k=4, n_shared=2, expert_ffn=128, n_dense_layers=1,
                        dense_ffn=768, max_ctx=192, prompt_len=48, cid=60)


@pytest.fixture(scope="module")
def moe():
    cfg = _cfg()
    w = synth.make_weights(cfg, seed=6)
    print("[moe] building engines", flush=True)
    ps = engine(cfg, w, max_block=17, prefill_chunk=64, moe_dedup=0)
    dd = engine(cfg, w, max_block=17, prefill_chunk=64, moe_dedup=1)
    yield cfg, w, ps, dd, Model(cfg, w)
    ps.close()
    dd.close()


def test_moe_injected_routing_matches_oracle_and_union(moe):
    cfg, w, ps, dd, ora = moe
    n = 64
    trace = synth.make_routing_trace(cfg["n_layers"], n, cfg["n_experts"], cfg["top_k"], seed=6)
    prompt = synth.make_prompt(cfg)
    block = list(synth.make_tokens(cfg["vocab"], 8, seed=6, stream=3))
    res = []
    for eng in (ps, dd):
        eng.set_routing(trace)
        eng.reset()
        eng.prefill(prompt)
        eng.verify(block)
        res.append((eng.read_logits(8), eng.read_union()))
        eng.accept()
        eng.set_routing(None)
    assert np.array_equal(res[0][0], res[1][0])            # per-slot == dedup, bitwise
    for l in range(1, cfg["n_layers"]):
        assert res[1][1][l] == len(set(trace[l, :8].reshape(-1).tolist()))
    ora.routing = {l: trace[l] for l in range(cfg["n_layers"])}
    cache = Cache(cfg)
    ora.forward(prompt, 0, cache)
    ref = ora.forward(block, len(prompt), cache)
    err = np.max(np.abs(res[0][0] - ref))
    print(f"[moe] max |dlogit| = {err:.3e}")
    assert err <= 3e-2
    for l in range(1, cfg["n_layers"]):
        assert ora.union[l] == res[1][1][l]
    ora.routing = None


@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_moe_per_slot_equals_dedup_router_choice(moe, n):
    cfg, w, ps, dd, _ = moe
    prompt = synth.make_prompt(cfg)
    block = list(synth.make_tokens(cfg["vocab"], n, seed=7, stream=n))
    out = []
    for eng in (ps, dd):
        eng.reset()
        eng.prefill(prompt)
        post = eng.verify(block)
        out.append((post, eng.read_logits(n)))
        eng.accept()
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])


def test_routing_switch_drops_captured_passes(moe):
    """A verify pass captured with injected expert ids, then the same shape
    with the router's own choice: the second pass must use the router (equal
    to an eager, graphs-off router-choice verify), not replay the injected
    graph; and an injection for fewer rows than a captured pass is refused."""
    cfg, w, ps, dd, _ = moe
    from self_speculative_decoding_amd import SSDError
    prompt = synth.make_prompt(cfg)
    block = list(synth.make_tokens(cfg["vocab"], 6, seed=8, stream=9))
    trace = synth.make_routing_trace(cfg["n_layers"], 6, cfg["n_experts"], cfg["top_k"], seed=8)

    def run(eng, ids):
        eng.set_routing(None)          # the prompt runs on the router's choice
        eng.reset()
        eng.prefill(prompt)
        eng.set_routing(ids)
        post = eng.verify(block)
        lg = eng.read_logits(len(block))
        eng.accept()
        return post, lg

    for eng in (ps, dd):
        injected = run(eng, trace)
        router = run(eng, None)
        eng.set_graphs(False)
        eager = run(eng, None)
        eng.set_graphs(True)
        assert router[0] == eager[0]
        assert np.array_equal(router[1], eager[1])
        assert not np.array_equal(router[1], injected[1])
        # a captured 6-row pass with injected ids, then ids for 4 rows only
        # (same mode, so the graph stays): the 6-row pass is refused, not replayed
        eng.set_routing(None)
        eng.reset()
        eng.prefill(prompt)
        eng.set_routing(trace)
        eng.verify(block)
        eng.accept()
        eng.set_routing(trace[:, :4])
        with pytest.raises(SSDError):
            eng.verify(block)
        eng.set_routing(None)


def test_moe_self_spec_lossless(moe):
    cfg, w, ps, dd, _ = moe
    from self_speculative_decoding_amd import skip_mask
    prompt = synth.make_prompt(cfg)
    for eng in (ps, dd):
        base, _ = eng.generate(prompt, 40)
        for k in (1, 3, 6):
            out, _ = eng.generate(prompt, 40, skip_mask(cfg["n_layers"], 0.34), k)
            assert out == base, k
    assert ps.generate(prompt, 40)[0] == dd.generate(prompt, 40)[0]


def test_moe_router_choice_matches_oracle_logits(moe):
    """Router-chosen experts: GPU logits follow the oracle (top-k decided in
    each side's own precision; random routers have no near-ties here)."""
    cfg, w, ps, dd, ora = moe
    prompt = synth.make_prompt(cfg)
    ps.reset()
    ps.prefill(prompt)
    got = ps.read_logits(1)[0]
    _, _, last = ora.prefill(prompt)
    assert np.max(np.abs(got - last)) <= 3e-2


def test_measurement_hooks_run_every_op(moe):
    """ssd_time_op on every operation of an MoE model (the bench's timing
    hook): each returns a positive time and leaves the engine usable; the MoE
    op runs the same kernels as a pass, its combine included."""
    cfg, w, ps, dd, ora = moe
    prompt = synth.make_prompt(cfg)
    for eng in (ps, dd):
        eng.reset()
        eng.prefill(prompt)
        moe_layer = cfg["n_dense_layers"]
        for op, layer in (("moe", moe_layer), ("qkv", moe_layer), ("o", moe_layer), ("attention", moe_layer),
                          ("gate_up", 0), ("down", 0), ("lm_head", 0)):
            for m in (1, 4):
                us = eng.time_op(op, layer, m, 3)
                print(f"[moe] time_op {op} layer {layer} m={m}: {us:.2f} us", flush=True)
                assert us > 0.0
        base, _ = eng.generate(prompt, 8)
        assert len(base) == 8
