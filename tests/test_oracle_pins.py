"""Pins of the oracle against facts the pages and mathematics fix (CPU only).

Each test names what it pins.  The oracle is never compared with itself:
the references are library routines (torch, transformers' Llama and
DeepSeek-V2 blocks), closed forms, invariants and brute force.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import synth
from oracle import Model, accept, accept_brute, bf16_round, skip_layers, skip_mask
from oracle.model import Cache, rmsnorm, rope, silu

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# skip set (MLX layer-skip blog, "Code")
# ---------------------------------------------------------------------------

def test_skip_tiny_config_is_layers_1_2():
    # The tiny workload drops layers 1-2 of 4; the blog's rule at 50 % gives exactly that.
    assert skip_layers(4, 0.5) == [1, 2]


def _skip_brute(n, frac):
    """Independent reading of the rule: the block size is the integer nearest
    n * frac (ties to the even one), at least 1; the block is the unique
    contiguous run of that size whose right margin equals its left margin or
    exceeds it by one."""
    t = n * frac
    cands = sorted(range(0, n + 1), key=lambda s: (abs(s - t), s % 2))
    size = min(n, max(1, cands[0]))
    best = [s for s in range(n - size + 1) if (n - s - size) - s in (0, 1)]
    assert len(best) == 1
    return list(range(best[0], best[0] + size))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 12, 32, 36])
@pytest.mark.parametrize("frac", [0.1, 0.2, 0.3, 0.4, 0.5, 0.25, 0.9])
def test_skip_matches_centred_block_brute_force(n, frac):
    assert skip_layers(n, frac) == _skip_brute(n, frac)
    m = skip_mask(n, frac)
    assert sum(m) == len(skip_layers(n, frac)) and len(m) == n


def test_skip_golden_table():
    # tests/golden/skip_sets.txt: the rule applied to the sweep's layer counts
    for line in open(f"{GOLDEN}/skip_sets.txt"):
        if not line.strip() or line.startswith("#"):
            continue
        n, f, lo, hi = line.split()
        assert skip_layers(int(n), float(f)) == list(range(int(lo), int(hi) + 1)), line


def test_skip_rounds_half_to_even():
    # n * frac = 2.5 rounds to 2 (Python's round), 3.5 to 4
    assert len(skip_layers(5, 0.5)) == 2
    assert len(skip_layers(7, 0.5)) == 4
    assert skip_layers(10, 0.01) == [4]          # at least one layer is skipped


# ---------------------------------------------------------------------------
# accept (mlx-dflash "Architecture"; LayerSkip summary 4.3.2)
# ---------------------------------------------------------------------------

def _accept_unique(d, p):
    """The a for which d[0..a) matches p[0..a) and (a == k or d[a] != p[a])."""
    k = len(d)
    sols = [a for a in range(k + 1)
            if all(d[i] == p[i] for i in range(a)) and (a == k or d[a] != p[a])]
    assert len(sols) == 1
    return sols[0]


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4])
def test_accept_exhaustive_v3(k):
    for d in itertools.product(range(3), repeat=k):
        for p in itertools.product(range(3), repeat=k + 1):
            a, em = accept(d, p)
            assert a == _accept_unique(d, p) == accept_brute(d, p)
            # advance by accepted length + 1: drafts d[0..a) then p[a]
            assert len(em) == a + 1 and em[:a] == list(d[:a]) and em[-1] == p[a]


def test_accept_rejects_bad_lengths():
    with pytest.raises(ValueError):
        accept([1, 2], [1, 2])


# ---------------------------------------------------------------------------
# elementwise numerics
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_f32_inputs():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000) * 10 ** g.uniform(-6, 6, 20000),
                        [1.0, -1.0, 0.0, 3.0e38 / 4]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa (1) wins
    assert bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 halfway between 1+2^-7 and 1+2^-6: even (1 + 2^-6) wins
    assert bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above the halfway point rounds up
    assert bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7


def test_rmsnorm_constant_vector_closed_form():
    c, eps = -0.37, 1e-5
    g = np.linspace(0.5, 2.0, 64)
    y = rmsnorm(np.full((1, 64), c), g, eps)
    np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * g, rtol=1e-14)


def test_rmsnorm_matches_torch():
    g = np.random.default_rng(2)
    x, w = g.standard_normal((5, 96)), g.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w), 1e-5)
    np.testing.assert_allclose(rmsnorm(x, w, 1e-5), ref.numpy(), rtol=1e-12, atol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-13, atol=1e-300)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(3).standard_normal((1, 3, 16))
    np.testing.assert_array_equal(rope(x, np.array([0]), 10000.0), x)


def test_rope_is_complex_rotation():
    # pair (i, i + hd/2) as z = a + i b is multiplied by exp(i * p * theta^(-2i/hd))
    hd, theta, p = 32, 10000.0, 37
    x = np.random.default_rng(4).standard_normal((1, 2, hd))
    z = x[..., :hd // 2] + 1j * x[..., hd // 2:]
    w = np.exp(1j * p * theta ** (-np.arange(hd // 2) * 2.0 / hd))
    r = z * w
    ref = np.concatenate([r.real, r.imag], axis=-1)
    np.testing.assert_allclose(rope(x, np.array([p]), theta), ref, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_only_on_offset():
    g = np.random.default_rng(5)
    q, k = g.standard_normal((1, 1, 64)), g.standard_normal((1, 1, 64))
    def score(m, n):
        return float(np.sum(rope(q, np.array([m]), 1e4) * rope(k, np.array([n]), 1e4)))
    assert abs(score(10, 3) - score(107, 100)) < 1e-10
    assert abs(score(10, 3) - score(9, 3)) > 1e-3


# ---------------------------------------------------------------------------
# whole decoder vs transformers' Llama (library routine) in float64
# ---------------------------------------------------------------------------

def _hf_llama(cfg, weights):
    from transformers import LlamaConfig, LlamaForCausalLM
    c = LlamaConfig(vocab_size=cfg["vocab"], hidden_size=cfg["d_model"],
                    intermediate_size=cfg["ffn_dim"], num_hidden_layers=cfg["n_layers"],
                    num_attention_heads=cfg["n_q_heads"], num_key_value_heads=cfg["n_kv_heads"],
                    head_dim=cfg["head_dim"], rms_norm_eps=cfg["rms_eps"],
                    rope_parameters={"rope_type": "default", "rope_theta": cfg["rope_theta"]},
                    tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                    max_position_embeddings=cfg["max_ctx"])
    c._attn_implementation = "eager"
    m = LlamaForCausalLM(c).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    sd = {"model.embed_tokens.weight": t(weights["embed"]), "model.norm.weight": t(weights["final_norm"]),
          "lm_head.weight": t(weights["lm_head"])}
    for l in range(cfg["n_layers"]):
        p, q = f"l{l}.", f"model.layers.{l}."
        sd.update({q + "input_layernorm.weight": t(weights[p + "attn_norm"]),
                   q + "post_attention_layernorm.weight": t(weights[p + "ffn_norm"]),
                   q + "self_attn.q_proj.weight": t(weights[p + "wq"]),
                   q + "self_attn.k_proj.weight": t(weights[p + "wk"]),
                   q + "self_attn.v_proj.weight": t(weights[p + "wv"]),
                   q + "self_attn.o_proj.weight": t(weights[p + "wo"]),
                   q + "mlp.gate_proj.weight": t(weights[p + "w_gate"]),
                   q + "mlp.up_proj.weight": t(weights[p + "w_up"]),
                   q + "mlp.down_proj.weight": t(weights[p + "w_down"])})
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in k for k in missing), (missing, unexpected)
    return m


def _random_gains(cfg, weights, seed):
    # unit gains would hide a gain applied to the wrong norm: use random gains here
    g = np.random.default_rng(seed)
    out = dict(weights)
    for name, shape, kind in synth.weight_specs(cfg):
        if kind == "gain":
            out[name] = (1.0 + 0.5 * g.standard_normal(shape)).astype(np.float32)
    return out


@pytest.mark.parametrize("which", ["micro", "tiny"])
def test_decoder_matches_transformers_llama(which):
    cfg = synth.micro_config() if which == "micro" else synth.config("tiny")
    w = _random_gains(cfg, synth.make_weights(cfg, seed=7), 8)
    # scale up the random matrices so attention is far from uniform
    for k in list(w):
        if k.endswith((".wq", ".wk")):
            w[k] = w[k] * 8
    toks = synth.make_tokens(cfg["vocab"], 40, seed=7, stream=1)
    ora = Model(cfg, w).forward(toks, 0, Cache(cfg))
    with torch.no_grad():
        ref = _hf_llama(cfg, w)(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    # transformers runs its RMSNorm and rotary tables in float32
    assert np.max(np.abs(ora - ref)) < 2e-5 * np.max(np.abs(ref))


def test_feature_tap_is_residual_after_layer():
    cfg = synth.micro_config(n_layers=4, feat_layers=(1, 2))
    cfg["out_scale"] = {}
    w = _random_gains(cfg, synth.make_weights(cfg, seed=9), 10)
    toks = synth.make_tokens(cfg["vocab"], 12, seed=9, stream=2)
    m = Model(cfg, w)
    m.forward(toks, 0, Cache(cfg))
    with torch.no_grad():
        hs = _hf_llama(cfg, {k: v for k, v in w.items() if k != "fc"})(
            torch.from_numpy(toks.astype(np.int64))[None], output_hidden_states=True).hidden_states
    # hidden_states[i + 1] is the output of 0-indexed layer i (before the final norm for i < L-1)
    cat = np.concatenate([hs[2][0].numpy(), hs[3][0].numpy()], axis=-1)
    ref = cat @ np.asarray(w["fc"], dtype=np.float64).T
    assert np.max(np.abs(m.features - ref)) < 2e-6 * np.max(np.abs(ref))


def test_attention_matches_torch_sdpa_gqa():
    cfg = synth.micro_config(n_q_heads=6, n_kv_heads=2, head_dim=8, d_model=48)
    w = synth.make_weights(cfg, seed=11)
    for k in list(w):
        if k.endswith((".wq", ".wk")):
            w[k] = w[k] * 10
    m = Model(cfg, w)
    cache = Cache(cfg)
    x = np.random.default_rng(12).standard_normal((9, 48))
    pos0 = 0
    h = m.attention_block(0, x, pos0, cache) - x
    # rebuild q, k, v independently of the block and call torch's SDPA
    from oracle.model import rmsnorm as rn_, rope as rp_
    n1 = rn_(x, np.asarray(w["l0.attn_norm"], np.float64), 1e-5)
    q = rp_((n1 @ np.asarray(w["l0.wq"], np.float64).T).reshape(9, 6, 8), np.arange(9), 1e4)
    k = rp_((n1 @ np.asarray(w["l0.wk"], np.float64).T).reshape(9, 2, 8), np.arange(9), 1e4)
    v = (n1 @ np.asarray(w["l0.wv"], np.float64).T).reshape(9, 2, 8)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(T(q), T(k), T(v), is_causal=True, enable_gqa=True)
    ref = o[0].numpy().transpose(1, 0, 2).reshape(9, 48) @ np.asarray(w["l0.wo"], np.float64).T
    np.testing.assert_allclose(h, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# cache, causality and decoding invariants
# ---------------------------------------------------------------------------

def _micro(seed=0, **kw):
    cfg = synth.micro_config(**kw)
    w = synth.make_weights(cfg, seed=seed)
    for k in list(w):
        if k.endswith((".wq", ".wk")):
            w[k] = w[k] * 6
    return cfg, Model(cfg, w)


def test_cached_decode_equals_full_reforward():
    cfg, m = _micro()
    toks = synth.make_tokens(cfg["vocab"], 20, seed=0, stream=3)
    full = m.forward(toks, 0, Cache(cfg))
    cache = Cache(cfg)
    rows = [m.forward(toks[:7], 0, cache)]
    for i in range(7, 20, 3):          # mixed block widths
        rows.append(m.forward(toks[i:i + 3], i, cache))
    np.testing.assert_allclose(np.concatenate(rows), full, rtol=1e-11, atol=1e-12)


def test_causality():
    cfg, m = _micro()
    a = synth.make_tokens(cfg["vocab"], 16, seed=0, stream=4)
    b = a.copy()
    b[10:] = (b[10:] + 1) % cfg["vocab"]
    la, lb = m.forward(a, 0, Cache(cfg)), m.forward(b, 0, Cache(cfg))
    np.testing.assert_array_equal(la[:10], lb[:10])
    assert np.max(np.abs(la[10:] - lb[10:])) > 1e-6


def test_greedy_tokens_are_argmax_of_teacher_forced():
    cfg, m = _micro()
    p = synth.make_prompt(cfg, seed=1)
    g, rows = m.greedy(p, 20)
    tf = m.teacher_forced(p, g)
    np.testing.assert_allclose(tf, rows, rtol=1e-10, atol=1e-11)
    assert g == [int(np.argmax(r)) for r in tf]


def test_zero_layers_reduce_to_head_of_embedding():
    cfg = synth.micro_config()
    w = synth.make_weights(cfg, seed=3)
    for l in range(cfg["n_layers"]):
        w[f"l{l}.wo"] = np.zeros_like(w[f"l{l}.wo"])
        w[f"l{l}.w_down"] = np.zeros_like(w[f"l{l}.w_down"])
    m = Model(cfg, w)
    toks = synth.make_tokens(cfg["vocab"], 5, seed=3, stream=5)
    E = np.asarray(w["embed"], np.float64)[toks]
    ref = torch.nn.functional.rms_norm(torch.from_numpy(E), (cfg["d_model"],), eps=1e-5).numpy() \
        @ np.asarray(w["lm_head"], np.float64).T
    np.testing.assert_allclose(m.forward(toks, 0, Cache(cfg)), ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# self-speculation: lossless, and the closed-form special cases
# ---------------------------------------------------------------------------

def test_self_spec_lossless_all_masks_micro():
    cfg, m = _micro(seed=5, n_layers=3)
    cfg["out_scale"] = {}
    p = synth.make_prompt(cfg, seed=5)
    ref, _ = m.greedy(p, 24)
    for mask in itertools.product([0, 1], repeat=3):
        skip = [l for l in range(3) if mask[l]]
        for k in range(0, 7):
            out, st = m.self_spec(p, 24, skip, k)
            assert out == ref, (skip, k)


def test_self_spec_lossless_tiny_config():
    cfg = synth.config("tiny")
    m = Model(cfg, synth.make_weights(cfg))
    p = synth.make_prompt(cfg)
    ref, _ = m.greedy(p, cfg["n_new"])
    out, st = m.self_spec(p, cfg["n_new"], cfg["skip_layers"], cfg["k"])
    assert out == ref
    assert st["accepted"] > 0           # the x0.1 layers make the draft useful


def test_empty_mask_accepts_every_draft():
    cfg, m = _micro(seed=6)
    p = synth.make_prompt(cfg, seed=6)
    N = 24
    for k in (1, 2, 3, 5):
        out, st = m.self_spec(p, N, [], k)
        assert all(a == k for a in st["a_hist"])
        assert st["cycles"] == math.ceil((N - 1) / (k + 1))


def test_zeroed_skipped_layers_make_draft_exact():
    cfg = synth.micro_config(n_layers=4)
    w = synth.make_weights(cfg, seed=8)
    for l in (1, 2):
        w[f"l{l}.wo"] = np.zeros_like(w[f"l{l}.wo"])
        w[f"l{l}.w_down"] = np.zeros_like(w[f"l{l}.w_down"])
    m = Model(cfg, w)
    out, st = m.self_spec(synth.make_prompt(cfg, seed=8), 24, [1, 2], 3)
    assert all(a == 3 for a in st["a_hist"])
    assert out == m.greedy(synth.make_prompt(cfg, seed=8), 24)[0]


def test_forced_wrong_draft_accepts_nothing():
    cfg, m = _micro(seed=9)
    V = cfg["vocab"]
    p = synth.make_prompt(cfg, seed=9)
    N = 20
    ref, _ = m.greedy(p, N)
    # every draft is replaced by the verifier-correct token + 1: first draft always rejected
    out, st = m.self_spec(p, N, [], 3, draft_fn=lambda j, t: (t + 1) % V)
    assert out == ref
    assert all(a == 0 for a in st["a_hist"]) and st["cycles"] == N - 1


def test_k0_is_plain_greedy():
    cfg, m = _micro(seed=10)
    p = synth.make_prompt(cfg, seed=10)
    out, st = m.self_spec(p, 18, [0], 0)
    assert out == m.greedy(p, 18)[0] and st["cycles"] == 17


# ---------------------------------------------------------------------------
# MoE expert FFN (speculative decoding for MoE models, abstract)
# ---------------------------------------------------------------------------

def _moe_cfg():
    return synth.config("dsv2-lite", n_layers=3, d_model=64, n_q_heads=4, n_kv_heads=2,
                        head_dim=16, vocab=96, n_experts=16, top_k=4, n_shared=2,
                        expert_ffn=24, dense_ffn=80, dtype="f32", max_ctx=64)


def _hf_moe_block(w):
    """transformers' DeepSeek-V2 MoE block (float64) holding layer 1's experts of w."""
    from transformers import DeepseekV2Config
    from transformers.models.deepseek_v2.modeling_deepseek_v2 import DeepseekV2Moe
    c = DeepseekV2Config(hidden_size=64, num_experts=16, num_experts_per_tok=4, n_shared_experts=2,
                         moe_intermediate_size=24, routed_scaling_factor=1.0, topk_method="greedy",
                         hidden_act="silu", mlp_bias=False)
    blk = DeepseekV2Moe(c).double()
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    with torch.no_grad():
        blk.gate.weight.copy_(t(w["l1.router"]))
        blk.experts.gate_up_proj.copy_(torch.cat([t(w["l1.exp_gate"]), t(w["l1.exp_up"])], dim=1))
        blk.experts.down_proj.copy_(t(w["l1.exp_down"]))
        blk.shared_experts.gate_proj.weight.copy_(t(w["l1.sh_gate"]).reshape(48, 64))
        blk.shared_experts.up_proj.weight.copy_(t(w["l1.sh_up"]).reshape(48, 64))
        blk.shared_experts.down_proj.weight.copy_(torch.cat([t(w["l1.sh_down"][0]), t(w["l1.sh_down"][1])], dim=1))
    return blk


def test_moe_layer_folded_norm_matches_transformers_on_the_normed_input():
    """The MoE feed-forward of a layer takes the stored input x * g and the
    rows' 1/rms factors (the ffn norm folded in, as every norm that feeds a
    product): it must equal transformers' DeepSeek-V2 MoE block applied to
    rmsnorm(x, g), router included.  A factor left off the router, the gate
    or the up product (or applied to the down product) fails it."""
    cfg = _moe_cfg()
    w = synth.make_weights(cfg, seed=29)
    w["l1.router"] = w["l1.router"] * 20            # peaked routing: no near-ties
    w["l1.ffn_norm"] = np.random.default_rng(31).uniform(0.5, 1.5, 64).astype(np.float32)
    m = Model(cfg, w)
    # residual rows with distinct scales, so that a missing 1/rms shows
    h = np.random.default_rng(30).standard_normal((6, 64)) * np.array([0.3, 1, 2, 5, 0.7, 3])[:, None]
    blk = _hf_moe_block(m.w)
    with torch.no_grad():
        ref = blk(torch.from_numpy(rmsnorm(h, m.w["l1.ffn_norm"], m.eps))[None])[0].numpy()
    xg, rstd = m.norm_input(h, m.w["l1.ffn_norm"])
    for dedup in (False, True):
        np.testing.assert_allclose(m.moe_ffn(1, xg, rstd, dedup=dedup), ref, rtol=2e-5, atol=2e-6)
    # without the 1/rms factors the output is visibly different
    assert not np.allclose(m.moe_ffn(1, xg), ref, rtol=1e-3)


def test_moe_block_matches_transformers_deepseek_v2():
    from transformers import DeepseekV2Config
    from transformers.models.deepseek_v2.modeling_deepseek_v2 import DeepseekV2Moe
    cfg = _moe_cfg()
    w = synth.make_weights(cfg, seed=13)
    w["l1.router"] = w["l1.router"] * 20            # peaked routing: no near-ties
    m = Model(cfg, w)
    c = DeepseekV2Config(hidden_size=64, num_experts=16, num_experts_per_tok=4, n_shared_experts=2,
                         moe_intermediate_size=24, routed_scaling_factor=1.0, topk_method="greedy",
                         hidden_act="silu", mlp_bias=False)
    blk = DeepseekV2Moe(c).double()
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    with torch.no_grad():
        blk.gate.weight.copy_(t(w["l1.router"]))
        blk.experts.gate_up_proj.copy_(torch.cat([t(w["l1.exp_gate"]), t(w["l1.exp_up"])], dim=1))
        blk.experts.down_proj.copy_(t(w["l1.exp_down"]))
        blk.shared_experts.gate_proj.weight.copy_(t(w["l1.sh_gate"]).reshape(48, 64))
        blk.shared_experts.up_proj.weight.copy_(t(w["l1.sh_up"]).reshape(48, 64))
        blk.shared_experts.down_proj.weight.copy_(torch.cat([t(w["l1.sh_down"][0]), t(w["l1.sh_down"][1])], dim=1))
    x = np.random.default_rng(14).standard_normal((7, 64))
    with torch.no_grad():
        ref = blk(torch.from_numpy(x)[None])[0].numpy()
    # transformers' router runs in float32
    np.testing.assert_allclose(m.moe_ffn(1, x), ref, rtol=2e-5, atol=2e-6)


def test_moe_router_topk_matches_torch_topk():
    cfg = _moe_cfg()
    m = Model(cfg, synth.make_weights(cfg, seed=15))
    x = np.random.default_rng(16).standard_normal((9, 64))
    probs, ids = m.route(1, x)
    tv, ti = torch.topk(torch.from_numpy(probs), 4, dim=-1)
    np.testing.assert_array_equal(ids, ti.numpy())
    np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=1e-14)


def test_moe_topk_ties_take_lower_id():
    cfg = _moe_cfg()
    m = Model(cfg, synth.make_weights(cfg, seed=17))
    m.w["l1.router"] = np.zeros_like(m.w["l1.router"])     # uniform probabilities
    _, ids = m.route(1, np.ones((2, 64)))
    np.testing.assert_array_equal(ids, [[0, 1, 2, 3]] * 2)


@pytest.mark.parametrize("n", [1, 3, 8])
def test_moe_dedup_equals_per_slot_and_union(n):
    cfg = _moe_cfg()
    m = Model(cfg, synth.make_weights(cfg, seed=18))
    trace = synth.make_routing_trace(cfg["n_layers"], n, 16, 4, seed=18)
    m.routing = {l: trace[l] for l in range(cfg["n_layers"])}
    x = np.random.default_rng(19).standard_normal((n, 64))
    a = m.moe_ffn(1, x, dedup=False)
    b = m.moe_ffn(1, x, dedup=True)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    assert m.union[1] == len(set(trace[1].reshape(-1).tolist()))


def test_routing_trace_rows_are_distinct_and_reuse_half():
    tr = synth.make_routing_trace(4, 8, 64, 6, seed=0, stream=1)
    for l in range(4):
        for t in range(8):
            assert len(set(tr[l, t].tolist())) == 6
    reuse = np.mean(tr[:, 1:] == tr[:, :-1])
    assert 0.3 < reuse < 0.7


def test_geometric_block_prefix():
    true = np.arange(100, 115, dtype=np.int32)
    for s in range(50):
        d, m = synth.make_geometric_block(true, 1000, 0.7, 16, seed=0, stream=s)
        a, _ = accept(d, list(true) + [0])
        assert a == m


# ---------------------------------------------------------------------------
# draft-length choice (speculative decoding for MoE models, abstract)
# ---------------------------------------------------------------------------

def test_kselect_hand_worked_example():
    from oracle import select_k, expected_tokens
    # flat verify cost 1.0, draft step 0.8, no overhead, alpha 0.9:
    # r0 = 1/1, r1 = 1.9/1.8 = 1.0556, r2 = 2.71/2.6 = 1.0423, r3 = 3.439/3.4 = 1.0115
    assert abs(expected_tokens(0.9, 2) - 2.71) < 1e-12
    k, r = select_k([1.0, 1.0, 1.0, 1.0], 0.8, 0.0, 0.9)
    assert k == 1 and abs(r - 1.9 / 1.8) < 1e-12
    # cheaper drafts push k up: t_draft 0.2 -> r3 = 3.439/1.6 beats r2 = 2.71/1.4
    assert select_k([1.0] * 6, 0.2, 0.0, 0.9)[0] == 5


def test_kselect_closed_forms():
    from oracle import select_k, expected_tokens
    # geometric sum closed form
    for a in (0.0, 0.3, 0.95):
        for k in range(8):
            cf = (1 - a ** (k + 1)) / (1 - a)
            assert abs(expected_tokens(a, k) - cf) < 1e-12
    # alpha = 0: one token per cycle whatever k, so the cheapest cycle wins
    tv = [1.0, 1.05, 1.1, 1.2]
    assert select_k(tv, 0.5, 0.1, 0.0) == (0, 1.0 / 1.1)
    # alpha = 1: E_k = k + 1
    k, r = select_k([1.0, 1.0, 1.0], 0.5, 0.0, 1.0)
    assert k == 2 and abs(r - 3 / 2.0) < 1e-12
    # exact ties (alpha = 0, free drafts, flat verify): the smallest k wins
    assert select_k([1.0, 1.0, 1.0], 0.0, 0.0, 0.0) == (0, 1.0)
    assert select_k([2.0, 1.0, 1.0, 1.0], 0.0, 0.0, 0.0) == (1, 1.0)


# ---------------------------------------------------------------------------
# skip set as a knapsack (MLX layer-skip blog, "Paper -> the idea")
# ---------------------------------------------------------------------------

def test_layer_cosines_closed_forms():
    from oracle import layer_cosines
    e = np.array([[1.0, 0.0], [0.0, 2.0]])
    same = e * 3.0                               # parallel: cos 1
    orth = np.array([[0.0, 5.0], [-1.0, 0.0]])   # orthogonal to the previous rows: cos 0
    neg = -orth                                  # opposite: cos -1
    got = layer_cosines(e, [same, orth, neg])
    np.testing.assert_allclose(got, [1.0, 0.0, -1.0], atol=1e-15)
    # 45 degrees
    np.testing.assert_allclose(layer_cosines(np.array([[1.0, 0.0]]), [np.array([[1.0, 1.0]])]), [2 ** -0.5])
    # the layer's value averages its rows: cos 1, 1 and 0 over three rows -> 2/3
    e3 = np.eye(3)
    out = np.array([[2.0, 0.0, 0.0], [0.0, 3.0, 0.0], [1.0, 0.0, 0.0]])
    np.testing.assert_allclose(layer_cosines(e3, [out]), [2.0 / 3.0], atol=1e-15)


def test_knapsack_brute_hand_example():
    from oracle import knapsack_skip_brute
    # values 6, 10, 12 with costs 1, 2, 3 and budget 5: keep {1, 2} (22)
    best, sets = knapsack_skip_brute([1, 2, 3], [6.0, 10.0, 12.0], 5)
    assert best == 22.0 and sets == [(1, 2)]
    # budget 0 keeps nothing; a large budget keeps everything
    assert knapsack_skip_brute([1, 2, 3], [6.0, 10.0, 12.0], 0) == (0.0, [()])
    assert knapsack_skip_brute([1, 2, 3], [6.0, 10.0, 12.0], 6)[0] == 28.0


# ---------------------------------------------------------------------------
# speculative sampling (LayerSkip summary 4.3.2: rejection-sampling accept)
# ---------------------------------------------------------------------------

def test_philox_matches_numpy_bit_generator():
    from oracle import philox4x64_10
    # numpy's Philox (4x64, 10 rounds) advances its counter before each block
    for ctr, key in (([0, 0, 0, 0], [0, 0]), ([5, 7, 0, 0], [11, 13]), ([2**62 + 5, 3, 9, 1], [2**62, 17])):
        bg = np.random.Philox(counter=ctr, key=key)
        got = [int(x) for x in bg.random_raw(4)]
        nxt = list(ctr)
        nxt[0] = (nxt[0] + 1) % 2**64
        if nxt[0] == 0:
            nxt[1] += 1
        assert philox4x64_10(nxt, key) == got


def test_draw_special_cases():
    from oracle import draw, uniform24
    assert draw([0, 0, 3.0, 0], 0.0)[0] == 2 and draw([0, 0, 3.0, 0], 0.99)[0] == 2
    for u in (0.0, 0.1, 0.5, 0.99):
        assert draw(np.ones(10), u)[0] == int(u * 10)
    for s in range(50):
        u = uniform24(7, s, 1, 2)
        assert 0.0 <= u < 1.0 and u * 2**24 == int(u * 2**24)


def _chi2_ok(counts, p, min_expected=5.0):
    """Pearson chi-square with bins of small expectation pooled; True unless the
    statistic exceeds its 0.999 quantile (Wilson-Hilferty approximation)."""
    counts, p = np.asarray(counts, float), np.asarray(p, float)
    n = counts.sum()
    order = np.argsort(p)
    cs, ps, acc_c, acc_p = [], [], 0.0, 0.0
    for i in order:
        acc_c += counts[i]
        acc_p += p[i]
        if acc_p * n >= min_expected:
            cs.append(acc_c); ps.append(acc_p); acc_c = acc_p = 0.0
    if acc_p > 0:
        cs[-1] += acc_c; ps[-1] += acc_p
    cs, ps = np.array(cs), np.array(ps)
    stat = np.sum((cs - n * ps) ** 2 / (n * ps))
    df = len(cs) - 1
    z = 3.090                                              # 0.999 normal quantile
    q = df * (1 - 2 / (9 * df) + z * np.sqrt(2 / (9 * df))) ** 3
    return stat <= q, stat, q


def test_spec_cycle_output_follows_the_target_distribution():
    """The speculative-sampling theorem on a small vocabulary: whatever the draft
    distribution, the first emitted token is distributed as p_0, the second
    (when emitted) as p_1, and draft 1 is accepted with probability
    sum_x min(p_0(x), q_1(x))."""
    from oracle import spec_cycle, probs
    rng = np.random.default_rng(3)
    V, k, T, N = 6, 2, 0.8, 12000
    tl = rng.normal(0, 1.5, (k + 1, V))
    dl = rng.normal(0, 1.5, (k, V))
    first, second, acc1 = np.zeros(V), np.zeros(V), 0
    for c in range(N):
        a, em, _ = spec_cycle(tl, dl, T, seed=99, cycle=c)
        first[em[0]] += 1
        if len(em) > 1:
            second[em[1]] += 1
        acc1 += a >= 1
    assert _chi2_ok(first, probs(tl[0], T))[0]
    assert _chi2_ok(second, probs(tl[1], T))[0]
    pa = np.sum(np.minimum(probs(tl[0], T), probs(dl[0], T)))
    assert abs(acc1 / N - pa) <= 4 * np.sqrt(pa * (1 - pa) / N)
    # a draft equal to the target is always accepted
    a, em, _ = spec_cycle(tl, tl[:k], T, seed=1, cycle=0)
    assert a == k


def _np_philox_word0(seed, ctr):
    """First output word of Philox4x64-10 at counter ctr (ctr[0] >= 1), key
    (seed, 0), from numpy's own generator (it advances the counter first)."""
    bg = np.random.Philox(counter=[ctr[0] - 1, ctr[1], ctr[2], ctr[3]], key=[seed, 0])
    return int(bg.random_raw(1)[0])


def test_uniform24_is_the_top_24_bits_of_numpys_philox_word():
    from oracle import uniform24
    odd = 0
    for c in range(1, 300):
        u = uniform24(17, c, c % 5, c % 3)
        w = _np_philox_word0(17, [c, c % 5, c % 3, 0])
        assert u * 2**24 == (w >> 40)
        odd += (w >> 40) & 1
    assert odd > 0


def test_probs_is_softmax_of_logits_over_temperature():
    from scipy.special import softmax
    from oracle import probs
    rng = np.random.default_rng(4)
    l = rng.normal(0, 3, 50)
    for T in (0.25, 0.6, 1.0, 2.5):
        assert np.allclose(probs(l, T), softmax(l / T), rtol=1e-12, atol=0)
    assert np.array_equal(probs(np.array([0.0, -np.inf, 0.0]), 1.0), np.array([0.5, 0.0, 0.5]))


def test_spec_cycle_decisions_on_constructed_cycles():
    """Cycles whose every decision follows from one Philox number (numpy's):
    (A) q_1 puts all mass on token 0 and p_0 half, so d_1 = 0 is accepted iff
    u(c, 1, accept) < 1/2; accepted, the bonus token comes from p_1 (uniform on
    {2, 3}) with u(c, 1, final); rejected, the residual is all on token 1.
    (B) q_1 uniform on {0, 1} and p_0 uniform on {2, 3}: d_1 = 0 iff
    u(c, 0, draft) < 1/2, always rejected, the final token is 2 iff
    u(c, 0, final) < 1/2."""
    from oracle import spec_cycle
    ninf = -np.inf
    seed = 5
    u = lambda c, slot, purpose: (_np_philox_word0(seed, [c, slot, purpose, 0]) >> 40) / 2**24
    tlA = np.array([[0.0, 0.0, ninf, ninf], [ninf, ninf, 0.0, 0.0]])
    dlA = np.array([[0.0, ninf, ninf, ninf]])
    tlB = np.array([[ninf, ninf, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    dlB = np.array([[0.0, 0.0, ninf, ninf]])
    seen = set()
    for c in range(1, 200):
        a, em, _ = spec_cycle(tlA, dlA, 1.0, seed, c)
        if u(c, 1, 1) < 0.5:
            want = (1, [0, 2 if u(c, 1, 2) < 0.5 else 3])
        else:
            want = (0, [1])
        assert (a, em) == want, c
        seen.add(tuple(em))
        a, em, _ = spec_cycle(tlB, dlB, 1.0, seed, c)
        assert (a, em) == (0, [2 if u(c, 0, 2) < 0.5 else 3]), c
        d = 0 if u(c, 0, 0) < 0.5 else 1
        assert spec_cycle(tlB, dlB, 1.0, seed, c, drafts=[d])[:2] == (a, em)
    assert seen == {(0, 2), (0, 3), (1,)}
