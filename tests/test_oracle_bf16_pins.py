"""Pins of the oracle's bf16 mode (CPU only).

The bf16 workloads store weights, every GEMM input, the K/V cache entries,
q after the rotary embedding, the attention output, the SwiGLU activation
and the feature-tap concat and output as bf16 (round to nearest, ties to
even), while norms, softmax and accumulations stay wide.  These tests pin the
oracle's bf16 arithmetic to independent references:

- the bf16 weight decoding against torch's bfloat16 on every bit pattern;
- the whole bf16 decoder against transformers' Llama run in float64 with the
  same rounding points inserted by hooks (a float64 bit-level rounding
  written here, not the oracle's), so every rounding point and every
  operation between them is checked, and the two sides differ only by
  float64 summation order;
- the MoE feed-forward of a bf16 model against transformers' DeepSeek-V2
  MoE block with the expert activation rounded the same way;
- that every value the oracle declares stored is a bf16 value.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import Model, decode_weight
from oracle.model import Cache


def _rne_bf16(x):
    """float64 -> nearest bf16 value (ties to even), on the float64 bit
    pattern: keep sign, exponent and the top 7 stored mantissa bits, round on
    the 45 dropped bits.  Finite normal values only."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    u = a.view(np.uint64)
    keep = u >> np.uint64(45)
    rem = u & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    out = ((keep + up.astype(np.uint64)) << np.uint64(45)).view(np.float64)
    return np.where(a == 0.0, a, out)


def _rne_t(t):
    return torch.from_numpy(_rne_bf16(t.detach().numpy()))


def _torch_w(a):
    """A stored weight as a float64 tensor, decoded by torch (bf16 bits viewed
    as torch.bfloat16), independently of the oracle's decoding."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _bf16_bits(x):
    """float values that are bf16-representable -> uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    assert np.array_equal(_rne_bf16(f.astype(np.float64)), f.astype(np.float64))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# weight decoding
# ---------------------------------------------------------------------------

def test_decode_weight_every_bf16_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns
        ours = decode_weight(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # the float32 path is the identity
    f = np.random.default_rng(0).standard_normal(100).astype(np.float32)
    assert np.array_equal(decode_weight(f), f.astype(np.float64))


def test_reference_rounding_matches_torch_on_float32_inputs():
    """The test's own float64 rounding agrees with torch's float32 -> bf16
    conversion wherever that conversion is a single rounding."""
    g = np.random.default_rng(1)
    x = (g.standard_normal(50000) * 10.0 ** g.uniform(-5, 5, 50000)).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]   # ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(_rne_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# bf16 models
# ---------------------------------------------------------------------------

def _bf16_model(cfg, seed, scale_qk=8.0):
    """bf16 weights of cfg with random bf16 norm gains and scaled-up q/k
    projections (attention far from uniform); all values exact bf16."""
    w = synth.make_weights(cfg, seed=seed)
    g = np.random.default_rng(seed + 1)
    out = {}
    for name, shape, kind in synth.weight_specs(cfg):
        if kind == "gain":
            gain = (1.0 + 0.5 * g.standard_normal(shape)).astype(np.float32)
            out[name] = _bf16_bits(_rne_bf16(gain.astype(np.float64)).astype(np.float32))
        elif name.endswith((".wq", ".wk")):
            out[name] = _bf16_bits(decode_weight(w[name]) * scale_qk)   # power of two: exact
        else:
            out[name] = w[name]
    return out


def _bf16_cfg(which):
    if which == "micro":
        return synth.micro_config(dtype="bf16")
    return synth.config("tiny", dtype="bf16", out_scale={})


class _FoldedNorm(torch.nn.Module):
    """The stored operand of a GEMM after a norm: bf16(x * g), with the
    per-row factor 1/sqrt(mean(x^2) + eps) applied to it in float64 (the
    product then equals the oracle's scaled product up to float64 rounding)."""

    def __init__(self, g, eps):
        super().__init__()
        self.g = _torch_w(g)
        self.eps = eps

    def forward(self, x):
        rstd = 1.0 / torch.sqrt(torch.mean(x * x, dim=-1, keepdim=True) + self.eps)
        return _rne_t(x * self.g) * rstd


class _Rotary64(torch.nn.Module):
    """cos / sin tables of the rotate-half rotary embedding in float64
    (transformers computes them in float32)."""

    def __init__(self, hd, theta):
        super().__init__()
        self.inv = theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)

    def forward(self, x, position_ids):
        f = position_ids[0].to(torch.float64)[:, None] * self.inv[None, :]
        emb = torch.cat([f, f], dim=-1)[None]
        return emb.cos(), emb.sin()


def _bf16_attention(module, query, key, value, attention_mask, scaling, dropout=0.0, **kw):
    """transformers' attention interface with q after the rotary embedding
    and the K/V entries stored as bf16; scores, mask and softmax in float64."""
    from transformers.models.llama.modeling_llama import repeat_kv
    q, k, v = _rne_t(query), _rne_t(key), _rne_t(value)
    k = repeat_kv(k, module.num_key_value_groups)
    v = repeat_kv(v, module.num_key_value_groups)
    s = torch.matmul(q, k.transpose(2, 3)) * scaling
    if attention_mask is not None:
        s = s + attention_mask.to(s.dtype)
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v).transpose(1, 2).contiguous(), p


def _hf_bf16_llama(cfg, w):
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
    t = _torch_w
    sd = {"model.embed_tokens.weight": t(w["embed"]), "lm_head.weight": t(w["lm_head"])}
    for l in range(cfg["n_layers"]):
        p, q = f"l{l}.", f"model.layers.{l}."
        sd.update({q + "self_attn.q_proj.weight": t(w[p + "wq"]), q + "self_attn.k_proj.weight": t(w[p + "wk"]),
                   q + "self_attn.v_proj.weight": t(w[p + "wv"]), q + "self_attn.o_proj.weight": t(w[p + "wo"]),
                   q + "mlp.gate_proj.weight": t(w[p + "w_gate"]), q + "mlp.up_proj.weight": t(w[p + "w_up"]),
                   q + "mlp.down_proj.weight": t(w[p + "w_down"])})
    m.load_state_dict(sd, strict=False)
    eps = cfg["rms_eps"]
    round_input = lambda mod, args: (_rne_t(args[0]),)
    for l, layer in enumerate(m.model.layers):
        layer.input_layernorm = _FoldedNorm(w[f"l{l}.attn_norm"], eps)
        layer.post_attention_layernorm = _FoldedNorm(w[f"l{l}.ffn_norm"], eps)
        layer.self_attn.o_proj.register_forward_pre_hook(round_input)     # attention output
        layer.mlp.down_proj.register_forward_pre_hook(round_input)        # silu(gate) * up
    m.model.norm = _FoldedNorm(w["final_norm"], eps)
    m.model.rotary_emb = _Rotary64(cfg["head_dim"], cfg["rope_theta"])
    return m


@pytest.mark.parametrize("which", ["micro", "tiny"])
def test_bf16_decoder_matches_transformers_llama_with_storage_rounding(which):
    """Bound: both sides round the same float64 values at the same points, so
    they differ by float64 summation order only (relative ~1e-15); a bf16
    rounding decision can change only for a value within that distance of a
    rounding midpoint (probability ~1e-12 per value).  1e-9 of the largest
    logit leaves a margin of six orders of magnitude, while any misplaced or
    missing rounding point moves the logits by ~1e-3 of their scale."""
    import transformers.models.llama.modeling_llama as hf_llama
    cfg = _bf16_cfg(which)
    w = _bf16_model(cfg, seed=21)
    toks = synth.make_tokens(cfg["vocab"], 40, seed=21, stream=1)
    ora = Model(cfg, w).forward(toks, 0, Cache(cfg))
    saved = hf_llama.eager_attention_forward
    hf_llama.eager_attention_forward = _bf16_attention
    try:
        with torch.no_grad():
            ref = _hf_bf16_llama(cfg, w)(torch.from_numpy(toks.astype(np.int64))[None],
                                         use_cache=False).logits[0].numpy()
    finally:
        hf_llama.eager_attention_forward = saved
    err = float(np.max(np.abs(ora - ref)))
    assert err <= 1e-9 * float(np.max(np.abs(ref))), err
    # the rounding points matter at this scale: without them the logits move
    ora_f32 = Model(dict(cfg, dtype="f32"), w).forward(toks, 0, Cache(cfg))
    assert np.max(np.abs(ora_f32 - ref)) > 1e-4 * np.max(np.abs(ref))


def test_bf16_feature_tap_matches_transformers_hidden_states():
    """fc . bf16(concat of the residual after the tapped layers), stored bf16."""
    import transformers.models.llama.modeling_llama as hf_llama
    cfg = synth.micro_config(n_layers=4, feat_layers=(1, 2), dtype="bf16")
    w = _bf16_model(cfg, seed=23)
    toks = synth.make_tokens(cfg["vocab"], 12, seed=23, stream=2)
    m = Model(cfg, w)
    m.forward(toks, 0, Cache(cfg))
    saved = hf_llama.eager_attention_forward
    hf_llama.eager_attention_forward = _bf16_attention
    try:
        with torch.no_grad():
            hs = _hf_bf16_llama(cfg, {k: v for k, v in w.items() if k != "fc"})(
                torch.from_numpy(toks.astype(np.int64))[None], use_cache=False,
                output_hidden_states=True).hidden_states
    finally:
        hf_llama.eager_attention_forward = saved
    cat = _rne_bf16(np.concatenate([hs[2][0].numpy(), hs[3][0].numpy()], axis=-1))
    ref = _rne_bf16(cat @ _torch_w(w["fc"]).numpy().T)
    # equal up to float64 order; a stored value may sit one bf16 step away
    # only where its float64 value lies on a rounding midpoint (not seen)
    assert np.array_equal(m.features, ref)


def test_bf16_moe_block_matches_transformers_deepseek_v2():
    """Routed and shared experts of a bf16 model: bf16 input rows, bf16
    weights, the SwiGLU activation stored bf16 before each down projection.
    transformers' router runs in float32, so the gate weights (and only
    they) differ at float32 rounding: bound 2e-5 relative."""
    from transformers import DeepseekV2Config
    from transformers.models.deepseek_v2.modeling_deepseek_v2 import DeepseekV2Moe
    cfg = synth.config("dsv2-lite", n_layers=3, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                       vocab=96, n_experts=16, top_k=4, n_shared=2, expert_ffn=24, dense_ffn=80,
                       dtype="bf16", max_ctx=64)
    w = synth.make_weights(cfg, seed=25)
    w["l1.router"] = _bf16_bits(decode_weight(w["l1.router"]) * 16.0)   # peaked routing, no near-ties
    m = Model(cfg, w)
    d, fe = 64, 24
    c = DeepseekV2Config(hidden_size=d, num_experts=16, num_experts_per_tok=4, n_shared_experts=2,
                         moe_intermediate_size=fe, routed_scaling_factor=1.0, topk_method="greedy",
                         hidden_act="silu", mlp_bias=False)
    blk = DeepseekV2Moe(c).double()
    t = _torch_w
    with torch.no_grad():
        blk.gate.weight.copy_(t(w["l1.router"]))
        blk.experts.gate_up_proj.copy_(torch.cat([t(w["l1.exp_gate"]), t(w["l1.exp_up"])], dim=1))
        blk.experts.down_proj.copy_(t(w["l1.exp_down"]))
        blk.shared_experts.gate_proj.weight.copy_(t(w["l1.sh_gate"]).reshape(2 * fe, d))
        blk.shared_experts.up_proj.weight.copy_(t(w["l1.sh_up"]).reshape(2 * fe, d))
        blk.shared_experts.down_proj.weight.copy_(torch.cat([t(w["l1.sh_down"][0]), t(w["l1.sh_down"][1])], dim=1))
    blk.shared_experts.down_proj.register_forward_pre_hook(lambda mod, args: (_rne_t(args[0]),))
    x = _rne_bf16(np.random.default_rng(26).standard_normal((7, d)))
    linear = torch.nn.functional.linear

    def rounded_down(inp, weight, bias=None):
        # the routed experts' down projections are the only [d, fe] products
        if tuple(weight.shape) == (d, fe):
            inp = _rne_t(inp)
        return linear(inp, weight, bias)

    torch.nn.functional.linear = rounded_down
    try:
        with torch.no_grad():
            ref = blk(torch.from_numpy(x)[None])[0].numpy()
    finally:
        torch.nn.functional.linear = linear
    for dedup in (False, True):
        np.testing.assert_allclose(m.moe_ffn(1, x, dedup=dedup), ref, rtol=2e-5, atol=2e-6)
    # the activation rounding is visible at this bound
    m32 = Model(dict(cfg, dtype="f32"), w)
    assert np.max(np.abs(m32.moe_ffn(1, x) - ref)) > 1e-4 * np.max(np.abs(ref))


def test_bf16_storage_points_hold_bf16_values():
    """Every operand the oracle declares stored is exactly a bf16 value: each
    GEMM input (normed inputs, attention output, SwiGLU activation, MoE rows,
    feature concat), q after the rotary embedding, the K/V cache entries
    read by attention and the features."""
    seen = {"lin": 0, "attend": 0}

    def is_bf16(a):
        return np.array_equal(_rne_bf16(a), a)

    class Probe(Model):
        def lin(self, x, W):
            assert is_bf16(x), "GEMM input not stored as bf16"
            seen["lin"] += 1
            return super().lin(x, W)

        def attend(self, q, Kc, Vc, pos):
            assert is_bf16(q) and is_bf16(Kc) and is_bf16(Vc), "q or K/V not stored as bf16"
            seen["attend"] += 1
            return super().attend(q, Kc, Vc, pos)

    cfg = synth.micro_config(n_layers=3, feat_layers=(0, 2), dtype="bf16")
    w = _bf16_model(cfg, seed=27)
    m = Probe(cfg, w)
    cache = Cache(cfg)
    toks = synth.make_tokens(cfg["vocab"], 10, seed=27, stream=3)
    m.forward(toks[:7], 0, cache)
    m.forward(toks[7:], 7, cache)
    assert is_bf16(m.features)
    for l in range(cfg["n_layers"]):
        assert is_bf16(cache.K[l]) and is_bf16(cache.V[l])
    # per forward: 7 products per layer (q, k, v, o, gate, up, down), head, fc
    assert seen["attend"] == 2 * 3 and seen["lin"] == 2 * (3 * 7 + 1 + 1)
    mcfg = synth.config("dsv2-lite", n_layers=2, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                        vocab=96, n_experts=8, top_k=2, n_shared=1, expert_ffn=24, dense_ffn=80,
                        dtype="bf16", max_ctx=32)
    mm = Probe(mcfg, synth.make_weights(mcfg, seed=28))
    for dedup in (False, True):
        mm.forward(synth.make_tokens(96, 5, seed=28, stream=4), 0, Cache(mcfg), dedup=dedup)
