#!/usr/bin/env python3
"""Greedy self-speculative decode benchmark on one MI355X.

Workload (default): Llama-3.1-8B-shaped bf16 decoder with seeded random
weights, a 1024-token uniform-random prompt and 512 greedy tokens; the draft
skips the contiguous middle 20 % of the layers and proposes k=3 tokens per
cycle.  A step is one whole decode (prefill + 512 tokens through
draft/verify/accept cycles).  ``value`` is decode tokens per second after the
prefill (tokens after the first / decode wall time).

Also reported: plain greedy tok/s measured back-to-back in the same process
(speedup = self-spec / greedy), the verify pass's HBM bandwidth (algorithmic
bytes of weights + KV per pass / HIP-event time of the pass), the roofline
of the dominant kernel (the gate/up GEMM at the verify width, timed with HIP
events on the library's stream), the skip x k sweep, and the CPU oracle's
decode rate on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama-8b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def weight_bytes_per_pass(cfg: dict) -> int:
    """Weights one full pass streams: every layer matrix plus the LM head
    (the embedding table is gathered, M rows only)."""
    import synth
    eb = 2 if cfg["dtype"] == "bf16" else 4
    tot = 0
    for name, shape, kind in synth.weight_specs(cfg):
        if name in ("embed", "fc") or kind == "gain":
            continue
        n = 1
        for s in shape:
            n *= s
        tot += n * eb
    return tot


def pass_bytes(cfg: dict, M: int, ctx: float, layers: int | None = None, head: bool = True) -> float:
    """Algorithmic HBM bytes of one pass of M rows ending at context ctx:
    weights once, K and V of positions [0, ctx) read once per layer, K/V of
    the M new rows written, logits written."""
    eb = 2 if cfg["dtype"] == "bf16" else 4
    L = cfg["n_layers"]
    per_layer_w = (weight_bytes_per_pass(cfg) - cfg["vocab"] * cfg["d_model"] * eb) / L
    nl = L if layers is None else layers
    kv_tok = 2 * cfg["n_kv_heads"] * cfg["head_dim"] * eb
    b = nl * (per_layer_w + kv_tok * ctx + kv_tok * M)
    if head:
        b += cfg["vocab"] * cfg["d_model"] * eb + M * cfg["vocab"] * 4
    return b


def speedup_frame(k: int, c_d: float, alpha: float, t_draft_ms: float, t_verify_ms: float,
                  t_base_ms: float) -> dict:
    """Expected-speedup frame of a cycle of k draft steps and one verify (time
    per pass = bytes / bandwidth + fixed time, MoE speculative decoding
    abstract; geometric acceptance): a cycle yields sum_{i<=k} alpha^i tokens
    in k draft steps + one verify.  Ceiling (every draft accepted) from the
    draft/full byte ratio c_d: (k + 1) / (k c_d + 1); break-even: the
    smallest alpha with sum_{i<=k} alpha^i >= k c_d + 1; prediction from the
    measured step times against a plain decode step of t_base_ms."""
    e_tok = sum(alpha ** i for i in range(k + 1))
    lo, hi = 0.0, 1.0
    for _ in range(60):
        mid = (lo + hi) / 2
        if sum(mid ** i for i in range(k + 1)) >= k * c_d + 1:
            hi = mid
        else:
            lo = mid
    return {"draft_byte_ratio": round(c_d, 4),
            "ceiling_alpha1": round((k + 1) / (k * c_d + 1), 4),
            "break_even_alpha": round(hi, 4),
            "alpha": round(alpha, 4),
            "predicted_speedup": round(e_tok / ((k * t_draft_ms + t_verify_ms) / t_base_ms), 4),
            "measured_speedup": None}


def _weights_progress(frac: float) -> None:
    log(f"weights {frac:.0%} generated")


def measured_traffic() -> float | None:
    """HBM bytes per launch of the gate/up GEMM from the committed hardware-
    counter summary, or None when the kernel sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_swiglu_llama8b_traffic.txt")
    try:
        txt = open(path).read()
    except OSError:
        return None
    csrc = os.path.join(ROOT, "self_speculative_decoding_amd", "csrc")
    sha = hashlib.sha256(open(os.path.join(csrc, "gemm.hip"), "rb").read() +
                         open(os.path.join(csrc, "device.h"), "rb").read()).hexdigest()
    rec_sha = nbytes = None
    for line in txt.splitlines():
        if line.startswith("kernel source sha256"):
            rec_sha = line.split(":")[-1].strip()
        if line.startswith("counter bytes per launch:"):
            nbytes = float(line.split(":")[1].split()[0])
    return nbytes if rec_sha == sha else None


def cpu_baseline(cfg, weights, prompt, budget_s: float) -> dict:
    """The oracle (float64 CPU decoder) timed on this host at the workload's
    own context: it prefills the workload's prompt itself (not timed), then
    greedy decode steps at context len(prompt), len(prompt)+1, ... are timed
    until about budget_s seconds of decode work (a bounded sample)."""
    import numpy as np
    from oracle import Model
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    log("cpu baseline: building the oracle model")
    m = Model(cfg, weights)
    P = len(prompt)
    t0 = time.perf_counter()
    cache, n, last = m.prefill(prompt)
    t_pre = time.perf_counter() - t0
    log(f"cpu baseline: oracle prefill of {P} tokens took {t_pre:.1f}s")
    tok = int(np.argmax(last))
    t0 = time.perf_counter()
    steps = 0
    while True:
        lg = m.forward([tok], n, cache)[0]
        n += 1
        steps += 1
        tok = int(np.argmax(lg))
        el = time.perf_counter() - t0
        log(f"cpu baseline: decode step {steps} at {el:.1f}s")
        if el >= budget_s or steps >= 64:
            break
    del m, cache
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": steps / el, "unit": "tok/s", "cores": int(cores), "kind": "oracle",
            "host": {"nproc": os.cpu_count(), "cpu": cpu_model},
            "sample": f"{steps} float64 greedy decode steps at context {P}-{P + steps - 1}, after the oracle's "
                      f"own prefill of the workload's {P}-token prompt ({t_pre:.0f} s, not timed); the sample "
                      f"is bounded to about {budget_s:.0f} s of decode work, so it holds fewer steps than a "
                      f"full 16-step sample would"}


def bench_pmc_probe(args) -> int:
    """Kernel sequence for `rocprofv3 --pmc` runs: 3 plain copies of 128 MiB
    (counter calibration), then 24 gate/up GEMM launches at m = 4 over the
    layers of a 4-layer model with the headline widths (940 MB of weights, more
    than the on-die caches hold), 3 read probes of the 1.05 GB LM head, and 24
    launches each of the QKV, o and down GEMMs at m = 4 (the other decode
    GEMMs, cycling over the same layers)."""
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = synth.config("llama-8b", n_layers=4)
    w = synth.make_weights(cfg, progress=_weights_progress)
    eng = Engine(make_cfg(cfg, max_block=6, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    eng.prefill(synth.make_prompt(cfg)[:64])
    res = {"copy_probe_us": eng.time_op("copy_probe", 0, 128, 3),
           "gate_up_m4_us": eng.time_op("gate_up", 0, 4, 24),
           "read_probe_us": eng.time_op("read_probe", 0, 4, 3)}
    for op in ("qkv", "o", "down"):
        res[op + "_m4_us"] = eng.time_op(op, 0, 4, 24)
    eng.close()
    res["copy_bytes"] = 128 << 20
    res["gate_up_bytes"] = 2 * cfg["ffn_dim"] * cfg["d_model"] * 2
    res["read_probe_gbs"] = round(cfg["vocab"] * cfg["d_model"] * 2 / res["read_probe_us"] / 1e3, 1)
    print(json.dumps(res), flush=True)
    return 0


def bench_attn_pmc_probe(args) -> int:
    """Kernel sequence for `rocprofv3 --pmc` runs on the decode attention:
    3 plain copies of 128 MiB (counter calibration), then the 8B-shaped
    model (4 layers, headline widths) after a 1024-token prompt, 24 attention
    launches at m = 4 (the k = 3 verify) and then 24 at m = 1, cycling over
    the layers.  Prints the K/V bytes each launch reads."""
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = synth.config("llama-8b", n_layers=4)
    w = synth.make_weights(cfg, progress=_weights_progress)
    eng = Engine(make_cfg(cfg, max_block=6, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    eng.prefill(synth.make_prompt(cfg))
    ctx = eng.context_length
    res = {"copy_probe_us": eng.time_op("copy_probe", 0, 128, 3),
           "attention_m4_us": eng.time_op("attention", 0, 4, 24),
           "attention_m1_us": eng.time_op("attention", 0, 1, 24)}
    eng.close()
    kv = lambda m: cfg["n_kv_heads"] * (ctx + m) * cfg["head_dim"] * 2 * 2
    res.update({"copy_bytes": 128 << 20, "context": ctx, "kv_bytes_m4": kv(4), "kv_bytes_m1": kv(1)})
    print(json.dumps(res), flush=True)
    return 0


def bench_trace_verify(args) -> int:
    """Kernel sequence for `rocprofv3 --kernel-trace`: the workload's model
    after its full prompt, then groups of 12 verify passes (host blocks of
    random tokens, each followed by the accept): llama-8b 4, 6 and 1 rows (the
    k = 3 and k = 5 cycles and plain decoding), qwen3-4b 4 and 1, qwen3-8b 16
    and 1, dsv2-lite 8 and 1 rows per-slot then deduplicated (synthetic
    routing).  Prints the mean verify time per group."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    widths = {"llama-8b": (4, 6, 1), "qwen3-4b": (4, 1), "qwen3-8b": (16, 1), "dsv2-lite": (8, 1)}[args.workload]
    cfg = synth.config(args.workload)
    w = synth.make_weights(cfg, progress=_weights_progress)
    eng = Engine(make_cfg(cfg, max_block=17, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    del w
    moe = cfg["n_experts"] > 0
    prompt = synth.make_prompt(cfg)
    toks = synth.make_tokens(cfg["vocab"], 400, seed=1, stream=5)
    res, i = {}, 0
    for mode in ((0, 1) if moe else (None,)):
        if moe:
            eng.set_moe_dedup(mode)
            eng.set_routing(None)
        eng.reset()
        eng.prefill(prompt)
        for m in widths:
            if moe:
                eng.set_routing(synth.make_routing_trace(cfg["n_layers"], m, cfg["n_experts"], cfg["top_k"], seed=0,
                                                         stream=m))
            ms = []
            for _ in range(12):
                st0 = eng.stats()
                eng.verify([int(t) for t in toks[i:i + m]])
                ms.append(eng.stats()["t_verify_ms"] - st0["t_verify_ms"])
                eng.accept()
                i = (i + m) % 380
            key = f"verify_m{m}_ms" + ("" if not moe else ("_dedup" if mode else "_per_slot"))
            res[key] = round(float(np.mean(ms[1:])), 4)
            log(f"{key}: {res[key]} ms, context {eng.context_length}")
    eng.close()
    print(json.dumps(res), flush=True)
    return 0


def bench_prefill(args) -> int:
    """Prefill (time to the first token) of the 1024-token prompt on the
    8B-shaped model (--prefill-layers of its 32 layers) in 64- and 256-row
    chunks: best of --steps prefills each, wall time including the first
    token's read-back.  Outside the decode rate; also the kernel sequence
    for counter runs of the prefill GEMMs."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = synth.config("llama-8b", n_layers=args.prefill_layers)
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    rows = {}
    for chunk in (64, 256):
        eng = Engine(make_cfg(cfg, max_block=4, prefill_chunk=chunk), [w[n] for n, _, _ in synth.weight_specs(cfg)])
        ts = []
        for _ in range(max(1, args.steps)):
            eng.reset()
            t = time.perf_counter()
            eng.prefill(prompt)
            ts.append(time.perf_counter() - t)
        eng.close()
        rows[f"chunk_{chunk}_ms"] = round(min(ts) * 1e3, 2)
        log(f"prefill chunk {chunk}: {rows[f'chunk_{chunk}_ms']} ms")
    flops = 2.0 * len(prompt) * sum(int(np.prod(sh)) for n, sh, kind in synth.weight_specs(cfg)
                                    if kind == "mat" and n not in ("embed", "lm_head"))
    line = {"metric": "prefill ms (time to first token), 8B-shaped bf16", "value": rows["chunk_256_ms"], "unit": "ms",
            "n_gpus": 1, "higher_is_better": False, "dtype": "bf16", "data": "synthetic", "vs_baseline": None,
            "config": {"workload": f"llama-8b-shaped bf16 random-init, {cfg['n_layers']} layers, "
                                   f"{len(prompt)}-token prompt, 64- and 256-row chunks"},
            "by_chunk": rows, "gemm_tflops_at_256": round(flops / (rows["chunk_256_ms"] * 1e-3) / 1e12, 1)}
    print(json.dumps(line), flush=True)
    return 0


def bench_moe_pmc_probe(args) -> int:
    """Kernel sequence for `rocprofv3 --pmc` runs on the MoE expert operation:
    3 plain copies of 128 MiB (counter calibration), then the expert op of
    every MoE layer of the DeepSeek-V2-Lite-shaped model twice over at n = 8
    rows with the synthetic routing trace, per-slot (--moe-dedup 0) or
    deduplicated (1).  Prints the requested expert bytes per layer op."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = dict(synth.config("dsv2-lite"), max_ctx=4096)   # room for a 128 MiB copy in the partial buffer
    L, E, K, n = cfg["n_layers"], cfg["n_experts"], cfg["top_k"], 8
    nd = cfg["n_dense_layers"]
    eb = cfg["expert_ffn"] * cfg["d_model"] * 3 * 2
    assert (cfg["max_ctx"] // 64) * 256 * cfg["n_q_heads"] * cfg["head_dim"] * 4 >= 128 << 20
    w = synth.make_weights(cfg, progress=_weights_progress)
    eng = Engine(make_cfg(cfg, max_block=9, prefill_chunk=256), [w[n_] for n_, _, _ in synth.weight_specs(cfg)])
    del w
    eng.prefill(synth.make_prompt(cfg)[:64])
    trace = synth.make_routing_trace(L, n, E, K, seed=0, stream=n)
    eng.set_moe_dedup(args.moe_dedup)
    eng.set_routing(trace)
    unions = [len(set(trace[l].reshape(-1).tolist())) for l in range(nd, L)]
    res = {"copy_probe_us": eng.time_op("copy_probe", 0, 128, 3),
           "moe_us": eng.time_op("moe", nd, n, 2 * (L - nd))}
    eng.close()
    routed = K * n if args.moe_dedup == 0 else float(np.mean(unions))
    res.update({"mode": "dedup" if args.moe_dedup else "per_slot", "n": n, "copy_bytes": 128 << 20,
                "expert_bytes": eb, "requested_bytes_per_layer": (routed + cfg["n_shared"]) * eb,
                "mean_union": float(np.mean(unions)), "layer_ops": 2 * (L - nd)})
    print(json.dumps(res), flush=True)
    return 0


def bench_verify_blocks(args) -> int:
    """Qwen3-8B-shaped target verifying 16-token blocks at context 2048 with the
    five-layer feature tap + fc on; drafts carry a geometric(p) correct prefix.
    Reports the verify pass time, its HBM bandwidth and tokens per verify."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = synth.config("qwen3-8b")
    B, P = cfg["block"], cfg["prompt_len"]
    log("qwen3-8b: generating weights")
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    eng = Engine(make_cfg(cfg, max_block=B, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    n_cont = 400
    true, _ = eng.generate(prompt, n_cont)
    log("greedy continuation ready")
    fc_bytes = cfg["d_model"] * len(cfg["feat_layers"]) * cfg["d_model"] * 2
    res = []
    for p in cfg["geo_p"]:
        eng.reset()
        eng.prefill(prompt)
        pos, a_list, ms = 0, [], []
        s = 0
        while pos + B < n_cont and s < args.blocks:
            d, m = synth.make_geometric_block(np.array(true[pos + 1:pos + B], np.int32), cfg["vocab"], p, B,
                                              seed=0, stream=1000 * int(p * 10) + s)
            st0 = eng.stats()
            eng.verify([true[pos]] + list(d))
            st1 = eng.stats()
            a, _ = eng.accept()
            if a != m:
                raise RuntimeError(f"accepted {a} but the block had a correct prefix of {m}")
            ms.append(st1["t_verify_ms"] - st0["t_verify_ms"])
            a_list.append(a)
            pos += a + 1
            s += 1
        ms = ms[1:] if len(ms) > 1 else ms        # first replay captures the graph
        v_ms = float(np.mean(ms))
        vb = pass_bytes(cfg, B, P + pos / 2) + fc_bytes
        res.append({"p": p, "blocks": s, "tokens_per_verify": round(float(np.mean(a_list)) + 1, 3),
                    "expected_tokens_per_verify": round((1 - p ** B) / (1 - p), 3),
                    "verify_ms": round(v_ms, 4), "gbs": round(vb / v_ms / 1e6, 1),
                    "frac": round(vb / v_ms / 1e6 / PEAK_HBM_GBS, 4),
                    "tok_s": round((float(np.mean(a_list)) + 1) / v_ms * 1e3, 1)})
        log(f"p={p}: {res[-1]}")
    ops = {}
    for op in ("gate_up", "down", "qkv", "o", "attention", "lm_head"):
        for m in (1, B):
            ops[f"{op}_m{m}"] = round(eng.time_op(op, 0, m, 30), 2)
    eng.close()
    line = {"metric": "verify-pass HBM GB/s (% of peak), 16-token blocks, Qwen3-8B-shaped bf16 + feature tap",
            "value": res[-1]["gbs"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16",
            "data": "synthetic", "vs_baseline": None,
            "config": {"workload": f"qwen3-8b-shaped bf16 random-init target, {P}-token prompt, verify blocks of {B} "
                                   f"with geometric correct prefix, feature tap layers {list(cfg['feat_layers'])} + fc"},
            "by_p": res, "ops_us": ops}
    print(json.dumps(line), flush=True)
    return 0


def bench_kselect(args) -> int:
    """Draft length from measured step times: fit t_draft, t_verify(k+1) and the
    per-cycle overhead on the 8B-shaped model, predict k*(alpha) and the rate
    for geometric acceptance alpha, then measure cycles of real draft passes
    followed by a verify of a block whose correct prefix is geometric(alpha)
    (so the acceptance is controlled while every pass runs in full)."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg, skip_mask, select_k
    cfg = synth.config("llama-8b")
    KMAX, V = 8, cfg["vocab"]
    frac = args.skip if args.skip is not None else cfg["skip_frac"]
    log("kselect: generating weights")
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    eng = Engine(make_cfg(cfg, max_block=KMAX + 1, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    del w
    mask = skip_mask(cfg["n_layers"], frac)
    true, _ = eng.generate(prompt, 40 * (KMAX + 1) + 8)
    _, st = eng.generate(prompt, 256, mask, 3)          # warm graphs; fit draft step and cycle overhead
    _, st = eng.generate(prompt, 256, mask, 3)
    t_draft = st["t_draft_ms"] / st["drafted"]
    t_cycle = (st["t_decode_ms"] - st["t_draft_ms"] - st["t_verify_ms"]) / st["cycles"]
    tv = []
    for k in range(KMAX + 1):
        ms = []
        for rep in range(4):
            eng.reset()
            eng.prefill(prompt)
            s0 = eng.stats()
            eng.verify(true[:k + 1])
            ms.append(eng.stats()["t_verify_ms"] - s0["t_verify_ms"])
            eng.accept()
        tv.append(float(np.median(ms[1:])))
    log(f"fitted: t_draft {t_draft:.3f} ms, t_cycle {t_cycle:.3f} ms, t_verify {[round(x, 3) for x in tv]}")
    rows = []
    for alpha in (0.5, 0.7, 0.8, 0.9, 0.95):
        k_pred, _ = select_k(tv, t_draft, t_cycle, alpha)
        meas = []
        for k in range(KMAX + 1):
            eng.reset()
            eng.prefill(prompt)
            pos, toks, cyc, gpu_ms, stream = 0, 0, 0, 0.0, 0
            s0 = eng.stats()
            while pos + k + 2 < len(true) and cyc < 40:
                if k > 0:
                    eng.draft(mask, k)                   # the real draft passes; tokens replaced below
                d, m = synth.make_geometric_block(np.array(true[pos + 1:pos + k + 1], np.int32), V, alpha,
                                                  k + 1, seed=1, stream=stream) if k > 0 else (np.zeros(0, np.int32), 0)
                stream += 1
                eng.verify([true[pos]] + [int(x) for x in d])
                a, em = eng.accept()
                if a != m or em != true[pos + 1:pos + a + 2]:
                    raise RuntimeError(f"accepted {a} of a prefix of {m}")
                pos += a + 1
                toks += a + 1
                cyc += 1
            s1 = eng.stats()
            gpu_ms = (s1["t_draft_ms"] - s0["t_draft_ms"]) + (s1["t_verify_ms"] - s0["t_verify_ms"]) + cyc * t_cycle
            e_k = sum(alpha ** i for i in range(k + 1))
            meas.append({"k": k, "tokens_per_cycle": round(toks / cyc, 3), "expected": round(e_k, 3),
                         "measured_tok_s": round(toks / gpu_ms * 1e3, 1),
                         "predicted_tok_s": round(e_k / (k * t_draft + tv[k] + t_cycle) * 1e3, 1)})
        k_meas = max(meas, key=lambda r: r["measured_tok_s"])["k"]
        rows.append({"alpha": alpha, "k_pred": k_pred, "k_measured": k_meas, "by_k": meas})
        log(f"alpha {alpha}: k* predicted {k_pred}, measured {k_meas}")
    eng.close()
    mono = all(rows[i]["k_pred"] <= rows[i + 1]["k_pred"] for i in range(len(rows) - 1))
    line = {"metric": "draft length k*(alpha) from fitted step times, predicted vs measured, 8B-shaped bf16",
            "value": sum(r["k_pred"] == r["k_measured"] for r in rows) / len(rows), "unit": "fraction of alphas where k* agrees",
            "n_gpus": 1, "higher_is_better": True, "dtype": "bf16", "data": "synthetic", "vs_baseline": None,
            "config": {"workload": f"llama-8b-shaped bf16 random-init, {len(prompt)}-token prompt, middle skip "
                                   f"{frac:.0%}, k = 0..{KMAX}, verify blocks with geometric(alpha) correct prefix"},
            "fit": {"t_draft_ms": round(t_draft, 4), "t_cycle_ms": round(t_cycle, 4), "t_verify_ms": [round(x, 4) for x in tv]},
            "k_pred_monotone": mono, "by_alpha": rows}
    print(json.dumps(line), flush=True)
    return 0


def bench_kvq(args) -> int:
    """LayerSkip early-exit draft (tail mask: the first E layers + the shared
    head) with and without exit-state reuse in the verify (SSD_OPT_KVQ), on the
    8B-shaped model: verify and draft step times, decode tok/s, losslessness;
    plus the early-exit inference rate (one E-layer pass per token)."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = synth.config("llama-8b")
    L, k = cfg["n_layers"], args.k if args.k is not None else 3
    n_new = args.n_new or 256
    log("kvq: generating weights")
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    eng = Engine(make_cfg(cfg, max_block=k + 1, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    del w
    base, _ = eng.generate(prompt, n_new)
    _, stb = eng.generate(prompt, n_new)
    base_tps = (n_new - 1) / stb["t_decode_ms"] * 1e3
    rows = []
    for E in (8, 12, 16, 24):
        mask = np.zeros(L, np.uint8)
        mask[E:] = 1
        r = {"E": E}
        for mode, on in (("full_verify", False), ("kvq_reuse", True)):
            eng.set_kvq(on)
            eng.generate(prompt, n_new, mask, k)                 # capture graphs
            out, st = eng.generate(prompt, n_new, mask, k)
            r[mode] = {"verify_ms": round(st["t_verify_ms"] / st["verify_passes"], 4),
                       "draft_step_ms": round(st["t_draft_ms"] / st["drafted"], 4),
                       "tok_s": round((n_new - 1) / st["t_decode_ms"] * 1e3, 2),
                       "acceptance": round(st["accepted"] / st["drafted"], 4),
                       "lossless": out == base}
        eng.set_kvq(False)
        r["early_exit_tok_s"] = round(1e3 / r["full_verify"]["draft_step_ms"], 1)
        r["verify_saving"] = round(1 - r["kvq_reuse"]["verify_ms"] / r["full_verify"]["verify_ms"], 4)
        rows.append(r)
        log(f"E={E}: {r}")
    eng.close()
    line = {"metric": "early-exit draft: verify ms with vs without exit-state reuse, 8B-shaped bf16",
            "value": rows[1]["kvq_reuse"]["verify_ms"], "unit": "ms", "n_gpus": 1, "higher_is_better": False,
            "dtype": "bf16", "data": "synthetic", "vs_baseline": None,
            "config": {"workload": f"llama-8b-shaped bf16 random-init, {len(prompt)}-token prompt, {n_new} tokens, "
                                   f"tail masks E in (8, 12, 16, 24), k={k}"},
            "greedy_tok_s": round(base_tps, 2), "by_E": rows}
    print(json.dumps(line), flush=True)
    return 0


def bench_sampling(args) -> int:
    """Speculative sampling on the 8B-shaped model: greedy decoding, plain
    sampling (one pass per token, a Philox draw from softmax(logits / T)) and
    self-speculative sampling (middle-skip draft sampled from its own
    distribution, rejection-sampling accept) at T = 1 and 0.6; tok/s, the
    acceptance rate and the cost per cycle over the greedy cycle."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg, skip_mask
    cfg = synth.config("llama-8b")
    L, k = cfg["n_layers"], args.k if args.k is not None else 3
    frac = args.skip if args.skip is not None else 0.2
    n_new = args.n_new or 256
    log("sampling: generating weights")
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    eng = Engine(make_cfg(cfg, max_block=k + 1, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    del w
    mask = skip_mask(L, frac)

    def run(*a, **kw):
        eng.generate(prompt, n_new, *a, **kw)                    # capture graphs
        out, st = eng.generate(prompt, n_new, *a, **kw)
        r = {"tok_s": round((n_new - 1) / st["t_decode_ms"] * 1e3, 2)}
        if st.get("drafted"):
            r["acceptance"] = round(st["accepted"] / st["drafted"], 4)
            r["cycle_ms"] = round(st["t_decode_ms"] / st["verify_passes"], 4)
        return out, r

    _, greedy = run()
    _, greedy_spec = run(mask, k)
    rows = {"greedy": greedy, "greedy_selfspec": greedy_spec}
    for T in (1.0, 0.6):
        eng.set_sampling(T, 2024)
        _, plain = run(greedy=0)
        out, spec = run(mask, k, greedy=0)
        assert all(0 <= t < cfg["vocab"] for t in out)
        spec["cycle_overhead_vs_greedy_ms"] = round(spec["cycle_ms"] - greedy_spec["cycle_ms"], 4)
        rows[f"T={T}"] = {"plain_sampling": plain, "spec_sampling": spec}
        log(f"T={T}: plain {plain}, spec {spec}")
    eng.close()
    line = {"metric": "self-speculative sampling decode throughput, 8B-shaped bf16",
            "value": rows["T=1.0"]["spec_sampling"]["tok_s"], "unit": "tokens/s", "n_gpus": 1,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic", "vs_baseline": None,
            "config": {"workload": f"llama-8b-shaped bf16 random-init, {len(prompt)}-token prompt, {n_new} tokens, "
                                   f"middle skip {frac}, k={k}"},
            "modes": rows}
    print(json.dumps(line), flush=True)
    return 0


def bench_knapsack(args) -> int:
    """Skip set as a knapsack on the 8B-shaped model: per-layer costs from
    measured op times, per-layer value 1 - cos(input, output) from a traced
    16-row verify pass, budgets matching the middle-skip fractions; compares
    the knapsack mask with the contiguous middle block (acceptance, tok/s)."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg, skip_mask, knapsack_skip
    cfg = synth.config("llama-8b")
    L, k, n_new = cfg["n_layers"], 3, args.n_new or 256
    log("knapsack: generating weights")
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    eng = Engine(make_cfg(cfg, max_block=17, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    del w
    true, _ = eng.generate(prompt, 20)
    eng.set_trace(True)
    eng.reset()
    eng.prefill(prompt)
    eng.verify(true[:16])
    cos = eng.layer_cosines(16)
    eng.set_trace(False)
    eng.reset()
    eng.prefill(prompt)
    # per-layer cost (units of 10 ns): attention block + FFN block at M = 1
    cost = []
    for l in range(L):
        us = sum(eng.time_op(op, l, 1, 20) for op in ("qkv", "attention", "o", "gate_up", "down"))
        cost.append(int(round(us * 100)))
    base, stb = eng.generate(prompt, n_new)
    base_tps = (n_new - 1) / stb["t_decode_ms"] * 1e3
    value = 1.0 - cos
    rows = []
    for frac in (0.1, 0.2, 0.3, 0.4, 0.5):
        mid = skip_mask(L, frac)
        budget = int(sum(c for c, m in zip(cost, mid) if not m))
        ks_mask, kept = knapsack_skip(cost, value, budget)
        r = {"skip_frac": frac, "budget_us": round(budget / 100, 2),
             "middle": [int(i) for i in np.nonzero(mid)[0]], "knapsack": [int(i) for i in np.nonzero(ks_mask)[0]]}
        for name, m in (("middle", mid), ("knapsack", ks_mask)):
            out, st = eng.generate(prompt, n_new, m, k)
            r[name + "_run"] = {"acceptance": round(st["accepted"] / st["drafted"], 4),
                                "tok_s": round((n_new - 1) / st["t_decode_ms"] * 1e3, 2),
                                "draft_step_ms": round(st["t_draft_ms"] / st["drafted"], 4),
                                "proxy_kept_value": round(float(sum(v for v, mm in zip(value, m) if not mm)), 6),
                                "lossless": out == base}
        rows.append(r)
        log(f"skip {frac}: middle {r['middle_run']} knapsack {r['knapsack_run']} skips {r['knapsack']}")
    eng.close()
    line = {"metric": "knapsack skip set vs middle block: draft acceptance at equal layer-time budget, 8B-shaped bf16",
            "value": rows[1]["knapsack_run"]["acceptance"], "unit": "acceptance (20 % budget)", "n_gpus": 1,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic", "vs_baseline": None,
            "config": {"workload": f"llama-8b-shaped bf16 random-init, {len(prompt)}-token prompt, {n_new} tokens, k={k}"},
            "greedy_tok_s": round(base_tps, 2), "layer_cos": [round(float(x), 6) for x in cos],
            "layer_cost_us": [c / 100 for c in cost], "by_budget": rows}
    print(json.dumps(line), flush=True)
    return 0


def bench_moe(args) -> int:
    """DeepSeek-V2-Lite-shaped MoE verify passes of n = 1..8 tokens with the
    synthetic routing trace: per-slot vs deduplicated expert reads, whole pass
    and one layer's expert operation alone (fitted bandwidths, u(n), r(n))."""
    import numpy as np
    import synth
    from self_speculative_decoding_amd import Engine, make_cfg
    cfg = synth.config("dsv2-lite")
    L, E, K = cfg["n_layers"], cfg["n_experts"], cfg["top_k"]
    eb = cfg["expert_ffn"] * cfg["d_model"] * 3 * 2             # one expert's gate/up/down bytes
    log("dsv2-lite: generating weights")
    w = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    eng = Engine(make_cfg(cfg, max_block=9, prefill_chunk=256), [w[n] for n, _, _ in synth.weight_specs(cfg)])
    rows = []
    for n in cfg["pass_sizes"]:
        trace = synth.make_routing_trace(L, n, E, K, seed=0, stream=n)
        ubar = float(np.mean([len(set(trace[l].reshape(-1).tolist())) for l in range(cfg["n_dense_layers"], L)])) / (K * n)
        r = {"n": n, "u_bar": round(ubar, 4)}
        for mode, dedup in (("per_slot", 0), ("dedup", 1)):
            eng.set_moe_dedup(dedup)
            eng.set_routing(None)
            eng.reset()
            eng.prefill(prompt)
            eng.set_routing(trace)
            block = list(synth.make_tokens(cfg["vocab"], n, seed=0, stream=100 + n))
            times = []
            for it in range(args.passes):
                st0 = eng.stats()
                eng.verify(block)
                st1 = eng.stats()
                eng.accept()
                times.append(st1["t_verify_ms"] - st0["t_verify_ms"])
            r[f"{mode}_pass_ms"] = round(float(np.mean(times[1:])), 4)
            us = eng.time_op("moe", cfg["n_dense_layers"], n, 52)
            unions = eng.read_union()
            req = (K * n if dedup == 0 else ubar * K * n) * eb + cfg["n_shared"] * eb
            r[f"{mode}_layer_us"] = round(us, 2)
            r[f"{mode}_layer_gbs"] = round(req / us / 1e3, 1)
        r["r"] = round(r["dedup_layer_gbs"] / r["per_slot_layer_gbs"], 4)
        rows.append(r)
        log(f"n={n}: {r}")
    eng.close()
    pred = next((r["n"] for r in rows if r["u_bar"] < r["r"]), None)
    meas = next((r["n"] for r in rows if r["dedup_pass_ms"] < r["per_slot_pass_ms"]), None)
    line = {"metric": "MoE verify pass ms, per-slot vs deduplicated expert reads, DeepSeek-V2-Lite-shaped bf16",
            "value": rows[-1]["dedup_pass_ms"], "unit": "ms", "n_gpus": 1, "higher_is_better": False,
            "dtype": "bf16", "data": "synthetic", "vs_baseline": None,
            "config": {"workload": "dsv2-lite-shaped bf16 MoE (27 layers, 64 experts top-6 + 2 shared, expert "
                                   "FFN 1408), verify passes of n=1..8 tokens, synthetic routing trace "
                                   "(reuse of the previous token's expert with probability 0.5)"},
            "predicted_crossover_n": pred, "measured_crossover_n": meas, "by_n": rows}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama-8b",
                    choices=["llama-8b", "qwen3-4b", "tiny", "qwen3-8b", "dsv2-lite"])
    ap.add_argument("--skip", type=float, default=None, help="draft skip fraction (default: workload's)")
    ap.add_argument("--k", type=int, default=None, help="draft length (default: workload's)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--n-new", type=int, default=None, help="tokens per decode (default: workload's)")
    ap.add_argument("--blocks", type=int, default=40, help="verify blocks per p (qwen3-8b)")
    ap.add_argument("--passes", type=int, default=12, help="verify passes per n and mode (dsv2-lite)")
    ap.add_argument("--knapsack", action="store_true",
                    help="knapsack skip set (cosine proxy, measured layer costs) vs the middle block")
    ap.add_argument("--kvq", action="store_true",
                    help="early-exit draft with vs without exit-state reuse in the verify")
    ap.add_argument("--sampling", action="store_true",
                    help="speculative sampling vs greedy and plain sampling (8B shape)")
    ap.add_argument("--kselect", action="store_true",
                    help="draft length from fitted step times: predicted vs measured k*(alpha)")
    ap.add_argument("--prefill", action="store_true", help="prefill time of the 1024-token prompt (8B shape)")
    ap.add_argument("--prefill-layers", type=int, default=32)
    ap.add_argument("--moe-pmc-probe", action="store_true",
                    help="MoE expert op kernel sequence for rocprofv3 --pmc (with --moe-dedup)")
    ap.add_argument("--moe-dedup", type=int, default=0, choices=(0, 1))
    ap.add_argument("--attn-pmc-probe", action="store_true",
                    help="kernel sequence for rocprofv3 --pmc on the decode attention (8B shape, context 1024)")
    ap.add_argument("--trace-verify", action="store_true",
                    help="kernel sequence for rocprofv3 --kernel-trace: groups of replayed verify graphs after "
                         "the workload's prompt (see bench_trace_verify)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short fixed kernel sequence for hardware-counter runs (copy probe, read probe, "
                         "gate/up GEMM at m=4 on a 4-layer model of the headline widths)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the decode path has no multi-GPU mode "
              "(pass --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from self_speculative_decoding_amd import Engine, make_cfg, skip_mask

    if args.trace_verify:
        return bench_trace_verify(args)
    if args.pmc_probe:
        return bench_pmc_probe(args)
    if args.moe_pmc_probe:
        return bench_moe_pmc_probe(args)
    if args.attn_pmc_probe:
        return bench_attn_pmc_probe(args)
    if args.prefill:
        return bench_prefill(args)
    if args.workload == "qwen3-8b":
        return bench_verify_blocks(args)
    if args.workload == "dsv2-lite":
        return bench_moe(args)
    if args.kselect:
        return bench_kselect(args)
    if args.kvq:
        return bench_kvq(args)
    if args.knapsack:
        return bench_knapsack(args)
    if args.sampling:
        return bench_sampling(args)
    cfg = synth.config(args.workload)
    frac = args.skip if args.skip is not None else cfg.get("skip_frac", 0.5)
    k = args.k if args.k is not None else cfg["k"]
    ks = list(cfg.get("ks", (k,)))
    fracs = list(cfg.get("skip_fracs", (frac,)))
    n_new, P = args.n_new or cfg["n_new"], cfg["prompt_len"]
    log(f"workload {args.workload}: generating weights")
    t = time.perf_counter()
    weights = synth.make_weights(cfg, progress=_weights_progress)
    prompt = synth.make_prompt(cfg)
    log(f"weights ready in {time.perf_counter() - t:.1f}s; uploading")
    eng = Engine(make_cfg(cfg, max_block=max(ks + [k]) + 1, prefill_chunk=256),
                 [weights[n] for n, _, _ in synth.weight_specs(cfg)])
    mask = skip_mask(cfg["n_layers"], frac)
    skipped = [int(i) for i in np.nonzero(mask)[0]]
    log(f"draft skips layers {skipped[0]}..{skipped[-1]} ({len(skipped)} of {cfg['n_layers']}), k={k}")

    for w in range(args.warmup):
        eng.generate(prompt, n_new, mask, k)
        eng.generate(prompt, n_new)
        log(f"warmup {w + 1}/{args.warmup} done")

    # ---- timed region: K self-speculative decodes ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_tps = []
    dec_ms = ver_ms = dr_ms = 0.0
    vpasses = cycles = acc = drafted = 0
    spec_out = None
    for i in range(args.steps):
        out, st = eng.generate(prompt, n_new, mask, k)
        spec_out = out
        dec_ms += st["t_decode_ms"]
        ver_ms += st["t_verify_ms"]
        dr_ms += st["t_draft_ms"]
        vpasses += st["verify_passes"]
        cycles += st["cycles"]
        acc += st["accepted"]
        drafted += st["drafted"]
        step_tps.append((n_new - 1) / st["t_decode_ms"] * 1e3)
        log(f"step {i + 1}/{args.steps}: {(n_new - 1) / st['t_decode_ms'] * 1e3:.1f} tok/s, "
            f"{st['cycles']} cycles, {st['accepted']}/{st['drafted']} drafts accepted")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = float(np.median(step_tps))       # median over the timed decodes
    mean_tps = args.steps * (n_new - 1) / (dec_ms / 1e3)

    # ---- plain greedy, back to back ----
    base_ms = base_pass_ms = 0.0
    base_passes = 0
    base_out = None
    base_steps = []
    for i in range(args.steps):
        out, st = eng.generate(prompt, n_new)
        base_out = out
        base_steps.append((n_new - 1) / st["t_decode_ms"] * 1e3)
        base_ms += st["t_decode_ms"]
        base_pass_ms += st["t_verify_ms"]
        base_passes += st["verify_passes"]
    base_tps = float(np.median(base_steps))
    lossless = spec_out == base_out
    log(f"greedy {base_tps:.1f} tok/s; self-spec {value:.1f} tok/s; lossless={lossless}")

    # ---- verify-pass bandwidth ----
    avg_ctx = P + n_new / 2.0
    vb = pass_bytes(cfg, k + 1, avg_ctx)
    v_ms = ver_ms / max(vpasses, 1)
    v_gbs = vb / (v_ms / 1e3) / 1e9
    bb = pass_bytes(cfg, 1, avg_ctx)
    b_ms = base_pass_ms / max(base_passes, 1)
    b_gbs = bb / (b_ms / 1e3) / 1e9

    # ---- dominant kernel: gate/up GEMM (+SwiGLU) at the verify width ----
    ops = {}
    for op in ("gate_up", "down", "qkv", "o", "attention", "lm_head"):
        for m in (1, k + 1):
            ops[f"{op}_m{m}"] = round(eng.time_op(op, 0, m, 50), 2)
    d, F = cfg["d_model"], cfg["ffn_dim"]
    gu_bytes = 2 * F * d * 2
    gu_us = eng.time_op("gate_up", 0, k + 1, 200)
    roof = {"bound": "hbm", "kernel": "gemm_bf16_kernel<EPI_SWIGLU> (gate/up GEMM + SwiGLU)",
            "m": k + 1, "achieved": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gu_bytes / (gu_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic() if args.workload == "llama-8b" else None,
            "bytes_per_launch": gu_bytes, "avg_us": round(gu_us, 2)}
    log(f"gate/up GEMM m={k + 1}: {gu_us:.1f} us = {roof['achieved']:.0f} GB/s")
    # achievable HBM bandwidth: a plain streaming read of the 1.05 GB LM head
    rp_us = min(eng.time_op("read_probe", 0, 4, 3) for _ in range(3))
    achievable = round(cfg["vocab"] * cfg["d_model"] * 2 / (rp_us * 1e-6) / 1e9, 1)

    # expected-speedup frame: ceiling (all drafts accepted) from byte ratios,
    # and the prediction from measured step times and the measured acceptance
    # under geometric acceptance
    c_d = pass_bytes(cfg, 1, avg_ctx, layers=cfg["n_layers"] - len(skipped)) / bb
    frame = speedup_frame(k, c_d, acc / max(drafted, 1), dr_ms / max(drafted, 1), v_ms, b_ms)

    # ---- skip x k sweep (one decode each) ----
    sweep = []
    if not args.no_sweep and len(fracs) * len(ks) > 1:
        for f in fracs:
            m_ = skip_mask(cfg["n_layers"], f)
            for kk in ks:
                out, st = eng.generate(prompt, n_new, m_, kk)
                tps = (n_new - 1) / (st["t_decode_ms"] / 1e3)
                sweep.append({"skip": f, "k": kk, "tok_s": round(tps, 2), "speedup": round(tps / base_tps, 4),
                              "acceptance": round(st["accepted"] / max(st["drafted"], 1), 4),
                              "tokens_per_cycle": round(st["emitted"] / max(st["cycles"], 1), 3),
                              "verify_ms": round(st["t_verify_ms"] / max(st["verify_passes"], 1), 3),
                              "draft_step_ms": round(st["t_draft_ms"] / max(st["drafted"], 1), 3),
                              "lossless": out == base_out})
                log(f"sweep skip={f} k={kk}: {tps:.1f} tok/s ({tps / base_tps:.3f}x)")
    eng.close()
    del eng
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, weights, prompt, args.cpu_budget)

    skipped_desc = f"{skipped[0]}-{skipped[-1]}"
    line = {
        "metric": "greedy self-spec decode tok/s + verify-pass HBM GB/s (% of peak), 8B-shaped bf16",
        "value": round(value, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 1), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": f"{args.workload}-shaped {cfg['dtype']} random-init decoder, {P}-token uniform "
                               f"prompt, {n_new} greedy tokens, self-spec middle skip {frac:.0%} "
                               f"(layers {skipped_desc}), k={k}",
                   "prompt_len": P, "n_new": n_new, "skip_frac": frac, "k": k, "parallelism": "none"},
        "greedy_tok_s": round(base_tps, 2), "speedup": round(value / base_tps, 4), "lossless": lossless,
        "acceptance": round(acc / max(drafted, 1), 4), "tokens_per_cycle": round(args.steps * (n_new - 1) / max(cycles, 1), 3),
        "verify_pass": {"m": k + 1, "ms": round(v_ms, 4), "bytes": int(vb), "gbs": round(v_gbs, 1),
                        "frac": round(v_gbs / PEAK_HBM_GBS, 4), "avg_ctx": avg_ctx},
        "decode_pass_m1": {"ms": round(b_ms, 4), "bytes": int(bb), "gbs": round(b_gbs, 1),
                           "frac": round(b_gbs / PEAK_HBM_GBS, 4)},
        "draft_step_ms": round(dr_ms / max(drafted, 1), 4),
        "roofline": roof, "achievable_gbs": achievable, "speedup_frame": frame,
        "mean_tok_s": round(mean_tps, 2), "ops_us": ops, "sweep": sweep, "cpu_baseline": cpu,
    }
    frame["measured_speedup"] = round(value / base_tps, 4)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
