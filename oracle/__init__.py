"""The oracle: a plain, slow CPU implementation of the greedy self-speculative
decode step, written from the pages that describe the method.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP library (no kernels, headers, tables or helpers) and never imports it;
the only module both sides use is ``synth`` (seeded random inputs).

Contents
--------
``skip.py``   the layer-skip draft's skip set (MLX layer-skip blog, "Code").
``accept.py`` greedy longest-prefix accept (mlx-dflash README, "Architecture";
              LayerSkip summary, 4.3.2).
``model.py``  the decoder, greedy decode, shared-cache self-speculation,
              MoE expert FFN (per-slot and deduplicated), feature tap.
``kselect.py`` draft length from measured step times under geometric
              acceptance (speculative decoding for MoE models, abstract).
``knapsack.py`` skip set as a knapsack over measured layer costs with a
              cosine-similarity proxy (MLX layer-skip blog, "Paper -> the idea").
``sampling.py`` speculative sampling: rejection-sampling accept with a
              Philox4x64-10 counter-based generator (LayerSkip summary 4.3.2).

Every floating-point step runs in float64.  For bf16 workloads values are
rounded to bf16 (nearest, ties to even) exactly where the GPU stores bf16:
weights, every GEMM input, the K/V cache entries and q after RoPE.

Parity unpinned: absolute logit values of the random-init models (the pages
print no worked logits); RoPE base, RMSNorm epsilon and the bf16 rounding
points are readings, not page facts.
"""
from .accept import accept, accept_brute
from .skip import skip_layers, skip_mask
from .model import Model, bf16_round, decode_weight
from .kselect import expected_tokens, select_k
from .knapsack import knapsack_skip_brute, layer_cosines
from .sampling import draw, philox4x64_10, probs, spec_cycle, uniform24
