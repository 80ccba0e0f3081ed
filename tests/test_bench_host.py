"""bench.py's host-side measurement arithmetic (no GPU): the bytes a draft
step and a verify pass stream, and the expected-speedup frame built on them
(time per pass = bytes / bandwidth + fixed time, MoE speculative decoding
abstract; geometric acceptance)."""
import sys

import numpy as np
import pytest

import synth
from _common import ROOT
from oracle import skip_layers

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _layer_and_head_bytes(cfg):
    """bf16 weight bytes of one layer and of the LM head, from the shapes."""
    d, hd = cfg["d_model"], cfg["head_dim"]
    q, kv, f = cfg["n_q_heads"] * hd, cfg["n_kv_heads"] * hd, cfg["ffn_dim"]
    layer = 2 * (d * (q + 2 * kv) + q * d + 2 * f * d + f * d)
    return layer, 2 * cfg["vocab"] * d


def test_pass_bytes_of_the_8b_shape():
    """436.2 MB per layer, a 1.051 GB head, 15.009 GB of weights per pass,
    plus 4 KiB of K and V per position and layer."""
    cfg = synth.config("llama-8b")
    layer, head = _layer_and_head_bytes(cfg)
    assert layer == 436207616 and head == 1050673152
    assert bench.weight_bytes_per_pass(cfg) == 32 * layer + head
    kv = 2 * cfg["n_kv_heads"] * cfg["head_dim"] * 2
    got = bench.pass_bytes(cfg, 4, 1280)
    want = 32 * (layer + kv * 1280 + kv * 4) + head + 4 * cfg["vocab"] * 4
    assert got == pytest.approx(want, rel=1e-12)


@pytest.mark.parametrize("frac", [0.1, 0.2, 0.3, 0.4, 0.5])
@pytest.mark.parametrize("k", [2, 3, 5])
def test_speedup_frame(frac, k):
    """Draft/full byte ratio from the kept layers; the ceiling equals the
    frame's own prediction at alpha = 1 with byte-proportional step times;
    the break-even alpha is the real root in [0, 1] of
    sum_{i<=k} a^i = k c_d + 1 (numpy.roots) and predicts a speedup of 1."""
    cfg = synth.config("llama-8b")
    layer, head = _layer_and_head_bytes(cfg)
    kept = cfg["n_layers"] - len(skip_layers(cfg["n_layers"], frac))
    c_d = bench.pass_bytes(cfg, 1, 0, layers=kept) / bench.pass_bytes(cfg, 1, 0)
    assert c_d == pytest.approx((kept * layer + head) / (cfg["n_layers"] * layer + head), abs=2e-4)

    t = 2.0   # a full pass, ms; the draft step streams c_d of its bytes
    at1 = bench.speedup_frame(k, c_d, 1.0, c_d * t, t, t)
    assert at1["ceiling_alpha1"] == pytest.approx(at1["predicted_speedup"], abs=2e-4)
    assert at1["ceiling_alpha1"] == pytest.approx((k + 1) / (k * c_d + 1), abs=1e-4)

    coeffs = np.ones(k + 1)
    coeffs[-1] -= k * c_d + 1
    roots = [r.real for r in np.roots(coeffs) if abs(r.imag) < 1e-9 and 0.0 <= r.real <= 1.0]
    assert len(roots) == 1
    be = at1["break_even_alpha"]
    assert be == pytest.approx(roots[0], abs=1e-4)
    at_be = bench.speedup_frame(k, c_d, be, c_d * t, t, t)
    assert at_be["predicted_speedup"] == pytest.approx(1.0, abs=1e-3)
    below = bench.speedup_frame(k, c_d, be - 0.02, c_d * t, t, t)
    assert below["predicted_speedup"] < 1.0


def test_speedup_frame_edges():
    """No acceptance: one token per cycle of k drafts + a verify; k = 0 is
    plain decoding (ceiling 1, break-even 0)."""
    f = bench.speedup_frame(3, 0.8, 0.0, 1.6, 2.0, 2.0)
    assert f["predicted_speedup"] == pytest.approx(1.0 / ((3 * 1.6 + 2.0) / 2.0), abs=1e-4)
    f0 = bench.speedup_frame(0, 0.8, 0.5, 1.6, 2.0, 2.0)
    assert f0["ceiling_alpha1"] == 1.0 and f0["break_even_alpha"] == pytest.approx(0.0, abs=1e-6)
    assert f0["predicted_speedup"] == pytest.approx(1.0)
