"""The decision-matched oracle used by the full-size GPU tests, checked on
the CPU against the plain oracle (tests/_matched.py).

Fed the oracle's own stored values it reproduces the plain oracle exactly;
a stored value one bf16 step off where the oracle's value is not near a
rounding midpoint is counted as a mismatch; the other neighbour of a value
near a midpoint is accepted and then followed."""
import numpy as np

import synth
from oracle import Model
from oracle.model import Cache, bf16_round
from _matched import WINDOW, MatchedModel

NAMES = ["xg_attn", "q", "k", "v", "att", "xg_ffn", "act"]


class Recorder(Model):
    def rn(self, x):
        r = bf16_round(x)
        self.rec.append((x.copy(), r.copy()))
        return r


def _setup():
    cfg = synth.micro_config(n_layers=2, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=256,
                             vocab=128, dtype="bf16")
    w = synth.make_weights(cfg, seed=31)
    toks = synth.make_tokens(cfg["vocab"], 12, seed=31, stream=1)
    rec = Recorder(cfg, w)
    rec.rec = []
    cache = Cache(cfg)
    rec.forward(toks[:8], 0, cache)              # prefix
    rec.rec = []
    ref = rec.forward(toks[8:], 8, cache)
    names = [NAMES[i % 7] for i in range(2 * 7)] + ["xg_head"]
    assert len(rec.rec) == len(names)
    return cfg, w, toks, rec.rec, names, ref


def _run(cfg, w, toks, expect):
    mm = MatchedModel(cfg, w)
    cache = Cache(cfg)
    Model.forward(mm, toks[:8], 0, cache)        # the same prefix, plain rounding (expect empty)
    lg = mm.run(toks[8:], 8, cache, expect)
    return mm, lg


def test_own_values_match_exactly():
    cfg, w, toks, rec, names, ref = _setup()
    mm, lg = _run(cfg, w, toks, [(n, r) for n, (x, r) in zip(names, rec)])
    assert np.array_equal(lg, ref)
    assert all(p.bad == 0 and p.ambiguous == 0 and p.exact == p.n for p in mm.points.values())


def _step(v, sign):
    """The bf16 value one step from v (away from zero for sign > 0)."""
    b = (np.float32(v).view(np.uint32) >> 16) + (1 if sign > 0 else -1)
    return float(np.uint32(b << 16).view(np.float32))


def test_off_by_one_step_away_from_a_midpoint_is_a_mismatch():
    cfg, w, toks, rec, names, ref = _setup()
    i = names.index("q")
    x, r = rec[i]
    j = tuple(np.argwhere((np.abs(x - r) < 1e-3 * np.abs(r)) & (np.abs(r) > 1e-3))[0])   # x right at a bf16 value
    bad = r.copy()
    bad[j] = _step(r[j], +1)
    expect = [(n, rv) for n, (xv, rv) in zip(names, rec)]
    expect[i] = ("q", bad)
    mm, _ = _run(cfg, w, toks, expect)
    assert mm.points["q"].bad == 1 and mm.points["q"].exact == 2 * x.size - 1    # q of both layers


def test_rounding_decisions_are_classified_by_distance_to_the_midpoint():
    """Crafted rows [value, 2]: delta = WINDOW * rms(row), the second element
    always exact; cases around the midpoint between 1 and 1 + 2^-7 and near 0."""
    cfg, w, toks, rec, names, ref = _setup()
    mm = MatchedModel(cfg, w)
    mid = 1.0 + 2.0 ** -8

    def run(v, g):
        mm.points = {}
        mm.expect = [("p", np.array([[g, 2.0]]))]
        out = mm.rn(np.array([[v, 2.0]]))
        assert out[0, 0] == g                                # the GPU's value is followed
        p = mm.points["p"]
        return p.exact - 1, p.ambiguous, p.bad

    d = WINDOW * np.sqrt((mid ** 2 + 4.0) / 2)               # delta of the midpoint rows
    assert run(mid + 0.5 * d, 1.0) == (0, 1, 0)               # nearest is 1 + 2^-7; 1 within delta
    assert run(mid - 0.5 * d, 1.0 + 2.0 ** -7) == (0, 1, 0)
    assert run(mid + 0.5 * d, 1.0 + 2.0 ** -7) == (1, 0, 0)
    assert run(mid + 1.5 * d, 1.0) == (0, 0, 1)               # outside delta
    assert run(1.0 + 2.0 ** -10, 1.0 + 2.0 ** -7) == (0, 0, 1)   # far from the midpoint
    assert run(mid + 0.5 * d, 1.0 + 2.0 ** -6) == (0, 0, 1)   # two steps away
    d0 = WINDOW * np.sqrt(2.0)                                # rows [~0, 2]
    assert run(0.25 * d0, float(bf16_round(-0.5 * d0))) == (0, 1, 0)   # near zero: any bf16 value within delta
    assert run(0.25 * d0, float(bf16_round(1.5 * d0))) == (0, 0, 1)
