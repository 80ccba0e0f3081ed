"""The allocation-free accept entry point against the context one (needs an MI355X).

ssd_test_accept_noalloc keeps its staging and counters in a static device
array shared by every call on the GPU; each call must still give exactly
what ssd_test_accept gives, also right after a larger call left its contents
there.  Collected last: a failure here hides no other test.
"""
import itertools

import numpy as np
import pytest

import synth
from _common import engine

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def eng():
    cfg = synth.config("tiny")
    print("[no-alloc] building engine", flush=True)
    e = engine(cfg, synth.make_weights(cfg))
    yield e
    e.close()


def _case(g, k, a):
    p = g.integers(0, 1000, k + 1).astype(np.int32)
    d = p[:k].copy()
    if a < k:
        d[a] = (d[a] + 1) % 1000
    return d, p


def test_noalloc_accept_equals_context_accept_on_calls_in_a_row(eng):
    from self_speculative_decoding_amd import test_accept_noalloc
    g = np.random.default_rng(11)
    # a larger call, then smaller ones: stale entries past k must not leak
    for k, a in ((31, 31), (20, 13), (5, 2), (3, 3), (0, 0), (17, 0)):
        d, p = _case(g, k, a)
        got = test_accept_noalloc(d, p)
        assert got == eng.test_accept(d, p) == a, (k, a, got)


def test_noalloc_accept_exhaustive_small_and_on_a_stream(eng):
    import torch
    from self_speculative_decoding_amd import test_accept_noalloc
    s = torch.cuda.Stream()
    for k in range(0, 4):
        for d in itertools.product(range(3), repeat=k):
            for p in itertools.product(range(3), repeat=k + 1):
                ref = eng.test_accept(d, p)
                assert test_accept_noalloc(d, p) == ref, (d, p)
                assert test_accept_noalloc(d, p, stream=s) == ref, (d, p)
