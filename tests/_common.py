"""Shared helpers for the tests: build engines and oracles from seeded inputs."""
import os

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ordered(cfg, weights):
    """Weights in the canonical C-ABI order."""
    return [weights[name] for name, _, _ in synth.weight_specs(cfg)]


def engine(cfg, weights, **kw):
    from self_speculative_decoding_amd import Engine, make_cfg
    return Engine(make_cfg(cfg, **kw), ordered(cfg, weights))


def bf16_bits_to_f32(a):
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
