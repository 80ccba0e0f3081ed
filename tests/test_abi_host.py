"""C-ABI library: loads, exports every declared symbol, and its host-only
logic (configuration checks, weight table, layout, skip mask, state machine)
behaves as documented.  No GPU needed: nothing here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import skip_mask as oracle_skip_mask
from _common import ROOT

ssd = pytest.importorskip("self_speculative_decoding_amd")


def _declared():
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(ssd.LIB_PATH)
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(ssd.EXPORTS) == names


def test_binding_fails_loudly_without_the_library(tmp_path):
    """The binding refuses to import when libssd.so is absent: no CPU or other
    fallback stands in for the HIP path."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "self_speculative_decoding_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "self_speculative_decoding_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import self_speculative_decoding_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libssd.so is missing" in r.stderr


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus 2 exits non-zero with a message
    before anything touches a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU only" in r.stdout + r.stderr


def test_bench_traffic_is_null_once_the_gemm_sources_change(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counter summary only while the
    gate/up kernel's sources hash as they did when the counters were taken."""
    import hashlib
    import shutil
    import sys
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "self_speculative_decoding_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for f in ("gemm.hip", "device.h"):
        shutil.copy(os.path.join(ROOT, "self_speculative_decoding_amd", "csrc", f), csrc / f)
    sha = hashlib.sha256((csrc / "gemm.hip").read_bytes() + (csrc / "device.h").read_bytes()).hexdigest()
    (tmp_path / "profiles" / "gemm_swiglu_llama8b_traffic.txt").write_text(
        f"counter bytes per launch: 235467858 (ratio 1.0019)\nkernel source sha256 (gemm.hip + device.h) when measured: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic() == 235467858.0
    (csrc / "gemm.hip").write_bytes((csrc / "gemm.hip").read_bytes() + b"\n// changed\n")
    assert bench.measured_traffic() is None


@pytest.mark.parametrize("name", ["tiny", "qwen3-4b", "llama-8b", "qwen3-8b", "dsv2-lite"])
def test_workload_cfgs_validate_and_weight_table_matches(name):
    cfg = synth.config(name)
    c = ssd.make_cfg(cfg)
    assert ssd.validate_cfg(c) == 0, ssd.lib.ssd_last_error()
    numels = ssd.weight_numels(c)
    specs = synth.weight_specs(cfg)
    assert numels == [int(np.prod(s)) for _, s, _ in specs]
    assert ssd.workspace_bytes(c) > 0


@pytest.mark.parametrize("name", ["tiny", "llama-8b", "qwen3-8b", "dsv2-lite"])
def test_weight_retention_and_packed_workspace(name):
    # bf16 models copy every matrix into the workspace at load; only the
    # embedding and the norm gains stay referenced.  float32 keeps all.
    cfg = synth.config(name)
    c = ssd.make_cfg(cfg)
    specs = synth.weight_specs(cfg)
    kept = [ssd.lib.ssd_weight_retained(ctypes.byref(c), i) for i in range(len(specs))]
    if cfg["dtype"] == "f32":
        assert kept == [1] * len(specs)
        return
    expect = [1 if (n == "embed" or n.endswith("norm")) else 0 for n, _, _ in specs]
    assert kept == expect
    packed = sum(int(np.prod(s)) for (n, s, _), k in zip(specs, kept) if k == 0) * 2
    assert ssd.workspace_bytes(c) > packed
    assert ssd.lib.ssd_weight_retained(ctypes.byref(c), len(specs)) == -1


def test_llama8b_weight_bytes():
    # 32 layers x 436.2 MB + embedding and LM head of 1.05 GB each
    assert abs(synth.weight_bytes(synth.config("llama-8b")) / 1e9 - 16.06) < 0.01


@pytest.mark.parametrize("field,value,status", [
    ("n_kv_heads", 3, -1), ("head_dim", 96, -5), ("dtype", 7, -1), ("max_block", 0, -1),
    ("max_block", 33, -1), ("prefill_chunk", 24, -1), ("vocab", 4100, -5), ("rms_eps", 0.0, -1),
])
def test_validate_rejects(field, value, status):
    c = ssd.make_cfg(synth.config("llama-8b"))
    setattr(c, field, value)
    assert ssd.validate_cfg(c) == status
    assert ssd.workspace_bytes(c) == -1
    assert ssd.lib.ssd_last_error()


def test_null_cfg():
    assert ssd.lib.ssd_validate_cfg(None) == -1


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 32, 36, 80])
@pytest.mark.parametrize("frac", [0.0, 0.1, 0.2, 0.25, 0.3, 0.4, 0.5, 0.9, 1.0])
def test_skip_mask_matches_oracle(n, frac):
    assert ssd.skip_mask(n, frac).tolist() == oracle_skip_mask(n, frac)


def test_skip_mask_rejects():
    m = np.zeros(4, np.uint8)
    assert ssd.lib.ssd_skip_mask(0, 0.5, m.ctypes.data_as(ctypes.c_void_p)) == -1
    assert ssd.lib.ssd_skip_mask(4, 1.5, m.ctypes.data_as(ctypes.c_void_p)) == -1
    assert ssd.lib.ssd_skip_mask(4, 0.5, None) == -1


def test_state_machine():
    L, R, D, V = ssd.ST_LOADED, ssd.ST_READY, ssd.ST_DRAFTED, ssd.ST_VERIFIED
    ok = {(L, ssd.OP_PREFILL): R, (R, ssd.OP_DRAFT): D, (D, ssd.OP_VERIFY): V,
          (R, ssd.OP_VERIFY_BLOCK): V, (D, ssd.OP_VERIFY_BLOCK): V, (V, ssd.OP_ACCEPT): R}
    for s in (L, R, D, V):
        assert ssd.check_transition(s, ssd.OP_RESET) == L
        for op in (ssd.OP_PREFILL, ssd.OP_DRAFT, ssd.OP_VERIFY, ssd.OP_VERIFY_BLOCK, ssd.OP_ACCEPT):
            assert ssd.check_transition(s, op) == ok.get((s, op), -2), (s, op)
    assert ssd.check_transition(L, 99) == -1


def test_strerror():
    for s in (0, -1, -2, -3, -4, -5):
        assert ssd.lib.ssd_strerror(s)


def test_select_k_matches_oracle_and_is_monotone_in_alpha():
    from oracle import select_k as ora_select_k
    rng = np.random.default_rng(11)
    for trial in range(200):
        kmax = int(rng.integers(0, 31))
        tv = np.cumsum(rng.uniform(0.0, 0.2, kmax + 1)) + rng.uniform(0.5, 2.0)
        if trial % 3 == 0:
            tv = rng.uniform(0.5, 2.0, kmax + 1)          # any positive table
        td, tc = float(rng.uniform(0.05, 1.5)), float(rng.uniform(0.0, 0.3))
        prev = -1
        for a in np.linspace(0.0, 1.0, 21):
            k, r = ssd.select_k(tv, td, tc, a)
            ko, ro = ora_select_k(list(tv), td, tc, a)
            assert k == ko and abs(r - ro) <= 1e-12 * ro, (trial, a)
            assert k >= prev, (trial, a)                   # non-decreasing in alpha
            prev = k
    # exact ties (alpha = 0, k * t_draft + t_verify[k] equal): the smallest k, as in the oracle
    for tv, want in (([1.0, 0.75, 0.5], 0), ([1.25, 0.75, 0.5], 1)):
        assert ssd.select_k(tv, 0.25, 0.0, 0.0) == ora_select_k(tv, 0.25, 0.0, 0.0) == (want, 1.0)


def test_select_k_rejects():
    c = ssd.lib
    tv = np.ones(4)
    k, r = ctypes.c_int32(), ctypes.c_double()
    p = tv.ctypes.data_as(ctypes.c_void_p)
    assert c.ssd_select_k(p, 3, 0.5, 0.0, 1.5, ctypes.byref(k), ctypes.byref(r)) == -1
    assert c.ssd_select_k(p, 3, 0.0, 0.0, 0.5, ctypes.byref(k), ctypes.byref(r)) == -1
    assert c.ssd_select_k(p, 32, 0.5, 0.0, 0.5, ctypes.byref(k), ctypes.byref(r)) == -1
    assert c.ssd_select_k(None, 3, 0.5, 0.0, 0.5, ctypes.byref(k), ctypes.byref(r)) == -1


def test_knapsack_skip_matches_brute_force():
    from oracle import knapsack_skip_brute
    rng = np.random.default_rng(5)
    for trial in range(150):
        n = int(rng.integers(1, 11))
        cost = rng.integers(0, 9, n)
        if trial % 4 == 0:
            cost[:] = 5                                     # uniform costs: top values win
        value = rng.uniform(0.0, 1.0, n)
        if trial % 5 == 0:
            value = np.round(value * 4) / 4                 # ties
        budget = int(rng.integers(0, int(cost.sum()) + 2))
        mask, kept = ssd.knapsack_skip(cost, value, budget)
        best, sets = knapsack_skip_brute(cost.tolist(), value.tolist(), budget)
        keep = tuple(int(i) for i in np.nonzero(mask == 0)[0])
        assert abs(kept - best) <= 1e-9, trial
        assert keep in sets, (trial, keep, sets)            # an optimal, feasible set


def test_knapsack_skip_rejects():
    c = np.ones(4, np.int32)
    v = np.ones(4)
    m = np.zeros(4, np.uint8)
    kv = ctypes.c_double()
    f = ssd.lib.ssd_knapsack_skip
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert f(P(c), P(v), 4, -1, P(m), ctypes.byref(kv)) == -1
    assert f(P(c), P(v), 4, 1 << 25, P(m), ctypes.byref(kv)) == -1
    bad = np.array([1, -1, 1, 1], np.int32)
    assert f(P(bad), P(v), 4, 3, P(m), ctypes.byref(kv)) == -1


def test_noalloc_accept_rejects_bad_arguments_before_any_hip_call():
    """Argument checks of the allocation-free accept run on the host: an
    out-of-range k or a NULL pointer returns SSD_E_ARG without a HIP call."""
    a = ctypes.c_int32(-7)
    p = np.zeros(40, np.int32)
    for k in (-1, ssd.SSD_MAX_BLOCK, 40):
        st = ssd.lib.ssd_test_accept_noalloc(p.ctypes.data_as(ctypes.c_void_p), p.ctypes.data_as(ctypes.c_void_p),
                                             k, None, ctypes.byref(a))
        assert st == -1 and a.value == -7
    assert ssd.lib.ssd_test_accept_noalloc(None, p.ctypes.data_as(ctypes.c_void_p), 3, None, ctypes.byref(a)) == -1
    assert ssd.lib.ssd_test_accept_noalloc(p.ctypes.data_as(ctypes.c_void_p), None, 3, None, ctypes.byref(a)) == -1
