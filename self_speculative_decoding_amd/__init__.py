"""Python binding of libssd.so, the MI355X greedy self-speculative decoding
library (C ABI declared in include/ssd.h).

Argument marshalling only: every step of the decode path runs in the
library's HIP kernels.  torch provides device memory (weights, workspace) and
the stream.  Importing this package fails loudly when libssd.so is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_MAX_FEAT = 8
SSD_MAX_BLOCK = 32
ST_LOADED, ST_READY, ST_DRAFTED, ST_VERIFIED = range(4)
OP_PREFILL, OP_DRAFT, OP_VERIFY, OP_VERIFY_BLOCK, OP_ACCEPT, OP_RESET = range(6)
OPS = dict(gate_up=0, down=1, qkv=2, o=3, lm_head=4, attention=5, moe=6, read_probe=7, copy_probe=8)

EXPORTS = ["ssd_validate_cfg", "ssd_n_weights", "ssd_weight_numel", "ssd_weight_retained", "ssd_workspace_bytes",
           "ssd_skip_mask", "ssd_check_transition", "ssd_strerror", "ssd_last_error",
           "ssd_load", "ssd_free", "ssd_reset", "ssd_state", "ssd_context_length",
           "ssd_prefill", "ssd_draft", "ssd_verify", "ssd_accept_rollback", "ssd_generate",
           "ssd_get_stats", "ssd_read_logits", "ssd_read_features", "ssd_set_routing",
           "ssd_read_union", "ssd_test_accept", "ssd_time_op", "ssd_set_option", "ssd_read_trace",
           "ssd_read_kv", "ssd_select_k", "ssd_knapsack_skip", "ssd_layer_cosines",
           "ssd_set_sampling", "ssd_test_spec_cycle", "ssd_test_accept_noalloc", "ssd_read_trace_point"]


class Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "vocab", "dtype")] + \
               [("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)] + \
               [(n, ctypes.c_int32) for n in
                ("max_ctx", "max_block", "prefill_chunk", "n_experts", "top_k", "n_shared", "expert_ffn",
                 "n_dense_layers", "dense_ffn", "moe_dedup", "n_feat")] + \
               [("feat_layers", ctypes.c_int32 * SSD_MAX_FEAT)]


class Buf(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("nbytes", ctypes.c_int64)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("cycles", "drafted", "accepted", "emitted", "verify_passes")] + \
               [(n, ctypes.c_double) for n in
                ("t_prefill_ms", "t_draft_ms", "t_verify_ms", "t_accept_ms", "t_decode_ms")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class SSDError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ssd status {status}: {msg}")
        self.status = status


def _load():
    # torch first: its HIP runtime (SONAME libamdhip64.so.7) is then the one
    # libssd.so binds to, so the process has a single HIP runtime and device
    # pointers from torch are valid inside the library.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python self_speculative_decoding_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pc = P(Cfg)
    sig = {
        "ssd_validate_cfg": (I32, [pc]),
        "ssd_n_weights": (I32, [pc]),
        "ssd_weight_numel": (I64, [pc, I32]),
        "ssd_weight_retained": (I32, [pc, I32]),
        "ssd_workspace_bytes": (I64, [pc]),
        "ssd_skip_mask": (I32, [I32, ctypes.c_double, VP]),
        "ssd_select_k": (I32, [VP, I32, ctypes.c_double, ctypes.c_double, ctypes.c_double, VP, VP]),
        "ssd_knapsack_skip": (I32, [VP, VP, I32, I64, VP, VP]),
        "ssd_layer_cosines": (I32, [VP, I32, VP]),
        "ssd_set_sampling": (I32, [VP, ctypes.c_float, ctypes.c_uint64]),
        "ssd_test_spec_cycle": (I32, [VP, VP, VP, I32, I32, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, I32, VP]),
        "ssd_check_transition": (I32, [I32, I32, P(I32)]),
        "ssd_strerror": (ctypes.c_char_p, [I32]),
        "ssd_last_error": (ctypes.c_char_p, []),
        "ssd_load": (I32, [pc, P(Buf), I32, Buf, VP, P(VP)]),
        "ssd_free": (None, [VP]),
        "ssd_reset": (I32, [VP]),
        "ssd_state": (I32, [VP]),
        "ssd_context_length": (I32, [VP]),
        "ssd_prefill": (I32, [VP, VP, I32, P(I32)]),
        "ssd_draft": (I32, [VP, VP, I32, VP]),
        "ssd_verify": (I32, [VP, VP, I32, VP]),
        "ssd_accept_rollback": (I32, [VP, P(I32), VP, P(I32)]),
        "ssd_generate": (I32, [VP, VP, I32, I32, I32, VP, I32, VP, P(Stats)]),
        "ssd_get_stats": (I32, [VP, P(Stats)]),
        "ssd_read_logits": (I32, [VP, VP, I32]),
        "ssd_read_features": (I32, [VP, VP, I32]),
        "ssd_set_routing": (I32, [VP, VP, I32]),
        "ssd_read_union": (I32, [VP, VP]),
        "ssd_test_accept": (I32, [VP, VP, VP, I32, P(I32)]),
        "ssd_test_accept_noalloc": (I32, [VP, VP, I32, VP, P(I32)]),
        "ssd_time_op": (I32, [VP, I32, I32, I32, I32, P(ctypes.c_float)]),
        "ssd_set_option": (I32, [VP, I32, I32]),
        "ssd_read_trace": (I32, [VP, VP, I32]),
        "ssd_read_trace_point": (I32, [VP, I32, I32, I32, VP]),
        "ssd_read_kv": (I32, [VP, I32, I32, I32, VP, VP]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


lib = _load()


def _check(status: int):
    if status != 0:
        raise SSDError(status, (lib.ssd_last_error() or b"").decode())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def make_cfg(cfg: dict, max_block: int | None = None, prefill_chunk: int = 128, moe_dedup: int = 0) -> Cfg:
    """C cfg from a workload dict (keys as in the synth module)."""
    c = Cfg()
    for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "vocab", "max_ctx"):
        setattr(c, n, int(cfg[n]))
    c.ffn_dim = int(cfg.get("ffn_dim", 0))
    c.dtype = 1 if cfg["dtype"] == "bf16" else 0
    c.rms_eps = float(cfg["rms_eps"])
    c.rope_theta = float(cfg["rope_theta"])
    c.max_block = int(max_block if max_block is not None else cfg.get("max_block", 17))
    c.prefill_chunk = int(prefill_chunk)
    for n in ("n_experts", "top_k", "n_shared", "expert_ffn", "n_dense_layers", "dense_ffn"):
        setattr(c, n, int(cfg.get(n, 0)))
    c.moe_dedup = int(moe_dedup)
    fl = list(cfg.get("feat_layers", ()))
    c.n_feat = len(fl)
    for i, l in enumerate(fl):
        c.feat_layers[i] = int(l)
    return c


def validate_cfg(c: Cfg) -> int:
    return lib.ssd_validate_cfg(ctypes.byref(c))


def workspace_bytes(c: Cfg) -> int:
    return lib.ssd_workspace_bytes(ctypes.byref(c))


def weight_numels(c: Cfg) -> list[int]:
    n = lib.ssd_n_weights(ctypes.byref(c))
    if n < 0:
        _check(validate_cfg(c) or -1)
    return [lib.ssd_weight_numel(ctypes.byref(c), i) for i in range(n)]


def skip_mask(n_layers: int, frac: float) -> np.ndarray:
    m = np.zeros(n_layers, dtype=np.uint8)
    _check(lib.ssd_skip_mask(n_layers, float(frac), _ptr(m)))
    return m


def select_k(t_verify, t_draft: float, t_cycle: float, alpha: float) -> tuple[int, float]:
    """Draft length maximising expected tokens per unit time (ssd_select_k).
    t_verify[k] = verify-pass time over k+1 tokens, k = 0..len-1."""
    tv = np.ascontiguousarray(t_verify, dtype=np.float64)
    k = ctypes.c_int32(-1)
    r = ctypes.c_double(0.0)
    _check(lib.ssd_select_k(_ptr(tv), len(tv) - 1, float(t_draft), float(t_cycle), float(alpha),
                            ctypes.byref(k), ctypes.byref(r)))
    return k.value, r.value


def knapsack_skip(cost, value, budget: int) -> tuple[np.ndarray, float]:
    """Skip mask keeping the layers of largest total value within the cost
    budget (ssd_knapsack_skip)."""
    c = np.ascontiguousarray(cost, dtype=np.int32)
    v = np.ascontiguousarray(value, dtype=np.float64)
    mask = np.zeros(len(c), dtype=np.uint8)
    kept = ctypes.c_double(0.0)
    _check(lib.ssd_knapsack_skip(_ptr(c), _ptr(v), len(c), int(budget), _ptr(mask), ctypes.byref(kept)))
    return mask, kept.value


def test_accept_noalloc(d, p, stream=None) -> int:
    """The accept kernel on host drafts and predictions with no context and no
    device allocation (ssd_test_accept_noalloc); stream: a torch stream or None."""
    dd = np.ascontiguousarray(d, dtype=np.int32)
    pp = np.ascontiguousarray(p, dtype=np.int32)
    a = ctypes.c_int32()
    s = None if stream is None else ctypes.c_void_p(stream.cuda_stream)
    _check(lib.ssd_test_accept_noalloc(_ptr(dd) if len(dd) else None, _ptr(pp), len(dd), s, ctypes.byref(a)))
    return a.value


def check_transition(state: int, op: int) -> int:
    nxt = ctypes.c_int32(-1)
    st = lib.ssd_check_transition(state, op, ctypes.byref(nxt))
    return nxt.value if st == 0 else st


class Engine:
    """One loaded model on one GPU.

    weights: arrays in the canonical order of include/ssd.h (float32, or uint16
    bf16 bit patterns), uploaded once to device memory with torch.
    """

    def __init__(self, cfg: Cfg, weights: list[np.ndarray], device: str = "cuda:0"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        numels = weight_numels(cfg)
        if len(weights) != len(numels):
            raise ValueError(f"expected {len(numels)} weights, got {len(weights)}")
        self._w = []
        bufs = (Buf * len(weights))()
        for i, (a, n) in enumerate(zip(weights, numels)):
            a = np.ascontiguousarray(a)
            if a.size != n:
                raise ValueError(f"weight {i}: {a.size} elements, expected {n}")
            host = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            t = host.to(self.device)
            self._w.append(t)
            bufs[i] = Buf(t.data_ptr(), t.numel() * t.element_size())
        nb = workspace_bytes(cfg)
        if nb < 0:
            _check(validate_cfg(cfg))
        self._ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
        # a stream of the library's own (default priority): graphs cannot be
        # captured on the null stream
        self.stream = torch.cuda.Stream(self.device)
        ctx = ctypes.c_void_p()
        torch.cuda.synchronize(self.device)
        _check(lib.ssd_load(ctypes.byref(cfg), bufs, len(weights), Buf(self._ws.data_ptr(), nb),
                            ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(ctx)))
        self.ctx = ctx
        # matrices the library copied into its packed layout are not read again
        for i in range(len(self._w)):
            if lib.ssd_weight_retained(ctypes.byref(cfg), i) == 0:
                self._w[i] = None
        self.L, self.V, self.d = cfg.n_layers, cfg.vocab, cfg.d_model

    def close(self):
        if getattr(self, "ctx", None) is not None and self.ctx.value:
            lib.ssd_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- state ------------------------------------------------------------------
    @property
    def state(self) -> int:
        return lib.ssd_state(self.ctx)

    @property
    def context_length(self) -> int:
        return lib.ssd_context_length(self.ctx)

    def reset(self):
        _check(lib.ssd_reset(self.ctx))

    def set_graphs(self, on: bool):
        _check(lib.ssd_set_option(self.ctx, 0, 1 if on else 0))

    def set_moe_dedup(self, on: bool):
        _check(lib.ssd_set_option(self.ctx, 1, 1 if on else 0))

    def set_trace(self, on: bool):
        _check(lib.ssd_set_option(self.ctx, 2, 1 if on else 0))

    def layer_cosines(self, rows: int) -> np.ndarray:
        """Per-layer mean cosine(input, output) of the last full pass (trace on)."""
        out = np.zeros(self.L, dtype=np.float64)
        _check(lib.ssd_layer_cosines(self.ctx, rows, _ptr(out)))
        return out

    def set_sampling(self, temperature: float, seed: int):
        _check(lib.ssd_set_sampling(self.ctx, float(temperature), int(seed)))

    def test_spec_cycle(self, target, draft, temperature: float, seed: int, cycle0: int, trials: int) -> np.ndarray:
        """Sampled cycles on host logits: rows [trials, k+2] = a, emitted tokens, -1."""
        t = np.ascontiguousarray(target, dtype=np.float32)
        k, V = t.shape[0] - 1, t.shape[1]
        d = np.ascontiguousarray(draft, dtype=np.float32).reshape(k, V) if k > 0 else np.zeros((1, V), np.float32)
        out = np.zeros((trials, k + 2), dtype=np.int32)
        _check(lib.ssd_test_spec_cycle(self.ctx, _ptr(t), _ptr(d), k, V, float(temperature), int(seed), int(cycle0),
                                       trials, _ptr(out)))
        return out

    def set_kvq(self, on: bool):
        """Exit-state reuse for tail-mask (early-exit) drafts (SSD_OPT_KVQ)."""
        _check(lib.ssd_set_option(self.ctx, 3, 1 if on else 0))

    def set_tile_groups(self, min_workgroups: int):
        """Long-pass GEMM grouping threshold (SSD_OPT_TILE_GROUPS; 0 = default)."""
        _check(lib.ssd_set_option(self.ctx, 4, int(min_workgroups)))

    def read_trace(self, rows: int) -> np.ndarray:
        out = np.zeros((self.L, rows, self.d), dtype=np.float32)
        _check(lib.ssd_read_trace(self.ctx, _ptr(out), rows))
        return out

    def read_trace_point(self, layer: int, point: int, rows: int) -> np.ndarray:
        """A stored operand of one layer of the last traced pass
        (ssd_read_trace_point): bf16 bits (uint16) or float32, [rows, width]."""
        c = self.cfg
        qo = c.n_q_heads * c.head_dim
        moe = c.n_experts > 0 and c.n_dense_layers <= layer < c.n_layers
        ffn = (c.top_k + c.n_shared) * c.expert_ffn if moe else (c.dense_ffn if c.n_experts > 0 else c.ffn_dim)
        width = {0: c.d_model, 1: qo, 2: qo, 3: c.d_model, 4: c.d_model, 5: ffn}[point]
        dt = np.float32 if point == 3 or c.dtype == 0 else np.uint16
        out = np.zeros((rows, width), dtype=dt)
        _check(lib.ssd_read_trace_point(self.ctx, layer, point, rows, _ptr(out)))
        return out

    def read_kv(self, layer: int, pos0: int, n: int):
        """K and V of one layer, [n_kv_heads, n, head_dim], cfg dtype."""
        dt = np.uint16 if self.cfg.dtype == 1 else np.float32
        k = np.zeros((self.cfg.n_kv_heads, n, self.cfg.head_dim), dtype=dt)
        v = np.zeros_like(k)
        _check(lib.ssd_read_kv(self.ctx, layer, pos0, n, _ptr(k), _ptr(v)))
        return k, v

    # -- the decode step --------------------------------------------------------------
    def prefill(self, tokens) -> int:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        nxt = ctypes.c_int32()
        _check(lib.ssd_prefill(self.ctx, _ptr(t), len(t), ctypes.byref(nxt)))
        return nxt.value

    def draft(self, mask, k: int) -> list[int]:
        m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
        out = np.zeros(max(k, 1), dtype=np.int32)
        _check(lib.ssd_draft(self.ctx, None if m is None else _ptr(m), k, _ptr(out)))
        return out[:k].tolist()

    def verify(self, block=None, m: int | None = None) -> list[int]:
        if block is not None:
            b = np.ascontiguousarray(block, dtype=np.int32)
            m = len(b)
        post = np.zeros(m, dtype=np.int32)
        _check(lib.ssd_verify(self.ctx, None if block is None else _ptr(b), m, _ptr(post)))
        return post.tolist()

    def accept(self) -> tuple[int, list[int]]:
        a, ne = ctypes.c_int32(), ctypes.c_int32()
        em = np.zeros(SSD_MAX_BLOCK + 1, dtype=np.int32)
        _check(lib.ssd_accept_rollback(self.ctx, ctypes.byref(a), _ptr(em), ctypes.byref(ne)))
        return a.value, em[:ne.value].tolist()

    def generate(self, prompt, n_new: int, mask=None, k: int = 0, greedy: int = 1):
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        out = np.zeros(n_new, dtype=np.int32)
        st = Stats()
        m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
        _check(lib.ssd_generate(self.ctx, _ptr(p), len(p), n_new, greedy, None if m is None else _ptr(m), k,
                                _ptr(out), ctypes.byref(st)))
        return out.tolist(), st.as_dict()

    def stats(self) -> dict:
        st = Stats()
        _check(lib.ssd_get_stats(self.ctx, ctypes.byref(st)))
        return st.as_dict()

    # -- hooks -------------------------------------------------------------------------
    def read_logits(self, rows: int) -> np.ndarray:
        out = np.zeros((rows, self.V), dtype=np.float32)
        _check(lib.ssd_read_logits(self.ctx, _ptr(out), rows))
        return out

    def read_features(self, rows: int) -> np.ndarray:
        out = np.zeros((rows, self.d), dtype=np.uint16)
        _check(lib.ssd_read_features(self.ctx, _ptr(out), rows))
        return out

    def set_routing(self, ids) -> None:
        if ids is None:
            _check(lib.ssd_set_routing(self.ctx, None, 0))
            return
        a = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib.ssd_set_routing(self.ctx, _ptr(a), a.shape[1]))

    def read_union(self) -> np.ndarray:
        out = np.zeros(self.L, dtype=np.int32)
        _check(lib.ssd_read_union(self.ctx, _ptr(out)))
        return out

    def test_accept(self, d, p) -> int:
        dd = np.ascontiguousarray(d, dtype=np.int32)
        pp = np.ascontiguousarray(p, dtype=np.int32)
        a = ctypes.c_int32()
        _check(lib.ssd_test_accept(self.ctx, _ptr(dd) if len(dd) else None, _ptr(pp), len(dd), ctypes.byref(a)))
        return a.value

    def time_op(self, op: str, layer: int, m: int, iters: int) -> float:
        us = ctypes.c_float()
        _check(lib.ssd_time_op(self.ctx, OPS[op], layer, m, iters, ctypes.byref(us)))
        return us.value
