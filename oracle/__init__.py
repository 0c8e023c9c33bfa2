"""Python access to the plain CPU oracle (``dflash_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py``; never by the product package.

The C library is compiled with gcc (``build()``); every function here only
marshals arguments.  Inputs are torch CPU tensors in the workload's storage
dtype (fp32 or bf16); outputs are numpy float64 arrays already rounded to the
storage precision (fp32 values for logits).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dflash_oracle.c")
# DFLASH_ORACLE_LIB points the loader at another build of the same source
# (the mutation test of the pins builds deliberately altered copies apart)
_LIB = os.environ.get("DFLASH_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
MAX_LAYERS = 64


def build(force: bool = True, src: str = _SRC, out: Optional[str] = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    out = out or _LIB
    if force or not os.path.exists(out):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-I", _HERE,
               "-o", out + ".tmp", src, "-lm"]
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        vp, i32, i64, dp = C.c_void_p, C.c_int32, C.c_int64, C.POINTER(C.c_double)
        L.orc_set_fp32_accumulation.argtypes = [i32]
        L.orc_set_threads.argtypes = [i32]
        L.orc_get_threads.restype = i32
        L.orc_round_bf16.restype = C.c_double
        L.orc_round_bf16.argtypes = [C.c_double]
        L.orc_round_array_bf16.argtypes = [vp, i64, vp]
        L.orc_feature_layers.argtypes = [i32, vp]
        L.orc_rmsnorm.argtypes = [vp, i32, vp, i32, C.c_double, vp]
        L.orc_rope.argtypes = [vp, i32, i64, C.c_double]
        L.orc_fuse_rows.argtypes = [vp, vp, i64, vp, i32, vp]
        L.orc_inject_rows.argtypes = [vp, vp, i64, vp, i32, i64, vp, vp]
        L.orc_draft_block.argtypes = [vp, vp, vp, i64, i32, vp, vp, vp, vp]
        L.orc_draft_layer.argtypes = [vp, i32, vp, vp, i64, vp, vp]
        L.orc_lm_head.argtypes = [vp, vp, i32, vp, vp, vp]
        L.orc_accept.argtypes = [vp, vp, i32, vp, vp]
        L.orc_target_forward.argtypes = [vp, vp, i32, i64, vp, vp, i64, vp, vp, vp, vp, vp]
        L.orc_target_forward_tree.argtypes = [vp, vp, vp, i32, i64, vp, vp, i64, vp, vp, vp, vp, vp]
        L.orc_target_layer.argtypes = [vp, i32, vp, i32, i64, vp, vp, vp, i64, vp]
        for f in ("orc_fuse_rows", "orc_inject_rows", "orc_draft_block", "orc_target_forward", "orc_draft_layer",
                  "orc_lm_head", "orc_target_forward_tree", "orc_target_layer"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


class _Model(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("hidden", C.c_int32), ("n_layers", C.c_int32),
        ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("ffn", C.c_int32), ("vocab", C.c_int32), ("block", C.c_int32), ("mask_id", C.c_int32),
        ("rope_base", C.c_double), ("eps", C.c_double),
        ("fc", C.c_void_p), ("fc_norm", C.c_void_p),
        ("attn_norm", C.c_void_p * MAX_LAYERS), ("wq", C.c_void_p * MAX_LAYERS),
        ("wk", C.c_void_p * MAX_LAYERS), ("wv", C.c_void_p * MAX_LAYERS),
        ("wo", C.c_void_p * MAX_LAYERS), ("mlp_norm", C.c_void_p * MAX_LAYERS),
        ("wg", C.c_void_p * MAX_LAYERS), ("wu", C.c_void_p * MAX_LAYERS),
        ("wd", C.c_void_p * MAX_LAYERS),
        ("final_norm", C.c_void_p), ("embed", C.c_void_p), ("lm_head", C.c_void_p),
    ]


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return t.data_ptr()


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


class Model:
    """An oracle view of a model given as a dict of CPU tensors (kept alive here)."""

    def __init__(self, shape, weights: Dict[str, torch.Tensor], n_layers: Optional[int] = None):
        self.shape = shape
        self.w = weights
        L = shape.draft_layers if n_layers is None else n_layers
        self.n_layers = L
        m = _Model()
        m.dtype = 0 if shape.dtype == "fp32" else 1
        m.hidden, m.n_layers = shape.hidden, L
        m.n_q_heads, m.n_kv_heads, m.head_dim = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
        m.ffn, m.vocab, m.block, m.mask_id = shape.ffn, shape.vocab, shape.block, shape.mask_id
        m.rope_base, m.eps = shape.rope_base, shape.eps
        m.fc, m.fc_norm = _ptr(weights.get("fc")), _ptr(weights.get("fc_norm"))
        for l in range(L):
            for name in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd"):
                getattr(m, name)[l] = _ptr(weights.get(f"{name}.{l}"))
        m.final_norm = _ptr(weights.get("final_norm"))
        m.embed, m.lm_head = _ptr(weights.get("embed")), _ptr(weights.get("lm_head"))
        self.s = m

    @property
    def ref(self):
        return C.byref(self.s)


def set_threads(n: int):
    """OpenMP threads of the oracle's loops (results do not depend on it)."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def set_fp32_accumulation(on: bool):
    lib().orc_set_fp32_accumulation(1 if on else 0)


def draft_noise_floor(model: Model, ctx_k, ctx_v, C_len: int, anchor: int, ref_logits: np.ndarray) -> float:
    """Largest logit difference between the oracle (fp64 accumulation) and the
    same oracle with fp32 accumulation: the drift two correct implementations
    show once storage rounding amplifies accumulation-order differences."""
    set_fp32_accumulation(True)
    try:
        alt = draft_block(model, ctx_k, ctx_v, C_len, anchor)
    finally:
        set_fp32_accumulation(False)
    return float(np.abs(alt["logits"].astype(np.float64) - ref_logits.astype(np.float64)).max())


def round_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    f = np.vectorize(lib().orc_round_bf16, otypes=[np.float64])
    return f(x)


def feature_layers(target_layers: int) -> List[int]:
    out = (C.c_int32 * 5)()
    lib().orc_feature_layers(target_layers, out)
    return list(out)


def rmsnorm(x: np.ndarray, gain: torch.Tensor, dtype: str, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_dptr(x), x.shape[-1], _ptr(gain), 0 if dtype == "fp32" else 1, eps, _dptr(out))
    return out


def rope(v: np.ndarray, pos: int, base: float) -> np.ndarray:
    v = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_dptr(v), v.shape[-1], pos, base)
    return v


def to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Oracle values (already rounded to the storage type) as a storage tensor; exact."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.float32 if dtype == "fp32" else torch.bfloat16).contiguous()


def fuse_rows(model: Model, slabs: Sequence[torch.Tensor], rows: Sequence[int]) -> np.ndarray:
    H = model.shape.hidden
    slabs = [s.contiguous() for s in slabs]
    assert len(slabs) == 5
    ld = slabs[0].stride(0)
    arr = (C.c_void_p * 5)(*[s.data_ptr() for s in slabs])
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows_a), H), dtype=np.float64)
    rc = lib().orc_fuse_rows(model.ref, arr, ld, rows_a.ctypes.data, len(rows_a), _dptr(out))
    assert rc == 0
    return out


def inject_rows(model: Model, fused: torch.Tensor, rows: Sequence[int], pos0: int):
    s = model.shape
    fused = fused.contiguous()
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    NK = s.n_kv_heads * s.head_dim
    k = np.empty((model.n_layers, len(rows_a), NK), dtype=np.float64)
    v = np.empty_like(k)
    rc = lib().orc_inject_rows(model.ref, _ptr(fused), fused.stride(0), rows_a.ctypes.data,
                               len(rows_a), pos0, _dptr(k), _dptr(v))
    assert rc == 0
    return k, v


def draft_block(model: Model, ctx_k: Optional[torch.Tensor], ctx_v: Optional[torch.Tensor],
                C_len: int, anchor: int, want_logits: bool = True, want_trace: bool = False):
    """ctx_k / ctx_v: storage tensors [L, >=C, nkv, d] (or None when C == 0)."""
    s = model.shape
    L, B, V, H = model.n_layers, s.block, s.vocab, s.hidden
    if C_len > 0:
        ctx_k = ctx_k.contiguous()
        ctx_v = ctx_v.contiguous()
        kp = (C.c_void_p * L)(*[ctx_k[l].data_ptr() for l in range(L)])
        vp = (C.c_void_p * L)(*[ctx_v[l].data_ptr() for l in range(L)])
    else:
        kp = vp = None
    logits = np.empty((B, V), dtype=np.float32) if want_logits else None
    tokens = np.empty(B, dtype=np.int32)
    gap = np.empty(B, dtype=np.float64)
    trace = np.empty((L + 1, B, H), dtype=np.float64) if want_trace else None
    rc = lib().orc_draft_block(model.ref, kp, vp, C_len, anchor,
                               logits.ctypes.data if logits is not None else None,
                               tokens.ctypes.data, gap.ctypes.data,
                               trace.ctypes.data if trace is not None else None)
    assert rc == 0
    return {"logits": logits, "tokens": tokens, "gap": gap, "trace": trace}


def draft_layer(model: Model, layer: int, ctx_k: Optional[torch.Tensor], ctx_v: Optional[torch.Tensor],
                C_len: int, x_in: np.ndarray) -> np.ndarray:
    """One draft layer alone: x_in [B, H] (storage values, e.g. another
    implementation's input to that layer); ctx_k / ctx_v: storage tensors
    [>=C, nkv, d] of that layer (or None when C == 0).  Returns [B, H]."""
    s = model.shape
    x_in = np.ascontiguousarray(x_in, dtype=np.float64)
    assert x_in.shape == (s.block, s.hidden)
    if C_len > 0:
        ctx_k, ctx_v = ctx_k.contiguous(), ctx_v.contiguous()
    out = np.empty_like(x_in)
    rc = lib().orc_draft_layer(model.ref, layer, _ptr(ctx_k) if C_len > 0 else None,
                               _ptr(ctx_v) if C_len > 0 else None, C_len, _dptr(x_in), _dptr(out))
    assert rc == 0
    return out


def lm_head(model: Model, x: np.ndarray):
    """Final RMSNorm + LM head + argmax of rows x [R, H] (storage values)."""
    s = model.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    R = x.shape[0]
    logits = np.empty((R, s.vocab), dtype=np.float32)
    tokens = np.empty(R, dtype=np.int32)
    gap = np.empty(R, dtype=np.float64)
    rc = lib().orc_lm_head(model.ref, _dptr(x), R, logits.ctypes.data, tokens.ctypes.data, gap.ctypes.data)
    assert rc == 0
    return {"logits": logits, "tokens": tokens, "gap": gap}


def accept(drafts: Sequence[int], target: Sequence[int]):
    d = np.ascontiguousarray(drafts, dtype=np.int32)
    g = np.ascontiguousarray(target, dtype=np.int32)
    assert d.shape == g.shape
    k, b = C.c_int32(), C.c_int32()
    lib().orc_accept(d.ctypes.data, g.ctypes.data, len(d), C.byref(k), C.byref(b))
    return k.value, b.value


class TargetCache:
    """Dense fp64 KV cache of the oracle's causal target."""

    def __init__(self, model: Model, cap: int):
        s = model.shape
        NK = s.n_kv_heads * s.head_dim
        self.cap = cap
        self.k = np.zeros((model.n_layers, cap, NK), dtype=np.float64)
        self.v = np.zeros_like(self.k)


def target_forward(model: Model, cache: TargetCache, tokens: Sequence[int], pos0: int,
                   capture: Optional[Sequence[int]] = None, want_logits: bool = False,
                   parent: Optional[Sequence[int]] = None):
    """Causal forward of `tokens` at pos0.. ([A] §1.1), or with `parent` the
    tree verification of [A] §8.2: row j sits at pos0 + depth(j), its K/V at
    cache slot pos0 + j, and it sees the cache before pos0 plus its ancestors."""
    s = model.shape
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(t)
    am = np.empty(n, dtype=np.int32)
    gap = np.empty(n, dtype=np.float64)
    cap_a = np.ascontiguousarray(capture, dtype=np.int32) if capture is not None else None
    hid = np.empty((5, n, s.hidden), dtype=np.float64) if capture is not None else None
    logits = np.empty((n, s.vocab), dtype=np.float32) if want_logits else None
    outs = (cache.cap, cap_a.ctypes.data if cap_a is not None else None,
            hid.ctypes.data if hid is not None else None,
            logits.ctypes.data if logits is not None else None, am.ctypes.data, gap.ctypes.data)
    if parent is None:
        rc = lib().orc_target_forward(model.ref, t.ctypes.data, n, pos0, _dptr(cache.k), _dptr(cache.v), *outs)
    else:
        par = np.ascontiguousarray(parent, dtype=np.int32)
        assert par.shape == t.shape
        rc = lib().orc_target_forward_tree(model.ref, t.ctypes.data, par.ctypes.data, n, pos0, _dptr(cache.k),
                                           _dptr(cache.v), *outs)
    assert rc == 0, "not a valid tree" if parent is not None else "capacity"
    return {"argmax": am, "gap": gap, "hidden": hid, "logits": logits}


def target_layer(model: Model, layer: int, x_in: np.ndarray, pos0: int, cache: TargetCache,
                 parent: Optional[Sequence[int]] = None) -> np.ndarray:
    """Layer `layer` of target_forward alone (causal, or tree with `parent`):
    rows x_in [n, H] (storage values) at pos0 over cache.k/v[layer] (keys
    before pos0); writes the rows' K/V into that layer's cache.  Returns [n, H]."""
    x_in = np.ascontiguousarray(x_in, dtype=np.float64)
    n = x_in.shape[0]
    par = np.ascontiguousarray(parent, dtype=np.int32) if parent is not None else None
    out = np.empty_like(x_in)
    rc = lib().orc_target_layer(model.ref, layer, _dptr(x_in), n, pos0,
                                par.ctypes.data if par is not None else None,
                                cache.k[layer].ctypes.data, cache.v[layer].ctypes.data, cache.cap, _dptr(out))
    assert rc == 0
    return out


# ---------------------------------------------------------------- generation loops

def greedy_generate(target: Model, prompt: Sequence[int], n_new: int, cap: Optional[int] = None):
    """Plain greedy decoding of the causal target ([A] §1.1): the prompt in one
    forward, then one token per forward.  Returns (tokens [n_new], gaps [n_new])
    where gaps[i] is the top-2 logit gap of the step that chose tokens[i]."""
    P = len(prompt)
    cache = TargetCache(target, cap or P + n_new + 1)
    r = target_forward(target, cache, prompt, 0)
    toks, gaps = [int(r["argmax"][-1])], [float(r["gap"][-1])]
    for i in range(1, n_new):
        r = target_forward(target, cache, [toks[-1]], P + i - 1)
        toks.append(int(r["argmax"][0]))
        gaps.append(float(r["gap"][0]))
    return np.array(toks, dtype=np.int32), np.array(gaps)


def spec_generate(target: Model, draft: Model, prompt: Sequence[int], n_new: int, drafts_fn=None):
    """DFlash speculative decoding with greedy block verification ([A] §2.2,
    §8.2; [B] 技术内幕; [C]):
      - the target runs over the prompt, capturing its five feature layers;
        the draft fuses them and injects them as context K/V;
      - each step drafts B-1 tokens from [anchor, mask ...] at C (or takes
        them from drafts_fn(C) -> B-1 ids, to force a pattern), the target
        verifies [anchor, d_1..d_{B-1}] causally, k leading drafts are
        accepted and the target's token after them is the bonus;
      - all B verified rows are fused and injected, then both caches keep
        C + k + 1 positions; the bonus is the next anchor.
    Returns (tokens [n_new], list of k per step)."""
    s = target.shape
    B, H = s.block, s.hidden
    P = len(prompt)
    cap = P + n_new + B
    sel = feature_layers(s.target_layers)
    NKs = (draft.n_layers, cap, s.n_kv_heads, s.head_dim)
    store = torch.float32 if s.dtype == "fp32" else torch.bfloat16
    ctx_k = torch.zeros(NKs, dtype=store)
    ctx_v = torch.zeros(NKs, dtype=store)
    cache = TargetCache(target, cap)

    def add_context(hidden, pos0):
        slabs = [to_storage(hidden[i], s.dtype) for i in range(5)]
        n = slabs[0].shape[0]
        fused = to_storage(fuse_rows(draft, slabs, range(n)), s.dtype)
        k, v = inject_rows(draft, fused, range(n), pos0)
        ctx_k[:, pos0:pos0 + n] = to_storage(k, s.dtype).reshape(draft.n_layers, n, s.n_kv_heads, s.head_dim)
        ctx_v[:, pos0:pos0 + n] = to_storage(v, s.dtype).reshape(draft.n_layers, n, s.n_kv_heads, s.head_dim)

    r = target_forward(target, cache, prompt, 0, capture=sel)
    add_context(r["hidden"], 0)
    anchor = int(r["argmax"][-1])
    out, ks = [anchor], []
    C = P
    while len(out) < n_new:
        if drafts_fn is None:
            d = draft_block(draft, ctx_k, ctx_v, C, anchor, want_logits=False)["tokens"]
        else:
            d = np.concatenate([[anchor], np.asarray(drafts_fn(C), dtype=np.int32)])
        vin = np.concatenate([[anchor], d[1:]]).astype(np.int32)
        r = target_forward(target, cache, vin, C, capture=sel)
        k, bonus = accept(d, r["argmax"])
        add_context(r["hidden"], C)   # all B verified rows; only C..C+k are kept
        out.extend(int(t) for t in d[1:k + 1])
        out.append(int(bonus))
        ks.append(k)
        anchor = int(bonus)
        C += k + 1
    return np.array(out[:n_new], dtype=np.int32), ks
