"""Python binding of libdflash (ctypes): argument marshalling only.

Every step of the DFlash draft path runs in the HIP kernels of
``libdflash.so``; this module only converts torch tensors to pointers, calls
the C ABI (``include/dflash.h``) and raises on error.  There is no fallback:
if the library is missing, importing the context class fails loudly.

PyTorch provides the device memory (weights, workspace, KV pool, outputs) and
the stream.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import torch

from .stats import spec_stats  # noqa: F401  (host-side bookkeeping)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")
MAX_LAYERS = 64

DFLASH_F32, DFLASH_BF16 = 0, 1
_STATUS = {0: "DFLASH_OK", -1: "DFLASH_ERR_INVAL", -2: "DFLASH_ERR_CAPACITY", -3: "DFLASH_ERR_HIP",
           -4: "DFLASH_ERR_UNSUPPORTED", -5: "DFLASH_ERR_STATE"}


class DFlashError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")


class Config(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("hidden", C.c_int32), ("target_layers", C.c_int32),
        ("draft_layers", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32), ("block", C.c_int32),
        ("mask_id", C.c_int32), ("page_size", C.c_int32), ("max_ctx", C.c_int32),
        ("max_rows", C.c_int32), ("rope_base", C.c_double), ("eps", C.c_double),
        ("page_seed", C.c_uint64),
    ]


class Weights(C.Structure):
    _fields_ = [
        ("fc", C.c_void_p), ("fc_norm", C.c_void_p),
        ("attn_norm", C.c_void_p * MAX_LAYERS), ("wq", C.c_void_p * MAX_LAYERS),
        ("wk", C.c_void_p * MAX_LAYERS), ("wv", C.c_void_p * MAX_LAYERS),
        ("wo", C.c_void_p * MAX_LAYERS), ("mlp_norm", C.c_void_p * MAX_LAYERS),
        ("wg", C.c_void_p * MAX_LAYERS), ("wu", C.c_void_p * MAX_LAYERS),
        ("wd", C.c_void_p * MAX_LAYERS),
        ("final_norm", C.c_void_p), ("embed", C.c_void_p), ("lm_head", C.c_void_p),
    ]


_lib = None


def lib():
    """Load libdflash.so (built in-tree by ``build.py``); raise if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libdflash.so not built at {LIB_PATH}; run block_diffusion_drafter_context_amd/build.py")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        st = C.c_int
        L.dflash_status_str.restype = C.c_char_p
        L.dflash_status_str.argtypes = [C.c_int]
        L.dflash_last_error.restype = C.c_char_p
        L.dflash_last_error.argtypes = [vp]
        L.dflash_feature_layers.restype = st
        L.dflash_feature_layers.argtypes = [i32, vp]
        L.dflash_page_table.restype = st
        L.dflash_page_table.argtypes = [vp, vp, i32]
        L.dflash_workspace_size.restype = st
        L.dflash_workspace_size.argtypes = [vp, C.POINTER(sz), C.POINTER(sz)]
        L.dflash_create.restype = st
        L.dflash_create.argtypes = [vp, vp, vp, sz, vp, sz, vp, C.POINTER(vp)]
        L.dflash_destroy.restype = st
        L.dflash_destroy.argtypes = [vp]
        L.dflash_length.restype = i32
        L.dflash_length.argtypes = [vp]
        L.dflash_fuse_context.restype = st
        L.dflash_fuse_context.argtypes = [vp, vp, i64, i32, vp, vp]
        L.dflash_fuse_context_static.restype = st
        L.dflash_fuse_context_static.argtypes = [vp, vp, i64, i32, vp, vp]
        L.dflash_inject_kv.restype = st
        L.dflash_inject_kv.argtypes = [vp, vp, i64, i32, i32, vp]
        L.dflash_draft_block.restype = st
        L.dflash_draft_block.argtypes = [vp, vp, vp, vp, vp]
        L.dflash_draft_block_ex.restype = st
        L.dflash_draft_block_ex.argtypes = [vp, vp, vp, vp, vp, i64, vp]
        L.dflash_verify_accept.restype = st
        L.dflash_verify_accept.argtypes = [vp, vp, vp, vp, vp]
        L.dflash_device_length_enable.restype = st
        L.dflash_device_length_enable.argtypes = [vp, vp]
        L.dflash_keep_accepted.restype = st
        L.dflash_keep_accepted.argtypes = [vp, vp, vp]
        L.dflash_set_length_async.restype = st
        L.dflash_set_length_async.argtypes = [vp, i32, vp]
        L.dflash_read_device_length.restype = st
        L.dflash_read_device_length.argtypes = [vp, vp, vp]
        L.dflash_rollback.restype = st
        L.dflash_rollback.argtypes = [vp, i32]
        L.dflash_load_kv.restype = st
        L.dflash_load_kv.argtypes = [vp, vp, vp, i32, i32, vp]
        L.dflash_read_kv.restype = st
        L.dflash_read_kv.argtypes = [vp, i32, i32, vp, vp, vp]
        L.dflash_target_forward.restype = st
        L.dflash_target_forward.argtypes = [vp, vp, i32, vp, vp, vp, i64, vp]
        L.dflash_trace_enable.restype = st
        L.dflash_trace_enable.argtypes = [vp, i32, i32]
        L.dflash_trace_read.restype = st
        L.dflash_trace_read.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(i32)]
        L.dflash_hbm_read_probe.restype = st
        L.dflash_hbm_read_probe.argtypes = [vp, i64, vp, C.POINTER(i64), vp]
        L.dflash_trace_read_each.restype = st
        L.dflash_trace_read_each.argtypes = [vp, C.POINTER(C.c_float), i32, C.POINTER(i32)]
        L.dflash_target_forward_ex.restype = st
        L.dflash_target_forward_ex.argtypes = [vp, vp, vp, i32, vp, vp, vp, i64, vp]
        L.dflash_target_forward_tree.restype = st
        L.dflash_target_forward_tree.argtypes = [vp, vp, vp, i32, vp, vp, vp, i64, vp]
        L.dflash_draft_topk.restype = st
        L.dflash_draft_topk.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp]
        L.dflash_build_tree.restype = st
        L.dflash_build_tree.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
        L.dflash_tree_accept.restype = st
        L.dflash_tree_accept.argtypes = [vp, vp, vp, vp, i32, vp, vp]
        L.dflash_sample_tokens.restype = st
        L.dflash_sample_tokens.argtypes = [vp, vp, i64, i32, C.c_float, C.c_uint64, vp, vp, vp]
        L.dflash_verify_sample.restype = st
        L.dflash_verify_sample.argtypes = [vp, vp, vp, vp, i64, C.c_float, C.c_uint64, vp, vp]
        L.dflash_tree_commit.restype = st
        L.dflash_tree_commit.argtypes = [vp, i32, i32, vp, vp, i64, vp]
        _lib = L
    return _lib


def feature_layers(target_layers: int):
    out = (C.c_int32 * 5)()
    st = lib().dflash_feature_layers(target_layers, out)
    if st:
        raise DFlashError(st, "feature_layers")
    return list(out)


def make_config(shape, max_ctx: int, max_rows: int = 16, page_seed: int = 0) -> Config:
    """Config from a workload shape (``dflash_inputs.Shape`` or any object with the same fields)."""
    c = Config()
    c.dtype = DFLASH_F32 if shape.dtype == "fp32" else DFLASH_BF16
    c.hidden, c.target_layers, c.draft_layers = shape.hidden, shape.target_layers, shape.draft_layers
    c.n_q_heads, c.n_kv_heads, c.head_dim = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    c.ffn, c.vocab, c.block, c.mask_id = shape.ffn, shape.vocab, shape.block, shape.mask_id
    c.page_size, c.max_ctx, c.max_rows = shape.page_size, max_ctx, max_rows
    c.rope_base, c.eps, c.page_seed = shape.rope_base, shape.eps, page_seed
    return c


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> int:
    """One launch of the library's streaming-read kernel over the device tensor
    buf (a measurement aid); returns the bytes it reads."""
    n = C.c_int64()
    st = lib().dflash_hbm_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), C.byref(n),
                                     _stream(stream))
    if st:
        raise DFlashError(st, "hbm_read_probe")
    return n.value


def workspace_size(cfg: Config):
    ws, kv = C.c_size_t(), C.c_size_t()
    st = lib().dflash_workspace_size(C.byref(cfg), C.byref(ws), C.byref(kv))
    if st:
        raise DFlashError(st, "workspace_size")
    return ws.value, kv.value


def page_table(cfg: Config):
    n = (cfg.max_ctx + cfg.page_size - 1) // cfg.page_size
    out = (C.c_int32 * max(n, 1))()
    st = lib().dflash_page_table(C.byref(cfg), out, max(n, 1))
    if st:
        raise DFlashError(st, "page_table")
    return list(out)[:n]


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return t.data_ptr()


def _capture_array(capture, hidden: int):
    """A host array of 5 device pointers with their common row stride, or (None, 0)."""
    if capture is None:
        return None, 0
    assert len(capture) == 5
    live = [t for t in capture if t is not None]
    ld = live[0].stride(0) if live else hidden
    assert all(t.stride(0) == ld for t in live)
    return (C.c_void_p * 5)(*[_p(t) for t in capture]), ld


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


class DFlash:
    """A libdflash context over device weights given as a dict of CUDA tensors.

    Weight names: fc, fc_norm, final_norm, embed, lm_head and per layer l:
    attn_norm.l, wq.l, wk.l, wv.l, wo.l, mlp_norm.l, wg.l, wu.l, wd.l.
    """

    def __init__(self, shape, weights: Dict[str, torch.Tensor], max_ctx: int, max_rows: int = 16,
                 page_seed: int = 0, device=None):
        self.shape = shape
        self.cfg = make_config(shape, max_ctx, max_rows, page_seed)
        self.weights = weights  # keep alive
        self.device = torch.device("cuda") if device is None else torch.device(device)
        w = Weights()
        w.fc, w.fc_norm = _p(weights.get("fc")), _p(weights.get("fc_norm"))
        for l in range(shape.draft_layers):
            for name in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd"):
                t = weights.get(f"{name}.{l}")
                getattr(w, name)[l] = _p(t)
        w.final_norm, w.embed, w.lm_head = _p(weights.get("final_norm")), _p(weights.get("embed")), _p(weights.get("lm_head"))
        self._w = w
        ws, kv = workspace_size(self.cfg)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
        self.kv_pool = torch.empty(max(kv, 256), dtype=torch.uint8, device=self.device)
        h = C.c_void_p()
        st = lib().dflash_create(C.byref(self.cfg), C.byref(w), self.workspace.data_ptr(), ws,
                                 self.kv_pool.data_ptr(), kv, _stream(), C.byref(h))
        if st:
            raise DFlashError(st, "create")
        self.h = h
        self.dtype = shape.torch_dtype

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:
            try:
                _lib.dflash_destroy(h)
            except Exception:  # interpreter shutdown: the library may already be gone
                pass
            self.h = None

    def _check(self, st: int, what: str):
        if st:
            msg = lib().dflash_last_error(self.h)
            raise DFlashError(st, f"{what}: {msg.decode() if msg else ''}")

    @property
    def length(self) -> int:
        return lib().dflash_length(self.h)

    def fuse_context(self, layer_hidden: Sequence[Optional[torch.Tensor]], out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
        """layer_hidden: one tensor [M, H] (or None) per target layer."""
        assert len(layer_hidden) == self.cfg.target_layers
        ref = next(t for t in layer_hidden if t is not None)
        M, ld = ref.shape[0], ref.stride(0)
        if out is None:
            out = torch.empty(M, self.shape.hidden, dtype=self.dtype, device=self.device)
        arr = (C.c_void_p * len(layer_hidden))(*[_p(t) for t in layer_hidden])
        self._check(lib().dflash_fuse_context(self.h, arr, ld, M, out.data_ptr(), _stream(stream)), "fuse_context")
        return out

    def fuse_context_static(self, layer_hidden: Sequence[Optional[torch.Tensor]], out: torch.Tensor, stream=None):
        """fuse_context for M <= 16 rows without context scratch (the library's
        static per-GPU array); out is caller-allocated [M, H]."""
        assert len(layer_hidden) == self.cfg.target_layers
        ref = next(t for t in layer_hidden if t is not None)
        M, ld = ref.shape[0], ref.stride(0)
        arr = (C.c_void_p * len(layer_hidden))(*[_p(t) for t in layer_hidden])
        self._check(lib().dflash_fuse_context_static(self.h, arr, ld, M, out.data_ptr(), _stream(stream)),
                    "fuse_context_static")
        return out

    def inject_kv(self, fused: torch.Tensor, pos0: Optional[int] = None, stream=None):
        """pos0: the current length (default); -1 with the device-resident length."""
        pos0 = self.length if pos0 is None else pos0
        self._check(lib().dflash_inject_kv(self.h, fused.data_ptr(), fused.stride(0), fused.shape[0], pos0,
                                           _stream(stream)), "inject_kv")

    def draft_block(self, anchor: torch.Tensor, tokens: Optional[torch.Tensor] = None, want_logits: bool = False,
                    logits: Optional[torch.Tensor] = None, layers_out: Optional[torch.Tensor] = None, stream=None):
        """anchor: device int32[1].  Returns (tokens int32[B], logits fp32[B, V] or None).
        layers_out: optional device tensor [Ld, B, H] (context dtype) that receives
        the residual stream after every draft layer."""
        B, V = self.shape.block, self.shape.vocab
        if tokens is None:
            tokens = torch.empty(B, dtype=torch.int32, device=self.device)
        if want_logits and logits is None:
            logits = torch.empty(B, V, dtype=torch.float32, device=self.device)
        if layers_out is None:
            st = lib().dflash_draft_block(self.h, anchor.data_ptr(), _p(logits), tokens.data_ptr(), _stream(stream))
        else:
            assert layers_out.shape[:2] == (self.shape.draft_layers, B) and layers_out.stride(0) == B * layers_out.stride(1)
            st = lib().dflash_draft_block_ex(self.h, anchor.data_ptr(), _p(logits), tokens.data_ptr(),
                                             layers_out.data_ptr(), layers_out.stride(1), _stream(stream))
        self._check(st, "draft_block")
        return tokens, logits

    def verify_accept(self, draft: torch.Tensor, target: torch.Tensor, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.device)
        self._check(lib().dflash_verify_accept(self.h, draft.data_ptr(), target.data_ptr(), out.data_ptr(),
                                               _stream(stream)), "verify_accept")
        return out

    def target_forward(self, tokens: torch.Tensor, argmax: Optional[torch.Tensor] = None, want_logits: bool = False,
                       logits: Optional[torch.Tensor] = None, capture: Optional[Sequence[Optional[torch.Tensor]]] = None,
                       stream=None, parent: Optional[torch.Tensor] = None,
                       layers_out: Optional[torch.Tensor] = None):
        """Causal forward of tokens (device int32[M], M <= 16) at positions length..length+M-1,
        or with parent (device int32[M], M <= 32) the tree-masked forward of dflash_target_forward_tree.
        capture: 5 tensors [>= M, H] with one common row stride (or None entries).
        layers_out: [Ld, M, H] device tensor receiving every layer's output (no capture then).
        Returns (argmax int32[M], logits fp32[M, V] or None)."""
        M, V = tokens.shape[0], self.shape.vocab
        if argmax is None:
            argmax = torch.empty(M, dtype=torch.int32, device=self.device)
        if want_logits and logits is None:
            logits = torch.empty(M, V, dtype=torch.float32, device=self.device)
        cap, ld = _capture_array(capture, self.shape.hidden)
        if layers_out is not None:
            assert capture is None and layers_out.shape[:2] == (self.shape.draft_layers, M)
            assert layers_out.stride(0) == M * layers_out.stride(1)
            st = lib().dflash_target_forward_ex(self.h, tokens.data_ptr(), _p(parent), M, _p(logits),
                                                argmax.data_ptr(), layers_out.data_ptr(), layers_out.stride(1),
                                                _stream(stream))
        elif parent is None:
            st = lib().dflash_target_forward(self.h, tokens.data_ptr(), M, _p(logits), argmax.data_ptr(), cap, ld,
                                             _stream(stream))
        else:
            st = lib().dflash_target_forward_tree(self.h, tokens.data_ptr(), parent.data_ptr(), M, _p(logits),
                                                  argmax.data_ptr(), cap, ld, _stream(stream))
        self._check(st, "target_forward")
        return argmax, logits

    # ---- tree verification (DDTree)
    def draft_topk(self, logits: torch.Tensor, K: int, ids: Optional[torch.Tensor] = None,
                   logp: Optional[torch.Tensor] = None, stream=None):
        """Top-K ids and log-probabilities of each row of logits (device fp32 [rows, >= V], rows <= 16)."""
        rows = logits.shape[0]
        if ids is None:
            ids = torch.empty(rows, K, dtype=torch.int32, device=self.device)
        if logp is None:
            logp = torch.empty(rows, K, dtype=torch.float32, device=self.device)
        self._check(lib().dflash_draft_topk(self.h, logits.data_ptr(), logits.stride(0), rows, K, ids.data_ptr(),
                                            logp.data_ptr(), _stream(stream)), "draft_topk")
        return ids, logp

    def build_tree(self, anchor: torch.Tensor, ids: torch.Tensor, logp: torch.Tensor, budget: int,
                   tokens: Optional[torch.Tensor] = None, parent: Optional[torch.Tensor] = None, stream=None):
        """Best-first verification tree: (tokens, parent), device int32[budget + 1]."""
        R, K = ids.shape
        if tokens is None:
            tokens = torch.empty(budget + 1, dtype=torch.int32, device=self.device)
        if parent is None:
            parent = torch.empty(budget + 1, dtype=torch.int32, device=self.device)
        self._check(lib().dflash_build_tree(self.h, anchor.data_ptr(), ids.data_ptr(), logp.data_ptr(), R, K, budget,
                                            tokens.data_ptr(), parent.data_ptr(), _stream(stream)), "build_tree")
        return tokens, parent

    def tree_accept(self, tokens: torch.Tensor, parent: torch.Tensor, target: torch.Tensor,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Device int32[17]: {k, bonus, path[0..14]}."""
        if out is None:
            out = torch.empty(17, dtype=torch.int32, device=self.device)
        self._check(lib().dflash_tree_accept(self.h, tokens.data_ptr(), parent.data_ptr(), target.data_ptr(),
                                             tokens.shape[0], out.data_ptr(), _stream(stream)), "tree_accept")
        return out

    # ---- non-greedy drafting and verification
    def sample_tokens(self, logits: torch.Tensor, temperature: float, seed: int,
                      tokens: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      want_lse: bool = False, stream=None):
        """Gumbel-max draws (device int32[rows]) of logits [rows, >= V] / T, and
        with lse (or want_lse) the rows' log-sum-exp (fp32[rows]).  Returns
        (tokens, lse or None)."""
        rows = logits.shape[0]
        if tokens is None:
            tokens = torch.empty(rows, dtype=torch.int32, device=self.device)
        if want_lse and lse is None:
            lse = torch.empty(rows, dtype=torch.float32, device=self.device)
        self._check(lib().dflash_sample_tokens(self.h, logits.data_ptr(), logits.stride(0), rows, float(temperature),
                                               seed, tokens.data_ptr(), _p(lse), _stream(stream)),
                    "sample_tokens")
        return tokens, lse

    def verify_sample(self, draft: torch.Tensor, draft_logits: torch.Tensor, target_logits: torch.Tensor,
                      temperature: float, seed: int, out: Optional[torch.Tensor] = None, stream=None):
        """Speculative sampling over a block: device int32[2] = {k, token}."""
        assert draft_logits.stride(0) == target_logits.stride(0)
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.device)
        self._check(lib().dflash_verify_sample(self.h, draft.data_ptr(), draft_logits.data_ptr(),
                                               target_logits.data_ptr(), draft_logits.stride(0),
                                               float(temperature), seed, out.data_ptr(), _stream(stream)),
                    "verify_sample")
        return out

    def tree_commit(self, pos0: int, M: int, result: torch.Tensor,
                    capture: Optional[Sequence[Optional[torch.Tensor]]] = None, stream=None):
        cap, ld = _capture_array(capture, self.shape.hidden)
        self._check(lib().dflash_tree_commit(self.h, pos0, M, result.data_ptr(), cap, ld, _stream(stream)),
                    "tree_commit")

    # ---- device-resident length (a step without host round trips; capturable)
    def enable_device_length(self, stream=None):
        self._check(lib().dflash_device_length_enable(self.h, _stream(stream)), "device_length_enable")

    def keep_accepted(self, result: torch.Tensor, stream=None):
        """length += result[0] + 1 on the device (result: a verify_accept output)."""
        self._check(lib().dflash_keep_accepted(self.h, result.data_ptr(), _stream(stream)), "keep_accepted")

    def set_length_async(self, new_len: int, stream=None):
        self._check(lib().dflash_set_length_async(self.h, new_len, _stream(stream)), "set_length_async")

    def read_device_length(self, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """Device int32[2]: {length, capacity-error flag}."""
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.device)
        self._check(lib().dflash_read_device_length(self.h, out.data_ptr(), _stream(stream)), "read_device_length")
        return out

    def rollback(self, new_len: int):
        self._check(lib().dflash_rollback(self.h, new_len), "rollback")

    def load_kv(self, k: torch.Tensor, v: torch.Tensor, pos0: Optional[int] = None, stream=None):
        """k, v: [Ld, M, nkv, d] contiguous device tensors (already rotated K)."""
        pos0 = self.length if pos0 is None else pos0
        assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
        self._check(lib().dflash_load_kv(self.h, k.data_ptr(), v.data_ptr(), k.shape[1], pos0, _stream(stream)),
                    "load_kv")

    def read_kv(self, pos0: int, M: int, stream=None):
        s = self.shape
        k = torch.empty(s.draft_layers, M, s.n_kv_heads, s.head_dim, dtype=self.dtype, device=self.device)
        v = torch.empty_like(k)
        self._check(lib().dflash_read_kv(self.h, pos0, M, k.data_ptr(), v.data_ptr(), _stream(stream)), "read_kv")
        return k, v
