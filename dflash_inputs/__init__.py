"""Seeded synthetic inputs for the DFlash draft path.

This module holds workload shapes and random draws only: no step of the
method's arithmetic lives here.  Both the HIP path (through its Python
binding) and the CPU oracle consume the exact same bytes produced here.

Workloads (shapes follow the Qwen3-8B / 27B-class targets and the context
lengths swept in the community benchmark of the DFlash llama.cpp merge):

* ``tiny_fp32``        hidden 256, 8 target layers, 2 draft layers, 4/2 heads x 64,
                       FFN 688, vocab 1024, context 128, fp32, seed 0
* ``qwen3_8b_4k``      hidden 4096, 36 target layers, 5 draft layers, 32/8 x 128,
                       FFN 12288, vocab 151936, context 4096, bf16, seed 1
* ``qwen3_8b_36k``     the same shape at context 36864, seed 1
* ``dense27b_36k``     hidden 5120, 64 target layers, 5 draft layers, 40/8 x 128,
                       FFN 17408, vocab 151936, context 36864, bf16, seed 2
* ``fusion_prefill_32k`` the 27B-class shape used for prefill-side fusion and
                       KV injection of 32768 context rows, bf16, seed 3
* ``toy_e2e``          toy target hidden 1024, 8 layers, 16/4 x 64, FFN 2816,
                       vocab 32000; draft of the same shape with 3 layers, seed 4

Every tensor is drawn from its own ``torch.Generator`` whose seed mixes the
workload seed with a stable tag, so any one tensor can be regenerated without
drawing the others.  Samples are fp32 and then rounded to the storage dtype.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    dtype: str  # 'fp32' | 'bf16'
    hidden: int
    target_layers: int
    draft_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    ctx: int
    seed: int
    block: int = 16
    rope_base: float = 10000.0
    eps: float = 1e-6
    w_std: float = 0.02
    page_size: int = 256

    @property
    def mask_id(self) -> int:
        # a dedicated mask token: the last id of the vocabulary
        return self.vocab - 1

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


SHAPES: Dict[str, Shape] = {
    "tiny_fp32": Shape("tiny_fp32", "fp32", 256, 8, 2, 4, 2, 64, 688, 1024, 128, 0),
    "qwen3_8b_4k": Shape("qwen3_8b_4k", "bf16", 4096, 36, 5, 32, 8, 128, 12288, 151936, 4096, 1),
    "qwen3_8b_36k": Shape("qwen3_8b_36k", "bf16", 4096, 36, 5, 32, 8, 128, 12288, 151936, 36864, 1),
    "dense27b_36k": Shape("dense27b_36k", "bf16", 5120, 64, 5, 40, 8, 128, 17408, 151936, 36864, 2),
    "fusion_prefill_32k": Shape("fusion_prefill_32k", "bf16", 5120, 64, 5, 40, 8, 128, 17408, 151936, 32768, 3),
    "toy_e2e": Shape("toy_e2e", "bf16", 1024, 8, 3, 16, 4, 64, 2816, 32000, 2048, 4),
}

# toy end-to-end loop: prompt length and number of generated tokens
TOY_PROMPT = 2048
TOY_GENERATE = 512
# synthetic target of the tiny workload agrees with each draft position w.p. 0.3
SYNTH_AGREE_P = 0.3


def _gen(seed: int, tag: str) -> torch.Generator:
    mixed = (seed * 0x9E3779B1 + zlib.crc32(tag.encode())) & 0x7FFFFFFFFFFFFFFF
    return torch.Generator().manual_seed(mixed)


def normal(shape, seed: int, tag: str, std: float, dtype: torch.dtype) -> torch.Tensor:
    """N(0, std^2) samples in fp32, rounded once to ``dtype`` (CPU tensor)."""
    x = torch.randn(tuple(shape), generator=_gen(seed, tag), dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype).contiguous()


def uniform_int(n: int, lo: int, hi: int, seed: int, tag: str) -> torch.Tensor:
    """n integers uniform in [lo, hi) (int32)."""
    return torch.randint(lo, hi, (n,), generator=_gen(seed, tag), dtype=torch.int64).to(torch.int32)


def random_tree(n: int, seed: int, tag: str) -> np.ndarray:
    """Parent array of a random rooted tree on n nodes in topological order:
    parent[0] = -1, parent[j] uniform in [0, j)."""
    u = uniform01(max(n, 1), seed, tag).numpy()
    par = np.array([-1] + [int(u[j] * j) for j in range(1, n)], dtype=np.int32)
    return par[:n]


def chain_tree(n: int) -> np.ndarray:
    """Parent array of a chain: node j's parent is j-1."""
    return np.arange(-1, n - 1, dtype=np.int32)


def uniform01(n: int, seed: int, tag: str) -> torch.Tensor:
    return torch.rand((n,), generator=_gen(seed, tag), dtype=torch.float64)


def draft_weights(s: Shape, need_draft: bool = True, need_lm: bool = True,
                  gains: str = "ones", layers: Optional[List[int]] = None) -> Dict[str, torch.Tensor]:
    """Random-init draft weights of shape ``s`` (row-major [out, in] matrices).

    gains='ones' gives unit RMSNorm gains (the workloads' setting); gains='random'
    draws them from U(0.5, 1.5) so tests can see a dropped or misplaced gain.
    Only W_k / W_v are drawn per layer when ``need_draft`` is False (injection only).
    """
    dt, H, std = s.torch_dtype, s.hidden, s.w_std
    nq, nkv, d, F = s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn
    w: Dict[str, torch.Tensor] = {}

    def gain(tag):
        if gains == "ones":
            return torch.ones(H, dtype=dt)
        g = torch.rand((H,), generator=_gen(s.seed, tag), dtype=torch.float32) + 0.5
        return g.to(dt)

    w["fc"] = normal((H, 5 * H), s.seed, "fc", std, dt)
    w["fc_norm"] = gain("fc_norm")
    for l in (range(s.draft_layers) if layers is None else layers):
        w[f"wk.{l}"] = normal((nkv * d, H), s.seed, f"wk.{l}", std, dt)
        w[f"wv.{l}"] = normal((nkv * d, H), s.seed, f"wv.{l}", std, dt)
        if need_draft:
            w[f"attn_norm.{l}"] = gain(f"attn_norm.{l}")
            w[f"wq.{l}"] = normal((nq * d, H), s.seed, f"wq.{l}", std, dt)
            w[f"wo.{l}"] = normal((H, nq * d), s.seed, f"wo.{l}", std, dt)
            w[f"mlp_norm.{l}"] = gain(f"mlp_norm.{l}")
            w[f"wg.{l}"] = normal((F, H), s.seed, f"wg.{l}", std, dt)
            w[f"wu.{l}"] = normal((F, H), s.seed, f"wu.{l}", std, dt)
            w[f"wd.{l}"] = normal((H, F), s.seed, f"wd.{l}", std, dt)
    if need_draft:
        w["final_norm"] = gain("final_norm")
    if need_lm:
        w["embed"] = normal((s.vocab, H), s.seed, "embed", std, dt)
        w["lm_head"] = normal((s.vocab, H), s.seed, "lm_head", std, dt)
    return w


def target_hidden(s: Shape, layer: int, rows: int, tag: str = "ctx") -> torch.Tensor:
    """Hidden state of target layer ``layer`` for ``rows`` tokens, N(0,1), [rows, H]."""
    return normal((rows, s.hidden), s.seed, f"hidden.{tag}.{layer}", 1.0, s.torch_dtype)


def fused_context(s: Shape, rows: int, tag: str = "fused") -> torch.Tensor:
    """Stand-in for fused context features (unit RMS, like an RMSNorm output), [rows, H]."""
    return normal((rows, s.hidden), s.seed, tag, 1.0, s.torch_dtype)


def context_kv(s: Shape, ctx: Optional[int] = None, tag: str = "kv"):
    """Stand-in for an already-injected draft KV cache.

    Returns K, V of shape [Ld, C, nkv, d].  Entries are N(0, (w_std*sqrt(H))^2),
    the distribution of a projection of unit-RMS features by N(0, w_std^2) weights.
    """
    C = s.ctx if ctx is None else ctx
    std = s.w_std * float(np.sqrt(s.hidden))
    shape = (s.draft_layers, C, s.n_kv_heads, s.head_dim)
    return (normal(shape, s.seed, tag + ".k", std, s.torch_dtype),
            normal(shape, s.seed, tag + ".v", std, s.torch_dtype))


def anchor_token(s: Shape, tag: str = "anchor") -> int:
    return int(uniform_int(1, 0, s.vocab, s.seed, tag)[0])


def target_coins(s: Shape, tag: str = "coins"):
    """Pre-drawn randomness of the synthetic target argmax for one block.

    u[j] ~ U(0,1) and r[j] in [1, V-1] for j = 1..B-1 (index 0 unused), and a
    free last token g_last ~ U[0, V).
    """
    B = s.block
    u = uniform01(B, s.seed, tag + ".u")
    r = uniform_int(B, 1, s.vocab, s.seed, tag + ".r")
    last = int(uniform_int(1, 0, s.vocab, s.seed, tag + ".last")[0])
    return u, r, last


def synthetic_target_argmax(drafts, u, r, last: int, vocab: int, p: float = SYNTH_AGREE_P):
    """Synthetic target argmax g[0..B-1] that agrees with the draft at each
    position with probability p: g[j-1] = d[j] if u[j] < p else (d[j] + r[j]) mod V.

    ``drafts`` is the full block output [B] (index 0 = anchor row, unused).
    Works on numpy arrays or torch tensors (device tensors stay on device).
    """
    if isinstance(drafts, torch.Tensor):
        d = drafts.to(torch.int64)
        uu = torch.as_tensor(u, device=d.device)
        rr = torch.as_tensor(r, device=d.device).to(torch.int64)
        alt = torch.remainder(d + rr, vocab)
        g_next = torch.where(uu < p, d, alt)
        g = torch.empty_like(d)
        g[:-1] = g_next[1:]
        g[-1] = last
        return g.to(torch.int32)
    d = np.asarray(drafts, dtype=np.int64)
    uu = np.asarray(u)
    rr = np.asarray(r, dtype=np.int64)
    g = np.empty_like(d)
    g[:-1] = np.where(uu[1:] < p, d[1:], (d[1:] + rr[1:]) % vocab)
    g[-1] = last
    return g.astype(np.int32)


def toy_prompt(s: Shape, n: int = TOY_PROMPT) -> torch.Tensor:
    """Seeded uniform-random prompt token ids (excluding the mask id)."""
    return uniform_int(n, 0, s.vocab - 1, s.seed, "prompt")


def toy_target_weights(s: Shape, gains: str = "ones") -> Dict[str, torch.Tensor]:
    """Random-init weights of the toy Llama-style target (same layer shape as
    the draft, ``s.target_layers`` layers, causal); shares embed / lm_head with
    the draft (drawn under the draft's tags)."""
    dt, H, std = s.torch_dtype, s.hidden, s.w_std
    nq, nkv, d, F = s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn
    w: Dict[str, torch.Tensor] = {}
    for l in range(s.target_layers):
        w[f"attn_norm.{l}"] = torch.ones(H, dtype=dt)
        w[f"wq.{l}"] = normal((nq * d, H), s.seed, f"t.wq.{l}", std, dt)
        w[f"wk.{l}"] = normal((nkv * d, H), s.seed, f"t.wk.{l}", std, dt)
        w[f"wv.{l}"] = normal((nkv * d, H), s.seed, f"t.wv.{l}", std, dt)
        w[f"wo.{l}"] = normal((H, nq * d), s.seed, f"t.wo.{l}", std, dt)
        w[f"mlp_norm.{l}"] = torch.ones(H, dtype=dt)
        w[f"wg.{l}"] = normal((F, H), s.seed, f"t.wg.{l}", std, dt)
        w[f"wu.{l}"] = normal((F, H), s.seed, f"t.wu.{l}", std, dt)
        w[f"wd.{l}"] = normal((H, F), s.seed, f"t.wd.{l}", std, dt)
    w["final_norm"] = torch.ones(H, dtype=dt)
    w["embed"] = normal((s.vocab, H), s.seed, "embed", std, dt)
    w["lm_head"] = normal((s.vocab, H), s.seed, "lm_head", std, dt)
    return w


def page_permutation(n_pages: int, seed: int) -> np.ndarray:
    """A seeded permutation of physical page ids (tests use it to scramble the page table)."""
    g = _gen(seed, "pages")
    return torch.randperm(n_pages, generator=g).numpy().astype(np.int32)
