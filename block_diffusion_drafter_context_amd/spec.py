"""Greedy, sampled and DFlash speculative generation over libdflash contexts.

Orchestration only: every step of the model runs in libdflash calls; torch
holds the device buffers and moves a few token ids between them.

A *target* is a ``DFlash`` context whose decoder stack is the target model
(its ``draft_layers`` field set to the target's layer count) used through
``target_forward``; a *draft* is a ``DFlash`` context holding the draft model
and its fusion weights.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import torch

from . import DFlash, feature_layers

ROWS = 16  # rows per target call: the largest block libdflash verifies at once


class _Capture:
    """Device buffers for the five captured target layers of one call."""

    def __init__(self, target: DFlash, rows: int = ROWS):
        s = target.shape
        self.sel = feature_layers(s.target_layers)
        self.slabs = [torch.empty(rows, s.hidden, dtype=target.dtype, device=target.device) for _ in range(5)]
        self.n_layers = s.target_layers

    def views(self, M: int):
        return [t[:M] for t in self.slabs]

    def layer_list(self, M: int):
        lst: List[Optional[torch.Tensor]] = [None] * self.n_layers
        for i, l in enumerate(self.sel):
            lst[l] = self.slabs[i][:M]
        return lst


def prefill(target: DFlash, prompt: torch.Tensor, draft: Optional[DFlash] = None,
            last_logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Run the prompt (device int32[P]) through the target in calls of up to 16
    rows; with a draft, fuse and inject every call's captured features as its
    context.  Returns the greedy first token as device int32[1]; last_logits
    (device fp32 [1, V]) receives the logits of the prompt's last row."""
    cap = _Capture(target)
    am = torch.empty(ROWS, dtype=torch.int32, device=target.device)
    fused = None
    if draft is not None:
        fused = torch.empty(ROWS, draft.shape.hidden, dtype=draft.dtype, device=draft.device)
    lg = None
    if last_logits is not None:
        lg = torch.empty(ROWS, target.shape.vocab, dtype=torch.float32, device=target.device)
    P = prompt.shape[0]
    M = 0
    for r0 in range(0, P, ROWS):
        M = min(ROWS, P - r0)
        last = r0 + M == P
        target.target_forward(prompt[r0:r0 + M], argmax=am[:M], capture=cap.views(M) if draft is not None else None,
                              logits=lg[:M] if last and lg is not None else None)
        if draft is not None:
            f = draft.fuse_context(cap.layer_list(M), out=fused[:M])
            draft.inject_kv(f, r0)
    if last_logits is not None:
        last_logits.copy_(lg[M - 1:M])
    return am[M - 1:M].clone()


def greedy_generate(target: DFlash, prompt: torch.Tensor, n_new: int) -> torch.Tensor:
    """Plain greedy decoding: one target row per call.  Device int32[n_new]."""
    out = torch.empty(n_new, dtype=torch.int32, device=target.device)
    out[0:1].copy_(prefill(target, prompt))
    for i in range(1, n_new):
        target.target_forward(out[i - 1:i], argmax=out[i:i + 1])
    return out


def spec_generate(target: DFlash, draft: DFlash, prompt: torch.Tensor, n_new: int,
                  drafts_fn: Optional[Callable[[int], Sequence[int]]] = None) -> Tuple[List[int], List[int]]:
    """DFlash speculative decoding with greedy block verification.

    Per step at context length C with anchor a (the last emitted token, at C):
    draft the block [a, mask, ...] (or take drafts_fn(C) -> B-1 ids), verify
    [a, d_1..d_{B-1}] with one causal target call, accept the k leading drafts
    that equal the target's tokens, emit them and the target's next token
    (bonus); fuse and inject all B verified rows into the draft, then keep
    C + k + 1 positions in both caches.  Returns (tokens, k of every step)."""
    B = draft.shape.block
    dev = target.device
    first = prefill(target, prompt, draft)
    cap = _Capture(target)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    vin = torch.empty(B, dtype=torch.int32, device=dev)
    g = torch.empty(B, dtype=torch.int32, device=dev)
    res = torch.empty(2, dtype=torch.int32, device=dev)
    fused = torch.empty(B, draft.shape.hidden, dtype=draft.dtype, device=dev)
    anchor = first.clone()
    out = [int(first.item())]
    ks: List[int] = []
    C = prompt.shape[0]
    while len(out) < n_new:
        if drafts_fn is None:
            draft.draft_block(anchor, tokens=tok)
        else:
            tok[1:].copy_(torch.tensor(list(drafts_fn(C)), dtype=torch.int32))
        vin[0:1].copy_(anchor)
        vin[1:].copy_(tok[1:])
        target.target_forward(vin, argmax=g, capture=cap.views(B))
        draft.verify_accept(vin, g, out=res)
        f = draft.fuse_context(cap.layer_list(B), out=fused)
        draft.inject_kv(f, C)
        host = torch.cat([res, vin]).cpu()
        k, bonus = int(host[0]), int(host[1])
        target.rollback(C + k + 1)
        draft.rollback(C + k + 1)
        out.extend(int(t) for t in host[3:3 + k])
        out.append(bonus)
        ks.append(k)
        anchor.copy_(res[1:2])
        C += k + 1
    return out[:n_new], ks


def spec_tree_generate(target: DFlash, draft: DFlash, prompt: torch.Tensor, n_new: int, K: int = 4,
                       budget: int = 15,
                       trees_fn: Optional[Callable[[int], Tuple[Sequence[int], Sequence[int]]]] = None
                       ) -> Tuple[List[int], List[int]]:
    """DFlash speculative decoding with tree verification (DDTree).

    Per step at context length C with anchor a: draft the block with logits,
    take the top-K tokens of every drafted position, build the best-first tree
    of `budget` nodes rooted at a (or take trees_fn(C) -> (node tokens after
    the root, parents), parents indexing [root, nodes...]), verify it with one
    tree-masked target call, accept the longest matching root path, move the
    accepted rows behind the root in the target's cache and captured features,
    fuse and inject those k + 1 rows into the draft, keep C + k + 1 positions
    in both caches.  Returns (tokens, k of every step)."""
    B = draft.shape.block
    dev = target.device
    first = prefill(target, prompt, draft)
    n_max = max(ROWS, budget + 1)  # a tree of more than 16 nodes is verified in two target passes
    cap = _Capture(target, n_max)
    lg = torch.empty(B, draft.shape.vocab, dtype=torch.float32, device=dev)
    dtok = torch.empty(B, dtype=torch.int32, device=dev)
    g = torch.empty(n_max, dtype=torch.int32, device=dev)
    res = torch.empty(17, dtype=torch.int32, device=dev)
    fused = torch.empty(ROWS, draft.shape.hidden, dtype=draft.dtype, device=dev)
    anchor = first.clone()
    out = [int(first.item())]
    ks: List[int] = []
    C = prompt.shape[0]
    while len(out) < n_new:
        if trees_fn is None:
            draft.draft_block(anchor, tokens=dtok, logits=lg)
            ids, lp = draft.draft_topk(lg[1:], K)
            ttok, tpar = draft.build_tree(anchor, ids, lp, budget)
        else:
            nodes, parents = trees_fn(C)
            ttok = torch.empty(len(nodes) + 1, dtype=torch.int32, device=dev)
            ttok[0:1].copy_(anchor)
            ttok[1:].copy_(torch.tensor(list(nodes), dtype=torch.int32))
            tpar = torch.tensor([-1] + list(parents), dtype=torch.int32, device=dev)
        M = ttok.shape[0]
        target.target_forward(ttok, argmax=g[:M], capture=cap.views(M), parent=tpar)
        target.tree_accept(ttok, tpar, g[:M], out=res)
        target.tree_commit(C, M, res, capture=cap.views(M))
        host = torch.cat([res, ttok]).cpu()
        k, bonus = int(host[0]), int(host[1])
        path = [int(j) for j in host[2:2 + k]]
        target.rollback(C + k + 1)
        f = draft.fuse_context(cap.layer_list(k + 1), out=fused[:k + 1])
        draft.inject_kv(f, C)
        out.extend(int(host[17 + j]) for j in path)
        out.append(bonus)
        ks.append(k)
        anchor.copy_(res[1:2])
        C += k + 1
    return out[:n_new], ks


def step_seed(seed: int, step: int) -> int:
    """The generator stream of one step: seed + (step + 1) * 0x9E3779B97F4A7C15 mod 2^64."""
    return (seed + (step + 1) * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF


def spec_sample_generate(target: DFlash, draft: DFlash, prompt: torch.Tensor, n_new: int, temperature: float,
                         seed: int, on_step: Optional[Callable[..., None]] = None) -> Tuple[List[int], List[int]]:
    """DFlash speculative decoding at temperature T with the speculative
    sampling rule.

    The first token is a Gumbel-max draw from the prompt's last target row
    (stream step_seed(seed, 0), row 0).  Per step s >= 1 at context length C
    with anchor a: draft the block with logits, draw d_1..d_{B-1} from the
    draft's rows 1..B-1 (stream step_seed(seed, s)), verify [a, d_1..d_{B-1}]
    with one causal target call for its logits, and apply the rule (same
    stream): k accepted drafts and the next token.  Fuse and inject all B
    verified rows into the draft and keep C + k + 1 positions in both caches.
    on_step(C, seed, block, draft_logits, target_logits, result), when given,
    sees every step's device buffers.  Returns (tokens, k of every step)."""
    B = draft.shape.block
    V = draft.shape.vocab
    dev = target.device
    first_lg = torch.empty(1, V, dtype=torch.float32, device=dev)
    prefill(target, prompt, draft, last_logits=first_lg)
    first = torch.empty(1, dtype=torch.int32, device=dev)
    draft.sample_tokens(first_lg, temperature, step_seed(seed, 0), tokens=first)
    cap = _Capture(target)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    vin = torch.empty(B, dtype=torch.int32, device=dev)
    g = torch.empty(B, dtype=torch.int32, device=dev)
    res = torch.empty(2, dtype=torch.int32, device=dev)
    dlg = torch.empty(B, V, dtype=torch.float32, device=dev)
    tlg = torch.empty(B, V, dtype=torch.float32, device=dev)
    fused = torch.empty(B, draft.shape.hidden, dtype=draft.dtype, device=dev)
    anchor = first.clone()
    out = [int(first.item())]
    ks: List[int] = []
    C = prompt.shape[0]
    step = 0
    while len(out) < n_new:
        step += 1
        sd = step_seed(seed, step)
        draft.draft_block(anchor, tokens=tok, logits=dlg)
        vin[0:1].copy_(anchor)
        draft.sample_tokens(dlg[1:], temperature, sd, tokens=vin[1:])
        target.target_forward(vin, argmax=g, logits=tlg, capture=cap.views(B))
        draft.verify_sample(vin, dlg, tlg, temperature, sd, out=res)
        if on_step is not None:
            on_step(C, sd, vin, dlg, tlg, res)
        f = draft.fuse_context(cap.layer_list(B), out=fused)
        draft.inject_kv(f, C)
        host = torch.cat([res, vin]).cpu()
        k, nxt = int(host[0]), int(host[1])
        target.rollback(C + k + 1)
        draft.rollback(C + k + 1)
        out.extend(int(t) for t in host[3:3 + k])
        out.append(nxt)
        ks.append(k)
        anchor.copy_(res[1:2])
        C += k + 1
    return out[:n_new], ks
