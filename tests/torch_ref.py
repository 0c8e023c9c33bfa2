"""An independent, library-layer formulation of the draft forward (tests only).

Built from torch's own layers (``F.rms_norm``, ``F.scaled_dot_product_attention``,
``F.silu``, complex multiplication for the rotary embedding) in float64, with
rounding to fp32 at the same storage points as the path.  It exists to pin the
C oracle on tiny shapes; it does not share code with either side.
"""
import math

import torch
import torch.nn.functional as F


def _r32(t):
    return t.to(torch.float32).to(torch.float64)


def rope_complex(x, pos, base):
    """x [..., n, d] float64, pos [n]: rotate pairs (i, i + d/2) by pos * base^(-2i/d)
    as multiplication of the complex number x_i + j*x_{i+d/2} by exp(j*angle)."""
    d = x.shape[-1]
    h = d // 2
    inv = torch.tensor([base ** (-2.0 * i / d) for i in range(h)], dtype=torch.float64)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    z = torch.complex(x[..., :h], x[..., h:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def draft_forward(shape, w, ctx_k, ctx_v, C, anchor):
    """fp32-storage draft forward; ctx_k/ctx_v [L, C, nkv, d] already rotated.
    Returns fp32 logits [B, V] as float64."""
    H, B, d = shape.hidden, shape.block, shape.head_dim
    nq, nkv = shape.n_q_heads, shape.n_kv_heads
    eps = shape.eps
    g = lambda k: w[k].to(torch.float64)
    toks = torch.tensor([anchor] + [shape.mask_id] * (B - 1))
    x = g("embed")[toks]
    pos = torch.arange(C, C + B)
    for l in range(shape.draft_layers):
        u = _r32(F.rms_norm(x, (H,), weight=g(f"attn_norm.{l}"), eps=eps))
        q = (u @ g(f"wq.{l}").T).view(B, nq, d).transpose(0, 1)          # [nq, B, d]
        k = (u @ g(f"wk.{l}").T).view(B, nkv, d).transpose(0, 1)         # [nkv, B, d]
        v = _r32((u @ g(f"wv.{l}").T).view(B, nkv, d).transpose(0, 1))
        q = _r32(rope_complex(q, pos, shape.rope_base))
        k = _r32(rope_complex(k, pos, shape.rope_base))
        if C > 0:
            k = torch.cat([ctx_k[l, :C].to(torch.float64).transpose(0, 1), k], dim=1)
            v = torch.cat([ctx_v[l, :C].to(torch.float64).transpose(0, 1), v], dim=1)
        rep = nq // nkv
        k = k.repeat_interleave(rep, dim=0)
        v = v.repeat_interleave(rep, dim=0)
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=1.0 / math.sqrt(d))[0]
        o = _r32(o.transpose(0, 1).reshape(B, nq * d))
        x = _r32(x + _r32(o @ g(f"wo.{l}").T))
        u = _r32(F.rms_norm(x, (H,), weight=g(f"mlp_norm.{l}"), eps=eps))
        h = _r32(F.silu(u @ g(f"wg.{l}").T) * (u @ g(f"wu.{l}").T))
        x = _r32(x + _r32(h @ g(f"wd.{l}").T))
    z = _r32(F.rms_norm(x, (H,), weight=g("final_norm"), eps=eps))
    return _r32(z @ g("lm_head").T)


def fuse(shape, w, slabs):
    """fp32-storage fusion: RMSNorm(W_fc . concat(slabs)) for all rows."""
    x = torch.cat([s.to(torch.float64) for s in slabs], dim=1)
    y = _r32(x @ w["fc"].to(torch.float64).T)
    return _r32(F.rms_norm(y, (shape.hidden,), weight=w["fc_norm"].to(torch.float64), eps=shape.eps))


def inject(shape, w, fused, pos0):
    """fp32-storage KV injection of all rows: K, V [L, M, nkv, d]."""
    M = fused.shape[0]
    c = fused.to(torch.float64)
    pos = torch.arange(pos0, pos0 + M)
    ks, vs = [], []
    for l in range(shape.draft_layers):
        k = (c @ w[f"wk.{l}"].to(torch.float64).T).view(M, shape.n_kv_heads, shape.head_dim)
        k = rope_complex(k.transpose(0, 1), pos, shape.rope_base).transpose(0, 1)
        v = (c @ w[f"wv.{l}"].to(torch.float64).T).view(M, shape.n_kv_heads, shape.head_dim)
        ks.append(_r32(k))
        vs.append(_r32(v))
    return torch.stack(ks), torch.stack(vs)


def target_forward(shape, w, tokens, n_layers, pos=None, visible=None):
    """fp32-storage causal forward of `tokens` from position 0 (a prefill of
    the whole sequence at once): the autoregressive model of [A] §1.1, written
    with an explicit lower-triangular visibility mask (key j is visible to
    query i iff j <= i, the query's own key included).  `pos` and `visible`
    ([n, n] bool) replace the positions 0..n-1 and that mask when given.
    Returns (logits [n, V], hidden [n_layers, n, H]) where hidden[l] is the
    residual stream right after decoder layer l (before any final norm)."""
    H, d = shape.hidden, shape.head_dim
    nq, nkv = shape.n_q_heads, shape.n_kv_heads
    eps = shape.eps
    g = lambda k: w[k].to(torch.float64)
    n = len(tokens)
    x = g("embed")[torch.as_tensor(list(tokens), dtype=torch.long)]
    if pos is None:
        pos = torch.arange(n)
    if visible is None:
        visible = torch.ones(n, n, dtype=torch.bool).tril()
    outs = []
    for l in range(n_layers):
        u = _r32(F.rms_norm(x, (H,), weight=g(f"attn_norm.{l}"), eps=eps))
        q = (u @ g(f"wq.{l}").T).view(n, nq, d).transpose(0, 1)
        k = (u @ g(f"wk.{l}").T).view(n, nkv, d).transpose(0, 1)
        v = _r32((u @ g(f"wv.{l}").T).view(n, nkv, d).transpose(0, 1))
        q = _r32(rope_complex(q, pos, shape.rope_base))
        k = _r32(rope_complex(k, pos, shape.rope_base))
        rep = nq // nkv
        k = k.repeat_interleave(rep, dim=0)
        v = v.repeat_interleave(rep, dim=0)
        o = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=visible,
                                           scale=1.0 / math.sqrt(d))[0]
        o = _r32(o.transpose(0, 1).reshape(n, nq * d))
        x = _r32(x + _r32(o @ g(f"wo.{l}").T))
        u = _r32(F.rms_norm(x, (H,), weight=g(f"mlp_norm.{l}"), eps=eps))
        h = _r32(F.silu(u @ g(f"wg.{l}").T) * (u @ g(f"wu.{l}").T))
        x = _r32(x + _r32(h @ g(f"wd.{l}").T))
        outs.append(x.clone())
    z = _r32(F.rms_norm(x, (H,), weight=g("final_norm"), eps=eps))
    return _r32(z @ g("lm_head").T), torch.stack(outs)


def tree_forward(shape, w, prefix, tree_tokens, parent, n_layers):
    """[A] §8.2 tree verification written as one masked prefill: the prefix
    (positions 0..P-1, causal) followed by the tree's rows, where row j sits
    at position P + (its number of ancestors) and sees the whole prefix, its
    ancestors and itself.  Ancestors are found by set closure over the parent
    relation (not by walking up).  Returns (logits, hidden) of the tree rows."""
    P, n = len(prefix), len(tree_tokens)
    anc = torch.eye(n, dtype=torch.bool)
    for j in range(1, n):
        anc[j, parent[j]] = True
    for _ in range(n):  # transitive closure: anc = anc OR anc.anc
        anc = anc | ((anc.double() @ anc.double()) > 0)
    vis = torch.zeros(P + n, P + n, dtype=torch.bool)
    vis[:P, :P] = torch.ones(P, P, dtype=torch.bool).tril()
    vis[P:, :P] = True
    vis[P:, P:] = anc
    pos = torch.cat([torch.arange(P), P + anc.sum(dim=1) - 1])
    lg, hid = target_forward(shape, w, list(prefix) + list(tree_tokens), n_layers, pos=pos, visible=vis)
    return lg[P:], hid[:, P:]
