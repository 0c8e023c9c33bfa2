"""Tree verification (DDTree, "DFlash 深度解析…" §8.2) through the C ABI against
the oracle:

* top-K of draft logits: ids exact (same fp32 logits on both sides, ties to
  the lower id), log-probabilities within 1e-5;
* the best-first tree: tokens and parents exact on the same fp32 inputs;
* the tree-masked target forward over seeded paged KV: logits, tokens,
  captured layers and the tree rows' KV against the oracle's tree forward;
  with a chain for parents it is bit-identical to the causal forward;
* acceptance: exact against the oracle's walk on random trees;
* compaction of the accepted rows: the KV slots and captured rows move
  bit for bit.
"""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from oracle import ddtree
from tests.gpu_helpers import assert_logits, assert_rows_close, assert_tokens, check_target_layers, dev

pytestmark = pytest.mark.gpu

TR_BF16 = di.Shape("tr_bf16", "bf16", hidden=512, target_layers=8, draft_layers=8, n_q_heads=8,
                   n_kv_heads=2, head_dim=128, ffn=1376, vocab=4000, ctx=300, seed=51)
TR_BF16_D64 = TR_BF16.replace(name="tr_bf16_d64", n_q_heads=16, n_kv_heads=4, head_dim=64, seed=52)
TR_FP32_G5 = di.Shape("tr_fp32_g5", "fp32", hidden=320, target_layers=8, draft_layers=8, n_q_heads=10,
                      n_kv_heads=2, head_dim=64, ffn=688, vocab=1024, ctx=300, seed=53)


@pytest.fixture(scope="module")
def dl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_drafter_context_amd as m
    m.lib()
    return m


def sync():
    torch.cuda.synchronize()


def _vocab_ctx(dl, V):
    """A small context whose vocabulary is V (top-K and tree build need only V)."""
    s = di.Shape(f"v{V}", "bf16", hidden=64, target_layers=8, draft_layers=1, n_q_heads=2, n_kv_heads=1,
                 head_dim=64, ffn=96, vocab=V, ctx=16, seed=5)
    return dl.DFlash(s, dev(di.draft_weights(s, need_draft=False, need_lm=False)), max_ctx=64)


def _logits(R, V, tag):
    x = di.normal((R, V), 61, tag, 2.0, torch.float32).numpy().copy()
    x[0] = 0.25                      # a row of equal values: ids 0..K-1
    for r in range(1, R):            # exact ties at and next to the top
        top = int(np.argmax(x[r]))
        x[r, (top * 7 + 3) % V] = x[r, top]
        x[r, (top + 11) % V] = x[r, top]
    return x


# ------------------------------------------------------------------ top-K

@pytest.mark.parametrize("V,K", [(151936, 16), (151936, 4), (32000, 1), (4000, 16), (1008, 7)])
def test_topk_matches_oracle(dl, V, K):
    ctx = _vocab_ctx(dl, V)
    x = _logits(15, V, f"topk{V}")
    buf = torch.full((15, V + 48), float("nan"), dtype=torch.float32)  # a row stride beyond V
    buf[:, :V] = torch.from_numpy(x)
    g = buf.cuda()
    print(f"[tree] top-k V={V} K={K}", flush=True)
    ids, lp = ctx.draft_topk(g[:, :V], K)
    sync()
    rid, rlp = ddtree.topk_logprobs(x, K)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(lp.cpu().numpy().astype(np.float64), rlp, rtol=1e-6, atol=1e-5)
    assert (lp.cpu().numpy() <= 0).all()


# ------------------------------------------------------------------ tree build

def _tree_inputs(R, K, V, ties):
    rng = np.random.default_rng(100 * R + K + (7 if ties else 0))
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(R)]).astype(np.int32)
    lp = -np.sort(rng.exponential(1.0, (R, K)), axis=1).astype(np.float32)
    if ties:
        lp[:, K // 2:] = lp[:, K // 2:K // 2 + 1]           # equal candidates within a depth
        lp[1::2] = lp[0]                                    # equal rows: equal scores across branches
        lp[:, 0] = np.where(np.arange(R) % 3 == 0, 0.0, lp[:, 0])  # log-probability 0: child == parent
    return ids, lp


@pytest.mark.parametrize("R,K,budget,ties", [(15, 4, 15, False), (15, 16, 15, True), (15, 1, 15, False),
                                             (3, 2, 6, True), (2, 3, 0, False), (15, 8, 9, True),
                                             (5, 2, 15, False), (15, 4, 22, False), (15, 16, 31, True),
                                             (4, 2, 30, False)])
def test_build_tree_matches_oracle(dl, R, K, budget, ties):
    V = 4000
    ctx = _vocab_ctx(dl, V)
    ids, lp = _tree_inputs(R, K, V, ties)
    anchor = torch.tensor([1234], dtype=torch.int32, device="cuda")
    tok, par = ctx.build_tree(anchor, torch.from_numpy(ids).cuda(), torch.from_numpy(lp).cuda(), budget)
    sync()
    ref = ddtree.build_tree(1234, ids, lp, budget)
    assert tok.cpu().numpy().tolist() == ref["tokens"].tolist()
    assert par.cpu().numpy().tolist() == ref["parent"].tolist()


def test_topk_then_tree_on_draft_logits(dl):
    """The two steps chained on device at the 8B vocabulary, checked against
    the oracle on the GPU's own intermediate values."""
    V = 151936
    ctx = _vocab_ctx(dl, V)
    x = di.normal((15, V), 62, "chain", 3.0, torch.float32)
    g = x.cuda()
    anchor = torch.tensor([77], dtype=torch.int32, device="cuda")
    for K in (2, 5, 16):
        ids, lp = ctx.draft_topk(g, K)
        tok, par = ctx.build_tree(anchor, ids, lp, 15)
        sync()
        rid, _ = ddtree.topk_logprobs(x.numpy(), K)
        assert np.array_equal(ids.cpu().numpy(), rid)
        ref = ddtree.build_tree(77, ids.cpu().numpy(), lp.cpu().numpy(), 15)
        assert tok.cpu().numpy().tolist() == ref["tokens"].tolist()
        assert par.cpu().numpy().tolist() == ref["parent"].tolist()


# ------------------------------------------------------------------ acceptance

def test_tree_accept_matches_oracle(dl):
    ctx = _vocab_ctx(dl, 1008)
    rng = np.random.default_rng(12)
    cases, outs = [], []
    for t in range(304):
        n = int(rng.integers(1, 17 if t % 2 else 33))       # trees of up to 32 nodes
        par = di.random_tree(n, t, "gacc").copy()
        tok = rng.integers(0, 3, n).astype(np.int32)        # duplicate siblings happen
        g = rng.integers(0, 3, n).astype(np.int32)
        if t % 10 == 0 and n > 2:                           # out-of-range parents read as the root
            par[n - 1] = n + 3 if t % 20 == 0 else -7
        if t >= 300:                                        # chains of 15..32 nodes that match all the way
            n = (15, 16, 17, 32)[t - 300]
            par, tok, g = di.chain_tree(n), np.full(n, 2, np.int32), np.full(n, 2, np.int32)
        d = [torch.from_numpy(a).cuda() for a in (tok, par, g)]
        outs.append(ctx.tree_accept(*d))
        cases.append((tok, par, g))
    sync()
    for (tok, par, g), o in zip(cases, outs):
        clean = np.array([-1] + [p if 0 <= p < j else 0 for j, p in enumerate(par) if j > 0], dtype=np.int32)
        k, bonus, path = ddtree.tree_accept(tok, clean, g)
        if k > 15:                                          # acceptance stops after 15 nodes
            k, path = 15, path[:15]
            bonus = int(g[path[-1]])
        got = o.cpu().numpy().tolist()
        assert got[:2] == [k, bonus] and got[2:2 + k] == path and all(v == 0 for v in got[2 + k:])


# ------------------------------------------------------------------ tree-masked target forward

def _target(dl, s, w, C, page_seed):
    ctx = dl.DFlash(s.replace(draft_layers=s.target_layers), dev(w), max_ctx=C + 64, page_seed=page_seed)
    k, v = di.context_kv(s.replace(draft_layers=s.target_layers), C, tag="tree_kv")
    if C:
        ctx.load_kv(k.cuda(), v.cuda())
    return ctx, k, v


def _oracle_tree(orc, m, s, k, v, C, n, tok, par, sel, fp32_acc=False):
    NK = s.n_kv_heads * s.head_dim
    L = s.target_layers
    cache = orc.TargetCache(m, C + n)
    if C:
        cache.k[:, :C] = k.reshape(L, C, NK).double().numpy()
        cache.v[:, :C] = v.reshape(L, C, NK).double().numpy()
    orc.set_fp32_accumulation(fp32_acc)
    try:
        r = orc.target_forward(m, cache, tok, C, capture=sel, want_logits=True, parent=par)
    finally:
        orc.set_fp32_accumulation(False)
    r["cache"] = cache
    return r


@pytest.mark.parametrize("shape", [TR_BF16, TR_BF16_D64, TR_FP32_G5])
@pytest.mark.parametrize("C,n", [(0, 16), (37, 16), (180, 16), (250, 9), (300, 1), (380, 12), (511, 16),
                                 (0, 23), (250, 32), (380, 17)])
def test_tree_forward_matches_oracle(dl, orc, shape, C, n):
    """At the stated bar, one layer at a time: every layer of the tree pass
    against the oracle's tree-masked layer on the GPU's own input to it (2 bf16
    ulps; fp32 1e-4), the tree rows' K/V against the oracle's (same bar), the
    logits against the oracle's LM head on the GPU's final residual (2e-2;
    fp32 1e-4 relative) with tokens exact except top-2 gaps below 1e-3.  Then
    the feature capture of the same pass, and end to end against the oracle's
    own tree forward (bf16: the band twice the stated bar that bf16 rounding
    compounding over 8 layers needs; the plain causal forward shows the same
    end-to-end deviation on these inputs).  C = 180 / 380 put the tree's slots
    across a 192-key split boundary (keys 192 and 384) and 511 at the end of a
    64-key chunk.  Trees of 17 to 32 nodes take two passes (nodes 16 and on see
    their ancestors among the first pass's nodes in the cache)."""
    s = shape
    w = di.toy_target_weights(s)
    ctx, k, v = _target(dl, s, w, C, page_seed=9)
    par = di.random_tree(n, s.seed + C + n, "fwd")
    tok = di.uniform_int(n, 0, s.vocab - 1, s.seed + C, "tree_tok").numpy()
    tok_d, par_d = torch.from_numpy(tok).cuda(), torch.from_numpy(par).cuda()
    L, NK = s.target_layers, s.n_kv_heads * s.head_dim
    print(f"[tree] forward {s.name} C={C} n={n}", flush=True)
    layers = torch.empty(L, n, s.hidden, dtype=s.torch_dtype, device="cuda")
    am, lg = ctx.target_forward(tok_d, want_logits=True, parent=par_d, layers_out=layers)
    gk, gv = ctx.read_kv(C, n)
    ctx.rollback(C)
    cap = [torch.empty(n, s.hidden, dtype=s.torch_dtype, device="cuda") for _ in range(5)]
    am2, lg2 = ctx.target_forward(tok_d, want_logits=True, capture=cap, parent=par_d)
    sync()
    assert ctx.length == C + n
    assert torch.equal(am, am2) and torch.equal(lg, lg2)  # capture does not change the pass
    m = orc.Model(s, w, n_layers=L)
    sel = orc.feature_layers(s.target_layers)
    cache = orc.TargetCache(m, C + n)
    if C:
        cache.k[:, :C] = k.reshape(L, C, NK).double().numpy()
        cache.v[:, :C] = v.reshape(L, C, NK).double().numpy()
    lg = lg.cpu().numpy()
    err, ulps = check_target_layers(orc, m, w, s, cache, C, tok, par, layers, lg, am.cpu().numpy())
    print(f"[tree] per layer worst {ulps:.2f} ulps; LM head max|dlogit| {err:.3g}", flush=True)
    assert_rows_close(gk.float().cpu().numpy().reshape(L * n, NK), cache.k[:, C:].reshape(L * n, NK), s.dtype,
                      "tree K given the GPU's layer inputs")
    assert_rows_close(gv.float().cpu().numpy().reshape(L * n, NK), cache.v[:, C:].reshape(L * n, NK), s.dtype,
                      "tree V given the GPU's layer inputs")
    gl = layers.cpu()
    for i, l in enumerate(sel):
        assert torch.equal(cap[i].cpu(), gl[l]), f"capture of layer {l}"
    # end to end
    ref = _oracle_tree(orc, m, s, k, v, C, n, tok, par, sel)
    e2e = float(np.abs(lg.astype(np.float64) - ref["logits"]).max())
    print(f"[tree] end to end max|dlogit| {e2e:.3g}", flush=True)
    if s.dtype == "fp32":
        assert_logits(lg, ref["logits"], "fp32")
        assert_tokens(am.cpu().numpy(), ref["argmax"], ref["gap"], lg, ref["logits"], "fp32")
    else:
        assert e2e <= 4e-2
        assert_tokens(am.cpu().numpy(), ref["argmax"], ref["gap"], lg, ref["logits"], "bf16", 2e-2)


@pytest.mark.parametrize("shape", [TR_BF16, TR_FP32_G5])
@pytest.mark.parametrize("C,n", [(0, 16), (200, 16), (250, 16), (0, 32), (250, 32)])
def test_chain_tree_is_the_causal_forward(dl, shape, C, n):
    """A tree that is a chain runs the same arithmetic as the causal forward:
    logits, tokens, captures and KV bit-identical.  32 nodes: one two-pass tree
    call against two 16-row causal calls."""
    s = shape
    ctx, _, _ = _target(dl, s, di.toy_target_weights(s), C, page_seed=3)
    tok = torch.from_numpy(di.uniform_int(n, 0, s.vocab - 1, s.seed, "chain").numpy()).cuda()
    outs = []
    for parent in (None, torch.from_numpy(di.chain_tree(n)).cuda()):
        ctx.rollback(C)
        cap = [torch.empty(n, s.hidden, dtype=s.torch_dtype, device="cuda") for _ in range(5)]
        am = torch.empty(n, dtype=torch.int32, device="cuda")
        lg = torch.empty(n, s.vocab, dtype=torch.float32, device="cuda")
        if parent is None:
            for r0 in range(0, n, 16):
                ctx.target_forward(tok[r0:r0 + 16], argmax=am[r0:r0 + 16], logits=lg[r0:r0 + 16],
                                   capture=[c[r0:r0 + 16] for c in cap])
        else:
            ctx.target_forward(tok, argmax=am, logits=lg, capture=cap, parent=parent)
        k, v = ctx.read_kv(C, n)
        sync()
        outs.append([am.cpu(), lg.cpu(), k.cpu(), v.cpu()] + [c.cpu() for c in cap])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ compaction

@pytest.mark.parametrize("shape", [TR_BF16, TR_FP32_G5])
@pytest.mark.parametrize("n", [16, 32])
def test_tree_commit_moves_accepted_rows(dl, orc, shape, n):
    s = shape
    C = 120
    ctx, _, _ = _target(dl, s, di.toy_target_weights(s), C, page_seed=5)
    x = di.normal((15, s.vocab), 63, "commit", 2.0, torch.float32)
    ids, lp = ddtree.topk_logprobs(x.numpy(), 3)
    t = ddtree.build_tree(17, ids, lp.astype(np.float32), n - 1)
    tok, par = torch.from_numpy(t["tokens"]).cuda(), torch.from_numpy(t["parent"]).cuda()
    cap = [torch.empty(n, s.hidden, dtype=s.torch_dtype, device="cuda") for _ in range(5)]
    am, _ = ctx.target_forward(tok, capture=cap, parent=par)
    # a target that follows the deepest branch (the accepted path is then that branch)
    leaf = int(np.argmax(t["depth"]))
    g = am.cpu().numpy().copy()
    u = leaf
    while t["parent"][u] >= 0:
        g[t["parent"][u]] = t["tokens"][u]
        u = t["parent"][u]
    res = ctx.tree_accept(tok, par, torch.from_numpy(g).cuda())
    k0, v0 = ctx.read_kv(C, n)
    c0 = [c.clone() for c in cap]
    ctx.tree_commit(C, n, res, capture=cap)
    k1, v1 = ctx.read_kv(C, n)
    sync()
    kk, bonus, path = ddtree.tree_accept(t["tokens"], t["parent"], g)
    assert res.cpu().numpy().tolist()[:2 + kk] == [kk, bonus] + path and kk == t["depth"][leaf] >= 2
    src = [0] + path
    for i in range(n):
        j = src[i] if i < len(src) else i            # destinations 0..k, the rest untouched
        assert torch.equal(k1[:, i], k0[:, j]) and torch.equal(v1[:, i], v0[:, j]), f"slot {C + i}"
        for b in range(5):
            assert torch.equal(cap[b][i], c0[b][j])
    ctx.rollback(C + 1 + kk)
    assert ctx.length == C + 1 + kk


def test_tree_errors(dl):
    ctx = _vocab_ctx(dl, 1008)
    z = torch.zeros(17, 17, dtype=torch.int32, device="cuda")
    f = torch.zeros(17, 17, dtype=torch.float32, device="cuda")
    a = torch.zeros(1, dtype=torch.int32, device="cuda")
    for R, K, budget in ((3, 1, 4), (15, 17, 3), (16, 2, 3), (15, 2, 32), (2, 2, -1)):
        with pytest.raises(dl.DFlashError):
            ctx.build_tree(a, z[:R, :K], f[:R, :K], budget)
    lg = torch.zeros(17, 1008, dtype=torch.float32, device="cuda")
    with pytest.raises(dl.DFlashError):
        ctx.draft_topk(lg, 4)                       # 17 rows
    with pytest.raises(dl.DFlashError):
        ctx.draft_topk(lg[:4], 17)                  # K > 16
    res = torch.zeros(17, dtype=torch.int32, device="cuda")
    with pytest.raises(dl.DFlashError):
        ctx.tree_commit(0, 4, res)                  # rows beyond the length
    t33 = torch.zeros(33, dtype=torch.int32, device="cuda")
    with pytest.raises(dl.DFlashError):
        ctx.tree_accept(t33, t33, t33)              # more than 32 nodes
    sync()
