"""Pins of the oracle's tree verification ("DFlash 深度解析…" §8.2, DDTree):
top-K log-probabilities, best-first candidate trees, the accepted path, the
tree-masked target forward and the compaction of accepted rows.  Each is held
against something other than itself: repeated argmax and a library logsumexp,
exhaustive enumeration of small candidate trees, a brute-force search for the
accepted node, causal decoding of every root path, torch's attention with an
explicit tree mask, and the linear (chain) case of [B] 技术内幕."""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import dflash_inputs as di
from oracle import ddtree
from tests import torch_ref

TREE = di.Shape("tree", "fp32", hidden=64, target_layers=8, draft_layers=8, n_q_heads=4,
                n_kv_heads=2, head_dim=16, ffn=96, vocab=128, ctx=24, seed=43)


def _logits(R, V, tag, ties=True):
    x = di.normal((R, V), 9, tag, 1.0, torch.float32).numpy().copy()
    if ties:  # planted exact ties, including at the top
        for r in range(R):
            top = int(np.argmax(x[r]))
            x[r, (top + 7) % V] = x[r, top]
            x[r, 3] = x[r, 5]
    return x


# ---------------------------------------------------------------- top-K

@pytest.mark.parametrize("K", [1, 4, 16])
def test_topk_is_repeated_argmax_and_logsumexp(K):
    x = _logits(6, 200, "topk")
    ids, logp = ddtree.topk_logprobs(x, K)
    for r in range(6):
        row = x[r].astype(np.float64).copy()
        want = []
        for _ in range(K):  # np.argmax returns the first (lowest) index of the maximum
            j = int(np.argmax(row))
            want.append(j)
            row[j] = -np.inf
        assert ids[r].tolist() == want
        lse = scipy.special.logsumexp(x[r].astype(np.float64))
        np.testing.assert_allclose(logp[r], x[r, want].astype(np.float64) - lse, rtol=0, atol=1e-12)
        assert np.all(np.diff(logp[r]) <= 0)


# ---------------------------------------------------------------- candidate trees

def _f32_logp(R, K, tag, ties):
    """Sorted fp32 log-probabilities of R positions (top K of a 40-way softmax)."""
    x = _logits(R, 40, tag, ties=ties)
    ids, lp = ddtree.topk_logprobs(x, K)
    return ids, lp.astype(np.float32)


def _all_nodes(R, K, lp32):
    """Every node of the full K-ary candidate tree of depth R with its fp32
    score accumulated root-down, one rounding per edge."""
    out = []
    for depth in range(1, R + 1):
        for path in itertools.product(range(K), repeat=depth):
            sc = np.float32(0.0)
            for d, r in enumerate(path):
                sc = np.float32(sc + lp32[d, r])
            out.append((path, sc))
    return out


@pytest.mark.parametrize("R,K,ties", [(1, 3, False), (2, 2, True), (3, 2, False), (4, 2, True),
                                      (2, 4, False), (3, 3, True), (5, 1, False)])
def test_tree_is_the_best_budget_nodes(R, K, ties):
    """Exhaustive: the built tree is the first `budget` nodes of the whole
    candidate tree sorted by (score desc, depth, rank path), in that order."""
    ids, lp32 = _f32_logp(R, K, f"tree{R}{K}", ties)
    nodes = sorted(_all_nodes(R, K, lp32), key=lambda t: (-float(t[1]), len(t[0]), t[0]))
    for budget in range(0, min(15, len(nodes)) + 1):
        t = ddtree.build_tree(77, ids, lp32, budget)
        assert t["paths"][1:] == [p for p, _ in nodes[:budget]]
        assert len(t["tokens"]) == budget + 1 and t["tokens"][0] == 77 and t["parent"][0] == -1
        for j in range(1, budget + 1):
            p = t["paths"][j]
            assert t["paths"][t["parent"][j]] == p[:-1] and t["parent"][j] < j
            assert t["tokens"][j] == ids[len(p) - 1, p[-1]]
            assert t["depth"][j] == len(p)


def test_tree_maximises_expected_accepted_drafts():
    """Over every node set of the same size that is a tree (closed under
    taking parents), the built one has the largest sum of path probabilities,
    the expected number of accepted drafts when positions are independent."""
    R, K, budget = 3, 2, 4
    ids, lp32 = _f32_logp(R, K, "opt", False)
    nodes = _all_nodes(R, K, lp32)
    val = {p: float(np.exp(np.float64(s))) for p, s in nodes}
    best = -1.0
    for sub in itertools.combinations([p for p, _ in nodes], budget):
        ss = set(sub)
        if all(len(p) == 1 or p[:-1] in ss for p in sub):
            best = max(best, sum(val[p] for p in sub))
    t = ddtree.build_tree(0, ids, lp32, budget)
    got = sum(val[p] for p in t["paths"][1:])
    assert got >= best - 1e-12


def test_top1_tree_is_the_linear_block():
    """With K = 1 the tree is the chain of per-position argmax drafts that
    linear DFlash verifies."""
    x = _logits(15, 64, "chain", ties=True)
    ids, lp = ddtree.topk_logprobs(x, 1)
    t = ddtree.build_tree(5, ids, lp.astype(np.float32), 15)
    assert t["parent"].tolist() == di.chain_tree(16).tolist()
    assert t["tokens"][1:].tolist() == [int(np.argmax(x[r])) for r in range(15)]


# ---------------------------------------------------------------- acceptance

def test_chain_acceptance_is_linear_acceptance(orc):
    rng = np.random.default_rng(3)
    par = di.chain_tree(16)
    for _ in range(900):
        g = rng.integers(0, 4, 16).astype(np.int32)
        d = rng.integers(0, 4, 16).astype(np.int32)
        k, bonus, path = ddtree.tree_accept(d, par, g)
        assert (k, bonus) == orc.accept(d, g)
        assert path == list(range(1, k + 1))


def test_acceptance_brute_force():
    """The accepted node is the deepest node whose every edge carries the
    target's greedy token after the edge's upper end (siblings distinct)."""
    rng = np.random.default_rng(4)
    for trial in range(400):
        n = int(rng.integers(1, 17))
        par = di.random_tree(n, trial, "acc")
        tok = np.zeros(n, dtype=np.int32)
        for u in range(n):  # distinct tokens among siblings, from a 3-token alphabet where possible
            kids = [j for j in range(1, n) if par[j] == u]
            perm = rng.permutation(max(3, len(kids)))
            for i, j in enumerate(kids):
                tok[j] = perm[i]
        g = rng.integers(0, 3, n).astype(np.int32)
        ok = [True] + [False] * (n - 1)
        for j in range(1, n):
            ok[j] = ok[par[j]] and tok[j] == g[par[j]]
        dep = ddtree.depths(par)
        v = max((j for j in range(n) if ok[j]), key=lambda j: dep[j])
        path = []
        u = v
        while u != 0:
            path.append(u)
            u = par[u]
        k, bonus, got = ddtree.tree_accept(tok, par, g)
        assert (k, bonus, got) == (int(dep[v]), int(g[v]), path[::-1])


# ---------------------------------------------------------------- tree-masked target forward

def _tree_case(seed, n):
    s = TREE
    w = di.toy_target_weights(s)
    P = 9
    prefix = di.uniform_int(P, 0, s.vocab - 1, seed, "prefix").numpy()
    par = di.random_tree(n, seed, "tree")
    tok = di.uniform_int(n, 0, s.vocab - 1, seed, "tree_tok").numpy()
    return s, w, P, prefix, par, tok


def _prefilled(orc, m, prefix, cap):
    cache = orc.TargetCache(m, cap)
    orc.target_forward(m, cache, prefix, 0)
    return cache


@pytest.mark.parametrize("seed,n", [(1, 12), (2, 16), (3, 1), (4, 5)])
def test_tree_rows_equal_their_path_decodes(orc, seed, n):
    """Every tree row computes exactly (bit for bit: same keys, same order)
    what a causal forward of its root path computes at the path's last
    position: logits, argmax, captured layers, and its cache slot holds the K/V
    that path decode stores at the row's position.  A row placed at pos0 + j
    instead of pos0 + depth, a causal instead of an ancestor mask, or a row
    missing its own key fails here."""
    s, w, P, prefix, par, tok = _tree_case(seed, n)
    m = orc.Model(s, w, n_layers=s.target_layers)
    sel = orc.feature_layers(s.target_layers)
    cache = _prefilled(orc, m, prefix, P + n)
    r = orc.target_forward(m, cache, tok, P, capture=sel, want_logits=True, parent=par)
    dep = ddtree.depths(par)
    for j in range(n):
        path = []
        u = j
        while u >= 0:
            path.append(u)
            u = par[u]
        path = path[::-1]
        c2 = _prefilled(orc, m, prefix, P + len(path))
        q = orc.target_forward(m, c2, tok[path], P, capture=sel, want_logits=True)
        assert np.array_equal(r["logits"][j], q["logits"][-1]), f"node {j}"
        assert r["argmax"][j] == q["argmax"][-1]
        assert np.array_equal(r["hidden"][:, j], q["hidden"][:, -1])
        assert np.array_equal(cache.k[:, P + j], c2.k[:, P + dep[j]])
        assert np.array_equal(cache.v[:, P + j], c2.v[:, P + dep[j]])


@pytest.mark.parametrize("seed,n", [(5, 16), (6, 7)])
def test_tree_forward_against_torch_masked_prefill(orc, seed, n):
    s, w, P, prefix, par, tok = _tree_case(seed, n)
    m = orc.Model(s, w, n_layers=s.target_layers)
    sel = orc.feature_layers(s.target_layers)
    cache = _prefilled(orc, m, prefix, P + n)
    r = orc.target_forward(m, cache, tok, P, capture=sel, want_logits=True, parent=par)
    lg, hid = torch_ref.tree_forward(s, w, prefix, tok, par, s.target_layers)
    lg, hid = lg.numpy(), hid.numpy()
    np.testing.assert_allclose(r["logits"], lg, rtol=1e-5, atol=1e-6)
    assert np.array_equal(r["argmax"], lg.argmax(axis=1))
    for i, l in enumerate(sel):
        np.testing.assert_allclose(r["hidden"][i], hid[l], rtol=1e-5, atol=1e-6, err_msg=f"captured layer {l}")


def test_chain_tree_is_the_causal_forward(orc):
    s, w, P, prefix, _, tok = _tree_case(7, 16)
    m = orc.Model(s, w, n_layers=s.target_layers)
    a = orc.target_forward(m, _prefilled(orc, m, prefix, P + 16), tok, P, want_logits=True,
                           parent=di.chain_tree(16))
    b = orc.target_forward(m, _prefilled(orc, m, prefix, P + 16), tok, P, want_logits=True)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["argmax"], b["argmax"])


@pytest.mark.parametrize("par", [[0, 0, 1], [-1, 1, 0], [-1, 0, 3], [-1, -1, 0]])
def test_tree_forward_rejects_non_trees(orc, par):
    s, w, P, prefix, _, _ = _tree_case(8, 3)
    m = orc.Model(s, w, n_layers=s.target_layers)
    with pytest.raises(AssertionError):
        orc.target_forward(m, _prefilled(orc, m, prefix, P + 3), [1, 2, 3], P, parent=par)


def test_compacted_cache_is_the_accepted_sequence_cache(orc):
    """After verification of a tree and acceptance of a path, moving the
    accepted rows behind the root leaves exactly the cache that a causal
    forward of [root, accepted tokens] writes."""
    s, w, P, prefix, _, _ = _tree_case(9, 0)
    m = orc.Model(s, w, n_layers=s.target_layers)
    x = _logits(15, s.vocab, "commit", ties=False)
    ids, lp = ddtree.topk_logprobs(x, 4)
    t = ddtree.build_tree(11, ids, lp.astype(np.float32), 15)
    cache = _prefilled(orc, m, prefix, P + 16)
    r = orc.target_forward(m, cache, t["tokens"], P, parent=t["parent"])
    # a target that agrees with the deepest branch it can: follow argmax-free choices
    g = r["argmax"].copy()
    leaf = int(np.argmax(t["depth"]))
    u = leaf
    while t["parent"][u] >= 0:
        g[t["parent"][u]] = t["tokens"][u]
        u = t["parent"][u]
    k, bonus, path = ddtree.tree_accept(t["tokens"], t["parent"], g)
    assert k == t["depth"][leaf] and k >= 2
    ck = ddtree.compact_rows(np.moveaxis(cache.k, 1, 0), P, path)
    cv = ddtree.compact_rows(np.moveaxis(cache.v, 1, 0), P, path)
    ref = _prefilled(orc, m, prefix, P + 1 + k)
    orc.target_forward(m, ref, [t["tokens"][0]] + [int(t["tokens"][j]) for j in path], P)
    assert np.array_equal(ck[:P + 1 + k], np.moveaxis(ref.k, 1, 0))
    assert np.array_equal(cv[:P + 1 + k], np.moveaxis(ref.v, 1, 0))


@pytest.mark.parametrize("tree", [True, False])
def test_target_layers_compose_to_the_forward(orc, tree):
    """The one-layer entry (used to check a GPU pass layer by layer) chained
    over every layer, then the LM head, is exactly the full forward."""
    s, w, P, prefix, par, tok = _tree_case(10, 11)
    par = par if tree else None
    m = orc.Model(s, w, n_layers=s.target_layers)
    sel = orc.feature_layers(s.target_layers)
    full = orc.target_forward(m, _prefilled(orc, m, prefix, P + 11), tok, P, capture=sel, want_logits=True,
                              parent=par)
    cache = _prefilled(orc, m, prefix, P + 11)
    x = w["embed"][list(tok)].double().numpy()
    hid = []
    for l in range(s.target_layers):
        x = orc.target_layer(m, l, x, P, cache, par)
        hid.append(x)
    head = orc.lm_head(m, x)
    assert np.array_equal(head["logits"], full["logits"]) and np.array_equal(head["tokens"], full["argmax"])
    for i, l in enumerate(sel):
        assert np.array_equal(hid[l], full["hidden"][i])
