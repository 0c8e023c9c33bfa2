"""Candidate trees for tree verification (DDTree), written plainly.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and ``__graft_entry__.smoke()``;
never by the product package.

"DFlash 深度解析…" §8.2 (DDTree tree verification) replaces the single chain of
drafts by a tree of candidates, checked by the target in one pass under a node
budget, so that a rejection at one depth can still be followed by another
branch.  The passage names the idea and the budget (16 or 22 nodes) but not the
construction.  Readings taken here (plainest ones the passage supports):

- The candidates at depth d (the token for position C+d, the anchor being the
  root at C) are the draft's top-K tokens of block row d, ordered by logit
  (ties: lower id first), with log-probabilities log_softmax(logits row d).
- A node's score is the sum of the log-probabilities along its root path: the
  drafter's probability that the whole path is right when positions are taken
  as independent.  The tree is the `budget` best nodes under the order
  (score descending, depth ascending, rank path lexicographically ascending).
  A child never scores above its parent and a later sibling never above an
  earlier one, so these nodes always form a tree, and they maximise the
  expected number of accepted drafts under that independence.
- Scores are fp32 sums (parent score + log-probability, one rounding each): the
  kernel's precision, since these floating-point values decide integers.
- Verification: starting at the root, follow the child whose token equals the
  target's greedy token after the current node; the followed nodes are accepted
  and the target's token after the last of them is the bonus.

Node order of a built tree is the selection order, so parent[j] < j.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np


def topk_logprobs(logits: np.ndarray, K: int):
    """Per row: the K largest logits' ids (ties: lower id first) and their
    log-probabilities under the row's softmax, in fp64 from the fp32 logits."""
    x = np.asarray(logits, dtype=np.float32)
    R, V = x.shape
    assert 1 <= K <= V
    ids = np.empty((R, K), dtype=np.int32)
    logp = np.empty((R, K), dtype=np.float64)
    for r in range(R):
        row = x[r].astype(np.float64)
        # value descending, then id ascending
        order = np.lexsort((np.arange(V), -row))[:K]
        m = row.max()
        lse = m + np.log(np.exp(row - m).sum())
        ids[r] = order
        logp[r] = row[order] - lse
    return ids, logp


def _key(score: np.float32, path: tuple):
    return (-float(score), len(path), path)


def build_tree(anchor: int, ids: np.ndarray, logp32: np.ndarray, budget: int) -> Dict[str, np.ndarray]:
    """The `budget` best non-root nodes of the candidate tree whose depth-d
    choices are ids[d-1, :] with log-probabilities logp32[d-1, :] (fp32).
    Best-first: a node is eligible once its parent is in the tree; the best
    eligible node (under the order above) joins next.  Returns tokens, parent,
    depth, rank paths and fp32 scores of the root and the chosen nodes."""
    ids = np.asarray(ids)
    lp = np.asarray(logp32, dtype=np.float32)
    R, K = ids.shape
    assert 0 <= budget <= sum(K ** d for d in range(1, R + 1))
    paths: List[tuple] = [()]
    scores: List[np.float32] = [np.float32(0.0)]
    index = {(): 0}
    for _ in range(budget):
        best = None
        for u, pu in enumerate(paths):
            if len(pu) == R:
                continue
            for r in range(K):
                pc = pu + (r,)
                if pc in index:
                    continue
                sc = np.float32(scores[u] + lp[len(pu), r])
                if best is None or _key(sc, pc) < _key(best[1], best[2]):
                    best = (u, sc, pc)
        u, sc, pc = best
        index[pc] = len(paths)
        paths.append(pc)
        scores.append(sc)
    n = len(paths)
    tokens = np.empty(n, dtype=np.int32)
    parent = np.empty(n, dtype=np.int32)
    tokens[0], parent[0] = anchor, -1
    for j in range(1, n):
        pc = paths[j]
        tokens[j] = ids[len(pc) - 1, pc[-1]]
        parent[j] = index[pc[:-1]]
    depth = np.array([len(p) for p in paths], dtype=np.int32)
    return {"tokens": tokens, "parent": parent, "depth": depth, "paths": paths,
            "score": np.array(scores, dtype=np.float32)}


def tree_accept(tokens: Sequence[int], parent: Sequence[int], target: Sequence[int]):
    """Walk from the root: while some child of the current node carries the
    target's greedy token after that node (target[node]), move to it (the
    lowest-index such child).  Returns (k, bonus, path): k accepted nodes, the
    target's token after the last one, and their node indices."""
    n = len(tokens)
    children: List[List[int]] = [[] for _ in range(n)]
    for j in range(1, n):
        children[parent[j]].append(j)
    cur, path = 0, []
    while True:
        nxt = [c for c in children[cur] if tokens[c] == target[cur]]
        if not nxt:
            break
        cur = nxt[0]
        path.append(cur)
    return len(path), int(target[cur]), path


def depths(parent: Sequence[int]) -> np.ndarray:
    d = np.zeros(len(parent), dtype=np.int32)
    for j in range(1, len(parent)):
        d[j] = d[parent[j]] + 1
    return d


def compact_rows(a: np.ndarray, pos0: int, path: Sequence[int]) -> np.ndarray:
    """After acceptance the accepted nodes' rows move behind the root: row
    pos0 + 1 + i takes row pos0 + path[i] (axis 0 of `a`, the slot axis).
    Returns a copy; rows from pos0 + 1 + len(path) on are left as they were."""
    out = np.array(a, copy=True)
    for i, j in enumerate(path):
        out[pos0 + 1 + i] = a[pos0 + j]
    return out
