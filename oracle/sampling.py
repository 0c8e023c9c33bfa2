"""Non-greedy drafting and verification, written plainly.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the CPU-baseline leg of
``bench.py``; never by the product package.

The rebasdaily DFlash2 page (section 先猜几个，再让主模型拍板) says DFlash2's
candidate selection pays off most under non-greedy samplers; the pages give no
rule for verifying a drafted block when the target samples.  Readings taken:

- Drafting at temperature T samples token j of the block from
  softmax(z_j / T) (z_j: the draft's fp32 logits of block row j) by the
  Gumbel-max method: argmax over x of z_j[x] / T + G, with G = -log(-log U)
  and U uniform in (0, 1) (ties: lower id).
- Verification is the speculative sampling rule of the literature (Leviathan,
  Kalman and Matias 2023; Chen et al. 2023): draft d_j, with draft
  probability q = softmax(z_j / T)[d_j] and target probability
  p = softmax(t_{j-1} / T)[d_j] (t_i: the target's logits of verified row i,
  which predict position C + i + 1), is accepted when U * q < p.  At the first
  rejection the target's token is drawn from max(0, p_{j-1} - q_j)
  renormalised; after 15 acceptances the bonus is drawn from softmax(t_15 / T).
  The emitted tokens then follow the target's own sampling distribution.
- A draw from unnormalised weights w with U: the first x whose running sum
  w[0] + .. + w[x] exceeds U * sum(w).
- Random numbers come from SplitMix64 (Steele, Lea and Flood 2014) used as a
  counter-based generator: draw n of stream `seed` is the generator's
  (n + 1)-th output, n = a * 2^32 + b for the draw's coordinates (a, b);
  a uniform keeps its top 24 bits, k * 2^-24 in [0, 1), or (k + 0.5) * 2^-24
  in (0, 1) where a logarithm follows.  Coordinates: Gumbel draw of block row r
  and token x: (r, x); acceptance draw of draft j: (2^20 + j, 0); the
  rejection / bonus draw: (2^20 + 64, 0).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
TAG_ACCEPT = 1 << 20
TAG_RESIDUAL = (1 << 20) + 64


def splitmix64(seed: int, n: int) -> int:
    """Output n (0-based) of the SplitMix64 stream started at `seed`."""
    z = (seed + (n + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def uniform(seed: int, a: int, b: int, open_interval: bool = False) -> float:
    k = splitmix64(seed, (a << 32) | b) >> 40
    return (k + 0.5) * 2.0 ** -24 if open_interval else k * 2.0 ** -24


def log_softmax(z: np.ndarray, T: float) -> np.ndarray:
    x = np.asarray(z, dtype=np.float64) / T
    m = x.max()
    return x - (m + np.log(np.exp(x - m).sum()))


def sample_tokens(logits: np.ndarray, T: float, seed: int) -> Dict[str, np.ndarray]:
    """Gumbel-max draws from softmax(row / T) for every row of the fp32 logits.
    Returns the tokens, the gap between the two largest perturbed scores (a
    draw closer than rounding can tell may come out either way) and each row's
    log-sum-exp of row / T."""
    z = np.asarray(logits, dtype=np.float32)
    R, V = z.shape
    tokens = np.empty(R, dtype=np.int32)
    gap = np.empty(R)
    lse = np.empty(R)
    for r in range(R):
        u = np.array([uniform(seed, r, x, open_interval=True) for x in range(V)])
        key = z[r].astype(np.float64) / T - np.log(-np.log(u))
        order = np.lexsort((np.arange(V), -key))
        tokens[r] = order[0]
        gap[r] = key[order[0]] - key[order[1]]
        x = z[r].astype(np.float64) / T
        lse[r] = x.max() + np.log(np.exp(x - x.max()).sum())
    return {"tokens": tokens, "gap": gap, "lse": lse}


def draw(weights: np.ndarray, u: float):
    """The first index whose running sum exceeds u * total, and how far u * total
    lies from the nearest running-sum boundary (relative to the total)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    t = u * c[-1]
    x = int(np.searchsorted(c, t, side="right"))
    x = min(x, len(c) - 1)
    margin = min(abs(c[x] - t), abs(t - (c[x - 1] if x > 0 else 0.0))) / c[-1]
    return x, margin


def speculative_step(p: np.ndarray, q: np.ndarray, d: int, u_accept: float, u_draw: float):
    """One position of the rule: accept draft d (drawn from q) when
    u_accept * q[d] < p[d]; otherwise draw from max(0, p - q).  Returns
    (accepted, token, accept margin, draw margin)."""
    acc_margin = abs(u_accept * q[d] - p[d])
    if u_accept * q[d] < p[d]:
        return True, d, acc_margin, np.inf
    w = np.maximum(0.0, p - q)
    x, m = draw(w, u_draw)
    return False, x, acc_margin, m


def verify_sample(draft: np.ndarray, draft_logits: np.ndarray, target_logits: np.ndarray, T: float,
                  seed: int) -> Dict[str, object]:
    """Speculative sampling over one drafted block: k accepted drafts and the
    token drawn after them (the rejection draw, or the bonus after all B - 1
    acceptances).  Margins of every decision taken are returned alongside."""
    d = np.asarray(draft)
    B = len(d)
    margins = []
    u_draw = uniform(seed, TAG_RESIDUAL, 0)
    for j in range(1, B):
        p = np.exp(log_softmax(target_logits[j - 1], T))
        q = np.exp(log_softmax(draft_logits[j], T))
        ok, tok, ma, md = speculative_step(p, q, int(d[j]), uniform(seed, TAG_ACCEPT + j, 0), u_draw)
        margins.append(ma)
        if not ok:
            return {"k": j - 1, "bonus": tok, "accept_margins": margins, "draw_margin": md}
    x, md = draw(np.exp(log_softmax(target_logits[B - 1], T)), u_draw)
    return {"k": B - 1, "bonus": x, "accept_margins": margins, "draw_margin": md}
