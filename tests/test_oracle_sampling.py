"""Pins of the oracle's non-greedy drafting and verification (oracle/sampling.py):
the generator against its published reference outputs, the Gumbel-max draw
against the softmax it samples, and the speculative sampling rule against the
property that defines it -- the emitted token follows the target's
distribution whatever the draft's -- integrated over its random numbers."""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from oracle import sampling as sp


def test_splitmix64_reference_outputs():
    """SplitMix64's published reference values: the first two outputs of seed
    0 and the first output of seed 1234567."""
    assert sp.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert sp.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert sp.splitmix64(1234567, 0) == 6457827717110365317


def test_uniforms_cover_the_unit_interval():
    u = np.array([sp.uniform(7, 3, x) for x in range(20000)])
    uo = np.array([sp.uniform(7, 3, x, open_interval=True) for x in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0 and uo.min() > 0.0 and uo.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01 and abs(np.var(u) - 1 / 12) < 0.005
    assert (uo - u == 0.5 * 2.0 ** -24).all()


def test_gumbel_draws_follow_the_softmax():
    """Rows with identical logits are independent draws: their frequencies
    match softmax(z / T) within sampling error."""
    z = np.array([1.0, 0.2, -0.5, 2.0, 0.0], dtype=np.float32)
    for T in (0.7, 1.0, 1.5):
        rows = np.tile(z, (6000, 1))
        r = sp.sample_tokens(rows, T, seed=11)
        f = np.bincount(r["tokens"], minlength=5) / len(rows)
        p = np.exp(sp.log_softmax(z, T))
        assert np.abs(f - p).max() < 4 * np.sqrt(p.max() / len(rows)), (T, f, p)
        assert np.allclose(r["lse"], np.log(np.exp(z.astype(np.float64) / T).sum()))


def test_low_temperature_draw_is_the_argmax():
    z = di.normal((8, 50), 3, "lowT", 1.0, torch.float32).numpy()
    r = sp.sample_tokens(z, 1e-4, seed=2)
    assert np.array_equal(r["tokens"], z.argmax(axis=1))


@pytest.mark.parametrize("case", range(4))
def test_speculative_step_emits_the_target_distribution(case):
    """Integrated over both random numbers (a midpoint grid of n x n values)
    and over the draft token drawn from q: the emitted token's probabilities
    equal p, for unrelated p and q, q wider than p, q missing part of p's
    support, and q == p (every draft accepted)."""
    rng = np.random.default_rng(case)
    V = 6
    p = rng.dirichlet(np.ones(V))
    q = [rng.dirichlet(np.ones(V)), np.full(V, 1 / V), np.r_[rng.dirichlet(np.ones(3)), 0, 0, 0], p][case]
    n = 400
    grid = (np.arange(n) + 0.5) / n
    out = np.zeros(V)
    accepted = 0.0
    for d in range(V):
        if q[d] == 0:
            continue
        for ua in grid:
            acc = ua * q[d] < p[d]
            if acc:
                out[d] += q[d] / n
                accepted += q[d] / n
                continue
            for ud in grid:
                _, tok, _, _ = sp.speculative_step(p, q, d, ua, ud)
                out[tok] += q[d] / n / n
    assert np.abs(out - p).max() < 3.0 / n, (out, p)
    assert abs(accepted - np.minimum(p, q).sum()) < 2.0 / n
    if case == 3:
        assert accepted == pytest.approx(1.0)


def test_chain_acceptance_extremes():
    """A target equal to the draft accepts every draft (k = 15, the bonus drawn
    from the last target row: a row peaked at one id gives that id); a target
    that gives the drafts no mass accepts none, and its token is never the
    rejected draft."""
    B, V = 16, 40
    z = di.normal((B, V), 5, "chainx", 1.0, torch.float32).numpy()
    d = sp.sample_tokens(z, 1.0, seed=9)["tokens"]
    r = sp.verify_sample(d, z, np.roll(z, -1, axis=0), 1.0, seed=9)
    assert r["k"] == B - 1
    # the bonus comes from the last target row: peaked at id 7 there, elsewhere as before
    t = np.roll(z, -1, axis=0)
    t[B - 1] = -30.0
    t[B - 1, 7] = 30.0
    r = sp.verify_sample(d, z, t, 1.0, seed=9)
    assert r["k"] == B - 1 and r["bonus"] == 7
    far = np.array(z, copy=True)
    for j in range(1, B):
        far[j - 1, d[j]] = -1e4
    r = sp.verify_sample(d, z, far, 1.0, seed=9)
    assert r["k"] == 0 and r["bonus"] != d[1]


def test_draw_is_the_inverse_cdf():
    w = np.array([0.0, 2.0, 0.0, 1.0, 1.0])
    assert sp.draw(w, 0.0)[0] == 1 and sp.draw(w, 0.49)[0] == 1
    assert sp.draw(w, 0.5)[0] == 3 and sp.draw(w, 0.74)[0] == 3
    assert sp.draw(w, 0.75)[0] == 4 and sp.draw(w, 0.999)[0] == 4
