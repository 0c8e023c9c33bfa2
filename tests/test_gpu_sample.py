"""Non-greedy drafting and verification through the C ABI against the oracle
(oracle/sampling.py), on the same fp32 logits:

* Gumbel-max draws: tokens exact except where the two best perturbed scores
  lie closer than 1e-3 (fp32 against fp64 keys), the rows' log-sum-exp of
  z / T within 1e-6 relative (fp64 sums, returned in fp32);
* the speculative sampling rule over a drafted block, computed in fp64 on both
  sides: k exact except where the deciding comparison U * q < p is closer than
  1e-9 of its sides, the drawn token exact except where U * total lies closer
  to a running-sum boundary than 1e-12 of sum(p) + sum(q) (the rounding of
  fp64 probabilities, which the residual max(0, p - q) keeps in absolute
  terms while its total shrinks where p and q nearly agree).
"""
import zlib

import numpy as np
import pytest
import torch

import dflash_inputs as di
from oracle import sampling as sp
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

GAP = 1e-3           # perturbed-score gap under which either draw may come out
ACCEPT_REL = 1e-9    # relative closeness of U * q and p under which either decision may come out
DRAW_EPS = 1e-12     # boundary distance, relative to sum(p) + sum(q), under which either draw may come out


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
    s = di.Shape(f"s{V}", "bf16", hidden=64, target_layers=8, draft_layers=1, n_q_heads=2, n_kv_heads=1,
                 head_dim=64, ffn=96, vocab=V, ctx=16, seed=7)
    return dl.DFlash(s, dev(di.draft_weights(s, need_draft=False, need_lm=False)), max_ctx=64)


def _padded(x):
    """fp32 rows on the device with a row stride 48 beyond V (NaN padding)."""
    R, V = x.shape
    buf = torch.full((R, V + 48), float("nan"), dtype=torch.float32)
    buf[:, :V] = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return buf.cuda()[:, :V]


# ------------------------------------------------------------------ drafting

@pytest.mark.parametrize("V,T,rows,scale", [(151936, 1.0, 16, 2.0), (4000, 0.6, 16, 3.0), (4000, 1.7, 9, 1.0),
                                            (1008, 0.05, 16, 1.0), (1008, 1.0, 1, 0.0)])
def test_sample_tokens_matches_oracle(dl, V, T, rows, scale):
    ctx = _vocab_ctx(dl, V)
    x = di.normal((rows, V), 71, f"samp{V}_{T}", scale, torch.float32).numpy()
    seed = 0x5EED0000 + V
    print(f"[sample] V={V} T={T} rows={rows}", flush=True)
    g = _padded(x)
    tok, lse = ctx.sample_tokens(g, T, seed, want_lse=True)
    tok_only, _ = ctx.sample_tokens(g, T, seed)                     # draws alone
    lse_only = torch.empty(rows, dtype=torch.float32, device="cuda")  # log-sum-exp alone (no token output)
    assert dl.lib().dflash_sample_tokens(ctx.h, g.data_ptr(), g.stride(0), rows, T, seed, None,
                                         lse_only.data_ptr(), None) == 0
    sync()
    assert torch.equal(tok, tok_only) and torch.equal(lse, lse_only)
    ref = sp.sample_tokens(x, T, seed)
    got = tok.cpu().numpy()
    ties = 0
    for r in range(rows):
        if got[r] != ref["tokens"][r]:
            assert ref["gap"][r] < GAP, f"row {r}: {got[r]} vs {ref['tokens'][r]}, gap {ref['gap'][r]:.3g}"
            ties += 1
    assert ties <= max(1, rows // 8)
    np.testing.assert_allclose(lse.cpu().numpy().astype(np.float64), ref["lse"], rtol=1e-6, atol=1e-6)


def test_sample_tokens_is_seeded(dl):
    """The same seed gives the same draws on every call; another seed moves
    them (a flat row over 4000 ids); draws land inside the vocabulary."""
    V = 4000
    ctx = _vocab_ctx(dl, V)
    x = torch.zeros(16, V, dtype=torch.float32, device="cuda")
    a, _ = ctx.sample_tokens(x, 1.0, 1)
    b, _ = ctx.sample_tokens(x, 1.0, 1)
    c, _ = ctx.sample_tokens(x, 1.0, 2)
    sync()
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert int(a.min()) >= 0 and int(a.max()) < V
    assert len(set(a.cpu().tolist())) > 8      # 16 independent rows of a flat row rarely collide


@pytest.mark.parametrize("seed,x,wins", [(301, 3207, False), (416, 2393, True)])
def test_gumbel_draws_near_one(dl, seed, x, wins):
    """Uniforms within 4 steps of 1 (U = 1 - 0.5 * 2^-24 for id 3207 at seed
    301, U = 1 - 3.5 * 2^-24 for id 2393 at seed 416; both need 25 bits, so an
    fp32 U would round to 1.0 and to 1 - 4 * 2^-24).  The id's logit is set so
    that its exact key trails (seed 301) or beats (seed 416) the best other key
    by 0.05; a perturbation taken from the rounded U lands on the other side
    (+inf, and 0.134 lower)."""
    V = 4000
    ctx = _vocab_ctx(dl, V)
    u = np.array([sp.uniform(seed, 0, i, open_interval=True) for i in range(V)])
    assert 1 - u[x] < 4 * 2.0 ** -24
    g = -np.log(-np.log(u))
    other = np.delete(g, x).max()
    z = np.zeros((1, V), np.float32)
    z[0, x] = other + (0.05 if wins else -0.05) - g[x]
    ref = sp.sample_tokens(z, 1.0, seed)
    assert (ref["tokens"][0] == x) == wins and ref["gap"][0] > 0.04
    tok, _ = ctx.sample_tokens(torch.from_numpy(z).cuda(), 1.0, seed)
    sync()
    assert int(tok[0]) == ref["tokens"][0]


# ------------------------------------------------------------------ verification

def _block(V, B, kind, tag, scale=2.0, noise=0.7):
    """Draft logits [B, V], target logits [B, V] and a draft block for one of:
    'near' (target row j - 1 = draft row j + noise: a mix of acceptances),
    'same' (target row j - 1 == draft row j: every draft accepted),
    'far' (the target gives every draft almost no mass: rejected at once)."""
    zd = di.normal((B, V), 81, f"vd{tag}", scale, torch.float32).numpy()
    zt = np.empty_like(zd)
    zt[:B - 1] = zd[1:]
    zt[B - 1] = di.normal((1, V), 81, f"vl{tag}", scale, torch.float32).numpy()[0]
    if kind == "near":
        zt += di.normal((B, V), 81, f"vn{tag}", noise, torch.float32).numpy()
    # drafts drawn from softmax(draft row) by numpy's own Gumbel draws (an input here)
    g = np.random.default_rng(zlib.crc32(tag.encode())).gumbel(size=(B - 1, V))
    d = np.zeros(B, dtype=np.int32)
    d[1:] = np.argmax(zd[1:].astype(np.float64) + g, axis=1)
    if kind == "far":
        for j in range(1, B):
            zt[j - 1, d[j]] = -60.0
    return zd.astype(np.float32), zt.astype(np.float32), d


def _check_verify(got, ref, dl_, tl_, d, T, seed):
    """k and the drawn token against the oracle's walk, with the closeness
    exemptions of the module docstring; returns the number of exempted cases."""
    k, tok = int(got[0]), int(got[1])
    if k != ref["k"]:
        j = min(k, ref["k"]) + 1                   # the first decision that differs
        p = np.exp(sp.log_softmax(tl_[j - 1], T))[d[j]]
        q = np.exp(sp.log_softmax(dl_[j], T))[d[j]]
        u = sp.uniform(seed, sp.TAG_ACCEPT + j, 0)
        assert abs(u * q - p) <= ACCEPT_REL * max(p, u * q), f"k {k} vs {ref['k']} at draft {j}: uq {u*q} p {p}"
        return 1
    if tok != ref["bonus"]:
        B = len(d)
        if k < B - 1:   # the residual's total, relative to which the oracle states its margin
            total = np.maximum(0.0, np.exp(sp.log_softmax(tl_[k], T)) - np.exp(sp.log_softmax(dl_[k + 1], T))).sum()
            tol = DRAW_EPS * 2.0 / total
        else:
            tol = DRAW_EPS
        assert ref["draw_margin"] < tol, f"k={k}: token {tok} vs {ref['bonus']}, margin {ref['draw_margin']} > {tol}"
        return 1
    return 0


@pytest.mark.parametrize("V", [151936, 4000])
@pytest.mark.parametrize("kind", ["near", "same", "far"])
def test_verify_sample_matches_oracle(dl, V, kind):
    ctx = _vocab_ctx(dl, V)
    B = 16
    seeds = range(12) if V > 100000 else range(40)
    exempt, ks = 0, []
    for case in range(2 if V > 100000 else 4):
        zd, zt, d = _block(V, B, kind, f"{kind}{V}_{case}")
        gd, gt, gdr = _padded(zd), _padded(zt), torch.from_numpy(d).cuda()
        for T in (1.0, 0.7) if case % 2 == 0 else (1.3,):
            print(f"[verify-sample] V={V} {kind} case {case} T={T}", flush=True)
            outs = [ctx.verify_sample(gdr, gd, gt, T, 1000 * case + s) for s in seeds]
            sync()
            for s, o in zip(seeds, outs):
                ref = sp.verify_sample(d, zd, zt, T, 1000 * case + s)
                exempt += _check_verify(o.cpu().numpy(), ref, zd, zt, d, T, 1000 * case + s)
                ks.append(ref["k"])
    print(f"[verify-sample] V={V} {kind}: k mean {np.mean(ks):.2f} min {min(ks)} max {max(ks)}; "
          f"{exempt} near-tie cases of {len(ks)}", flush=True)
    assert exempt <= max(1, len(ks) // 50)
    if kind == "same":
        assert min(ks) == B - 1
    if kind == "far":
        assert max(ks) == 0
    if kind == "near":
        assert max(ks) > min(ks)                   # the cases exercise both rejection and the residual draw


def test_verify_sample_arbitrary_drafts(dl):
    """Drafts not drawn from q (some of them far in q's tail): the rule still
    reads q and p at the given ids; k and the token match the oracle."""
    V, B = 4000, 16
    ctx = _vocab_ctx(dl, V)
    zd, zt, _ = _block(V, B, "near", "arb", noise=0.3)
    rng = np.random.default_rng(5)
    exempt = n = 0
    for case in range(6):
        d = np.zeros(B, dtype=np.int32)
        d[1:] = rng.integers(0, V, B - 1)
        d[1:case + 1] = np.argmax(zt[:case], axis=1)   # a likely prefix of length `case`
        gdr = torch.from_numpy(d).cuda()
        outs = [ctx.verify_sample(gdr, _padded(zd), _padded(zt), 1.0, 77 + s) for s in range(10)]
        sync()
        for s, o in enumerate(outs):
            ref = sp.verify_sample(d, zd, zt, 1.0, 77 + s)
            exempt += _check_verify(o.cpu().numpy(), ref, zd, zt, d, 1.0, 77 + s)
            n += 1
    assert exempt <= 2, f"{exempt} near-tie cases of {n}"


def test_sample_errors(dl):
    ctx = _vocab_ctx(dl, 1008)
    lg = torch.zeros(17, 1008, dtype=torch.float32, device="cuda")
    d = torch.zeros(16, dtype=torch.int32, device="cuda")
    for T in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(dl.DFlashError):
            ctx.sample_tokens(lg[:4], T, 1)
        with pytest.raises(dl.DFlashError):
            ctx.verify_sample(d, lg[:16], lg[:16], T, 1)
    with pytest.raises(dl.DFlashError):
        ctx.sample_tokens(lg, 1.0, 1)                     # 17 rows
    narrow = torch.zeros(16, 1000, dtype=torch.float32, device="cuda")
    with pytest.raises(dl.DFlashError):
        ctx.sample_tokens(narrow, 1.0, 1)                 # row stride below V
    with pytest.raises(dl.DFlashError):
        ctx.verify_sample(d, narrow, narrow, 1.0, 1)
    # misaligned int32 / fp32 buffers are refused before anything is enqueued
    L, ok = dl.lib(), torch.zeros(16, dtype=torch.int32, device="cuda")
    assert L.dflash_sample_tokens(ctx.h, lg.data_ptr(), lg.stride(0), 4, 1.0, 1, ok.data_ptr() + 2, None, None) != 0
    assert L.dflash_sample_tokens(ctx.h, lg.data_ptr(), lg.stride(0), 4, 1.0, 1, None, ok.data_ptr() + 1, None) != 0
    assert L.dflash_verify_sample(ctx.h, d.data_ptr() + 2, lg.data_ptr(), lg.data_ptr(), lg.stride(0), 1.0, 1,
                                  ok.data_ptr(), None) != 0
    assert L.dflash_verify_sample(ctx.h, d.data_ptr(), lg.data_ptr(), lg.data_ptr(), lg.stride(0), 1.0, 1,
                                  ok.data_ptr() + 2, None) != 0
    sync()


def test_sampled_position_follows_the_target_distribution(dl):
    """The GPU path of one drafted position end to end -- d_1 drawn from q by
    dflash_sample_tokens, then dflash_verify_sample -- emits at position 1 a
    token distributed as p = softmax(target row 0 / T) whatever q: token
    frequencies over 6000 seeds within 4.5 standard errors of p, and the
    acceptance rate P(k >= 1) within 4.5 standard errors of sum(min(p, q))."""
    V, B, T, N = 16, 16, 0.8, 6000
    ctx = _vocab_ctx(dl, V)
    zd = di.normal((B, V), 91, "dist_d", 1.5, torch.float32).numpy()
    zt = di.normal((B, V), 91, "dist_t", 1.5, torch.float32).numpy()
    zt[0, :4] = zd[1, :4] + 0.3                    # overlapping mass on a few ids
    p = np.exp(sp.log_softmax(zt[0], T))
    q = np.exp(sp.log_softmax(zd[1], T))
    gd, gt = torch.from_numpy(zd).cuda(), torch.from_numpy(zt).cuda()
    toks = torch.zeros(N, B, dtype=torch.int32, device="cuda")
    res = torch.empty(N, 2, dtype=torch.int32, device="cuda")
    for i in range(N):
        ctx.sample_tokens(gd[1:], T, 0xD157 + i, tokens=toks[i, 1:])
        ctx.verify_sample(toks[i], gd, gt, T, 0xD157 + i, out=res[i])
    sync()
    t, r = toks.cpu().numpy(), res.cpu().numpy()
    emitted = np.where(r[:, 0] >= 1, t[:, 1], r[:, 1])
    f = np.bincount(emitted, minlength=V) / N
    se = np.sqrt(p * (1 - p) / N)
    print(f"[sample dist] max |f - p| / se = {np.max(np.abs(f - p) / np.maximum(se, 1e-12)):.2f}", flush=True)
    assert (np.abs(f - p) <= 4.5 * se + 1.0 / N).all(), (f, p)
    a = float(np.minimum(p, q).sum())
    acc = float((r[:, 0] >= 1).mean())
    assert abs(acc - a) <= 4.5 * np.sqrt(a * (1 - a) / N), (acc, a)
    fq = np.bincount(t[:, 1], minlength=V) / N       # the drafts themselves follow q
    assert (np.abs(fq - q) <= 4.5 * np.sqrt(q * (1 - q) / N) + 1.0 / N).all(), (fq, q)


def test_sampling_masked_vocabulary(dl):
    """Ids with -inf logits (a masked vocabulary): never drawn, no mass in the
    log-sum-exp, p = q = 0 there; draws, lse and the rule match the oracle."""
    V, B = 4000, 16
    ctx = _vocab_ctx(dl, V)
    rng = np.random.default_rng(17)
    mask = rng.random(V) < 0.5
    zd = di.normal((B, V), 93, "mask_d", 2.0, torch.float32).numpy()
    zt = np.roll(zd, -1, axis=0) + di.normal((B, V), 93, "mask_t", 0.7, torch.float32).numpy()
    zd[:, mask] = -np.inf
    zt[:, mask] = -np.inf
    gd, gt = _padded(zd), _padded(zt)
    tok, lse = ctx.sample_tokens(gd[1:], 1.0, 55, want_lse=True)
    sync()
    ref = sp.sample_tokens(zd[1:], 1.0, 55)
    got = tok.cpu().numpy()
    assert not mask[got].any()
    assert ((got == ref["tokens"]) | (ref["gap"] < GAP)).all()
    np.testing.assert_allclose(lse.cpu().numpy().astype(np.float64), ref["lse"], rtol=1e-6, atol=1e-6)
    d = np.zeros(B, dtype=np.int32)
    d[1:] = got
    exempt = 0
    for s in range(20):
        o = ctx.verify_sample(torch.from_numpy(d).cuda(), gd, gt, 1.0, 300 + s).cpu().numpy()
        r = sp.verify_sample(d, zd, zt, 1.0, 300 + s)
        assert not mask[o[1]]
        exempt += _check_verify(o, r, zd, zt, d, 1.0, 300 + s)
    assert exempt <= 1


def test_verify_sample_short_block(dl):
    """A context whose block is 8 rows: the rule walks drafts 1..7, reads 15
    log-sum-exp rows, and draws the bonus from target row 7."""
    V, B = 1008, 8
    s = di.Shape("s1008b8", "bf16", hidden=64, target_layers=8, draft_layers=1, n_q_heads=2, n_kv_heads=1,
                 head_dim=64, ffn=96, vocab=V, ctx=16, seed=7, block=B)
    ctx = dl.DFlash(s, dev(di.draft_weights(s, need_draft=False, need_lm=False)), max_ctx=64)
    ks, exempt = [], 0
    for kind in ("near", "same", "far"):
        zd, zt, d = _block(V, B, kind, f"short_{kind}")
        gd, gt, gdr = _padded(zd), _padded(zt), torch.from_numpy(d).cuda()
        for seed in range(16):
            o = ctx.verify_sample(gdr, gd, gt, 0.9, seed).cpu().numpy()
            r = sp.verify_sample(d, zd, zt, 0.9, seed)
            exempt += _check_verify(o, r, zd, zt, d, 0.9, seed)
            ks.append(r["k"])
            if kind == "same":
                assert r["k"] == B - 1
    assert exempt <= 1 and max(ks) == B - 1 and min(ks) == 0


def test_sampling_graph_replay(dl):
    """The non-greedy calls hold no host read, so a step of them can be
    captured in a HIP graph: draws of the drafted positions, then the rule.
    Every replay (with eager work of the same context in between, fresh logits
    copied in before each) equals the eager calls on the same inputs bit for
    bit."""
    V, B = 4000, 16
    ctx = _vocab_ctx(dl, V)
    cases = []
    for i in range(3):
        zd, zt, _ = _block(V, B, "near", f"graph{i}")
        cases.append((torch.from_numpy(zd).cuda(), torch.from_numpy(zt).cuda()))
    dlg = torch.empty(B, V, dtype=torch.float32, device="cuda")
    tlg = torch.empty(B, V, dtype=torch.float32, device="cuda")
    blk = torch.zeros(B, dtype=torch.int32, device="cuda")
    res = torch.empty(2, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()

    def step():
        ctx.sample_tokens(dlg[1:], 0.8, 4242, tokens=blk[1:], stream=s)
        ctx.verify_sample(blk, dlg, tlg, 0.8, 4242, out=res, stream=s)

    eager = []
    for zd, zt in cases:
        dlg.copy_(zd)
        tlg.copy_(zt)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            step()
        s.synchronize()
        eager.append((blk.clone(), res.clone()))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, (zd, zt) in enumerate(cases):
            dlg.copy_(zd)
            tlg.copy_(zt)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(blk, eager[i][0]) and torch.equal(res, eager[i][1]), (rep, i)
            # eager work of the same context between replays (its own draws)
            ctx.sample_tokens(dlg[:4], 1.3, 99 + rep)
            torch.cuda.synchronize()
