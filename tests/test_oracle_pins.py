"""Pins of the CPU oracle against facts the pages and mathematics fix.

Each test targets a plausible mistake (dropped term, wrong index or sign,
transposed operand, wrong pairing) and fails on it.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dflash_inputs as di
from tests import torch_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MICRO = di.Shape("micro", "fp32", hidden=64, target_layers=8, draft_layers=2, n_q_heads=4,
                 n_kv_heads=2, head_dim=16, ffn=96, vocab=128, ctx=24, seed=11)


def micro_model(orc, shape=MICRO, gains="random", **over):
    w = di.draft_weights(shape, gains=gains)
    w.update(over)
    return orc.Model(shape, w), w


# ---------------------------------------------------------------- layer choice

def test_feature_layers_tiny_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "feature_layers_tiny.json")))
    assert orc.feature_layers(g["target_layers"]) == g["layers"]


@pytest.mark.parametrize("L", list(range(8, 81)))
def test_feature_layers_span(orc, L):
    s = orc.feature_layers(L)
    # second layer to the third-from-last output, strictly increasing, near-uniform steps
    assert s[0] == 1 and s[-1] == L - 2
    assert all(b > a for a, b in zip(s, s[1:]))
    step = (L - 3) / 4
    assert all(abs(s[i] - (1 + i * step)) <= 0.5 for i in range(5))


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    # exact halfway patterns: low 16 bits = 0x8000, both parities of the kept bit
    bits = rng.integers(0x3F000000, 0x42000000, 4000, dtype=np.uint32)
    half = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, half, -half, np.float32([0.0, 1.0, -2.5, 65504.0])])
    ours = orc.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_matches_library(orc):
    rng = np.random.default_rng(1)
    for n in (7, 64, 4096):
        x = rng.standard_normal(n) * 3.0
        g = torch.from_numpy(rng.uniform(0.5, 1.5, n).astype(np.float32))
        x32 = x.astype(np.float32).astype(np.float64)
        ours = orc.rmsnorm(x32, g, "fp32", 1e-6)
        ref = F.rms_norm(torch.from_numpy(x32), (n,), weight=g.double(), eps=1e-6).float().double().numpy()
        np.testing.assert_allclose(ours, ref, rtol=2e-7, atol=1e-30)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_zero_and_norm(orc):
    rng = np.random.default_rng(2)
    v = rng.standard_normal(128)
    assert np.array_equal(orc.rope(v, 0, 10000.0), v)
    r = orc.rope(v, 36879, 10000.0)
    h = 64
    np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, v[:h] ** 2 + v[h:] ** 2, rtol=1e-12)


def test_rope_is_complex_rotation(orc):
    """Pairs (i, i+d/2) rotate by pos * base^(-2i/d), as complex multiplication."""
    rng = np.random.default_rng(3)
    d, base = 16, 10000.0
    v = rng.standard_normal(d)
    for pos in (1, 7, 4097):
        ref = torch_ref.rope_complex(torch.from_numpy(v)[None, None, :], torch.tensor([pos]), base)[0, 0].numpy()
        np.testing.assert_allclose(orc.rope(v, pos, base), ref, rtol=1e-12, atol=1e-12)
    # the lowest pair turns by exactly `pos` radians, the next by pos*base^(-2/d)
    e = np.zeros(d); e[0] = 1.0
    r = orc.rope(e, 3, base)
    assert math.isclose(math.atan2(r[d // 2], r[0]), 3.0 - 2 * math.pi * round(3.0 / (2 * math.pi)), abs_tol=1e-12)
    e = np.zeros(d); e[1] = 1.0
    r = orc.rope(e, 1, base)
    assert math.isclose(math.atan2(r[d // 2 + 1], r[1]), base ** (-2.0 / d), rel_tol=1e-12)


def test_rope_relative(orc):
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = orc.rope(q, 100, 10000.0) @ orc.rope(k, 37, 10000.0)
    b = orc.rope(q, 5100, 10000.0) @ orc.rope(k, 5037, 10000.0)
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


# ---------------------------------------------------------------- fusion

@pytest.mark.parametrize("sel", [0, 2, 4])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fuse_selection_closed_form(orc, sel, dtype):
    """W_fc = [0 .. I .. 0] (identity in block `sel`) => c = RMSNorm(h_sel)."""
    s = MICRO.replace(dtype=dtype)
    H = s.hidden
    fc = torch.zeros(H, 5 * H)
    fc[:, sel * H:(sel + 1) * H] = torch.eye(H)
    w = di.draft_weights(s, gains="random")
    w["fc"] = fc.to(s.torch_dtype)
    m = orc.Model(s, w)
    slabs = [di.target_hidden(s, l, 9) for l in range(5)]
    out = orc.fuse_rows(m, slabs, range(9))
    ref = F.rms_norm(slabs[sel].double(), (H,), weight=w["fc_norm"].double(), eps=s.eps)
    ref = ref.to(s.torch_dtype).double().numpy()
    tol = 2 ** -7 if dtype == "bf16" else 2e-7
    np.testing.assert_allclose(out, ref, rtol=tol, atol=0)
    if dtype == "bf16":
        assert (out == ref).mean() > 0.99


def test_fuse_brute_force(orc):
    w = di.draft_weights(MICRO, gains="random")
    m = orc.Model(MICRO, w)
    slabs = [di.target_hidden(MICRO, l, 13) for l in range(5)]
    out = orc.fuse_rows(m, slabs, range(13))
    ref = torch_ref.fuse(MICRO, w, slabs).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)


def test_fuse_slab_permutation_invariance(orc):
    """Swapping two slabs together with the matching column blocks of W_fc changes nothing."""
    s, H = MICRO, MICRO.hidden
    w = di.draft_weights(s, gains="random")
    slabs = [di.target_hidden(s, l, 6) for l in range(5)]
    a = orc.fuse_rows(orc.Model(s, w), slabs, range(6))
    w2 = dict(w)
    fc = w["fc"].clone()
    fc[:, 1 * H:2 * H], fc[:, 3 * H:4 * H] = w["fc"][:, 3 * H:4 * H], w["fc"][:, 1 * H:2 * H]
    w2["fc"] = fc.contiguous()
    sl2 = [slabs[0], slabs[3], slabs[2], slabs[1], slabs[4]]
    b = orc.fuse_rows(orc.Model(s, w2), sl2, range(6))
    np.testing.assert_allclose(a, b, rtol=1e-6)


def test_fuse_unit_mean_square(orc):
    s = MICRO
    w = di.draft_weights(s, gains="ones")
    slabs = [di.target_hidden(s, l, 8) for l in range(5)]
    out = orc.fuse_rows(orc.Model(s, w), slabs, range(8))
    np.testing.assert_allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-5)


# ---------------------------------------------------------------- injection

def test_inject_brute_force(orc):
    w = di.draft_weights(MICRO, gains="random")
    m = orc.Model(MICRO, w)
    fused = di.fused_context(MICRO, 11)
    k, v = orc.inject_rows(m, fused, range(11), pos0=37)
    rk, rv = torch_ref.inject(MICRO, w, fused, 37)
    L, M = MICRO.draft_layers, 11
    np.testing.assert_allclose(k, rk.reshape(L, M, -1).numpy(), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(v, rv.reshape(L, M, -1).numpy(), rtol=1e-6, atol=1e-6)


def test_inject_selection_closed_form(orc):
    """W_k = W_v = [I 0] picks the first nkv*d features: v = c[:NK], k = RoPE(c[:NK]) per head
    at position pos0 + row, in every layer."""
    s = MICRO
    NK = s.n_kv_heads * s.head_dim
    sel = torch.zeros(NK, s.hidden)
    sel[:, :NK] = torch.eye(NK)
    w = di.draft_weights(s)
    for l in range(s.draft_layers):
        w[f"wk.{l}"] = sel.clone()
        w[f"wv.{l}"] = sel.clone()
    fused = di.fused_context(s, 5)
    rows = [0, 3, 4]
    k, v = orc.inject_rows(orc.Model(s, w), fused, rows, pos0=1000)
    c = fused.double().numpy()
    for l in range(s.draft_layers):
        for i, r in enumerate(rows):
            np.testing.assert_array_equal(v[l, i], c[r, :NK])
            for h in range(s.n_kv_heads):
                seg = c[r, h * s.head_dim:(h + 1) * s.head_dim]
                exp = orc.rope(seg, 1000 + r, s.rope_base).astype(np.float32).astype(np.float64)
                np.testing.assert_array_equal(k[l, i, h * s.head_dim:(h + 1) * s.head_dim], exp)


# ---------------------------------------------------------------- draft block

def _ctx(s, C, seed_tag="kv"):
    return di.context_kv(s.replace(ctx=C), tag=seed_tag)


@pytest.mark.parametrize("C", [0, 1, 24])
def test_draft_block_brute_force(orc, C):
    m, w = micro_model(orc)
    k, v = _ctx(MICRO, C)
    out = orc.draft_block(m, k, v, C, anchor=17)
    ref = torch_ref.draft_forward(MICRO, w, k, v, C, 17).numpy()
    np.testing.assert_allclose(out["logits"], ref, rtol=1e-5, atol=1e-6)
    assert np.array_equal(out["tokens"], ref.argmax(axis=1))


def test_draft_block_tiny_workload_brute_force(orc):
    s = di.SHAPES["tiny_fp32"]
    w = di.draft_weights(s)
    m = orc.Model(s, w)
    k, v = di.context_kv(s)
    anchor = di.anchor_token(s)
    out = orc.draft_block(m, k, v, s.ctx, anchor)
    ref = torch_ref.draft_forward(s, w, k, v, s.ctx, anchor).numpy()
    rel = np.abs(out["logits"] - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert rel.max() < 1e-5


def test_context_row_order_invariance(orc):
    """Injected context keys enter a softmax over a set: permuting the stored
    rows of K and V together leaves the draft unchanged."""
    m, w = micro_model(orc)
    C = 24
    k, v = _ctx(MICRO, C)
    perm = torch.randperm(C, generator=torch.Generator().manual_seed(5))
    a = orc.draft_block(m, k, v, C, 3)
    b = orc.draft_block(m, k[:, perm].contiguous(), v[:, perm].contiguous(), C, 3)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-5, atol=1e-6)


def test_context_present_in_every_layer(orc):
    """KV injection reaches every layer: changing only layer l's context values
    changes the residual stream from layer l on and not before."""
    m, w = micro_model(orc)
    C = 24
    k, v = _ctx(MICRO, C)
    base = orc.draft_block(m, k, v, C, 3, want_trace=True)["trace"]
    for l in range(MICRO.draft_layers):
        v2 = v.clone()
        v2[l] *= 2
        tr = orc.draft_block(m, k, v2, C, 3, want_trace=True)["trace"]
        assert np.array_equal(tr[: l + 1], base[: l + 1])
        assert np.abs(tr[l + 1] - base[l + 1]).max() > 1e-3


def test_gqa_head_mapping(orc):
    """nq=4, nkv=2 equals nq=4, nkv=4 with each kv head duplicated for its group
    (query heads 0,1 -> kv head 0; 2,3 -> kv head 1)."""
    s = MICRO
    w = di.draft_weights(s, gains="random")
    d = s.head_dim
    s4 = s.replace(n_kv_heads=4)
    w4 = dict(w)
    for l in range(s.draft_layers):
        for name in ("wk", "wv"):
            blk = w[f"{name}.{l}"].view(2, d, s.hidden)
            w4[f"{name}.{l}"] = blk.repeat_interleave(2, dim=0).reshape(4 * d, s.hidden).contiguous()
    C = 24
    k, v = _ctx(s, C)
    k4 = k.repeat_interleave(2, dim=2).contiguous()
    v4 = v.repeat_interleave(2, dim=2).contiguous()
    a = orc.draft_block(orc.Model(s, w), k, v, C, 9)
    b = orc.draft_block(orc.Model(s4, w4), k4, v4, C, 9)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-6, atol=1e-7)


def test_single_key_returns_its_value(orc):
    """B = 1 and C = 0: softmax over one key is 1, so attention returns v itself.
    With W_o = I-like selection the layer output is x + v (pinned via a 1-layer model)."""
    s = MICRO.replace(block=1, draft_layers=1, n_q_heads=2, n_kv_heads=2, hidden=32)
    w = di.draft_weights(s, gains="ones")
    NQ = s.n_q_heads * s.head_dim
    w["wo.0"] = torch.eye(s.hidden, NQ).contiguous()
    w["wd.0"] = torch.zeros(s.hidden, s.ffn)
    m = orc.Model(s, w)
    out = orc.draft_block(m, None, None, 0, 5, want_trace=True)
    tr = out["trace"]
    x0 = w["embed"][5].double()
    u = F.rms_norm(x0, (s.hidden,), eps=s.eps).float().double()
    vv = (u @ w["wv.0"].double().T).float().double()
    np.testing.assert_allclose(tr[1, 0], (x0 + vv).float().double().numpy(), rtol=1e-6, atol=1e-7)


def test_block_is_bidirectional(orc):
    """Row 0 (the anchor) sees the mask rows after it: its logits with a
    16-row block differ from a 1-row block; under a causal mask they would not."""
    m16, w = micro_model(orc)
    s1 = MICRO.replace(block=1)
    m1 = orc.Model(s1, w)
    C = 24
    k, v = _ctx(MICRO, C)
    a = orc.draft_block(m16, k, v, C, 4)["logits"][0]
    b = orc.draft_block(m1, k, v, C, 4)["logits"][0]
    assert np.abs(a - b).max() > 1e-4


def test_softmax_scale_two_keys(orc):
    """Two keys, one query head, d = 16: p = sigmoid((s1 - s2)/sqrt(d)).
    Checked through a 1-layer model whose only attention input is controlled."""
    s = MICRO.replace(block=1, draft_layers=1, n_q_heads=1, n_kv_heads=1, hidden=16, head_dim=16)
    H = 16
    w = di.draft_weights(s, gains="ones")
    w["wq.0"] = torch.eye(H)
    w["wk.0"] = torch.zeros(H, H)
    w["wv.0"] = torch.zeros(H, H)
    w["wo.0"] = torch.eye(H)
    w["wd.0"] = torch.zeros(H, s.ffn)
    m = orc.Model(s, w)
    # context: key 0 = e0 * 4, key 1 = 0; values e1 * 1 and e2 * 1 (position baked in already)
    k = torch.zeros(1, 2, 1, H)
    v = torch.zeros(1, 2, 1, H)
    k[0, 0, 0, 0] = 4.0
    v[0, 0, 0, 1] = 1.0
    v[0, 1, 0, 2] = 1.0
    out = orc.draft_block(m, k, v, 2, 7, want_trace=True)["trace"]
    x0 = w["embed"][7].double()
    u = F.rms_norm(x0, (H,), eps=s.eps).float().double()
    q = torch_ref.rope_complex(u.view(1, 1, H), torch.tensor([2]), s.rope_base).view(H).float().double()
    sc = np.array([4.0 * q[0].item(), 0.0, 0.0]) / 4.0  # block key is zero (W_k = 0)
    p = np.exp(sc - sc.max()); p /= p.sum()
    o = np.zeros(H); o[1] = p[0]; o[2] = p[1]
    o = o.astype(np.float32).astype(np.float64)
    exp = (x0.numpy() + o).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(out[1, 0], exp, rtol=1e-6, atol=1e-7)


def test_argmax_ties_lowest_index(orc):
    s = MICRO
    w = di.draft_weights(s, gains="random")
    lm = torch.zeros(s.vocab, s.hidden)
    vec = torch.randn(s.hidden, generator=torch.Generator().manual_seed(0))
    for r in (5, 9, 77):
        lm[r] = vec
    w["lm_head"] = lm
    out = orc.draft_block(orc.Model(s, w), *_ctx(s, 24), 24, 1)
    for j in range(s.block):
        lg = out["logits"][j]
        top = np.flatnonzero(lg == lg.max())
        assert out["tokens"][j] == top[0]
        assert len(top) >= 2 and out["gap"][j] == 0.0


# ---------------------------------------------------------------- acceptance

def test_accept_exhaustive_patterns(orc):
    rng = np.random.default_rng(6)
    B = 16
    for pat in range(1 << (B - 1)):
        d = rng.integers(0, 1000, B)
        g = d.copy()
        g[:-1] = d[1:]
        g[-1] = rng.integers(0, 1000)
        for j in range(1, B):
            if not (pat >> (j - 1)) & 1:
                g[j - 1] = d[j] + 1  # mismatch at draft position j
        lead = 0
        while lead < B - 1 and (pat >> lead) & 1:
            lead += 1
        k, bonus = orc.accept(d, g)
        assert k == lead and bonus == g[lead]


def test_accept_statistics_synthetic_target(orc):
    """With the synthetic target agreeing w.p. 0.3 per position, k is the
    number of leading agreements: P(k) = 0.7 * 0.3^k for k < 15, E[k] = sum 0.3^j."""
    s = di.SHAPES["tiny_fp32"]
    rng = np.random.default_rng(7)
    n = 40000
    ks = np.empty(n, dtype=np.int64)
    for t in range(n):
        d = rng.integers(0, s.vocab, s.block)
        u = rng.random(s.block)
        r = rng.integers(1, s.vocab, s.block)
        g = di.synthetic_target_argmax(d, u, r, int(rng.integers(0, s.vocab)), s.vocab)
        ks[t] = orc.accept(d, g)[0]
    mean = sum(0.3 ** j for j in range(1, 16))
    assert abs(ks.mean() - mean) < 5 * math.sqrt(0.6 / n)
    assert abs((ks == 0).mean() - 0.7) < 5 * math.sqrt(0.21 / n)
    assert abs((ks == 1).mean() - 0.21) < 5 * math.sqrt(0.17 / n)


# ---------------------------------------------------------------- causal target / lossless loop

def test_target_prefill_equals_decode(orc):
    s = MICRO.replace(draft_layers=2)
    w = di.toy_target_weights(s.replace(target_layers=2))
    m = orc.Model(s, w, n_layers=2)
    toks = di.uniform_int(10, 0, s.vocab - 1, 3, "t").numpy()
    c1 = orc.TargetCache(m, 16)
    a = orc.target_forward(m, c1, toks, 0, capture=[0, 1, 1, 1, 1])
    c2 = orc.TargetCache(m, 16)
    outs, hids = [], []
    for i, t in enumerate(toks):
        r = orc.target_forward(m, c2, [t], i, capture=[0, 1, 1, 1, 1])
        outs.append(r["argmax"][0])
        hids.append(r["hidden"][:, 0])
    assert np.array_equal(a["argmax"], np.array(outs))
    assert np.array_equal(a["hidden"], np.stack(hids, axis=1))
    assert np.array_equal(c1.k, c2.k)


TOYLET = di.Shape("toylet", "fp32", hidden=64, target_layers=8, draft_layers=2, n_q_heads=4,
                  n_kv_heads=2, head_dim=16, ffn=96, vocab=128, ctx=20, seed=21)


@pytest.fixture(scope="module")
def toylet(orc):
    s = TOYLET
    tm = orc.Model(s, di.toy_target_weights(s), n_layers=s.target_layers)
    dw = di.draft_weights(s)
    dm = orc.Model(s, dw)
    prompt = di.uniform_int(s.ctx, 0, s.vocab - 1, s.seed, "prompt").numpy()
    greedy, _ = orc.greedy_generate(tm, prompt, 40)
    return tm, dm, prompt, greedy


@pytest.mark.parametrize("mode", ["dflash", "perfect", "null", "prefix"])
def test_spec_decode_is_lossless(orc, toylet, mode):
    """Greedy block verification emits exactly the target's greedy tokens
    whatever the drafts are ([C]: lossless greedy verification): drafts from
    the DFlash draft model, all correct (k = 15 every block), all wrong
    (k = 0), and correct up to a random length."""
    tm, dm, prompt, greedy = toylet
    P, V = len(prompt), TOYLET.vocab
    rng = np.random.default_rng(5)

    def truth(C):  # greedy tokens at positions C+1..C+15 (past the end: anything)
        return [int(greedy[p - P]) if p - P < len(greedy) else 0 for p in range(C + 1, C + 16)]

    fn = {"dflash": None,
          "perfect": truth,
          "null": lambda C: [(t + 1) % V for t in truth(C)],
          "prefix": lambda C: [t if j < r else (t + 1) % V
                               for r in [int(rng.integers(0, 16))] for j, t in enumerate(truth(C))]}[mode]
    out, ks = orc.spec_generate(tm, dm, prompt, len(greedy), drafts_fn=fn)
    assert np.array_equal(out, greedy)
    if mode == "perfect":
        assert ks[:-1] == [15] * (len(ks) - 1) and len(ks) == math.ceil((len(greedy) - 1) / 16)
    if mode == "null":
        assert ks == [0] * (len(greedy) - 1)
    if mode == "prefix":
        assert len(set(ks)) > 3


# ---------------------------------------------------------------- causal target vs an independent formulation

CAUSAL = di.Shape("causal", "fp32", hidden=64, target_layers=8, draft_layers=8, n_q_heads=4,
                  n_kv_heads=2, head_dim=16, ffn=96, vocab=128, ctx=24, seed=41)


@pytest.mark.parametrize("chunks", [[24], [7, 1, 16], [1] * 8 + [16]])
def test_target_forward_brute_force(orc, chunks):
    """The oracle's causal forward ([A] §1.1 autoregressive generation, §1.2
    verification of a block in one causal pass) against torch's attention with
    an explicit lower-triangular mask over the whole sequence: logits, argmax
    and the five captured layers (the residual stream right AFTER each selected
    layer).  The oracle runs the sequence as one prefill, or as calls of 1 and
    16 rows appended to its cache, so a row that misses its own key or a
    capture taken before the layer fails here."""
    s = CAUSAL
    w = di.toy_target_weights(s)
    m = orc.Model(s, w, n_layers=s.target_layers)
    toks = di.uniform_int(s.ctx, 0, s.vocab - 1, s.seed, "causal").numpy()
    sel = orc.feature_layers(s.target_layers)
    cache = orc.TargetCache(m, s.ctx)
    lg, am, hid, pos = [], [], [], 0
    for n in chunks:
        r = orc.target_forward(m, cache, toks[pos:pos + n], pos, capture=sel, want_logits=True)
        lg.append(r["logits"])
        am.append(r["argmax"])
        hid.append(r["hidden"])
        pos += n
    assert pos == s.ctx
    lg, am, hid = np.concatenate(lg), np.concatenate(am), np.concatenate(hid, axis=1)
    ref_lg, ref_hid = torch_ref.target_forward(s, w, toks, s.target_layers)
    ref_lg, ref_hid = ref_lg.numpy(), ref_hid.numpy()
    np.testing.assert_allclose(lg, ref_lg, rtol=1e-5, atol=1e-6)
    assert np.array_equal(am, ref_lg.argmax(axis=1))
    for i, l in enumerate(sel):
        np.testing.assert_allclose(hid[i], ref_hid[l], rtol=1e-5, atol=1e-6, err_msg=f"captured layer {l}")


def test_target_first_row_sees_only_itself(orc):
    """Row 0 of a prefill attends to its own key alone, so its output does not
    depend on the tokens after it; row j depends on token j (its own key)."""
    s = CAUSAL
    w = di.toy_target_weights(s)
    m = orc.Model(s, w, n_layers=s.target_layers)
    toks = di.uniform_int(6, 0, s.vocab - 1, s.seed, "own").numpy()
    alt = toks.copy()
    alt[3] = (alt[3] + 1) % s.vocab
    a = orc.target_forward(m, orc.TargetCache(m, 6), toks, 0, want_logits=True)["logits"]
    b = orc.target_forward(m, orc.TargetCache(m, 6), alt, 0, want_logits=True)["logits"]
    assert np.array_equal(a[:3], b[:3])
    assert np.abs(a[3] - b[3]).max() > 1e-4 and np.abs(a[5] - b[5]).max() > 1e-4


# ---------------------------------------------------------------- fusion storage rounding (bf16)

def test_fuse_rounds_linear_output_before_norm(orc):
    """bf16 storage contract of the fusion ([A] §2.2 rms_norm(linear(concat))):
    the Linear's output is stored (rounded to bf16) and the RMSNorm reads the
    stored values.  Written here with torch's own matmul, bf16 conversion and
    rms_norm; leaving out the rounding between the two changes about a quarter
    of the bf16 outputs."""
    s = MICRO.replace(dtype="bf16")
    H = s.hidden
    w = di.draft_weights(s, gains="random", need_draft=False, need_lm=False)
    slabs = [di.target_hidden(s, l, 32) for l in range(5)]
    out = orc.fuse_rows(orc.Model(s, w), slabs, range(32))
    x = torch.cat([t.double() for t in slabs], dim=1)
    y = (x @ w["fc"].double().T).to(torch.bfloat16).double()
    ref = F.rms_norm(y, (H,), weight=w["fc_norm"].double(), eps=s.eps).to(torch.bfloat16).double().numpy()
    # torch converts float64 -> float32 -> bfloat16, which can differ from a
    # direct rounding only at exact bf16 halfway points of the float32 value
    assert (out != ref).mean() < 2e-3


# ---------------------------------------------------------------- per-layer entry points

def test_draft_layers_compose_to_the_block(orc):
    """Chaining the one-layer entry and the LM-head entry reproduces the full
    draft block exactly (they expose the block's own steps)."""
    s = MICRO
    m, w = micro_model(orc)
    C = 24
    k, v = _ctx(s, C)
    full = orc.draft_block(m, k, v, C, 9, want_trace=True)
    x = full["trace"][0]
    for l in range(s.draft_layers):
        x = orc.draft_layer(m, l, k[l], v[l], C, x)
        assert np.array_equal(x, full["trace"][l + 1])
    head = orc.lm_head(m, x)
    assert np.array_equal(head["logits"], full["logits"]) and np.array_equal(head["tokens"], full["tokens"])
    m0 = orc.Model(s, w)
    x0 = orc.draft_block(m0, None, None, 0, 9, want_trace=True)["trace"]
    assert np.array_equal(orc.draft_layer(m0, 0, None, None, 0, x0[0]), x0[1])
