"""The causal target forward (the verify side of a speculative step) and the
toy end-to-end greedy loop, through the C ABI, against the CPU oracle.

* parity: logits, tokens, captured feature layers and the paged KV cache of a
  chain of target calls of ragged row counts vs one oracle forward;
* batch invariance: a row's results are bit-identical whether it is verified
  alone or inside a block (the property that makes speculative output equal
  greedy output bit for bit);
* the toy workload (target hidden 1024, 8 layers, 16/4 heads x 64, FFN 2816,
  vocab 32000; 3-layer draft; 2048-token prompt, 512 tokens): speculative
  decoding == greedy decoding, with DFlash drafts and with forced all-right,
  all-wrong and random-prefix drafts; GPU greedy vs oracle greedy.
"""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from tests.gpu_helpers import (assert_logits, assert_rows_close, assert_tokens, bf16_logit_tol, dev,
                               drift_ulps)

pytestmark = pytest.mark.gpu

T_BF16 = di.Shape("t_bf16", "bf16", hidden=512, target_layers=8, draft_layers=8, n_q_heads=8,
                  n_kv_heads=2, head_dim=128, ffn=1376, vocab=4000, ctx=300, seed=31)
T_BF16_D64 = T_BF16.replace(name="t_bf16_d64", n_q_heads=16, n_kv_heads=4, head_dim=64, seed=32)
T_FP32_G5 = di.Shape("t_fp32_g5", "fp32", hidden=320, target_layers=8, draft_layers=8, n_q_heads=10,
                     n_kv_heads=2, head_dim=64, ffn=688, vocab=1024, ctx=300, seed=33)
TOY = di.SHAPES["toy_e2e"]


@pytest.fixture(scope="module")
def dl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_drafter_context_amd as m
    m.lib()
    return m


def sync():
    torch.cuda.synchronize()


def target_ctx(dl, s, w, max_ctx, page_seed=7):
    return dl.DFlash(s.replace(draft_layers=s.target_layers), dev(w), max_ctx=max_ctx, page_seed=page_seed)


def run_chunks(dl, ctx, s, toks, chunks, sel_capture=True):
    """Target calls over toks in the given row counts; returns argmax, logits, captures."""
    am, lg, caps = [], [], [[] for _ in range(5)]
    pos = 0
    for M in chunks:
        cap = [torch.empty(M, s.hidden, dtype=s.torch_dtype, device="cuda") for _ in range(5)]
        t = torch.from_numpy(np.asarray(toks[pos:pos + M], dtype=np.int32)).cuda()
        a, l = ctx.target_forward(t, want_logits=True, capture=cap if sel_capture else None)
        am.append(a)
        lg.append(l)
        for i in range(5):
            caps[i].append(cap[i])
        pos += M
    sync()
    return (torch.cat(am).cpu().numpy(), torch.cat(lg).cpu().numpy(),
            [torch.cat(c).float().cpu().numpy() for c in caps])


def oracle_noise_floor(orc, m, toks, ref, sel):
    """How far the oracle itself moves when it accumulates dot products in fp32
    instead of fp64 (same definition, same bf16 rounding points): the largest
    logit change, and per captured layer the largest row change in bf16 ulps.
    Layer after layer, bf16 rounding turns accumulation-order differences into
    whole-ulp differences, so two correct implementations drift by about this."""
    orc.set_fp32_accumulation(True)
    try:
        alt_cache = orc.TargetCache(m, len(toks))
        alt = orc.target_forward(m, alt_cache, toks, 0, capture=sel, want_logits=True)
    finally:
        orc.set_fp32_accumulation(False)
    lg = float(np.abs(alt["logits"].astype(np.float64) - ref["logits"].astype(np.float64)).max())
    n = alt_cache.k.shape[0] * alt_cache.k.shape[1]
    kv = max(drift_ulps(alt_cache.k.reshape(n, -1), ref["cache"].k.reshape(n, -1)),
             drift_ulps(alt_cache.v.reshape(n, -1), ref["cache"].v.reshape(n, -1)))
    return lg, [drift_ulps(alt["hidden"][i], ref["hidden"][i]) for i in range(5)], kv


# ------------------------------------------------------------------ parity

@pytest.mark.parametrize("shape", [T_BF16, T_BF16_D64, T_FP32_G5])
def test_target_forward_matches_oracle(dl, orc, shape):
    """300 tokens in calls of 16, 5, 1, 16, ... rows (splits of 192 keys are
    crossed; the page table is shuffled)."""
    s = shape
    w = di.toy_target_weights(s)
    toks = di.uniform_int(s.ctx, 0, s.vocab - 1, s.seed, "prompt").numpy()
    chunks, n = [], 0
    for M in [16, 5, 1, 16, 16, 3, 16, 7, 16, 16, 2, 16, 11] * 4:
        M = min(M, s.ctx - n)
        if M <= 0:
            break
        chunks.append(M)
        n += M
    assert n == s.ctx
    ctx = target_ctx(dl, s, w, max_ctx=s.ctx + 64)
    am, lg, caps = run_chunks(dl, ctx, s, toks, chunks)
    assert ctx.length == s.ctx

    m = orc.Model(s, w, n_layers=s.target_layers)
    sel = orc.feature_layers(s.target_layers)
    cache = orc.TargetCache(m, s.ctx)
    ref = orc.target_forward(m, cache, toks, 0, capture=sel, want_logits=True)
    ref["cache"] = cache
    noise, hid_ulps, kv_ulps = (oracle_noise_floor(orc, m, toks, ref, sel) if s.dtype == "bf16"
                                else (None, [0.0] * 5, 0.0))
    assert_logits(lg, ref["logits"], s.dtype, noise)
    assert_tokens(am, ref["argmax"], ref["gap"], lg, ref["logits"], s.dtype, noise)
    for i in range(5):
        assert_rows_close(caps[i], ref["hidden"][i], s.dtype, f"captured layer {sel[i]}",
                          ulps=max(2.0, 2.0 * hid_ulps[i]))
    gk, gv = ctx.read_kv(0, s.ctx)
    sync()
    L, NK = s.target_layers, s.n_kv_heads * s.head_dim
    tol = max(2.0, 2.0 * kv_ulps)
    assert_rows_close(gk.float().cpu().numpy().reshape(L * s.ctx, NK), cache.k.reshape(L * s.ctx, NK), s.dtype, "K",
                      ulps=tol)
    assert_rows_close(gv.float().cpu().numpy().reshape(L * s.ctx, NK), cache.v.reshape(L * s.ctx, NK), s.dtype, "V",
                      ulps=tol)


# ------------------------------------------------------------------ batch invariance

@pytest.mark.parametrize("shape", [T_BF16, T_FP32_G5])
@pytest.mark.parametrize("C", [0, 37, 250, 256, 600])
def test_target_forward_is_batch_invariant(dl, shape, C):
    s = shape
    w = di.toy_target_weights(s)
    ctx = target_ctx(dl, s, w, max_ctx=C + 64)
    toks = di.uniform_int(C + 16, 0, s.vocab - 1, s.seed + C, "binv").numpy()
    if C:
        run_chunks(dl, ctx, s, toks[:C], [16] * (C // 16) + ([C % 16] if C % 16 else []), sel_capture=False)
    results = []
    for split in ([16], [1] * 16, [7, 9], [3, 13]):
        ctx.rollback(C)
        am, lg, caps = run_chunks(dl, ctx, s, toks[C:], split)
        k, v = ctx.read_kv(C, 16)
        sync()
        results.append((am, lg, caps, k.cpu(), v.cpu()))
    a0 = results[0]
    for r in results[1:]:
        assert np.array_equal(r[0], a0[0])
        assert np.array_equal(r[1], a0[1])
        for i in range(5):
            assert np.array_equal(r[2][i], a0[2][i])
        assert torch.equal(r[3], a0[3]) and torch.equal(r[4], a0[4])


def test_target_forward_errors(dl):
    s = T_FP32_G5
    ctx = target_ctx(dl, s, di.toy_target_weights(s), max_ctx=40)
    t = torch.zeros(17, dtype=torch.int32, device="cuda")
    with pytest.raises(dl.DFlashError):
        ctx.target_forward(t)                     # more than 16 rows
    for _ in range(2):
        ctx.target_forward(t[:16])
    with pytest.raises(dl.DFlashError):
        ctx.target_forward(t[:16])                # 48 > max_ctx: nothing written
    assert ctx.length == 32
    with pytest.raises(dl.DFlashError):           # no fusion weights in a target context
        ctx.fuse_context([torch.zeros(4, s.hidden, device="cuda")] * s.target_layers)
    sync()
    # a capture of a feature layer the stack does not have is refused, nothing enqueued
    short = dl.DFlash(s.replace(draft_layers=4), dev(di.toy_target_weights(s)), max_ctx=40)
    sel = dl.feature_layers(s.target_layers)
    cap = [torch.empty(2, s.hidden, dtype=s.torch_dtype, device="cuda") if l >= 4 else None for l in sel]
    with pytest.raises(dl.DFlashError) as e:
        short.target_forward(t[:2], capture=cap)
    assert e.value.status == -1 and short.length == 0
    short.target_forward(t[:2], capture=[c if l < 4 else None for c, l in zip(cap, sel)])
    sync()
    assert short.length == 2


# ------------------------------------------------------------------ toy end-to-end

@pytest.fixture(scope="module")
def toy(dl):
    s = TOY
    tw = dev(di.toy_target_weights(s))
    dw = dev(di.draft_weights(s))
    prompt = di.toy_prompt(s).cuda()
    n_new = di.TOY_GENERATE
    cap = prompt.shape[0] + n_new + 2 * s.block

    def fresh():
        tgt = dl.DFlash(s.replace(draft_layers=s.target_layers), tw, max_ctx=cap, page_seed=11)
        drf = dl.DFlash(s, dw, max_ctx=cap, page_seed=12)
        return tgt, drf

    from block_diffusion_drafter_context_amd import spec
    tgt, _ = fresh()
    greedy = spec.greedy_generate(tgt, prompt, n_new).cpu().numpy()
    return {"fresh": fresh, "prompt": prompt, "n_new": n_new, "greedy": greedy, "spec": spec}


@pytest.mark.parametrize("mode", ["dflash", "perfect", "null", "prefix"])
def test_toy_spec_equals_greedy(toy, mode):
    """Greedy block verification is lossless: the speculative loop emits the
    GPU's own greedy tokens bit for bit, whatever the drafts."""
    greedy, P, V = toy["greedy"], toy["prompt"].shape[0], TOY.vocab
    rng = np.random.default_rng(9)

    def truth(C):
        return [int(greedy[p - P]) if p - P < len(greedy) else 0 for p in range(C + 1, C + 16)]

    fn = {"dflash": None,
          "perfect": truth,
          "null": lambda C: [(t + 1) % V for t in truth(C)],
          "prefix": lambda C: [t if j < r else (t + 1) % V
                               for r in [int(rng.integers(0, 16))] for j, t in enumerate(truth(C))]}[mode]
    tgt, drf = toy["fresh"]()
    out, ks = toy["spec"].spec_generate(tgt, drf, toy["prompt"], toy["n_new"], drafts_fn=fn)
    print(f"[toy {mode}] steps {len(ks)} mean k {np.mean(ks):.3f} tokens/step {len(out) / max(len(ks), 1):.2f}",
          flush=True)
    first_bad = next((i for i in range(len(out)) if out[i] != greedy[i]), None)
    assert first_bad is None, f"spec diverges from greedy at generated token {first_bad}"
    if mode == "perfect":
        assert all(k == 15 for k in ks[:-1])
    if mode == "null":
        assert ks == [0] * (toy["n_new"] - 1)


@pytest.fixture(scope="module")
def toy_oracle(orc):
    """The oracle's greedy tokens (one token per forward), plus one teacher-forced
    forward over prompt + those tokens in fp64 and in fp32 accumulation: its
    logits at the generated positions and their drift (the bf16 noise floor)."""
    s = TOY
    m = orc.Model(s, di.toy_target_weights(s), n_layers=s.target_layers)
    prompt = di.toy_prompt(s).numpy()
    toks, gaps = orc.greedy_generate(m, prompt, di.TOY_GENERATE)
    P = len(prompt)
    seq = np.concatenate([prompt, toks[:-1]]).astype(np.int32)
    ref = orc.target_forward(m, orc.TargetCache(m, len(seq)), seq, 0, want_logits=True)
    assert np.array_equal(ref["argmax"][P - 1:], toks)  # the oracle is batch invariant
    orc.set_fp32_accumulation(True)
    try:
        alt = orc.target_forward(m, orc.TargetCache(m, len(seq)), seq, 0, want_logits=True)
    finally:
        orc.set_fp32_accumulation(False)
    logits = ref["logits"][P - 1:].copy()
    noise = float(np.abs(alt["logits"][P - 1:].astype(np.float64) - logits).max())
    del ref, alt
    return prompt, toks, gaps, logits, noise


def test_toy_greedy_matches_oracle(dl, toy, toy_oracle):
    """The GPU target, teacher-forced on the oracle's greedy sequence, picks the
    oracle's token at every generated position except near-ties (oracle top-2
    gap inside the bf16 logit band, with the GPU's token inside the band of the
    oracle's maximum); the free-running GPU greedy sequence equals the oracle's
    up to its first near-tie."""
    prompt, otoks, ogaps, ologits, noise = toy_oracle
    band = bf16_logit_tol(noise)
    P, n = len(prompt), len(otoks)
    seq = np.concatenate([prompt, otoks[:-1]]).astype(np.int32)
    tgt, _ = toy["fresh"]()
    am = torch.empty(len(seq), dtype=torch.int32, device="cuda")
    seq_d = torch.from_numpy(seq).cuda()
    for r0 in range(0, len(seq), 16):
        M = min(16, len(seq) - r0)
        tgt.target_forward(seq_d[r0:r0 + M], argmax=am[r0:r0 + M])
    sync()
    pred = am.cpu().numpy()[P - 1:]
    nex = assert_tokens(pred, otoks, ogaps, ref_logits=ologits, dtype="bf16", noise_floor=noise)
    print(f"[toy oracle] noise floor {noise:.4f}; teacher-forced near-tie mismatches {nex} of {n}", flush=True)
    g = toy["greedy"]
    first = next((i for i in range(n) if g[i] != otoks[i]), n)
    print(f"[toy oracle] free-running greedy agrees for the first {first} of {n} tokens", flush=True)
    assert first == n or ogaps[first] < band, f"free-running greedy diverges at {first} (gap {ogaps[first]:.3g})"


def _assert_teacher_forced_greedy(toy, o, band):
    """Every emitted token o[i] is the target's greedy token given prompt +
    o[:i] (teacher-forced in 16-row calls), or its logit lies within `band`
    of that token's.  Returns the indices where they differ."""
    P, V = toy["prompt"].shape[0], TOY.vocab
    ref, _ = toy["fresh"]()
    seq = torch.cat([toy["prompt"], torch.tensor(o[:-1], dtype=torch.int32, device="cuda")])
    am = torch.empty(seq.shape[0], dtype=torch.int32, device="cuda")
    lg = torch.empty(seq.shape[0], V, dtype=torch.float32, device="cuda")
    for r0 in range(0, seq.shape[0], 16):
        M = min(16, seq.shape[0] - r0)
        ref.target_forward(seq[r0:r0 + M], argmax=am[r0:r0 + M], logits=lg[r0:r0 + M])
    sync()
    pred = am[P - 1:].cpu().numpy()
    lgp = lg[P - 1:].cpu().numpy()
    mism = np.flatnonzero(o != pred)
    for i in mism:
        gap = float(lgp[i, pred[i]] - lgp[i, o[i]])
        assert gap <= band, f"token {i}: emitted {o[i]} is {gap:.3g} below the greedy logit"
    return mism


@pytest.mark.parametrize("mode", ["ddtree", "branch", "ddtree22"])
def test_toy_tree_spec_is_lossless(toy, mode):
    """Tree verification ([A] §8.2) keeps greedy output: every emitted token is
    the target's greedy token given the emitted prefix (teacher-forced in
    16-row calls, which equal one-row decoding bit for bit), except at
    near-ties inside the bf16 logit band, where the tree pass and the chain
    pass may order two logits differently (their attention sums run in a
    different order).  'ddtree': trees built from the draft's top-4 per
    position (budget 15); 'ddtree22': budget 22 (two target passes per
    step); 'branch': a wrong 5-node chain first and the right 10-node chain
    second, so acceptance has to take the second branch."""
    P, V, n_new = toy["prompt"].shape[0], TOY.vocab, toy["n_new"]
    greedy = toy["greedy"]

    def truth(C):
        return [int(greedy[p - P]) if p - P < len(greedy) else 0 for p in range(C + 1, C + 11)]

    def branch(C):
        t = truth(C)
        nodes = [(x + 1) % V for x in t[:5]] + t
        parents = [0, 1, 2, 3, 4] + [0] + list(range(6, 15))
        return nodes, parents

    tgt, drf = toy["fresh"]()
    out, ks = toy["spec"].spec_tree_generate(tgt, drf, toy["prompt"], n_new, K=4,
                                             budget=22 if mode == "ddtree22" else 15,
                                             trees_fn=branch if mode == "branch" else None)
    print(f"[toy tree {mode}] steps {len(ks)} mean k {np.mean(ks):.3f}", flush=True)
    o = np.asarray(out)
    mism = _assert_teacher_forced_greedy(toy, o, bf16_logit_tol())
    print(f"[toy tree {mode}] near-tie tokens {len(mism)} of {len(o)}", flush=True)
    if mode == "branch":
        # the forced branch holds the precomputed greedy tokens, so it is right
        # until the emitted sequence leaves greedy at a near-tie; until then
        # every step accepts the whole second branch
        first = next((i for i in range(len(o)) if o[i] != greedy[i]), len(o))
        pos, checked = 1, 0
        for k in ks:
            if pos + 11 > min(first, len(greedy)):
                break
            assert k == 10, f"step at generated token {pos}: accepted {k} of the right 10-node branch"
            pos += k + 1
            checked += 1
        print(f"[toy tree branch] greedy until token {first}; {checked} steps accepted the second branch", flush=True)
        # each such step also relies on the previous step's compaction (the
        # accepted branch's K/V moved behind the root), or its verify would drift
        assert checked >= 1 or first < 12


def test_toy_sampled_spec_matches_oracle(toy):
    """Speculative sampling at T = 1 through the whole loop (draft, draws,
    verify pass, rule, fuse, inject, rollback): at every step (k, next token)
    is the oracle's rule on that step's fp32 logits, and on the first steps
    the drafts are the oracle's Gumbel-max draws from the draft's rows (near
    ties aside); the emitted tokens are each step's accepted drafts and its
    next token."""
    from oracle import sampling as sp
    B = TOY.block
    steps = []
    stats = {"draw_ties": 0, "rule_ties": 0}

    def on_step(C, sd, vin, dlg, tlg, res):
        blk, d_l, t_l, r = vin.cpu().numpy(), dlg.cpu().numpy(), tlg.cpu().numpy(), res.cpu().numpy()
        if len(steps) < 3:
            ref = sp.sample_tokens(d_l[1:], 1.0, sd)
            for j in np.flatnonzero(ref["tokens"] != blk[1:]):
                assert ref["gap"][j] < 1e-3, f"step at C={C}: draft {j + 1} {blk[j + 1]} vs {ref['tokens'][j]}"
                stats["draw_ties"] += 1
        ref = sp.verify_sample(blk, d_l, t_l, 1.0, sd)
        if (int(r[0]), int(r[1])) != (ref["k"], ref["bonus"]):
            assert min(ref["accept_margins"] + [ref["draw_margin"]]) < 1e-9, (C, r, ref)
            stats["rule_ties"] += 1
        steps.append((blk[1:1 + int(r[0])].tolist(), int(r[1])))

    tgt, drf = toy["fresh"]()
    out, ks = toy["spec"].spec_sample_generate(tgt, drf, toy["prompt"], 64, 1.0, 1234, on_step=on_step)
    print(f"[toy sampled] steps {len(ks)} mean k {np.mean(ks):.3f}; {stats}", flush=True)
    assert stats["draw_ties"] <= 1 and stats["rule_ties"] <= 1
    emitted = [out[0]]
    for acc, nxt in steps:
        emitted += acc + [nxt]
    assert emitted[:len(out)] == out
    assert ks == [len(a) for a, _ in steps] and all(0 <= k <= B - 1 for k in ks)


def test_toy_sampled_spec_low_temperature_is_greedy(toy):
    """At T = 1e-4 the draws and the rule reduce to argmaxes: the sampled loop
    emits the target's greedy tokens, teacher-forced, except where two logits
    lie within the bf16 band (or within 1e-4 * 17, the reach of a Gumbel
    perturbation at that temperature)."""
    tgt, drf = toy["fresh"]()
    out, ks = toy["spec"].spec_sample_generate(tgt, drf, toy["prompt"], toy["n_new"], 1e-4, 5)
    o = np.asarray(out)
    mism = _assert_teacher_forced_greedy(toy, o, bf16_logit_tol() + 17e-4)
    print(f"[toy sampled T=1e-4] steps {len(ks)} mean k {np.mean(ks):.3f}; near-tie tokens {len(mism)} of {len(o)}",
          flush=True)
    assert len(mism) <= len(o) // 20


@pytest.mark.parametrize("tree", [False, True])
def test_toy_target_layers_match_oracle(dl, orc, tree):
    """The toy target at the stated bar, layer by layer: 16 rows (a causal
    block, or a 16-node random tree) over 2048 cached positions of seeded K/V,
    each of the 8 layers against the oracle's layer on the GPU's own input to
    it (2 bf16 ulps), the logits against the oracle's LM head on the GPU's
    final residual (2e-2) with tokens exact except top-2 gaps below 1e-3."""
    from tests.gpu_helpers import check_target_layers
    s = TOY.replace(draft_layers=TOY.target_layers)
    C, M, L = di.TOY_PROMPT, 16, TOY.target_layers
    w = di.toy_target_weights(TOY)
    ctx = dl.DFlash(s, dev(w), max_ctx=C + 64, page_seed=13)
    k, v = di.context_kv(s, C, tag="toy_target_kv")
    ctx.load_kv(k.cuda(), v.cuda())
    toks = di.uniform_int(M, 0, s.vocab - 1, s.seed, "toy_rows").numpy()
    par = di.random_tree(M, s.seed, "toy_tree") if tree else None
    layers = torch.empty(L, M, s.hidden, dtype=s.torch_dtype, device="cuda")
    am, lg = ctx.target_forward(torch.from_numpy(toks).cuda(), want_logits=True, layers_out=layers,
                                parent=torch.from_numpy(par).cuda() if tree else None)
    sync()
    m = orc.Model(s, w, n_layers=L)
    NK = s.n_kv_heads * s.head_dim
    cache = orc.TargetCache(m, C + M)
    cache.k[:, :C] = k.reshape(L, C, NK).double().numpy()
    cache.v[:, :C] = v.reshape(L, C, NK).double().numpy()
    err, ulps = check_target_layers(orc, m, w, s, cache, C, toks, par, layers, lg.cpu().numpy(), am.cpu().numpy())
    print(f"[toy target {'tree' if tree else 'chain'}] per layer worst {ulps:.2f} ulps; LM head max|dlogit| {err:.3g}",
          flush=True)
