"""Parity at the workloads' full sizes, in the launch configuration the bench
times: the Qwen3-8B-shaped draft at 4096 and 36864 context, the 27B-class draft
at 36864 context (complete blocks against the oracle), and prefill-side fusion
and injection of 32768 rows (sampled rows / positions the oracle computes one
by one, including the ragged last tile)."""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from tests.gpu_helpers import assert_logits, assert_rows_close, assert_tokens, check_layers, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_drafter_context_amd as m
    m.lib()
    return m


def _draft_case(dl, orc, s, C):
    w = di.draft_weights(s)
    ctx = dl.DFlash(s, dev(w), max_ctx=C + 64, page_seed=17)
    k, v = di.context_kv(s, C)
    ctx.load_kv(k.cuda(), v.cuda())
    anchor = di.anchor_token(s)
    a = torch.tensor([anchor], dtype=torch.int32, device="cuda")
    layers = torch.empty(s.draft_layers, s.block, s.hidden, dtype=s.torch_dtype, device="cuda")
    tok, lg = ctx.draft_block(a, want_logits=True, layers_out=layers)
    torch.cuda.synchronize()
    print(f"[fullsize] {s.name} C={C}: gpu done", flush=True)
    m = orc.Model(s, w)
    # the stated bar, layer by layer on identical inputs
    err, ulps = check_layers(orc, m, w, s, k, v, C, anchor, layers, lg.cpu().numpy(), tok.cpu().numpy())
    print(f"[fullsize] {s.name} C={C}: per layer, worst {ulps:.2f} bf16 ulps of the row max; LM head given "
          f"the GPU's final residual max|dlogit| {err:.3g}", flush=True)
    # end to end (bf16 rounding compounds over the layers): a separate, widened band
    ref = orc.draft_block(m, k, v, C, anchor)
    noise = orc.draft_noise_floor(m, k, v, C, anchor, ref["logits"])
    lg = lg.cpu().numpy()
    print(f"[fullsize] {s.name} C={C}: end to end max|dlogit| {np.abs(lg - ref['logits']).max():.3g}, "
          f"oracle fp32-vs-fp64 drift {noise:.3g}", flush=True)
    assert_logits(lg, ref["logits"], s.dtype, noise)
    n_ex = assert_tokens(tok.cpu().numpy(), ref["tokens"], ref["gap"], lg, ref["logits"], s.dtype, noise)
    print(f"[fullsize] {s.name} C={C}: exempt near-tie token mismatches {n_ex}/{s.block}", flush=True)
    # the per-step verification against the synthetic target
    u, r, last = di.target_coins(s)
    g = di.synthetic_target_argmax(tok.cpu().numpy(), u.numpy(), r.numpy(), last, s.vocab)
    res = ctx.verify_accept(tok, torch.from_numpy(g).cuda()).cpu().tolist()
    assert tuple(res) == orc.accept(tok.cpu().numpy(), g)
    return ctx, w


@pytest.mark.timeout(900)
def test_qwen3_8b_4k_draft(dl, orc):
    _draft_case(dl, orc, di.SHAPES["qwen3_8b_4k"], 4096)


@pytest.mark.timeout(900)
def test_qwen3_8b_36k_draft(dl, orc):
    _draft_case(dl, orc, di.SHAPES["qwen3_8b_36k"], 36864)


@pytest.mark.timeout(1200)
def test_dense27b_36k_draft(dl, orc):
    _draft_case(dl, orc, di.SHAPES["dense27b_36k"], 36864)


@pytest.mark.timeout(900)
def test_qwen3_8b_step_fuse_inject_16(dl, orc):
    """Per-step path at full size: fuse the 16 verified rows' target features,
    and inject 16 rows after a 4096-token context (skinny-GEMM kernels).  The
    injection input is a generated stand-in for fused features, so each call is
    checked against the oracle on identical inputs."""
    s = di.SHAPES["qwen3_8b_4k"]
    w = di.draft_weights(s, need_draft=False, need_lm=False)
    ctx = dl.DFlash(s, dev(w), max_ctx=4096 + 64, max_rows=16, page_seed=4)
    k, v = di.context_kv(s, 4096)
    ctx.load_kv(k.cuda(), v.cuda())
    sel = orc.feature_layers(s.target_layers)
    hid = {l: di.target_hidden(s, l, 16, tag="step") for l in sel}
    fused = ctx.fuse_context([hid[l].cuda() if l in hid else None for l in range(s.target_layers)])
    feat = di.fused_context(s, 16, tag="verified")
    ctx.inject_kv(feat.cuda(), 4096)
    gk, gv = ctx.read_kv(4096, 16)
    torch.cuda.synchronize()
    m = orc.Model(s, w)
    rf = orc.fuse_rows(m, [hid[l] for l in sel], range(16))
    assert_rows_close(fused.float().cpu().numpy(), rf, s.dtype, "fuse16")
    rk, rv = orc.inject_rows(m, feat, range(16), 4096)
    L = s.draft_layers
    assert_rows_close(gk.float().cpu().numpy().reshape(L * 16, -1), rk.reshape(L * 16, -1), s.dtype, "K16")
    assert_rows_close(gv.float().cpu().numpy().reshape(L * 16, -1), rv.reshape(L * 16, -1), s.dtype, "V16")
    # the injected rows did not disturb the context before them
    k0, v0 = ctx.read_kv(4000, 96)
    torch.cuda.synchronize()
    assert torch.equal(k0.cpu(), k[:, 4000:4096]) and torch.equal(v0.cpu(), v[:, 4000:4096])


@pytest.mark.timeout(1200)
def test_prefill_fuse_inject_32k_sampled(dl, orc):
    """Fusion GEMM (M=32768, K=25600, N=5120) and injection of 32768 rows into
    256-token pages, checked on sampled rows including the ragged edges."""
    s = di.SHAPES["fusion_prefill_32k"]
    M = s.ctx
    w = di.draft_weights(s, need_draft=False, need_lm=False)
    ctx = dl.DFlash(s, dev(w), max_ctx=M, max_rows=M, page_seed=8)
    sel = orc.feature_layers(s.target_layers)
    hid = {l: di.target_hidden(s, l, M) for l in sel}
    dev_hid = [hid[l].cuda() if l in hid else None for l in range(s.target_layers)]
    fused = ctx.fuse_context(dev_hid)
    torch.cuda.synchronize()
    del dev_hid
    rows = [0, 1, 63, 64, 4095, 17000, 32704, M - 1]
    m = orc.Model(s, w)
    rf = orc.fuse_rows(m, [hid[l] for l in sel], rows)
    assert_rows_close(fused[rows].float().cpu().numpy(), rf, s.dtype, "fuse32k")
    # injection of synthetic fused features (independent of the fusion output)
    feat = di.fused_context(s, M, tag="prefill")
    ctx.inject_kv(feat.cuda(), 0)
    torch.cuda.synchronize()
    rk, rv = orc.inject_rows(m, feat, rows, 0)
    L = s.draft_layers
    for i, r in enumerate(rows):
        gk, gv = ctx.read_kv(r, 1)
        assert_rows_close(gk.float().cpu().numpy().reshape(L, -1), rk[:, i], s.dtype, f"K pos {r}")
        assert_rows_close(gv.float().cpu().numpy().reshape(L, -1), rv[:, i], s.dtype, f"V pos {r}")


@pytest.mark.timeout(1500)
def test_qwen3_8b_target_verify_4k(dl, orc):
    """The verify side of a step at the Qwen3-8B target shape ([A] §1.2
    parallel verification; [B] 技术内幕): a causal forward of 16 rows through 36
    target layers (hidden 4096, 32/8 heads x 128, FFN 12288, vocab 151936)
    over a 4096-token paged target KV cache of seeded values, capturing the
    five feature layers the draft fuses.  The oracle's dense cache holds the
    same bytes (no oracle prefill).  Logits, tokens and captured layers are
    compared with the oracle's causal forward under the bf16 band that its
    own fp32-vs-fp64 drift sets over 36 layers."""
    from tests.gpu_helpers import bf16_logit_tol, drift_ulps
    s = di.SHAPES["qwen3_8b_4k"].replace(name="qwen3_8b_target", draft_layers=36)
    C, M = 4096, 16
    w = di.toy_target_weights(s)
    ctx = dl.DFlash(s, dev(w), max_ctx=C + 64, page_seed=23)
    k, v = di.context_kv(s, C, tag="target_kv")
    ctx.load_kv(k.cuda(), v.cuda())
    toks = di.uniform_int(M, 0, s.vocab, s.seed, "verify_rows")
    sel = orc.feature_layers(s.target_layers)
    cap = [torch.empty(M, s.hidden, dtype=s.torch_dtype, device="cuda") for _ in range(5)]
    am, lg = ctx.target_forward(toks.cuda(), want_logits=True, capture=cap)
    torch.cuda.synchronize()
    assert ctx.length == C + M
    print(f"[fullsize] target verify 36 layers, C={C}, {M} rows: gpu done", flush=True)
    m = orc.Model(s, w, n_layers=36)
    NK = s.n_kv_heads * s.head_dim

    def run_oracle():
        cache = orc.TargetCache(m, C + M)
        cache.k[:, :C] = k.reshape(36, C, NK).double().numpy()
        cache.v[:, :C] = v.reshape(36, C, NK).double().numpy()
        return orc.target_forward(m, cache, toks.numpy(), C, capture=sel, want_logits=True)

    ref = run_oracle()
    orc.set_fp32_accumulation(True)
    try:
        alt = run_oracle()
    finally:
        orc.set_fp32_accumulation(False)
    noise = float(np.abs(alt["logits"].astype(np.float64) - ref["logits"].astype(np.float64)).max())
    lg = lg.cpu().numpy()
    err = float(np.abs(lg - ref["logits"]).max())
    print(f"[fullsize] target verify: max|dlogit| {err:.3g}, oracle fp32-vs-fp64 drift {noise:.3g}", flush=True)
    assert_logits(lg, ref["logits"], s.dtype, noise)
    n_ex = assert_tokens(am.cpu().numpy(), ref["argmax"], ref["gap"], lg, ref["logits"], s.dtype, noise)
    print(f"[fullsize] target verify: exempt near-tie token mismatches {n_ex}/{M}", flush=True)
    for i in range(5):
        ulps = drift_ulps(alt["hidden"][i], ref["hidden"][i])
        assert_rows_close(cap[i].float().cpu().numpy(), ref["hidden"][i], s.dtype, f"captured layer {sel[i]}",
                          ulps=max(2.0, 2.0 * ulps))
