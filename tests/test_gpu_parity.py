"""Parity of the HIP path (through the C ABI) with the CPU oracle, at sizes the
oracle finishes in seconds: several tiles, ragged tails and edge cases."""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from tests.gpu_helpers import (MID_BF16, MID_BF16_D64, MID_BF16_H352, MID_FP32_G5, assert_logits,
                               assert_rows_close, assert_tokens, check_layers, dev)

pytestmark = pytest.mark.gpu

TINY = di.SHAPES["tiny_fp32"]


@pytest.fixture(scope="module")
def dl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_drafter_context_amd as m
    m.lib()
    return m


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ acceptance

@pytest.mark.parametrize("B", [16, 7, 2])
def test_accept_matches_oracle(dl, orc, B):
    s = TINY.replace(block=B)
    ctx = dl.DFlash(s, dev(di.draft_weights(s, need_draft=False, need_lm=False)), max_ctx=64)
    rng = np.random.default_rng(B)
    for trial in range(300):
        d = rng.integers(0, 50, B).astype(np.int32)
        g = d.copy()
        g[:-1] = d[1:]
        g[-1] = rng.integers(0, 50)
        flip = rng.random(B) < (trial % 7) / 7.0
        g = np.where(flip, (g + 1 + rng.integers(0, 5, B)) % 60, g).astype(np.int32)
        out = ctx.verify_accept(torch.from_numpy(d).cuda(), torch.from_numpy(g).cuda())
        sync()
        assert tuple(out.cpu().tolist()) == orc.accept(d, g)


# ------------------------------------------------------------------ fusion

@pytest.mark.parametrize("shape,M", [(TINY, 1), (TINY, 3), (TINY, 16), (TINY, 17), (TINY, 128), (TINY, 130),
                                     (MID_BF16, 1), (MID_BF16, 16), (MID_BF16, 100), (MID_BF16, 300),
                                     (MID_BF16_H352, 17), (MID_BF16_H352, 300), (MID_FP32_G5, 40)])
def test_fuse_matches_oracle(dl, orc, shape, M):
    w = di.draft_weights(shape, gains="random", need_draft=False, need_lm=False)
    ctx = dl.DFlash(shape, dev(w), max_ctx=64, max_rows=max(M, 16))
    sel = orc.feature_layers(shape.target_layers)
    hidden = {l: di.target_hidden(shape, l, M) for l in sel}
    layer_ptrs = [hidden[l].cuda() if l in hidden else None for l in range(shape.target_layers)]
    out = ctx.fuse_context(layer_ptrs)
    sync()
    ref = orc.fuse_rows(orc.Model(shape, w), [hidden[l] for l in sel], range(M))
    assert_rows_close(out.float().cpu().numpy(), ref, shape.dtype, f"fuse M={M}")


def test_fuse_strided_rows(dl, orc):
    """Hidden states with a row stride larger than H (a view into a wider buffer)."""
    s = MID_BF16
    M = 24
    w = di.draft_weights(s, need_draft=False, need_lm=False)
    ctx = dl.DFlash(s, dev(w), max_ctx=64, max_rows=M)
    sel = orc.feature_layers(s.target_layers)
    wide = {l: di.normal((M, s.hidden + 64), s.seed, f"wide.{l}", 1.0, s.torch_dtype) for l in sel}
    views = [wide[l].cuda()[:, 32:32 + s.hidden] if l in wide else None for l in range(s.target_layers)]
    out = ctx.fuse_context(views)
    sync()
    ref = orc.fuse_rows(orc.Model(s, w), [wide[l][:, 32:32 + s.hidden].contiguous() for l in sel], range(M))
    assert_rows_close(out.float().cpu().numpy(), ref, s.dtype, "strided fuse")


# ------------------------------------------------------------------ injection

@pytest.mark.parametrize("shape", [TINY, MID_BF16, MID_BF16_D64, MID_BF16_H352])
def test_inject_matches_oracle(dl, orc, shape):
    """Injections of 300 rows (prefill GEMM), 16 and 5 rows (skinny), 270 rows at
    the unaligned position 321 (crossing a page boundary) and 1 row, into a
    shuffled page table; every position read back and compared with the oracle."""
    w = di.draft_weights(shape, gains="random", need_draft=False, need_lm=False)
    ctx = dl.DFlash(shape, dev(w), max_ctx=1024, max_rows=600, page_seed=99)
    m = orc.Model(shape, w)
    pos = 0
    ks, vs = [], []
    for M in (300, 16, 5, 270, 1):
        fused = di.fused_context(shape, M, tag=f"fused{pos}")
        ctx.inject_kv(fused.cuda(), pos)
        k, v = orc.inject_rows(m, fused, range(M), pos)
        ks.append(k)
        vs.append(v)
        pos += M
    assert ctx.length == pos
    gk, gv = ctx.read_kv(0, pos)
    sync()
    rk, rv = np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)
    L = shape.draft_layers
    assert_rows_close(gk.float().cpu().numpy().reshape(L * pos, -1), rk.reshape(L * pos, -1), shape.dtype, "K")
    assert_rows_close(gv.float().cpu().numpy().reshape(L * pos, -1), rv.reshape(L * pos, -1), shape.dtype, "V")


def test_load_read_roundtrip(dl):
    s = MID_BF16
    ctx = dl.DFlash(s, dev(di.draft_weights(s, need_draft=False, need_lm=False)), max_ctx=2000, page_seed=5)
    k, v = di.context_kv(s, 777)
    ctx.load_kv(k.cuda(), v.cuda())
    gk, gv = ctx.read_kv(0, 777)
    sync()
    assert torch.equal(gk.cpu(), k) and torch.equal(gv.cpu(), v)


# ------------------------------------------------------------------ draft block

def _draft_pair(dl, orc, shape, C, anchor, page_seed=3, w=None):
    w = di.draft_weights(shape, gains="random") if w is None else w
    ctx = dl.DFlash(shape, dev(w), max_ctx=max(C, 1) + 64, page_seed=page_seed)
    k = v = None
    if C > 0:
        k, v = di.context_kv(shape, C)
        ctx.load_kv(k.cuda(), v.cuda())
    a = torch.tensor([anchor], dtype=torch.int32, device="cuda")
    layers = torch.empty(shape.draft_layers, shape.block, shape.hidden, dtype=shape.torch_dtype, device="cuda")
    tokens, logits = ctx.draft_block(a, want_logits=True, layers_out=layers)
    sync()
    m = orc.Model(shape, w)
    # the stated bar layer by layer on identical inputs, then the end-to-end comparison
    check_layers(orc, m, w, shape, k, v, C, anchor, layers, logits.cpu().numpy(), tokens.cpu().numpy())
    ref = orc.draft_block(m, k, v, C, anchor)
    ref["noise"] = orc.draft_noise_floor(m, k, v, C, anchor, ref["logits"]) if shape.dtype == "bf16" else None
    return tokens.cpu().numpy(), logits.cpu().numpy(), ref, ctx


@pytest.mark.parametrize("shape,C", [(TINY, 0), (TINY, 1), (TINY, 128), (TINY, 200),
                                     (MID_FP32_G5, 100),
                                     (MID_BF16, 0), (MID_BF16, 1), (MID_BF16, 63), (MID_BF16, 64),
                                     (MID_BF16, 255), (MID_BF16, 256), (MID_BF16, 257), (MID_BF16, 1000),
                                     (MID_BF16_D64, 300)])
def test_draft_block_matches_oracle(dl, orc, shape, C):
    tok, lg, ref, _ = _draft_pair(dl, orc, shape, C, anchor=shape.vocab // 3)
    assert_logits(lg, ref["logits"], shape.dtype, ref["noise"])
    assert_tokens(tok, ref["tokens"], ref["gap"], lg, ref["logits"], shape.dtype, ref["noise"])


@pytest.mark.parametrize("B", [7, 2])
def test_draft_short_block(dl, orc, B):
    s = MID_BF16.replace(block=B)
    tok, lg, ref, _ = _draft_pair(dl, orc, s, 130, anchor=11)
    assert tok.shape == (B,) and lg.shape == (B, s.vocab)
    assert_logits(lg, ref["logits"], s.dtype, ref["noise"])
    assert_tokens(tok, ref["tokens"], ref["gap"], lg, ref["logits"], s.dtype, ref["noise"])


@pytest.mark.parametrize("B", [16, 5])
def test_draft_lm_head_partial_tile(dl, orc, B):
    """Vocabulary 1008 ends in half a 32-column LM-head tile; a short block
    leaves rows the logits buffer does not have.  Tokens must not depend on
    whether logits are requested."""
    s = MID_BF16_H352.replace(block=B)
    w = di.draft_weights(s, gains="random")
    tok, lg, ref, ctx = _draft_pair(dl, orc, s, 300, anchor=5, w=w)
    assert lg.shape == (B, s.vocab)
    assert_logits(lg, ref["logits"], s.dtype, ref["noise"])
    assert_tokens(tok, ref["tokens"], ref["gap"], lg, ref["logits"], s.dtype, ref["noise"])
    a = torch.tensor([5], dtype=torch.int32, device="cuda")
    t_off, _ = ctx.draft_block(a, want_logits=False)
    sync()
    assert torch.equal(t_off.cpu(), torch.as_tensor(np.asarray(tok)).to(t_off.dtype))


def test_layer_capture_changes_nothing(dl):
    """The per-layer copy is an extra store in the down projection's epilogue:
    tokens and logits are bit-identical with and without it."""
    s = MID_BF16
    ctx = dl.DFlash(s, dev(di.draft_weights(s)), max_ctx=600)
    k, v = di.context_kv(s, 400)
    ctx.load_kv(k.cuda(), v.cuda())
    a = torch.tensor([9], dtype=torch.int32, device="cuda")
    t1, l1 = ctx.draft_block(a, want_logits=True)
    t1, l1 = t1.clone(), l1.clone()
    layers = torch.empty(s.draft_layers, s.block, s.hidden, dtype=s.torch_dtype, device="cuda")
    t2, l2 = ctx.draft_block(a, want_logits=True, layers_out=layers)
    sync()
    assert torch.equal(t1, t2) and torch.equal(l1, l2)
    st = dl.lib().dflash_draft_block_ex(ctx.h, a.data_ptr(), None, t2.data_ptr(), layers.data_ptr(), s.hidden - 1,
                                        None)
    assert st == -1  # layer_ld below H: refused before anything is enqueued


def test_draft_deterministic_and_logits_optional(dl, orc):
    s = MID_BF16
    w = di.draft_weights(s)
    ctx = dl.DFlash(s, dev(w), max_ctx=600)
    k, v = di.context_kv(s, 500)
    ctx.load_kv(k.cuda(), v.cuda())
    a = torch.tensor([7], dtype=torch.int32, device="cuda")
    t1, l1 = ctx.draft_block(a, want_logits=True)
    t1, l1 = t1.clone(), l1.clone()
    t2, _ = ctx.draft_block(a, want_logits=False)
    t3, l3 = ctx.draft_block(a, want_logits=True)
    sync()
    assert torch.equal(t1, t2) and torch.equal(t1, t3) and torch.equal(l1, l3)


def test_tiny_full_chain(dl, orc):
    """The tiny workload end to end: 128 context rows of target features ->
    fusion -> injection -> one draft block -> acceptance against the
    synthetic target, every stage compared with the oracle chain."""
    s = TINY
    w = di.draft_weights(s)
    m = orc.Model(s, w)
    ctx = dl.DFlash(s, dev(w), max_ctx=s.ctx + 16, max_rows=s.ctx, page_seed=1)
    sel = orc.feature_layers(s.target_layers)
    assert sel == [1, 2, 4, 5, 6]
    hidden = {l: di.target_hidden(s, l, s.ctx) for l in range(s.target_layers)}
    fused = ctx.fuse_context([hidden[l].cuda() for l in range(s.target_layers)])
    ctx.inject_kv(fused, 0)
    anchor = di.anchor_token(s)
    tok, lg = ctx.draft_block(torch.tensor([anchor], dtype=torch.int32, device="cuda"), want_logits=True)
    sync()
    rf = orc.fuse_rows(m, [hidden[l] for l in sel], range(s.ctx))
    assert_rows_close(fused.cpu().numpy(), rf, s.dtype, "fused")
    rk, rv = orc.inject_rows(m, orc.to_storage(rf, s.dtype), range(s.ctx), 0)
    to_kv = lambda a: orc.to_storage(a, s.dtype).view(s.draft_layers, s.ctx, s.n_kv_heads, s.head_dim)
    ref = orc.draft_block(m, to_kv(rk), to_kv(rv), s.ctx, anchor)
    assert_logits(lg.cpu().numpy(), ref["logits"], s.dtype)
    assert_tokens(tok.cpu().numpy(), ref["tokens"], ref["gap"], lg.cpu().numpy(), ref["logits"], s.dtype)
    u, r, last = di.target_coins(s)
    g = di.synthetic_target_argmax(tok.cpu().numpy(), u.numpy(), r.numpy(), last, s.vocab)
    res = ctx.verify_accept(tok, torch.from_numpy(g).cuda())
    sync()
    assert tuple(res.cpu().tolist()) == orc.accept(ref["tokens"], g)


def test_rollback_equals_shorter_injection(dl):
    """Injecting all B verified rows then rolling back to C+k+1 leaves the same
    draft as injecting only the k+1 kept rows (bit-identical)."""
    s = MID_BF16
    w = dev(di.draft_weights(s))
    C = 200
    k, v = di.context_kv(s, C)
    fused = di.fused_context(s, 16, tag="verified").cuda()
    a = torch.tensor([5], dtype=torch.int32, device="cuda")
    outs = []
    for keep in (None, 4):
        ctx = dl.DFlash(s, w, max_ctx=C + 32)
        ctx.load_kv(k.cuda(), v.cuda())
        if keep is None:
            ctx.inject_kv(fused, C)
            ctx.rollback(C + 4)
        else:
            ctx.inject_kv(fused[:keep].contiguous(), C)
        assert ctx.length == C + 4
        outs.append(ctx.draft_block(a, want_logits=True))
    sync()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_error_paths(dl):
    s = TINY
    ctx = dl.DFlash(s, dev(di.draft_weights(s)), max_ctx=40, max_rows=32)
    f = di.fused_context(s, 32).cuda()
    with pytest.raises(dl.DFlashError) as e:
        ctx.inject_kv(f, pos0=3)
    assert e.value.status == -5
    ctx.inject_kv(f, 0)
    with pytest.raises(dl.DFlashError) as e:
        ctx.inject_kv(f[:16].contiguous(), 32)
    assert e.value.status == -2 and ctx.length == 32
    with pytest.raises(dl.DFlashError) as e:
        ctx.rollback(33)
    assert e.value.status == -1 and ctx.length == 32
    ctx.rollback(10)
    assert ctx.length == 10
    with pytest.raises(dl.DFlashError):
        ctx.read_kv(5, 6)


def test_trace_records(dl):
    """Per-launch trace durations: one record per draft call, all positive, and
    their sum equals the summed total; capacity bounds the count."""
    import ctypes as C
    s = TINY
    ctx = dl.DFlash(s, dev(di.draft_weights(s)), max_ctx=200)
    k, v = di.context_kv(s, 100)
    ctx.load_kv(k.cuda(), v.cuda())
    a = torch.tensor([3], dtype=torch.int32, device="cuda")
    L = dl.lib()
    assert L.dflash_trace_enable(ctx.h, 7, 8) == 0
    for _ in range(5):
        ctx.draft_block(a)
    buf = (C.c_float * 8)()
    n = C.c_int32()
    assert L.dflash_trace_read_each(ctx.h, buf, 8, C.byref(n)) == 0
    assert n.value == 5 and all(x > 0 for x in buf[:5])
    tot, m = C.c_double(), C.c_int32()
    assert L.dflash_trace_read(ctx.h, C.byref(tot), C.byref(m)) == 0
    assert m.value == 5 and abs(tot.value - sum(buf[:5])) <= 1e-3 * tot.value + 1e-6
    assert L.dflash_trace_read_each(ctx.h, buf, 2, C.byref(n)) == 0 and n.value == 2
    assert L.dflash_trace_enable(ctx.h, 0, 0) == 0


def test_hbm_read_probe(dl):
    """The streaming-read measurement aid reads the whole-round prefix of its
    buffer and rejects a misaligned one."""
    buf = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    n = dl.hbm_read_probe(buf, sink)
    sync()
    assert 0 < n <= buf.numel() and n % (16 * 64 * 16) == 0
    assert dl.hbm_read_probe(buf[:1024], sink) == 0  # too small for one round per wave: nothing launched
    with pytest.raises(dl.DFlashError) as e:
        dl.hbm_read_probe(buf[1:], sink)
    assert e.value.status == -1
