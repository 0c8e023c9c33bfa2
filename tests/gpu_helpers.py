"""Shared helpers of the GPU parity tests: device copies, tolerances, checks."""
import numpy as np
import torch

import dflash_inputs as di

# a bf16 shape small enough for the oracle in seconds that still spans several
# tiles, ragged K (FFN 1376 = 43 chunks of 32) and a vocab that is not a power of two
MID_BF16 = di.Shape("mid_bf16", "bf16", hidden=512, target_layers=12, draft_layers=2, n_q_heads=8,
                    n_kv_heads=2, head_dim=128, ffn=1376, vocab=4000, ctx=300, seed=21)
MID_BF16_D64 = MID_BF16.replace(name="mid_bf16_d64", n_q_heads=8, n_kv_heads=4, head_dim=64, seed=22)
# hidden 352 is a multiple of 32 but not of 64: the prefill GEMMs take their
# 32-deep K-step path and a partial 256-column tile
MID_BF16_H352 = di.Shape("mid_bf16_h352", "bf16", hidden=352, target_layers=10, draft_layers=2, n_q_heads=4,
                         n_kv_heads=2, head_dim=64, ffn=704, vocab=1008, ctx=300, seed=24)
MID_FP32_G5 = di.Shape("mid_fp32_g5", "fp32", hidden=320, target_layers=9, draft_layers=1, n_q_heads=10,
                       n_kv_heads=2, head_dim=64, ffn=688, vocab=1024, ctx=100, seed=23)

# Token exactness is required except where the oracle's top-2 gap is below the
# noise two correct implementations can differ by.  fp32: 1e-3.  bf16: the
# logit tolerance 2e-2 -- with bf16 storage points, fp32 instead of fp64
# accumulation alone (same definition, same rounding points) moves logits by
# ~1e-2, so gaps below that can reorder.  A mismatching GPU token must still be
# a near-argmax of the oracle's logits (within the same band).
TIE_GAP = {"fp32": 1e-3, "bf16": 2e-2}


def dev(w):
    return {k: v.cuda() for k, v in w.items()}


def bf16_ulp(x):
    x = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 7)


def drift_ulps(alt, ref):
    """Largest per-row difference between two oracle variants, in bf16 ulps of the row max."""
    alt = np.asarray(alt, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    return float((np.abs(alt - ref).max(axis=1) / bf16_ulp(np.abs(ref).max(axis=1))).max())


def assert_rows_close(got, ref, dtype, what="", ulps=2.0):
    """fp32: per-row max|d| / max|ref| <= 1e-4.  bf16 intermediates: per-row
    max|d| <= `ulps` (default 2) bf16 ulps of the row's max magnitude."""
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    err = np.abs(got - ref).max(axis=1)
    mx = np.abs(ref).max(axis=1)
    if dtype == "fp32":
        bad = err > 1e-4 * np.maximum(mx, 1e-30)
    else:
        bad = err > ulps * bf16_ulp(mx)
    assert not bad.any(), f"{what}: rows {np.flatnonzero(bad)[:8]} err {err[bad][:8]} rowmax {mx[bad][:8]}"


def bf16_logit_tol(noise_floor=None):
    """bf16 logits: 2e-2 absolute, widened to twice the oracle's own fp32-vs-fp64
    accumulation drift when that is larger (deep / wide shapes)."""
    return 2e-2 if noise_floor is None else max(2e-2, 2.0 * noise_floor)


def assert_logits(got, ref, dtype, noise_floor=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "fp32":
        rel = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert rel.max() <= 1e-4, f"fp32 logits relative error {rel.max():.3g}"
    else:
        err = np.abs(got - ref).max()
        tol = bf16_logit_tol(noise_floor)
        assert err <= tol, f"bf16 logits absolute error {err:.3g} > {tol:.3g} (noise floor {noise_floor})"


def assert_tokens(got, ref, gap, logits=None, ref_logits=None, dtype="bf16", noise_floor=None):
    """Returns the number of exempt mismatches."""
    got, ref = np.asarray(got), np.asarray(ref)
    tol = TIE_GAP[dtype] if dtype == "fp32" else bf16_logit_tol(noise_floor)
    mism = np.flatnonzero(got != ref)
    for j in mism:
        extra = ""
        if logits is not None:
            extra = (f"; row max|dlogit| {np.abs(np.asarray(logits[j], np.float64) - ref_logits[j]).max():.3g}, "
                     f"all rows {np.abs(np.asarray(logits, np.float64) - ref_logits).max():.3g}")
        assert gap[j] < tol, f"token mismatch at row {j}: gpu {got[j]} oracle {ref[j]} gap {gap[j]:.3g}{extra}"
        if ref_logits is not None:
            short = float(ref_logits[j].max()) - float(ref_logits[j][got[j]])
            assert short < tol, f"row {j}: gpu token {got[j]} is {short:.3g} below the oracle max"
    return len(mism)


def check_layers(orc, model, w, shape, ctx_k, ctx_v, C, anchor, layers, logits, tokens):
    """Parity at the stated bar, one launch group at a time: each draft layer's
    GPU input (the embedding rows, then the GPU's own previous layer output)
    goes through the oracle's one-layer step, and the GPU's output of that layer
    must be within 2 bf16 ulps of the row maximum (fp32: 1e-4 relative); the
    GPU's final residual goes through the oracle's LM head, and the GPU logits
    must be within 2e-2 absolute (fp32: 1e-4 relative), tokens exact except
    where the oracle's top-2 gap is below 1e-3.  Returns the largest logit
    difference and the largest per-layer difference in ulps of the row max."""
    L, B, H = shape.draft_layers, shape.block, shape.hidden
    gl = layers.float().cpu().numpy().astype(np.float64).reshape(L, B, H)
    ids = [anchor] + [shape.mask_id] * (B - 1)
    x_in = w["embed"][ids].double().numpy()
    worst_ulps = 0.0
    for l in range(L):
        kl = ctx_k[l] if C > 0 else None
        vl = ctx_v[l] if C > 0 else None
        ref = orc.draft_layer(model, l, kl, vl, C, x_in)
        if shape.dtype == "bf16":
            worst_ulps = max(worst_ulps, float((np.abs(gl[l] - ref).max(axis=1)
                                                / bf16_ulp(np.abs(ref).max(axis=1))).max()))
        assert_rows_close(gl[l], ref, shape.dtype, f"draft layer {l} given the GPU's input")
        x_in = gl[l]
    head = orc.lm_head(model, gl[L - 1])
    lg = np.asarray(logits, dtype=np.float64)
    ref_lg = head["logits"].astype(np.float64)
    if shape.dtype == "fp32":
        rel = np.abs(lg - ref_lg).max(axis=1) / np.abs(ref_lg).max(axis=1)
        assert rel.max() <= 1e-4, f"LM head logits relative error {rel.max():.3g}"
        err = float(rel.max())
    else:
        err = float(np.abs(lg - ref_lg).max())
        assert err <= 2e-2, f"LM head logits absolute error {err:.3g} given the GPU's final residual"
    tok = np.asarray(tokens)
    for j in np.flatnonzero(tok != head["tokens"]):
        assert head["gap"][j] < 1e-3, (f"row {j}: gpu token {tok[j]} vs oracle {head['tokens'][j]} "
                                       f"(oracle top-2 gap {head['gap'][j]:.3g}) given the GPU's final residual")
    return err, worst_ulps


def check_target_layers(orc, model, w, shape, cache, C, tokens, parent, layers, logits, argmax):
    """check_layers for the causal / tree target forward: layer l of the oracle
    (its tree mask when parent is given) runs on the GPU's input to that layer
    over `cache` (an oracle TargetCache holding the same keys before C, into
    which each layer's rows are written), and must land within 2 bf16 ulps of
    the GPU's output (fp32: 1e-4 relative); the oracle's LM head on the GPU's
    final residual bounds logits at 2e-2 (fp32: 1e-4 relative) with tokens
    exact except where its top-2 gap is below 1e-3.  Returns the largest logit
    difference, the worst per-layer ulps and the oracle's rows of every layer."""
    L, n, H = layers.shape[0], layers.shape[1], shape.hidden
    gl = layers.float().cpu().numpy().astype(np.float64).reshape(L, n, H)
    x_in = w["embed"][list(np.asarray(tokens))].double().numpy()
    worst = 0.0
    for l in range(L):
        ref = orc.target_layer(model, l, x_in, C, cache, parent)
        if shape.dtype == "bf16":
            worst = max(worst, float((np.abs(gl[l] - ref).max(axis=1) / bf16_ulp(np.abs(ref).max(axis=1))).max()))
        assert_rows_close(gl[l], ref, shape.dtype, f"target layer {l} given the GPU's input")
        x_in = gl[l]
    head = orc.lm_head(model, gl[L - 1])
    lg = np.asarray(logits, dtype=np.float64)
    ref_lg = head["logits"].astype(np.float64)
    if shape.dtype == "fp32":
        err = float((np.abs(lg - ref_lg).max(axis=1) / np.abs(ref_lg).max(axis=1)).max())
        assert err <= 1e-4, f"LM head logits relative error {err:.3g}"
    else:
        err = float(np.abs(lg - ref_lg).max())
        assert err <= 2e-2, f"LM head logits absolute error {err:.3g} given the GPU's final residual"
    am = np.asarray(argmax)
    for j in np.flatnonzero(am != head["tokens"]):
        assert head["gap"][j] < 1e-3, (f"row {j}: gpu token {am[j]} vs oracle {head['tokens'][j]} "
                                       f"(oracle top-2 gap {head['gap'][j]:.3g}) given the GPU's final residual")
    return err, worst
