"""Shared helpers of the GPU parity tests: device copies, tolerances, checks."""
import numpy as np
import torch

import dflash_inputs as di

# a bf16 shape small enough for the oracle in seconds that still spans several
# tiles, ragged K (FFN 1376 = 43 chunks of 32) and a vocab that is not a power of two
MID_BF16 = di.Shape("mid_bf16", "bf16", hidden=512, target_layers=12, draft_layers=2, n_q_heads=8,
                    n_kv_heads=2, head_dim=128, ffn=1376, vocab=4000, ctx=300, seed=21)
MID_BF16_D64 = MID_BF16.replace(name="mid_bf16_d64", n_q_heads=8, n_kv_heads=4, head_dim=64, seed=22)
MID_FP32_G5 = di.Shape("mid_fp32_g5", "fp32", hidden=320, target_layers=9, draft_layers=1, n_q_heads=10,
                       n_kv_heads=2, head_dim=64, ffn=688, vocab=1024, ctx=100, seed=23)

TIE_GAP = 1e-3


def dev(w):
    return {k: v.cuda() for k, v in w.items()}


def bf16_ulp(x):
    x = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(x)) - 7)


def assert_rows_close(got, ref, dtype, what=""):
    """fp32: per-row max|d| / max|ref| <= 1e-4.  bf16 intermediates: per-row
    max|d| <= 2 bf16 ulps of the row's max magnitude."""
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    err = np.abs(got - ref).max(axis=1)
    mx = np.abs(ref).max(axis=1)
    if dtype == "fp32":
        bad = err > 1e-4 * np.maximum(mx, 1e-30)
    else:
        bad = err > 2 * bf16_ulp(mx)
    assert not bad.any(), f"{what}: rows {np.flatnonzero(bad)[:8]} err {err[bad][:8]} rowmax {mx[bad][:8]}"


def assert_logits(got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if dtype == "fp32":
        rel = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
        assert rel.max() <= 1e-4, f"fp32 logits relative error {rel.max():.3g}"
    else:
        err = np.abs(got - ref).max()
        assert err <= 2e-2, f"bf16 logits absolute error {err:.3g}"


def assert_tokens(got, ref, gap):
    got, ref = np.asarray(got), np.asarray(ref)
    mism = np.flatnonzero(got != ref)
    for j in mism:
        assert gap[j] < TIE_GAP, f"token mismatch at row {j}: gpu {got[j]} oracle {ref[j]} gap {gap[j]}"
    return len(mism)
