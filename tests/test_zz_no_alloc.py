"""The allocation-free 16-row fusion (dflash_fuse_context_static) against the
workspace-scratch entry point (dflash_fuse_context) through the C ABI: two
calls in a row, the second with fewer rows, each bit-identical to the existing
entry point (same kernels, same summation order) and within the bf16 bar of
the oracle."""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from tests.gpu_helpers import MID_BF16, assert_rows_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_drafter_context_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("shape", [MID_BF16, di.SHAPES["qwen3_8b_4k"]])
def test_static_fuse_equals_workspace_fuse(dl, orc, shape):
    s = shape
    w = di.draft_weights(s, need_draft=False, need_lm=False, gains="random")
    ctx = dl.DFlash(s, dev(w), max_ctx=64, max_rows=16)
    sel = orc.feature_layers(s.target_layers)
    for call, M in enumerate((16, 5)):
        hid = {l: di.target_hidden(s, l, M, tag=f"static{call}") for l in sel}
        layers = [hid[l].cuda() if l in hid else None for l in range(s.target_layers)]
        ref = ctx.fuse_context(layers)
        out = torch.full((M, s.hidden), float("nan"), dtype=s.torch_dtype, device="cuda")
        ctx.fuse_context_static(layers, out)
        torch.cuda.synchronize()
        print(f"[no-alloc] {s.name} call {call}: M={M}", flush=True)
        assert torch.equal(out, ref), f"call {call}: static scratch result differs from the workspace result"
        rf = orc.fuse_rows(orc.Model(s, w), [hid[l] for l in sel], range(M))
        assert_rows_close(out.float().cpu().numpy(), rf, s.dtype, f"static fuse call {call}")


def test_static_fuse_rejects_more_than_16_rows(dl):
    s = MID_BF16
    ctx = dl.DFlash(s, dev(di.draft_weights(s, need_draft=False, need_lm=False)), max_ctx=64, max_rows=32)
    layers = [torch.zeros(17, s.hidden, dtype=s.torch_dtype, device="cuda")] * s.target_layers
    out = torch.empty(17, s.hidden, dtype=s.torch_dtype, device="cuda")
    with pytest.raises(dl.DFlashError) as e:
        ctx.fuse_context_static(layers, out)
    assert e.value.status == -2
    torch.cuda.synchronize()
