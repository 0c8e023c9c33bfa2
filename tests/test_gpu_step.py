"""The device-resident step ([B] 技术内幕: draft, verify, keep the anchor and
the accepted drafts, inject the verified rows' context, draft again) with the
context length on the device, eagerly and captured in a HIP graph.

* A graph-replayed step loop equals the same loop run eagerly, bit for bit:
  tokens, accept results, the device length and every KV page position.
* The draft with the device-resident length equals the host-length draft.
* An injection past the capacity writes nothing and raises the error word.
"""
import numpy as np
import pytest
import torch

import dflash_inputs as di
from tests.gpu_helpers import MID_BF16, dev

pytestmark = pytest.mark.gpu

S = MID_BF16
C0 = 300
STEPS = 8


@pytest.fixture(scope="module")
def dl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_diffusion_drafter_context_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def w():
    return dev(di.draft_weights(S))


def prefilled(dl, w, page_seed=5):
    ctx = dl.DFlash(S, w, max_ctx=C0 + 16 * (STEPS + 2), max_rows=C0, page_seed=page_seed)
    sel = dl.feature_layers(S.target_layers)
    hid = [di.target_hidden(S, l, C0).cuda() if l in sel else None for l in range(S.target_layers)]
    ctx.inject_kv(ctx.fuse_context(hid), 0)
    return ctx


class Step:
    """Static buffers of one device-resident step (what a graph captures)."""

    def __init__(self, dl, ctx):
        self.ctx = ctx
        B = S.block
        sel = dl.feature_layers(S.target_layers)
        self.hid = [torch.empty(16, S.hidden, dtype=S.torch_dtype, device="cuda") if l in sel else None
                    for l in range(S.target_layers)]
        self.fused = torch.empty(16, S.hidden, dtype=S.torch_dtype, device="cuda")
        self.anchor = torch.tensor([7], dtype=torch.int32, device="cuda")
        self.tok = torch.empty(B, dtype=torch.int32, device="cuda")
        self.g = torch.empty(B, dtype=torch.int32, device="cuda")
        self.res = torch.empty(2, dtype=torch.int32, device="cuda")
        # synthetic target: agrees with the first drafts, then breaks (k varies with the drafts)
        self.sel_idx = torch.tensor(list(range(1, B)) + [0], dtype=torch.int64, device="cuda")
        self.add = torch.tensor([0, 0, 0] + [j % 3 for j in range(3, B - 1)] + [11], dtype=torch.int32, device="cuda")

    def load(self, i):  # the verified rows' target features of step i (outside the graph)
        for l, t in enumerate(self.hid):
            if t is not None:
                t.copy_(di.target_hidden(S, l, 16, tag=f"step{i}").cuda())

    def __call__(self):
        c = self.ctx
        c.draft_block(self.anchor, tokens=self.tok)
        torch.index_select(self.tok, 0, self.sel_idx, out=self.g)
        self.g.add_(self.add).remainder_(S.vocab)
        c.verify_accept(self.tok, self.g, out=self.res)
        c.fuse_context(self.hid, out=self.fused)
        c.inject_kv(self.fused, -1)
        c.keep_accepted(self.res)
        self.anchor.copy_(self.res[1:2])


def run(dl, w, graph):
    ctx = prefilled(dl, w)
    ctx.enable_device_length()
    st = Step(dl, ctx)
    g = None
    if graph:
        warm = prefilled(dl, w, page_seed=9)  # load every kernel before capture
        warm.enable_device_length()
        ws = Step(dl, warm)
        ws.load(0)
        ws()
        torch.cuda.synchronize()
        st.load(0)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            st()
        torch.cuda.synchronize()
    toks, ress, lens = [], [], []
    for i in range(STEPS):
        st.load(i)
        if graph:
            g.replay()
        else:
            st()
        lens.append(ctx.read_device_length().clone())
        toks.append(st.tok.clone())
        ress.append(st.res.clone())
    torch.cuda.synchronize()
    # every position an injection wrote: step i writes 16 rows at the length
    # after step i - 1 (lengths only grow), so the last step's rows end here
    written = int(lens[-2][0]) + 16
    k, v = ctx.read_kv(0, written)
    torch.cuda.synchronize()
    return ([t.cpu() for t in toks], [r.cpu() for r in ress], [int(x[0]) for x in lens], k.cpu(), v.cpu())


def test_graph_replay_equals_eager_steps(dl, w):
    eager = run(dl, w, graph=False)
    graph = run(dl, w, graph=True)
    ks = [int(r[0]) for r in eager[1]]
    print(f"[step] accepted k per step {ks}; lengths {eager[2]}", flush=True)
    assert len(set(ks)) > 1 or ks[0] > 0  # the synthetic target lets some drafts through
    assert eager[2][-1] == C0 + sum(k + 1 for k in ks)
    for i in range(STEPS):
        assert torch.equal(eager[0][i], graph[0][i]), f"step {i} tokens"
        assert torch.equal(eager[1][i], graph[1][i]), f"step {i} accept result"
    assert eager[2] == graph[2]
    assert torch.equal(eager[3], graph[3]) and torch.equal(eager[4], graph[4])


def test_device_length_draft_equals_host_length_draft(dl, w):
    ctx = prefilled(dl, w)
    a = torch.tensor([7], dtype=torch.int32, device="cuda")
    t_h, l_h = ctx.draft_block(a, want_logits=True)
    t_h, l_h = t_h.clone(), l_h.clone()
    ctx.enable_device_length()
    assert ctx.length == -1
    # with C = 300 and max_ctx = 460 both attention plans use 192-key splits
    t_d, l_d = ctx.draft_block(a, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(t_h, t_d) and torch.equal(l_h, l_d)
    with pytest.raises(dl.DFlashError) as e:
        ctx.rollback(10)
    assert e.value.status == -5


def test_device_length_capacity_guard(dl, w):
    ctx = prefilled(dl, w)
    ctx.enable_device_length()
    cap = C0 + 16 * (STEPS + 2)
    ctx.set_length_async(cap - 8)
    before = ctx.read_kv(cap - 16, 16)
    f = di.fused_context(S, 16, tag="over").cuda()
    ctx.inject_kv(f, -1)  # 16 rows at cap - 8 do not fit: nothing written
    lw = ctx.read_device_length()
    after = ctx.read_kv(cap - 16, 16)
    torch.cuda.synchronize()
    assert lw.cpu().tolist() == [cap - 8, 1]
    # never-written pool memory may hold NaN patterns: compare the bits
    assert all(torch.equal(b.view(torch.int16), a.view(torch.int16)) for b, a in zip(before, after))
    res = torch.tensor([15, 3], dtype=torch.int32, device="cuda")
    ctx.keep_accepted(res)  # clamped to the capacity
    assert int(ctx.read_device_length()[0]) == cap
