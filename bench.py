#!/usr/bin/env python3
"""Throughput of the DFlash draft step on one MI355X.

One step = one pass of the whole draft-side hot path over one block:
  draft_block (embed, every draft layer, LM head + argmax)
  -> verify_accept against a synthetic target argmax
  -> fuse_context of the 16 verified rows' target features (5 layers, Linear + RMSNorm)
  -> inject_kv of those 16 rows into every layer's paged draft KV cache
  -> keep C + k + 1 positions (then back to C so every step sees the same context)
with the context length held on the device, so no step reads anything back.
Inputs are seeded synthetic tensors of the Qwen3-8B-shaped draft (hidden 4096,
36 target layers, 5 draft layers, 32/8 heads x 128, FFN 12288, vocab 151936,
bf16) with a 4096-token injected context, already resident in HBM.

Prints progress to stderr and ONE JSON line to stdout.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DFlash 16-token draft blocks/s + drafted tok/s at 8B shape, 4K/36K ctx; % HBM peak"
HBM_PEAK = 8.0e12       # MI355X HBM3E, bytes/s
BF16_PEAK = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(s, C):
    """Algorithmic HBM bytes of one draft block and of one full step."""
    e = s.elem_bytes
    H, F, V, nq, nkv, d, L = s.hidden, s.ffn, s.vocab, s.n_q_heads, s.n_kv_heads, s.head_dim, s.draft_layers
    layer_w = (H * nq * d + 2 * H * nkv * d + nq * d * H + 3 * H * F) * e
    lm = V * H * e
    kv = L * C * 2 * nkv * d * e
    draft = L * layer_w + lm + kv + 2 * H * e
    fuse16 = 5 * H * H * e + 16 * 5 * H * e + 16 * H * e
    inject16 = L * 2 * nkv * d * H * e + 16 * H * e + L * 16 * 2 * nkv * d * e
    return {"draft": draft, "lm_head": lm + 16 * H * e, "layer_weights": L * layer_w, "kv": kv,
            "fuse16": fuse16, "inject16": inject16, "step": draft + fuse16 + inject16}


def cpu_identity():
    """Model name, sockets, physical cores and logical CPUs of the host (from
    lscpu, else /proc/cpuinfo); fields that cannot be read are left out."""
    import subprocess
    info = {}
    try:
        txt = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        kv = dict(l.split(":", 1) for l in txt.splitlines() if ":" in l)
        kv = {a.strip(): b.strip() for a, b in kv.items()}
        if "Model name" in kv:
            info["cpu_model"] = kv["Model name"]
        if "Socket(s)" in kv:
            info["sockets"] = int(kv["Socket(s)"])
            if "Core(s) per socket" in kv:
                info["physical_cores"] = int(kv["Core(s) per socket"]) * info["sockets"]
        if "CPU(s)" in kv:
            info["logical_cpus"] = int(kv["CPU(s)"])
    except Exception:
        pass
    if "cpu_model" not in info and os.path.exists("/proc/cpuinfo"):
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except Exception:
        pass
    return info


def profiled_traffic(workload):
    """HBM bytes per draft pass and per LM-head launch from the committed
    counter passes ({"draft_pass": ..., "lm_head": ...}), or None when they
    were taken on another workload or on different kernel sources."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "draft_pass_qwen3_8b_4k_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("workload") != workload:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return {"draft_pass": rec["traffic_bytes_per_pass"], "lm_head": rec["lm_head_traffic_bytes_per_launch"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_8b_4k")
    ap.add_argument("--long-ctx", type=int, default=36864, help="second context length measured (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-side fusion/injection GEMM timing")
    ap.add_argument("--no-27b", action="store_true", help="skip the 27B-class draft pass at 36K context")
    ap.add_argument("--no-toy", action="store_true", help="skip the toy end-to-end speculative loop")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the target verify pass at the Qwen3-8B target shape (36 layers)")
    ap.add_argument("--kv-rotate", type=int, default=4,
                    help="independent contexts (KV caches, anchors) the 4K steps rotate through, so the 256 MB "
                         "Infinity Cache cannot hold one context's KV between its steps")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="after timing, copy this many GiB device-to-device (plain copy kernel for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (each GPU would run its own "
              "sequences' draft steps independently). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_diffusion_drafter_context_amd as dl
    import dflash_inputs as di

    torch.cuda.set_device(0)
    s = di.SHAPES[args.workload]
    C = s.ctx
    t0 = time.time()
    w_cpu = di.draft_weights(s)
    w = {k: v.cuda() for k, v in w_cpu.items()}
    torch.cuda.synchronize()
    log(f"[bench] weights {sum(v.numel() for v in w.values()) * s.elem_bytes / 1e9:.2f} GB ready in {time.time() - t0:.1f}s")

    sel = dl.feature_layers(s.target_layers)

    def prepare(ctx_len, tag):
        ctx = dl.DFlash(s, w, max_ctx=ctx_len + 64, max_rows=max(ctx_len, 16))
        chunk = 8192
        for r0 in range(0, ctx_len, chunk):
            M = min(chunk, ctx_len - r0)
            hid = {l: di.normal((M, s.hidden), s.seed, f"hidden.{tag}.{l}.{r0}", 1.0, s.torch_dtype).cuda()
                   for l in sel}
            fused = ctx.fuse_context([hid.get(l) for l in range(s.target_layers)])
            ctx.inject_kv(fused, r0)
        torch.cuda.synchronize()
        return ctx

    step_hidden = [di.target_hidden(s, l, 16, tag="step").cuda() if l in sel else None
                   for l in range(s.target_layers)]
    u, r, last = di.target_coins(s)
    # the synthetic target argmax of a block, as two device ops per step:
    # g[j] = (d[j+1] + r'[j]) mod V for j < B-1, with r'[j] = 0 where the
    # target agrees (u[j+1] < p) and r[j+1] otherwise; g[B-1] = last is set
    # once when the buffer is made
    B = s.block
    add = torch.tensor([0 if float(u[j]) < di.SYNTH_AGREE_P else int(r[j]) for j in range(1, B)],
                       dtype=torch.int32, device="cuda")

    def synthetic_target(tokens, g_buf):
        torch.add(tokens[1:B], add, out=g_buf[:B - 1])
        g_buf[:B - 1].remainder_(s.vocab)
        return g_buf

    def make_step(ctx, C0):
        """One device-resident step on ctx (its length lives on the device):
        draft -> synthetic target -> accept -> fuse the 16 verified rows ->
        inject them at the length -> keep the anchor and the k accepted rows ->
        back to C0 (every step sees the same context) -> the bonus token is the
        next anchor, read in place from the accept result {k, bonus}.  No host
        read anywhere, so steps are enqueued back to back and the step can be
        captured in a HIP graph (static buffers)."""
        tok = torch.empty(B, dtype=torch.int32, device="cuda")
        g = torch.full((B,), last, dtype=torch.int32, device="cuda")
        res = torch.tensor([0, di.anchor_token(s)], dtype=torch.int32, device="cuda")
        anchor = res[1:2]  # the first step's anchor, then each step's bonus token
        fused = torch.empty(16, s.hidden, dtype=s.torch_dtype, device="cuda")

        def step():
            ctx.draft_block(anchor, tokens=tok)
            synthetic_target(tok, g)
            ctx.verify_accept(tok, g, out=res)
            ctx.fuse_context(step_hidden, out=fused)
            ctx.inject_kv(fused, -1)
            ctx.keep_accepted(res)
            ctx.set_length_async(C0)

        step.res = res
        return step

    def timed(ctxs, C0, steps, warmup, trace_cls=None):
        """Eager device-resident steps rotating through the contexts in ctxs
        (a list, or one context); no host synchronisation inside the loop."""
        if not isinstance(ctxs, list):
            ctxs = [ctxs]
        made = [make_step(c, C0) for c in ctxs]
        for i in range(warmup):
            made[i % len(made)]()
        torch.cuda.synchronize()
        if trace_cls is not None:
            for c in ctxs:
                st = dl.lib().dflash_trace_enable(c.h, trace_cls, steps * 8)
                assert st == 0
        t = time.perf_counter()
        for i in range(steps):
            made[i % len(made)]()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        trace = None
        if trace_cls is not None:
            import ctypes as C_
            tot_ms, tot_n = 0.0, 0
            for c in ctxs:
                ms, n = C_.c_double(), C_.c_int32()
                dl.lib().dflash_trace_read(c.h, C_.byref(ms), C_.byref(n))
                tot_ms += ms.value
                tot_n += n.value
                dl.lib().dflash_trace_enable(c.h, 0, 0)
            trace = (tot_ms, tot_n)
        return dt, trace

    def accept_stats(ctxs, C0, n=32):
        """Mean accepted k over n steps (host reads after each step; untimed)."""
        made = [make_step(c, C0) for c in ctxs]
        ks = []
        for i in range(n):
            m = made[i % len(made)]
            m()
            ks.append(int(m.res[0].item()))
        return float(np.mean(ks))

    def graph_timed(ctxs, C0, steps, warmup):
        """The same step captured once per context in a HIP graph and replayed."""
        made = [make_step(c, C0) for c in ctxs]
        for m in made:  # every kernel loaded before capture
            m()
        torch.cuda.synchronize()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        graphs = []
        for m in made:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=cs):
                m()
            graphs.append(gr)
        torch.cuda.synchronize()
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t

    # ---- headline: context C, LM head traced live over the timed region
    t0 = time.time()
    ctxs = [prepare(C, f"ctx{i}" if i else "ctx") for i in range(max(args.kv_rotate, 1))]
    for c_ in ctxs:
        c_.enable_device_length()
    ctx = ctxs[0]
    log(f"[bench] {len(ctxs)} contexts, prefill fuse+inject of {C} rows each, done in {time.time() - t0:.1f}s")
    # the whole draft call of every step is bracketed by HIP events on the
    # library's stream over the timed region
    dt, tr = timed(ctxs, C, args.steps, args.warmup, trace_cls=7)
    ab = alg_bytes(s, C)
    bps = args.steps / dt
    dr_ms = tr[0] / max(tr[1], 1)
    dr_ach = ab["draft"] / (dr_ms * 1e-3)
    log(f"[bench] {args.steps} steps in {dt:.3f}s: {bps:.1f} blocks/s; draft pass {dr_ms * 1e3:.1f} us/call")
    # the pass's dominant kernel, the LM head (+ argmax), in a short traced run of the same steps
    _, tr_lm = timed(ctxs, C, 50, 5, trace_cls=1)
    lm_ms = tr_lm[0] / max(tr_lm[1], 1)
    lm_ach = ab["lm_head"] / (lm_ms * 1e-3)
    traffic = profiled_traffic(args.workload)

    out = {
        "metric": METRIC,
        "value": round(bps, 2),
        "unit": "draft blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) target features, N(0,0.02) random-init weights)",
        "config": {"workload": args.workload, "hidden": s.hidden, "target_layers": s.target_layers,
                   "draft_layers": s.draft_layers, "heads": f"{s.n_q_heads}/{s.n_kv_heads}x{s.head_dim}",
                   "ffn": s.ffn, "vocab": s.vocab, "ctx": C, "block": s.block,
                   "step": "device-resident: draft_block+synthetic target+verify_accept+fuse(16)+inject(16)"
                           "+keep_accepted+rewind, no host read",
                   "kv_contexts_rotated": len(ctxs)},
        "drafted_tok_per_s": round(15 * bps, 1),
        "hbm_frac_step": round(ab["step"] * bps / HBM_PEAK, 4),
        "alg_bytes_per_step": ab["step"],
        "mean_accept_k": None,
        "roofline": {"bound": "hbm",
                     "kernel": "the draft pass: embed, 5 x (QKV+RoPE, split-KV attention, merge, O+residual, "
                               "gate/up+SwiGLU, down+residual), LM head+argmax (32 launches)",
                     "achieved": round(dr_ach / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(dr_ach / HBM_PEAK, 4), "traffic": traffic["draft_pass"] if traffic else None,
                     "alg_bytes_per_launch": ab["draft"], "avg_launch_us": round(dr_ms * 1e3, 2),
                     "dominant_kernel": {"kernel": "skinny_wg_kernel<OpLMHeadWG> (LM head + argmax)",
                                         "achieved": round(lm_ach / 1e9, 1), "frac": round(lm_ach / HBM_PEAK, 4),
                                         "traffic": traffic["lm_head"] if traffic else None,
                                         "alg_bytes_per_launch": ab["lm_head"],
                                         "avg_launch_us": round(lm_ms * 1e3, 2)}},
    }

    if args.copy_calibration_gib > 0:
        n = int(args.copy_calibration_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n
        del src, dst

    def draft_percentiles(ctxs_, C0, n=200):
        """p10 / p50 / p90 of single draft-pass durations (HIP events), in us;
        steps rotate through the contexts as in the timed region."""
        import ctypes as C_
        if not isinstance(ctxs_, list):
            ctxs_ = [ctxs_]
        made = [make_step(c, C0) for c in ctxs_]
        for c in ctxs_:
            assert dl.lib().dflash_trace_enable(c.h, 7, n) == 0
        for i in range(n):
            made[i % len(made)]()
        v = []
        for c in ctxs_:
            buf = (C_.c_float * n)()
            cnt = C_.c_int32()
            assert dl.lib().dflash_trace_read_each(c.h, buf, n, C_.byref(cnt)) == 0
            dl.lib().dflash_trace_enable(c.h, 0, 0)
            v.extend(buf[:cnt.value])
        v = np.array(v, dtype=np.float64) * 1e3
        return [round(float(np.percentile(v, q)), 1) for q in (10, 50, 90)]

    out["draft_pass_us_p10_p50_p90"] = draft_percentiles(ctxs, C)
    p50 = out["draft_pass_us_p10_p50_p90"][1]
    # the draft call alone: blocks/s = 1 / median pass; 15 drafted tokens or 16 block positions per block
    out["draft_pass_blocks_per_s"] = round(1e6 / p50, 1)
    out["draft_pass_drafted_tok_per_s"] = round(15e6 / p50, 1)
    out["draft_pass_block_positions_per_s"] = round(16e6 / p50, 1)
    out["draft_pass_hbm_frac_p50"] = round(alg_bytes(s, C)["draft"] / (p50 * 1e-6) / HBM_PEAK, 4)
    log(f"[bench] draft pass p10/p50/p90 {out['draft_pass_us_p10_p50_p90']} us")
    out["mean_accept_k"] = round(accept_stats(ctxs, C), 4)
    # the same step captured in a HIP graph per context and replayed
    dtg = graph_timed(ctxs, C, args.steps, args.warmup)
    out["graph_step"] = {"blocks_per_s": round(args.steps / dtg, 2), "us_per_step": round(dtg / args.steps * 1e6, 1),
                         "hbm_frac_step": round(ab["step"] * args.steps / dtg / HBM_PEAK, 4)}
    log(f"[bench] graph-replayed step: {json.dumps(out['graph_step'])}")

    # ---- the chip's practical streaming-read rate, next to the 8 TB/s spec
    probe_buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    probe_sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        probe_bytes = dl.hbm_read_probe(probe_buf, probe_sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dl.hbm_read_probe(probe_buf, probe_sink)
    e1.record()
    torch.cuda.synchronize()
    probe_gbps = probe_bytes / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    out["hbm_read_ceiling"] = {"GBps": round(probe_gbps, 1), "frac_of_peak": round(probe_gbps * 1e9 / HBM_PEAK, 4),
                               "bytes": probe_bytes, "lm_head_frac_of_ceiling": round(lm_ach / 1e9 / probe_gbps, 4),
                               "kernel": "read_probe_kernel: 16-byte non-temporal loads, 4 waves per CU, one contiguous "
                                         "range per wave, 16 KB in flight per wave"}
    log(f"[bench] streaming-read ceiling {json.dumps(out['hbm_read_ceiling'])}")
    del probe_buf, probe_sink

    # ---- per-kernel-class breakdown (separate short traced runs, not the timed region)
    if not args.no_breakdown:
        per_layer = {"qkv": (4, (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim * s.hidden * s.elem_bytes),
                     "attn": (6, ab["kv"] // s.draft_layers),
                     "o_proj": (5, s.n_q_heads * s.head_dim * s.hidden * s.elem_bytes),
                     "gate_up": (2, 2 * s.ffn * s.hidden * s.elem_bytes),
                     "down": (3, s.ffn * s.hidden * s.elem_bytes),
                     "lm_head": (1, ab["lm_head"]),
                     "draft": (7, ab["draft"]),
                     "fuse16": (8, ab["fuse16"]),
                     "inject16": (9, ab["inject16"])}
        bd = {}
        for name, (cls, byts) in per_layer.items():
            _, tr2 = timed(ctxs, C, 32, 4, trace_cls=cls)
            us = tr2[0] / max(tr2[1], 1) * 1e3
            bd[name] = {"us": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1)}
        out["breakdown_ctx"] = bd
        log(f"[bench] breakdown {json.dumps(bd)}")

    # ---- long context
    if args.long_ctx:
        del ctx
        ctxs.clear()
        torch.cuda.empty_cache()
        t0 = time.time()
        ctx2 = prepare(args.long_ctx, "long")
        ctx2.enable_device_length()
        log(f"[bench] prefill of {args.long_ctx} rows done in {time.time() - t0:.1f}s")
        dt2, tr2 = timed(ctx2, args.long_ctx, args.steps, args.warmup, trace_cls=7)
        ab2 = alg_bytes(s, args.long_ctx)
        bps2 = args.steps / dt2
        dr_us = tr2[0] / max(tr2[1], 1) * 1e3
        pct = draft_percentiles(ctx2, args.long_ctx)
        out["long_ctx"] = {"ctx": args.long_ctx, "blocks_per_s": round(bps2, 2),
                           "draft_pass_us_p10_p50_p90": pct,
                           "draft_pass_blocks_per_s": round(1e6 / pct[1], 1),
                           "draft_pass_hbm_frac_p50": round(ab2["draft"] / (pct[1] * 1e-6) / HBM_PEAK, 4),
                           "drafted_tok_per_s": round(15 * bps2, 1),
                           "hbm_frac_step": round(ab2["step"] * bps2 / HBM_PEAK, 4),
                           "draft_pass_us": round(dr_us, 1),
                           "draft_pass_hbm_frac": round(ab2["draft"] / (dr_us * 1e-6) / HBM_PEAK, 4)}
        log(f"[bench] long ctx: {json.dumps(out['long_ctx'])}")
        del ctx2

    # ---- 27B-class draft pass at 36864 tokens of injected context (the draft call alone)
    if not args.no_27b:
        if "ctx" in locals():
            del ctx
        ctxs.clear()
        torch.cuda.empty_cache()
        import ctypes as C_
        s3 = di.SHAPES["dense27b_36k"]
        t0 = time.time()
        w3_cpu = di.draft_weights(s3)
        w3 = {k: v.cuda() for k, v in w3_cpu.items()}
        ctx3 = dl.DFlash(s3, w3, max_ctx=s3.ctx + 64)
        k3, v3 = di.context_kv(s3, s3.ctx)
        ctx3.load_kv(k3.cuda(), v3.cuda())
        if args.no_cpu_baseline:
            del w3_cpu, k3, v3
        a3 = torch.tensor([di.anchor_token(s3)], dtype=torch.int32, device="cuda")
        t3 = torch.empty(s3.block, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] 27B-class context of {s3.ctx} tokens ready in {time.time() - t0:.1f}s")
        for _ in range(args.warmup):
            ctx3.draft_block(a3, tokens=t3)
        torch.cuda.synchronize()
        n3 = args.steps
        assert dl.lib().dflash_trace_enable(ctx3.h, 7, n3) == 0
        for _ in range(n3):
            ctx3.draft_block(a3, tokens=t3)
        buf = (C_.c_float * n3)()
        cnt = C_.c_int32()
        assert dl.lib().dflash_trace_read_each(ctx3.h, buf, n3, C_.byref(cnt)) == 0
        dl.lib().dflash_trace_enable(ctx3.h, 0, 0)
        v = np.array(buf[:cnt.value], dtype=np.float64) * 1e3
        pct3 = [round(float(np.percentile(v, q)), 1) for q in (10, 50, 90)]
        ab3 = alg_bytes(s3, s3.ctx)["draft"]
        out["dense27b_36k"] = {"workload": "dense27b_36k", "hidden": s3.hidden, "ffn": s3.ffn, "heads": "40/8x128",
                               "ctx": s3.ctx, "draft_pass_us_p10_p50_p90": pct3,
                               "draft_pass_blocks_per_s": round(1e6 / pct3[1], 1),
                               "draft_pass_drafted_tok_per_s": round(15e6 / pct3[1], 1),
                               "alg_bytes_per_pass": ab3,
                               "draft_pass_hbm_frac_p50": round(ab3 / (pct3[1] * 1e-6) / HBM_PEAK, 4)}
        log(f"[bench] 27B-class @36K: {json.dumps(out['dense27b_36k'])}")
        del ctx3, w3
        torch.cuda.empty_cache()

    # ---- the verify side at the Qwen3-8B target shape: a causal forward of 16
    # rows through 36 layers over a 4096-token paged target cache (random
    # device-side weights and cache: an HBM-bound pass, values do not matter)
    if not args.no_verify:
        if "ctx" in locals():
            del ctx
        ctxs.clear()
        torch.cuda.empty_cache()
        import ctypes as C_
        sv = s.replace(name="qwen3_8b_target", draft_layers=36)
        Lv, Cv = sv.draft_layers, s.ctx
        gen = torch.Generator(device="cuda").manual_seed(sv.seed)
        t0 = time.time()

        def rnd(*shape, std=sv.w_std):
            return (torch.randn(*shape, generator=gen, device="cuda") * std).to(torch.bfloat16)
        H_, nq_, nkv_, d_, F_ = sv.hidden, sv.n_q_heads, sv.n_kv_heads, sv.head_dim, sv.ffn
        wv = {"final_norm": torch.ones(H_, dtype=torch.bfloat16, device="cuda"),
              "embed": rnd(sv.vocab, H_), "lm_head": rnd(sv.vocab, H_)}
        for l in range(Lv):
            wv[f"attn_norm.{l}"] = torch.ones(H_, dtype=torch.bfloat16, device="cuda")
            wv[f"mlp_norm.{l}"] = torch.ones(H_, dtype=torch.bfloat16, device="cuda")
            wv[f"wq.{l}"], wv[f"wk.{l}"], wv[f"wv.{l}"] = rnd(nq_ * d_, H_), rnd(nkv_ * d_, H_), rnd(nkv_ * d_, H_)
            wv[f"wo.{l}"], wv[f"wg.{l}"], wv[f"wu.{l}"], wv[f"wd.{l}"] = rnd(H_, nq_ * d_), rnd(F_, H_), rnd(F_, H_), rnd(H_, F_)
        ctxv = dl.DFlash(sv, wv, max_ctx=Cv + 64)
        kv_std = sv.w_std * float(np.sqrt(H_))
        ctxv.load_kv(rnd(Lv, Cv, nkv_, d_, std=kv_std), rnd(Lv, Cv, nkv_, d_, std=kv_std))
        vt = torch.randint(0, sv.vocab, (16,), generator=gen, device="cuda", dtype=torch.int64).to(torch.int32)
        va = torch.empty(16, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] 8B-shape target (36 layers) with {Cv} cached tokens ready in {time.time() - t0:.1f}s")
        for _ in range(args.warmup):
            ctxv.target_forward(vt, argmax=va)
            ctxv.rollback(Cv)
        torch.cuda.synchronize()
        nv = max(20, args.steps // 4)
        assert dl.lib().dflash_trace_enable(ctxv.h, 10, nv) == 0
        for _ in range(nv):
            ctxv.target_forward(vt, argmax=va)
            ctxv.rollback(Cv)
        buf = (C_.c_float * nv)()
        cnt = C_.c_int32()
        assert dl.lib().dflash_trace_read_each(ctxv.h, buf, nv, C_.byref(cnt)) == 0
        dl.lib().dflash_trace_enable(ctxv.h, 0, 0)
        vus = np.array(buf[:cnt.value], dtype=np.float64) * 1e3
        layer_w = (H_ * nq_ * d_ + 2 * H_ * nkv_ * d_ + nq_ * d_ * H_ + 3 * H_ * F_) * 2
        vbytes = Lv * layer_w + sv.vocab * H_ * 2 + Lv * Cv * 2 * nkv_ * d_ * 2 + Lv * 16 * 2 * nkv_ * d_ * 2
        pv = [round(float(np.percentile(vus, q)), 1) for q in (10, 50, 90)]
        out["target_verify"] = {"workload": "qwen3_8b target, 36 layers, 16 rows over 4096 cached tokens",
                                "us_p10_p50_p90": pv, "alg_bytes_per_pass": vbytes,
                                "hbm_frac_p50": round(vbytes / (pv[1] * 1e-6) / HBM_PEAK, 4),
                                "verified_rows_per_s": round(16e6 / pv[1], 1)}
        log(f"[bench] target verify: {json.dumps(out['target_verify'])}")

        # tree verification (DDTree) on the same target: top-4 candidates of 15
        # drafted positions (seeded stand-in logits at the 8B vocabulary), the
        # best-first tree of 15 nodes, its tree-masked verify pass, acceptance
        # and the compaction of the accepted rows
        lgt = torch.randn(15, sv.vocab, generator=gen, device="cuda") * 3.0
        res = torch.empty(17, dtype=torch.int32, device="cuda")

        def tree_step():
            ids, lp = ctxv.draft_topk(lgt, 4)
            tt, tp = ctxv.build_tree(vt[:1], ids, lp, 15)
            ctxv.target_forward(tt, argmax=va, parent=tp)
            ctxv.tree_accept(tt, tp, va, out=res)
            ctxv.tree_commit(Cv, 16, res)
            ctxv.rollback(Cv)
        for _ in range(args.warmup):
            tree_step()
        torch.cuda.synchronize()
        per_cls = {}
        for cls, n_per in ((10, 1), (11, 4)):
            assert dl.lib().dflash_trace_enable(ctxv.h, cls, nv * n_per) == 0
            for _ in range(nv):
                tree_step()
            buf = (C_.c_float * (nv * n_per))()
            assert dl.lib().dflash_trace_read_each(ctxv.h, buf, nv * n_per, C_.byref(cnt)) == 0
            dl.lib().dflash_trace_enable(ctxv.h, 0, 0)
            per_cls[cls] = np.array(buf[:cnt.value], dtype=np.float64).reshape(nv, n_per) * 1e3
        helpers = np.median(per_cls[11], axis=0)
        tv = float(np.median(per_cls[10]))
        out["ddtree"] = {"workload": "qwen3_8b target, tree of 16 nodes (top-4 per depth, 15 depths) over 4096 cached "
                                     "tokens, vocab 151936",
                         "topk_us": round(float(helpers[0]), 1), "build_us": round(float(helpers[1]), 1),
                         "verify_tree_us_p50": round(tv, 1), "accept_us": round(float(helpers[2]), 1),
                         "commit_us": round(float(helpers[3]), 1),
                         "overhead_vs_chain_verify_us": round(float(helpers.sum()) + tv - pv[1], 1)}
        log(f"[bench] ddtree: {json.dumps(out['ddtree'])}")

        # the same with a budget of 22 nodes (the pages' larger budget): 23 rows,
        # verified in one 23-row tree pass (two 16-row passes where the kernels
        # cannot take 32 rows; the trace then holds two records per step)
        va32 = torch.empty(32, dtype=torch.int32, device="cuda")

        def tree22_step():
            ids, lp = ctxv.draft_topk(lgt, 4)
            tt, tp = ctxv.build_tree(vt[:1], ids, lp, 22)
            ctxv.target_forward(tt, argmax=va32[:23], parent=tp)
            ctxv.tree_accept(tt, tp, va32[:23], out=res)
            ctxv.tree_commit(Cv, 23, res)
            ctxv.rollback(Cv)
        for _ in range(args.warmup):
            tree22_step()
        torch.cuda.synchronize()
        assert dl.lib().dflash_trace_enable(ctxv.h, 10, 2 * nv) == 0
        for _ in range(nv):
            tree22_step()
        buf = (C_.c_float * (2 * nv))()
        assert dl.lib().dflash_trace_read_each(ctxv.h, buf, 2 * nv, C_.byref(cnt)) == 0
        dl.lib().dflash_trace_enable(ctxv.h, 0, 0)
        passes = cnt.value // nv
        t22 = np.array(buf[:passes * nv], dtype=np.float64).reshape(nv, passes).sum(axis=1) * 1e3
        out["ddtree22"] = {"workload": "as ddtree with a tree of 23 nodes (budget 22)",
                           "passes": int(passes),
                           "verify_tree_us_p50": round(float(np.median(t22)), 1),
                           "vs_chain_verify": round(float(np.median(t22)) / pv[1], 3)}
        log(f"[bench] ddtree22: {json.dumps(out['ddtree22'])}")

        # non-greedy verification at the 8B vocabulary (T = 1): Gumbel-max draws
        # of the 15 drafted positions from seeded stand-in draft logits, then the
        # speculative sampling rule against target logits near the draft's
        lgd = torch.randn(16, sv.vocab, generator=gen, device="cuda") * 3.0
        lgv = torch.roll(lgd, -1, 0) + torch.randn(16, sv.vocab, generator=gen, device="cuda")
        dsm = torch.zeros(16, dtype=torch.int32, device="cuda")
        rsm = torch.empty(nv, 2, dtype=torch.int32, device="cuda")

        def sample_step(i, r):
            ctxv.sample_tokens(lgd[1:], 1.0, i, tokens=dsm[1:])
            ctxv.verify_sample(dsm, lgd, lgv, 1.0, i, out=r)
        for i in range(args.warmup):
            sample_step(i, rsm[0])
        torch.cuda.synchronize()
        assert dl.lib().dflash_trace_enable(ctxv.h, 12, 2 * nv) == 0
        for i in range(nv):
            sample_step(1000 + i, rsm[i])
        buf = (C_.c_float * (2 * nv))()
        assert dl.lib().dflash_trace_read_each(ctxv.h, buf, 2 * nv, C_.byref(cnt)) == 0
        dl.lib().dflash_trace_enable(ctxv.h, 0, 0)
        su = np.median(np.array(buf[:cnt.value], dtype=np.float64).reshape(nv, 2) * 1e3, axis=0)
        ksm = rsm[:, 0].float().mean().item()
        out["sampled_verify"] = {"workload": "T = 1, 15 drafted positions, vocab 151936 (fp32 logits), "
                                             "target rows near the draft's",
                                 "sample_drafts_us": round(float(su[0]), 1), "verify_rule_us": round(float(su[1]), 1),
                                 "mean_k": round(ksm, 2),
                                 "logit_bytes_per_step": 2 * 16 * sv.vocab * 4 + 15 * sv.vocab * 4}
        log(f"[bench] sampled verify: {json.dumps(out['sampled_verify'])}")
        del ctxv, wv
        torch.cuda.empty_cache()

    # ---- toy end-to-end greedy speculative loop against plain greedy decoding
    if not args.no_toy:
        from block_diffusion_drafter_context_amd import spec
        st = di.SHAPES["toy_e2e"]
        tw = {k: v.cuda() for k, v in di.toy_target_weights(st).items()}
        dw = {k: v.cuda() for k, v in di.draft_weights(st).items()}
        prompt = di.toy_prompt(st).cuda()
        n_new = di.TOY_GENERATE
        cap = prompt.shape[0] + n_new + 2 * st.block

        def fresh():
            return (dl.DFlash(st.replace(draft_layers=st.target_layers), tw, max_ctx=cap),
                    dl.DFlash(st, dw, max_ctx=cap))

        def wall(fn):
            torch.cuda.synchronize()
            t = time.perf_counter()
            r = fn()
            torch.cuda.synchronize()
            return r, time.perf_counter() - t

        tgt, _ = fresh()
        spec.greedy_generate(tgt, prompt, 8)  # warm-up of every kernel shape
        tgt, _ = fresh()
        _, t_pre = wall(lambda: spec.prefill(tgt, prompt))
        tgt, drf = fresh()
        _, t_pre_s = wall(lambda: spec.prefill(tgt, prompt, drf))
        tgt, _ = fresh()
        greedy, t_g = wall(lambda: spec.greedy_generate(tgt, prompt, n_new).cpu().tolist())
        tgt, drf = fresh()
        (sp, ks), t_s = wall(lambda: spec.spec_generate(tgt, drf, prompt, n_new))
        P = prompt.shape[0]

        def truth(C0):
            return [int(greedy[p - P]) if p - P < len(greedy) else 0 for p in range(C0 + 1, C0 + st.block)]

        tgt, drf = fresh()
        (spp, ksp), t_p = wall(lambda: spec.spec_generate(tgt, drf, prompt, n_new, drafts_fn=truth))
        out["toy_e2e"] = {
            "workload": "toy_e2e", "prompt": P, "generated": n_new,
            "note": "wall times include the prompt prefill (16-row target calls, plus fuse/inject for the draft in "
                    "the speculative loops); decode rates subtract the matching prefill time. The draft is "
                    "random-init, so its blocks are rarely accepted; the target-drafts run feeds the target's own "
                    "greedy tokens as drafts (every block accepted)",
            "prefill_s": round(t_pre, 4), "prefill_with_draft_s": round(t_pre_s, 4),
            "greedy_s": round(t_g, 4), "greedy_decode_tok_per_s": round(n_new / max(t_g - t_pre, 1e-9), 1),
            "spec_s": round(t_s, 4), "spec_steps": len(ks), "spec_mean_accept_k": round(float(np.mean(ks)), 3),
            "spec_tokens_per_step": round(len(sp) / max(len(ks), 1), 3), "spec_equals_greedy": sp == greedy,
            "spec_decode_tok_per_s": round(n_new / max(t_s - t_pre_s, 1e-9), 1),
            "target_drafts_s": round(t_p, 4), "target_drafts_steps": len(ksp),
            "target_drafts_equals_greedy": spp == greedy,
            "target_drafts_decode_tok_per_s": round(n_new / max(t_p - t_pre_s, 1e-9), 1)}
        log(f"[bench] toy end to end: {json.dumps(out['toy_e2e'])}")
        del tw, dw

    # ---- prefill side: fusion and injection of 32768 context rows (27B-class shape)
    if not args.no_prefill:
        if "ctx" in locals():
            del ctx
        ctxs.clear()
        torch.cuda.empty_cache()
        ps = di.SHAPES["fusion_prefill_32k"]
        Mp = ps.ctx
        wp = {k: v.cuda() for k, v in di.draft_weights(ps, need_draft=False, need_lm=False).items()}
        pctx = dl.DFlash(ps, wp, max_ctx=Mp + 64, max_rows=Mp)
        psel = dl.feature_layers(ps.target_layers)
        gen = torch.Generator(device="cuda").manual_seed(ps.seed)
        slabs = {l: torch.randn(Mp, ps.hidden, generator=gen, device="cuda").to(torch.bfloat16) for l in psel}
        hid = [slabs.get(l) for l in range(ps.target_layers)]
        fused = torch.empty(Mp, ps.hidden, dtype=torch.bfloat16, device="cuda")

        def time_ms(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        fuse_ms = time_ms(lambda: pctx.fuse_context(hid, out=fused))
        # the GEMM alone (without its row RMSNorm), from the library's own event trace
        dl.lib().dflash_trace_enable(pctx.h, 8, 8)
        for _ in range(5):
            pctx.fuse_context(hid, out=fused)
        import ctypes as C_
        tms, tn = C_.c_double(), C_.c_int32()
        dl.lib().dflash_trace_read(pctx.h, C_.byref(tms), C_.byref(tn))
        dl.lib().dflash_trace_enable(pctx.h, 0, 0)
        gemm_ms = tms.value / max(tn.value, 1)

        def inject():
            pctx.rollback(0)
            pctx.inject_kv(fused, 0)

        inject_ms = time_ms(inject)
        fl_fuse = 2.0 * Mp * 5 * ps.hidden * ps.hidden
        # vendor reference for the same contraction: torch.matmul (hipBLASLt) on
        # the materialised concatenation [rows, 5H] x [5H, H]
        a_cat = torch.cat([slabs[l] for l in psel], dim=1)
        w_t = wp["fc"].t().contiguous()
        ref_out = torch.empty(Mp, ps.hidden, dtype=torch.bfloat16, device="cuda")
        ref_ms = time_ms(lambda: torch.matmul(a_cat, w_t, out=ref_out))
        del a_cat, w_t, ref_out
        n_inj = ps.draft_layers * 2 * ps.n_kv_heads * ps.head_dim
        fl_inj = 2.0 * Mp * ps.hidden * n_inj
        out["prefill"] = {
            "workload": "fusion_prefill_32k", "rows": Mp, "hidden": ps.hidden, "concat_k": 5 * ps.hidden,
            "fuse_gemm_ms": round(gemm_ms, 3), "fuse_gemm_tflops": round(fl_fuse / (gemm_ms * 1e-3) / 1e12, 1),
            "fuse_gemm_mfma_frac": round(fl_fuse / (gemm_ms * 1e-3) / BF16_PEAK, 4),
            "fuse_with_norm_ms": round(fuse_ms, 3),
            "torch_matmul_same_gemm_ms": round(ref_ms, 3),
            "torch_matmul_same_gemm_tflops": round(fl_fuse / (ref_ms * 1e-3) / 1e12, 1),
            "inject_ms": round(inject_ms, 3), "inject_tflops": round(fl_inj / (inject_ms * 1e-3) / 1e12, 1),
            "inject_mfma_frac": round(fl_inj / (inject_ms * 1e-3) / BF16_PEAK, 4)}
        log(f"[bench] prefill: {json.dumps(out['prefill'])}")
        del pctx, slabs, hid, fused, wp
        torch.cuda.empty_cache()

    # ---- CPU oracle baseline: full steps of the oracle on a bounded sample
    # (steps until 10 s have elapsed, at most 30; the anchor follows each step's bonus token)
    if not args.no_cpu_baseline:
        # threads pinned close together (read by the OpenMP runtime when the
        # oracle library loads)
        os.environ.setdefault("OMP_PROC_BIND", "close")
        import oracle as orc
        m = orc.Model(s, w_cpu)
        k, v = di.context_kv(s, C)
        hid16 = [di.target_hidden(s, l, 16, tag="step") for l in sel]

        def oracle_steps(n_max, budget_s):
            anchor = di.anchor_token(s)
            n_cpu = 0
            t = time.perf_counter()
            while n_cpu < n_max and (n_cpu == 0 or time.perf_counter() - t < budget_s):
                ref = orc.draft_block(m, k, v, C, anchor, want_logits=False)
                g = di.synthetic_target_argmax(ref["tokens"], u.numpy(), r.numpy(), last, s.vocab)
                _, anchor = orc.accept(ref["tokens"], g)
                f16 = orc.fuse_rows(m, hid16, range(16))
                orc.inject_rows(m, orc.to_storage(f16, s.dtype), range(16), C)
                n_cpu += 1
            return n_cpu, (time.perf_counter() - t) / n_cpu

        threads = orc.get_threads()
        n_cpu, cpu_s = oracle_steps(30, 10.0)
        host = cpu_identity()
        out["cpu_baseline"] = {"value": round(1.0 / cpu_s, 5), "unit": "draft blocks/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{n_cpu} full steps (draft block at C={C} + accept + fuse/inject of 16 rows, "
                                         f"anchor from each step's bonus), fp64 oracle, {cpu_s * n_cpu:.1f}s in all, "
                                         f"{cpu_s:.2f}s per step, {threads} OpenMP threads "
                                         f"(OMP_PROC_BIND={os.environ.get('OMP_PROC_BIND')})",
                               **host}
        log(f"[bench] cpu oracle: {n_cpu} steps, {cpu_s:.2f}s per step with {threads} threads; host {host}")
        # the same step on one thread
        orc.set_threads(1)
        n1, s1 = oracle_steps(1, 0.0)
        orc.set_threads(threads)
        out["cpu_baseline"]["single_thread"] = {"value": round(1.0 / s1, 5), "unit": "draft blocks/s",
                                                "sample": f"{n1} full step on 1 thread, {s1:.2f}s"}
        log(f"[bench] cpu oracle, 1 thread: {s1:.2f}s per step")
        other = {}
        # the 8B shape at 36864 tokens of context: one draft block
        if args.long_ctx:
            kl, vl = di.context_kv(s, args.long_ctx)
            t = time.perf_counter()
            orc.draft_block(m, kl, vl, args.long_ctx, di.anchor_token(s), want_logits=False)
            dt_ = time.perf_counter() - t
            other[f"{args.workload}@{args.long_ctx}"] = {"value": round(1.0 / dt_, 5), "unit": "draft blocks/s",
                                                         "sample": f"1 draft block at C={args.long_ctx}, {dt_:.2f}s"}
            del kl, vl
        # the 27B-class draft block at 36864 tokens
        if "w3_cpu" in locals():
            m3 = orc.Model(s3, w3_cpu)
            t = time.perf_counter()
            orc.draft_block(m3, k3, v3, s3.ctx, di.anchor_token(s3), want_logits=False)
            dt_ = time.perf_counter() - t
            other["dense27b_36k"] = {"value": round(1.0 / dt_, 5), "unit": "draft blocks/s",
                                     "sample": f"1 draft block at C={s3.ctx}, {dt_:.2f}s"}
            del m3, w3_cpu, k3, v3
        # prefill fusion + injection of 32768 rows, timed on a 16-row subset and
        # scaled linearly in rows (each row's fusion and injection is independent)
        if not args.no_prefill:
            ps = di.SHAPES["fusion_prefill_32k"]
            wp_cpu = di.draft_weights(ps, need_draft=False, need_lm=False)
            mp = orc.Model(ps, wp_cpu)
            psel = dl.feature_layers(ps.target_layers)
            rows = 16
            slabs = [di.target_hidden(ps, l, rows, tag="cpu") for l in psel]
            t = time.perf_counter()
            fz = orc.fuse_rows(mp, slabs, range(rows))
            orc.inject_rows(mp, orc.to_storage(fz, ps.dtype), range(rows), 0)
            dt_ = time.perf_counter() - t
            full_s = dt_ * ps.ctx / rows
            fl = 2.0 * ps.ctx * ps.hidden * (5 * ps.hidden + ps.draft_layers * 2 * ps.n_kv_heads * ps.head_dim)
            other["fusion_prefill_32k"] = {"value": round(full_s, 1), "unit": "s per 32768-row fuse+inject",
                                           "tflops": round(fl / full_s / 1e12, 5),
                                           "sample": f"fuse+inject of {rows} of {ps.ctx} rows in {dt_:.2f}s, "
                                                     f"scaled by {ps.ctx // rows} (extrapolated, not measured whole)"}
            del mp, wp_cpu
        out["cpu_baseline"]["other_configs"] = other
        log(f"[bench] cpu oracle, other configs: {json.dumps(other)}")

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
