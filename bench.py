"""Benchmark of the Lizard hybrid attention layer on one MI355X.

One step = one forward pass (the chunked gated branch, window + sink
softmax and hybrid sum, all in one kernel launch) of the Llama-3-8B-shaped
prefill layer: B=4, H=32, L=4096, d=128, chunk 64, w=64, m=4, alpha=0.5,
bf16 operands with fp32 accumulation, inference mode (no lse / y_anchor /
state outputs).  Inputs are seeded synthetic tensors resident in HBM.

Prints one JSON line: tokens/s (B*L per second), the forward kernel's
position on the HBM roofline (algorithmic bytes / average launch time) and
its MFMA fraction, the float64 CPU oracle timed on a bounded sample of the
same workload, and secondary objects for the decode step (batch 64, H=32,
1024 steps after a 2048-token prefill: HBM GB/s) and the backward pass
(B=8, H=32, L=2048).

Timing of every leg: the leg's inputs are generated on the host first
(seconds, during which the GPU idles and its clock drops), then the leg's
own step runs back to back for a fixed --prewarm-ms of wall time (reported
as "prewarm_ms"; 0 turns it off) so the clock is settled again, then
exactly --warmup untimed steps, then exactly --steps timed steps between
HIP events on the launch stream, one event after every step: the mean is
the total over the steps, the median and minimum are those of the
per-step intervals.  In a --only run the leg's timed launches are the last
launches of its kernels in the process (what the profile summaries
average).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-attn fwd tokens/s + %MFMA peak (L=4k,H=32,d=128); decode GB/s % peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["subquadratic_attention_amd/csrc/lizard_fwd.hip", "subquadratic_attention_amd/csrc/lizard_common.hpp",
                  "subquadratic_attention_amd/csrc/lizard_decode.hip", "subquadratic_attention_amd/csrc/lizard_bwd.hip"]


def source_hash(paths: str) -> str:
    """Hash of the kernel sources a counter record was taken on (comma-separated
    paths, in order; the same hash as the profile summaries record)."""
    h = hashlib.sha256()
    for path in paths.split(","):
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work (per head-token / per (b, h) decode step)
# ---------------------------------------------------------------------------

def fwd_bytes_per_head_token(d: int, elem: int = 2) -> int:
    # q, k, v and y in the element type, log_g in float32
    return 3 * elem * d + 4 * d + elem * d


def fwd_logit_bytes_per_head_token(d: int, elem: int = 2) -> int:
    # q, k, v, the gate logits and y, all in the element type
    return 5 * elem * d


def fwd_flops_per_head_token(d: int, C: int = 64, w: int = 64, m: int = 4) -> int:
    # readout + carry 4 d^2, intra causal pairs (C+1)(dk+dv), window+sink logits 2(w+m)d, window values 2wd
    return 4 * d * d + (C + 1) * 2 * d + 2 * (w + m) * d + 2 * w * d


def bwd_bytes_per_head_token(d: int, elem: int = 2) -> int:
    # reads q, k, v, dy (elem), log_g (f32), lse (f32); writes dq, dk, dv (elem), dlog_g (f32)
    return 4 * elem * d + 4 * d + 4 + 3 * elem * d + 4 * d


def bwd_flops_per_head_token(d: int, C: int = 64, w: int = 64, m: int = 4) -> int:
    return 10 * d * d + 5 * (C + 1) * d + 6 * (w + m) * d + 4 * w * d


def decode_bytes_per_bh(d: int, w: int, elem: int = 2) -> int:
    # state read + write (f32), window keys and values except the incoming token, q/k/v/log_g in,
    # ring slot write, y out
    return 2 * 4 * d * d + 2 * elem * (w - 1) * d + 3 * elem * d + 4 * d + 2 * elem * d + elem * d


# ---------------------------------------------------------------------------

def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(rec["source"]):
        return None
    return rec.get("hbm_bytes_per_launch")


PREWARM_MS = 300.0


def prewarm(fn, ms: float):
    """Run fn back to back for `ms` milliseconds of wall time (in batches of
    8 calls, each batch waited for), so the GPU clock has settled before the
    warm-up and timed steps."""
    import torch

    if ms <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_steps(fn, steps: int, warmup: int, prewarm_ms: float = None):
    """Prewarm, `warmup` untimed steps, then `steps` timed steps with an event
    after each.  Returns {"mean", "median", "min"} in ms per step (the mean
    over the whole region, the median and minimum over the per-step
    intervals) and the number of timed steps."""
    import torch

    prewarm(fn, PREWARM_MS if prewarm_ms is None else prewarm_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return {"mean": ev[0].elapsed_time(ev[-1]) / steps, "median": median, "min": per[0], "steps": steps}


def time_region(fn, steps: int, warmup: int, prewarm_ms: float = None):
    """Mean ms per step (see time_steps)."""
    return time_steps(fn, steps, warmup, prewarm_ms)["mean"]


def stats_us(t):
    return {"mean_us": round(t["mean"] * 1e3, 2), "median_us": round(t["median"] * 1e3, 2),
            "min_us": round(t["min"] * 1e3, 2), "timed_steps": t["steps"]}


def bench_fwd(sqa, si, steps, warmup, logit=False, workload="llama3_8b_prefill_bf16"):
    import torch

    w = si.WORKLOADS[workload]
    st = si.storage_inputs(w, with_logit=logit)
    x = {}
    for k, v in st.items():
        import numpy as np

        x[k] = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() if v.dtype == np.uint16 else \
            torch.from_numpy(v).cuda()
    del st
    out = {"y": torch.empty_like(x["q"])}

    def step():
        if logit:
            sqa.lizard_attn_fwd_logit(x["q"], x["k"], x["v"], x["gate_logit"], x["meta_k"], window=w.window,
                                      alpha=w.alpha, out=out)
        else:
            sqa.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window, alpha=w.alpha,
                                out=out)

    t = time_steps(step, steps, warmup)
    head_tokens = w.B * w.H * w.L
    elem = 2 if w.dtype == "bf16" else 4
    alg_bytes = head_tokens * (fwd_logit_bytes_per_head_token(w.d, elem) if logit else
                               fwd_bytes_per_head_token(w.d, elem))
    alg_flops = head_tokens * fwd_flops_per_head_token(w.d, w.chunk, w.window, w.n_meta)
    del x, out
    torch.cuda.empty_cache()
    return w, t, alg_bytes, alg_flops


def bench_fwd_logit(sqa, si, steps, warmup):
    """The same prefill with the gates fed as bf16 logits (log-sigmoid in the
    kernel's prologue): 1,280 instead of 1,536 algorithmic bytes per head-token."""
    w, t, alg_bytes, _ = bench_fwd(sqa, si, steps, warmup, logit=True)
    ms = t["mean"]
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"workload": "llama3_8b_prefill_bf16, gate logits in bf16", "ms": round(ms, 5), **stats_us(t),
            "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1), "alg_bytes": alg_bytes, "gbps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic("lizard_fwd", "llama3_8b_prefill_logit_bf16")}


def bench_train_step(sqa, si, workload, steps, warmup):
    """One training step of the layer: the training forward (y, lse and the
    chunk-start states) and the backward reading those states, with a seeded
    upstream gradient.  Returns (workload, timing)."""
    import numpy as np
    import torch

    w = si.WORKLOADS[workload]
    st = si.storage_inputs(w, with_dy=True)
    x = {k: (torch.from_numpy(v.view(np.int16)).view(torch.bfloat16) if v.dtype == np.uint16 else
             torch.from_numpy(v)).cuda() for k, v in st.items()}
    del st
    q = x["q"]
    fout = {"y": torch.empty_like(q), "lse": torch.empty((w.B, w.H, w.L), device="cuda", dtype=torch.float32),
            "chunk_states": torch.empty((w.B, w.H, (w.L + 63) // 64, w.d, w.d), device="cuda", dtype=q.dtype)}
    gout = {key: torch.empty_like(x[src]) for key, src in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dlog_g", "log_g"))}
    gout["dmeta"] = torch.empty(tuple(x["meta_k"].shape), device="cuda", dtype=torch.float32)
    ws = torch.empty(max(16, sqa.lizard_attn_bwd_workspace_size(w.B, w.H, w.L, w.d, window=w.window,
                                                                n_meta=w.n_meta, dtype=sqa._dtype_code(q))),
                     device="cuda", dtype=torch.uint8)

    def step():
        sqa.lizard_attn_fwd_train(x["q"], x["k"], x["v"], x["meta_k"], log_g=x["log_g"], window=w.window,
                                  alpha=w.alpha, out=fout)
        sqa.lizard_attn_bwd_train(x["q"], x["k"], x["v"], x["meta_k"], fout["lse"], fout["chunk_states"], x["dy"],
                                  log_g=x["log_g"], window=w.window, alpha=w.alpha, workspace=ws, out=gout)

    step()
    t = time_steps(step, steps, warmup)
    del x, fout, gout, ws
    torch.cuda.empty_cache()
    return w, t


def bench_fp32_ablation(sqa, si, steps, warmup):
    """The pages' one speed claim is that the log-space form, whose gate
    factors fold into bf16 matrix-core operands, raises training throughput
    over a float32 fallback.  Measured here two ways, each with the same
    kernels built for bf16 operands (bf16 MFMA, fp32 accumulate) and for
    fp32 operands (fp32 MFMA), at d=64, the largest head dim the fp32 build
    has: the inference forward on the prefill shapes (B=4, H=32, L=4096) and
    the training step (training forward + backward reading its chunk
    states) on the backward's shapes (B=8, H=32, L=2048)."""
    res = {}
    for name in ("prefill_d64_bf16", "prefill_d64_f32"):
        w, t, alg_bytes, _ = bench_fwd(sqa, si, steps, warmup, workload=name)
        ms = t["mean"]
        res[name] = {"ms": round(ms, 5), **stats_us(t), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
                     "gbps": round(alg_bytes / (ms * 1e-3) / 1e9, 1)}
    res["bf16_over_fp32"] = round(res["prefill_d64_bf16"]["tokens_per_s"] / res["prefill_d64_f32"]["tokens_per_s"], 3)
    train = {}
    for name in ("train_d64_bf16", "train_d64_f32"):
        w, t = bench_train_step(sqa, si, name, steps, warmup)
        train[name] = {"ms": round(t["mean"], 5), **stats_us(t),
                       "tokens_per_s": round(w.B * w.L / (t["mean"] * 1e-3), 1)}
    train["bf16_over_fp32"] = round(train["train_d64_bf16"]["tokens_per_s"] / train["train_d64_f32"]["tokens_per_s"], 3)
    train["pages_claim"] = "training throughput up to +32 % (de page) / +32-36 % (it page) for bf16 over fp32"
    res["train_step"] = train
    return res


def bench_long_ctx(sqa, si, steps, warmup):
    """Long-context prefill (B=1, H=32, L=32768, gates N(2,2)).  One head's
    sequence is a chain of chunks, so a one-pass schedule would run one
    workgroup per (head, value slice), 64 for the whole GPU; both calls timed
    here cut each sequence into segments run side by side.  lizard_attn_fwd
    takes a stream-ordered workspace of its own on every call (inside the
    timed region); lizard_attn_fwd_split uses one the caller allocated once,
    outside it."""
    import numpy as np
    import torch

    w = si.WORKLOADS["long_ctx_32k_bf16"]
    st = si.storage_inputs(w)
    x = {k: (torch.from_numpy(v.view(np.int16)).view(torch.bfloat16) if v.dtype == np.uint16 else
             torch.from_numpy(v)).cuda() for k, v in st.items()}
    del st
    out = {"y": torch.empty_like(x["q"])}
    need = sqa.lizard_attn_fwd_split_workspace_size(w.B, w.H, w.L, w.d, window=w.window, n_meta=w.n_meta)
    ws = torch.empty(max(need, 1), device="cuda", dtype=torch.uint8)

    def split():
        sqa.lizard_attn_fwd_split(x["q"], x["k"], x["v"], x["meta_k"], log_g=x["log_g"], window=w.window,
                                  alpha=w.alpha, workspace=ws, out=out)

    def named():
        sqa.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window, alpha=w.alpha, out=out)

    # the named call first, the split call last (its launches are then the
    # last ones of the process, which the profile summary averages)
    t_named = time_steps(named, steps, warmup)
    t_split = time_steps(split, steps, warmup)
    alg_bytes = w.B * w.H * w.L * fwd_bytes_per_head_token(w.d)
    del x, out, ws
    torch.cuda.empty_cache()
    res = {"workload": "long_ctx_32k_bf16 (B=1, H=32, L=32768, d=128, gates N(2,2))", "steps": steps,
           "segments_workspace_bytes": need}
    for name, call, t in (("split", "lizard_attn_fwd_split", t_split), ("named", "lizard_attn_fwd", t_named)):
        ms = t["mean"]
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        res[name] = {"call": call, "ms": round(ms, 5), **stats_us(t), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
                     "gbps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    res["named_over_split"] = round(t_named["mean"] / t_split["mean"], 3)
    return res


def bench_decode(sqa, si, reps=3):
    """1024 back-to-back steps after a 2048-token prefill (prefill untimed)."""
    import numpy as np
    import torch

    w = si.WORKLOADS["decode_b64_bf16"]
    st = si.storage_inputs(w)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() if a.dtype == np.uint16 else \
            torch.from_numpy(np.ascontiguousarray(a)).cuda()

    L0, steps = w.L, w.steps
    pre = {k: dev(np.ascontiguousarray(st[k][:, :, :L0])) for k in ("q", "k", "v", "log_g")}
    meta = dev(st["meta_k"])
    # decode inputs laid out [step, B, H, d] so each step reads a contiguous slice
    dec = {k: dev(np.ascontiguousarray(st[k][:, :, L0:].transpose(2, 0, 1, 3))) for k in ("q", "k", "v", "log_g")}
    ring0 = {k: dev(np.ascontiguousarray(st[k][:, :, L0 - w.window:L0])) for k in ("k", "v")}
    del st
    res = sqa.lizard_attn_fwd(pre["q"], pre["k"], pre["v"], pre["log_g"], meta, window=w.window, alpha=w.alpha,
                              need_state=True)
    state0 = res["state"]
    del pre, res
    y = torch.empty((steps, w.B, w.H, w.d), device="cuda", dtype=torch.bfloat16)
    state = torch.empty_like(state0)
    kr = torch.empty_like(ring0["k"])
    vr = torch.empty_like(ring0["v"])
    # (L0 - w) is a multiple of w, so slot p mod w of the ring is row p - (L0 - w)

    def run_all(per_step_events=None, flush=None):
        state.copy_(state0)
        kr.copy_(ring0["k"])
        vr.copy_(ring0["v"])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            if flush is not None:
                flush()
            if per_step_events is not None:
                per_step_events[i][0].record()
            sqa.lizard_decode_step(L0 + i, dec["q"][i], dec["k"][i], dec["v"][i], dec["log_g"][i], meta, state, kr,
                                   vr, alpha=w.alpha, y_t=y[i])
            if per_step_events is not None:
                per_step_events[i][1].record()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    prewarm(run_all, PREWARM_MS)
    run_all()  # warm-up
    # cache-flushed: 512 MiB read between steps evicts the 256 MB last-level cache
    # (a read, so that no dirty lines of the flush are written back while the
    # decode kernel runs); only the decode kernel is timed (per-step events)
    scratch = torch.ones((512 << 20) // 4, device="cuda", dtype=torch.int32)
    sink = torch.empty((), device="cuda", dtype=torch.int64)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    run_all(per_step_events=ev, flush=lambda: torch.sum(scratch, dim=0, out=sink))
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms_flushed = sum(per) / steps
    bytes_step = w.B * w.H * decode_bytes_per_bh(w.d, w.window)
    out = {
        "workload": "decode_b64_bf16", "B": w.B, "H": w.H, "d": w.d, "window": w.window, "n_meta": w.n_meta,
        "prefill": L0, "steps": steps,
        "alg_bytes_per_step": bytes_step,
        "flushed_us_per_step": round(ms_flushed * 1e3, 2),
        "flushed_p50_us": round(per[steps // 2] * 1e3, 2),
        "flushed_min_us": round(per[0] * 1e3, 2),
        "flushed_gbps": round(bytes_step / (ms_flushed * 1e-3) / 1e9, 1),
        "flushed_frac_hbm_peak": round(bytes_step / (ms_flushed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "traffic": read_traffic("lizard_decode", "decode_b64_bf16"),
    }
    # serving form: the same 1024 tokens as 256 calls of T = 4 tokens per row
    # (lizard_decode_tokens, positions on the device); the state is read and
    # written once per call
    T = 4
    pos_all = (L0 + T * torch.arange(steps // T, device="cuda", dtype=torch.int64))[:, None].repeat(1, w.B).contiguous()
    dec4 = {kk: vv.view(steps // T, T, w.B, w.H, w.d).permute(0, 2, 3, 1, 4).contiguous() for kk, vv in dec.items()}
    y4 = torch.empty((steps // T, w.B, w.H, T, w.d), device="cuda", dtype=torch.bfloat16)

    def run_tokens():
        state.copy_(state0)
        kr.copy_(ring0["k"])
        vr.copy_(ring0["v"])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps // T):
            sqa.lizard_decode_tokens(pos_all[i], dec4["q"][i], dec4["k"][i], dec4["v"][i], dec4["log_g"][i], meta,
                                     state, kr, vr, alpha=w.alpha, y=y4[i])
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    run_tokens()
    ms_tok = sum(run_tokens() for _ in range(reps)) / reps
    # per call: the state once, then per token the window, inputs and output
    bytes_call = w.B * w.H * (decode_bytes_per_bh(w.d, w.window) + (T - 1) * (decode_bytes_per_bh(w.d, w.window)
                                                                               - 2 * 4 * w.d * w.d))
    out["tokens4"] = {"T": T, "us_per_token": round(ms_tok * 1e3, 2), "tokens_per_s": round(w.B / (ms_tok * 1e-3), 1),
                      "alg_bytes_per_call": bytes_call,
                      "gbps": round(bytes_call / (T * ms_tok * 1e-3) / 1e9, 1)}
    # the same 1024 steps recorded once into a HIP graph (torch.cuda.graph)
    # and replayed: no host launch per token (the positions are kernel
    # arguments, so a replay repeats the recorded steps from the restored
    # state); its outputs must equal the eager run's bit for bit
    y_eager = y.clone()
    state.copy_(state0)
    kr.copy_(ring0["k"])
    vr.copy_(ring0["v"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            sqa.lizard_decode_step(L0 + i, dec["q"][i], dec["k"][i], dec["v"][i], dec["log_g"][i], meta, state, kr,
                                   vr, alpha=w.alpha, y_t=y[i])

    def run_graph():
        state.copy_(state0)
        kr.copy_(ring0["k"])
        vr.copy_(ring0["v"])
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        graph.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    y.fill_(float("nan"))
    ms_graph = [run_graph() for _ in range(reps + 1)][1:]
    out["graph"] = {"us_per_step": round(sum(ms_graph) / reps * 1e3, 2), "replays": reps, "steps_per_replay": steps,
                    "equals_eager_bitwise": bool(torch.equal(y, y_eager))}
    del graph, y_eager
    # back to back last: `reps` runs of the 1024 steps, the mean over all of
    # them (these are the last launches of the one-token kernel)
    prewarm(run_all, PREWARM_MS)
    runs = [run_all() for _ in range(reps)]
    ms_b2b = sum(runs) / reps
    out.update({"us_per_step": round(ms_b2b * 1e3, 2), "best_run_us_per_step": round(min(runs) * 1e3, 2),
                "timed_steps": reps * steps, "tokens_per_s": round(w.B / (ms_b2b * 1e-3), 1),
                "gbps": round(bytes_step / (ms_b2b * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(bytes_step / (ms_b2b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    del dec, dec4, y4, pos_all, ring0, y, state, state0, kr, vr, scratch, sink
    torch.cuda.empty_cache()
    return out


def bench_decode_graph_b1(sqa, reps, steps=256):
    """One sequence (B = 1, H = 32, d = 128, window 64, 4 sinks): a decode
    step moves 5.3 MB, under a microsecond of HBM time, so one host launch
    per token bounds the eager loop; the same steps as one HIP graph.
    Seeded synthetic state, rings and tokens (timing only)."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(20250709)
    B, H, d, wnd, m = 1, 32, 128, 64, 4

    def rn(*shape, sd=1.0):
        return torch.randn(*shape, device="cuda", generator=g) * sd

    state0 = rn(B, H, d, d, sd=0.05)
    kr0 = rn(B, H, wnd, d, sd=0.125).bfloat16()
    vr0 = rn(B, H, wnd, d, sd=0.125).bfloat16()
    meta = rn(H, m, d, sd=0.125).bfloat16()
    q, k, v = (rn(steps, B, H, d, sd=0.125).bfloat16() for _ in range(3))
    lg = torch.nn.functional.logsigmoid(rn(steps, B, H, d) + 3.0)
    y = torch.empty((steps, B, H, d), device="cuda", dtype=torch.bfloat16)
    state, kr, vr = state0.clone(), kr0.clone(), vr0.clone()
    p0 = 4096

    def launch_all():
        for i in range(steps):
            sqa.lizard_decode_step(p0 + i, q[i], k[i], v[i], lg[i], meta, state, kr, vr, alpha=0.5, y_t=y[i])

    def timed(fn):
        state.copy_(state0)
        kr.copy_(kr0)
        vr.copy_(vr0)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    prewarm(launch_all, PREWARM_MS)   # the host's launch path and the GPU clock settled
    timed(launch_all)
    eager = [timed(launch_all) for _ in range(reps)]
    y_eager = y.clone()
    state.copy_(state0)
    kr.copy_(kr0)
    vr.copy_(vr0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch_all()
    timed(graph.replay)
    replayed = [timed(graph.replay) for _ in range(reps)]
    ms_e, ms_g = sum(eager) / reps, sum(replayed) / reps
    bytes_step = B * H * decode_bytes_per_bh(d, wnd)
    res = {"workload": "decode B=1 H=32 d=128 window 64, 4 sinks (seeded synthetic)", "steps": steps,
           "alg_bytes_per_step": bytes_step, "eager_us_per_step": round(ms_e * 1e3, 2),
           "graph_us_per_step": round(ms_g * 1e3, 2), "graph_speedup": round(ms_e / ms_g, 2),
           "graph_gbps": round(bytes_step / (ms_g * 1e-3) / 1e9, 1),
           "equals_eager_bitwise": bool(torch.equal(y, y_eager))}
    del graph, q, k, v, lg, y, y_eager, state, kr, vr, state0, kr0, vr0
    torch.cuda.empty_cache()
    return res


def bench_bwd(sqa, si, steps, warmup, logit=False):
    import numpy as np
    import torch

    w = si.WORKLOADS["train_bwd_bf16"]
    st = si.storage_inputs(w, with_dy=True, with_logit=logit)
    x = {k: (torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() if v.dtype == np.uint16 else
             torch.from_numpy(v).cuda()) for k, v in st.items()}
    del st
    if logit:
        fw = sqa.lizard_attn_fwd_logit(x["q"], x["k"], x["v"], x["gate_logit"], x["meta_k"], window=w.window,
                                       alpha=w.alpha, need_lse=True)
    else:
        fw = sqa.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window, alpha=w.alpha,
                                 need_lse=True)
    ws = torch.empty(max(16, sqa.lizard_attn_bwd_workspace_size(w.B, w.H, w.L, w.d, window=w.window,
                                                                 n_meta=w.n_meta, dtype=sqa.LIZARD_BF16)),
                     device="cuda", dtype=torch.uint8)
    gname = "gate_logit" if logit else "log_g"
    out = {key: torch.empty_like(x[src]) for key, src in (("dq", "q"), ("dk", "k"), ("dv", "v"),
                                                          ("dgate_logit" if logit else "dlog_g", gname))}
    out["dmeta"] = torch.empty(tuple(x["meta_k"].shape), device="cuda", dtype=torch.float32)

    def step():
        if logit:
            sqa.lizard_attn_bwd_logit(x["q"], x["k"], x["v"], x["gate_logit"], x["meta_k"], fw["lse"], x["dy"],
                                      window=w.window, alpha=w.alpha, workspace=ws, out=out)
        else:
            sqa.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], fw["lse"], x["dy"],
                                window=w.window, alpha=w.alpha, workspace=ws, out=out)

    step()
    t_saved = None
    if not logit:
        # the same backward reading the chunk-start states a training forward
        # kept (timed first: the plain backward's launches are then the last
        # ones of the process)
        tr = sqa.lizard_attn_fwd_train(x["q"], x["k"], x["v"], x["meta_k"], log_g=x["log_g"], window=w.window,
                                       alpha=w.alpha)

        def step_saved():
            sqa.lizard_attn_bwd_train(x["q"], x["k"], x["v"], x["meta_k"], tr["lse"], tr["chunk_states"], x["dy"],
                                      log_g=x["log_g"], window=w.window, alpha=w.alpha, workspace=ws, out=out)

        t_saved = time_steps(step_saved, steps, warmup)
        del tr
    t = time_steps(step, steps, warmup)
    ms = t["mean"]
    head_tokens = w.B * w.H * w.L
    # with logits: the gate in and its gradient out in bf16 instead of float32
    alg_bytes = head_tokens * (bwd_bytes_per_head_token(w.d) - (4 * w.d if logit else 0))
    alg_flops = head_tokens * bwd_flops_per_head_token(w.d, w.chunk, w.window, w.n_meta)
    res = {
        "workload": "train_bwd_bf16" + (", gate logits in bf16" if logit else ""), "B": w.B, "H": w.H, "L": w.L, "d": w.d,
        "ms": round(ms, 4), **stats_us(t), "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1),
        "alg_bytes": alg_bytes, "gbps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "tflops": round(alg_flops / (ms * 1e-3) / 1e12, 2),
        "frac_mfma_peak": round(alg_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "workspace_bytes": int(ws.numel()),
        "traffic": read_traffic("lizard_bwd", "train_bwd_logit_bf16" if logit else "train_bwd_bf16"),
    }
    if t_saved is not None:
        res["ms_with_saved_states"] = round(t_saved["mean"], 4)
        res["with_saved_states"] = stats_us(t_saved)
    del x, fw, ws, out
    torch.cuda.empty_cache()
    return res


def bench_stage1(sqa, si, steps, warmup):
    """One synthetic stage-1 attention-transfer step on the backward workload's
    shapes (B=8, H=32, L=2048, d=128, bf16): the causal softmax teacher, the
    layer's training forward (lse and chunk-start states kept), the
    output-matching loss and the layer's backward reading those states.  Also
    timed: the same step with the plain forward and a backward that recomputes
    the states, and the teacher alone (causal QK^T and PV flops)."""
    import numpy as np
    import torch

    w = si.WORKLOADS["train_bwd_bf16"]
    st = si.storage_inputs(w)
    x = {k: (torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() if v.dtype == np.uint16 else
             torch.from_numpy(v).cuda()) for k, v in st.items()}
    del st
    ws = torch.empty(max(16, sqa.lizard_attn_bwd_workspace_size(w.B, w.H, w.L, w.d, window=w.window,
                                                                n_meta=w.n_meta, dtype=sqa.LIZARD_BF16)),
                     device="cuda", dtype=torch.uint8)
    tout = {"y": torch.empty_like(x["q"])}
    fout = {"y": torch.empty_like(x["q"]),
            "lse": torch.empty((w.B, w.H, w.L), device="cuda", dtype=torch.float32),
            "chunk_states": torch.empty((w.B, w.H, (w.L + 63) // 64, w.d, w.d), device="cuda",
                                        dtype=torch.bfloat16)}
    dy = torch.empty_like(x["q"])
    loss_bh = torch.empty((w.B, w.H), device="cuda", dtype=torch.float32)
    gout = {key: torch.empty_like(x[src]) for key, src in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dlog_g", "log_g"))}
    gout["dmeta"] = torch.empty(tuple(x["meta_k"].shape), device="cuda", dtype=torch.float32)

    def teacher():
        sqa.lizard_softmax_attn_fwd(x["q"], x["k"], x["v"], out=tout)

    def step():
        teacher()
        sqa.lizard_attn_fwd_train(x["q"], x["k"], x["v"], x["meta_k"], log_g=x["log_g"], window=w.window,
                                  alpha=w.alpha, out=fout)
        sqa.lizard_transfer_loss(fout["y"], tout["y"], dy=dy, loss_bh=loss_bh)
        sqa.lizard_attn_bwd_train(x["q"], x["k"], x["v"], x["meta_k"], fout["lse"], fout["chunk_states"], dy,
                                  log_g=x["log_g"], window=w.window, alpha=w.alpha, workspace=ws, out=gout)

    def step_recompute():
        teacher()
        sqa.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], window=w.window, alpha=w.alpha,
                            need_lse=True, out=fout)
        sqa.lizard_transfer_loss(fout["y"], tout["y"], dy=dy, loss_bh=loss_bh)
        sqa.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta_k"], fout["lse"], dy, window=w.window,
                            alpha=w.alpha, workspace=ws, out=gout)

    ms_t = time_region(teacher, 3 * steps, warmup)
    ms_r = time_region(step_recompute, steps, warmup)
    ms = time_region(step, steps, warmup)
    t_flops = w.B * w.H * 2 * w.L * (w.L + 1) * w.d    # causal pairs x (QK^T + PV) x 2 flops
    res = {"workload": "train_bwd_bf16 shapes, teacher = causal softmax attention", "ms": round(ms, 4),
           "tokens_per_s": round(w.B * w.L / (ms * 1e-3), 1), "loss": round(float(loss_bh.sum()), 6),
           "ms_recomputing_states": round(ms_r, 4),
           "teacher_ms": round(ms_t, 4), "teacher_tflops": round(t_flops / (ms_t * 1e-3) / 1e12, 1),
           "teacher_frac_mfma_peak": round(t_flops / (ms_t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del x, ws, tout, fout, dy, loss_bh, gout
    torch.cuda.empty_cache()
    return res


def cpu_baseline(si, target_s: float = 15.0):
    """The float64 oracle (oracle.lizard_fwd) on a bounded sample: whole-length
    heads of the 4K prefill workload, one BLAS thread."""
    import numpy as np

    import oracle

    from threadpoolctl import threadpool_limits

    w = si.WORKLOADS["llama3_8b_prefill_bf16"]
    n = 0
    elapsed = 0.0
    with threadpool_limits(limits=1):
        while elapsed < target_s and n < w.B * w.H:
            b, h = divmod(n, w.H)
            s = si.slice_inputs(w, b, h)
            mk = si.meta_keys(w, h)[None]
            t0 = time.perf_counter()
            oracle.lizard_fwd(s["q"][None], s["k"][None], s["v"][None], s["log_g"][None], mk, w.window, w.alpha)
            elapsed += time.perf_counter() - t0
            n += 1
    head_tokens_per_s = n * w.L / elapsed
    return {
        "value": round(head_tokens_per_s / w.H, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": f"{n} whole (b,h) heads x L={w.L} of the 4K prefill workload in {elapsed:.1f} s "
                  f"(float64 numpy, 1 thread); tokens/s = head-tokens/s / H",
        "host_cpus": os.cpu_count(), "np_version": np.__version__,
    }


def main():
    global PREWARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=PREWARM_MS,
                    help="wall time each leg's step runs back to back before its warm-up (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-logit", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-stage1", action="store_true")
    ap.add_argument("--no-long-ctx", action="store_true")
    ap.add_argument("--only", choices=["fwd", "decode", "bwd", "fwd_logit", "bwd_logit", "fp32_ablation", "stage1",
                                       "long_ctx", "decode_b1"],
                    default=None,
                    help="run one leg only (for profiler runs); prints that leg's record")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the layer's kernels run on a single MI355X; "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import seeded_inputs as si
    import subquadratic_attention_amd as sqa

    sqa.load_library()
    torch.cuda.init()
    PREWARM_MS = max(0.0, args.prewarm_ms)

    if args.copy_calibration:
        src = torch.empty(1 << 30, device="cuda", dtype=torch.uint8).fill_(3)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30}), flush=True)
        del src, dst

    if args.only == "decode":
        print(json.dumps({"prewarm_ms": PREWARM_MS, **bench_decode(sqa, si)}), flush=True)
        return
    if args.only == "decode_b1":
        print(json.dumps(bench_decode_graph_b1(sqa, 3)), flush=True)
        return
    if args.only == "bwd":
        print(json.dumps(bench_bwd(sqa, si, args.steps, args.warmup)), flush=True)
        return
    if args.only == "fwd_logit":
        print(json.dumps(bench_fwd_logit(sqa, si, args.steps, args.warmup)), flush=True)
        return
    if args.only == "bwd_logit":
        print(json.dumps(bench_bwd(sqa, si, args.steps, args.warmup, logit=True)), flush=True)
        return
    if args.only == "stage1":
        print(json.dumps(bench_stage1(sqa, si, args.steps, args.warmup)), flush=True)
        return
    if args.only == "long_ctx":
        print(json.dumps(bench_long_ctx(sqa, si, args.steps, args.warmup)), flush=True)
        return
    if args.only == "fp32_ablation":
        print(json.dumps(bench_fp32_ablation(sqa, si, args.steps, args.warmup)), flush=True)
        return

    w, t, alg_bytes, alg_flops = bench_fwd(sqa, si, args.steps, args.warmup)
    ms = t["mean"]
    print(f"# fwd done: {ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    tokens = w.B * w.L
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_ms": PREWARM_MS,
        "ms_per_step": round(ms, 5),
        "step_stats": stats_us(t),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_prefill_bf16", "B": w.B, "H": w.H, "L": w.L, "d": w.d, "chunk": w.chunk,
                   "window": w.window, "n_meta": w.n_meta, "alpha": w.alpha, "mode": "inference (y only)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("lizard_fwd", "llama3_8b_prefill_bf16"),
                     "kernel": "lizard_fwd_kernel<bf16,128,64>", "alg_bytes_per_launch": alg_bytes},
        "mfma": {"achieved_tflops": round(tflops, 2), "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "alg_flops_per_launch": alg_flops,
                 "frac_ceiling_at_hbm_bound": round(fwd_flops_per_head_token(w.d) / fwd_bytes_per_head_token(w.d)
                                                    * HBM_PEAK_GBS / 1e3 / BF16_PEAK_TFLOPS, 4)},
    }
    if args.only == "fwd":
        print(json.dumps(rec), flush=True)
        return
    if not args.no_logit:
        rec["fwd_logit"] = bench_fwd_logit(sqa, si, args.steps, args.warmup)
        print("# fwd_logit done", file=sys.stderr, flush=True)
    if not args.no_ablation:
        rec["fp32_ablation"] = bench_fp32_ablation(sqa, si, args.steps, args.warmup)
        print("# fp32 ablation done", file=sys.stderr, flush=True)
    if not args.no_long_ctx:
        rec["long_ctx"] = bench_long_ctx(sqa, si, args.steps, args.warmup)
        print("# long_ctx done", file=sys.stderr, flush=True)
    if not args.no_decode:
        rec["decode"] = bench_decode(sqa, si)
        # one sequence, eager and as a HIP graph (a leg of its own: its launches
        # of the same kernel stay out of the batch-64 decode's profile)
        rec["decode_b1"] = bench_decode_graph_b1(sqa, 3)
        print("# decode done", file=sys.stderr, flush=True)
    if not args.no_bwd:
        try:
            rec["bwd"] = bench_bwd(sqa, si, args.steps, args.warmup)
            if not args.no_logit:
                rec["bwd_logit"] = bench_bwd(sqa, si, args.steps, args.warmup, logit=True)
        except sqa.LizardError as e:
            rec["bwd"] = {"error": str(e)}
        print("# bwd done", file=sys.stderr, flush=True)
    if not args.no_stage1:
        rec["stage1"] = bench_stage1(sqa, si, args.steps, args.warmup)
        print("# stage1 done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(si)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
