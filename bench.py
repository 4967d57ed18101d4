"""Benchmark of the MSA forward path on one MI355X.

One step = the whole prefill hot path on the 128K-token workload (B=1,
N=T=131072, Hq=64, G=8, d=128, Bk=128, k=16, needles planted): fused index
scoring + block max + top-k, then KV-outer sparse attention with inversion and
combine, as one msa_prefill call (the two halves of successive row windows
overlapped on two streams); the same step as the two calls msa_select_blocks
+ msa_sparse_attn_prefill is timed with events for the stage breakdown.  Inputs are
generated on the device before timing.  Printed: one JSON line with the
prefill throughput (algorithmic TFLOP/s), the roofline of the kernel that takes
the most time per step (and of the other stage kernels; per-kernel times from
the library's own HIP events on each launch stream), the decode leg (B=16 x 256K cache, GB/s), the standalone
top-k leg on the materialised 128K scores (us), and the CPU oracle baseline
on a bounded sample of rows.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--only prefill]
    python bench.py --block-size 64 --only prefill   # 64-key blocks, k = 32
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_long_index_amd import accounting as acc  # noqa: E402
from block_sparse_long_index_amd import ops  # noqa: E402
from msa_inputs import WORKLOADS, make_inputs, sample_rows  # noqa: E402

METRIC = "MSA prefill eff. TFLOP/s & decode HBM GB/s at 128K; top-k select µs (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counter_traffic(kernel):
    """Bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE from rocprofv3,
    copy-calibrated) from the committed counter summaries under profiles/:
    a line `traffic: <kernel> | sources: <files> | sha256: <hex> | fetch_bytes:
    <n> | write_bytes: <n>`.  None when no summary names the kernel or when
    its source files changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        for line in open(path):
            if not line.startswith("traffic: "):
                continue
            f = dict(x.strip().split(": ", 1) for x in line.strip().split(" | "))
            if f.get("traffic") != kernel:
                continue
            h = hashlib.sha256()
            for src in f["sources"].split(","):
                with open(os.path.join(ROOT, "block_sparse_long_index_amd", "csrc",
                                       src.strip()), "rb") as fh:
                    h.update(fh.read())
            if h.hexdigest() != f["sha256"]:
                return None
            return int(f["fetch_bytes"]) + int(f["write_bytes"])
    return None


def kernel_times(fn, steps, between=None):
    """fn() run `steps` times with the library's per-kernel timing on (HIP
    events recorded by the library on each kernel's own launch stream):
    {kind: {avg_launch_ms, launches_per_step, ms_per_step}}.  between(): work
    run before each step, outside the library (not timed)."""
    torch.cuda.synchronize()
    ops.timing_begin(1 << 18)
    t0 = time.perf_counter()
    for _ in range(steps):
        if between is not None:
            between()
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    t = ops.timing_end()
    out = {k: {"avg_launch_ms": ms / n, "launches_per_step": n / steps, "ms_per_step": ms / steps}
           for k, (ms, n) in t.items()}
    out["wall_ms_per_step"] = wall * 1e3
    return out


def roof(kernel, bound, achieved, peak, unit, traffic=None, **extra):
    r = {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
         "frac": achieved / peak, "traffic": traffic}
    r.update(extra)
    return r


def ev():
    return torch.cuda.Event(enable_timing=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo) and the threads this
    process may run on."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name, len(os.sched_getaffinity(0))


def config_leg(name, steps, warmup, cpu=False):
    """One more prefill workload (select + attention per step), timed like the
    headline leg: per-step wall time between synchronisations, and the two
    calls' times from events on the launch stream."""
    w = WORKLOADS[name]
    log("[bench] config leg", name, "generating")
    inp = make_inputs(w, device="cuda")
    qI, kI, q, K, V = inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"]
    idx = torch.empty(w.B, w.G, w.T, w.k, dtype=torch.int32, device="cuda")
    O = torch.empty_like(q)
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws = torch.empty(max(1, ops.workspace_bytes(ops.OP_ATTN_PREFILL, d)), dtype=torch.uint8,
                     device="cuda")
    nsel = ops.workspace_bytes(ops.OP_SELECT_BLOCKS, d)
    ws_sel = torch.empty(nsel, dtype=torch.uint8, device="cuda") if nsel else None

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        ops.select_blocks(qI, kI, w.k, out=idx, workspace=ws_sel, Bk=w.Bk)
        if evs is not None:
            evs[1].record()
        ops.sparse_attn_prefill(q, K, V, idx, out=O, workspace=ws, Bk=w.Bk)
        if evs is not None:
            evs[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[ev(), ev(), ev()] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    sel = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    att = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    del ws, ws_sel
    wall1, equal = time_one_call(w, inp, idx, O, steps, warmup)
    fl = acc.prefill_flops(w)
    tf = fl["total"] / wall1 / 1e12
    log("[bench] %s %.3f ms/step in one call, %.1f TFLOP/s (two calls %.3f ms: select %.3f, "
        "attention %.3f)" % (name, wall1 * 1e3, tf, wall * 1e3, sel, att))
    extra = {"cpu_baseline": cpu_full(w, inp)} if cpu else {}
    del inp, qI, kI, q, K, V, idx, O
    torch.cuda.empty_cache()
    return {"workload": name, "steps": steps, "ms_per_step": wall1 * 1e3, "flops": fl["total"],
            "TFLOPs": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
            "one_call_equal_two_calls": equal,
            "two_calls": {"ms_per_step": wall * 1e3, "select_ms": sel, "attention_ms": att,
                          "index_flops": fl["index"], "main_flops": fl["main"],
                          "select_TFLOPs": fl["index"] / (sel * 1e-3) / 1e12,
                          "attention_TFLOPs": fl["main"] / (att * 1e-3) / 1e12}, **extra}


def time_one_call(w, inp, idx_ref, O_ref, steps, warmup):
    """The whole prefill as one msa_prefill call per step (selection and
    attention of successive row windows overlapped on two streams): wall time
    per step between synchronisations, and whether its outputs equal the two
    separate calls' (idx_ref, O_ref)."""
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws1 = torch.empty(max(1, ops.workspace_bytes(ops.OP_PREFILL, d)), dtype=torch.uint8,
                      device="cuda")
    idx1, O1 = torch.empty_like(idx_ref), torch.empty_like(O_ref)

    def one_call():
        ops.prefill(inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"], w.k, out=(idx1, O1),
                    workspace=ws1, Bk=w.Bk)

    for _ in range(max(1, warmup)):
        one_call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_call()
    torch.cuda.synchronize()
    wall1 = (time.perf_counter() - t0) / steps
    equal = bool(torch.equal(idx1, idx_ref) and torch.equal(O1, O_ref))
    del ws1, idx1, O1
    return wall1, equal


def with_block_size(w, args):
    """The workload with --block-size / --k applied (the same token budget by
    default: k = 2048 / Bk)."""
    if args.block_size == w.Bk and args.k is None:
        return w
    k = args.k if args.k is not None else 2048 // args.block_size
    return w.replace(Bk=args.block_size, k=k, name="%s_bk%d" % (w.name, args.block_size))


def prefill_leg(args):
    w = with_block_size(WORKLOADS[args.workload], args)
    log("[bench] generating", w.name)
    inp = make_inputs(w, device="cuda")
    qI, kI, q, K, V = inp["qI"], inp["kI"], inp["q"], inp["K"], inp["V"]
    idx = torch.empty(w.B, w.G, w.T, w.k, dtype=torch.int32, device="cuda")
    O = torch.empty_like(q)
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws = torch.empty(max(1, ops.workspace_bytes(ops.OP_ATTN_PREFILL, d)), dtype=torch.uint8,
                     device="cuda")
    nsel = ops.workspace_bytes(ops.OP_SELECT_BLOCKS, d)
    ws_sel = torch.empty(nsel, dtype=torch.uint8, device="cuda") if nsel else None
    torch.cuda.synchronize()

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        ops.select_blocks(qI, kI, w.k, out=idx, workspace=ws_sel, Bk=w.Bk)
        if evs is not None:
            evs[1].record()
        ops.sparse_attn_prefill(q, K, V, idx, out=O, workspace=ws, Bk=w.Bk)
        if evs is not None:
            evs[2].record()

    log("[bench] warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] timing", args.steps, "steps")
    events = [[ev(), ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    att_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    fl = acc.prefill_flops(w)
    res = dict(w=w, inp=inp, idx=idx, O=O, wall=wall, sel_ms=sel_ms, att_ms=att_ms, flops=fl)
    log("[bench] prefill %.3f ms/step (select %.3f, attention %.3f)"
        % (1e3 * wall / args.steps, sel_ms.mean(), att_ms.mean()))
    # the same steps again with the library timing each kernel launch
    res["kernels"] = kernel_times(step, args.steps)
    log("[bench] per kernel:", {k: round(v["ms_per_step"], 3) for k, v in res["kernels"].items()
                                if isinstance(v, dict)})
    # the headline step: the same work as one call (msa_prefill)
    del ws, ws_sel
    wall1, res["one_call_equal"] = time_one_call(w, inp, idx, O, args.steps, args.warmup)
    res["wall1"] = wall1 * args.steps
    log("[bench] prefill, one call: %.3f ms/step (outputs equal to the two calls: %s)"
        % (1e3 * wall1, res["one_call_equal"]))
    return res


def backward_leg(args, pre):
    """Stage-4 backward (msa_sparse_attn_backward) on the prefill leg's
    inputs and selection, with O and lse from the forward and a seeded dO;
    timed with events on the launch stream."""
    from msa_inputs import make_grad_output
    w, inp, idx = pre["w"], pre["inp"], pre["idx"]
    q, K, V = inp["q"], inp["K"], inp["V"]
    O, lse = ops.sparse_attn_prefill(q, K, V, idx, return_lse=True, Bk=w.Bk)
    dO = make_grad_output(w, device="cuda")
    outs = (torch.empty(q.shape, dtype=torch.float32, device="cuda"),
            torch.empty(K.shape, dtype=torch.float32, device="cuda"),
            torch.empty(K.shape, dtype=torch.float32, device="cuda"))
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws = torch.empty(ops.workspace_bytes(ops.OP_ATTN_BACKWARD, d), dtype=torch.uint8,
                     device="cuda")
    for _ in range(max(1, args.warmup)):
        ops.sparse_attn_backward(q, K, V, idx, O, lse, dO, out=outs, workspace=ws, Bk=w.Bk)
    torch.cuda.synchronize()
    events = [(ev(), ev()) for _ in range(args.steps)]
    for e0, e1 in events:
        e0.record()
        ops.sparse_attn_backward(q, K, V, idx, O, lse, dO, out=outs, workspace=ws, Bk=w.Bk)
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in events])
    fl = acc.backward_flops(w.N, w.T, w.Hq, w.d_h, w.Bk, w.k, w.B)
    tf = fl / (ms.mean() * 1e-3) / 1e12
    log("[bench] backward %.3f ms (%.1f TFLOP/s)" % (ms.mean(), tf))
    return {"workload": w.name, "Bk": w.Bk, "k": w.k, "ms": float(ms.mean()),
            "ms_min": float(ms.min()), "flops": fl, "TFLOPs": tf,
            "frac_bf16_peak": tf / PEAK_BF16_TFLOPS, "outputs": "dq, dK, dV fp32"}


def index_kl_leg(args, pre):
    """Index-branch KL alignment backward (msa_index_kl_backward) on the
    prefill leg's inputs, selection and main lse; events on the launch
    stream.  Work: the teacher's main scores for every head (2 d_h FLOP per
    (row, head, support key)) plus the index scores twice (proxy lse, then
    the gradient pass) and the two gradient products (2 d_I FLOP each per
    (row, group, support key))."""
    w, inp, idx = pre["w"], pre["inp"], pre["idx"]
    _, lse = ops.sparse_attn_prefill(inp["q"], inp["K"], inp["V"], idx, return_lse=True, Bk=w.Bk)
    outs = (torch.empty(inp["qI"].shape, dtype=torch.float32, device="cuda"),
            torch.empty(inp["kI"].shape, dtype=torch.float32, device="cuda"))
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws = torch.empty(ops.workspace_bytes(ops.OP_INDEX_KL_BACKWARD, d), dtype=torch.uint8,
                     device="cuda")
    call = lambda: ops.index_kl_backward(inp["qI"], inp["kI"], inp["q"], inp["K"], idx, lse,
                                         out=outs, workspace=ws, Bk=w.Bk)
    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    events = [(ev(), ev()) for _ in range(args.steps)]
    for e0, e1 in events:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in events])
    fl = acc.index_kl_flops(w.N, w.T, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k, w.B)
    tf = fl / (ms.mean() * 1e-3) / 1e12
    log("[bench] index KL backward %.3f ms (%.1f TFLOP/s)" % (ms.mean(), tf))
    return {"workload": w.name, "Bk": w.Bk, "k": w.k, "ms": float(ms.mean()),
            "ms_min": float(ms.min()), "flops": fl, "TFLOPs": tf,
            "frac_bf16_peak": tf / PEAK_BF16_TFLOPS, "outputs": "dqI, dkI fp32"}


def train_leg(args, pre):
    """Both training backwards in one call (msa_train_backward) on the same
    inputs as the two legs above; events on the launch stream.  Work: the
    stage-4 backward's five products plus the index branch's four (the
    teacher is the backward's own weights)."""
    from msa_inputs import make_grad_output
    w, inp, idx = pre["w"], pre["inp"], pre["idx"]
    q, K, V = inp["q"], inp["K"], inp["V"]
    O, lse = ops.sparse_attn_prefill(q, K, V, idx, return_lse=True, Bk=w.Bk)
    dO = make_grad_output(w, device="cuda")
    outs = (torch.empty(q.shape, dtype=torch.float32, device="cuda"),
            torch.empty(K.shape, dtype=torch.float32, device="cuda"),
            torch.empty(K.shape, dtype=torch.float32, device="cuda"),
            torch.empty(inp["qI"].shape, dtype=torch.float32, device="cuda"),
            torch.empty(inp["kI"].shape, dtype=torch.float32, device="cuda"))
    d = ops.dims(w.B, w.T, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws = torch.empty(ops.workspace_bytes(ops.OP_TRAIN_BACKWARD, d), dtype=torch.uint8,
                     device="cuda")
    call = lambda: ops.train_backward(q, K, V, inp["qI"], inp["kI"], idx, O, lse, dO, out=outs,
                                      workspace=ws, Bk=w.Bk)
    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    events = [(ev(), ev()) for _ in range(args.steps)]
    for e0, e1 in events:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in events])
    fl = acc.train_flops(w.N, w.T, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k, w.B)
    tf = fl / (ms.mean() * 1e-3) / 1e12
    log("[bench] fused training backward %.3f ms (%.1f TFLOP/s)" % (ms.mean(), tf))
    return {"workload": w.name, "Bk": w.Bk, "k": w.k, "ms": float(ms.mean()),
            "ms_min": float(ms.min()), "flops": fl, "TFLOPs": tf,
            "frac_bf16_peak": tf / PEAK_BF16_TFLOPS,
            "outputs": "dq, dK, dV, dqI, dkI fp32"}


def topk_leg(args, pre):
    """Stage 3 alone on materialised scores of the same workload."""
    w, inp = pre["w"], pre["inp"]
    S = ops.index_scores(inp["qI"], inp["kI"])
    idx = torch.empty(w.B, w.G, w.T, w.k, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(2):
        ops.select_blocks_from_scores(S, w.k, w.N, out=idx)
    evs = [(ev(), ev()) for _ in range(args.topk_reps)]
    for a, b in evs:
        a.record()
        ops.select_blocks_from_scores(S, w.k, w.N, out=idx)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    same = bool(torch.equal(idx, pre["idx"]))
    kt = kernel_times(lambda: ops.select_blocks_from_scores(S, w.k, w.N, out=idx),
                      args.topk_reps)
    # torch.topk over the same rows, as context only (full rows, no local rule)
    tk = []
    for _ in range(3):
        a, b = ev(), ev()
        a.record()
        torch.topk(S, w.k - 1, dim=-1)
        b.record()
        torch.cuda.synchronize()
        tk.append(a.elapsed_time(b) * 1e3)
    del S
    torch.cuda.empty_cache()
    by = acc.topk_bytes(w)
    med = float(np.median(us))
    # the launch's kernel: two rows per wave for rows of at most 1024 blocks
    # and k <= 16, else one row per wave
    nb = (w.N + w.Bk - 1) // w.Bk
    kname = "topk_pair_kernel" if (w.k <= 16 and nb <= 1024) else "topk_rows_kernel"
    return {"workload": w.name, "rows": w.B * w.G * w.T, "us_p50": med,
            "us_p95": float(np.percentile(us, 95)), "bytes": by["total"],
            "GBps": by["total"] / med / 1e3, "frac_hbm": by["total"] / med / 1e3 / PEAK_HBM_GBS,
            "matches_fused_select": same, "torch_topk_us": float(np.median(tk)),
            "roofline": roof(kname, "hbm",
                             by["total"] / (kt["topk"]["avg_launch_ms"] * 1e-3) / 1e9,
                             PEAK_HBM_GBS, "GB/s", counter_traffic(kname),
                             bytes_per_launch=by["total"],
                             avg_launch_ms=kt["topk"]["avg_launch_ms"])}


def fp8_leg(args, pre):
    """The index branch on 8-bit (E4M3) q^I / k^I: the fused select alone on the
    same prefill workload (its selection must equal the bf16 one: the inputs
    are integers, exact in both formats), and the step with it."""
    w, inp = pre["w"], pre["inp"]
    q8 = inp["qI"].float().to(torch.float8_e4m3fn)
    k8 = inp["kI"].float().to(torch.float8_e4m3fn)
    idx = torch.empty_like(pre["idx"])
    for _ in range(2):
        ops.select_blocks(q8, k8, w.k, out=idx)
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        ops.select_blocks(q8, k8, w.k, out=idx)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    same = bool(torch.equal(idx, pre["idx"]))
    fl = acc.prefill_flops(w)
    att = float(pre["att_ms"].mean())
    step = ms + att
    ach = fl["index"] / (ms * 1e-3) / 1e12
    del q8, k8
    return {"select_ms": ms, "select_TFLOPs": ach,
            "roofline": {"kernel": "index_tile_kernel (fp8 inputs)", "bound": "mfma",
                         "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / PEAK_FP8_TFLOPS},
            "matches_bf16_selection": same,
            "step_ms": step, "step_TFLOPs": fl["total"] / (step * 1e-3) / 1e12,
            "note": "step = fp8 select + the bf16 attention of the same run"}


def decode_leg(args, fp8=False, cpu=False):
    w = WORKLOADS["decode_256k_b16"]
    if not fp8:  # the fp8 index calls take 128-key blocks
        w = with_block_size(w, args)
    log("[bench] generating", w.name, "(fp8 index keys)" if fp8 else "")
    inp = make_inputs(w, device="cuda")
    qI, kI, K, V = inp["qI"], inp["kI"], inp["K"], inp["V"]
    if fp8:
        qI = qI.float().to(torch.float8_e4m3fn)
        kI = kI.float().to(torch.float8_e4m3fn)
        inp["qI"], inp["kI"] = qI, kI
    q = inp["q"][:, 0].contiguous()
    idx = torch.empty(w.B, w.G, 1, w.k, dtype=torch.int32, device="cuda")
    O = torch.empty_like(q)
    d = ops.dims(w.B, 1, w.N, w.Hq, w.G, w.k, Bk=w.Bk)
    ws_s = torch.empty(ops.workspace_bytes(ops.OP_SELECT_BLOCKS, d), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(ops.workspace_bytes(ops.OP_ATTN_DECODE, d), dtype=torch.uint8,
                       device="cuda")
    # a 1 GiB read evicts the 256 MB last-level cache and leaves it clean (a
    # write flush would leave dirty lines whose write-back lands in the step)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def two_calls():
        ops.select_blocks(qI, kI, w.k, out=idx, workspace=ws_s, Bk=w.Bk)
        ops.sparse_attn_decode(q, K, V, idx, out=O, workspace=ws_a, Bk=w.Bk)

    # the step as one msa_decode (msa_decode_fp8) call
    idx1, O1 = torch.empty_like(idx), torch.empty_like(O)
    ws_1 = torch.empty(ops.workspace_bytes(ops.OP_DECODE, d), dtype=torch.uint8, device="cuda")

    def one_call():
        ops.decode(qI, kI, q, K, V, w.k, out=(idx1, O1), workspace=ws_1, Bk=w.Bk)

    def timed(step):
        for _ in range(3):
            step()
        times = []
        for _ in range(args.decode_reps):
            torch.sum(flush, dim=0, out=sink)
            a, b = ev(), ev()
            a.record()
            step()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        return np.array(times)

    us2 = timed(two_calls)
    us = timed(one_call)
    by = acc.decode_bytes(w, index_bytes=1 if fp8 else 2)
    med = float(np.median(us))
    out = {"workload": w.name, "us_p50": med, "us_p95": float(np.percentile(us, 95)),
           "bytes": by["total"], "GBps": by["total"] / med / 1e3,
           "frac_hbm": by["total"] / med / 1e3 / PEAK_HBM_GBS,
           "step": ("one msa_decode%s call: index-key scan, then one workgroup per (sequence, "
                    "group) selecting, attending and merging its blocks" % ("_fp8" if fp8 else "")),
           "note": "last-level cache flushed before each step"}
    out["two_calls"] = {"us_p50": float(np.median(us2)),
                        "GBps": by["total"] / float(np.median(us2)) / 1e3,
                        "calls": "msa_select_blocks%s, then msa_sparse_attn_decode"
                                 % ("_fp8" if fp8 else ""),
                        "idx_equal": bool(torch.equal(idx1, idx)),
                        "O_max_abs_diff": float((O1.float() - O.float()).abs().max())}
    kt = kernel_times(one_call, args.decode_reps,
                      between=lambda: torch.sum(flush, dim=0, out=sink))
    out["kernel_us_per_step"] = {k: v["ms_per_step"] * 1e3 for k, v in kt.items()
                                 if isinstance(v, dict)}
    if "decode_scan" in kt:
        sc = kt["decode_scan"]["avg_launch_ms"]
        ach = by["index_keys"] / (sc * 1e-3) / 1e9
        out["roofline"] = roof("decode_scan_kernel<%s, %d> (stages 1-2: index-key scan)"
                               % ("true" if fp8 else "false", w.Bk), "hbm", ach, PEAK_HBM_GBS,
                               "GB/s", counter_traffic("decode_scan_kernel<%s, %d>"
                                                       % ("true" if fp8 else "false", w.Bk)),
                               bytes_per_launch=by["index_keys"], avg_launch_ms=sc)
    if "decode_attn" in kt:
        da = kt["decode_attn"]["avg_launch_ms"]
        ach = by["kv"] / (da * 1e-3) / 1e9
        out["roofline_attention"] = roof(
            "decode_attn_kernel<%d> (stage 4: selected K/V blocks)" % (w.Hq // w.G), "hbm", ach,
            PEAK_HBM_GBS, "GB/s", counter_traffic("decode_attn_kernel<%d>" % (w.Hq // w.G)),
            bytes_per_launch=by["kv"], avg_launch_ms=da)
    if "decode_step" in kt:
        da = kt["decode_step"]["avg_launch_ms"]
        ach = by["kv"] / (da * 1e-3) / 1e9
        parts = 2 if w.B * w.G < 256 else 1  # workgroups per (sequence, group) row
        name = "decode_step_kernel<%d, %d>" % (w.Hq // w.G, parts)
        out["roofline_attention"] = roof(
            name + " (stages 3-4: selection, selected K/V blocks, merge; with its merge kernel)",
            "hbm", ach, PEAK_HBM_GBS, "GB/s", counter_traffic(name),
            bytes_per_launch=by["kv"], avg_launch_ms=da)
    if cpu and not fp8:
        out["cpu_baseline"] = cpu_full(w, inp)
    del inp, flush
    torch.cuda.empty_cache()
    return out


def cpu_leg(args, pre):
    """The oracle as it stands, on host cores, on a bounded sample of rows of
    the same workload; scaled to TFLOP/s by the sample's algorithmic FLOPs."""
    import oracle
    w, inp = pre["w"], pre["inp"]
    d = oracle.dims_of(w.B, w.T, w.N, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)
    kI = inp["kI"].cpu()
    K = inp["K"].cpu()
    V = inp["V"].cpu()

    def run(nrows, seed):
        rb, rt = sample_rows(w, nrows, seed=seed)
        rbd, rtd = rb.cuda(), rt.cuda()
        qI_rows = inp["qI"][rbd, rtd].cpu()
        q_rows = inp["q"][rbd, rtd].cpu()
        t0 = time.perf_counter()
        ref = oracle.forward(d, rb.numpy(), rt.numpy(), qI_rows, kI, q_rows, K, V)
        sec = time.perf_counter() - t0
        p = (w.N - w.T) + rt.numpy()
        L = p // w.Bk
        nsel = np.minimum(L, w.k - 1) * w.Bk + p % w.Bk + 1
        flops = float((2 * w.G * w.d_I * (p + 1) + 4 * w.Hq * w.d_h * nsel).sum())
        return rb, rt, ref, sec, flops

    _, _, _, sec0, fl0 = run(16, 1)
    rate = fl0 / max(sec0, 1e-6)
    target = args.cpu_seconds
    n = int(min(4096, max(32, 16 * target / max(sec0, 1e-3))))
    log("[bench] cpu oracle: %d rows (probe %.2fs for 16 rows)" % (n, sec0))
    rb, rt, ref, sec, fl = run(n, 2)
    # parity of the same rows while we have them
    idx = pre["idx"]
    got = idx.permute(0, 2, 1, 3)[rb.cuda(), rt.cuda()].cpu().numpy()
    O = pre["O"][rb.cuda(), rt.cuda()].float().cpu().numpy()
    err = np.abs(O - ref["O"])
    parity = {"rows": int(n), "idx_exact": bool(np.array_equal(got, ref["idx"])),
              "O_max_abs": float(err.max()), "O_mean_abs": float(err.mean())}
    del rate
    model, _ = cpu_model()
    return {"value": fl / sec / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "cpu_model": model, "kind": "oracle", "seconds": sec,
            "sample": "%d query rows (all %d groups, %d heads) of %s: edge positions plus "
                      "uniform rows; fp64 plain C, OpenMP over rows" % (n, w.G, w.Hq, w.name)}, parity


def cpu_full(w, inp):
    """The oracle on every row of a small workload (the 2K prefill, the 256K x
    16 decode step) from host copies of its inputs."""
    import oracle
    model, _ = cpu_model()
    d = oracle.dims_of(w.B, w.T, w.N, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)
    rb = np.repeat(np.arange(w.B), w.T)
    rt = np.tile(np.arange(w.T), w.B)
    host = {k: inp[k].cpu() for k in ("qI", "kI", "q", "K", "V")}
    t0 = time.perf_counter()
    oracle.forward(d, rb, rt, host["qI"][rb, rt], host["kI"], host["q"][rb, rt], host["K"],
                   host["V"])
    sec = time.perf_counter() - t0
    if w.T == 1:
        val, unit = acc.decode_bytes(w)["total"] / sec / 1e9, "GB/s"
    else:
        val, unit = acc.prefill_flops(w)["total"] / sec / 1e12, "TFLOP/s"
    log("[bench] cpu oracle, every row of %s: %.2f s" % (w.name, sec))
    return {"value": val, "unit": unit, "seconds": sec, "cores": oracle.threads(),
            "cpu_model": model, "kind": "oracle",
            "sample": "every row (%d) of %s; fp64 plain C, OpenMP over rows" % (rb.size, w.name)}


def cpu_train_leg(args, pre):
    """The oracle's two backward functions, as they stand, on host cores, on
    a bounded sample of rows of the prefill workload (their selection from
    the oracle's own stages 1-3, outside the timed region); scaled to
    TFLOP/s by the sample's algorithmic FLOPs (the accounting of the GPU
    legs).  dK / dV and dk^I are accumulated for an 8-block window."""
    import oracle
    from msa_inputs import make_grad_output
    w, inp = pre["w"], pre["inp"]
    d = oracle.dims_of(w.B, w.T, w.N, w.Hq, w.G, w.d_h, w.d_I, w.Bk, w.k)
    kI, K, V = inp["kI"].cpu(), inp["K"].cpu(), inp["V"].cpu()
    dO = make_grad_output(w, device="cuda")
    out = {}
    for leg in ("backward", "index_kl_backward"):
        n = 16
        while True:
            rb, rt = sample_rows(w, n, seed=5)
            rbd, rtd = rb.cuda(), rt.cuda()
            S = oracle.block_scores(d, rb.numpy(), rt.numpy(), inp["qI"][rbd, rtd].cpu(), kI)
            idx = oracle.select(d, rt.numpy(), S)
            q_rows = inp["q"][rbd, rtd].cpu()
            t0 = time.perf_counter()
            if leg == "backward":
                oracle.attend_backward(d, rb.numpy(), rt.numpy(), q_rows, dO[rbd, rtd].cpu(), K,
                                       V, idx, blk_lo=w.NB - 8, nblk=8)
            else:
                oracle.index_kl_backward(d, rb.numpy(), rt.numpy(), inp["qI"][rbd, rtd].cpu(), kI,
                                         q_rows, K, idx, blk_lo=w.NB - 8, nblk=8)
            sec = time.perf_counter() - t0
            if sec * 2 > args.cpu_seconds / 3 or n >= 4096:
                break
            n = int(min(4096, max(2 * n, n * (args.cpu_seconds / 3) / max(sec, 1e-3))))
        p = (w.N - w.T) + rt.numpy()
        nsel = np.minimum(p // w.Bk, w.k - 1) * w.Bk + p % w.Bk + 1
        if leg == "backward":
            fl = float(10 * w.Hq * w.d_h * nsel.sum())
        else:
            fl = float((2 * w.Hq * w.d_h + 8 * w.G * w.d_I) * nsel.sum())
        log("[bench] cpu oracle %s: %d rows, %.2fs" % (leg, len(rb), sec))
        out[leg] = {"value": fl / sec / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
                    "kind": "oracle", "seconds": sec,
                    "sample": "%d query rows (all %d groups, %d heads) of %s; fp64 plain C, "
                              "OpenMP" % (len(rb), w.G, w.Hq, w.name)}
    # the fused call's work done by the oracle's two functions: per support
    # key, its FLOPs over the sum of the two functions' times for theirs
    fb, fk = 10 * w.Hq * w.d_h, 2 * w.Hq * w.d_h + 8 * w.G * w.d_I
    ft = 10 * w.Hq * w.d_h + 8 * w.G * w.d_I
    rate = ft / (fb / out["backward"]["value"] + fk / out["index_kl_backward"]["value"])
    out["train_backward"] = {"value": rate, "unit": "TFLOP/s", "cores": oracle.threads(),
                             "kind": "oracle",
                             "sample": "the two samples above: the oracle's backward and "
                                       "index KL functions' times per support key, added"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--only", default="",
                    help="prefill | decode | topk | fp8 | backward | configs (skip the other legs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--decode-reps", type=int, default=30)
    ap.add_argument("--block-size", type=int, default=128, choices=(32, 64, 128),
                    help="Bk of the prefill and bf16 decode legs (default 128)")
    ap.add_argument("--k", type=int, default=None,
                    help="blocks per query and group (default: 2048 / block size)")
    ap.add_argument("--topk-reps", type=int, default=10)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 2K, 32K and 1M prefill legs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if "RANK" in os.environ and int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is single-GPU only", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    ops.lib()
    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": src.numel() * 4}))
        return

    out = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if args.only in ("", "prefill", "topk", "fp8", "backward"):
        pre = prefill_leg(args)
        w = pre["w"]
        fl = pre["flops"]
        ms2 = 1e3 * pre["wall"] / args.steps
        ms = 1e3 * pre["wall1"] / args.steps
        sel = float(pre["sel_ms"].mean())
        att = float(pre["att_ms"].mean())
        out.update({"value": fl["total"] / (ms * 1e-3) / 1e12, "ms_per_step": ms})
        out["config"] = {"workload": w.name, "B": w.B, "N": w.N, "T": w.T, "Hq": w.Hq,
                         "G": w.G, "d_h": w.d_h, "d_I": w.d_I, "Bk": w.Bk, "k": w.k,
                         "needles": w.needles, "seed": w.seed}
        fused = w.Bk == 128
        kt = pre["kernels"]
        s4 = acc.stage4_bytes(w)
        pb = acc.partial_bytes(w)
        rl = []
        if "kv_outer" in kt:
            ko = kt["kv_outer"]
            n = ko["launches_per_step"]
            ach = fl["main"] / (ko["ms_per_step"] * 1e-3) / 1e12
            rl.append(roof("kv_outer_kernel<%d, %d> (stage 4 KV-outer attention, one launch per "
                           "stage of rows and group)" % (w.Hq // w.G, w.Bk // 32), "mfma", ach,
                           PEAK_BF16_TFLOPS, "TFLOP/s",
                           counter_traffic("kv_outer_kernel<%d, %d>" % (w.Hq // w.G, w.Bk // 32)),
                           flops_per_launch=fl["main"] / n, avg_launch_ms=ko["avg_launch_ms"],
                           launches_per_step=n, ms_per_step=ko["ms_per_step"],
                           algorithmic_stage4_bytes=s4["total"],
                           partial_bytes_written=pb["partials"] / n))
        sel_k = kt.get("select")
        sel_avg = sel_k["avg_launch_ms"] if sel_k else sel
        ach_s = fl["index"] / (sel_k["ms_per_step"] if sel_k else sel) / 1e9
        rl.append(roof("index_tile_kernel (fused select: scores, block max, top-k)" if fused else
                       "index_tile_kernel (block scores, written) + top-k kernel, window "
                       "after window", "mfma", ach_s, PEAK_BF16_TFLOPS, "TFLOP/s",
                       counter_traffic("index_tile_kernel<8, 15, false, false, 128>")
                       if fused and w.G == 8 else None,
                       flops_per_launch=fl["index"], avg_launch_ms=sel_avg,
                       ms_per_step=sel_k["ms_per_step"] if sel_k else sel))
        if "combine" in kt:
            co = kt["combine"]
            ach_c = pb["combine"] / (co["ms_per_step"] * 1e-3) / 1e9
            rl.append(roof("combine_kernel<%d, false> (stage 4 partial combine)" % (w.Hq // w.G),
                           "hbm", ach_c, PEAK_HBM_GBS, "GB/s",
                           counter_traffic("combine_kernel<%d, false>" % (w.Hq // w.G)),
                           bytes_per_launch=pb["combine"] / co["launches_per_step"],
                           bytes_note="the KV-outer schedule's partials read once, idx read, "
                                      "O and lse written",
                           avg_launch_ms=co["avg_launch_ms"],
                           launches_per_step=co["launches_per_step"],
                           ms_per_step=co["ms_per_step"]))
        # the kernel that takes the most time per step
        out["roofline"] = max(rl, key=lambda r: r["ms_per_step"])
        out["rooflines"] = rl
        out["kernel_ms_per_step"] = {k: v["ms_per_step"] for k, v in kt.items()
                                     if isinstance(v, dict)}
        out["kernel_timing_note"] = ("per-kernel times: HIP events the library records on each "
                                     "launch's stream over %d more steps of the two calls "
                                     "(%.3f ms per step with the events)"
                                     % (args.steps, kt["wall_ms_per_step"]))
        out["step"] = ("one msa_prefill call: fused select and KV-outer attention of "
                       "successive row windows overlapped on two streams")
        out["two_calls"] = {"ms_per_step": ms2, "TFLOPs": fl["total"] / (ms2 * 1e-3) / 1e12,
                            "one_call_outputs_equal": pre["one_call_equal"],
                            "calls": "msa_select_blocks, then msa_sparse_attn_prefill"}
        out["stages"] = {"select_ms": sel, "attention_ms": att,
                         "attention_TFLOPs": fl["main"] / (att * 1e-3) / 1e12,
                         "index_flops": fl["index"], "main_flops": fl["main"]}
        if not fused:
            log("[bench] Bk = %d: the top-k, fp8 and CPU legs run at Bk = 128 only" % w.Bk)
        if args.only in ("", "topk") and fused:
            log("[bench] top-k leg")
            out["topk"] = topk_leg(args, pre)
        if args.only in ("", "fp8") and fused:
            log("[bench] fp8 index leg")
            out["fp8_index"] = fp8_leg(args, pre)
        if args.only in ("", "backward"):
            log("[bench] backward leg")
            out["backward"] = backward_leg(args, pre)
            log("[bench] index KL backward leg")
            out["index_kl_backward"] = index_kl_leg(args, pre)
            log("[bench] fused training backward leg")
            out["train_backward"] = train_leg(args, pre)
        if not args.no_cpu and args.only == "" and fused:
            log("[bench] cpu baseline")
            out["cpu_baseline"], out["parity_sample"] = cpu_leg(args, pre)
            log("[bench] cpu baseline of the backward calls")
            cb = cpu_train_leg(args, pre)
            out["backward"]["cpu_baseline"] = cb["backward"]
            out["index_kl_backward"]["cpu_baseline"] = cb["index_kl_backward"]
            out["train_backward"]["cpu_baseline"] = cb["train_backward"]
        del pre
        torch.cuda.empty_cache()
    if args.only in ("", "configs") and not args.no_configs and args.block_size == 128 \
            and args.k is None:
        out["prefill_configs"] = [config_leg("prefill_2k", max(args.steps, 20), args.warmup,
                                             cpu=not args.no_cpu),
                                  config_leg("prefill_32k", args.steps, args.warmup),
                                  config_leg("prefill_1m", 3, 1)]
    if args.only in ("", "decode"):
        log("[bench] decode leg")
        out["decode"] = decode_leg(args, cpu=not args.no_cpu and args.only == "")
        out["decode_fp8_index"] = decode_leg(args, fp8=True)
        if args.only == "decode":
            out.update({"value": out["decode"]["GBps"], "unit": "GB/s",
                        "ms_per_step": out["decode"]["us_p50"] / 1e3,
                        "config": {"workload": out["decode"]["workload"]}})
    print(json.dumps(out))


if __name__ == "__main__":
    main()
