"""Benchmark: MonarchAttention layer calls on one MI355X.

Default (--mode fwd): one step = one full forward call (block-mean keys,
T x (L-step, R-step), L-apply) over one batch of seeded synthetic Q/K/V
already resident in HBM.  --mode train: one step = the training forward
(which keeps its state; the workload's iteration count, one for the 720p
latent, or --iters) plus the backward pass for a seeded upstream gradient
(dq, dk, dv).  Prints ONE JSON line with tokens/s (value),
layer-calls/s, the roofline of the dominant kernel (timed with HIP events on
the launch stream inside the timed region) and the CPU oracle timed on a
bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload latent720p] [--mode fwd|train]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MonarchAttention fwd tokens/s & layer-calls/s at 1 MI355X; % MFMA/HBM roofline"
METRIC_TRAIN = ("MonarchAttention {iters}-iteration training step (fwd + bwd) tokens/s at 1 MI355X; "
                "% MFMA/HBM roofline")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# every kernel source (headers and the library's translation unit), in a fixed order
KERNEL_SOURCES = sorted(os.path.relpath(p, ROOT) for p in
                        glob.glob(os.path.join(ROOT, "structured_attention_video_monarch_amd", "csrc", "*"))
                        if p.endswith((".h", ".hip")))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(wl):
    """Per launch: (flops, bytes) each kernel must do by the method's definition.

    flops: the method's own products, per (batch, head), e = element bytes,
    N = b1*b2 key tokens, Nq query tokens (N for the square layer):
      k_kbar       0
      k_lse        2*Nq*b1*d    (L logits)
      k_aggregate  2*Nq*b1*d    (L^T q per tile)
      k_rstep      4*t*N*b2*d   (R logits + R V)
      k_apply      2*Nq*b1*d    (L U)
    Logit recomputation in k_aggregate/k_apply and padding are not counted.
    bytes: only the layer's own tensors (q, k, v, out; in training also dy,
    dq, dk, dv) that the kernel must read or write, each once:
      k_kbar K; k_lse Q; k_aggregate Q; k_rstep K, V; k_apply Q, O.
    The implementation's intermediates (block-mean keys, log-sum-exps,
    aggregated queries Qh, U = R V, next keys and entropies, and the
    backward's) are not algorithmic bytes; ``intermediate_bytes`` models the
    forward's, and the rocprofv3 counters measure all of them.
    """
    e = 2 if wl.dtype == "bf16" else 4
    BH, N, d, b1, b2, t = wl.B * wl.H, wl.N, wl.d, wl.b1, wl.b2, wl.tiles
    Nq = wl.Nq   # query tokens (== N for the square layer; a chunk against cached keys has fewer)
    nd, nqd = N * d * e, Nq * d * e
    return {
        "k_kbar": (0.0, BH * nd),
        "k_lse": (BH * 2.0 * Nq * b1 * d, BH * nqd),
        "k_aggregate": (BH * 2.0 * Nq * b1 * d, BH * nqd),
        "k_rstep": (BH * 4.0 * t * N * b2 * d, BH * 2 * nd),
        "k_apply": (BH * 2.0 * Nq * b1 * d, BH * 2 * nqd),
        # backward (the one-iteration form), chain-rule products only (no logit
        # recomputation, no stored s*dl), per (batch, head); the row side
        # has the Nq query tokens, the key side t*N rows (tile, key block, a2):
        #   kb_du       dU = L^T dy                      2 Nq b1 d;  q, dy
        #   kb_rside_a  dR = dU v^T, dQh = dz k          4 t N b2 d; k, v
        #   kb_dq       <dy,U>, <q,G>, L G, dl Kbar      8 Nq b1 d;  q, dy, y in, dq out
        #   kb_dkbar    dKbar = dl^T q                   2 Nq b1 d;  q
        #   kb_rside_b  dv = R^T dU, dk_R = dz^T Qh      4 t N b2 d; k, v in, dk, dv out
        "kb_du": (BH * 2.0 * Nq * b1 * d, BH * 2 * nqd),
        "kb_rside_a": (BH * 4.0 * t * N * b2 * d, BH * 2 * nd),
        "kb_dq": (BH * 8.0 * Nq * b1 * d, BH * 4 * nqd),
        "kb_dkbar": (BH * 2.0 * Nq * b1 * d, BH * nqd),
        "kb_dkbar_reduce": (0.0, 0.0),
        "kb_rside_b": (BH * 4.0 * t * N * b2 * d, BH * 4 * nd),
        # early stopping: the objective per head reads only log-sum-exps
        "k_objective": (0.0, 0.0),
    }


def intermediate_bytes(wl):
    """Per launch of each forward kernel (one-iteration form): the bytes of
    the implementation's intermediates it reads or writes, per (batch, head),
    e = element bytes:
      k_kbar       b1*d*e (block means out)
      k_lse        b1*d*e (block means) + 4*Nq (log-sum-exps out)
      k_aggregate  b1*d*e + 4*Nq + t*N*d*e (Qh out)
      k_rstep      t*N*d*e (Qh in) + t*N*d*e (U out)
      k_apply      b1*d*e + 4*Nq + t*N*d*e (U in)
    """
    e = 2 if wl.dtype == "bf16" else 4
    BH, N, Nq, d, b1, t = wl.B * wl.H, wl.N, wl.Nq, wl.d, wl.b1, wl.tiles
    kb, ls, tnd = b1 * d * e, 4 * Nq, t * N * d * e
    return {"k_kbar": BH * kb, "k_lse": BH * (kb + ls), "k_aggregate": BH * (kb + ls + tnd),
            "k_rstep": BH * 2 * tnd, "k_apply": BH * (kb + ls + tnd)}


def step_work(wl, mode, launches):
    """Per step: (flops, bytes) of each kernel, summed over its launches.

    The forward kernels and the one-iteration backward do the same work at
    every launch (algorithmic_work x launches), except that with T >= 2 only
    the last R-step reads V (the earlier ones form R K).  The backward through
    T >= 2 iterations runs its kernels in two forms, per (batch, head):
      last iteration (once):  kb_du, kb_rside_a, kb_dq, kb_rside_b as above;
      each earlier iteration (T-1 times), with cotangents dKt, dH instead of dU:
        kb_rside_a  dR = dKt k^T, dQh = dz k      4 t N b2 d; k
        kb_dq       <q,G>, L G, dl Kt              6 Nq b1 d; q
        kb_rside_b  dk_R = dz^T Qh + R^T dKt       4 t N b2 d; k
        kb_dktil    dKt, dH of the R-step before   2 Nq b1 d; q   (T-1 launches)
      kb_dkbar and its reduction once, at the first iteration; dq, dk and dv
      are written once.
    """
    per = algorithmic_work(wl)
    tot = {kn: (per[kn][0] * n, per[kn][1] * n) for kn, n in launches.items() if kn in per}
    T = wl.iters
    if T < 2:
        return tot
    e = 2 if wl.dtype == "bf16" else 4
    BH, N, Nq, d, b1, b2, t = wl.B * wl.H, wl.N, wl.Nq, wl.d, wl.b1, wl.b2, wl.tiles
    nd, nqd = N * d * e, Nq * d * e
    m = T - 1
    if "k_rstep" in tot:
        n = launches["k_rstep"]
        tot["k_rstep"] = (tot["k_rstep"][0], BH * (n * nd + nd))
    if mode != "train":
        return tot
    tot["kb_rside_a"] = (BH * 4.0 * t * N * b2 * d * T, BH * (2 * nd + m * nd))
    tot["kb_dq"] = (per["kb_dq"][0] + m * BH * 6.0 * Nq * b1 * d, BH * (4 * nqd + m * nqd))
    tot["kb_rside_b"] = (BH * 4.0 * t * N * b2 * d * T, BH * (4 * nd + m * nd))
    tot["kb_dktil"] = (m * BH * 2.0 * Nq * b1 * d, m * BH * nqd)
    return tot


def roofline_entry(name, flops, nbytes, avg_s, dtype, traffic):
    """Roofline of one kernel from its algorithmic flops and bytes (per
    launch) and its average launch duration: MFMA-bound when its flops take
    longer at peak than its bytes do, else HBM-bound.  ``traffic`` is the
    measured HBM bytes per launch (or None); it is reported with its ratio
    to the algorithmic bytes."""
    peak_f = (PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS) * 1e12
    peak_b = PEAK_HBM_GBS * 1e9
    if flops <= 0 and nbytes <= 0:
        return {"kernel": name, "bound": "none", "achieved": None, "peak": None, "unit": None,
                "frac": None, "traffic": traffic}
    if flops / peak_f >= nbytes / peak_b:
        ach = flops / avg_s / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / (peak_f / 1e12), 4), "traffic": traffic}
    ach = nbytes / avg_s / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, seed, budget_s=30.0):
    """The oracle as it is, on a bounded sample: whole heads, one at a time,
    until about budget_s seconds have passed (at least one head)."""
    import oracle
    from structured_attention_video_monarch_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    done, spent = 0, 0.0
    while done < wl.B * wl.H and (done == 0 or spent < budget_s):
        b, h = divmod(done, wl.H)
        x = I.make_inputs(wl.with_(B=1), seed, heads=[h], want_bits=False)
        t0 = time.perf_counter()
        oracle.monarch_head(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], wl.b1, wl.b2, wl.tiles, wl.iters)
        spent += time.perf_counter() - t0
        done += 1
    per_call = spent / done * wl.B * wl.H
    return {"value": round(wl.B * wl.Nq / per_call, 1), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {wl.B * wl.H} heads of one {wl.name} call, fp64 numpy oracle, "
                      f"{spent:.1f} s; full call extrapolated as heads x per-head time"}


def cpu_baseline_train(wl, seed, budget_s=30.0):
    """The forward and gradient oracles on a bounded sample: whole heads."""
    import oracle
    from structured_attention_video_monarch_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    done, spent = 0, 0.0
    while done < wl.B * wl.H and (done == 0 or spent < budget_s):
        b, h = divmod(done, wl.H)
        x = I.make_inputs(wl.with_(B=1), seed, heads=[h], want_bits=False)
        dy = I.make_cotangent(wl.with_(B=1), seed, heads=[h], want_bits=False)["dy"][0, 0]
        t0 = time.perf_counter()
        oracle.monarch_head(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], wl.b1, wl.b2, wl.tiles, wl.iters)
        oracle.monarch_head_grad(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], dy, wl.b1, wl.b2, wl.tiles, wl.iters)
        spent += time.perf_counter() - t0
        done += 1
    per_call = spent / done * wl.B * wl.H
    return {"value": round(wl.B * wl.Nq / per_call, 1), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {wl.B * wl.H} heads of one {wl.name} training step (forward and "
                      f"gradient oracles, fp64 numpy), {spent:.1f} s; full step extrapolated as "
                      f"heads x per-head time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="latent720p")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--mode", choices=["fwd", "train"], default="fwd",
                    help="fwd: forward layer call; train: training forward + backward")
    ap.add_argument("--iters", type=int, default=0,
                    help="override the workload's iteration count (0: keep it)")
    ap.add_argument("--tol", type=float, default=None,
                    help="iterate until the objective gain per token is <= tol (at most --iters or the "
                         "workload's count; each head stops on its own)")
    ap.add_argument("--graph", action="store_true",
                    help="forward: also capture one call in a HIP graph and report the time per replay "
                         "(the value then comes from the replays; per-kernel figures from the eager run)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (float32 read + write), "
                         "to scale HBM byte counters (FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the forward pass "
              "has no multi-GPU path in this library.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "launches": 3}), flush=True)
        return

    import structured_attention_video_monarch_amd as M
    from structured_attention_video_monarch_amd import inputs as I

    wl = I.get_workload(args.workload)
    if args.iters:
        wl = wl.with_(iters=args.iters)
    dev = torch.device("cuda:0")
    t0 = time.time()
    x = I.make_inputs(wl, args.seed, want_f32=(wl.dtype == "f32"))
    if wl.dtype == "bf16":
        q, k, v = (torch.from_numpy(x[n + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
                   for n in "qkv")
    else:
        q, k, v = (torch.from_numpy(x[n]).to(dev) for n in "qkv")
    del x
    print(f"[bench] inputs {wl.name} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    out = torch.empty_like(q)
    dtc = M.MONARCH_BF16 if wl.dtype == "bf16" else M.MONARCH_F32
    nb = M.monarch_attn_kv_workspace_bytes(wl.B, wl.H, wl.fq or wl.f, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2,
                                           wl.tiles, wl.iters, dtc)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        M.monarch_attn_fwd_ws(q, k, v, out, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters,
                              ws, stream)

    iters_used = None
    if args.tol is not None:
        if args.mode == "train":
            print("bench.py: --tol applies to the forward only", file=sys.stderr)
            sys.exit(2)
        del ws
        iters_used = torch.empty((wl.B, wl.H), dtype=torch.int32, device=dev)
        if wl.kv:
            nb = M.monarch_attn_adaptive_kv_workspace_bytes(wl.B, wl.H, wl.fq, wl.f, wl.h, wl.w, wl.d, wl.b1,
                                                            wl.b2, wl.tiles, wl.iters, dtc)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)

            def step():
                M.monarch_attn_fwd_adaptive_kv(q, k, v, out, wl.fq, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles,
                                               wl.iters, args.tol, iters_used=iters_used, workspace=ws,
                                               stream=stream)
        else:
            nb = M.monarch_attn_adaptive_workspace_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2,
                                                         wl.tiles, wl.iters, dtc)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)

            def step():
                M.monarch_attn_fwd_adaptive(q, k, v, out, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters,
                                            args.tol, iters_used=iters_used, workspace=ws, stream=stream)

    if wl.kv and args.tol is None:
        def step():
            M.monarch_attn_fwd_kv(q, k, v, out, wl.fq, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles,
                                  wl.iters, workspace=ws, stream=stream)

    if args.mode == "train":
        del ws
        dyx = I.make_cotangent(wl, args.seed, want_f32=(wl.dtype == "f32"))
        if wl.dtype == "bf16":
            dy = torch.from_numpy(dyx["dy_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            dy = torch.from_numpy(dyx["dy"]).to(dev)
        del dyx
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        if wl.kv:
            # a chunk of frames against cached keys: the chunk's training step
            sb = M.monarch_attn_train_state_bytes_kv(wl.B, wl.H, wl.fq, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2,
                                                     wl.tiles, wl.iters, dtc)
            state = torch.empty(sb, dtype=torch.uint8, device=dev)
            targs = (wl.fq, wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters)

            def step():
                M.monarch_attn_fwd_train_kv(q, k, v, out, *targs, state, stream)
                M.monarch_attn_bwd_kv(q, k, v, out, dy, dq, dk, dv, *targs, state, stream)
        else:
            sb = M.monarch_attn_train_state_bytes(wl.B, wl.H, wl.f, wl.h, wl.w, wl.d, wl.b1, wl.b2, wl.tiles,
                                                  wl.iters, dtc)
            state = torch.empty(sb, dtype=torch.uint8, device=dev)
            targs = (wl.f, wl.h, wl.w, wl.b1, wl.b2, wl.tiles, wl.iters)

            def step():
                M.monarch_attn_fwd_train(q, k, v, out, *targs, state, stream)
                M.monarch_attn_bwd(q, k, v, out, dy, dq, dk, dv, *targs, state, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    # the headline: K steps with no per-kernel events
    M.monarch_attn_profile_enable(False)
    M.monarch_attn_profile_collect()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    ms_step = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {args.steps} steps, {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    # the per-kernel breakdown: K more steps, HIP events around every launch
    # on the launch stream
    M.monarch_attn_profile_enable(True)
    ev2, ev3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev2.record(stream)
    for _ in range(args.steps):
        step()
    ev3.record(stream)
    torch.cuda.synchronize(dev)
    M.monarch_attn_profile_enable(False)
    per_kernel = M.monarch_attn_profile_collect()
    ms_step_events = ev2.elapsed_time(ev3) / args.steps
    print(f"[bench] {args.steps} steps with per-kernel events, {ms_step_events:.4f} ms/step",
          file=sys.stderr, flush=True)

    graph_rec = None
    if args.graph:
        if args.mode != "fwd" or args.tol is not None:
            print("bench.py: --graph times the forward with a fixed iteration count", file=sys.stderr)
            sys.exit(2)
        # capture on a side stream (the step functions launch on `stream`)
        eager_stream = stream
        stream = torch.cuda.Stream(dev)
        stream.wait_stream(eager_stream)
        with torch.cuda.stream(stream):
            step()  # one call off the capture
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize(dev)
        for _ in range(args.warmup):
            graph.replay()
        cur = torch.cuda.current_stream(dev)
        torch.cuda.synchronize(dev)
        ev0.record(cur)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(cur)
        torch.cuda.synchronize(dev)
        ms_graph = ev0.elapsed_time(ev1) / args.steps
        print(f"[bench] {args.steps} graph replays, {ms_graph:.4f} ms/step", file=sys.stderr, flush=True)
        graph_rec = {"eager_ms_per_step": round(ms_step, 5),
                     "replay_ms_per_step": round(ms_graph, 5)}
        ms_step = ms_graph

    kernels = {}
    for full, (ms, n) in per_kernel.items():
        short = full.split(" ")[0]
        if n:
            kernels[short] = {"avg_ms": round(ms / n, 5), "launches_per_step": n / args.steps,
                              "ms_per_step": round(ms / args.steps, 5)}
    # work per launch: the kernel's work per step over its launches per step
    tot = step_work(wl, args.mode, {kn: rec["launches_per_step"] for kn, rec in kernels.items()})
    work = {kn: (tot[kn][0] / kernels[kn]["launches_per_step"], tot[kn][1] / kernels[kn]["launches_per_step"])
            for kn in kernels}
    dom = max(kernels, key=lambda kname: kernels[kname]["ms_per_step"])
    launches = kernels[dom]["launches_per_step"]
    fl, by = work[dom]
    roof = roofline_entry(dom, fl, by, kernels[dom]["avg_ms"] / 1e3, wl.dtype,
                          # the counters are taken on one-iteration runs: later iterations'
                          # launches read the aggregated keys as well, so they have no figure
                          read_traffic(dom, wl.name) if wl.iters == 1 else None)
    roof["launches_per_step"] = launches
    roof["alg_bytes"] = by
    roof["alg_flops"] = fl
    inter = intermediate_bytes(wl).get(dom) if args.mode == "fwd" and wl.iters == 1 else None
    roof["intermediate_bytes"] = inter
    roof["traffic_over_alg_bytes"] = (round(roof["traffic"] / by, 3)
                                      if roof["traffic"] is not None and by > 0 else None)
    if iters_used is not None:
        roof["note"] = ("early stopping: launches after every head has stopped return at once and are "
                        "counted in the per-launch average")
    for kname, rec in kernels.items():
        f2, b2 = work[kname]
        r = roofline_entry(kname, f2, b2, rec["avg_ms"] / 1e3, wl.dtype, None)
        rec.update({"bound": r["bound"], "frac": r["frac"]})

    total_flops = sum(work[kn][0] * kernels[kn]["launches_per_step"] for kn in kernels)
    res = {
        "metric": METRIC if args.mode == "fwd" else METRIC_TRAIN.format(iters=wl.iters),
        "value": round(wl.B * wl.Nq / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "f": wl.f, "h": wl.h, "w": wl.w,
                   "N": wl.N, "Nq": wl.Nq, "fq": wl.fq or wl.f, "d": wl.d, "b1": wl.b1, "b2": wl.b2,
                   "tiles": wl.tiles,
                   "iters": wl.iters, "spike_frac": wl.spike_frac, "mode": args.mode},
        "early_stop": (None if iters_used is None else
                       {"tol": args.tol, "max_iters": wl.iters,
                        "iters_used_mean": round(float(iters_used.float().mean().item()), 3),
                        "iters_used_max": int(iters_used.max().item())}),
        "layer_calls_per_s": round(1e3 / ms_step, 2),
        "ms_per_step_with_kernel_events": round(ms_step_events, 5),
        "path_alg_tflops": round(total_flops / (ms_step / 1e3) / 1e12, 2),
        "path_frac_of_mfma_peak": round(total_flops / (ms_step / 1e3) / 1e12 /
                                        (PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS), 4),
        "roofline": roof,
        "kernels": kernels,
        "kernel_source_hash": kernel_source_hash(),
    }
    if graph_rec is not None:
        res["graph"] = graph_rec
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = (cpu_baseline(wl, args.seed, args.cpu_budget) if args.mode == "fwd"
                               else cpu_baseline_train(wl, args.seed, args.cpu_budget))
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
