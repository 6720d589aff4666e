#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet + HLA hot path on one MI355X.

Headline: routed GDN+HLA prefill at T = 32768 (B = 1, H = 16, d = 128, C = 64, bf16 inputs,
float32 states), one step = hla_chunk_transitions -> hla_route_mix -> hla_gdn_prefill
(chunk_init = routed states).  Reports tokens/s, whole-step MFMA utilisation, a roofline
record of the dominant kernel (the gated composition) timed with HIP events on its own
stream, and the CPU oracle's throughput on a bounded sample.  Secondary records (same
JSON line): decode step tokens/s with HBM GB/s, native chunkwise prefill, Tail-Replay
state rebuild, the routed prefill's backward pass at T = 8192.  All inputs are seeded synthetic tensors of the workloads' shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]

Hardware counters behind the roofline records come from rocprofv3 passes over one line at a
time (each counter set a run of its own, after a 1 GiB device copy that calibrates
FETCH_SIZE / WRITE_SIZE), summarised into profiles/counters.json with a hash of the kernel
sources; a line reports them only while its sources are unchanged:

    cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o c -- \\
        python3 <repo>/bench.py --counter-run <line>
    (the same with WRITE_SIZE, and for the MFMA lines SQ_INSTS_VALU_MFMA_MOPS_BF16
     SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS GRBM_GUI_ACTIVE)
    python3 bench.py --counter-write <line> <f>/c_counter_collection.csv <w>/c_counter_collection.csv ...

Kernel-time tables (warm-up and timed dispatches apart) come from a kernel trace of
``--only <line>`` through ``--trace-summary``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (GDN+HLA, T=32K) with MFMA util %; decode tokens/s with HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
C = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- FLOP / byte models
def flops_transitions(n_chunks, dk, dv):
    """UT chunk form per 64-token piece: K K^T, the W/U products, the K^T D [W|U] product."""
    return n_chunks * (2 * C * C * dk + 2 * C * C * (dk + dv) + 2 * C * dk * (dk + dv))


def flops_routed_output(n_chunks, dk, dv):
    """Per 64-token piece: Q K^T, P [W|U], Qp S~ (W|U come from the transitions pass)."""
    return n_chunks * (2 * C * C * dk + 2 * C * C * (dk + dv) + 2 * C * dk * dv)


def flops_reps_pool(n_windows, window, dk):
    """Learned representatives, pooling pass, per window: Q, K, V projections of its tokens,
    the in-window scores and P V (the mean over rows is additions)."""
    return n_windows * (3 * 2 * window * dk * dk + 2 * 2 * window * window * dk)


def flops_reps_project(n_windows, dk, with_wr=True):
    return n_windows * 2 * dk * dk * (2 if with_wr else 1)


def flops_gates(pairs, n_rep, dk):
    return pairs * 2 * n_rep * dk


def flops_compose(pairs, dk, dv):
    """One gated composition step: S (dv x dk) times A (dk x dk)."""
    return pairs * 2 * dk * dk * dv


def compose_alg_bytes(n_chunks, W):
    """Algorithmic HBM bytes of one composition launch: every chunk's transition pair
    (At prepared, Bc; bf16) read once, however many query chunks route to it; the gates
    (float32) and mask (byte) of every (query, history) chunk pair read; every routed state
    (float32) written once."""
    e = 2
    n_q = W.B * W.H * n_chunks
    return n_q * (W.dk * W.dk + W.dk * W.dv) * e + n_q * n_chunks * (4 + 1) + n_q * W.dk * W.dv * 4


def sha_of(*paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- helpers
def to_dev(storage, dtype, torch):
    import numpy as np
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(storage, dtype=np.float32)).cuda()


def rel_err(got, ref):
    """max|got - ref| / max|ref| (a comparison of two results, not part of the method)."""
    import numpy as np
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / scale if scale > 0 else float(np.max(np.abs(got)))


def timed_kernels(fn, steps, warmup, torch, hla):
    """timed() with the library's per-kernel HIP-event timing on: (seconds per call, average
    milliseconds per launch of each kernel kind that ran)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    hla.timing_enable(True)
    dt = timed(fn, steps, 0, torch)
    names = (("chunk", hla.KERNEL_CHUNK), ("scan", hla.KERNEL_SCAN), ("prefill", hla.KERNEL_PREFILL),
             ("bwd_reps", hla.KERNEL_BWD_REPS))
    kms = {}
    for name, kid in names:
        ms, n = hla.timing_read(kid)
        if n:
            kms[name] = round(ms / n, 4)
    hla.timing_enable(False)
    return dt, kms


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def gemm_ceiling(torch, n=16384):
    """TFLOP/s of a plain bf16 GEMM (torch.matmul, n x n x n, standard normal operands) on
    the same GPU: what the matrix cores sustain on dense random data under the board's
    power limit, beside the published peak."""
    a = torch.randn(n, n, device="cuda").bfloat16()
    b = torch.randn(n, n, device="cuda").bfloat16()
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del a, b, c
    torch.cuda.empty_cache()
    return dict(op=f"torch.matmul bf16 {n}x{n}x{n}, N(0,1) operands", ms=round(ms, 3),
                tflops=round(2 * n ** 3 / (ms / 1e3) / 1e12, 1))


def kernel_counters(line, kms, kinds):
    """Counter figures of the kernels behind the timed kinds {kind: avg ms} of a line."""
    out = {}
    for kind, kernel in kinds:
        if kind in kms:
            cf = counter_figures(line, kernel, kms[kind] / 1e3)
            if cf:
                out[kernel] = cf
    return out or None


# ----------------------------------------------------------------------------- routed prefill
def bench_routed_prefill(args, torch, hla, inputs, Cw=C, gates_in=None, tau=None, x=None, tag="routed_prefill",
                         handoff=True, pooler=None, window=32):
    """The routed prefill step at chunk size Cw (64-token pieces underneath), with the
    router's computed gates or caller gates; handoff passes W | U from the transitions
    call to the output call.  With ``pooler`` (seeded weights) the step also computes the
    learned window representatives (hla_chunk_reps) that the router scores."""
    W = inputs.WORKLOADS["routed_prefill"]
    tau = W.tau if tau is None else tau
    N = math.ceil(W.T / Cw)
    if x is None:
        x = routed_inputs(inputs)
    q, k, v = (to_dev(a, W.dtype, torch) for a in (x.q, x.k, x.v))
    beta, alpha = to_dev(x.beta, "f32", torch), to_dev(x.alpha, "f32", torch)
    dev = k.device
    At = torch.empty((W.B, W.H, N, W.dk, W.dk), dtype=k.dtype, device=dev)
    Bc = torch.empty((W.B, W.H, N, W.dk, W.dv), dtype=k.dtype, device=dev)
    d = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, hla.HLA_BF16, Cw)
    ws = torch.empty(hla.workspace_bytes(hla.FN_ROUTE_MIX, d, Cw), dtype=torch.uint8, device=dev)
    ws_t = hla._workspace(hla.workspace_bytes(hla.FN_CHUNK_TRANSITIONS, d), dev)
    ws_p = hla._workspace(hla.workspace_bytes(hla.FN_GDN_PREFILL, d), dev) if Cw != C else None
    wu = hla._workspace(hla.workspace_bytes(hla.FN_WU_HANDOFF, d), dev) if handoff else None
    g_in = None if gates_in is None else torch.from_numpy(gates_in).to(dev)
    n_rep = Cw if pooler is None else Cw // window
    if pooler is not None:
        Wd = {n: to_dev(a, W.dtype, torch) for n, a in pooler.items()}
        reps = torch.empty((W.B, N * n_rep, W.H, W.dk), dtype=k.dtype, device=dev)
        ws_r = hla._workspace(hla.workspace_bytes(hla.FN_CHUNK_REPS, d, n_rep), dev)
    out = dict(gates=torch.empty((W.B, W.H, N, N), dtype=torch.float32, device=dev),
               mask=torch.empty((W.B, W.H, N, N), dtype=torch.uint8, device=dev),
               active_idx=torch.empty((W.B, W.H, N, N), dtype=torch.int32, device=dev),
               active_cnt=torch.empty((W.B, W.H, N), dtype=torch.int32, device=dev),
               n_eff=torch.empty((W.B, W.H, N), dtype=torch.float32, device=dev),
               S_routed=torch.empty((W.B, W.H, N, W.dk, W.dv), dtype=torch.float32, device=dev))
    o = torch.empty((W.B, W.T, W.H, W.dv), dtype=torch.float32, device=dev)

    def step():
        hla.chunk_transitions(k, v, beta, alpha, At=At, Bc=Bc, C=Cw, ws=ws_t, wu=wu)
        r_in = k
        if pooler is not None:
            r_in = hla.chunk_reps(k, Wd, window=window, C=Cw, out=reps, ws=ws_r)
        hla.route_mix(q, r_in, At, Bc, n_rep=n_rep, tau=tau, gates_in=g_in, out=out, ws=ws, C=Cw)
        hla.gdn_prefill(q, k, v, beta, alpha, chunk_init=out["S_routed"], want_state=False, o=o, ws=ws_p, C=Cw,
                        wu=wu)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    pairs = int(out["active_cnt"].sum().item())
    hla.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    comp_ms, comp_n = hla.timing_read(hla.KERNEL_COMPOSE)
    per_kernel = {name: hla.timing_read(kid) for name, kid in
                  (("chunk", hla.KERNEL_CHUNK), ("gates", hla.KERNEL_GATES), ("compose", hla.KERNEL_COMPOSE),
                   ("reps", hla.KERNEL_REPS))}
    hla.timing_enable(False)

    n_pieces = W.B * W.H * math.ceil(W.T / C)
    fl_comp = flops_compose(pairs, W.dk, W.dv)
    fl_total = (fl_comp + flops_transitions(n_pieces, W.dk, W.dv) + flops_routed_output(n_pieces, W.dk, W.dv)
                + (flops_gates(pairs, n_rep, W.dk) if gates_in is None else 0))
    n_windows = W.B * W.H * N * n_rep
    if pooler is not None:
        fl_total += flops_reps_pool(n_windows, window, W.dk) + flops_reps_project(n_windows, W.dk)
    if Cw != C:  # composing the C / 64 piece maps of every chunk: [I|0] through C/64 pieces
        fl_total += W.B * W.H * N * (Cw // C) * 2 * W.dk * W.dk * (W.dk + W.dv)
    comp_avg_s = comp_ms / comp_n / 1e3
    achieved = fl_comp / comp_avg_s / 1e12
    cf = counter_figures(tag, "compose_bf16_kernel", comp_avg_s, flops=fl_comp,
                         nbytes=compose_alg_bytes(N, W)) if tag == "routed_prefill" else None
    traffic = cf["hbm_bytes_per_launch"] if cf and "hbm_bytes_per_launch" in cf else None
    tokens = W.B * W.T
    res = dict(
        value=tokens / dt, ms_per_step=dt * 1e3,
        mfma_util_pct=100.0 * fl_total / dt / (PEAK_BF16_TFLOPS * 1e12),
        step_tflops=fl_total / dt / 1e12, active_pairs=pairs,
        kernel_ms={kname: round(ms / n, 4) for kname, (ms, n) in per_kernel.items() if n > 0},
        roofline=dict(kernel="compose_bf16_kernel", bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=traffic,
                      flops_per_launch=fl_comp, avg_launch_ms=round(comp_avg_s * 1e3, 4), launches=comp_n,
                      counters=cf),
    )
    if tag == "routed_prefill":
        gc = gemm_ceiling(torch)
        res["roofline"]["library_gemm"] = dict(gc, frac_of_peak=round(gc["tflops"] / PEAK_BF16_TFLOPS, 4),
                                               compose_vs_gemm=round(achieved / gc["tflops"], 3))
    if pooler is not None:
        rms, rn = per_kernel["reps"]
        r_ach = flops_reps_pool(n_windows, window, W.dk) / (rms / rn / 1e3) / 1e12
        res["reps_pool"] = dict(kernel="reps_pool_kernel", bound="mfma", window=window, n_rep=n_rep,
                                avg_launch_ms=round(rms / rn, 4), achieved=round(r_ach, 2), peak=PEAK_BF16_TFLOPS,
                                unit="TFLOP/s", frac=round(r_ach / PEAK_BF16_TFLOPS, 4),
                                flops_per_launch=flops_reps_pool(n_windows, window, W.dk))
    log(f"[{tag}] {dt*1e3:.3f} ms/step, {tokens/dt/1e6:.3f} M tok/s, compose {comp_avg_s*1e3:.3f} ms "
        f"({achieved:.0f} TFLOP/s), step MFMA util {res['mfma_util_pct']:.1f}%, active pairs {pairs}")
    del q, k, v, At, Bc, out, o, ws, ws_t, ws_p, g_in
    torch.cuda.empty_cache()
    return res, x


def _sub(args):
    return argparse.Namespace(steps=max(3, args.steps // 2), warmup=1)


def bench_routed_c256(args, torch, hla, inputs, x):
    """The pages' default chunk size, C = 256 (64-token pieces composed four at a time)."""
    W = inputs.WORKLOADS["routed_prefill"]
    r, _ = bench_routed_prefill(_sub(args), torch, hla, inputs, Cw=256, x=x, tag="routed_prefill_C256")
    return dict(workload="routed_prefill C=256", C=256, tau=W.tau, ms_per_step=r["ms_per_step"],
                tokens_per_s=r["value"], mfma_util_pct=r["mfma_util_pct"], active_pairs=r["active_pairs"],
                compose_ms=r["roofline"]["avg_launch_ms"])


def bench_routed_skip(args, torch, hla, inputs, x):
    """C = 64 with skip-heavy caller gates at tau = 0.1: how skipping cuts the composition."""
    W = inputs.WORKLOADS["routed_prefill"]
    N = math.ceil(W.T / C)
    G = inputs.gen_gates(W.B, W.H, N, seed=0, stream=inputs.STREAM["routed_prefill"], mode="skip_heavy")
    r, _ = bench_routed_prefill(_sub(args), torch, hla, inputs, Cw=C, gates_in=G, tau=0.1, x=x,
                                tag="routed_prefill_skip")
    dense_pairs = W.B * W.H * N * (N - 1) // 2
    return dict(workload="routed_prefill C=64, caller gates sigmoid(N(-4, 3)), tau=0.1",
                C=C, tau=0.1, ms_per_step=r["ms_per_step"], tokens_per_s=r["value"],
                active_pairs=r["active_pairs"], active_frac=r["active_pairs"] / dense_pairs,
                compose_ms=r["roofline"]["avg_launch_ms"], compose_tflops_active=r["roofline"]["achieved"])


def bench_routed_learned_reps(args, torch, hla, inputs, x, window=32):
    """C = 64 with learned window representatives (seeded weights), C / window per chunk."""
    W = inputs.WORKLOADS["routed_prefill"]
    pooler = inputs.gen_pooler_weights(W.H, W.dk, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"])
    tag = "routed_prefill_learned_reps" + ("" if window == 32 else f"_w{window}")
    r, _ = bench_routed_prefill(_sub(args), torch, hla, inputs, Cw=C, x=x, tag=tag, pooler=pooler, window=window)
    return dict(
        workload=f"routed_prefill C=64, learned representatives (window {window}, {C // window} per chunk), "
                 "seeded weights",
        C=C, tau=W.tau, ms_per_step=r["ms_per_step"], tokens_per_s=r["value"], mfma_util_pct=r["mfma_util_pct"],
        active_pairs=r["active_pairs"], kernel_ms=r["kernel_ms"], reps_pool=r["reps_pool"])


def flops_reps_bwd(n_tokens_heads, dk):
    """Algorithmic matrix work of the learned-representative backward per token and head:
    the recomputed projections Q, K, V (3 x 2 dk^2), dX = dQ Wq + dK Wk + dV Wv (3 x 2 dk^2)
    and the weight gradients dQ^T X, dK^T X, dV^T X (3 x 2 dk^2); the window attention and the
    per-window vectors are not counted."""
    return n_tokens_heads * 18 * dk * dk


def bench_reps_backward(args, torch, hla, inputs, x, window=32):
    """hla_chunk_reps_backward at the long-context shape (B=1, T=32768, H=16, dk=128, bf16,
    per-head seeded weights with the folded query projection, window 32): from a seeded
    gradient of every representative row to dk and the five weight gradients."""
    W = inputs.WORKLOADS["routed_prefill"]
    pooler = inputs.gen_pooler_weights(W.H, W.dk, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"])
    Wd = {n: to_dev(a, W.dtype, torch) for n, a in pooler.items()}
    k = to_dev(x.k, W.dtype, torch)
    N = math.ceil(W.T / C)
    dreps = to_dev(inputs.gen_cotangent((W.B, N * (C // window), W.H, W.dk), seed=0, name="dreps"), "f32", torch)
    d = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dk, hla.HLA_BF16, C)
    ws = torch.empty(hla.workspace_bytes(hla.FN_CHUNK_REPS_BACKWARD, d, 1), dtype=torch.uint8, device=k.device)
    step = lambda: hla.chunk_reps_backward(k, Wd, dreps, window=window, ws=ws)
    steps = max(3, args.steps // 2)
    dt, kms = timed_kernels(step, steps, 2, torch, hla)
    ms = kms.get("bwd_reps", dt * 1e3)
    fl = flops_reps_bwd(W.B * W.T * W.H, W.dk)
    ach = fl / (ms / 1e3) / 1e12
    res = dict(workload=f"learned-representative backward, B={W.B} T={W.T} H={W.H} dk={W.dk} bf16, window {window}, "
                        "per-head weights with the folded query projection",
               ms_per_step=round(dt * 1e3, 3), kernel_ms=round(ms, 3), workspace_gib=round(ws.numel() / 2**30, 2),
               roofline=dict(kernel="reps_bwd_tile_kernel + reps_bwd_reduce_kernel", bound="mfma",
                             achieved=round(ach, 2), peak=PEAK_FP32_MFMA_TFLOPS, unit="TFLOP/s",
                             frac=round(ach / PEAK_FP32_MFMA_TFLOPS, 4), flops_per_call=fl))
    log(f"[learned_reps_backward] {dt*1e3:.3f} ms/call, kernels {ms:.3f} ms ({ach:.1f} TFLOP/s fp32 MFMA)")
    del ws, k, dreps, Wd
    torch.cuda.empty_cache()
    return res


def routed_inputs(inputs):
    W = inputs.WORKLOADS["routed_prefill"]
    log(f"[routed_prefill] generating inputs B={W.B} T={W.T} H={W.H} d={W.dk}")
    return inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"],
                             plant_period=W.plant_period)


# secondary lines, in the order the default run measures them; each takes the routed inputs
SECONDARY = {
    "routed_prefill_C256": bench_routed_c256,
    "routed_prefill_skip": bench_routed_skip,
    "routed_prefill_learned_reps": bench_routed_learned_reps,
    "routed_prefill_learned_reps_w64": lambda args, torch, hla, inputs, x: bench_routed_learned_reps(
        args, torch, hla, inputs, x, window=64),
    "gdn2_routed_prefill": lambda args, torch, hla, inputs, x: bench_gdn2_routed(args, torch, hla, inputs, x),
    "routed_prefill_backward": lambda args, torch, hla, inputs, x: bench_prefill_backward(args, torch, hla, inputs, x),
    "gdn2_routed_prefill_backward": lambda args, torch, hla, inputs, x: bench_gdn2_prefill_backward(
        args, torch, hla, inputs, x),
    "learned_reps_backward": bench_reps_backward,
    "decode": lambda args, torch, hla, inputs, x: bench_decode(args, torch, hla, inputs),
    "gdn2_decode": lambda args, torch, hla, inputs, x: bench_decode(args, torch, hla, inputs, gdn2=True),
    "native_prefill": lambda args, torch, hla, inputs, x: bench_native_prefill(args, torch, hla, inputs),
    "tail_replay": lambda args, torch, hla, inputs, x: _tail_replay_line(args, torch, hla, inputs),
    "decode_skip": lambda args, torch, hla, inputs, x: bench_decode(args, torch, hla, inputs, skip=True),
}

# lines run only when named with --only: the backward at the full 32768 tokens, in one call
# within a 64 GiB workspace (history segments replayed from checkpoints), and beside it with
# the about 200 GiB workspace in which every chunk pair has its own state slots
ONLY_LINES = {
    "routed_prefill_backward_T32K": lambda args, torch, hla, inputs, x: bench_prefill_backward(
        args, torch, hla, inputs, x, T=inputs.WORKLOADS["routed_prefill"].T, ws_gib=64),
}


# ----------------------------------------------------------------------------- decode
def bench_decode(args, torch, hla, inputs, gdn2=False, skip=False, warm=8):
    """Decode at Bs=256, H=16 with 64 cached chunks per sequence; ``gdn2`` runs the Gated
    DeltaNet-2 live update (channel-wise gates per token) instead of Gated DeltaNet's.
    ``skip``: skip-heavy caller gates (sigmoid(N(-4, 3)) per cached chunk) at tau = 0.1, the
    pages' threshold, so that skipped chunks are never read ([HLA] Methodology paragraph 4:
    thresholding cuts memory traffic)."""
    W = inputs.WORKLOADS["decode"]
    tag = "gdn2_decode" if gdn2 else ("decode_skip" if skip else "decode")
    tau = 0.1 if skip else W.tau
    Bs, H, dk, dv, n_cap = W.B, W.H, W.dk, W.dv, W.n_cache
    log(f"[decode] generating {n_cap} cached chunks per sequence for Bs={Bs} H={H}")
    hist = inputs.gen_tokens(Bs, n_cap * C, H, dk, dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["decode"],
                             with_q=False)
    k = to_dev(hist.k, W.dtype, torch)
    v = to_dev(hist.v, W.dtype, torch)
    beta, alpha = to_dev(hist.beta, "f32", torch), to_dev(hist.alpha, "f32", torch)
    del hist
    At_cache, Bc_cache = hla.chunk_transitions(k, v, beta, alpha)        # [Bs, H, n_cap, dk, dk|dv]
    reps = k.view(Bs, n_cap, C, H, dk).permute(0, 3, 1, 2, 4).contiguous()  # chunk keys as representatives
    del k, v, beta, alpha
    n_cache = torch.full((Bs,), n_cap, dtype=torch.int32, device="cuda")
    S = torch.zeros((Bs, H, dk, dv), dtype=torch.float32, device="cuda")
    A = torch.eye(dk, dtype=torch.float32, device="cuda").repeat(Bs, H, 1, 1).contiguous()
    o = torch.empty((Bs, H, dv), dtype=torch.float32, device="cuda")
    n_tok = 32  # distinct token sets, cycled over the timed steps
    toks = [inputs.gen_decode_tokens(Bs, H, dk, dv, step=s, dtype=W.dtype, seed=0, stream=inputs.STREAM["decode"])
            for s in range(n_tok)]
    toks = [{kk: to_dev(vv, W.dtype if kk in ("q", "k", "v") else "f32", torch) for kk, vv in t.items()} for t in toks]
    if gdn2:
        for s_, t in enumerate(toks):
            g = inputs.gen_gdn2_decode_gates(Bs, H, dk, dv, step=s_, seed=0, stream=inputs.STREAM["decode"])
            t.update({n: to_dev(g[n], "f32", torch) for n in ("a", "b", "w")})
    it = [0]
    g_in, n_active = None, Bs * H * n_cap
    if skip:
        import numpy as np
        G = inputs.gen_gates(Bs, H, n_cap, seed=0, stream=inputs.STREAM["decode"], mode="skip_heavy")[:, :, -1, :]
        G = np.ascontiguousarray(G)
        n_active = int((G >= np.float32(tau)).sum())
        g_in = torch.from_numpy(G).cuda()

    def step():
        t = toks[it[0] % n_tok]
        it[0] += 1
        if gdn2:
            hla.gdn2_decode(t["q"], t["k"], t["v"], t["a"], t["b"], t["w"], S, At_cur=A, At_cache=At_cache,
                            Bc_cache=Bc_cache, reps_cache=reps, n_cache=n_cache, tau=tau, o=o)
        else:
            hla.gdn_decode(t["q"], t["k"], t["v"], t["beta"], t["alpha"], S, At_cur=A, At_cache=At_cache,
                           Bc_cache=Bc_cache, reps_cache=reps, n_cache=n_cache, tau=tau, o=o, gates_in=g_in)

    steps = args.decode_steps
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    hla.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    dec_ms, dec_n = hla.timing_read(hla.KERNEL_DECODE)
    hla.timing_enable(False)
    e = 2  # bf16 bytes
    # per (sequence, head): live state and live transition read and written, the token
    # vectors and gates, the output; the representatives (computed gates) or the caller's
    # gates; and every active cached chunk's (At_j, Bc_j), read once
    per_seqhead = (2 * dk * dv * 4 + 2 * dk * dk * 4 + (2 * dk + dv) * e + ((2 * dk + dv) * 4 if gdn2 else 2 * 4)
                   + dv * 4 + (n_cap * 4 if skip else n_cap * C * dk * e))
    bytes_step = Bs * H * per_seqhead + n_active * (dk * dk + dk * dv) * e
    bytes_dense = Bs * H * (per_seqhead + n_cap * (dk * dk + dk * dv) * e)  # the same call, every chunk kept
    kern_s = dec_ms / dec_n / 1e3
    res = dict(workload=tag, Bs=Bs, H=H, cached_chunks=n_cap, steps=steps, ms_per_step=dt * 1e3, tau=tau,
               tokens_per_s=Bs / dt, hbm_gbs=bytes_step / kern_s / 1e9,
               roofline=dict(kernel="decode_kernel", bound="hbm", achieved=round(bytes_step / kern_s / 1e9, 1),
                             peak=PEAK_HBM_GBS, unit="GB/s", frac=round(bytes_step / kern_s / 1e9 / PEAK_HBM_GBS, 4),
                             bytes_per_launch=bytes_step, avg_launch_ms=round(kern_s * 1e3, 4),
                             traffic=None, counters=None),
               note="no commit while timing; live chunk extends past 64 tokens so every step does the same work")
    if tag == "decode":
        cf = counter_figures("decode", "decode_kernel", kern_s, nbytes=bytes_step)
        res["roofline"].update(counters=cf, traffic=cf["hbm_bytes_per_launch"] if cf else None)
    if skip:
        res.update(active_chunk_frac=n_active / (Bs * H * n_cap), bytes_per_step=bytes_step,
                   dense_bytes_per_step=bytes_dense, bytes_frac_of_dense=bytes_step / bytes_dense,
                   gates="caller gates sigmoid(N(-4, 3)) per cached chunk")
    log(f"[{tag}] {dt*1e3:.3f} ms/step, {Bs/dt:.0f} tok/s, kernel {kern_s*1e3:.3f} ms, "
        f"{bytes_step/kern_s/1e9:.0f} GB/s")
    del At_cache, Bc_cache, reps, S, A, toks, g_in
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- native prefill
def bench_native_prefill(args, torch, hla, inputs, steps=20, warmup=3):
    W = inputs.WORKLOADS["native_prefill"]
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["native_prefill"])
    q, k, v = (to_dev(a, W.dtype, torch) for a in (x.q, x.k, x.v))
    beta, alpha = to_dev(x.beta, "f32", torch), to_dev(x.alpha, "f32", torch)
    d = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, hla.HLA_BF16)
    ws = torch.empty(hla.workspace_bytes(hla.FN_GDN_PREFILL, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((W.B, W.T, W.H, W.dv), dtype=torch.float32, device="cuda")
    S = torch.empty((W.B, W.H, W.dk, W.dv), dtype=torch.float32, device="cuda")
    dt, kms = timed_kernels(lambda: hla.gdn_prefill(q, k, v, beta, alpha, o=o, S_final=S, ws=ws), steps, warmup,
                            torch, hla)
    bytes_alg = W.B * W.T * W.H * (2 * W.dk * 2 + W.dv * 2 + 2 * 4 + W.dv * 4) + W.B * W.H * W.dk * W.dv * 4
    res = dict(workload="native_prefill", B=W.B, T=W.T, H=W.H, ms_per_step=dt * 1e3, tokens_per_s=W.B * W.T / dt,
               algorithmic_gbs=bytes_alg / dt / 1e9, hbm_frac=round(bytes_alg / dt / 1e9 / PEAK_HBM_GBS, 4),
               kernel_ms=kms, counters=kernel_counters("native_prefill", kms,
                                                       (("chunk", "ut_kernel"), ("prefill", "state_kernel"))))
    log(f"[native_prefill] {dt*1e3:.3f} ms, {W.B*W.T/dt/1e6:.2f} M tok/s, {bytes_alg/dt/1e9:.0f} GB/s algorithmic")
    return res


# ----------------------------------------------------------------------------- Gated DeltaNet-2
# fp32 vector peak, as published: 256 CUs x 4 SIMDs x 16 lanes x 2 flop per FMA x 2 (packed
# fp32: two FMAs per lane and instruction) x 2.4 GHz = 157.3 TFLOP/s.  The library is compiled
# without packed-fp32 instructions, so its own ceiling is half that; records give both.
PEAK_FP32_VALU_TFLOPS = 256 * 4 * 16 * 2 * 2 * 2.4e9 / 1e12
PEAK_FP32_VALU_UNPACKED_TFLOPS = PEAK_FP32_VALU_TFLOPS / 2
# dense fp32 matrix-core peak, as published
PEAK_FP32_MFMA_TFLOPS = 157.3


def bytes_gdn2_passes(B, T, H, dk, dv, N):
    """Algorithmic HBM bytes of the two bf16 Gated DeltaNet-2 chunk passes, each input read
    once and each output written once: the maps pass reads k, v (bf16) and the channel-wise
    alpha, b (dk) and w (dv) (float32) and writes every chunk's At and Bc (bf16); the
    outputs pass reads q, k, v, alpha, b, w and every chunk's float32 start state and
    writes o (float32)."""
    th, chunks = B * T * H, B * H * N
    gates = 4 * (2 * dk + dv)
    maps = th * (2 * dk + 2 * dv + gates) + chunks * 2 * (dk * dk + dk * dv)
    outs = th * (2 * dk + 2 * dk + 2 * dv + gates + 4 * dv) + chunks * 4 * dk * dv
    return maps, outs


def bench_gdn2_routed(args, torch, hla, inputs, x):
    """The routed prefill step under the Gated DeltaNet-2 recurrence at the long-context
    shape: GDN-2 chunk maps, the HLA router and composition, GDN-2 chunk outputs."""
    W = inputs.WORKLOADS["routed_prefill"]
    log(f"[gdn2_routed_prefill] generating channel-wise gates B={W.B} T={W.T} H={W.H}")
    g = inputs.gen_gdn2_gates(W.B, W.T, W.H, W.dk, W.dv, seed=0, stream=inputs.STREAM["routed_prefill"])
    ga, gb, gw = (to_dev(g[n], "f32", torch) for n in ("a", "b", "w"))
    del g
    q, k, v = (to_dev(a, W.dtype, torch) for a in (x.q, x.k, x.v))
    dev = k.device
    N = math.ceil(W.T / C)
    d = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, hla.HLA_BF16, C)
    At = torch.empty((W.B, W.H, N, W.dk, W.dk), dtype=k.dtype, device=dev)
    Bc = torch.empty((W.B, W.H, N, W.dk, W.dv), dtype=k.dtype, device=dev)
    ws = torch.empty(hla.workspace_bytes(hla.FN_ROUTE_MIX, d, C), dtype=torch.uint8, device=dev)
    out = dict(gates=torch.empty((W.B, W.H, N, N), dtype=torch.float32, device=dev),
               mask=torch.empty((W.B, W.H, N, N), dtype=torch.uint8, device=dev),
               active_idx=torch.empty((W.B, W.H, N, N), dtype=torch.int32, device=dev),
               active_cnt=torch.empty((W.B, W.H, N), dtype=torch.int32, device=dev),
               n_eff=torch.empty((W.B, W.H, N), dtype=torch.float32, device=dev),
               S_routed=torch.empty((W.B, W.H, N, W.dk, W.dv), dtype=torch.float32, device=dev))
    o = torch.empty((W.B, W.T, W.H, W.dv), dtype=torch.float32, device=dev)

    def step():
        hla.gdn2_chunk_transitions(k, v, ga, gb, gw, At=At, Bc=Bc)
        hla.route_mix(q, k, At, Bc, n_rep=C, tau=W.tau, out=out, ws=ws)
        hla.gdn2_prefill(q, k, v, ga, gb, gw, chunk_init=out["S_routed"], want_state=False, o=o)

    steps = max(3, args.steps // 2)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    hla.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    ch_ms, ch_n = hla.timing_read(hla.KERNEL_CHUNK)
    cm_ms, cm_n = hla.timing_read(hla.KERNEL_COMPOSE)
    hla.timing_enable(False)
    maps_b, outs_b = bytes_gdn2_passes(W.B, W.T, W.H, W.dk, W.dv, N)
    chunk_s = ch_ms / ch_n / 1e3 * 2  # two chunk passes per step
    ach = (maps_b + outs_b) / chunk_s / 1e9
    # HBM bytes of the two passes from the committed counters (FETCH_SIZE + WRITE_SIZE, copy
    # calibrated), when they were taken on the current sources
    ks = read_counters("gdn2_routed_prefill") or {}
    kp = [ks.get(f"gdn2_wy_kernel<{W.dk}, {W.dv}, {o}>") for o in ("false", "true")]
    traffic = sum(k["hbm_bytes"] for k in kp) if all(k and "hbm_bytes" in k for k in kp) else None
    res = dict(workload="routed_prefill under Gated DeltaNet-2 (channel-wise decay, erase and write gates), "
                        "B=1 T=32768 H=16 d=128 C=64",
               ms_per_step=dt * 1e3, tokens_per_s=W.B * W.T / dt, compose_ms=round(cm_ms / cm_n, 4),
               chunk_passes_ms=round(chunk_s * 1e3, 4),
               chunk_roofline=dict(kernel="gdn2_wy_kernel (maps + outputs)", bound="hbm", achieved=round(ach, 1),
                                   peak=PEAK_HBM_GBS, unit="GB/s", frac=round(ach / PEAK_HBM_GBS, 4),
                                   traffic=traffic, bytes_per_step=maps_b + outs_b, maps_bytes=maps_b,
                                   outputs_bytes=outs_b))
    if traffic:
        res["chunk_roofline"].update(counter_hbm_gbs=round(traffic / chunk_s / 1e9, 1),
                                     traffic_over_algorithmic=round(traffic / (maps_b + outs_b), 3))
    log(f"[gdn2_routed_prefill] {dt*1e3:.3f} ms/step, {W.B*W.T/dt/1e6:.3f} M tok/s, chunk passes "
        f"{chunk_s*1e3:.3f} ms ({ach:.0f} GB/s of algorithmic bytes), compose {cm_ms/cm_n:.3f} ms")
    del q, k, v, ga, gb, gw, At, Bc, out, o, ws
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- backward
BWD_T = 8192


def flops_chunk_bwd(n_pieces_heads, dk, dv):
    """Algorithmic work of the per-piece reverse through the UT form ([HLA] Methodology
    paragraph 1), per (piece, head), as matrix products at 2 m n k, each product with a
    triangular factor (A0, P, dP, X, H) at half: both parts recompute A0 (C^2 dk), W and U
    (C^2 (dk + dv)) and end in the common tail (G and F: C^2 (dk + dv); T1: 2 C^2 (dk + dv);
    H: C^3; H'K and H'^T K: 2 C^2 dk).  The maps part adds dY, dKB and dK_ab (4 C dk^2 +
    4 C dk dv); the outputs part adds P (C^2 dk), E (2 C dk dv), dE and dP (2 C^2 dv), dQ
    (2 C dk dv + C^2 dk), dK_P (C^2 dk), dM0 (4 C dk dv) and dW (2 C dk dv).  The blocked
    inverse and the per-token sums are not counted."""
    c = C
    tail = c * c * (dk + dv) + 2 * c * c * (dk + dv) + c ** 3 + 2 * c * c * dk
    common = c * c * dk + c * c * (dk + dv) + tail
    maps = common + 4 * c * dk * dk + 4 * c * dk * dv
    outs = common + c * c * dk + 2 * c * dk * dv + 2 * c * c * dv + 2 * c * dk * dv + c * c * dk + c * c * dk \
        + 4 * c * dk * dv + 2 * c * dk * dv
    return n_pieces_heads * (maps + outs)


def flops_router_bwd(pairs, n_rep, dk):
    """Per history pair: the scores twice (query side and key side) and the two gradient
    accumulations, 2 n_rep dk each."""
    return pairs * 4 * 2 * n_rep * dk


def state_traffic(pairs, dk, dv, ms):
    """The per-pair state bytes each composition-backward pass moves by design (bf16 dk x dv
    matrices: the replay writes M_{j-1} and D_j, the adjoint reads D_j and writes g lambda_j,
    the reduce reads M_{j-1} and g lambda_j), and the HBM rate they make per pass: context
    for the matrix-core fractions, since these passes are bound by that traffic."""
    per = pairs * dk * dv * 2
    out = {}
    for name, n in (("bwd_save", 2), ("bwd_adjoint", 2), ("bwd_reduce", 2)):
        if name in ms:
            gbs = n * per / (ms[name] / 1e3) / 1e9
            out[name] = dict(bytes=n * per, achieved=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4))
    return dict(unit="GB/s", peak=PEAK_HBM_GBS, **out)


def bench_prefill_backward(args, torch, hla, inputs, x, T=BWD_T, ws_gib=None):
    """The routed-prefill backward (hla_prefill_backward) at B=1, T tokens (8192 by default),
    H=16, d=128, C=64, bf16, computed gates at tau = 1e-3: recomputed chunk maps and gates,
    composition replay, chunk outputs reverse, composition adjoint and sums, chunk maps
    reverse, router backward and the per-token sums.  The workspace is the one-pass size
    (every chunk pair its own state slots) or, with `ws_gib` below that, `ws_gib` GiB, in
    which the composition backward runs its history steps in segments replayed from
    checkpoints; the one-pass size is then timed beside it."""
    W = inputs.WORKLOADS["routed_prefill"]
    q, k, v = (to_dev(a[:, :T], W.dtype, torch) for a in (x.q, x.k, x.v))
    beta, alpha = to_dev(x.beta[:, :T], "f32", torch), to_dev(x.alpha[:, :T], "f32", torch)
    dO = to_dev(inputs.gen_cotangent((W.B, T, W.H, W.dv), seed=0, name="dO"), "f32", torch)
    dev = k.device
    N = math.ceil(T / C)
    d = hla.make_dims(W.B, T, W.H, T, W.dk, W.dv, hla.HLA_BF16, C)
    one_pass = hla.workspace_bytes(hla.FN_PREFILL_BACKWARD, d)
    main_bytes = one_pass if ws_gib is None else min(one_pass, int(ws_gib * 2**30))
    steps = max(3, args.steps // 4)
    names = (("bwd_chunk", hla.KERNEL_BWD_CHUNK), ("bwd_save", hla.KERNEL_BWD_SAVE),
             ("bwd_adjoint", hla.KERNEL_BWD_ADJOINT), ("bwd_reduce", hla.KERNEL_BWD_REDUCE),
             ("bwd_router", hla.KERNEL_BWD_ROUTER), ("fwd_chunk", hla.KERNEL_CHUNK), ("fwd_gates", hla.KERNEL_GATES),
             ("fwd_compose", hla.KERNEL_COMPOSE))

    def measure(nbytes):
        """ms per step, per-kernel ms per step and composition segments per step."""
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        log(f"[routed_prefill_backward] T={T}: workspace {nbytes / 2**30:.2f} GiB")
        step = lambda: hla.prefill_backward(q, k, v, beta, alpha, dO, tau=W.tau, ws=ws)
        step()
        torch.cuda.synchronize()
        hla.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        dt_ = (time.perf_counter() - t0) / steps
        per = {n: hla.timing_read(kid) for n, kid in names}
        hla.timing_enable(False)
        del ws
        torch.cuda.empty_cache()
        ms_ = {n: tot / steps for n, (tot, cnt) in per.items() if cnt > 0}
        return dt_, ms_, per["bwd_adjoint"][1] // steps  # one adjoint launch per segment

    dt, ms, segments = measure(main_bytes)
    # active pairs from the router's own mask (a gate gradient can underflow to zero far
    # back in a long chain, so it does not count them); after the timed calls, so that in a
    # kernel trace every kernel's first dispatch is the warm-up call's
    At, Bc = hla.chunk_transitions(k, v, beta, alpha)
    pairs = int(hla.route_mix(q, k, At, Bc, tau=W.tau)["active_cnt"].sum().item())
    del At, Bc
    fl_chunk = flops_chunk_bwd(W.B * N * W.H, W.dk, W.dv)
    fl_pair = flops_compose(pairs, W.dk, W.dv)
    ach = fl_chunk / (ms["bwd_chunk"] / 1e3) / 1e12
    mfma = {n: dict(achieved=round(fl_pair / (ms[n] / 1e3) / 1e12, 1),
                    frac=round(fl_pair / (ms[n] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4))
            for n in ("bwd_save", "bwd_adjoint", "bwd_reduce")}
    # roofline record of the kernel that takes the most time: the chunk reverse (fp32 matrix
    # cores) or one of the composition passes (bf16 matrix cores)
    kernels = {"bwd_chunk": ("chunk_bwd_out_ut_kernel + chunk_bwd_map_ut_kernel (reverse through the UT form)",
                             "mfma", fl_chunk, PEAK_FP32_MFMA_TFLOPS),
               "bwd_save": ("compose_replay_kernel (+ prep_bwd_kernel)", "mfma", fl_pair, PEAK_BF16_TFLOPS),
               "bwd_adjoint": ("compose_adjoint_kernel", "mfma", fl_pair, PEAK_BF16_TFLOPS),
               "bwd_reduce": ("compose_grad_reduce_kernel (+ chain_sum_kernel)", "mfma", fl_pair, PEAK_BF16_TFLOPS)}
    dom = max(kernels, key=lambda n: ms[n])
    kname, bound, fl_dom, peak = kernels[dom]
    ach_dom = fl_dom / (ms[dom] / 1e3) / 1e12
    res = dict(workload=f"routed prefill backward (GDN + HLA), B={W.B} T={T} H={W.H} d={W.dk} C={C} bf16, "
                        f"computed gates tau={W.tau}",
               ms_per_step=round(dt * 1e3, 3), tokens_per_s=round(W.B * T / dt, 1), active_pairs=pairs,
               workspace_gib=round(main_bytes / 2**30, 2), history_segments=segments,
               kernel_ms={n: round(v, 3) for n, v in ms.items()},
               roofline=dict(kernel=kname, bound=bound, achieved=round(ach_dom, 2), peak=round(peak, 1),
                             unit="TFLOP/s", frac=round(ach_dom / peak, 4), flops_per_launch=fl_dom,
                             avg_launch_ms=round(ms[dom], 4)),
               chunk_reverse=dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_FP32_MFMA_TFLOPS,
                                  unit="TFLOP/s", frac=round(ach / PEAK_FP32_MFMA_TFLOPS, 4), flops_per_step=fl_chunk),
               composition_mfma=dict(flops_per_pass=fl_pair, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", **mfma),
               composition_state_traffic=state_traffic(pairs, W.dk, W.dv, ms),
               router_tflops=round(flops_router_bwd(pairs, C, W.dk) / (ms["bwd_router"] / 1e3) / 1e12, 2),
               min_workspace_gib=round(hla.workspace_bytes(hla.FN_PREFILL_BACKWARD_MIN, d) / 2**30, 2))
    log(f"[routed_prefill_backward T={T}] {dt*1e3:.3f} ms/step, {W.B*T/dt/1e6:.3f} M tok/s in "
        f"{main_bytes / 2**30:.1f} GiB ({segments} history segments); chunk reverse "
        f"{ms['bwd_chunk']:.3f} ms ({ach:.1f} TFLOP/s fp32 MFMA); replay {ms['bwd_save']:.3f}, adjoint "
        f"{ms['bwd_adjoint']:.3f}, reduce {ms['bwd_reduce']:.3f}, router {ms['bwd_router']:.3f} ms")
    if main_bytes < one_pass:
        dt1, ms1, _ = measure(one_pass)
        res["one_pass"] = dict(workspace_gib=round(one_pass / 2**30, 2), ms_per_step=round(dt1 * 1e3, 3),
                               tokens_per_s=round(W.B * T / dt1, 1), kernel_ms={n: round(v, 3) for n, v in ms1.items()})
        log(f"[routed_prefill_backward T={T}] one pass in {one_pass / 2**30:.1f} GiB: {dt1*1e3:.3f} ms/step")
    del q, k, v, beta, alpha, dO
    torch.cuda.empty_cache()
    return res


def flops_gdn2_chunk_bwd(n_tokens_heads, dk, dv):
    """Algorithmic work of the Gated DeltaNet-2 per-chunk reverse, per token and head and per
    row of a state column: the forward step once (a o x, k . x' and the update: 7 flops) and
    its reverse (k . dx and (b o k) . dx: 5; the key, decay and erase-gate parts and the dx
    update: 12); the dv state columns add q dO and the query part (3).  Map columns: dk + dv;
    state columns: dv.  The checkpoint replay and the column sums are not counted."""
    return n_tokens_heads * dk * (dv * 27 + (dk + dv) * 24)


def bench_gdn2_prefill_backward(args, torch, hla, inputs, x, T=BWD_T):
    """The Gated DeltaNet-2 routed-prefill backward (hla_gdn2_prefill_backward) at B=1,
    T tokens (8192 by default), H=16, d=128, C=64, bf16, channel-wise gates, computed router
    gates at tau = 1e-3, with the one-pass workspace: recomputed GDN-2 chunk maps and gates,
    the composition replay, adjoint and sums (shared with Gated DeltaNet), the GDN-2 chunk
    reverse per state column (float32 VALU) and the router backward."""
    W = inputs.WORKLOADS["routed_prefill"]
    log(f"[gdn2_routed_prefill_backward] generating channel-wise gates B={W.B} T={T} H={W.H}")
    g = inputs.gen_gdn2_gates(W.B, T, W.H, W.dk, W.dv, seed=0, stream=inputs.STREAM["routed_prefill"])
    ga, gb, gw = (to_dev(g[n], "f32", torch) for n in ("a", "b", "w"))
    del g
    # the first T tokens as their own [B, T, H, d] arrays, like the gates
    q, k, v = (to_dev(a[:, :T].copy(), W.dtype, torch) for a in (x.q, x.k, x.v))
    dO = to_dev(inputs.gen_cotangent((W.B, T, W.H, W.dv), seed=0, name="dO"), "f32", torch)
    dev = k.device
    d = hla.make_dims(W.B, T, W.H, T, W.dk, W.dv, hla.HLA_BF16, C)
    ws = torch.empty(hla.workspace_bytes(hla.FN_GDN2_PREFILL_BACKWARD, d), dtype=torch.uint8, device=dev)
    step = lambda: hla.gdn2_prefill_backward(q, k, v, ga, gb, gw, dO, tau=W.tau, ws=ws)
    steps = max(3, args.steps // 4)
    step()
    torch.cuda.synchronize()
    hla.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    names = (("bwd_chunk", hla.KERNEL_BWD_CHUNK), ("bwd_save", hla.KERNEL_BWD_SAVE),
             ("bwd_adjoint", hla.KERNEL_BWD_ADJOINT), ("bwd_reduce", hla.KERNEL_BWD_REDUCE),
             ("bwd_router", hla.KERNEL_BWD_ROUTER), ("fwd_chunk", hla.KERNEL_CHUNK), ("fwd_gates", hla.KERNEL_GATES))
    per = {n: hla.timing_read(kid) for n, kid in names}
    hla.timing_enable(False)
    ms = {n: tot / steps for n, (tot, cnt) in per.items() if cnt > 0}
    fl = flops_gdn2_chunk_bwd(W.B * T * W.H, W.dk, W.dv)
    ach = fl / (ms["bwd_chunk"] / 1e3) / 1e12
    res = dict(workload=f"Gated DeltaNet-2 routed prefill backward, B={W.B} T={T} H={W.H} d={W.dk} C={C} bf16, "
                        f"channel-wise gates, computed gates tau={W.tau}",
               ms_per_step=round(dt * 1e3, 3), tokens_per_s=round(W.B * T / dt, 1),
               workspace_gib=round(ws.numel() / 2**30, 2), kernel_ms={n: round(v, 3) for n, v in ms.items()},
               chunk_reverse=dict(kernel="gdn2_chunk_bwd_kernel (outputs and maps, per state column)", bound="alu",
                                  achieved=round(ach, 2), peak=round(PEAK_FP32_VALU_TFLOPS, 1), unit="TFLOP/s",
                                  frac=round(ach / PEAK_FP32_VALU_TFLOPS, 4),
                                  frac_of_unpacked_peak=round(ach / PEAK_FP32_VALU_UNPACKED_TFLOPS, 4),
                                  flops_per_step=fl))
    log(f"[gdn2_routed_prefill_backward T={T}] {dt*1e3:.3f} ms/step, {W.B*T/dt/1e6:.3f} M tok/s; chunk reverse "
        f"{ms['bwd_chunk']:.3f} ms ({ach:.1f} TFLOP/s fp32 VALU); replay {ms['bwd_save']:.3f}, adjoint "
        f"{ms['bwd_adjoint']:.3f}, reduce {ms['bwd_reduce']:.3f}, router {ms['bwd_router']:.3f} ms")
    del ws, q, k, v, ga, gb, gw, dO
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- Tail-Replay
def bench_tail_replay(args, torch, hla, inputs, steps=20, warmup=3, full_prefix=True):
    """[TR]: the state of a 32768-token prefix rebuilt from its last 3277 tokens alone (a
    suffix view of the allocation, state-only), against the full-prefix state-only prefill
    on the GPU.  Returns the record and the two states of TAIL_PAIRS on the host, for the
    oracle leg."""
    W = inputs.WORKLOADS["tail_replay"]
    L = W.replay
    log(f"[tail_replay] generating B={W.B} T={W.T} H={W.H} (replay {L})")
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["tail_replay"],
                          with_q=False)
    k, v = to_dev(x.k, W.dtype, torch), to_dev(x.v, W.dtype, torch)
    beta, alpha = to_dev(x.beta, "f32", torch), to_dev(x.alpha, "f32", torch)
    del x
    ks, vs, bs, als = k[:, -L:], v[:, -L:], beta[:, -L:], alpha[:, -L:]
    S = torch.empty((W.B, W.H, W.dk, W.dv), dtype=torch.float32, device="cuda")
    d_rep = hla.make_dims(W.B, L, W.H, W.T, W.dk, W.dv, hla.HLA_BF16)
    ws_rep = hla._workspace(hla.workspace_bytes(hla.FN_GDN_PREFILL, d_rep), "cuda")
    dt_rep, kms = timed_kernels(lambda: hla.gdn_prefill(None, ks, vs, bs, als, want_o=False, S_final=S, ws=ws_rep),
                                steps, warmup, torch, hla)
    if not full_prefix:
        return dict(ms_replay=dt_rep * 1e3, kernel_ms=kms), None
    d_full = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, hla.HLA_BF16)
    ws_full = hla._workspace(hla.workspace_bytes(hla.FN_GDN_PREFILL, d_full), "cuda")
    S2 = torch.empty_like(S)
    dt_full = timed(lambda: hla.gdn_prefill(None, k, v, beta, alpha, want_o=False, S_final=S2, ws=ws_full), 5, 1, torch)
    Sh, S2h = S.cpu().numpy(), S2.cpu().numpy()
    bytes_alg = W.B * L * W.H * (W.dk * 2 + W.dv * 2 + 2 * 4) + W.B * W.H * W.dk * W.dv * 4
    res = dict(workload="tail_replay", B=W.B, H=W.H, prefix=W.T, replay=L, ms_replay=dt_rep * 1e3,
               ms_full_prefix_state=dt_full * 1e3, speedup_vs_full=dt_full / dt_rep,
               replay_tokens_per_s=W.B * L / dt_rep, algorithmic_gbs=bytes_alg / dt_rep / 1e9,
               hbm_frac=round(bytes_alg / dt_rep / 1e9 / PEAK_HBM_GBS, 4),
               rel_err_vs_gpu_full_prefix=rel_err(Sh, S2h), kernel_ms=kms,
               counters=kernel_counters("tail_replay", kms, (("chunk", "ut_kernel"), ("prefill", "state_kernel"))),
               note="rel_err_vs_gpu_full_prefix compares the rebuilt states of all sequences with the GPU's "
                    "full-prefix states; the oracle leg adds both against the oracle and the P11 bound")
    log(f"[tail_replay] replay {dt_rep*1e3:.3f} ms vs full-prefix state {dt_full*1e3:.3f} ms "
        f"({dt_full/dt_rep:.1f}x), rebuilt vs full-prefix state {res['rel_err_vs_gpu_full_prefix']:.2e}")
    del k, v, beta, alpha, ws_rep, ws_full
    torch.cuda.empty_cache()
    states = (Sh[[b for b, _ in TAIL_PAIRS], [h for _, h in TAIL_PAIRS]],
              S2h[[b for b, _ in TAIL_PAIRS], [h for _, h in TAIL_PAIRS]])
    return res, states


_TAIL_STATES = {}


def _tail_replay_line(args, torch, hla, inputs):
    res, _TAIL_STATES["states"] = bench_tail_replay(args, torch, hla, inputs)
    return res


# ----------------------------------------------------------------------------- CPU oracle
TAIL_PAIRS = [(0, 0), (0, 1)]  # (b, h) of the Tail-Replay workload the oracle checks and times


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        return 1


def oracle_samples(n_query_chunks, small=False, tail_states=None):
    """The oracle (as it stands, never tuned) timed on a bounded sample of every workload
    the GPU lines measure, each stage extrapolated to the full workload by its own work
    ratio.  ``small`` shrinks the samples (the single-thread run).  ``tail_states``: the
    GPU's rebuilt and full-prefix states of TAIL_PAIRS, compared with the oracle's."""
    import numpy as np

    import oracle
    from gated_deltanet_hybrid_amd import inputs
    out = {}
    # routed prefill (the headline): the first n_query_chunks chunks of head 0
    W = inputs.WORKLOADS["routed_prefill"]
    Tn = n_query_chunks * C
    x = inputs.gen_tokens(1, W.T, 1, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"],
                          plant_period=W.plant_period, t_range=(0, Tn))
    q, k, v = (x.f64(n)[0, :, 0] for n in ("q", "k", "v"))
    beta, alpha = x.f64("beta")[0, :, 0], x.f64("alpha")[0, :, 0]
    t0 = time.perf_counter()
    A, B = oracle.chunk_transitions(k, v, beta, alpha, C)
    t1 = time.perf_counter()
    r = oracle.router_gates(q, k, C, C, W.tau)
    t2 = time.perf_counter()
    S = oracle.routed_states(A, B, r["ghat"], r["mask"])
    t3 = time.perf_counter()
    oracle.routed_outputs(q, k, v, beta, alpha, C, S)
    t4 = time.perf_counter()
    N = W.N
    pairs_s, pairs_f = n_query_chunks * (n_query_chunks - 1) / 2, N * (N - 1) / 2
    per_head = ((t1 - t0) * N / n_query_chunks + (t2 - t1) * pairs_f / pairs_s + (t3 - t2) * pairs_f / pairs_s
                + (t4 - t3) * N / n_query_chunks)
    full = per_head * W.H * W.B
    out["routed_prefill"] = dict(
        value=W.B * W.T / full, unit="tokens/s",
        sample=f"routed prefill of the first {Tn} tokens ({n_query_chunks} chunks) of head 0, {t4 - t0:.1f} s; "
               f"stages extrapolated to B={W.B}, H={W.H}, T={W.T} by chunk count (transitions, outputs) or "
               f"chunk-pair count (gates, composition)",
        sample_seconds=round(t4 - t0, 2), extrapolated_seconds=round(full, 1))
    # native prefill: a few heads of batch row 0, whole sequence, outputs and final state
    W = inputs.WORKLOADS["native_prefill"]
    nh = 2 if small else 4
    x = inputs.gen_tokens(1, W.T, nh, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["native_prefill"])
    t0 = time.perf_counter()
    oracle.gdn_recurrent(*(x.f64(n)[0].swapaxes(0, 1) for n in ("q", "k", "v", "beta", "alpha")))
    dt = time.perf_counter() - t0
    full = dt * W.B * W.H / nh
    out["native_prefill"] = dict(value=W.B * W.T / full, unit="tokens/s",
                                 sample=f"{nh} of {W.B * W.H} (batch row, head) sequences of {W.T} tokens, "
                                        f"{dt:.1f} s, extrapolated by sequence count",
                                 sample_seconds=round(dt, 2), extrapolated_seconds=round(full, 1))
    # decode: one step of a few (sequence, head) pairs, each composing its 64 cached chunks
    W = inputs.WORKLOADS["decode"]
    ns = 4 if small else 8
    At_s, Bc_s = inputs.gen_transitions(1, ns, W.n_cache, W.dk, W.dv, dtype=W.dtype, seed=31)
    reps = inputs.gen_tokens(1, W.n_cache * C, ns, W.dk, W.dk, dtype=W.dtype, seed=32, with_q=False)
    R = reps.f64("k")[0].reshape(W.n_cache, C, ns, W.dk).transpose(2, 0, 1, 3)
    Am = inputs.to_f64(At_s, W.dtype)[0].transpose(0, 1, 3, 2)
    Bm = inputs.to_f64(Bc_s, W.dtype)[0].transpose(0, 1, 3, 2)
    tok = inputs.gen_decode_tokens(1, ns, W.dk, W.dv, step=0, dtype=W.dtype, seed=0, stream=inputs.STREAM["decode"])
    tq, tk, tv = (inputs.to_f64(tok[n], W.dtype)[0] for n in ("q", "k", "v"))
    t0 = time.perf_counter()
    for i in range(ns):
        oracle.decode_step(tq[i], tk[i], tv[i], float(tok["beta"][0, i]), float(tok["alpha"][0, i]),
                           np.zeros((W.dv, W.dk)), np.eye(W.dk), Am[i], Bm[i], R[i], W.tau)
    dt = time.perf_counter() - t0
    step_s = dt * W.B * W.H / ns
    out["decode"] = dict(value=W.B / step_s, unit="tokens/s",
                         sample=f"one step of {ns} (sequence, head) pairs with {W.n_cache} cached chunks each, "
                                f"{dt:.2f} s, extrapolated to Bs={W.B} x H={W.H} by pair count",
                         sample_seconds=round(dt, 3), extrapolated_seconds=round(step_s, 2))
    # Tail-Replay: the replay of the last L tokens and the full-prefix recurrence
    W = inputs.WORKLOADS["tail_replay"]
    L = W.replay
    pairs = TAIL_PAIRS[:1] if small else TAIL_PAIRS
    nh = max(h for _, h in pairs) + 1
    x = inputs.gen_tokens(1, W.T, nh, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["tail_replay"],
                          with_q=False)
    kk, vv, bb, aa = (np.stack([x.f64(n)[b, :, h] for b, h in pairs]) for n in ("k", "v", "beta", "alpha"))
    t0 = time.perf_counter()
    _, S_rep = oracle.gdn_recurrent(None, kk[:, -L:], vv[:, -L:], bb[:, -L:], aa[:, -L:])
    t1 = time.perf_counter()
    _, S_pre = oracle.gdn_recurrent(None, kk[:, :-L], vv[:, :-L], bb[:, :-L], aa[:, :-L])
    _, S_full = oracle.gdn_recurrent(None, kk[:, -L:], vv[:, -L:], bb[:, -L:], aa[:, -L:], S0=S_pre)
    t2 = time.perf_counter()
    rep_full = (t1 - t0) * W.B * W.H / len(pairs)
    rec = dict(value=W.B * L / rep_full, unit="tokens/s (replayed)",
               sample=f"{len(pairs)} of {W.B * W.H} sequences: replay of the last {L} tokens {t1 - t0:.1f} s, "
                      f"full {W.T}-token prefix {t2 - t1:.1f} s; replay extrapolated by sequence count",
               sample_seconds=round(t2 - t0, 2), extrapolated_seconds=round(rep_full, 1),
               full_prefix_seconds_per_sequence=round((t2 - t1) / len(pairs), 2))
    if tail_states is not None:
        # parity of the GPU's rebuilt state against the same-suffix replay, and its distance
        # from the full-prefix state next to the [TR] bound of the replay (P11): the two
        # differ by at most (prod of the suffix alphas) ||S_{T-L}||_2
        S_gpu, S_gpu_full = tail_states
        cmp = []
        for i, (b, h) in enumerate(pairs):
            lb = oracle.tail_replay_bound_log10(aa[i, -L:], S_pre[i])
            cmp.append(dict(b=b, h=h, rel_err_vs_oracle_replay=rel_err(S_gpu[i], S_rep[i].T),
                            rel_err_vs_oracle_full_prefix=rel_err(S_gpu[i], S_full[i].T),
                            gpu_full_prefix_rel_err_vs_oracle=rel_err(S_gpu_full[i], S_full[i].T),
                            oracle_replay_vs_full_rel=rel_err(S_rep[i], S_full[i]),
                            p11_bound_log10=round(lb, 1)))
        rec["parity"] = cmp
    out["tail_replay"] = rec
    return out


def cpu_baseline(n_query_chunks, tail_states=None):
    """The oracle on every workload's sample: on all of the host's BLAS threads in this
    process, then single-threaded in a child process whose thread counts are set before
    numpy loads.  The headline value is the routed prefill on all threads."""
    import subprocess
    multi = oracle_samples(n_query_chunks, tail_states=tail_states)
    threads = _blas_threads()
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    single = None
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-samples", str(max(64, n_query_chunks // 4))],
                           env=env, capture_output=True, text=True, timeout=900)
        if r.returncode == 0:
            single = json.loads(r.stdout.strip().splitlines()[-1])
        else:
            log(f"[cpu_baseline] single-thread run failed: {r.stderr[-500:]}")
    except Exception as e:  # the baseline is a report; a failed child does not end the bench
        log(f"[cpu_baseline] single-thread run failed: {e}")
    head = multi["routed_prefill"]
    try:
        cpu_model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        cpu_model = None
    return dict(value=head["value"], unit="tokens/s", cores=threads, kind="oracle", sample=head["sample"],
                sample_seconds=head["sample_seconds"], extrapolated_seconds=head["extrapolated_seconds"],
                host_cpus=os.cpu_count(), affinity_cpus=len(os.sched_getaffinity(0)), cpu_model=cpu_model,
                per_workload={"threads": threads, **multi},
                single_thread=None if single is None else {"threads": single.pop("threads"), **single})


# ----------------------------------------------------------------------------- counters
# Hardware counters behind the roofline records, from rocprofv3 passes over short runs of
# one line each (one counter set per pass, FETCH_SIZE and WRITE_SIZE scaled by their own
# reading for a 1 GiB device copy), summarised into profiles/counters.json together with a
# hash of the kernel sources of that line; a line reports them only while those sources
# are unchanged.
COUNTER_SOURCES = {line: ["gated_deltanet_hybrid_amd/csrc/" + f for f in files] for line, files in (
    ("routed_prefill", ("chunk.hip", "route.hip", "compose.hip")),
    ("native_prefill", ("prefill.hip",)),
    ("tail_replay", ("prefill.hip",)),
    ("decode", ("decode.hip",)),
    ("gdn2_routed_prefill", ("gdn2.hip", "route.hip", "compose.hip")))}
CALIB_BYTES = 1 << 30
COUNTER_LINES = ("routed_prefill", "native_prefill", "tail_replay", "decode", "gdn2_routed_prefill")


def counter_run(line, torch, hla, inputs):
    """The line's timed call, once untimed and twice more, then a plain 1 GiB device copy
    (read 1 GiB, write 1 GiB) twice, which calibrates FETCH_SIZE / WRITE_SIZE."""
    args = argparse.Namespace(steps=2, warmup=1, decode_steps=2)
    if line == "routed_prefill":
        bench_routed_prefill(args, torch, hla, inputs)
    elif line == "native_prefill":
        bench_native_prefill(args, torch, hla, inputs, steps=2, warmup=1)
    elif line == "tail_replay":
        bench_tail_replay(args, torch, hla, inputs, steps=2, warmup=1, full_prefix=False)
    elif line == "decode":
        bench_decode(args, torch, hla, inputs, warm=1)
    elif line == "gdn2_routed_prefill":
        bench_gdn2_routed(args, torch, hla, inputs, routed_inputs(inputs))
    else:
        sys.exit(f"no counter run for {line}; lines: {', '.join(COUNTER_LINES)}")
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[counters] {line} done")


def _counter_rows(csv_path):
    """{(dispatch id, kernel name): {counter: summed value}} of one rocprofv3 counter file."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        c = per.setdefault(key, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


_MANGLED_ARGS = (("DF16b", "bf16"), ("f", "float"))


def kernel_key(name):
    """A readable key of a library kernel's trace name, template arguments kept:
    'void hla::ut_kernel<128, 128>(hla::UtArgs)' -> 'ut_kernel<128, 128>', and the mangled
    names the demangler leaves alone (bf16 template arguments) decoded the same way,
    '_ZN3hla13decode_kernelIDF16bLi128E...Lb0EEEv...' -> 'decode_kernel<bf16, 128, ..., false>'."""
    import re
    if name.startswith("_ZN3hla"):
        m = re.match(r"_ZN3hla(\d+)", name)
        n = int(m.group(1))
        ident = name[m.end():m.end() + n]
        rest = name[m.end() + n:]
        args = []
        if rest.startswith("I"):
            rest = rest[1:]
            while rest and not rest.startswith("E"):
                m2 = re.match(r"L([ib])(\d+)E", rest)
                if m2:
                    args.append(m2.group(2) if m2.group(1) == "i" else ("true" if m2.group(2) == "1" else "false"))
                    rest = rest[m2.end():]
                    continue
                for code, txt in _MANGLED_ARGS:
                    if rest.startswith(code):
                        args.append(txt)
                        rest = rest[len(code):]
                        break
                else:
                    args.append("?")
                    break
        return ident + (f"<{', '.join(args)}>" if args else "")
    s = name.replace("void ", "", 1).replace("hla::", "")
    depth = 0
    for i, ch in enumerate(s):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return s[:i]
    return s


def _short(name):
    return kernel_key(name).split("<")[0]


def counter_write(line, csv_paths):
    """Per-kernel means over the line's dispatches of every counter in the given passes,
    HBM bytes scaled by the calibration copy, into profiles/counters.json."""
    sums, counts, calib = {}, {}, {}
    for pth in csv_paths:
        rows = _counter_rows(pth)
        # the calibration copies are the run's last two runtime copy-buffer dispatches
        copies = sorted((i, v) for (i, n), v in rows.items() if n.startswith("__amd_rocclr_copyBuffer"))[-2:]
        if len(copies) != 2:
            sys.exit(f"{pth}: the two calibration copies are missing")
        for cn in copies[0][1]:
            calib[cn] = (copies[0][1][cn] + copies[1][1][cn]) / 2
        for (_, n), v in rows.items():
            if "hla" not in n:
                continue
            k = kernel_key(n)
            for cn, cv in v.items():
                sums.setdefault(k, {}).setdefault(cn, 0.0)
                sums[k][cn] += cv
                counts.setdefault(k, {}).setdefault(cn, 0)
                counts[k][cn] += 1
    out = {}
    for k, cs in sums.items():
        rec = {}
        for cn, tot in cs.items():
            mean = tot / counts[k][cn]
            rec[cn.lower() + "_mean"] = round(mean, 1)
            if cn in ("FETCH_SIZE", "WRITE_SIZE") and cn in calib:
                scale = CALIB_BYTES / (calib[cn] * 1024.0)
                rec[("fetch" if cn == "FETCH_SIZE" else "write") + "_bytes"] = round(mean * 1024.0 * scale)
                rec[cn.lower() + "_calib_factor"] = round(scale, 4)
            if cn == "SQ_INSTS_VALU_MFMA_MOPS_BF16":
                rec["mfma_bf16_flops"] = round(mean * 512)
        rec["dispatches"] = max(counts[k].values())
        if "fetch_bytes" in rec and "write_bytes" in rec:
            rec["hbm_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
        out[k] = rec
    path = os.path.join(ROOT, "profiles", "counters.json")
    allrec = json.load(open(path)) if os.path.exists(path) else {}
    allrec[line] = dict(source_sha=sha_of(*COUNTER_SOURCES[line]), sources=COUNTER_SOURCES[line], kernels=out,
                        calib_copy_bytes=CALIB_BYTES, calib_raw={k: round(v, 1) for k, v in calib.items()})
    with open(path, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(allrec[line], indent=1))


def read_counters(line):
    """The committed counter summary of a line's kernels, or None when a kernel source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(line)
    except Exception:
        return None
    if not rec or line not in COUNTER_SOURCES or rec.get("source_sha") != sha_of(*COUNTER_SOURCES[line]):
        return None
    return rec["kernels"]


def counter_figures(line, kernel, avg_launch_s, flops=None, nbytes=None):
    """Counter-derived rates of one kernel next to the algorithmic ones: HBM bytes per launch
    (FETCH_SIZE + WRITE_SIZE) over the live average launch time, and bf16 MFMA FLOP per launch
    (512 per SQ_INSTS_VALU_MFMA_MOPS_BF16) over the same time."""
    ks = read_counters(line)
    if not ks:
        return None
    hits = [n for n in ks if n == kernel or n.split("<")[0] == kernel]
    if len(hits) != 1:
        return None
    k = ks[hits[0]]
    out = dict(source="profiles/counters.json", kernel=hits[0])
    if "hbm_bytes" in k:
        out.update(hbm_bytes_per_launch=k["hbm_bytes"], fetch_bytes=k["fetch_bytes"], write_bytes=k["write_bytes"],
                   hbm_gbs=round(k["hbm_bytes"] / avg_launch_s / 1e9, 1),
                   hbm_frac=round(k["hbm_bytes"] / avg_launch_s / 1e9 / PEAK_HBM_GBS, 4))
        if nbytes:
            out["hbm_bytes_over_algorithmic"] = round(k["hbm_bytes"] / nbytes, 3)
    if "mfma_bf16_flops" in k:
        tf = k["mfma_bf16_flops"] / avg_launch_s / 1e12
        out.update(mfma_flops_per_launch=k["mfma_bf16_flops"], mfma_tflops=round(tf, 1),
                   mfma_frac=round(tf / PEAK_BF16_TFLOPS, 4))
        if flops:
            out["mfma_flops_over_algorithmic"] = round(k["mfma_bf16_flops"] / flops, 3)
    if "sq_valu_mfma_busy_cycles_mean" in k and "grbm_gui_active_mean" in k:
        # busy cycles summed over the chip's 1024 SIMDs against the kernel's GPU-active cycles on all
        # of them (GRBM_GUI_ACTIVE is summed over the 8 XCDs: one eighth of it is the kernel's cycles)
        out["mfma_busy_frac"] = round(k["sq_valu_mfma_busy_cycles_mean"] / (k["grbm_gui_active_mean"] / 8 * 256 * 4), 4)
    for cn in ("sq_valu_mfma_busy_cycles_mean", "sq_busy_cycles_mean", "grbm_gui_active_mean",
               "sq_lds_bank_conflict_mean", "sq_insts_lds_mean", "sq_waves_mean"):
        if cn in k:
            out[cn] = k[cn]
    return out


def trace_summary(csv_path, skip, take, title, command, per_call=""):
    """Markdown table of a rocprofv3 kernel trace: per kernel, calls in time order, the first
    `skip` as warm-up and the next `take` as the timed ones.  A call is one dispatch, or m
    consecutive dispatches for kernels listed in `per_call` as "kernel=m;..." (a kernel
    launched once per history segment); its time is then the sum over them."""
    import csv
    mult = dict((k, int(m)) for k, m in (e.rsplit("=", 1) for e in per_call.split(";") if e))
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if "hla" not in r["Kernel_Name"]:
            continue
        per.setdefault(kernel_key(r["Kernel_Name"]), []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    lines = [f"# {title}", "", "Command, on one MI355X (`<repo>` is the checkout, `<out>` an output folder):", "",
             f"    {command}", "",
             f"Per kernel, calls in time order: the first {skip} are warm-up, the next {take} the timed ones "
             "the bench line averages; durations in microseconds."]
    if mult:
        lines.append("Kernels launched several times per call (once per history segment) are summed over "
                     "the call's launches: " + ", ".join(f"`{k}` x {m}" for k, m in mult.items()) + ".")
    lines += ["", "| kernel | timed | avg (us) | min (us) | max (us) | warm-up avg (us) | other dispatches |",
              "|---|---|---|---|---|---|---|"]
    rows = []
    for name, ds in per.items():
        ds.sort()
        m = mult.get(name, 1)
        calls = [sum(d for _, d in ds[i:i + m]) for i in range(0, m * (skip + take), m) if i + m <= len(ds)]
        warm, timed = calls[:skip], calls[skip:skip + take]
        rest = len(ds) - m * (len(warm) + len(timed))
        if not timed:
            continue
        td = [d / 1e3 for d in timed]
        wa = sum(warm) / len(warm) / 1e3 if warm else float("nan")
        rows.append((sum(td), f"| `{name}` | {len(td)} | {sum(td) / len(td):.1f} | {min(td):.1f} | {max(td):.1f} | "
                              f"{wa:.1f} | {rest} |"))
    lines += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    print("\n".join(lines))


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-secondary", action="store_true", help="only the headline routed prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--oracle-chunks", type=int, default=512, help="query chunks of the oracle sample (512 = all of head 0)")
    ap.add_argument("--counter-run", metavar="LINE",
                    help="run one line's timed call three times and a 1 GiB calibration copy (under rocprofv3 --pmc)")
    ap.add_argument("--counter-write", nargs="+", metavar=("LINE", "CSV"),
                    help="summarise the counter passes of LINE (rocprofv3 counter_collection.csv files) into "
                         "profiles/counters.json")
    ap.add_argument("--trace-summary", nargs="+", metavar="CSV SKIP TAKE TITLE COMMAND [PER_CALL]",
                    help="markdown table of a rocprofv3 kernel trace, warm-up and timed dispatches apart")
    ap.add_argument("--only", metavar="LINES",
                    help="profiling aid: run only these comma-separated lines (routed_prefill or a secondary "
                         "name) and print their results as one JSON object instead of the bench line")
    ap.add_argument("--oracle-samples", type=int, metavar="CHUNKS",
                    help="the oracle leg alone on the CPU (used for the single-thread run): time every "
                         "workload's oracle sample and print one JSON object")
    args = ap.parse_args()
    if args.oracle_samples:
        rec = oracle_samples(args.oracle_samples, small=True)
        print(json.dumps({"threads": _blas_threads(), **rec}), flush=True)
        return
    if args.counter_write:
        counter_write(args.counter_write[0], args.counter_write[1:])
        return
    if args.trace_summary:
        if len(args.trace_summary) not in (5, 6):
            sys.exit("--trace-summary takes CSV SKIP TAKE TITLE COMMAND [PER_CALL]")
        c, sk, tk, title, cmd = args.trace_summary[:5]
        trace_summary(c, int(sk), int(tk), title, cmd, *args.trace_summary[5:])
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: every (batch, head) of this path is independent, so --gpus {args.gpus} "
              "would only shard heads without communication; only --gpus 1 is measured here.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_deltanet_hybrid_amd import hla, inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hla.library()
    torch.cuda.set_device(0)
    if args.counter_run:
        counter_run(args.counter_run, torch, hla, inputs)
        return

    if args.only:
        names = args.only.split(",")
        extra = {**SECONDARY, **ONLY_LINES}
        unknown = [n for n in names if n != "routed_prefill" and n not in extra]
        if unknown:
            print(f"unknown lines {unknown}; known: routed_prefill, {', '.join(extra)}", file=sys.stderr)
            sys.exit(2)
        x = routed_inputs(inputs) if any(n.startswith(("routed", "gdn2_routed", "learned")) for n in names) else None
        out = {}
        for n in names:
            out[n] = bench_routed_prefill(args, torch, hla, inputs, x=x)[0] if n == "routed_prefill" else \
                extra[n](args, torch, hla, inputs, x)
        print(json.dumps(out), flush=True)
        return

    head, x = bench_routed_prefill(args, torch, hla, inputs)
    secondary = {}
    if not args.no_secondary:
        for name, fn in SECONDARY.items():
            secondary[name] = fn(args, torch, hla, inputs, x)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[cpu_baseline] oracle samples of every workload ({args.oracle_chunks} chunks of the headline)")
        cpu = cpu_baseline(args.oracle_chunks, tail_states=_TAIL_STATES.get("states"))
        # GPU / oracle throughput per workload (all-thread oracle)
        gpu_rates = {"routed_prefill": head["value"],
                     "native_prefill": secondary.get("native_prefill", {}).get("tokens_per_s"),
                     "decode": secondary.get("decode", {}).get("tokens_per_s"),
                     "tail_replay": secondary.get("tail_replay", {}).get("replay_tokens_per_s")}
        for name, rate in gpu_rates.items():
            if rate and name in cpu["per_workload"]:
                cpu["per_workload"][name]["gpu_speedup"] = round(rate / cpu["per_workload"][name]["value"], 1)
        parity = cpu["per_workload"]["tail_replay"].pop("parity", None)
        if parity is not None and "tail_replay" in secondary:
            secondary["tail_replay"]["vs_oracle"] = parity
        log(f"[cpu_baseline] {cpu['value']:.1f} tokens/s (sample {cpu['sample_seconds']} s)")

    W = inputs.WORKLOADS["routed_prefill"]
    line = {
        "metric": METRIC,
        "value": round(head["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "routed_prefill (GDN + HLA, T=32K)", "B": W.B, "T": W.T, "H": W.H, "dk": W.dk,
                   "dv": W.dv, "C": W.C, "tau": W.tau, "parallelism": "single GPU"},
        "mfma_util_pct": round(head["mfma_util_pct"], 2),
        "step_tflops": round(head["step_tflops"], 1),
        "kernel_ms": head["kernel_ms"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
