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

HBM traffic of the composition kernel (the roofline record's ``traffic``), from two counter
passes over one routed-prefill step plus a 1 GiB calibration copy:

    cd /tmp && rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <f> -o t -- \
        python3 <repo>/bench.py --traffic-run
    cd /tmp && rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <w> -o t -- \
        python3 <repo>/bench.py --traffic-run
    python3 bench.py --traffic-write <f>/t_counter_collection.csv <w>/t_counter_collection.csv
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


def sha_of(*paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_key, sources):
    """HBM bytes per launch from the committed counter summary, or None when the kernel
    source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != sha_of(*sources):
        return None
    return rec.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- helpers
def to_dev(storage, dtype, torch):
    import numpy as np
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(storage).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(storage, dtype=np.float32)).cuda()


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


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
    traffic = read_traffic(TRAFFIC_KEY, TRAFFIC_SOURCES)
    tokens = W.B * W.T
    res = dict(
        value=tokens / dt, ms_per_step=dt * 1e3,
        mfma_util_pct=100.0 * fl_total / dt / (PEAK_BF16_TFLOPS * 1e12),
        step_tflops=fl_total / dt / 1e12, active_pairs=pairs,
        kernel_ms={kname: round(ms / n, 4) for kname, (ms, n) in per_kernel.items() if n > 0},
        roofline=dict(kernel="compose_bf16_kernel", bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=traffic,
                      flops_per_launch=fl_comp, avg_launch_ms=round(comp_avg_s * 1e3, 4), launches=comp_n),
    )
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


def bench_routed_learned_reps(args, torch, hla, inputs, x):
    """C = 64 with learned window representatives (window 32, seeded weights)."""
    W = inputs.WORKLOADS["routed_prefill"]
    pooler = inputs.gen_pooler_weights(W.H, W.dk, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"])
    r, _ = bench_routed_prefill(_sub(args), torch, hla, inputs, Cw=C, x=x, tag="routed_prefill_learned_reps",
                                pooler=pooler, window=32)
    return dict(
        workload="routed_prefill C=64, learned representatives (window 32, 2 per chunk), seeded weights",
        C=C, tau=W.tau, ms_per_step=r["ms_per_step"], tokens_per_s=r["value"], mfma_util_pct=r["mfma_util_pct"],
        active_pairs=r["active_pairs"], kernel_ms=r["kernel_ms"], reps_pool=r["reps_pool"])


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
    "gdn2_routed_prefill": lambda args, torch, hla, inputs, x: bench_gdn2_routed(args, torch, hla, inputs, x),
    "routed_prefill_backward": lambda args, torch, hla, inputs, x: bench_prefill_backward(args, torch, hla, inputs, x),
    "decode": lambda args, torch, hla, inputs, x: bench_decode(args, torch, hla, inputs),
    "gdn2_decode": lambda args, torch, hla, inputs, x: bench_decode(args, torch, hla, inputs, gdn2=True),
    "native_prefill": lambda args, torch, hla, inputs, x: bench_native_prefill(args, torch, hla, inputs),
    "tail_replay": lambda args, torch, hla, inputs, x: bench_tail_replay(args, torch, hla, inputs),
}

# lines run only when named with --only: the backward at the full 32768 tokens needs about
# 200 GiB of workspace in one pass (three per-pair states of the composition backward grow
# as N^2); the line also times it in query-chunk groups within 64 GiB
ONLY_LINES = {
    "routed_prefill_backward_T32K": lambda args, torch, hla, inputs, x: bench_prefill_backward(
        args, torch, hla, inputs, x, T=inputs.WORKLOADS["routed_prefill"].T, grouped_gib=64),
}


# ----------------------------------------------------------------------------- decode
def bench_decode(args, torch, hla, inputs, gdn2=False):
    """Decode at Bs=256, H=16 with 64 cached chunks per sequence; ``gdn2`` runs the Gated
    DeltaNet-2 live update (channel-wise gates per token) instead of Gated DeltaNet's."""
    W = inputs.WORKLOADS["decode"]
    tag = "gdn2_decode" if gdn2 else "decode"
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

    def step():
        t = toks[it[0] % n_tok]
        it[0] += 1
        if gdn2:
            hla.gdn2_decode(t["q"], t["k"], t["v"], t["a"], t["b"], t["w"], S, At_cur=A, At_cache=At_cache,
                            Bc_cache=Bc_cache, reps_cache=reps, n_cache=n_cache, tau=W.tau, o=o)
        else:
            hla.gdn_decode(t["q"], t["k"], t["v"], t["beta"], t["alpha"], S, At_cur=A, At_cache=At_cache,
                           Bc_cache=Bc_cache, reps_cache=reps, n_cache=n_cache, tau=W.tau, o=o)

    steps = args.decode_steps
    for _ in range(8):
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
    per_seqhead = (2 * dk * dv * 4 + 2 * dk * dk * 4 + n_cap * (dk * dk + dk * dv) * e + n_cap * C * dk * e
                   + (2 * dk + dv) * e + ((2 * dk + dv) * 4 if gdn2 else 2 * 4) + dv * 4)
    bytes_step = Bs * H * per_seqhead
    kern_s = dec_ms / dec_n / 1e3
    res = dict(workload=tag, Bs=Bs, H=H, cached_chunks=n_cap, steps=steps, ms_per_step=dt * 1e3,
               tokens_per_s=Bs / dt, hbm_gbs=bytes_step / kern_s / 1e9,
               roofline=dict(kernel="decode_kernel", bound="hbm", achieved=round(bytes_step / kern_s / 1e9, 1),
                             peak=PEAK_HBM_GBS, unit="GB/s", frac=round(bytes_step / kern_s / 1e9 / PEAK_HBM_GBS, 4),
                             bytes_per_launch=bytes_step, avg_launch_ms=round(kern_s * 1e3, 4)),
               note="no commit while timing; live chunk extends past 64 tokens so every step does the same work")
    log(f"[{tag}] {dt*1e3:.3f} ms/step, {Bs/dt:.0f} tok/s, kernel {kern_s*1e3:.3f} ms, "
        f"{bytes_step/kern_s/1e9:.0f} GB/s")
    del At_cache, Bc_cache, reps, S, A, toks
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- native prefill
def bench_native_prefill(args, torch, hla, inputs):
    W = inputs.WORKLOADS["native_prefill"]
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["native_prefill"])
    q, k, v = (to_dev(a, W.dtype, torch) for a in (x.q, x.k, x.v))
    beta, alpha = to_dev(x.beta, "f32", torch), to_dev(x.alpha, "f32", torch)
    d = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, hla.HLA_BF16)
    ws = torch.empty(hla.workspace_bytes(hla.FN_GDN_PREFILL, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((W.B, W.T, W.H, W.dv), dtype=torch.float32, device="cuda")
    S = torch.empty((W.B, W.H, W.dk, W.dv), dtype=torch.float32, device="cuda")
    dt = timed(lambda: hla.gdn_prefill(q, k, v, beta, alpha, o=o, S_final=S, ws=ws), 20, 3, torch)
    bytes_alg = W.B * W.T * W.H * (2 * W.dk * 2 + W.dv * 2 + 2 * 4 + W.dv * 4) + W.B * W.H * W.dk * W.dv * 4
    res = dict(workload="native_prefill", B=W.B, T=W.T, H=W.H, ms_per_step=dt * 1e3, tokens_per_s=W.B * W.T / dt,
               algorithmic_gbs=bytes_alg / dt / 1e9, hbm_frac=round(bytes_alg / dt / 1e9 / PEAK_HBM_GBS, 4))
    log(f"[native_prefill] {dt*1e3:.3f} ms, {W.B*W.T/dt/1e6:.2f} M tok/s, {bytes_alg/dt/1e9:.0f} GB/s algorithmic")
    return res


# ----------------------------------------------------------------------------- Gated DeltaNet-2
# fp32 vector peak, as published: 256 CUs x 4 SIMDs x 16 lanes x 2 flop per FMA x 2 (packed
# fp32: two FMAs per lane and instruction) x 2.4 GHz = 157.3 TFLOP/s.  The library is compiled
# without packed-fp32 instructions, so its own ceiling is half that; records give both.
PEAK_FP32_VALU_TFLOPS = 256 * 4 * 16 * 2 * 2 * 2.4e9 / 1e12
PEAK_FP32_VALU_UNPACKED_TFLOPS = PEAK_FP32_VALU_TFLOPS / 2


def flops_gdn2_pass(n_tokens_heads, dk, dv, outputs):
    """Token-loop chunk pass per token and head: every column of the map [P | Q] (dk + dv
    columns) or of the state (dv columns) takes k.(D x) (dk FMA), D x (dk mul), the erase
    (dk FMA) and the write (dk FMA; none for P columns); outputs add q . x (dk FMA)."""
    if outputs:
        return n_tokens_heads * dv * dk * (2 + 1 + 2 + 2 + 2)
    return n_tokens_heads * (dk * dk * (2 + 1 + 2) + dv * dk * (2 + 1 + 2 + 2))


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
    th = W.B * W.T * W.H
    fl_pass = flops_gdn2_pass(th, W.dk, W.dv, False) + flops_gdn2_pass(th, W.dk, W.dv, True)
    chunk_s = ch_ms / ch_n / 1e3 * 2  # two chunk passes per step
    ach = fl_pass / chunk_s / 1e12
    res = dict(workload="routed_prefill under Gated DeltaNet-2 (channel-wise decay, erase and write gates), "
                        "B=1 T=32768 H=16 d=128 C=64",
               ms_per_step=dt * 1e3, tokens_per_s=W.B * W.T / dt, compose_ms=round(cm_ms / cm_n, 4),
               chunk_passes_ms=round(chunk_s * 1e3, 4),
               chunk_roofline=dict(kernel="gdn2_chunk_kernel (maps + outputs)", bound="alu", achieved=round(ach, 2),
                                   peak=round(PEAK_FP32_VALU_TFLOPS, 1), unit="TFLOP/s",
                                   frac=round(ach / PEAK_FP32_VALU_TFLOPS, 4), flops_per_step=fl_pass,
                                   frac_of_unpacked_peak=round(ach / PEAK_FP32_VALU_UNPACKED_TFLOPS, 4)))
    log(f"[gdn2_routed_prefill] {dt*1e3:.3f} ms/step, {W.B*W.T/dt/1e6:.3f} M tok/s, chunk passes "
        f"{chunk_s*1e3:.3f} ms ({ach:.1f} TFLOP/s fp32 VALU), compose {cm_ms/cm_n:.3f} ms")
    del q, k, v, ga, gb, gw, At, Bc, out, o, ws
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- backward
BWD_T = 8192


def flops_chunk_bwd(n_tokens_heads, dk, dv):
    """Algorithmic work of the per-chunk reverse, per token and head: every column runs the
    forward step once (k . x and the update, 4 dk) and its reverse (k . dx, dx . x_prev, the
    two-term key gradient and the dx update, 10 dk); the dv state columns add q dO and the
    query gradient (4 dk).  Map columns: dk + dv; state columns: dv.  The checkpoint replay
    the kernel adds (a second forward step) is not counted."""
    return n_tokens_heads * dk * (dv * 18 + (dk + dv) * 14)


def flops_router_bwd(pairs, n_rep, dk):
    """Per history pair: the scores twice (query side and key side) and the two gradient
    accumulations, 2 n_rep dk each."""
    return pairs * 4 * 2 * n_rep * dk


def bench_prefill_backward(args, torch, hla, inputs, x, T=BWD_T, grouped_gib=None):
    """The routed-prefill backward (hla_prefill_backward) at B=1, T tokens (8192 by default),
    H=16, d=128, C=64, bf16, computed gates at tau = 1e-3: recomputed chunk maps and gates,
    composition replay, chunk outputs reverse, composition adjoint and sums, chunk maps
    reverse, router backward and the per-token sums.  With `grouped_gib` the step is also
    timed with a workspace of that many GiB, which runs the query chunks in groups."""
    W = inputs.WORKLOADS["routed_prefill"]
    q, k, v = (to_dev(a[:, :T], W.dtype, torch) for a in (x.q, x.k, x.v))
    beta, alpha = to_dev(x.beta[:, :T], "f32", torch), to_dev(x.alpha[:, :T], "f32", torch)
    dO = to_dev(inputs.gen_cotangent((W.B, T, W.H, W.dv), seed=0, name="dO"), "f32", torch)
    dev = k.device
    N = math.ceil(T / C)
    d = hla.make_dims(W.B, T, W.H, T, W.dk, W.dv, hla.HLA_BF16, C)
    ws = torch.empty(hla.workspace_bytes(hla.FN_PREFILL_BACKWARD, d), dtype=torch.uint8, device=dev)
    log(f"[routed_prefill_backward] T={T}: workspace {ws.numel() / 2**30:.2f} GiB")
    step = lambda: hla.prefill_backward(q, k, v, beta, alpha, dO, tau=W.tau, ws=ws)
    g = step()
    # active pairs from the router's own mask (a gate gradient can underflow to zero far
    # back in a long chain, so it does not count them)
    At, Bc = hla.chunk_transitions(k, v, beta, alpha)
    pairs = int(hla.route_mix(q, k, At, Bc, tau=W.tau)["active_cnt"].sum().item())
    del At, Bc
    torch.cuda.synchronize()
    steps = max(3, args.steps // 4)
    hla.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    names = (("bwd_chunk", hla.KERNEL_BWD_CHUNK), ("bwd_save", hla.KERNEL_BWD_SAVE),
             ("bwd_adjoint", hla.KERNEL_BWD_ADJOINT), ("bwd_reduce", hla.KERNEL_BWD_REDUCE),
             ("bwd_router", hla.KERNEL_BWD_ROUTER), ("fwd_chunk", hla.KERNEL_CHUNK), ("fwd_gates", hla.KERNEL_GATES),
             ("fwd_compose", hla.KERNEL_COMPOSE))
    per = {n: hla.timing_read(kid) for n, kid in names}
    hla.timing_enable(False)
    ms = {n: tot / steps for n, (tot, cnt) in per.items() if cnt > 0}
    th = W.B * T * W.H
    fl_chunk = flops_chunk_bwd(th, W.dk, W.dv)
    fl_pair = flops_compose(pairs, W.dk, W.dv)
    ach = fl_chunk / (ms["bwd_chunk"] / 1e3) / 1e12
    mfma = {n: dict(achieved=round(fl_pair / (ms[n] / 1e3) / 1e12, 1),
                    frac=round(fl_pair / (ms[n] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4))
            for n in ("bwd_save", "bwd_adjoint", "bwd_reduce")}
    # roofline record of the kernel that takes the most time: the chunk reverse (fp32 VALU)
    # or one of the composition passes (bf16 matrix cores)
    kernels = {"bwd_chunk": ("chunk_bwd_kernel (outputs + maps reverse)", "alu", fl_chunk, PEAK_FP32_VALU_TFLOPS),
               "bwd_save": ("compose_save_kernel (+ prep_bwd_kernel)", "mfma", fl_pair, PEAK_BF16_TFLOPS),
               "bwd_adjoint": ("compose_adjoint_kernel", "mfma", fl_pair, PEAK_BF16_TFLOPS),
               "bwd_reduce": ("compose_grad_reduce_kernel (+ chain_sum_kernel)", "mfma", fl_pair, PEAK_BF16_TFLOPS)}
    dom = max(kernels, key=lambda n: ms[n])
    kname, bound, fl_dom, peak = kernels[dom]
    ach_dom = fl_dom / (ms[dom] / 1e3) / 1e12
    res = dict(workload=f"routed prefill backward (GDN + HLA), B={W.B} T={T} H={W.H} d={W.dk} C={C} bf16, "
                        f"computed gates tau={W.tau}",
               ms_per_step=round(dt * 1e3, 3), tokens_per_s=round(W.B * T / dt, 1), active_pairs=pairs,
               kernel_ms={n: round(v, 3) for n, v in ms.items()},
               roofline=dict(kernel=kname, bound=bound, achieved=round(ach_dom, 2), peak=round(peak, 1),
                             unit="TFLOP/s", frac=round(ach_dom / peak, 4), flops_per_launch=fl_dom,
                             avg_launch_ms=round(ms[dom], 4)),
               chunk_reverse=dict(bound="alu", achieved=round(ach, 2), peak=round(PEAK_FP32_VALU_TFLOPS, 1),
                                  unit="TFLOP/s", frac=round(ach / PEAK_FP32_VALU_TFLOPS, 4), flops_per_step=fl_chunk,
                                  frac_of_unpacked_peak=round(ach / PEAK_FP32_VALU_UNPACKED_TFLOPS, 4)),
               composition_mfma=dict(flops_per_pass=fl_pair, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", **mfma),
               router_tflops=round(flops_router_bwd(pairs, C, W.dk) / (ms["bwd_router"] / 1e3) / 1e12, 2))
    log(f"[routed_prefill_backward T={T}] {dt*1e3:.3f} ms/step, {W.B*T/dt/1e6:.3f} M tok/s; chunk reverse "
        f"{ms['bwd_chunk']:.3f} ms ({ach:.1f} TFLOP/s fp32 VALU); save {ms['bwd_save']:.3f}, adjoint "
        f"{ms['bwd_adjoint']:.3f}, reduce {ms['bwd_reduce']:.3f}, router {ms['bwd_router']:.3f} ms")
    res["workspace_gib"] = round(ws.numel() / 2**30, 2)
    if grouped_gib is not None and grouped_gib * 2**30 < ws.numel():
        del ws, g
        torch.cuda.empty_cache()
        ws = torch.empty(int(grouped_gib * 2**30), dtype=torch.uint8, device=dev)
        g = step()
        torch.cuda.synchronize()
        hla.timing_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        dtg = (time.perf_counter() - t0) / steps
        groups = hla.timing_read(hla.KERNEL_BWD_SAVE)[1] // steps  # one save launch per group
        hla.timing_enable(False)
        res["grouped"] = dict(workspace_gib=grouped_gib, groups=groups, ms_per_step=round(dtg * 1e3, 3),
                              tokens_per_s=round(W.B * T / dtg, 1),
                              min_workspace_gib=round(hla.workspace_bytes(hla.FN_PREFILL_BACKWARD_MIN, d) / 2**30, 2))
        log(f"[routed_prefill_backward T={T}] in {groups} query-chunk groups within {grouped_gib} GiB: "
            f"{dtg*1e3:.3f} ms/step")
    del q, k, v, beta, alpha, dO, ws, g
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- Tail-Replay
def bench_tail_replay(args, torch, hla, inputs):
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
    ws_rep = torch.empty(hla.workspace_bytes(hla.FN_GDN_PREFILL, d_rep), dtype=torch.uint8, device="cuda")
    dt_rep = timed(lambda: hla.gdn_prefill(None, ks, vs, bs, als, want_o=False, S_final=S, ws=ws_rep), 20, 3, torch)
    d_full = hla.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, hla.HLA_BF16)
    ws_full = torch.empty(hla.workspace_bytes(hla.FN_GDN_PREFILL, d_full), dtype=torch.uint8, device="cuda")
    S2 = torch.empty_like(S)
    dt_full = timed(lambda: hla.gdn_prefill(None, k, v, beta, alpha, want_o=False, S_final=S2, ws=ws_full), 5, 1, torch)
    res = dict(workload="tail_replay", B=W.B, H=W.H, prefix=W.T, replay=L, ms_replay=dt_rep * 1e3,
               ms_full_prefix_state=dt_full * 1e3, speedup_vs_full=dt_full / dt_rep,
               replay_tokens_per_s=W.B * L / dt_rep)
    log(f"[tail_replay] replay {dt_rep*1e3:.3f} ms vs full-prefix state {dt_full*1e3:.3f} ms "
        f"({dt_full/dt_rep:.1f}x)")
    del k, v, beta, alpha, ws_rep, ws_full
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- CPU oracle
def cpu_baseline(x, n_query_chunks):
    """The oracle (as is) on the routed prefill of the first n_query_chunks chunks of head 0,
    each stage extrapolated to the full workload by its own work ratio."""
    import numpy as np

    import oracle
    from gated_deltanet_hybrid_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = 1
    W = inputs.WORKLOADS["routed_prefill"]
    Tn = n_query_chunks * C
    q, k, v = (x.f64(n)[0, :Tn, 0] for n in ("q", "k", "v"))
    beta, alpha = x.f64("beta")[0, :Tn, 0], x.f64("alpha")[0, :Tn, 0]
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
    return dict(value=W.B * W.T / full, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"routed prefill of the first {Tn} tokens ({n_query_chunks} chunks) of head 0, "
                       f"{t4 - t0:.1f} s; stages extrapolated to B={W.B}, H={W.H}, T={W.T} by chunk count "
                       f"(transitions, outputs) or chunk-pair count (gates, composition)",
                sample_seconds=round(t4 - t0, 2), extrapolated_seconds=round(full, 1),
                host_cpus=os.cpu_count())


# ----------------------------------------------------------------------------- HBM traffic
TRAFFIC_KEY = "compose_routed_prefill"
TRAFFIC_SOURCES = ["gated_deltanet_hybrid_amd/csrc/compose.hip"]
CALIB_BYTES = 1 << 30


def traffic_run(torch, hla, inputs):
    """One warm-up and one timed routed-prefill step, then a plain 1 GiB device copy (read
    1 GiB, write 1 GiB) that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    args = argparse.Namespace(steps=1, warmup=1)
    bench_routed_prefill(args, torch, hla, inputs)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[traffic] done")


def _per_dispatch(csv_path, counter):
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"], int(r["Grid_Size"]))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def _mean_of(per, pred):
    """Mean counter value over the dispatches whose kernel name passes ``pred`` and whose
    grid is the largest among those (the calibration copy, not incidental small copies)."""
    sel = [(g, v) for (_, name, g), v in per.items() if pred(name)]
    if not sel:
        return None, 0
    gmax = max(g for g, _ in sel)
    vals = [v for g, v in sel if g == gmax]
    return sum(vals) / len(vals), len(vals)


def traffic_write(fetch_csv, write_csv):
    """HBM bytes per composition launch from the two counter passes (KiB per dispatch),
    each scaled by the same counter's reading for the calibration copy of known size."""
    is_copy = lambda n: "copy" in n.lower() and "hla::" not in n
    is_comp = lambda n: "compose_bf16_kernel" in n
    f, w = _per_dispatch(fetch_csv, "FETCH_SIZE"), _per_dispatch(write_csv, "WRITE_SIZE")
    f_copy, n_fc = _mean_of(f, is_copy)
    w_copy, n_wc = _mean_of(w, is_copy)
    f_comp, n_f = _mean_of(f, is_comp)
    w_comp, n_w = _mean_of(w, is_comp)
    if None in (f_copy, w_copy, f_comp, w_comp):
        sys.exit("traffic: a calibration copy or composition dispatch is missing from the counter files")
    k_fetch = CALIB_BYTES / (f_copy * 1024.0)
    k_write = CALIB_BYTES / (w_copy * 1024.0)
    fetch_b = f_comp * 1024.0 * k_fetch
    write_b = w_comp * 1024.0 * k_write
    rec = dict(source_sha=sha_of(*TRAFFIC_SOURCES), hbm_bytes_per_launch=round(fetch_b + write_b),
               fetch_bytes=round(fetch_b), write_bytes=round(write_b), fetch_kib_raw=round(f_comp, 1),
               write_kib_raw=round(w_comp, 1), calib_fetch_factor=round(k_fetch, 4),
               calib_write_factor=round(k_write, 4), calib_copy_bytes=CALIB_BYTES, launches=[n_f, n_w],
               kernel="compose_bf16_kernel", workload="routed_prefill B=1 H=16 T=32768 d=128 C=64 bf16")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = json.load(open(path)) if os.path.exists(path) else {}
    allrec[TRAFFIC_KEY] = rec
    with open(path, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


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
    ap.add_argument("--traffic-run", action="store_true", help="one routed-prefill step plus a calibration copy (under rocprofv3 --pmc)")
    ap.add_argument("--traffic-write", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from the two counter passes")
    ap.add_argument("--only", metavar="LINES",
                    help="profiling aid: run only these comma-separated lines (routed_prefill or a secondary "
                         "name) and print their results as one JSON object instead of the bench line")
    args = ap.parse_args()
    if args.traffic_write:
        traffic_write(*args.traffic_write)
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
    if args.traffic_run:
        traffic_run(torch, hla, inputs)
        return

    if args.only:
        names = args.only.split(",")
        extra = {**SECONDARY, **ONLY_LINES}
        unknown = [n for n in names if n != "routed_prefill" and n not in extra]
        if unknown:
            print(f"unknown lines {unknown}; known: routed_prefill, {', '.join(extra)}", file=sys.stderr)
            sys.exit(2)
        x = routed_inputs(inputs) if any(n.startswith(("routed", "gdn2_routed")) for n in names) else None
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
        log(f"[cpu_baseline] oracle on {args.oracle_chunks} chunks of one head")
        cpu = cpu_baseline(x, args.oracle_chunks)
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
