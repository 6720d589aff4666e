"""Backward of the learned representatives and of the router on them, on the GPU through
the C ABI (hla_chunk_reps_backward, hla_router_backward), against the gradient oracles
(oracle.grad_reps, oracle.grad.router_backward: float64 autograd pinned by finite
differences and closed forms).

Bars as everywhere: max|diff| / max|ref| <= 1e-4 (float32 inputs), <= 2e-2 (bf16 inputs).
The last test chains the three backward calls (routed prefill with the forward's gates,
router, pooler) into the gradient of a routed prefill on learned representatives and holds
it to the same chain of oracles."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, dev, f32, host, note, token_tensors

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, dk, window, C, T, shared weights, with Wr
    ("bf16", 128, 32, 64, 5 * 64 - 37, False, True),
    ("f32", 64, 8, 64, 2 * 64 + 13, True, False),
    ("bf16", 128, 64, 64, 3 * 64 - 20, False, False),
    ("bf16", 64, 16, 128, 2 * 128 - 50, True, True),
    ("f32", 128, 64, 64, 128 + 70, False, True),
    ("bf16", 128, 8, 64, 9, False, True),
]
IDS = [f"{c[0]}-dk{c[1]}-w{c[2]}-C{c[3]}-T{c[4]}{'-shared' if c[5] else ''}{'-Wr' if c[6] else ''}" for c in CASES]
NAMES = ("Wq", "Wk", "Wv", "Wp", "Wr")


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def _weights(H, dk, dtype, shared, with_wr, seed):
    Ws = inputs.gen_pooler_weights(H, dk, dtype=dtype, seed=seed, shared=shared)
    dev_w = {n: dev(a, dtype) for n, a in Ws.items() if with_wr or n != "Wr"}
    f64 = {n: inputs.to_f64(a, dtype) for n, a in Ws.items()}
    return dev_w, f64


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_chunk_reps_backward(case):
    dtype, dk, window, C, T, shared, with_wr = case
    note(f"chunk reps backward {case}")
    B, H = 2, 2
    N = math.ceil(T / C)
    x = inputs.gen_tokens(B, T, H, dk, dk, dtype=dtype, seed=181)
    _, k, _, _, _ = token_tensors(x)
    Wd, W64 = _weights(H, dk, dtype, shared, with_wr, seed=182)
    dreps = inputs.gen_cotangent((B, N * (C // window), H, dk), seed=183, name="dreps")
    r = hla().chunk_reps_backward(k, Wd, f32(dreps), window=window, C=C)
    torch.cuda.synchronize()
    acc = {}
    for b in range(B):
        for h in range(H):
            hw = 0 if shared else h
            ref = oracle.window_reps_backward(x.f64("k")[b, :, h], C, window, *(W64[n][hw] for n in NAMES[:4]),
                                              dreps[b, :, h].astype(np.float64),
                                              Wr=W64["Wr"][hw] if with_wr else None)
            assert_close(host(r["dk"])[b, :, h], ref["dk"], dtype, f"dk b{b} h{h}")
            for n in NAMES:
                if ref["d" + n] is None:
                    continue
                key = n if shared else (n, h)  # shared weights sum over the heads too
                acc[key] = acc.get(key, 0.0) + ref["d" + n]
    for n in NAMES:
        if n == "Wr" and not with_wr:
            assert r["dWr"] is None
            continue
        got = host(r["d" + n])
        if shared:
            assert_close(got[0], acc[n], dtype, f"d{n} (shared)")
        else:
            for h in range(H):
                assert_close(got[h], acc[(n, h)], dtype, f"d{n} h{h}")


@pytest.mark.parametrize("learned", [True, False])
def test_router_backward(learned):
    dtype, dk, B, H, T = "bf16", 128, 2, 2, 6 * 64 - 21
    C = 64
    note(f"router backward, learned={learned}")
    N = math.ceil(T / C)
    x = inputs.gen_tokens(B, T, H, dk, dk, dtype=dtype, seed=191)
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    if learned:
        window = 16
        Wd, _ = _weights(H, dk, dtype, False, True, seed=192)
        reps, n_rep = h.chunk_reps(k, Wd, window=window), C // window
    else:
        reps, n_rep = k, C
    At, Bc = h.chunk_transitions(k, v, beta, alpha)
    fw = h.route_mix(q, reps, At, Bc, n_rep=n_rep, tau=1e-3)
    dG = f32(inputs.gen_cotangent((B, H, N, N), seed=193, name="dgates"))
    dG = dG * fw["mask"].float()  # a skipped pair passes nothing
    r = h.router_backward(q, reps, n_rep, fw["gates"], dG)
    torch.cuda.synchronize()
    reps64 = host(reps)
    for b in range(B):
        for hh in range(H):
            ref = oracle.router_backward(x.f64("q")[b, :, hh], reps64[b, :, hh], n_rep, C, host(dG)[b, hh])
            assert_close(host(r["dq"])[b, :, hh], ref["dq"], dtype, f"dq b{b} h{hh}")
            want = np.zeros((N * n_rep, dk))
            m = min(N * n_rep, ref["dreps"].shape[0])
            want[:m] = ref["dreps"][:m]
            assert_close(host(r["dreps"])[b, :, hh], want, dtype, f"dreps b{b} h{hh}")
            assert np.all(host(r["dreps"])[b, (N - 1) * n_rep:, hh] == 0.0)


def test_learned_reps_prefill_backward_chain():
    """Gradient of the routed prefill on learned representatives, as three calls: the
    routed-prefill backward with the forward's gates (dgates and the chunk-local parts), the
    router backward (dq, dreps) and the pooler backward (dk, dW); against the same chain of
    oracles in float64."""
    dtype, dk, dv, B, H, T, window, C = "bf16", 128, 128, 1, 2, 5 * 64 - 9, 32, 64
    note("learned-representative prefill backward chain")
    N = math.ceil(T / C)
    n_rep = C // window
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=201, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    Wd, W64 = _weights(H, dk, dtype, False, True, seed=202)
    dO = inputs.gen_cotangent((B, T, H, dv), seed=203, name="dO")
    h = hla()
    reps = h.chunk_reps(k, Wd, window=window)
    At, Bc = h.chunk_transitions(k, v, beta, alpha)
    fw = h.route_mix(q, reps, At, Bc, n_rep=n_rep, tau=1e-3)
    g1 = h.prefill_backward(q, k, v, beta, alpha, f32(dO), tau=1e-3, gates_in=fw["gates"])
    g2 = h.router_backward(q, reps, n_rep, fw["gates"], g1["dgates"])
    g3 = h.chunk_reps_backward(k, Wd, g2["dreps"], window=window)
    torch.cuda.synchronize()
    for hh in range(H):
        qq, kk, vv, bb, aa = (x.f64(n)[0, :, hh] for n in ("q", "k", "v", "beta", "alpha"))
        Wh = [W64[n][hh] for n in NAMES]
        reps_o = oracle.window_reps(kk, C, window, *Wh[:4]) @ Wh[4]
        gates_o = oracle.router_gates(qq, reps_o, n_rep, C, 1e-3)["gates"]
        r1 = oracle.hla_prefill_backward(qq, kk, vv, bb, aa, C, 1e-3, dO[0, :, hh].astype(np.float64),
                                         gates_in=gates_o)
        r2 = oracle.router_backward(qq, reps_o, n_rep, C, r1["dgates"])
        r3 = oracle.window_reps_backward(kk, C, window, *Wh[:4], r2["dreps"], Wr=Wh[4])
        assert_close(host(g1["dq"] + g2["dq"])[0, :, hh], r1["dq"] + r2["dq"], dtype, "dq")
        assert_close(host(g1["dk"] + g3["dk"])[0, :, hh], r1["dk"] + r3["dk"], dtype, "dk")
        for n in ("dv", "dbeta", "dalpha"):
            assert_close(host(g1[n])[0, :, hh], r1[n], dtype, n)
        for n in NAMES:
            assert_close(host(g3["d" + n])[hh], r3["d" + n], dtype, "d" + n)


def test_learned_reps_gdn2_prefill_backward_chain():
    """The same three-call chain under the Gated DeltaNet-2 recurrence: its routed-prefill
    backward with the forward's gates, then the (shared) router and pooler backward."""
    dtype, dk, dv, B, H, T, window, C = "bf16", 128, 64, 1, 2, 4 * 64 - 21, 16, 64
    note("learned-representative gated deltanet-2 prefill backward chain")
    n_rep = C // window
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=211, alpha_mode="slow")
    q, k, v, _, _ = token_tensors(x)
    gg = inputs.gen_gdn2_gates(B, T, H, dk, dv, seed=212, alpha_mode="slow")
    ga, gb, gw = (f32(gg[n]) for n in ("a", "b", "w"))
    Wd, W64 = _weights(H, dk, dtype, True, True, seed=213)  # one weight set shared by the heads
    dO = inputs.gen_cotangent((B, T, H, dv), seed=214, name="dO")
    h = hla()
    reps = h.chunk_reps(k, Wd, window=window)
    At, Bc = h.gdn2_chunk_transitions(k, v, ga, gb, gw)
    fw = h.route_mix(q, reps, At, Bc, n_rep=n_rep, tau=1e-3)
    g1 = h.gdn2_prefill_backward(q, k, v, ga, gb, gw, f32(dO), tau=1e-3, gates_in=fw["gates"])
    g2 = h.router_backward(q, reps, n_rep, fw["gates"], g1["dgates"])
    g3 = h.chunk_reps_backward(k, Wd, g2["dreps"], window=window)
    torch.cuda.synchronize()
    Wh = [W64[n][0] for n in NAMES]
    dW = {n: 0.0 for n in NAMES}
    for hh in range(H):
        qq, kk, vv = (x.f64(n)[0, :, hh] for n in ("q", "k", "v"))
        aa, bb, ww = (gg[n][0, :, hh].astype(np.float64) for n in ("a", "b", "w"))
        reps_o = oracle.window_reps(kk, C, window, *Wh[:4]) @ Wh[4]
        gates_o = oracle.router_gates(qq, reps_o, n_rep, C, 1e-3)["gates"]
        r1 = oracle.gdn2_hla_prefill_backward(qq, kk, vv, aa, bb, ww, C, 1e-3, dO[0, :, hh].astype(np.float64),
                                              gates_in=gates_o)
        r2 = oracle.router_backward(qq, reps_o, n_rep, C, r1["dgates"])
        r3 = oracle.window_reps_backward(kk, C, window, *Wh[:4], r2["dreps"], Wr=Wh[4])
        assert_close(host(g1["dq"] + g2["dq"])[0, :, hh], r1["dq"] + r2["dq"], dtype, "dq")
        assert_close(host(g1["dk"] + g3["dk"])[0, :, hh], r1["dk"] + r3["dk"], dtype, "dk")
        for n in ("dv", "da", "db", "dw"):
            assert_close(host(g1[n])[0, :, hh], r1[n], dtype, n)
        for n in NAMES:
            dW[n] = dW[n] + r3["d" + n]
    for n in NAMES:
        assert_close(host(g3["d" + n])[0], dW[n], dtype, "d" + n + " (shared)")
