"""Backward pass on the GPU, through the C ABI, against the gradient oracle (oracle.grad,
float64 autograd pinned by finite differences).

Bars as everywhere: max|diff| / max|ref| <= 1e-4 (float32), <= 2e-2 (bf16) for every
gradient tensor; skipped pairs get exactly zero gate gradient."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, dev, f32, host, note

pytestmark = pytest.mark.gpu
C = 64


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


COMPOSE_CASES = [("f32", 64, 128, 7), ("bf16", 128, 128, 7), ("bf16", 64, 64, 9), ("bf16", 128, 64, 33)]


@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("mode,tau", [("uniform", 1e-3), ("skip_heavy", 0.1)])
@pytest.mark.parametrize("case", COMPOSE_CASES, ids=[f"{c[0]}-dk{c[1]}-dv{c[2]}-N{c[3]}" for c in COMPOSE_CASES])
def test_compose_backward(case, mode, tau, with_s0):
    dtype, dk, dv, N = case
    note(f"compose backward {case} {mode} tau={tau} S0={with_s0}")
    B, H = 2, 2
    At_s, Bc_s = inputs.gen_transitions(B, H, N, dk, dv, dtype=dtype, seed=31)
    G = inputs.gen_gates(B, H, N, seed=32, mode=mode)
    S0 = inputs.gen_state(B, H, dk, dv, seed=33) if with_s0 else None
    dS = inputs.gen_cotangent((B, H, N, dk, dv), seed=34, name="dS")
    h = hla()
    At, Bc = dev(At_s, dtype), dev(Bc_s, dtype)
    S0d = None if S0 is None else f32(S0)
    r = h.route_mix(None, None, At, Bc, tau=tau, gates_in=f32(G), T=N * C, S0=S0d)
    g = h.compose_backward(At, Bc, r["gates"], r["mask"], f32(dS), S0=S0d, want_states=True)
    torch.cuda.synchronize()
    A = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    for b in range(B):
        for hh in range(H):
            fw = oracle.router_gates(np.zeros((N * C, dk)), np.zeros((N * C, dk)), C, C, tau,
                                     gates_in=G[b, hh].astype(np.float64))
            s0 = None if S0 is None else S0[b, hh].astype(np.float64).T
            ref = oracle.routed_states_backward(A[b, hh], Bm[b, hh], fw["ghat"], fw["mask"],
                                                dS[b, hh].astype(np.float64).transpose(0, 2, 1), S0=s0)
            Sr = oracle.routed_states(A[b, hh], Bm[b, hh], fw["ghat"], fw["mask"], S0=s0)
            assert_close(host(g["S_routed"])[b, hh], Sr.transpose(0, 2, 1), dtype, "recomputed S_routed")
            assert_close(host(g["dAt"])[b, hh], ref["dA"].transpose(0, 2, 1), dtype, "dAt")
            assert_close(host(g["dBc"])[b, hh], ref["dB"].transpose(0, 2, 1), dtype, "dBc")
            dg = host(g["dgates"])[b, hh]
            assert_close(dg, ref["dghat"], dtype, "dgates")
            assert np.all(dg[~fw["mask"]] == 0.0)
            assert_close(host(g["dS0"])[b, hh], ref["dS0"].T, dtype, "dS0")


def _tok(x, name, b, h):
    return x.f64(name)[b, :, h]


CHUNK_CASES = [("f32", 64, 128, 3 * C + 17), ("bf16", 128, 128, 150), ("bf16", 128, 64, C), ("bf16", 64, 64, 1),
               ("f32", 128, 128, 2 * C)]


@pytest.mark.parametrize("parts", ["out", "map", "both"])
@pytest.mark.parametrize("case", CHUNK_CASES, ids=[f"{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}" for c in CHUNK_CASES])
def test_chunk_backward(case, parts):
    dtype, dk, dv, T = case
    note(f"chunk backward {case} {parts}")
    B, H = 2, 2
    N = -(-T // C)
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=41, alpha_mode="slow")
    q, k, v, beta, alpha = (dev(x.q, dtype), dev(x.k, dtype), dev(x.v, dtype), f32(x.beta), f32(x.alpha))
    want_out, want_map = parts in ("out", "both"), parts in ("map", "both")
    init = inputs.gen_cotangent((B, H, N, dk, dv), seed=42, name="S0", scale=0.5) if want_out else None
    dO = inputs.gen_cotangent((B, T, H, dv), seed=43, name="dO") if want_out else None
    dAt = inputs.gen_cotangent((B, H, N, dk, dk), seed=44, name="At") if want_map else None
    dBc = inputs.gen_cotangent((B, H, N, dk, dv), seed=45, name="Bc") if want_map else None
    g = hla().chunk_backward(q, k, v, beta, alpha, chunk_init=None if init is None else f32(init),
                             dO=None if dO is None else f32(dO), dAt=None if dAt is None else f32(dAt),
                             dBc=None if dBc is None else f32(dBc))
    torch.cuda.synchronize()
    for b in range(B):
        for hh in range(H):
            qq, kk, vv, bb, aa = (_tok(x, n, b, hh) for n in ("q", "k", "v", "beta", "alpha"))
            ref = {n: 0.0 for n in ("dq", "dk", "dv", "dbeta", "dalpha")}
            if want_out:
                ro = oracle.chunk_outputs_backward(qq, kk, vv, bb, aa, C, init[b, hh].astype(np.float64).transpose(0, 2, 1),
                                                   dO[b, :, hh].astype(np.float64))
                for n in ref:
                    ref[n] = ref[n] + ro[n]
                assert_close(host(g["dchunk_init"])[b, hh], ro["dS_routed"].transpose(0, 2, 1), dtype, "dchunk_init")
            if want_map:
                rm = oracle.chunk_transitions_backward(kk, vv, bb, aa, C, dAt[b, hh].astype(np.float64).transpose(0, 2, 1),
                                                       dBc[b, hh].astype(np.float64).transpose(0, 2, 1))
                for n in ("dk", "dv", "dbeta", "dalpha"):
                    ref[n] = ref[n] + rm[n]
            if want_out:
                assert_close(host(g["dq"])[b, :, hh], ref["dq"], dtype, "dq")
            else:
                assert np.all(host(g["dq"])[b, :, hh] == 0.0)
            for n, key in (("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"), ("dalpha", "dalpha")):
                assert_close(host(g[key])[b, :, hh], ref[n], dtype, n)
