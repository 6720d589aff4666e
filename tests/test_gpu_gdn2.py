"""GPU parity of the Gated DeltaNet-2 path (hla_gdn2_chunk_transitions, hla_gdn2_prefill and
hla_route_mix on their maps) against the oracle, through the C ABI.

Bars as everywhere: max|diff| / max|ref| <= 1e-4 for float32 inputs and 2e-2 for bf16
inputs (the chunk pass itself runs in float32; bf16 enters through the inputs and the bf16
chunk maps); masks and active lists bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, dev, f32, host, note, token_tensors

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, dk, dv, T
    ("f32", 64, 64, 70),
    ("f32", 128, 64, 130),
    ("bf16", 128, 128, 200),
    ("bf16", 64, 128, 100),
    ("bf16", 128, 64, 256),
]
IDS = [f"{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}" for c in CASES]
C = 64


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def gen(case, B=2, H=2, seed=0, T=None):
    dtype, dk, dv, T0 = case
    T = T0 if T is None else T
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=seed, alpha_mode="slow")
    g = inputs.gen_gdn2_gates(B, T, H, dk, dv, seed=seed, alpha_mode="slow")
    return x, g


def seq(x, g, b, h):
    return (x.f64("q")[b, :, h], x.f64("k")[b, :, h], x.f64("v")[b, :, h],
            g["a"][b, :, h].astype(np.float64), g["b"][b, :, h].astype(np.float64),
            g["w"][b, :, h].astype(np.float64))


def gates_dev(g):
    return f32(g["a"]), f32(g["b"]), f32(g["w"])


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_gdn2_chunk_transitions(case):
    note(f"gdn2 transitions {case}")
    dtype = case[0]
    x, g = gen(case, seed=81)
    q, k, v, _, _ = token_tensors(x)
    At, Bc = hla().gdn2_chunk_transitions(k, v, *gates_dev(g))
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            A, Bm = oracle.gdn2_chunk_transitions(*seq(x, g, b, h)[1:], C)
            assert_close(host(At[b, h]), A.transpose(0, 2, 1), dtype, f"At b{b} h{h}")
            assert_close(host(Bc[b, h]), Bm.transpose(0, 2, 1), dtype, f"Bc b{b} h{h}")


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("with_s0", [False, True])
def test_gdn2_native_prefill(case, with_s0):
    note(f"gdn2 native {case} S0={with_s0}")
    dtype, dk, dv = case[:3]
    x, g = gen(case, seed=82)
    q, k, v, _, _ = token_tensors(x)
    S0 = inputs.gen_state(2, 2, dk, dv, seed=83) if with_s0 else None
    o, S = hla().gdn2_prefill(q, k, v, *gates_dev(g), S0=None if S0 is None else f32(S0))
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            o_ref, S_ref = oracle.gdn2_recurrent(*seq(x, g, b, h), S0=None if S0 is None else S0[b, h].T.astype(np.float64))
            assert_close(host(o)[b, :, h], o_ref, dtype, f"o b{b} h{h}")
            assert_close(host(S)[b, h], S_ref.T, dtype, f"S b{b} h{h}")


@pytest.mark.parametrize("case", [CASES[1], CASES[2]], ids=[IDS[1], IDS[2]])
def test_gdn2_routed_prefill(case):
    note(f"gdn2 routed {case}")
    dtype = case[0]
    x, g = gen(case, B=1, seed=84, T=5 * C - 11)
    q, k, v, _, _ = token_tensors(x)
    r = hla().gdn2_hla_prefill(q, k, v, *gates_dev(g), tau=1e-3)
    torch.cuda.synchronize()
    for h in range(2):
        ref = oracle.gdn2_hla_prefill(*seq(x, g, 0, h), C, 1e-3)
        np.testing.assert_allclose(host(r["gates"])[0, h], ref["gates"], atol=2e-5, rtol=0)
        near = np.abs(ref["gates"] - 1e-3) <= 1e-6
        assert np.array_equal(host(r["mask"])[0, h].astype(bool)[~near], ref["mask"][~near])
        assert_close(host(r["S_routed"])[0, h], ref["S_routed"].transpose(0, 2, 1), dtype, "S_routed")
        assert_close(host(r["o"])[0, :, h], ref["o"], dtype, "routed o")


def test_gdn2_routed_caller_gates_larger_chunks():
    # C = 256 (64-token piece maps composed four at a time), skip-heavy caller gates
    Cw, dk, dv, T = 256, 128, 128, 4 * 256 - 30
    note(f"gdn2 routed C={Cw}")
    x, g = gen(("bf16", dk, dv, T), B=1, seed=85)
    q, k, v, _, _ = token_tensors(x)
    N = math.ceil(T / Cw)
    G = inputs.gen_gates(1, 2, N, seed=86, mode="uniform")
    h = hla()
    At, Bc = h.gdn2_chunk_transitions(k, v, *gates_dev(g), C=Cw)
    r = h.route_mix(q, k, At, Bc, n_rep=Cw, tau=0.4, gates_in=f32(G), C=Cw)
    o, _ = h.gdn2_prefill(q, k, v, *gates_dev(g), chunk_init=r["S_routed"], want_state=False, C=Cw)
    torch.cuda.synchronize()
    for hh in range(2):
        ref = oracle.gdn2_hla_prefill(*seq(x, g, 0, hh), Cw, 0.4, gates_in=G[0, hh].astype(np.float64))
        np.testing.assert_array_equal(host(r["mask"])[0, hh].astype(bool), ref["mask"])
        assert_close(host(At[0, hh]), ref["A"].transpose(0, 2, 1), "bf16", "At C=256")
        assert_close(host(r["S_routed"])[0, hh], ref["S_routed"].transpose(0, 2, 1), "bf16", "S_routed")
        assert_close(host(o)[0, :, hh], ref["o"], "bf16", "routed o")


def test_gdn2_tail_replay_state_only():
    # state-only prefill of a suffix given as a token window (q unused)
    dtype, dk, dv, T, L = "bf16", 128, 128, 300, 77
    note("gdn2 tail replay")
    x, g = gen((dtype, dk, dv, T), seed=87)
    q, k, v, _, _ = token_tensors(x)
    ga, gb, gw = gates_dev(g)
    s = slice(T - L, T)
    _, S = hla().gdn2_prefill(None, k[:, s], v[:, s], ga[:, s], gb[:, s], gw[:, s], want_o=False)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            args = seq(x, g, b, h)
            _, S_ref = oracle.gdn2_recurrent(None, *(a[T - L:] for a in args[1:]))
            assert_close(host(S)[b, h], S_ref.T, dtype, "replayed state")


def test_gdn2_native_prefill_many_pieces():
    # 21 pieces scanned in order from the GDN-2 piece maps
    dtype, dk, dv, T = "bf16", 128, 128, 20 * C + 3
    note("gdn2 native many pieces")
    x, g = gen((dtype, dk, dv, T), B=1, seed=99)
    q, k, v, _, _ = token_tensors(x)
    o, S = hla().gdn2_prefill(q, k, v, *gates_dev(g))
    torch.cuda.synchronize()
    for h in range(2):
        o_ref, S_ref = oracle.gdn2_recurrent(*seq(x, g, 0, h))
        assert_close(host(o)[0, :, h], o_ref, dtype, f"o h{h}")
        assert_close(host(S)[0, h], S_ref.T, dtype, f"S h{h}")


def test_gdn2_pieces_beyond_one_per_cu():
    # 2 x 4 x 40 = 320 pieces: more than one workgroup per CU can take at once, so the bf16
    # passes loop over pieces and prefetch the next piece's inputs; the last piece is ragged
    dtype, dk, dv, T = "bf16", 128, 128, 40 * C - 5
    B, H, N = 2, 4, 40
    note("gdn2 pieces beyond one per CU")
    x, g = gen((dtype, dk, dv, T), B=B, H=H, seed=97)
    q, k, v, _, _ = token_tensors(x)
    rng = np.random.default_rng(98)
    init = (0.05 * rng.standard_normal((B, H, N, dk, dv))).astype(np.float32)
    h = hla()
    At, Bc = h.gdn2_chunk_transitions(k, v, *gates_dev(g))
    o, _ = h.gdn2_prefill(q, k, v, *gates_dev(g), chunk_init=f32(init), want_state=False)
    torch.cuda.synchronize()
    for b, hh in [(0, 0), (1, 3), (1, 1)]:
        args = seq(x, g, b, hh)
        A_ref, B_ref = oracle.gdn2_chunk_transitions(*args[1:], C)
        assert_close(host(At[b, hh]), A_ref.transpose(0, 2, 1), dtype, f"At b{b} h{hh}")
        assert_close(host(Bc[b, hh]), B_ref.transpose(0, 2, 1), dtype, f"Bc b{b} h{hh}")
        o_ref = oracle.gdn2_routed_outputs(*args, C, init[b, hh].astype(np.float64).transpose(0, 2, 1))
        assert_close(host(o)[b, :, hh], o_ref, dtype, f"o b{b} h{hh}")


def test_gdn2_collapsed_gates_match_gdn():
    # b = w = beta and a = alpha broadcast: both GPU paths compute the same Gated DeltaNet
    dtype, dk, dv, T = "f32", 64, 64, 150
    note("gdn2 collapsed")
    x = inputs.gen_tokens(1, T, 2, dk, dv, dtype=dtype, seed=88, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    ga = alpha[..., None].expand(1, T, 2, dk).contiguous()
    gb = beta[..., None].expand(1, T, 2, dk).contiguous()
    gw = beta[..., None].expand(1, T, 2, dv).contiguous()
    h = hla()
    o2, S2 = h.gdn2_prefill(q, k, v, ga, gb, gw)
    o1, S1 = h.gdn_prefill(q, k, v, beta, alpha)
    torch.cuda.synchronize()
    assert_close(host(o2), host(o1), dtype, "o")
    assert_close(host(S2), host(S1), dtype, "S")


def test_gdn2_full_size_sampled_transitions():
    # B=1, H=16, T=32768, d=128: sampled chunk maps against the oracle
    W = inputs.WORKLOADS["routed_prefill"]
    note("gdn2 full size")
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"],
                          plant_period=W.plant_period, with_q=False)
    g = inputs.gen_gdn2_gates(W.B, W.T, W.H, W.dk, W.dv, seed=0, stream=inputs.STREAM["routed_prefill"])
    k, v = dev(x.k, W.dtype), dev(x.v, W.dtype)
    At, Bc = hla().gdn2_chunk_transitions(k, v, *gates_dev(g))
    torch.cuda.synchronize()
    rng = np.random.default_rng(89)
    N = W.T // C
    for h, c in [(int(rng.integers(W.H)), int(rng.integers(N))) for _ in range(6)] + [(W.H - 1, N - 1)]:
        s = slice(c * C, (c + 1) * C)
        A, Bm = oracle.gdn2_chunk_transition(x.f64("k")[0, s, h], x.f64("v")[0, s, h],
                                             g["a"][0, s, h].astype(np.float64), g["b"][0, s, h].astype(np.float64),
                                             g["w"][0, s, h].astype(np.float64))
        assert_close(host(At[0, h, c]), A.T, W.dtype, f"At h{h} c{c}")
        assert_close(host(Bc[0, h, c]), Bm.T, W.dtype, f"Bc h{h} c{c}")


def _tok(t, x, g, dtype):
    """Token t of every (sequence, head) as decode inputs."""
    q, k, v = (dev(np.ascontiguousarray(getattr(x, n)[:, t]), dtype) for n in ("q", "k", "v"))
    return q, k, v, f32(g["a"][:, t]), f32(g["b"][:, t]), f32(g["w"][:, t])


@pytest.mark.parametrize("case", [CASES[0], CASES[2]], ids=[IDS[0], IDS[2]])
def test_gdn2_decode_native_equals_recurrence(case):
    note(f"gdn2 decode native {case}")
    dtype, dk, dv = case[:3]
    Bs, H, T = 2, 2, 40
    x, g = gen((dtype, dk, dv, T), B=Bs, H=H, seed=90)
    S0 = inputs.gen_state(Bs, H, dk, dv, seed=91)
    S = f32(S0)
    outs = []
    for t in range(T):
        outs.append(host(hla().gdn2_decode(*_tok(t, x, g, dtype), S)))
    torch.cuda.synchronize()
    for b in range(Bs):
        for h in range(H):
            o_ref, S_ref = oracle.gdn2_recurrent(*seq(x, g, b, h), S0=S0[b, h].T.astype(np.float64))
            assert_close(np.stack([o[b, h] for o in outs]), o_ref, dtype, "decode o")
            assert_close(host(S)[b, h], S_ref.T, dtype, "decode state")


def test_gdn2_decode_routed_with_commits_equals_routed_prefill():
    # token-by-token decode, committing every C tokens, with the prefill gate rows as caller
    # gates, reproduces the routed prefill outputs
    dtype, dk, dv = "bf16", 128, 128
    note("gdn2 decode routed commits")
    Bs, H, N = 2, 2, 3
    T = N * C
    x, g = gen((dtype, dk, dv, T), B=Bs, H=H, seed=92)
    G = inputs.gen_gates(Bs, H, N, seed=93, mode="uniform")
    tau = 0.2
    S = torch.zeros((Bs, H, dk, dv), dtype=torch.float32, device="cuda")
    A = torch.eye(dk, dtype=torch.float32, device="cuda").repeat(Bs, H, 1, 1).contiguous()
    Ac = torch.zeros((Bs, H, N, dk, dk), dtype=torch.bfloat16, device="cuda")
    Bcc = torch.zeros((Bs, H, N, dk, dv), dtype=torch.bfloat16, device="cuda")
    nc = torch.zeros((Bs,), dtype=torch.int32, device="cuda")
    outs = []
    for t in range(T):
        i = t // C
        gin = np.zeros((Bs, H, N), np.float32)
        gin[:, :, :i] = G[:, :, i, :i]
        o = hla().gdn2_decode(*_tok(t, x, g, dtype), S, At_cur=A, At_cache=Ac, Bc_cache=Bcc, n_cache=nc,
                              gates_in=f32(gin), tau=tau, commit=(t % C == C - 1))
        outs.append(host(o))
    torch.cuda.synchronize()
    assert host(nc).tolist() == [N] * Bs
    got = np.stack(outs, axis=2)  # [Bs, H, T, dv]
    for b in range(Bs):
        for h in range(H):
            ref = oracle.gdn2_hla_prefill(*seq(x, g, b, h), C, tau, gates_in=G[b, h].astype(np.float64))
            assert_close(got[b, h], ref["o"], dtype, "decode routed o")


def test_gdn2_decode_computed_gates():
    dtype, dk, dv = "bf16", 128, 64
    note("gdn2 decode computed gates")
    Bs, H, n_cap, n_rep = 3, 2, 5, 64
    At_s, Bc_s = inputs.gen_transitions(Bs, H, n_cap, dk, dv, dtype=dtype, seed=94)
    reps_x = inputs.gen_tokens(Bs, n_cap * n_rep, H, dk, dk, dtype=dtype, seed=95)
    reps = reps_x.k.reshape(Bs, n_cap, n_rep, H, dk).transpose(0, 3, 1, 2, 4).copy()
    x, g = gen((dtype, dk, dv, 1), B=Bs, H=H, seed=96)
    S0 = inputs.gen_state(Bs, H, dk, dv, seed=97)
    A0 = (np.eye(dk)[None, None] + 0.05 * inputs.gen_state(Bs, H, dk, dk, seed=98)).astype(np.float32)
    n_cache = np.array([5, 2, 0], np.int32)
    S, A, nc = f32(S0), f32(A0), torch.from_numpy(n_cache).cuda()
    go = torch.empty((Bs, H, n_cap), dtype=torch.float32, device="cuda")
    o = hla().gdn2_decode(*_tok(0, x, g, dtype), S, At_cur=A, At_cache=dev(At_s, dtype), Bc_cache=dev(Bc_s, dtype),
                          reps_cache=dev(reps, dtype), n_cache=nc, tau=0.3, gates_out=go)
    torch.cuda.synchronize()
    Am = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    R = inputs.to_f64(reps, dtype)
    for b in range(Bs):
        for h in range(H):
            ncb = n_cache[b]
            qv, kv, vv, av, bv, wv = (arr[0] for arr in seq(x, g, b, h))
            r = oracle.gdn2_decode_step(qv, kv, vv, av, bv, wv, S0[b, h].astype(np.float64).T,
                                        A0[b, h].astype(np.float64).T, Am[b, h, :ncb], Bm[b, h, :ncb], R[b, h, :ncb], 0.3)
            assert_close(host(o)[b, h], r["o"], dtype, f"o b{b} h{h}")
            np.testing.assert_allclose(host(go)[b, h, :ncb], r["gates"], atol=2e-5)
            assert_close(host(S)[b, h], r["B_cur"].T, dtype, "live state")
            assert_close(host(A)[b, h], r["A_cur"].T, dtype, "live transition")
