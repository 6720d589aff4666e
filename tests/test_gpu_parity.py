"""GPU parity of every C-ABI entry point against the CPU oracle, at sizes the oracle
finishes in seconds (several chunks plus a ragged tail).  Bars: max|diff| / max|ref|
<= 1e-4 for float32 inputs and <= 2e-2 for bfloat16 inputs (float32 accumulation);
masks and active lists bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, dev, f32, host, note, token_tensors

pytestmark = pytest.mark.gpu
C = 64

CASES = [
    # dtype, dk, dv, T, alpha mode
    ("f32", 64, 64, 256, "config"),
    ("f32", 64, 64, 200, "slow"),
    ("f32", 128, 128, 100, "slow"),
    ("bf16", 128, 128, 256, "config"),
    ("bf16", 128, 128, 200, "slow"),
    ("bf16", 64, 128, 130, "slow"),
    ("bf16", 128, 64, 70, "slow"),
    ("bf16", 64, 64, 150, "config"),
]
IDS = [f"{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}-{c[4]}" for c in CASES]


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def gen(case, B=2, H=2, seed=0, T=None):
    dtype, dk, dv, T0, mode = case
    return inputs.gen_tokens(B, T or T0, H, dk, dv, dtype=dtype, seed=seed, alpha_mode=mode)


def seq(x, b, h):
    """Per-(b, h) float64 arrays of the oracle."""
    q = None if x.q is None else x.f64("q")[b, :, h]
    return q, x.f64("k")[b, :, h], x.f64("v")[b, :, h], x.f64("beta")[b, :, h], x.f64("alpha")[b, :, h]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_chunk_transitions(case):
    note(f"chunk_transitions {case}")
    x = gen(case)
    q, k, v, beta, alpha = token_tensors(x)
    At, Bc = hla().chunk_transitions(k, v, beta, alpha)
    torch.cuda.synchronize()
    At, Bc = host(At), host(Bc)
    for b in range(2):
        for h in range(2):
            _, kk, vv, bb, aa = seq(x, b, h)
            A, B = oracle.chunk_transitions(kk, vv, bb, aa, C)
            assert_close(At[b, h], A.transpose(0, 2, 1), case[0], f"At b{b} h{h}")
            assert_close(Bc[b, h], B.transpose(0, 2, 1), case[0], f"Bc b{b} h{h}")


@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_native_prefill(case, with_s0):
    note(f"native prefill {case} S0={with_s0}")
    dtype, dk, dv = case[:3]
    x = gen(case, seed=1)
    q, k, v, beta, alpha = token_tensors(x)
    S0 = inputs.gen_state(2, 2, dk, dv, seed=3) if with_s0 else None
    o, S = hla().gdn_prefill(q, k, v, beta, alpha, S0=None if S0 is None else f32(S0))
    torch.cuda.synchronize()
    tr = lambda a: a.transpose(0, 2, 1, 3)  # [B,T,H,d] -> [B,H,T,d]
    o_ref, S_ref = oracle.gdn_recurrent(tr(x.f64("q")), tr(x.f64("k")), tr(x.f64("v")),
                                        x.f64("beta").transpose(0, 2, 1), x.f64("alpha").transpose(0, 2, 1),
                                        S0=None if S0 is None else S0.astype(np.float64).transpose(0, 1, 3, 2))
    assert_close(host(o), o_ref.transpose(0, 2, 1, 3), dtype, "o")
    assert_close(host(S), S_ref.transpose(0, 1, 3, 2), dtype, "S_final")


@pytest.mark.parametrize("case", [CASES[1], CASES[4]], ids=[IDS[1], IDS[4]])
def test_prefill_resumes_from_final_state(case):
    # prefill(x[:T1]) then prefill(x[T1:], S0 = S_final) equals the plain recurrence over x
    note(f"resume {case}")
    dtype, dk, dv, T = case[:4]
    x = gen(case, seed=2)
    q, k, v, beta, alpha = token_tensors(x)
    T1 = 64 + 37
    h = hla()
    o1, S1 = h.gdn_prefill(q[:, :T1], k[:, :T1], v[:, :T1], beta[:, :T1], alpha[:, :T1])
    o2, S2 = h.gdn_prefill(q[:, T1:], k[:, T1:], v[:, T1:], beta[:, T1:], alpha[:, T1:], S0=S1)
    torch.cuda.synchronize()
    for b in range(2):
        for hh in range(2):
            o_ref, S_ref = oracle.gdn_recurrent(*seq(x, b, hh))
            assert_close(np.concatenate([host(o1)[b, :, hh], host(o2)[b, :, hh]]), o_ref, dtype, "o")
            assert_close(host(S2)[b, hh], S_ref.T, dtype, "S_final")


@pytest.mark.parametrize("case", [CASES[1], CASES[4]], ids=[IDS[1], IDS[4]])
def test_tail_replay_state_only(case):
    # state-only prefill of a suffix window from a zero state ([TR] Tail-Replay)
    note(f"tail replay {case}")
    dtype, dk, dv, T = case[:4]
    x = gen(case, seed=4, T=300)
    _, k, v, beta, alpha = token_tensors(x)
    L = 77
    o, S = hla().gdn_prefill(None, k[:, -L:], v[:, -L:], beta[:, -L:], alpha[:, -L:], want_o=False)
    torch.cuda.synchronize()
    assert o is None
    for b in range(2):
        for hh in range(2):
            _, kk, vv, bb, aa = seq(x, b, hh)
            S_rep, _ = oracle.tail_replay(kk, vv, bb, aa, L)
            assert_close(host(S)[b, hh], S_rep.T, dtype, "S_replay")


def _check_lists(mask, aidx, acnt):
    N = mask.shape[-1]
    for i in range(N):
        act = np.nonzero(mask[i])[0]
        assert acnt[i] == len(act)
        np.testing.assert_array_equal(aidx[i, :len(act)], act)
        assert np.all(aidx[i, len(act):] == -1)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_route_mix_computed_gates_and_routed_prefill(case):
    note(f"route computed {case}")
    dtype, dk, dv, T = case[:4]
    x = gen(case, seed=5)
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    r = h.hla_prefill(q, k, v, beta, alpha, tau=1e-3)
    torch.cuda.synchronize()
    N = math.ceil(T / C)
    for b in range(2):
        for hh in range(2):
            ref = oracle.hla_prefill(*seq(x, b, hh), C, 1e-3)
            g = host(r["gates"])[b, hh]
            np.testing.assert_allclose(g, ref["gates"], atol=2e-5, rtol=0)
            near = np.abs(ref["gates"] - 1e-3) <= 1e-6
            m = host(r["mask"])[b, hh].astype(bool)
            assert np.array_equal(m[~near], ref["mask"][~near])
            _check_lists(m, host(r["active_idx"])[b, hh].astype(int), host(r["active_cnt"])[b, hh].astype(int))
            np.testing.assert_allclose(host(r["n_eff"])[b, hh], ref["n_eff"], rtol=1e-4, atol=1e-5)
            assert_close(host(r["S_routed"])[b, hh], ref["S_routed"].transpose(0, 2, 1), dtype, "S_routed")
            assert_close(host(r["o"])[b, :, hh], ref["o"], dtype, "routed o")
            assert ref["count"].sum() == N * (N - 1) // 2


@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("tau", [0.1, 1e-3])
@pytest.mark.parametrize("case", [CASES[1], CASES[4], CASES[5]], ids=[IDS[1], IDS[4], IDS[5]])
def test_route_mix_caller_gates_isolated(case, tau, with_s0):
    # caller gates (skip-heavy) and generated transitions: the composition alone, with the
    # same rounded A/B on both sides; masks and lists must be bit-exact
    note(f"route caller gates {case} tau={tau} S0={with_s0}")
    dtype, dk, dv = case[:3]
    B, H, N = 2, 2, 7
    T = N * C - 20
    At_s, Bc_s = inputs.gen_transitions(B, H, N, dk, dv, dtype=dtype, seed=6)
    G = inputs.gen_gates(B, H, N, seed=7, mode="skip_heavy")
    S0 = inputs.gen_state(B, H, dk, dv, seed=8) if with_s0 else None
    r = hla().route_mix(None, None, dev(At_s, dtype), dev(Bc_s, dtype), tau=tau, gates_in=f32(G), T=T,
                        S0=None if S0 is None else f32(S0))
    torch.cuda.synchronize()
    A = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)   # math orientation
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    for b in range(B):
        for hh in range(H):
            ref = oracle.router_gates(np.zeros((T, dk)), np.zeros((T, dk)), C, C, tau, gates_in=G[b, hh].astype(np.float64))
            m = host(r["mask"])[b, hh].astype(bool)
            np.testing.assert_array_equal(m, ref["mask"])
            np.testing.assert_array_equal(host(r["gates"])[b, hh], ref["gates"].astype(np.float32))
            _check_lists(m, host(r["active_idx"])[b, hh].astype(int), host(r["active_cnt"])[b, hh].astype(int))
            np.testing.assert_allclose(host(r["n_eff"])[b, hh], ref["n_eff"], rtol=1e-5, atol=1e-6)
            s0 = None if S0 is None else S0[b, hh].astype(np.float64).T
            Sr = oracle.routed_states(A[b, hh], Bm[b, hh], ref["ghat"], ref["mask"], S0=s0)
            assert_close(host(r["S_routed"])[b, hh], Sr.transpose(0, 2, 1), dtype, "S_routed")


@pytest.mark.parametrize("case", [CASES[0], CASES[4]], ids=[IDS[0], IDS[4]])
def test_decode_native_equals_recurrence(case):
    note(f"decode native {case}")
    dtype, dk, dv = case[:3]
    Bs, H, T = 3, 2, 40
    x = inputs.gen_tokens(Bs, T, H, dk, dv, dtype=dtype, seed=9, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    S = torch.zeros((Bs, H, dk, dv), dtype=torch.float32, device="cuda")
    h = hla()
    outs = []
    for t in range(T):
        o = h.gdn_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), beta[:, t].contiguous(),
                         alpha[:, t].contiguous(), S)
        outs.append(host(o))
    torch.cuda.synchronize()
    tr = lambda a: a.transpose(0, 2, 1, 3)
    o_ref, S_ref = oracle.gdn_recurrent(tr(x.f64("q")), tr(x.f64("k")), tr(x.f64("v")),
                                        x.f64("beta").transpose(0, 2, 1), x.f64("alpha").transpose(0, 2, 1))
    assert_close(np.stack(outs, axis=2), o_ref, dtype, "decode o")
    assert_close(host(S), S_ref.transpose(0, 1, 3, 2), dtype, "decode state")


@pytest.mark.parametrize("case", [CASES[1], CASES[4], CASES[6]], ids=[IDS[1], IDS[4], IDS[6]])
def test_decode_routed_with_commits_equals_routed_prefill(case):
    # token-by-token decode, committing every C tokens, with the prefill gate row of the
    # current chunk as caller gates, reproduces the routed prefill outputs
    note(f"decode routed commit {case}")
    dtype, dk, dv = case[:3]
    Bs, H, N = 2, 2, 3
    T = N * C
    x = inputs.gen_tokens(Bs, T, H, dk, dv, dtype=dtype, seed=10, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    G = inputs.gen_gates(Bs, H, N, seed=11, mode="uniform")
    tau = 0.2
    n_cap = N
    S = torch.zeros((Bs, H, dk, dv), dtype=torch.float32, device="cuda")
    A = torch.eye(dk, dtype=torch.float32, device="cuda").repeat(Bs, H, 1, 1).contiguous()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Ac = torch.zeros((Bs, H, n_cap, dk, dk), dtype=tdt, device="cuda")
    Bcc = torch.zeros((Bs, H, n_cap, dk, dv), dtype=tdt, device="cuda")
    nc = torch.zeros((Bs,), dtype=torch.int32, device="cuda")
    h = hla()
    outs = []
    for t in range(T):
        i = t // C
        gin = np.zeros((Bs, H, n_cap), np.float32)
        gin[:, :, :i] = G[:, :, i, :i]
        o = h.gdn_decode(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), beta[:, t].contiguous(),
                         alpha[:, t].contiguous(), S, At_cur=A, At_cache=Ac, Bc_cache=Bcc, n_cache=nc,
                         gates_in=f32(gin), tau=tau, commit=(t % C == C - 1))
        outs.append(host(o))
    torch.cuda.synchronize()
    assert host(nc).tolist() == [N] * Bs
    got = np.stack(outs, axis=2)  # [Bs, H, T, dv]
    for b in range(Bs):
        for hh in range(H):
            ref = oracle.hla_prefill(*seq(x, b, hh), C, tau, gates_in=G[b, hh].astype(np.float64))
            assert_close(got[b, hh], ref["o"], dtype, "decode routed o")


@pytest.mark.parametrize("case", [CASES[0], CASES[4]], ids=[IDS[0], IDS[4]])
def test_decode_computed_gates(case):
    # one step against a generated cache; gates from the token's q and the cached reps
    note(f"decode computed gates {case}")
    dtype, dk, dv = case[:3]
    Bs, H, n_cap, n_rep = 3, 2, 6, 64
    At_s, Bc_s = inputs.gen_transitions(Bs, H, n_cap, dk, dv, dtype=dtype, seed=12)
    reps_x = inputs.gen_tokens(Bs, n_cap * n_rep, H, dk, dk, dtype=dtype, seed=13)
    reps = reps_x.k.reshape(Bs, n_cap, n_rep, H, dk).transpose(0, 3, 1, 2, 4).copy()  # [Bs,H,n_cap,n_rep,dk]
    tok = inputs.gen_decode_tokens(Bs, H, dk, dv, step=0, dtype=dtype, seed=14)
    S0 = inputs.gen_state(Bs, H, dk, dv, seed=15)
    A0 = (np.eye(dk)[None, None] + 0.05 * inputs.gen_state(Bs, H, dk, dk, seed=16)).astype(np.float32)
    n_cache = np.array([6, 3, 0], np.int32)
    S, A, nc = f32(S0), f32(A0), torch.from_numpy(n_cache).cuda()
    go = torch.empty((Bs, H, n_cap), dtype=torch.float32, device="cuda")
    o = hla().gdn_decode(dev(tok["q"], dtype), dev(tok["k"], dtype), dev(tok["v"], dtype), f32(tok["beta"]),
                         f32(tok["alpha"]), S, At_cur=A, At_cache=dev(At_s, dtype), Bc_cache=dev(Bc_s, dtype),
                         reps_cache=dev(reps, dtype), n_cache=nc, tau=0.3, gates_out=go)
    torch.cuda.synchronize()
    Am = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    R = inputs.to_f64(reps, dtype)
    for b in range(Bs):
        for hh in range(H):
            ncb = n_cache[b]
            r = oracle.decode_step(inputs.to_f64(tok["q"], dtype)[b, hh], inputs.to_f64(tok["k"], dtype)[b, hh],
                                   inputs.to_f64(tok["v"], dtype)[b, hh], float(tok["beta"][b, hh]),
                                   float(tok["alpha"][b, hh]), S0[b, hh].astype(np.float64).T,
                                   A0[b, hh].astype(np.float64).T, Am[b, hh, :ncb], Bm[b, hh, :ncb], R[b, hh, :ncb], 0.3)
            assert_close(host(o)[b, hh], r["o"], dtype, f"o b{b} h{hh}")
            np.testing.assert_allclose(host(go)[b, hh, :ncb], r["gates"], atol=2e-5)
            assert np.all(host(go)[b, hh, ncb:] == 0)
            assert_close(host(S)[b, hh], r["B_cur"].T, dtype, "live state")
            assert_close(host(A)[b, hh], r["A_cur"].T, dtype, "live transition")
