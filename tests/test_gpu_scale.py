"""GPU parity beyond one tile of work, through the C ABI.

* Routed prefill over tens of chunks (several query groups of the composition kernel,
  chains of up to 39 history chunks, ragged last chunk), with computed and with skip-heavy
  caller gates.
* The four benchmark workloads at their full sizes and in the launch configuration the
  benchmark times, checked on sampled outputs that the oracle computes one by one.

Bars as everywhere: max|diff| / max|ref| <= 1e-4 (float32 inputs), <= 2e-2 (bfloat16
inputs, float32 accumulation); masks and active lists bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close as _assert_close, dev, f32, host, note, token_tensors

pytestmark = pytest.mark.gpu
C = 64


def assert_close(got, ref, dtype, what, tol=None):
    """The parity bar, with the measured error printed (run with -s to see it)."""
    e = _assert_close(got, ref, dtype, what, tol=tol)
    note(f"    {what}: max|diff|/max|ref| = {e:.2e}")
    return e


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def seq(x, b, h, t0=0, t1=None):
    """Per-(b, h) float64 oracle arrays of tokens [t0, t1)."""
    sl = slice(t0, t1)
    q = None if x.q is None else x.f64("q")[b, sl, h]
    return q, x.f64("k")[b, sl, h], x.f64("v")[b, sl, h], x.f64("beta")[b, sl, h], x.f64("alpha")[b, sl, h]


def check_row(i, g_gpu, m_gpu, idx_gpu, cnt_gpu, ref, tau):
    """Gates, mask and active list of query chunk i against the oracle's row i."""
    np.testing.assert_allclose(g_gpu[:i], ref["gates"][i, :i], atol=2e-5, rtol=0)
    near = np.abs(ref["gates"][i, :i] - tau) <= 1e-6
    m = m_gpu[:i].astype(bool)
    assert np.array_equal(m[~near], ref["mask"][i, :i][~near])
    act = np.nonzero(m)[0]
    assert cnt_gpu == len(act)
    np.testing.assert_array_equal(idx_gpu[:len(act)], act)
    assert np.all(idx_gpu[len(act):] == -1)


# ----------------------------------------------------------------------------- many chunks
MANY = [
    # dtype, dk, dv, T (ragged), alpha mode, with S0
    ("bf16", 128, 128, 40 * C - 23, "slow", False),
    ("bf16", 128, 128, 21 * C - 5, "slow", True),
    ("bf16", 64, 128, 21 * C - 40, "slow", False),
    ("bf16", 128, 64, 21 * C - 1, "slow", True),
    ("f32", 64, 64, 21 * C - 17, "slow", False),
]
MANY_IDS = [f"{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}-S0{int(c[5])}" for c in MANY]


@pytest.mark.parametrize("case", MANY, ids=MANY_IDS)
def test_routed_prefill_many_chunks(case):
    dtype, dk, dv, T, mode, with_s0 = case
    note(f"routed many chunks {case}")
    B, H = 1, 2
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=21, alpha_mode=mode)
    q, k, v, beta, alpha = token_tensors(x)
    S0 = inputs.gen_state(B, H, dk, dv, seed=22) if with_s0 else None
    r = hla().hla_prefill(q, k, v, beta, alpha, tau=1e-3, S0=None if S0 is None else f32(S0))
    torch.cuda.synchronize()
    N = math.ceil(T / C)
    for hh in range(H):
        s0 = None if S0 is None else S0[0, hh].astype(np.float64).T
        ref = oracle.hla_prefill(*seq(x, 0, hh), C, 1e-3, S0=s0)
        m, idx, cnt = host(r["mask"])[0, hh], host(r["active_idx"])[0, hh].astype(int), host(r["active_cnt"])[0, hh]
        for i in range(N):
            check_row(i, host(r["gates"])[0, hh, i], m[i], idx[i], int(cnt[i]), ref, 1e-3)
        assert_close(host(r["S_routed"])[0, hh], ref["S_routed"].transpose(0, 2, 1), dtype, "S_routed")
        assert_close(host(r["o"])[0, :, hh], ref["o"], dtype, "routed o")


@pytest.mark.parametrize("case", [MANY[0], MANY[2], MANY[3]], ids=[MANY_IDS[0], MANY_IDS[2], MANY_IDS[3]])
def test_route_mix_many_chunks_caller_gates(case):
    # skip-heavy caller gates: many query groups meet runs of skipped history chunks
    dtype, dk, dv, T = case[:4]
    note(f"route caller gates many chunks {case}")
    B, H = 1, 2
    N = math.ceil(T / C)
    At_s, Bc_s = inputs.gen_transitions(B, H, N, dk, dv, dtype=dtype, seed=23)
    G = inputs.gen_gates(B, H, N, seed=24, mode="skip_heavy")
    tau = 0.1
    r = hla().route_mix(None, None, dev(At_s, dtype), dev(Bc_s, dtype), tau=tau, gates_in=f32(G), T=T)
    torch.cuda.synchronize()
    A = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    for hh in range(H):
        ref = oracle.router_gates(np.zeros((T, dk)), np.zeros((T, dk)), C, C, tau, gates_in=G[0, hh].astype(np.float64))
        np.testing.assert_array_equal(host(r["mask"])[0, hh].astype(bool), ref["mask"])
        skipped = np.tril(np.ones((N, N), bool), -1) & ~ref["mask"]
        assert skipped.sum() > N  # the case really exercises skipping
        Sr = oracle.routed_states(A[0, hh], Bm[0, hh], ref["ghat"], ref["mask"])
        assert_close(host(r["S_routed"])[0, hh], Sr.transpose(0, 2, 1), dtype, "S_routed")


# ----------------------------------------------------------------------------- full sizes
def _check_router_all_rows(r, b, hh, ref, tau, N):
    """Every row of one head's router outputs against the oracle: history gates (atol
    2e-5), the diagonal 1 and the upper triangle 0, the mask (bit-exact away from tau),
    active lists and counts (bit-exact, from the GPU's own mask) and n_eff."""
    g = host(r["gates"][b, hh])
    m = host(r["mask"][b, hh]).astype(bool)
    idx = host(r["active_idx"][b, hh]).astype(np.int64)
    cnt = host(r["active_cnt"][b, hh]).astype(np.int64)
    low = np.tril(np.ones((N, N), bool), -1)
    np.testing.assert_allclose(g[low], ref["gates"][low], atol=2e-5, rtol=0)
    assert np.all(np.diag(g) == 1.0) and np.all(g[np.triu(np.ones((N, N), bool), 1)] == 0.0)
    near = low & (np.abs(ref["gates"] - tau) <= 1e-6)
    assert np.array_equal(m[low & ~near], ref["mask"][low & ~near])
    assert not m[~low].any()
    np.testing.assert_array_equal(cnt, m.sum(axis=1))
    for i in range(N):
        act = np.nonzero(m[i])[0]
        np.testing.assert_array_equal(idx[i, :len(act)], act)
        assert np.all(idx[i, len(act):] == -1)
    np.testing.assert_allclose(host(r["n_eff"][b, hh]), ref["n_eff"], rtol=1e-4, atol=1e-5)
    return int(near.sum())


def _router_refs(x, pairs, tau):
    """The oracle's full gate matrices of several (b, h) sequences, in threads."""
    from concurrent.futures import ThreadPoolExecutor

    def one(p):
        b, hh = p
        return oracle.router_gates(x.f64("q")[b, :, hh], x.f64("k")[b, :, hh], C, C, tau)
    with ThreadPoolExecutor(8) as ex:
        return dict(zip(pairs, ex.map(one, pairs)))


def _routed_rows(x, r, o, b, hh, rows, ref, dtype):
    """Routed states and outputs of query chunks ``rows`` of (b, hh) against the oracle:
    transitions token by token, the composition of each row alone, the chunk's outputs
    from its routed state."""
    qh, kh, vh, bh, ah = seq(x, b, hh)
    A, Bm = oracle.chunk_transitions(kh, vh, bh, ah, C)
    T = qh.shape[0]
    for i in rows:
        note(f"  head {hh} query chunk {i}")
        only_i = np.zeros_like(ref["mask"])
        only_i[i] = ref["mask"][i]
        S_i = oracle.routed_states(A[:i + 1], Bm[:i + 1], ref["ghat"][:i + 1, :i + 1], only_i[:i + 1, :i + 1])[i]
        assert_close(host(r["S_routed"][b, hh, i]), S_i.T, dtype, f"S_routed h{hh} i{i}")
        s, e = i * C, min((i + 1) * C, T)
        o_i, _ = oracle.gdn_recurrent(qh[s:e], kh[s:e], vh[s:e], bh[s:e], ah[s:e], S0=S_i)
        assert_close(host(o[b, s:e, hh]), o_i, dtype, f"o h{hh} chunk {i}")


def _routed_calls(x, W, N):
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    At = torch.empty((W.B, W.H, N, W.dk, W.dk), dtype=k.dtype, device="cuda")
    Bc = torch.empty((W.B, W.H, N, W.dk, W.dv), dtype=k.dtype, device="cuda")
    h.chunk_transitions(k, v, beta, alpha, At=At, Bc=Bc)
    r = h.route_mix(q, k, At, Bc, n_rep=C, tau=W.tau)
    o, _ = h.gdn_prefill(q, k, v, beta, alpha, chunk_init=r["S_routed"], want_state=False)
    torch.cuda.synchronize()
    return r, o


def test_routed_prefill_full_size_sampled():
    """B=1, H=16, T=32768, d=128, 512 chunks, bf16, tau=1e-3, planted x8 signal: the three
    calls the benchmark times.  Every head's 512 x 512 gates, mask, active lists, counts
    and n_eff against the oracle's; the routed states and outputs of query chunks
    {1, 300, 511} of heads {0, 15}."""
    W = inputs.WORKLOADS["routed_prefill"]
    note("routed prefill full size")
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["routed_prefill"],
                          plant_period=W.plant_period)
    N = W.N
    r, o = _routed_calls(x, W, N)
    refs = _router_refs(x, [(0, hh) for hh in range(W.H)], W.tau)
    for hh in range(W.H):
        note(f"  router rows, head {hh}")
        assert refs[(0, hh)]["mask"][np.tril_indices(N, -1)].all()  # dense at these distributions
        assert _check_router_all_rows(r, 0, hh, refs[(0, hh)], W.tau, N) == 0
    for hh in (0, W.H - 1):
        _routed_rows(x, r, o, 0, hh, [1, 300, N - 1], refs[(0, hh)], W.dtype)


def test_routed_prefill_full_length_slow_decay():
    """B=1, H=8, T=32768 (512 chunks), bf16, slow decay (median alpha ~ 0.95, so the chunk
    maps are far from zero and every step of a 511-step chain matters), computed gates:
    B H is a multiple of 8, so the composition takes its XCD-ordered dispatch.  All router
    rows of heads {0, 7}; routed states and outputs of query chunks {1, 257, 511}."""
    W = inputs.Workload("routed_slow", B=1, T=32768, H=8, dk=128, dv=128, C=C, dtype="bf16", tau=1e-3)
    note("routed prefill full length, slow decay")
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=5, stream=inputs.STREAM["routed_prefill"],
                          alpha_mode="slow")
    N = W.N
    r, o = _routed_calls(x, W, N)
    pairs = [(0, 0), (0, W.H - 1)]
    refs = _router_refs(x, pairs, W.tau)
    for b, hh in pairs:
        _check_router_all_rows(r, b, hh, refs[(b, hh)], W.tau, N)
        _routed_rows(x, r, o, b, hh, [1, 257, N - 1], refs[(b, hh)], W.dtype)


@pytest.mark.parametrize("T,with_s0", [(16 * C + 37, True), (40 * C - 5, False)])
def test_native_prefill_many_pieces(T, with_s0):
    """17 and 40 pieces of 64 tokens (ragged last piece), outputs and final state, and the
    state-only call.  Slow decay, so each piece's start state carries its history."""
    dtype, dk, dv, B, H = "bf16", 128, 64, 1, 2
    note(f"native prefill T={T} S0={with_s0}")
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=101, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    S0 = inputs.gen_state(B, H, dk, dv, seed=102) if with_s0 else None
    h = hla()
    o, S = h.gdn_prefill(q, k, v, beta, alpha, S0=None if S0 is None else f32(S0))
    _, S_only = h.gdn_prefill(None, k, v, beta, alpha, S0=None if S0 is None else f32(S0), want_o=False)
    torch.cuda.synchronize()
    for hh in range(H):
        o_ref, S_ref = oracle.gdn_recurrent(*seq(x, 0, hh), S0=None if S0 is None else S0[0, hh].T.astype(np.float64))
        assert_close(host(o[0, :, hh]), o_ref, dtype, f"o h{hh}")
        assert_close(host(S[0, hh]), S_ref.T, dtype, f"S_final h{hh}")
        assert_close(host(S_only[0, hh]), S_ref.T, dtype, f"state-only S_final h{hh}")


def test_native_prefill_full_size_sampled():
    """B=4, H=16, T=4096, d=128, bf16: the benchmark's call, then outputs and final state
    of (b, h) in {(0, 0), (2, 9), (3, 15)} against the sequential recurrence."""
    W = inputs.WORKLOADS["native_prefill"]
    note("native prefill full size")
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["native_prefill"])
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    d = h.make_dims(W.B, W.T, W.H, W.T, W.dk, W.dv, h.HLA_BF16)
    ws = torch.empty(h.workspace_bytes(h.FN_GDN_PREFILL, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((W.B, W.T, W.H, W.dv), dtype=torch.float32, device="cuda")
    S = torch.empty((W.B, W.H, W.dk, W.dv), dtype=torch.float32, device="cuda")
    h.gdn_prefill(q, k, v, beta, alpha, o=o, S_final=S, ws=ws)
    torch.cuda.synchronize()
    for b, hh in ((0, 0), (2, 9), (3, 15)):
        o_ref, S_ref = oracle.gdn_recurrent(*seq(x, b, hh))
        assert_close(host(o[b, :, hh]), o_ref, W.dtype, f"o b{b} h{hh}")
        assert_close(host(S[b, hh]), S_ref.T, W.dtype, f"S_final b{b} h{hh}")


def test_tail_replay_full_size_sampled():
    """B=8, H=16, prefix 32768: the benchmark's suffix-view call (last 3277 tokens, rows
    strided by the full prefix length) against the replay of the same suffix for
    (b, h) in {(0, 0), (5, 7), (7, 15)}."""
    W = inputs.WORKLOADS["tail_replay"]
    L = W.replay
    note("tail replay full size")
    x = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["tail_replay"],
                          with_q=False, t_range=(W.T - L, W.T))
    tdt = torch.bfloat16
    k = torch.zeros((W.B, W.T, W.H, W.dk), dtype=tdt, device="cuda")
    v = torch.zeros((W.B, W.T, W.H, W.dv), dtype=tdt, device="cuda")
    beta = torch.zeros((W.B, W.T, W.H), dtype=torch.float32, device="cuda")
    alpha = torch.ones((W.B, W.T, W.H), dtype=torch.float32, device="cuda")
    k[:, -L:] = dev(x.k, W.dtype)
    v[:, -L:] = dev(x.v, W.dtype)
    beta[:, -L:] = f32(x.beta)
    alpha[:, -L:] = f32(x.alpha)
    h = hla()
    S = torch.empty((W.B, W.H, W.dk, W.dv), dtype=torch.float32, device="cuda")
    d = h.make_dims(W.B, L, W.H, W.T, W.dk, W.dv, h.HLA_BF16)
    ws = torch.empty(h.workspace_bytes(h.FN_GDN_PREFILL, d), dtype=torch.uint8, device="cuda")
    h.gdn_prefill(None, k[:, -L:], v[:, -L:], beta[:, -L:], alpha[:, -L:], want_o=False, S_final=S, ws=ws)
    torch.cuda.synchronize()
    picks = ((0, 0), (5, 7), (7, 15))
    for b, hh in picks:
        _, kk, vv, bb, aa = seq(x, b, hh)
        _, S_ref = oracle.gdn_recurrent(None, kk, vv, bb, aa)
        assert_close(host(S[b, hh]), S_ref.T, W.dtype, f"S_replay b{b} h{hh}")
    # [TR]: the rebuilt state against the full 32768-token prefix state.  They differ by at
    # most (prod of the suffix alphas) ||S_{T-L}||_2 (about 1e-3000 here), so the bf16 bar
    # plus that bound holds
    note("tail replay vs full prefix")
    xp = inputs.gen_tokens(W.B, W.T, W.H, W.dk, W.dv, dtype=W.dtype, seed=0, stream=inputs.STREAM["tail_replay"],
                           with_q=False, t_range=(0, W.T - L))
    kk, vv, bb, aa = (np.stack([xp.f64(n)[b, :, hh] for b, hh in picks]) for n in ("k", "v", "beta", "alpha"))
    _, S_pre = oracle.gdn_recurrent(None, kk, vv, bb, aa)
    for i, (b, hh) in enumerate(picks):
        _, ks_, vs_, bs_, as_ = seq(x, b, hh)
        _, S_full = oracle.gdn_recurrent(None, ks_, vs_, bs_, as_, S0=S_pre[i])
        lb = oracle.tail_replay_bound_log10(as_, S_pre[i])
        assert lb < -100
        bound_rel = 10.0 ** lb / np.max(np.abs(S_full))
        e = assert_close(host(S[b, hh]), S_full.T, W.dtype, f"S_replay vs full prefix b{b} h{hh}",
                         tol=2e-2 + bound_rel)
        note(f"    bound log10 {lb:.0f}, rel err vs full prefix {e:.2e}")


def test_decode_full_size_sampled():
    """Bs=256, H=16, d=128, 64 cached chunks, bf16 caches, tau=1e-3: three decode steps
    in the benchmark's launch configuration.  The cache holds 8 seeded sequences' chunk
    transitions and representatives repeated 32 times over the batch; sequences
    {0, 131, 255} and heads {0, 15} are checked after every step against the oracle's
    decode step on the same rounded cache."""
    W = inputs.WORKLOADS["decode"]
    Bs, H, dk, dv, n_cap = W.B, W.H, W.dk, W.dv, W.n_cache
    note("decode full size")
    distinct = 8
    At_s, Bc_s = inputs.gen_transitions(distinct, H, n_cap, dk, dv, dtype=W.dtype, seed=31)
    reps_x = inputs.gen_tokens(distinct, n_cap * C, H, dk, dk, dtype=W.dtype, seed=32, with_q=False)
    reps_s = reps_x.k.reshape(distinct, n_cap, C, H, dk).transpose(0, 3, 1, 2, 4).copy()
    rep = Bs // distinct
    At_cache = dev(At_s, W.dtype).repeat(rep, 1, 1, 1, 1).contiguous()
    Bc_cache = dev(Bc_s, W.dtype).repeat(rep, 1, 1, 1, 1).contiguous()
    reps = dev(reps_s, W.dtype).repeat(rep, 1, 1, 1, 1).contiguous()
    n_cache = torch.full((Bs,), n_cap, dtype=torch.int32, device="cuda")
    S = torch.zeros((Bs, H, dk, dv), dtype=torch.float32, device="cuda")
    A = torch.eye(dk, dtype=torch.float32, device="cuda").repeat(Bs, H, 1, 1).contiguous()
    o = torch.empty((Bs, H, dv), dtype=torch.float32, device="cuda")
    Am = inputs.to_f64(At_s, W.dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, W.dtype).transpose(0, 1, 2, 4, 3)
    R = inputs.to_f64(reps_s, W.dtype)
    picks = [(b, hh) for b in (0, 131, 255) for hh in (0, H - 1)]
    live = {p: (np.zeros((dv, dk)), np.eye(dk)) for p in picks}
    h = hla()
    for step in range(3):
        tok = inputs.gen_decode_tokens(Bs, H, dk, dv, step=step, dtype=W.dtype, seed=0, stream=inputs.STREAM["decode"])
        h.gdn_decode(dev(tok["q"], W.dtype), dev(tok["k"], W.dtype), dev(tok["v"], W.dtype), f32(tok["beta"]),
                     f32(tok["alpha"]), S, At_cur=A, At_cache=At_cache, Bc_cache=Bc_cache, reps_cache=reps,
                     n_cache=n_cache, tau=W.tau, o=o)
        torch.cuda.synchronize()
        for b, hh in picks:
            src = b % distinct
            B_cur, A_cur = live[(b, hh)]
            ref = oracle.decode_step(inputs.to_f64(tok["q"], W.dtype)[b, hh], inputs.to_f64(tok["k"], W.dtype)[b, hh],
                                     inputs.to_f64(tok["v"], W.dtype)[b, hh], float(tok["beta"][b, hh]),
                                     float(tok["alpha"][b, hh]), B_cur, A_cur, Am[src, hh], Bm[src, hh], R[src, hh],
                                     W.tau)
            live[(b, hh)] = (ref["B_cur"], ref["A_cur"])
            assert_close(host(o[b, hh]), ref["o"], W.dtype, f"o step {step} b{b} h{hh}")
    for b, hh in picks:
        assert_close(host(S[b, hh]), live[(b, hh)][0].T, W.dtype, f"live state b{b} h{hh}")
        assert_close(host(A[b, hh]), live[(b, hh)][1].T, W.dtype, f"live transition b{b} h{hh}")
