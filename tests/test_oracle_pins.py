"""Pins for the CPU oracle: closed forms, invariants, library routines and brute force.

Each pin is chosen so that a plausible mistake in the oracle (a dropped beta or alpha, a
wrong sign in the erase, an off-by-one token, a transposed outer product, a wrong
composition order, g applied to only half of the map) fails at least one of them.
Shapes use dk != dv so that transposed operands fail loudly.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_seq(rng, T, dk, dv, slow=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal(T) + (-3.0 if slow else 2.0)))
    return q, k, v, beta, alpha


# ----------------------------------------------------------------------------- P6 closed forms
def test_single_token_closed_form():
    # T = 1 from a zero state: S = beta v k^T, so o = beta (k . q) v.
    rng = np.random.default_rng(1)
    q, k, v, beta, alpha = _rand_seq(rng, 1, 5, 3)
    o, S = oracle.gdn_recurrent(q, k, v, beta, alpha)
    np.testing.assert_allclose(o[0], beta[0] * (k[0] @ q[0]) * v[0], rtol=1e-14)
    np.testing.assert_allclose(S, beta[0] * np.outer(v[0], k[0]), rtol=1e-14)


def test_orthonormal_keys_store_exactly():
    # alpha = beta = 1 with orthonormal keys: S_T = sum_t v_t k_t^T and S_T k_s = v_s.
    rng = np.random.default_rng(2)
    dk, dv, T = 6, 4, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:T]
    v = rng.standard_normal((T, dv))
    _, S = oracle.gdn_recurrent(None, k, v, np.ones(T), np.ones(T))
    np.testing.assert_allclose(S, v.T @ k, atol=1e-13)
    for s in range(T):
        np.testing.assert_allclose(S @ k[s], v[s], atol=1e-13)


def test_delta_rule_overwrites_same_key():
    # alpha = beta = 1, the same key written twice: the second value replaces the first
    # (the erase term has a minus sign).
    k = np.array([[0.6, 0.8, 0.0], [0.6, 0.8, 0.0]])
    v = np.array([[1.0, 2.0], [-3.0, 5.0]])
    _, S = oracle.gdn_recurrent(None, k, v, np.ones(2), np.ones(2))
    np.testing.assert_allclose(S, np.outer(v[1], k[1]), atol=1e-15)


def test_beta_zero_is_pure_decay():
    # beta = 0: S_t = (prod_{s<=t} alpha_s) S0 and o_t = S_t q_t.
    rng = np.random.default_rng(3)
    q, k, v, _, alpha = _rand_seq(rng, 7, 4, 3)
    S0 = rng.standard_normal((3, 4))
    o, S = oracle.gdn_recurrent(q, k, v, np.zeros(7), alpha, S0=S0)
    gam = np.cumprod(alpha)
    np.testing.assert_allclose(S, gam[-1] * S0, rtol=1e-13)
    for t in range(7):
        np.testing.assert_allclose(o[t], gam[t] * S0 @ q[t], rtol=1e-12)


def test_scalar_recurrence_closed_form():
    # d = 1: s_t = a_t s_{t-1} + b_t with a_t = alpha_t (1 - beta_t k_t^2), b_t = beta_t v_t k_t,
    # whose solution is s_T = sum_t b_t prod_{u>t} a_u (+ prod a * s0).
    rng = np.random.default_rng(4)
    T = 9
    k = rng.choice([-1.0, 1.0], size=(T, 1))
    v = rng.standard_normal((T, 1))
    beta = rng.uniform(0.1, 0.9, T)
    alpha = rng.uniform(0.5, 1.0, T)
    s0 = np.array([[0.7]])
    q = np.ones((T, 1))
    o, S = oracle.gdn_recurrent(q, k, v, beta, alpha, S0=s0)
    a = alpha * (1 - beta * k[:, 0] ** 2)
    b = beta * v[:, 0] * k[:, 0]
    for t in range(T):
        expect = np.prod(a[:t + 1]) * 0.7 + sum(b[u] * np.prod(a[u + 1:t + 1]) for u in range(t + 1))
        np.testing.assert_allclose(o[t, 0], expect, rtol=1e-12)


def test_stability_bound():
    # ||S_t||_F <= alpha_t ||S_{t-1}||_F + beta_t ||v_t|| (I - beta k k^T has norm <= 1).
    rng = np.random.default_rng(5)
    q, k, v, beta, alpha = _rand_seq(rng, 40, 6, 5, slow=True)
    S = rng.standard_normal((5, 6))
    for t in range(40):
        _, S_new = oracle.gdn_recurrent(None, k[t:t + 1], v[t:t + 1], beta[t:t + 1], alpha[t:t + 1], S0=S)
        assert np.linalg.norm(S_new) <= alpha[t] * np.linalg.norm(S) + beta[t] * np.linalg.norm(v[t]) + 1e-12
        S = S_new


# ----------------------------------------------------------------------------- P2 identity
def test_alpha_one_beta_zero_is_identity():
    rng = np.random.default_rng(6)
    q, k, v, _, _ = _rand_seq(rng, 12, 4, 3)
    S0 = rng.standard_normal((3, 4))
    o, S = oracle.gdn_recurrent(q, k, v, np.zeros(12), np.ones(12), S0=S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, q @ S0.T, rtol=1e-14)
    A, B = oracle.chunk_transitions(k, v, np.zeros(12), np.ones(12), 4)
    np.testing.assert_array_equal(A, np.broadcast_to(np.eye(4), A.shape))
    np.testing.assert_array_equal(B, 0.0)


# ----------------------------------------------------------------------------- P1 / P7 chunks
@pytest.mark.parametrize("C", [1, 3, 4, 16, 21])
def test_chunk_transitions_compose_to_sequential(C):
    rng = np.random.default_rng(7)
    T, dk, dv = 21, 5, 3
    q, k, v, beta, alpha = _rand_seq(rng, T, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    _, S_seq = oracle.gdn_recurrent(None, k, v, beta, alpha, S0=S0)
    A, B = oracle.chunk_transitions(k, v, beta, alpha, C)
    assert A.shape[0] == math.ceil(T / C)
    S = S0
    for j in range(A.shape[0]):
        S = S @ A[j] + B[j]
    np.testing.assert_allclose(S, S_seq, atol=1e-12)


def test_transition_of_one_token():
    rng = np.random.default_rng(8)
    _, k, v, beta, alpha = _rand_seq(rng, 1, 4, 2)
    A, B = oracle.chunk_transition(k, v, beta, alpha)
    np.testing.assert_allclose(A, alpha[0] * (np.eye(4) - beta[0] * np.outer(k[0], k[0])), atol=1e-15)
    np.testing.assert_allclose(B, beta[0] * np.outer(v[0], k[0]), atol=1e-15)


def test_transitions_compose_over_halves():
    # The map of a 2C chunk is (A1 A2, B1 A2 + B2) of its halves.
    rng = np.random.default_rng(9)
    _, k, v, beta, alpha = _rand_seq(rng, 16, 5, 4)
    A, B = oracle.chunk_transition(k, v, beta, alpha)
    A1, B1 = oracle.chunk_transition(k[:8], v[:8], beta[:8], alpha[:8])
    A2, B2 = oracle.chunk_transition(k[8:], v[8:], beta[8:], alpha[8:])
    np.testing.assert_allclose(A, A1 @ A2, atol=1e-13)
    np.testing.assert_allclose(B, B1 @ A2 + B2, atol=1e-13)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_all_ones_gates_reproduce_native(C):
    # g = 1 everywhere: the routed prefill equals native GDN, for every chunk size.
    rng = np.random.default_rng(10)
    T, dk, dv = 64, 6, 4
    q, k, v, beta, alpha = _rand_seq(rng, T, dk, dv)
    N = math.ceil(T / C)
    out = oracle.hla_prefill(q, k, v, beta, alpha, C, tau=1e-3, gates_in=np.ones((N, N)))
    o_ref, _ = oracle.gdn_recurrent(q, k, v, beta, alpha)
    np.testing.assert_allclose(out["o"], o_ref, atol=1e-12)


def test_all_zero_gates_isolate_chunks():
    # g = 0: every query chunk starts from S0 and sees only its own tokens.
    rng = np.random.default_rng(11)
    T, C, dk, dv = 40, 8, 5, 3
    q, k, v, beta, alpha = _rand_seq(rng, T, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    N = T // C
    out = oracle.hla_prefill(q, k, v, beta, alpha, C, tau=1e-3, gates_in=np.zeros((N, N)), S0=S0)
    for i in range(N):
        np.testing.assert_array_equal(out["S_routed"][i], S0)
        o_i, _ = oracle.gdn_recurrent(q[i * C:(i + 1) * C], k[i * C:(i + 1) * C], v[i * C:(i + 1) * C],
                                      beta[i * C:(i + 1) * C], alpha[i * C:(i + 1) * C], S0=S0)
        np.testing.assert_allclose(out["o"][i * C:(i + 1) * C], o_i, atol=1e-14)
    assert out["count"].sum() == 0


def test_resumable_prefill():
    rng = np.random.default_rng(12)
    q, k, v, beta, alpha = _rand_seq(rng, 30, 4, 3)
    o, S = oracle.gdn_recurrent(q, k, v, beta, alpha)
    o1, S1 = oracle.gdn_recurrent(q[:13], k[:13], v[:13], beta[:13], alpha[:13])
    o2, S2 = oracle.gdn_recurrent(q[13:], k[13:], v[13:], beta[13:], alpha[13:], S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, atol=1e-14)
    np.testing.assert_allclose(S2, S, atol=1e-14)


def test_batched_recurrence_matches_per_sequence():
    rng = np.random.default_rng(13)
    seqs = [_rand_seq(rng, 9, 4, 3) for _ in range(3)]
    stacked = [np.stack([s[i] for s in seqs]) for i in range(5)]
    o, S = oracle.gdn_recurrent(*stacked)
    for b, s in enumerate(seqs):
        ob, Sb = oracle.gdn_recurrent(*s)
        np.testing.assert_allclose(o[b], ob, atol=1e-15)
        np.testing.assert_allclose(S[b], Sb, atol=1e-15)


# ----------------------------------------------------------------------------- P5 brute force
def _brute_force_chunk_output(q, k, v, beta, alpha, C, i, selected, S0):
    """o of chunk i = the plain recurrence over the selected history chunks' tokens
    (in time order) followed by chunk i's tokens."""
    idx = [t for j in sorted(selected) for t in range(j * C, (j + 1) * C)]
    _, S = oracle.gdn_recurrent(None, k[idx], v[idx], beta[idx], alpha[idx], S0=S0) if idx else (None, S0)
    sl = slice(i * C, (i + 1) * C)
    o, _ = oracle.gdn_recurrent(q[sl], k[sl], v[sl], beta[sl], alpha[sl], S0=S)
    return o


@pytest.mark.parametrize("C,T", [(1, 5), (2, 8), (4, 16), (3, 12)])
def test_brute_force_binary_gates(C, T):
    rng = np.random.default_rng(20 + C)
    dk, dv = 4, 3
    q, k, v, beta, alpha = _rand_seq(rng, T, dk, dv)
    S0 = 0.3 * rng.standard_normal((dv, dk))
    N = T // C
    g = (rng.uniform(size=(N, N)) < 0.5).astype(float)
    out = oracle.hla_prefill(q, k, v, beta, alpha, C, tau=0.5, gates_in=g, S0=S0)
    for i in range(N):
        sel = [j for j in range(i) if g[i, j] == 1.0]
        np.testing.assert_allclose(out["o"][i * C:(i + 1) * C],
                                   _brute_force_chunk_output(q, k, v, beta, alpha, C, i, sel, S0), atol=1e-12)


@pytest.mark.parametrize("C,T", [(1, 5), (2, 8), (4, 16)])
def test_brute_force_fractional_gates(C, T):
    # Fractional gates: the output equals the expectation over independent Bernoulli(g_ij)
    # selections of history chunks (affine maps preserve convex combinations).
    rng = np.random.default_rng(30 + C)
    dk, dv = 4, 3
    q, k, v, beta, alpha = _rand_seq(rng, T, dk, dv)
    S0 = 0.3 * rng.standard_normal((dv, dk))
    N = T // C
    g = rng.uniform(0.05, 0.95, size=(N, N))
    out = oracle.hla_prefill(q, k, v, beta, alpha, C, tau=1e-3, gates_in=g, S0=S0)
    for i in range(N):
        expect = np.zeros((C, dv))
        for bits in itertools.product([0, 1], repeat=i):
            p = np.prod([g[i, j] if b else 1 - g[i, j] for j, b in enumerate(bits)])
            sel = [j for j, b in enumerate(bits) if b]
            expect += p * _brute_force_chunk_output(q, k, v, beta, alpha, C, i, sel, S0)
        np.testing.assert_allclose(out["o"][i * C:(i + 1) * C], expect, atol=1e-12)


def test_replay_composition_matches_transition_composition():
    rng = np.random.default_rng(40)
    T, C = 48, 8
    q, k, v, beta, alpha = _rand_seq(rng, T, 5, 4)
    N = T // C
    g = rng.uniform(size=(N, N))
    r = oracle.router_gates(q, k, C, C, tau=0.2, gates_in=g)
    A, B = oracle.chunk_transitions(k, v, beta, alpha, C)
    S0 = rng.standard_normal((4, 5))
    S1 = oracle.routed_states(A, B, r["ghat"], r["mask"], S0=S0)
    S2 = oracle.routed_states_by_replay(k, v, beta, alpha, C, r["ghat"], r["mask"], S0=S0)
    np.testing.assert_allclose(S1, S2, atol=1e-12)


# ----------------------------------------------------------------------------- router
def test_log_mean_exp_is_logsumexp_minus_log_n():
    rng = np.random.default_rng(50)
    s = 30 * rng.standard_normal((7, 13))
    np.testing.assert_allclose(oracle.log_mean_exp(s), scipy.special.logsumexp(s, axis=-1) - np.log(13), rtol=1e-13)


def test_router_gates_against_library_routines():
    rng = np.random.default_rng(51)
    T, C, dk = 40, 8, 6
    q, k, _, _, _ = _rand_seq(rng, T, dk, 2)
    r = oracle.router_gates(q, k, C, C, tau=1e-3)
    N = T // C
    for i in range(N):
        qbar = q[i * C:(i + 1) * C].sum(axis=0) / C
        for j in range(N):
            if j < i:
                s = k[j * C:(j + 1) * C] @ qbar / np.sqrt(dk)
                expect = scipy.special.expit(scipy.special.logsumexp(s) - np.log(C))
            else:
                expect = 1.0 if j == i else 0.0
            np.testing.assert_allclose(r["gates"][i, j], expect, rtol=1e-13)
    assert r["mask"].sum() == N * (N - 1) // 2


def test_router_identical_reps_reduce_to_single_score():
    # If every representative of a chunk equals r, the pooled score is exactly qbar.r/sqrt(dk).
    rng = np.random.default_rng(52)
    T, C, dk = 24, 8, 4
    q = rng.standard_normal((T, dk))
    rows = rng.standard_normal((3, dk))
    reps = np.repeat(rows, 5, axis=0)  # n_rep = 5 identical rows per chunk
    r = oracle.router_gates(q, reps, 5, C, tau=0.0)
    qbar2 = q[16:24].mean(axis=0)
    np.testing.assert_allclose(r["gates"][2, 1], scipy.special.expit(qbar2 @ rows[1] / 2.0), rtol=1e-13)


def test_threshold_skips_strictly_below_tau_without_renormalising():
    tau = np.float32(0.1)
    g = np.zeros((4, 4))
    g[1, 0] = float(tau)                      # exactly tau: kept
    g[2, 0] = float(np.nextafter(tau, 0))     # just below: skipped
    g[2, 1] = 0.7
    g[3, :3] = [0.05, 0.3, 0.2]
    r = oracle.router_gates(np.zeros((4, 2)), np.zeros((4, 2)), 1, 1, tau=tau, gates_in=g)
    assert r["mask"][1, 0] and not r["mask"][2, 0] and r["mask"][2, 1]
    assert list(r["active"][3]) == [1, 2]
    assert r["ghat"][3, 1] == 0.3 and r["ghat"][3, 2] == 0.2  # no renormalisation
    np.testing.assert_array_equal(r["count"], [0, 1, 1, 2])
    np.testing.assert_array_equal(np.diag(r["gates"]), 1.0)
    assert np.all(np.triu(r["gates"], 1) == 0)


def test_n_eff_cases():
    np.testing.assert_allclose(oracle.n_eff(np.full(7, 0.3)), 7.0)
    np.testing.assert_allclose(oracle.n_eff(np.array([0, 0, 0.9, 0])), 1.0)
    assert oracle.n_eff(np.zeros(5)) == 0.0
    np.testing.assert_allclose(oracle.n_eff(np.array([1.0, 1.0, 0.0])), 2.0)


# ----------------------------------------------------------------------------- P10 decode
def test_native_decode_equals_recurrence():
    rng = np.random.default_rng(60)
    q, k, v, beta, alpha = _rand_seq(rng, 10, 4, 3)
    o_ref, S_ref = oracle.gdn_recurrent(q, k, v, beta, alpha)
    S = np.zeros((3, 4))
    for t in range(10):
        r = oracle.decode_step(q[t], k[t], v[t], beta[t], alpha[t], S, None, None, None, None, 0.0)
        S = r["B_cur"]
        np.testing.assert_allclose(r["o"], o_ref[t], atol=1e-14)
    np.testing.assert_allclose(S, S_ref, atol=1e-14)


def test_routed_decode_with_commits_equals_routed_prefill():
    # Decode token by token, committing every C tokens, with the prefill's gate row for the
    # current chunk: the outputs equal the routed prefill's.
    rng = np.random.default_rng(61)
    T, C, dk, dv = 24, 4, 5, 3
    q, k, v, beta, alpha = _rand_seq(rng, T, dk, dv)
    N = T // C
    g = rng.uniform(0.0, 1.0, size=(N, N))
    pre = oracle.hla_prefill(q, k, v, beta, alpha, C, tau=0.2, gates_in=g)
    cA, cB = np.zeros((0, dk, dk)), np.zeros((0, dv, dk))
    A_cur, B_cur = np.eye(dk), np.zeros((dv, dk))
    for t in range(T):
        i = t // C
        r = oracle.decode_step(q[t], k[t], v[t], beta[t], alpha[t], B_cur, A_cur, cA, cB, None, 0.2,
                               gates_in=g[i, :i], commit=(t % C == C - 1))
        np.testing.assert_allclose(r["o"], pre["o"][t], atol=1e-12)
        A_cur, B_cur, cA, cB = r["A_cur"], r["B_cur"], r["cache_A"], r["cache_B"]
    np.testing.assert_allclose(cA, pre["A"], atol=1e-12)
    np.testing.assert_allclose(cB, pre["B"], atol=1e-12)


def test_decode_gates_equal_prefill_gates_for_constant_query():
    # With q constant over the query chunk, its mean is that q: decode and prefill gates agree.
    rng = np.random.default_rng(62)
    T, C, dk = 20, 4, 6
    q, k, _, _, _ = _rand_seq(rng, T, dk, 2)
    q[16:20] = q[16]
    r = oracle.router_gates(q, k, C, C, tau=0.0)
    reps = k[:16].reshape(4, C, dk)
    d = oracle.decode_step(q[16], k[16], np.zeros(2), 0.5, 0.5, np.zeros((2, dk)), np.eye(dk),
                           np.zeros((4, dk, dk)), np.zeros((4, 2, dk)), reps, 0.0)
    np.testing.assert_allclose(d["gates"], r["gates"][4, :4], rtol=1e-13)


# ----------------------------------------------------------------------------- P11 Tail-Replay
def test_tail_replay_error_bound():
    # ||S_full - S_replay||_2 <= (prod_{suffix} alpha) ||S_{T-L}||_2.
    rng = np.random.default_rng(70)
    T, L = 60, 20
    _, k, v, beta, alpha = _rand_seq(rng, T, 5, 4, slow=True)
    S_rep, S_full = oracle.tail_replay(k, v, beta, alpha, L)
    _, S_pre = oracle.gdn_recurrent(None, k[:T - L], v[:T - L], beta[:T - L], alpha[:T - L])
    bound = 10.0 ** oracle.tail_replay_bound_log10(alpha[T - L:], S_pre)
    err = np.linalg.norm(S_full - S_rep, 2)
    assert err <= bound * (1 + 1e-12) + 1e-14
    assert err > 0.1 * bound  # the bound is not vacuous here
    # equality case: one token with k orthogonal to the prefix state's rows (beta = 0), so
    # the only difference is alpha times the starting state
    S0 = rng.standard_normal((4, 5))
    _, S_a = oracle.gdn_recurrent(None, np.zeros((1, 5)), np.zeros((1, 4)), np.zeros(1), np.array([0.3]), S0=S0)
    assert math.isclose(np.linalg.norm(S_a, 2), 10.0 ** oracle.tail_replay_bound_log10([0.3], S0), rel_tol=1e-12)
    # With L = T the replay is the full prefill.
    S_rep2, S_full2 = oracle.tail_replay(k, v, beta, alpha, T)
    np.testing.assert_array_equal(S_rep2, S_full2)


# ----------------------------------------------------------------------------- inputs / golden
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(80)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = inputs.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_slices_agree_with_full_draw():
    full = inputs.gen_tokens(2, 9000, 2, 8, 4, dtype="bf16", seed=3)
    part = inputs.gen_tokens(2, 9000, 2, 8, 4, dtype="bf16", seed=3, t_range=(8100, 9000))
    for name in ("q", "k", "v", "beta", "alpha"):
        np.testing.assert_array_equal(getattr(full, name)[:, 8100:], getattr(part, name))


def test_generator_distributions():
    x = inputs.gen_tokens(1, 4096, 2, 64, 64, dtype="f32", seed=0)
    np.testing.assert_allclose(np.linalg.norm(x.f64("k"), axis=-1), 1.0, rtol=1e-6)
    assert 0.10 < np.median(x.alpha) < 0.14           # exp(-softplus(N(0,1)+2)) has median ~0.119
    assert 0.45 < np.median(x.beta) < 0.55
    p = inputs.gen_tokens(1, 8192, 1, 16, 16, dtype="bf16", seed=0, plant_period=4096)
    planted = np.abs(p.f64("v")[0, [4095, 8191], 0]).mean()
    assert planted > 3 * np.abs(p.f64("v")[0, :4000, 0]).mean()


def test_golden_affine_memory_accounting():
    # Chunk summaries are two d x d matrices (A_c and B_c) at 2 bytes per element.
    g = json.load(open(os.path.join(GOLDEN, "affine_memory.json")))
    T, d = g["context_tokens"], g["head_dim"]
    kv = 2 * T * d * 2
    assert kv == g["kv_bytes_per_layer_head"]
    from gated_deltanet_hybrid_amd.layout import transition_cache_bytes
    for C, frac in g["affine_fraction_of_kv"].items():
        assert transition_cache_bytes(n_chunks=T // int(C), dk=d, dv=d, dtype="bf16") == frac * kv
