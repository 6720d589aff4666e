"""Oracle functions (float64 numpy).  Test infrastructure only; see the package docstring.

Every array is float64.  Per-(batch, head) functions take token-major arrays:
q, k [T, dk], v [T, dv], beta, alpha [T]; the math state S is [dv, dk].
"""
from __future__ import annotations

import math

import numpy as np

# Readings of the pages that no printed value can confirm (reported as parity unpinned).
PARITY_UNPINNED = (
    "router score pooling is log-MEAN-exp (HLA Overview) rather than log-sum-exp "
    "(HLA Methodology paragraph 2); the two differ by log(n_rep)",
    "representatives are the history chunk's raw keys, or (window_reps) the learned "
    "pooler with seeded random weights: trained weights are not on the pages",
    "the pooler's self-attention is one head, scaled by 1/sqrt(dk), over the keys of the "
    "window, with no causal mask inside a completed window; every projection is dk x dk",
    "the decode-time gate query is the token's own q; the prefill gate query is the mean "
    "of q over the query chunk",
    "gates are per (batch, head)",
    "Gated DeltaNet-2: the decay acts before the edit, the read uses k_t and the erase "
    "is (S' k_t)(b_t o k_t)^T, the write (w_t o v_t) k_t^T (the pages give no formula)",
)


# --------------------------------------------------------------------------- O1
def gdn_recurrent(q, k, v, beta, alpha, S0=None):
    """Token-by-token gated delta rule.

    For each token t:  S <- alpha_t * S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    then o_t = S q_t (the read sees token t's own write).  [HLA] Methodology paragraph 1:
    decay and edit the old state, then add the key-value write.

    Leading batch dimensions are allowed: q [..., T, dk], beta [..., T], S0 [..., dv, dk].
    Returns (o [..., T, dv], S_final [..., dv, dk]).  q may be None (state only).
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, dk = k.shape[-2], k.shape[-1]
    dv = v.shape[-1]
    batch = k.shape[:-2]
    S = np.zeros(batch + (dv, dk)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = None if q is None else np.zeros(batch + (T, dv))
    for t in range(T):
        kt = k[..., t, :]
        vt = v[..., t, :]
        bt = np.asarray(beta)[..., t][..., None, None]
        at = np.asarray(alpha)[..., t][..., None, None]
        Sk = np.einsum("...ij,...j->...i", S, kt)                  # S k_t  [dv]
        S = at * (S - bt * Sk[..., :, None] * kt[..., None, :]) + bt * vt[..., :, None] * kt[..., None, :]
        if q is not None:
            o[..., t, :] = np.einsum("...ij,...j->...i", S, q[..., t, :])
    return o, S


# --------------------------------------------------------------------------- chunks
def chunk_bounds(T, C):
    """Chunks start at token 0 of the processed range; the last one may be partial."""
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def chunk_transition(k, v, beta, alpha):
    """Exact affine map of one chunk, built token by token (never through UT/WY).

    [HLA] Methodology paragraph 1 and Key Contributions 2: because the per-token updates
    are affine, a whole chunk is one affine map S -> S A + B.  A is the product of the
    per-token linear parts alpha_t (I - beta_t k_t k_t^T) in token order; B is the state
    the chunk produces from a zero start.  Returns (A [dk, dk], B [dv, dk]).
    """
    dk = k.shape[-1]
    A = np.eye(dk)
    for t in range(k.shape[0]):
        kt = k[t]
        A = alpha[t] * (A - beta[t] * np.outer(A @ kt, kt))
    _, B = gdn_recurrent(None, k, v, beta, alpha)
    return A, B


def chunk_transitions(k, v, beta, alpha, C):
    """(A [N, dk, dk], B [N, dv, dk]) for every chunk of one (batch, head) sequence."""
    A, B = [], []
    for s, e in chunk_bounds(k.shape[0], C):
        a, b = chunk_transition(k[s:e], v[s:e], beta[s:e], alpha[s:e])
        A.append(a)
        B.append(b)
    return np.stack(A), np.stack(B)


# --------------------------------------------------------------------------- O3 router
def log_mean_exp(s, axis=-1):
    """log(mean(exp(s))) computed with the max shifted out."""
    m = np.max(s, axis=axis, keepdims=True)
    return np.squeeze(m, axis) + np.log(np.mean(np.exp(s - m), axis=axis))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def n_eff(g):
    """Order-2 effective number of accessed chunks, (sum g)^2 / sum g^2 ([HLA] Key
    Contributions 3, Methodology paragraph 4: inverse sum of squares); 0 if all are 0."""
    g = np.asarray(g, np.float64)
    den = np.sum(g * g, axis=-1)
    num = np.sum(g, axis=-1) ** 2
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def window_rep(X, Wq, Wk, Wv, Wp):
    """One representative from the keys X [n, dk] of one pooling window ([HLA] Methodology
    paragraph 2): self-attention inside the window, mean-pool of its token outputs, then a
    learned projection.  Weights are [out, in]: a row vector x maps to W @ x.
      Q = X Wq^T, K = X Wk^T, V = X Wv^T
      P = row-softmax(Q K^T / sqrt(dk))      (every token attends to the whole window)
      O = P V;   rep = Wp (mean over the n token rows of O)."""
    n, dk = X.shape
    Q, K, V = X @ Wq.T, X @ Wk.T, X @ Wv.T
    s = Q @ K.T / math.sqrt(dk)
    s = s - s.max(axis=1, keepdims=True)
    P = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    O = P @ V
    return Wp @ O.mean(axis=0)


def window_reps(k, C, window, Wq, Wk, Wv, Wp):
    """Representatives of every chunk for one (batch, head) sequence: chunk c is split into
    C / window pooling windows of consecutive tokens, one representative each, rows
    [c n_rep, (c + 1) n_rep) with n_rep = C / window.  A window cut by the end of the
    sequence pools the tokens it has; one with no tokens gets a zero row."""
    T, dk = k.shape
    assert C % window == 0
    n_rep = C // window
    bounds = chunk_bounds(T, C)
    reps = np.zeros((len(bounds) * n_rep, dk))
    for c, (s, e) in enumerate(bounds):
        for w in range(n_rep):
            lo, hi = s + w * window, min(s + (w + 1) * window, e)
            if hi > lo:
                reps[c * n_rep + w] = window_rep(k[lo:hi], Wq, Wk, Wv, Wp)
    return reps


def router_gates(q, reps, n_rep, C, tau, gates_in=None, Wr=None):
    """Query-chunk x history-chunk gates for one (batch, head) sequence.

    q [T, dk]; reps [(N-1) * n_rep or more, dk]: chunk j's representatives are rows
    [j n_rep, (j + 1) n_rep).  [HLA] Overview (log-mean-exp pooled routing gates) and
    Methodology paragraphs 2-4:
      * query of chunk i = mean of q over the chunk's tokens, then projected by Wr
        [dk, dk] when given (the router's learned query projection);
      * l_ij = log-mean-exp over chunk j's representatives r of (qbar_i . r) / sqrt(dk);
      * g_ij = sigmoid(l_ij) for j < i, independent (no normalisation over j);
      * the current chunk has weight 1, future chunks are masked (weight 0);
      * a history gate below tau is set to zero without renormalisation.  The pages fix
        no precision for this test; tau crosses the C boundary as a float32 and the gates
        it is compared with are float32 outputs, so the comparison is taken in float32:
        keep iff float32(g) >= float32(tau).  A gate within float32 rounding of tau may go
        either way, which is why exact mask parity is checked on caller gates that both
        sides read as the same float32 numbers.
    ``gates_in`` [N, N] replaces the computed history gates (entries j < i).
    Returns dict(gates [N,N], mask [N,N] bool (history only), ghat [N,N], active (list of
    ascending index arrays), count [N], n_eff [N]).
    """
    T, dk = q.shape
    bounds = chunk_bounds(T, C)
    N = len(bounds)
    g = np.zeros((N, N))
    if gates_in is None:
        qbar = np.stack([q[s:e].mean(axis=0) for s, e in bounds])
        if Wr is not None:
            qbar = qbar @ Wr.T
        for i in range(N):
            for j in range(i):
                r = reps[j * n_rep:(j + 1) * n_rep]
                g[i, j] = _sigmoid(log_mean_exp(r @ qbar[i] / math.sqrt(dk)))
    else:
        g = np.tril(np.asarray(gates_in, np.float64), -1)
    np.fill_diagonal(g, 1.0)
    hist = np.tril(np.ones((N, N), bool), -1)
    mask = hist & (g.astype(np.float32) >= np.float32(tau))
    ghat = np.where(mask, g, 0.0)
    active = [np.nonzero(mask[i])[0] for i in range(N)]
    return dict(gates=g, mask=mask, ghat=ghat, active=active,
                count=mask.sum(axis=1), n_eff=n_eff(ghat))


# --------------------------------------------------------------------------- O4 / O5
def routed_states(A, B, ghat, mask, S0=None):
    """Initial state of every query chunk i, composed chronologically over history chunks.

    [HLA] Methodology paragraph 3: the gate interpolates the chunk's full transition with
    the identity, S -> g (S A_j + B_j) + (1 - g) S, so g = 1 applies the chunk and g = 0
    leaves the state untouched; chunks compose in time order ([HLA] Methodology paragraph
    1: affine maps compose).  Masked chunks are skipped.  Returns [N, dv, dk].
    """
    N, dv, dk = B.shape
    out = np.zeros((N, dv, dk))
    for i in range(N):
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
        for j in range(i):
            if mask[i, j]:
                S = ghat[i, j] * (S @ A[j] + B[j]) + (1.0 - ghat[i, j]) * S
        out[i] = S
    return out


def routed_states_by_replay(k, v, beta, alpha, C, ghat, mask, S0=None):
    """Same as ``routed_states`` but applies chunk j by replaying its tokens (no A, B)."""
    bounds = chunk_bounds(k.shape[0], C)
    N, dv, dk = len(bounds), v.shape[1], k.shape[1]
    out = np.zeros((N, dv, dk))
    for i in range(N):
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
        for j in range(i):
            if mask[i, j]:
                s, e = bounds[j]
                _, Sj = gdn_recurrent(None, k[s:e], v[s:e], beta[s:e], alpha[s:e], S0=S)
                S = ghat[i, j] * Sj + (1.0 - ghat[i, j]) * S
        out[i] = S
    return out


def routed_outputs(q, k, v, beta, alpha, C, S_routed):
    """Outputs of every chunk i: the plain recurrence over chunk i's own tokens started
    from its routed state (the current chunk has weight one).  Returns o [T, dv]."""
    o = np.zeros((q.shape[0], v.shape[1]))
    for i, (s, e) in enumerate(chunk_bounds(q.shape[0], C)):
        o[s:e], _ = gdn_recurrent(q[s:e], k[s:e], v[s:e], beta[s:e], alpha[s:e], S0=S_routed[i])
    return o


def hla_prefill(q, k, v, beta, alpha, C, tau, reps=None, n_rep=None, gates_in=None, S0=None, Wr=None):
    """Whole routed prefill for one (batch, head): transitions, gates, states, outputs."""
    if reps is None:
        reps, n_rep = k, C
    A, B = chunk_transitions(k, v, beta, alpha, C)
    r = router_gates(q, reps, n_rep, C, tau, gates_in=gates_in, Wr=Wr)
    S = routed_states(A, B, r["ghat"], r["mask"], S0=S0)
    o = routed_outputs(q, k, v, beta, alpha, C, S)
    return dict(A=A, B=B, S_routed=S, o=o, **r)


# --------------------------------------------------------------------------- O6 decode
def decode_step(q, k, v, beta, alpha, B_cur, A_cur, cache_A, cache_B, cache_reps, tau,
                gates_in=None, commit=False, Wr=None):
    """One single-token decode step for one (sequence, head).

    [HLA] Key Contributions 3 (dynamic autoregressive decoding) with Methodology
    paragraphs 2-4.  The live chunk is the affine map (A_cur, B_cur) of the tokens since
    the last cached chunk; this token extends it.  Gates over the cached chunks use the
    token's own q.  The routed state S~ composes the gated cached chunks from zero; the
    output reads the live chunk applied after it: o = (S~ A_cur + B_cur) q.
    ``A_cur is None`` selects native GDN: B_cur is the full-prefix state, o = B_cur q.
    cache_A [Nc, dk, dk], cache_B [Nc, dv, dk], cache_reps [Nc, n_rep, dk].  Wr [dk, dk]
    projects the gate query when given.
    Returns dict(o, B_cur, A_cur, gates, ghat, cache_A, cache_B) after the step (and the
    optional commit, which appends the live chunk and resets it to (I, 0)).
    """
    dk = k.shape[0]
    lin = alpha * (np.eye(dk) - beta * np.outer(k, k))
    return decode_read(q, B_cur @ lin + beta * np.outer(v, k), None if A_cur is None else A_cur @ lin,
                       cache_A, cache_B, cache_reps, tau, gates_in=gates_in, commit=commit, Wr=Wr)


def decode_read(q, B_cur, A_cur, cache_A, cache_B, cache_reps, tau, gates_in=None, commit=False, Wr=None):
    """The decode step after the live chunk (A_cur, B_cur) has taken the token: gates over
    the cached chunks, the routed state and the output (see decode_step)."""
    dk = q.shape[0]
    if A_cur is None:
        return dict(o=B_cur @ q, B_cur=B_cur, A_cur=None)
    Nc = cache_A.shape[0]
    g = np.zeros(Nc)
    qr = q if Wr is None else Wr @ q
    for j in range(Nc):
        if gates_in is None:
            g[j] = _sigmoid(log_mean_exp(cache_reps[j] @ qr / math.sqrt(dk)))
        else:
            g[j] = gates_in[j]
    keep = g.astype(np.float32) >= np.float32(tau)
    ghat = np.where(keep, g, 0.0)
    S = np.zeros_like(B_cur)
    for j in range(Nc):
        if keep[j]:
            S = ghat[j] * (S @ cache_A[j] + cache_B[j]) + (1.0 - ghat[j]) * S
    o = (S @ A_cur + B_cur) @ q
    out = dict(o=o, gates=g, ghat=ghat, S_routed=S)
    if commit:
        cache_A = np.concatenate([cache_A, A_cur[None]])
        cache_B = np.concatenate([cache_B, B_cur[None]])
        A_cur, B_cur = np.eye(dk), np.zeros_like(B_cur)
    out.update(B_cur=B_cur, A_cur=A_cur, cache_A=cache_A, cache_B=cache_B)
    return out


# --------------------------------------------------------------------------- O7
def tail_replay(k, v, beta, alpha, L):
    """[TR]: rebuild the recurrent state of a T-token prefix by replaying only its last L
    tokens from a zero state.  Returns (S_replay, S_full), both [..., dv, dk]."""
    T = k.shape[-2]
    _, S_rep = gdn_recurrent(None, k[..., T - L:, :], v[..., T - L:, :],
                             beta[..., T - L:], alpha[..., T - L:])
    _, S_full = gdn_recurrent(None, k, v, beta, alpha)
    return S_rep, S_full


def tail_replay_bound_log10(alpha_suffix, S_prefix):
    """log10 of the error bound of a replay from zero ([TR] state rebuild).

    Every token's linear part alpha_t (I - beta_t k_t k_t^T) has 2-norm alpha_t when
    beta_t is in [0, 1] and k_t has unit length, and the replay differs from the full
    recurrence only by the state it starts from (zero instead of S_{T-L}).  So
    ||S_full - S_replay||_2 <= (prod of alpha over the suffix) ||S_{T-L}||_2.  Taken in
    log10, because the product underflows float64 for long suffixes.
    alpha_suffix [L]; S_prefix [dv, dk], the state in front of the suffix.
    """
    nrm = np.linalg.norm(np.asarray(S_prefix, np.float64), 2)
    if nrm == 0.0:
        return -math.inf
    return float(np.sum(np.log10(np.asarray(alpha_suffix, np.float64))) + math.log10(nrm))
