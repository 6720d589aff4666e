"""GPU parity of the learned chunk representatives (hla_chunk_reps), through the C ABI.

The oracle pools every window in float64 ([HLA] Methodology paragraph 2); the library folds
the router's query projection into its output, r' = Wr^T r, which the oracle pins show is
what the router needs ((Wr q) . r = q . (Wr^T r)).  Bars: max|diff| / max|ref| <= 2e-2 for
bf16 (float32 accumulation of bf16 products, with Q, K, P and V rounded to bf16 between the
products) and 1e-4 for float32.  Gates downstream of the representatives are held to the
bound their error implies: log-mean-exp moves by at most the largest change of its
arguments and the sigmoid's slope is at most 1/4, so for query chunk i and history chunk j
|dg_ij| <= max over j's representatives r of |qbar_i . dr| / (4 sqrt(dk)), plus 1e-5 for
the float32 gate arithmetic itself.
"""
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
    ("bf16", 64, 16, 128, 3 * 128 - 50, True, False),
    ("bf16", 128, 8, 256, 2 * 256 - 3, False, True),
    ("bf16", 128, 32, 64, 33, False, False),
    ("f32", 64, 32, 64, 200, False, True),
    ("f32", 128, 16, 64, 130, True, True),
    ("bf16", 128, 64, 128, 3 * 128 - 40, False, True),
    ("bf16", 64, 64, 64, 4 * 64 - 23, True, False),
    ("f32", 128, 64, 64, 2 * 64 + 9, False, True),
]
IDS = [f"{c[0]}-dk{c[1]}-w{c[2]}-C{c[3]}-T{c[4]}{'-shared' if c[5] else ''}{'-Wr' if c[6] else ''}" for c in CASES]


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def weights(H, dk, dtype, shared, with_wr, seed, r_scale=None):
    Ws = inputs.gen_pooler_weights(H, dk, dtype=dtype, seed=seed, shared=shared, r_scale=r_scale)
    dev_w = {n: dev(a, dtype) for n, a in Ws.items() if with_wr or n != "Wr"}
    f64 = {n: inputs.to_f64(a, dtype) for n, a in Ws.items()}
    return dev_w, f64


def oracle_reps(k64, f64, h, C, window, with_wr):
    """float64 representatives of one (batch, head) sequence, in the library's folded form."""
    hw = 0 if f64["Wq"].shape[0] == 1 else h
    r = oracle.window_reps(k64, C, window, f64["Wq"][hw], f64["Wk"][hw], f64["Wv"][hw], f64["Wp"][hw])
    return r @ f64["Wr"][hw] if with_wr else r


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_chunk_reps(case):
    dtype, dk, window, C, T, shared, with_wr = case
    note(f"chunk reps {case}")
    B, H = 2, 3
    x = inputs.gen_tokens(B, T, H, dk, dk, dtype=dtype, seed=71, with_q=False)
    k = dev(x.k, dtype)
    Wd, W64 = weights(H, dk, dtype, shared, with_wr, seed=72)
    reps = hla().chunk_reps(k, Wd, window=window, C=C)
    torch.cuda.synchronize()
    N = math.ceil(T / C)
    assert reps.shape == (B, N * (C // window), H, dk)
    got = host(reps)
    k64 = x.f64("k")
    for b in range(B):
        for h in range(H):
            ref = oracle_reps(k64[b, :, h], W64, h, C, window, with_wr)
            assert_close(got[b, :, h], ref, dtype, f"reps b{b} h{h}")
            empty = np.all(ref == 0, axis=1)
            assert np.all(got[b, empty, h] == 0)


def test_chunk_reps_token_window_view():
    # keys given as a window of a longer allocation (ld_T > T): only rows [0, T) are read
    dtype, dk, window, C, T, ld = "bf16", 128, 32, 64, 150, 300
    note("chunk reps token window")
    x = inputs.gen_tokens(1, ld, 2, dk, dk, dtype=dtype, seed=73, with_q=False)
    k = dev(x.k, dtype)[:, :T]
    Wd, W64 = weights(2, dk, dtype, False, True, seed=74)
    got = host(hla().chunk_reps(k, Wd, window=window, C=C))
    for h in range(2):
        ref = oracle_reps(x.f64("k")[0, :T, h], W64, h, C, window, True)
        assert_close(got[0, :, h], ref, dtype, f"reps h{h}")


def test_chunk_reps_full_size_sampled():
    # the benchmark's shape (B=1, H=16, T=32768, d=128, C=64, window 32): sampled windows
    dtype, dk, window, C, T, H = "bf16", 128, 32, 64, 32768, 16
    note("chunk reps full size")
    W = inputs.WORKLOADS["routed_prefill"]
    assert (W.T, W.H, W.dk) == (T, H, dk)
    x = inputs.gen_tokens(1, T, H, dk, dk, dtype=dtype, seed=0, stream=inputs.STREAM["routed_prefill"],
                          plant_period=W.plant_period, with_q=False)
    k = dev(x.k, dtype)
    Wd, W64 = weights(H, dk, dtype, False, True, seed=75)
    got = host(hla().chunk_reps(k, Wd, window=window, C=C))
    rng = np.random.default_rng(76)
    k64 = x.f64("k")
    n_rows = T // window
    picks = [(int(rng.integers(H)), int(rng.integers(n_rows))) for _ in range(24)] + [(0, 0), (H - 1, n_rows - 1)]
    ref = np.stack([oracle.window_rep(k64[0, r * window:(r + 1) * window, h], W64["Wq"][h], W64["Wk"][h],
                                      W64["Wv"][h], W64["Wp"][h]) @ W64["Wr"][h] for h, r in picks])
    assert_close(np.stack([got[0, r, h] for h, r in picks]), ref, dtype, "sampled reps")


def _gate_bound(qbar, d_reps, n_rep, dk):
    """[Nq, Nj] bound on the gate error that the representatives' error d_reps implies."""
    s = np.abs(qbar @ d_reps.T) / math.sqrt(dk)  # [Nq, Nj * n_rep]
    return s.reshape(len(qbar), -1, n_rep).max(axis=2) / 4 + 1e-5


@pytest.mark.parametrize("C,T", [(64, 7 * 64 - 20), (256, 6 * 256 - 40)])
def test_routed_prefill_with_learned_reps(C, T):
    dtype, dk, dv, window = "bf16", 128, 128, 32
    note(f"routed prefill learned reps C={C} T={T}")
    B, H = 1, 2
    n_rep = C // window
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=77, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    # a large query projection spreads the gates over (0, 1), as trained routers do
    Wd, W64 = weights(H, dk, dtype, False, True, seed=78, r_scale=400.0)
    # oracle representatives and gates first; tau sits in the middle of the widest gap
    # between the central half of all history gates, so no gate lies near the threshold
    per_head, gall = [], []
    for h in range(H):
        args = [x.f64(n)[0, :, h] for n in ("q", "k", "v", "beta", "alpha")]
        reps64 = oracle.window_reps(args[1], C, window, W64["Wq"][h], W64["Wk"][h], W64["Wv"][h], W64["Wp"][h])
        per_head.append((args, reps64))
        g = oracle.router_gates(args[0], reps64, n_rep, C, 0.0, Wr=W64["Wr"][h])["gates"]
        gall.append(g[np.tril_indices(g.shape[0], -1)])
    gs = np.sort(np.concatenate(gall))
    lo, hi = len(gs) // 4, max(len(gs) * 3 // 4, len(gs) // 4 + 1)
    i = lo + int(np.argmax(np.diff(gs[lo:hi + 1])))
    tau, half_gap = float((gs[i] + gs[i + 1]) / 2), float((gs[i + 1] - gs[i]) / 2)
    r = hla().hla_prefill(q, k, v, beta, alpha, tau=tau, C=C, pooler=Wd, window=window)
    torch.cuda.synchronize()
    for h in range(H):
        args, reps64 = per_head[h]
        ref = oracle.hla_prefill(*args, C, tau, reps=reps64, n_rep=n_rep, Wr=W64["Wr"][h])
        d_reps = host(r["reps"])[0, :, h] - reps64 @ W64["Wr"][h]
        qbar = np.stack([args[0][s:e].mean(axis=0) for s, e in oracle.chunk_bounds(T, C)])
        N = len(qbar)
        bound = _gate_bound(qbar, d_reps, n_rep, dk)[:, :N]
        g = host(r["gates"])[0, h]
        hist = np.tril(np.ones_like(g, bool), -1)
        assert np.all(np.abs(g - ref["gates"])[hist] <= bound[hist])
        assert bound[hist].max() < half_gap  # every gate is decided the same way on both sides
        np.testing.assert_array_equal(host(r["mask"])[0, h].astype(bool), ref["mask"])
        assert_close(host(r["S_routed"])[0, h], ref["S_routed"].transpose(0, 2, 1), dtype, "S_routed")
        assert_close(host(r["o"])[0, :, h], ref["o"], dtype, "routed o")
    assert 0 < sum(int(np.sum(gg >= tau)) for gg in gall) < sum(len(gg) for gg in gall)  # tau splits the gates


def test_decode_with_learned_reps():
    # reps of committed chunks from hla_chunk_reps fill the decode cache; the decode gates
    # use the token's q against them, i.e. (Wr q) . r
    dtype, dk, dv, window, C = "bf16", 128, 128, 32, 64
    note("decode learned reps")
    Bs, H, n_cap = 2, 2, 4
    n_rep = C // window
    hist = inputs.gen_tokens(Bs, n_cap * C, H, dk, dv, dtype=dtype, seed=79, with_q=False)
    Wd, W64 = weights(H, dk, dtype, False, True, seed=80, r_scale=50.0)
    reps = hla().chunk_reps(dev(hist.k, dtype), Wd, window=window, C=C)  # [Bs, n_cap*n_rep, H, dk]
    cache = reps.view(Bs, n_cap, n_rep, H, dk).permute(0, 3, 1, 2, 4).contiguous()
    At_s, Bc_s = inputs.gen_transitions(Bs, H, n_cap, dk, dv, dtype=dtype, seed=81)
    tok = inputs.gen_decode_tokens(Bs, H, dk, dv, step=0, dtype=dtype, seed=82)
    S0 = inputs.gen_state(Bs, H, dk, dv, seed=83)
    n_cache = np.array([4, 2], np.int32)
    S, A, nc = f32(S0), f32(np.tile(np.eye(dk, dtype=np.float32), (Bs, H, 1, 1))), torch.from_numpy(n_cache).cuda()
    go = torch.empty((Bs, H, n_cap), dtype=torch.float32, device="cuda")
    o = hla().gdn_decode(dev(tok["q"], dtype), dev(tok["k"], dtype), dev(tok["v"], dtype), f32(tok["beta"]),
                         f32(tok["alpha"]), S, At_cur=A, At_cache=dev(At_s, dtype), Bc_cache=dev(Bc_s, dtype),
                         reps_cache=cache, n_cache=nc, tau=0.0, gates_out=go)
    torch.cuda.synchronize()
    Am = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    q64 = inputs.to_f64(tok["q"], dtype)
    for b in range(Bs):
        for h in range(H):
            ncb = n_cache[b]
            r64 = oracle.window_reps(hist.f64("k")[b, :, h], C, window, W64["Wq"][h], W64["Wk"][h], W64["Wv"][h],
                                     W64["Wp"][h]).reshape(n_cap, n_rep, dk)
            ref = oracle.decode_step(q64[b, h], inputs.to_f64(tok["k"], dtype)[b, h],
                                     inputs.to_f64(tok["v"], dtype)[b, h], float(tok["beta"][b, h]),
                                     float(tok["alpha"][b, h]), S0[b, h].astype(np.float64).T, np.eye(dk),
                                     Am[b, h, :ncb], Bm[b, h, :ncb], r64[:ncb], 0.0, Wr=W64["Wr"][h])
            d_reps = host(cache)[b, h, :ncb].reshape(-1, dk) - (r64[:ncb] @ W64["Wr"][h]).reshape(-1, dk)
            bound = _gate_bound(q64[b, h][None], d_reps, n_rep, dk)[0]
            assert np.all(np.abs(host(go)[b, h, :ncb] - ref["gates"]) <= bound)
            assert_close(host(o)[b, h], ref["o"], dtype, f"decode o b{b} h{h}")
