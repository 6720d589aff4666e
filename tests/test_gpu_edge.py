"""Degenerate and extreme cases of the path on the GPU, through the C ABI, against the oracle.

* one token (one partial chunk, no history for the router);
* exactly one full chunk, and one full chunk plus one token;
* a threshold above every gate (every history pair skipped);
* decode with the largest cache a call accepts (1024 slots), about half of them active;
* learned representatives and Gated DeltaNet-2 on one token.

Bars as everywhere: max|diff| / max|ref| <= 1e-4 (float32), <= 2e-2 (bf16); masks and
lists bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, dev, f32, host, note, token_tensors

pytestmark = pytest.mark.gpu
C = 64


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def seq(x, b, h):
    return tuple(x.f64(n)[b, :, h] for n in ("q", "k", "v", "beta", "alpha"))


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128)])
@pytest.mark.parametrize("T", [1, C, C + 1])
def test_short_sequences(dtype, dk, dv, T):
    """Transitions, native prefill (outputs, state, state-only) and the routed prefill on
    one token, one full chunk, and one chunk plus one token."""
    note(f"short T={T} {dtype} dk={dk} dv={dv}")
    x = inputs.gen_tokens(2, T, 2, dk, dv, dtype=dtype, seed=111, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    S0 = inputs.gen_state(2, 2, dk, dv, seed=112)
    h = hla()
    At, Bc = h.chunk_transitions(k, v, beta, alpha)
    o, S = h.gdn_prefill(q, k, v, beta, alpha, S0=f32(S0))
    _, S_only = h.gdn_prefill(None, k, v, beta, alpha, S0=f32(S0), want_o=False)
    r = h.hla_prefill(q, k, v, beta, alpha, tau=1e-3)
    torch.cuda.synchronize()
    N = -(-T // C)
    assert At.shape[2] == N and r["gates"].shape[-1] == N
    for b in range(2):
        for hh in range(2):
            qq, kk, vv, bb, aa = seq(x, b, hh)
            A, Bm = oracle.chunk_transitions(kk, vv, bb, aa, C)
            assert_close(host(At[b, hh]), A.transpose(0, 2, 1), dtype, "At")
            assert_close(host(Bc[b, hh]), Bm.transpose(0, 2, 1), dtype, "Bc")
            o_ref, S_ref = oracle.gdn_recurrent(qq, kk, vv, bb, aa, S0=S0[b, hh].T.astype(np.float64))
            assert_close(host(o[b, :, hh]), o_ref, dtype, "o")
            assert_close(host(S[b, hh]), S_ref.T, dtype, "S_final")
            assert_close(host(S_only[b, hh]), S_ref.T, dtype, "state-only S_final")
            ref = oracle.hla_prefill(qq, kk, vv, bb, aa, C, 1e-3)
            np.testing.assert_array_equal(host(r["mask"])[b, hh].astype(bool), ref["mask"])
            assert host(r["active_cnt"])[b, hh].tolist() == ref["count"].tolist()
            assert_close(host(r["S_routed"])[b, hh], ref["S_routed"].transpose(0, 2, 1), dtype, "S_routed")
            assert_close(host(r["o"])[b, :, hh], ref["o"], dtype, "routed o")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_threshold_above_every_gate(dtype):
    """tau = 2 skips every history pair: every routed state is S0, lists are empty, N_eff is 0."""
    dk, dv, T = 64, 128, 5 * C - 9
    note(f"tau above every gate {dtype}")
    x = inputs.gen_tokens(1, T, 2, dk, dv, dtype=dtype, seed=113, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    S0 = inputs.gen_state(1, 2, dk, dv, seed=114)
    r = hla().hla_prefill(q, k, v, beta, alpha, tau=2.0, S0=f32(S0))
    torch.cuda.synchronize()
    N = -(-T // C)
    assert not host(r["mask"]).any()
    assert (host(r["active_cnt"]) == 0).all() and (host(r["active_idx"]) == -1).all()
    assert (host(r["n_eff"]) == 0).all()
    for hh in range(2):
        np.testing.assert_array_equal(host(r["S_routed"])[0, hh], np.broadcast_to(S0[0, hh], (N, dk, dv)))
        ref = oracle.hla_prefill(*seq(x, 0, hh), C, 2.0, S0=S0[0, hh].T.astype(np.float64))
        assert_close(host(r["o"])[0, :, hh], ref["o"], dtype, "routed o")


def test_decode_largest_cache():
    """n_cap = 1024 cached chunks (the largest a call accepts), caller gates of which about
    half pass tau = 0.5, and the routed read against the oracle."""
    dtype, dk, dv, n_cap = "bf16", 64, 64, 1024
    note("decode largest cache")
    Bs, H = 1, 2
    At_s, Bc_s = inputs.gen_transitions(Bs, H, n_cap, dk, dv, dtype=dtype, seed=115, norm=0.999, b_scale=0.05)
    G = inputs.gen_gates(Bs, H, n_cap + 1, seed=116, mode="uniform")[:, :, -1, :n_cap].copy()
    tok = inputs.gen_decode_tokens(Bs, H, dk, dv, step=0, dtype=dtype, seed=117)
    S0 = inputs.gen_state(Bs, H, dk, dv, seed=118)
    S, A = f32(S0), f32(np.tile(np.eye(dk, dtype=np.float32), (Bs, H, 1, 1)))
    nc = torch.full((Bs,), n_cap, dtype=torch.int32, device="cuda")
    go = torch.empty((Bs, H, n_cap), dtype=torch.float32, device="cuda")
    o = hla().gdn_decode(dev(tok["q"], dtype), dev(tok["k"], dtype), dev(tok["v"], dtype), f32(tok["beta"]),
                         f32(tok["alpha"]), S, At_cur=A, At_cache=dev(At_s, dtype), Bc_cache=dev(Bc_s, dtype),
                         n_cache=nc, gates_in=f32(G), tau=0.5, gates_out=go)
    torch.cuda.synchronize()
    Am = inputs.to_f64(At_s, dtype).transpose(0, 1, 2, 4, 3)
    Bm = inputs.to_f64(Bc_s, dtype).transpose(0, 1, 2, 4, 3)
    for hh in range(H):
        ref = oracle.decode_step(inputs.to_f64(tok["q"], dtype)[0, hh], inputs.to_f64(tok["k"], dtype)[0, hh],
                                 inputs.to_f64(tok["v"], dtype)[0, hh], float(tok["beta"][0, hh]),
                                 float(tok["alpha"][0, hh]), S0[0, hh].astype(np.float64).T, np.eye(dk), Am[0, hh],
                                 Bm[0, hh], None, 0.5, gates_in=G[0, hh].astype(np.float64))
        assert 300 < int(ref["ghat"].astype(bool).sum()) < 724
        np.testing.assert_array_equal(host(go)[0, hh], G[0, hh])
        assert_close(host(o)[0, hh], ref["o"], dtype, f"o h{hh}")


def test_learned_reps_and_gdn2_on_one_token():
    dtype, dk, dv = "bf16", 128, 128
    note("reps and gdn2 on one token")
    x = inputs.gen_tokens(1, 1, 2, dk, dv, dtype=dtype, seed=119)
    q, k, v, _, _ = token_tensors(x)
    W = inputs.gen_pooler_weights(2, dk, dtype=dtype, seed=120)
    reps = hla().chunk_reps(k, {n: dev(a, dtype) for n, a in W.items()}, window=32, C=C)
    g = inputs.gen_gdn2_gates(1, 1, 2, dk, dv, seed=121)
    o, S = hla().gdn2_prefill(q, k, v, f32(g["a"]), f32(g["b"]), f32(g["w"]))
    torch.cuda.synchronize()
    W64 = {n: inputs.to_f64(a, dtype) for n, a in W.items()}
    for hh in range(2):
        r = oracle.window_reps(x.f64("k")[0, :, hh], C, 32, W64["Wq"][hh], W64["Wk"][hh], W64["Wv"][hh], W64["Wp"][hh])
        assert np.all(r[1] == 0)
        assert_close(host(reps)[0, :, hh], r @ W64["Wr"][hh], dtype, "reps")
        o_ref, S_ref = oracle.gdn2_recurrent(x.f64("q")[0, :, hh], x.f64("k")[0, :, hh], x.f64("v")[0, :, hh],
                                             g["a"][0, :, hh].astype(np.float64), g["b"][0, :, hh].astype(np.float64),
                                             g["w"][0, :, hh].astype(np.float64))
        assert_close(host(o)[0, :, hh], o_ref, dtype, "gdn2 o")
        assert_close(host(S)[0, hh], S_ref.T, dtype, "gdn2 S")
