"""Backward of the Gated DeltaNet-2 path on the GPU (hla_gdn2_chunk_backward,
hla_gdn2_prefill_backward), through the C ABI, against the gradient oracle
(oracle.grad_gdn2: float64 autograd, pinned by finite differences, by the collapse to the
Gated DeltaNet gradients and by a closed form).

Bars as everywhere: max|diff| / max|ref| <= 1e-4 (float32 inputs), <= 2e-2 (bf16 inputs)
for every gradient tensor; skipped pairs get exactly zero gate gradient."""
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


def _gen(dtype, B, T, H, dk, dv, seed, alpha_mode="slow"):
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=seed, alpha_mode="slow")
    g = inputs.gen_gdn2_gates(B, T, H, dk, dv, seed=seed + 1, alpha_mode=alpha_mode)
    q, k, v = (dev(getattr(x, n), dtype) for n in ("q", "k", "v"))
    return x, g, q, k, v, (f32(g["a"]), f32(g["b"]), f32(g["w"]))


def _seq(x, g, b, h, sl=slice(None)):
    return tuple(x.f64(n)[b, sl, h] for n in ("q", "k", "v")) + \
        tuple(g[n][b, sl, h].astype(np.float64) for n in ("a", "b", "w"))


CHUNK_CASES = [("f32", 64, 128, 3 * C + 17), ("bf16", 128, 128, 150), ("bf16", 128, 64, C), ("bf16", 64, 64, 1),
               ("f32", 128, 128, 2 * C)]


@pytest.mark.parametrize("parts", ["out", "map", "both"])
@pytest.mark.parametrize("case", CHUNK_CASES, ids=[f"{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}" for c in CHUNK_CASES])
def test_gdn2_chunk_backward(case, parts):
    dtype, dk, dv, T = case
    note(f"gdn2 chunk backward {case} {parts}")
    B, H = 2, 2
    N = -(-T // C)
    x, g, q, k, v, gates = _gen(dtype, B, T, H, dk, dv, seed=141)
    want_out, want_map = parts in ("out", "both"), parts in ("map", "both")
    init = inputs.gen_cotangent((B, H, N, dk, dv), seed=142, name="S0", scale=0.5) if want_out else None
    dO = inputs.gen_cotangent((B, T, H, dv), seed=143, name="dO") if want_out else None
    dAt = inputs.gen_cotangent((B, H, N, dk, dk), seed=144, name="At") if want_map else None
    dBc = inputs.gen_cotangent((B, H, N, dk, dv), seed=145, name="Bc") if want_map else None
    r = hla().gdn2_chunk_backward(q, k, v, *gates, chunk_init=None if init is None else f32(init),
                                  dO=None if dO is None else f32(dO), dAt=None if dAt is None else f32(dAt),
                                  dBc=None if dBc is None else f32(dBc))
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "da", "db", "dw")
    for b in range(B):
        for hh in range(H):
            qq, kk, vv, aa, bb, ww = _seq(x, g, b, hh)
            ref = {n: 0.0 for n in names}
            if want_out:
                ro = oracle.gdn2_chunk_outputs_backward(qq, kk, vv, aa, bb, ww, C,
                                                        init[b, hh].astype(np.float64).transpose(0, 2, 1),
                                                        dO[b, :, hh].astype(np.float64))
                for n in names:
                    ref[n] = ref[n] + ro[n]
                assert_close(host(r["dchunk_init"])[b, hh], ro["dS_routed"].transpose(0, 2, 1), dtype, "dchunk_init")
            if want_map:
                rm = oracle.gdn2_chunk_transitions_backward(kk, vv, aa, bb, ww, C,
                                                            dAt[b, hh].astype(np.float64).transpose(0, 2, 1),
                                                            dBc[b, hh].astype(np.float64).transpose(0, 2, 1))
                for n in names[1:]:
                    ref[n] = ref[n] + rm[n]
            if want_out:
                assert_close(host(r["dq"])[b, :, hh], ref["dq"], dtype, "dq")
            else:
                assert np.all(host(r["dq"])[b, :, hh] == 0.0)
            for n in names[1:]:
                assert_close(host(r[n])[b, :, hh], ref[n], dtype, f"{n} b{b} h{hh}")


def test_gdn2_chunk_backward_workload_decay():
    """The workloads' fast decay (a near exp(-softplus(x + 2))): per-channel products far
    below one within a chunk."""
    dtype, dk, dv, T = "bf16", 128, 128, 2 * C + 9
    note("gdn2 chunk backward, workload decay")
    B, H = 1, 2
    N = -(-T // C)
    x, g, q, k, v, gates = _gen(dtype, B, T, H, dk, dv, seed=146, alpha_mode="config")
    init = inputs.gen_cotangent((B, H, N, dk, dv), seed=147, name="S0", scale=0.5)
    dO = inputs.gen_cotangent((B, T, H, dv), seed=148, name="dO")
    dAt = inputs.gen_cotangent((B, H, N, dk, dk), seed=149, name="At")
    dBc = inputs.gen_cotangent((B, H, N, dk, dv), seed=150, name="Bc")
    r = hla().gdn2_chunk_backward(q, k, v, *gates, chunk_init=f32(init), dO=f32(dO), dAt=f32(dAt), dBc=f32(dBc))
    torch.cuda.synchronize()
    for hh in range(H):
        qq, kk, vv, aa, bb, ww = _seq(x, g, 0, hh)
        ro = oracle.gdn2_chunk_outputs_backward(qq, kk, vv, aa, bb, ww, C, init[0, hh].astype(np.float64).transpose(0, 2, 1),
                                                dO[0, :, hh].astype(np.float64))
        rm = oracle.gdn2_chunk_transitions_backward(kk, vv, aa, bb, ww, C, dAt[0, hh].astype(np.float64).transpose(0, 2, 1),
                                                    dBc[0, hh].astype(np.float64).transpose(0, 2, 1))
        assert_close(host(r["dq"])[0, :, hh], ro["dq"], dtype, "dq")
        for n in ("dk", "dv", "da", "db", "dw"):
            assert_close(host(r[n])[0, :, hh], ro[n] + rm[n], dtype, n)


PREFILL_CASES = [("f32", 64, 128, 4 * C + 9), ("bf16", 128, 128, 5 * C - 3), ("bf16", 64, 64, 3 * C)]


@pytest.mark.parametrize("gates", ["computed", "caller"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}" for c in PREFILL_CASES])
def test_gdn2_prefill_backward(case, gates):
    """The whole Gated DeltaNet-2 routed-prefill backward against the one-graph oracle."""
    dtype, dk, dv, T = case
    note(f"gdn2 prefill backward {case} {gates}")
    B, H = 1, 2
    N = -(-T // C)
    x, g, q, k, v, gd = _gen(dtype, B, T, H, dk, dv, seed=151)
    S0 = inputs.gen_state(B, H, dk, dv, seed=152)
    dO = inputs.gen_cotangent((B, T, H, dv), seed=153, name="dO")
    G = inputs.gen_gates(B, H, N, seed=154, mode="uniform") if gates == "caller" else None
    tau = 0.3 if G is not None else 1e-3
    r = hla().gdn2_prefill_backward(q, k, v, *gd, f32(dO), tau=tau, gates_in=None if G is None else f32(G),
                                    S0=f32(S0))
    torch.cuda.synchronize()
    skipped = 0
    hist = np.tril(np.ones((N, N), bool), -1)
    for hh in range(H):
        ref = oracle.gdn2_hla_prefill_backward(*_seq(x, g, 0, hh), C, tau, dO[0, :, hh].astype(np.float64),
                                               S0=S0[0, hh].astype(np.float64).T,
                                               gates_in=None if G is None else G[0, hh].astype(np.float64))
        for n in ("dq", "dk", "dv", "da", "db", "dw"):
            assert_close(host(r[n])[0, :, hh], ref[n], dtype, f"{n} h{hh}")
        assert_close(host(r["dS0"])[0, hh], ref["dS0"].T, dtype, "dS0")
        dgg = host(r["dgates"])[0, hh]
        assert_close(dgg, ref["dgates"], dtype, "dgates")
        assert np.all(dgg[~ref["mask"]] == 0.0)
        skipped += int(hist.sum() - ref["mask"][hist].sum())
    if gates == "caller":
        assert skipped > 0


def test_gdn2_prefill_backward_segments_and_window():
    """B = 2 inputs that are a token window of a longer allocation (ld_T > T), the smallest
    workspace (history segments replayed from checkpoints): against one pass (bf16 bar) and
    against the oracle."""
    dtype, dk, dv, H, T, ld = "bf16", 128, 64, 2, 7 * C - 11, 7 * C + 40
    note("gdn2 prefill backward, segments and token window")
    x, g, qf, kf, vf, gf = _gen(dtype, 2, ld, H, dk, dv, seed=161)
    off = 25
    sl = slice(off, off + T)
    q, k, v = (t[:, sl] for t in (qf, kf, vf))
    gd = tuple(t[:, sl] for t in gf)
    dO = inputs.gen_cotangent((2, T, H, dv), seed=162, name="dO")
    h = hla()
    d = h.make_dims(2, T, H, ld, dk, dv, 1, C)
    full, mn = h.workspace_bytes(h.FN_GDN2_PREFILL_BACKWARD, d), h.workspace_bytes(h.FN_GDN2_PREFILL_BACKWARD_MIN, d)
    assert mn < full
    one = h.gdn2_prefill_backward(q, k, v, *gd, f32(dO), tau=1e-3)
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    seg = h.gdn2_prefill_backward(q, k, v, *gd, f32(dO), tau=1e-3, ws=ws)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "da", "db", "dw", "dS0", "dgates")
    for n in names:
        assert_close(host(seg[n]), host(one[n]), dtype, f"{n} (segments vs one pass)")
    for b in range(2):
        hh = b  # one head per batch row
        ref = oracle.gdn2_hla_prefill_backward(*_seq(x, g, b, hh, sl), C, 1e-3, dO[b, :, hh].astype(np.float64))
        for n in ("dq", "dk", "dv", "da", "db", "dw"):
            assert_close(host(seg[n])[b, :, hh], ref[n], dtype, f"{n} b{b}")
        assert_close(host(seg["dgates"])[b, hh], ref["dgates"], dtype, "dgates")
        assert_close(host(seg["dS0"])[b, hh], ref["dS0"].T, dtype, "dS0")


def test_gdn2_backward_collapses_to_gated_deltanet():
    """Scalar gates (a = alpha, b = w = beta on every channel): the Gated DeltaNet-2
    backward agrees with the Gated DeltaNet backward (its own kernels) on dq, dk, dv, dS0
    and dgates, and its channel sums give dalpha and dbeta."""
    dtype, dk, dv, B, H, T = "f32", 64, 128, 1, 2, 3 * C + 5
    note("gdn2 backward, collapse to gated deltanet")
    x = inputs.gen_tokens(B, T, H, dk, dv, dtype=dtype, seed=171, alpha_mode="slow")
    q, k, v = (dev(getattr(x, n), dtype) for n in ("q", "k", "v"))
    beta, alpha = f32(x.beta), f32(x.alpha)
    a = alpha[..., None].expand(B, T, H, dk).contiguous()
    bg = beta[..., None].expand(B, T, H, dk).contiguous()
    w = beta[..., None].expand(B, T, H, dv).contiguous()
    dO = f32(inputs.gen_cotangent((B, T, H, dv), seed=172, name="dO"))
    S0 = f32(inputs.gen_state(B, H, dk, dv, seed=173))
    h = hla()
    g2 = h.gdn2_prefill_backward(q, k, v, a, bg, w, dO, tau=1e-3, S0=S0)
    g1 = h.prefill_backward(q, k, v, beta, alpha, dO, tau=1e-3, S0=S0)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dS0", "dgates"):
        assert_close(host(g2[n]), host(g1[n]), dtype, n)
    assert_close(host(g2["da"]).sum(-1), host(g1["dalpha"]), dtype, "dalpha")
    assert_close(host(g2["db"]).sum(-1) + host(g2["dw"]).sum(-1), host(g1["dbeta"]), dtype, "dbeta")
