"""GPU parity at chunk sizes C = 128 and 256 (bf16), through the C ABI.

A chunk of C tokens is C / 64 pieces of 64 tokens whose maps the library composes; the
oracle builds every C-token chunk's map token by token, routes over C-token chunks and
runs each chunk's tokens from its routed state.  Bars as everywhere: max|diff| / max|ref|
<= 2e-2 for bf16 inputs with float32 accumulation; masks and active lists bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, f32, host, note, token_tensors

pytestmark = pytest.mark.gpu

CASES = [
    # C, dk, dv, T (ragged)
    (128, 128, 128, 5 * 128 - 37),
    (256, 128, 128, 4 * 256 - 100),
    (256, 64, 128, 3 * 256 - 1),
    (128, 128, 64, 6 * 128 - 64),
]
IDS = [f"C{c[0]}-dk{c[1]}-dv{c[2]}-T{c[3]}" for c in CASES]


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def seq(x, b, h):
    return x.f64("q")[b, :, h], x.f64("k")[b, :, h], x.f64("v")[b, :, h], x.f64("beta")[b, :, h], x.f64("alpha")[b, :, h]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_chunk_transitions_larger_chunks(case):
    C, dk, dv, T = case
    note(f"transitions C={C} {case}")
    x = inputs.gen_tokens(2, T, 2, dk, dv, dtype="bf16", seed=41, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    At, Bc = hla().chunk_transitions(k, v, beta, alpha, C=C)
    torch.cuda.synchronize()
    assert At.shape[2] == math.ceil(T / C)
    for b in range(2):
        for hh in range(2):
            A, Bm = oracle.chunk_transitions(*seq(x, b, hh)[1:], C)
            assert_close(host(At[b, hh]), A.transpose(0, 2, 1), "bf16", f"At b{b} h{hh}")
            assert_close(host(Bc[b, hh]), Bm.transpose(0, 2, 1), "bf16", f"Bc b{b} h{hh}")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_routed_prefill_larger_chunks(case):
    C, dk, dv, T = case
    note(f"routed C={C} {case}")
    x = inputs.gen_tokens(1, T, 2, dk, dv, dtype="bf16", seed=42, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    r = hla().hla_prefill(q, k, v, beta, alpha, tau=1e-3, C=C)
    torch.cuda.synchronize()
    N = math.ceil(T / C)
    for hh in range(2):
        ref = oracle.hla_prefill(*seq(x, 0, hh), C, 1e-3)
        np.testing.assert_allclose(host(r["gates"])[0, hh], ref["gates"], atol=2e-5, rtol=0)
        near = np.abs(ref["gates"] - 1e-3) <= 1e-6
        m = host(r["mask"])[0, hh].astype(bool)
        assert np.array_equal(m[~near], ref["mask"][~near])
        aidx, acnt = host(r["active_idx"])[0, hh].astype(int), host(r["active_cnt"])[0, hh].astype(int)
        for i in range(N):
            act = np.nonzero(m[i])[0]
            assert acnt[i] == len(act)
            np.testing.assert_array_equal(aidx[i, :len(act)], act)
        assert_close(host(r["S_routed"])[0, hh], ref["S_routed"].transpose(0, 2, 1), "bf16", "S_routed")
        assert_close(host(r["o"])[0, :, hh], ref["o"], "bf16", "routed o")


def test_route_caller_gates_larger_chunks():
    # skip-heavy caller gates over C = 256 chunks; outputs through the segmented scan
    C, dk, dv, T = 256, 128, 128, 6 * 256 - 30
    note(f"routed caller gates C={C}")
    x = inputs.gen_tokens(1, T, 2, dk, dv, dtype="bf16", seed=43, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    N = math.ceil(T / C)
    G = inputs.gen_gates(1, 2, N, seed=44, mode="uniform")
    tau = 0.4
    r = hla().hla_prefill(q, k, v, beta, alpha, tau=tau, gates_in=f32(G), C=C)
    torch.cuda.synchronize()
    for hh in range(2):
        ref = oracle.hla_prefill(*seq(x, 0, hh), C, tau, gates_in=G[0, hh].astype(np.float64))
        np.testing.assert_array_equal(host(r["mask"])[0, hh].astype(bool), ref["mask"])
        assert (~ref["mask"][np.tril_indices(N, -1)]).any()  # some pairs are skipped
        assert_close(host(r["S_routed"])[0, hh], ref["S_routed"].transpose(0, 2, 1), "bf16", "S_routed")
        assert_close(host(r["o"])[0, :, hh], ref["o"], "bf16", "routed o")


def test_native_prefill_does_not_depend_on_chunk_size():
    # the native prefill runs on 64-token pieces whatever C the dims name: identical results
    T, dk, dv = 777, 128, 128
    x = inputs.gen_tokens(2, T, 2, dk, dv, dtype="bf16", seed=45, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    o64, S64 = h.gdn_prefill(q, k, v, beta, alpha, C=64)
    o256, S256 = h.gdn_prefill(q, k, v, beta, alpha, C=256)
    torch.cuda.synchronize()
    assert torch.equal(o64, o256) and torch.equal(S64, S256)
