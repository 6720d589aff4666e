"""The W | U hand-off from hla_chunk_transitions to hla_gdn_prefill (bf16), through the C ABI.

The transitions pass stores every 64-token piece's W = X diag(beta gamma) K and
U = X diag(beta) V in the bf16 operand form the output pass multiplies with, so an output
pass that reads them computes exactly what one that rebuilds them computes: outputs must
be bit-identical with and without the buffer, and match the oracle to the bf16 bar."""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_deltanet_hybrid_amd import inputs
from gpu_util import assert_close, host, note, token_tensors

pytestmark = pytest.mark.gpu


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


@pytest.mark.parametrize("C,dk,dv,T", [(64, 128, 128, 9 * 64 - 21), (64, 64, 128, 5 * 64), (256, 128, 64, 3 * 256 - 77)])
def test_routed_outputs_identical_with_handoff(C, dk, dv, T):
    note(f"hand-off routed C={C} dk={dk} dv={dv} T={T}")
    h = hla()
    x = inputs.gen_tokens(2, T, 2, dk, dv, dtype="bf16", seed=61, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    ref = h.hla_prefill(q, k, v, beta, alpha, tau=1e-3, C=C, handoff=False)
    got = h.hla_prefill(q, k, v, beta, alpha, tau=1e-3, C=C, handoff=True)
    torch.cuda.synchronize()
    assert torch.equal(ref["At"], got["At"]) and torch.equal(ref["Bc"], got["Bc"])
    assert torch.equal(ref["S_routed"], got["S_routed"])
    assert torch.equal(ref["o"], got["o"])
    for b in range(2):
        for hh in range(2):
            args = (x.f64(n)[b, :, hh] for n in ("q", "k", "v", "beta", "alpha"))
            r = oracle.hla_prefill(*args, C, 1e-3)
            assert_close(host(got["o"])[b, :, hh], r["o"], "bf16", f"routed o b{b} h{hh}")


def test_native_prefill_takes_caller_handoff():
    # native mode: the caller's buffer replaces the workspace copy; outputs unchanged
    T, dk, dv = 11 * 64 - 5, 128, 128
    note(f"hand-off native T={T}")
    h = hla()
    x = inputs.gen_tokens(1, T, 3, dk, dv, dtype="bf16", seed=62, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    wu = h.wu_buffer(k, v, beta, alpha)
    assert wu is not None and wu.numel() == 1 * 3 * math.ceil(T / 64) * 64 * (dk + dv) * 2
    h.chunk_transitions(k, v, beta, alpha, wu=wu)
    o1, S1 = h.gdn_prefill(q, k, v, beta, alpha, wu=wu)
    o0, S0 = h.gdn_prefill(q, k, v, beta, alpha)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)


def test_float32_has_no_handoff():
    x = inputs.gen_tokens(1, 100, 1, 64, 64, dtype="f32", seed=63)
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    assert h.wu_buffer(k, v, beta, alpha) is None
    with pytest.raises(h.HlaError):
        h.chunk_transitions(k, v, beta, alpha, wu=torch.empty(1 << 20, dtype=torch.uint8, device=k.device))
