"""Guard bands: every output and workspace buffer handed to an entry point sits inside a
larger allocation whose bytes before and after it hold a canary pattern; after the call the
guard bands must still hold it (no kernel writes outside the buffers it was given) and the
buffer itself must be fully written (no canary left in an output).

The cases run several workgroups per kernel and a ragged last chunk; the Gated DeltaNet-2
case has more pieces than CUs, so its workgroups loop over pieces."""
import math

import pytest
import torch

from gated_deltanet_hybrid_amd import inputs
from gpu_util import dev, f32, note, token_tensors

pytestmark = pytest.mark.gpu
C = 64
G = 4096  # guard elements on each side (16 KiB or more: keeps every buffer 16-byte aligned)
CANARY_INT = {torch.int32: 0x5A5A5A5A, torch.uint8: 0xA5}


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


def _fill(t):
    t.fill_(float("nan") if t.is_floating_point() else CANARY_INT[t.dtype])
    return t


def _bits(t):
    if t.is_floating_point():
        return t.view(torch.int16 if t.element_size() == 2 else torch.int32)
    return t


class Guarded:
    """Buffers carved out of canary-filled allocations with G guard elements on each side."""

    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype, output=True):
        n = math.prod(shape)
        full = _fill(torch.empty(n + 2 * G, dtype=dtype, device="cuda"))
        view = full[G:G + n].view(shape)
        self.bufs.append((full, n, output))
        return view

    def check(self, what):
        torch.cuda.synchronize()
        for i, (full, n, output) in enumerate(self.bufs):
            ref = _bits(_fill(torch.empty(G, dtype=full.dtype, device="cuda")))
            assert torch.equal(_bits(full[:G]), ref), f"{what}: buffer {i} written below its start"
            assert torch.equal(_bits(full[G + n:]), ref), f"{what}: buffer {i} written past its end"
            if output:
                body = full[G:G + n]
                left = torch.isnan(body) if body.is_floating_point() else body == CANARY_INT[body.dtype]
                assert not left.any(), f"{what}: buffer {i} has elements left unwritten"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_routed_prefill_guards(dtype):
    B, H, T, d = 1, 8, 13 * C - 21, 128 if dtype == "bf16" else 64
    note(f"guards: routed prefill {dtype}")
    x = inputs.gen_tokens(B, T, H, d, d, dtype=dtype, seed=151, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    N = math.ceil(T / C)
    g = Guarded()
    tdt = k.dtype
    At, Bc = g((B, H, N, d, d), tdt), g((B, H, N, d, d), tdt)
    dims = h.make_dims(B, T, H, T, d, d, 1 if dtype == "bf16" else 0, C)
    ws_t = g((max(h.workspace_bytes(h.FN_CHUNK_TRANSITIONS, dims), 16),), torch.uint8, output=False)
    h.chunk_transitions(k, v, beta, alpha, At=At, Bc=Bc, ws=ws_t)
    out = dict(gates=g((B, H, N, N), torch.float32), mask=g((B, H, N, N), torch.uint8),
               active_idx=g((B, H, N, N), torch.int32), active_cnt=g((B, H, N), torch.int32),
               n_eff=g((B, H, N), torch.float32), S_routed=g((B, H, N, d, d), torch.float32))
    ws_r = g((h.workspace_bytes(h.FN_ROUTE_MIX, dims, C),), torch.uint8, output=False)
    r = h.route_mix(q, k, At, Bc, n_rep=C, tau=1e-3, out=out, ws=ws_r)
    o = g((B, T, H, d), torch.float32)
    h.gdn_prefill(q, k, v, beta, alpha, chunk_init=r["S_routed"], want_state=False, o=o)
    S = g((B, H, d, d), torch.float32)
    ws_p = g((max(h.workspace_bytes(h.FN_GDN_PREFILL, dims), 16),), torch.uint8, output=False)
    o2 = g((B, T, H, d), torch.float32)
    h.gdn_prefill(q, k, v, beta, alpha, o=o2, S_final=S, ws=ws_p)
    g.check(f"routed prefill {dtype}")


def test_gdn2_guards():
    B, H, T, d = 2, 8, 20 * C - 5, 128  # 320 pieces
    note("guards: gated deltanet-2")
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=152, alpha_mode="slow")
    q, k, v, _, _ = token_tensors(x)
    gg = inputs.gen_gdn2_gates(B, T, H, d, d, seed=153, alpha_mode="slow")
    ga, gb, gw = (f32(gg[n]) for n in ("a", "b", "w"))
    h = hla()
    N = math.ceil(T / C)
    g = Guarded()
    At, Bc = g((B, H, N, d, d), torch.bfloat16), g((B, H, N, d, d), torch.bfloat16)
    h.gdn2_chunk_transitions(k, v, ga, gb, gw, At=At, Bc=Bc)
    init = f32(0.05 * torch.randn(B, H, N, d, d, generator=torch.Generator().manual_seed(154)).numpy())
    o = g((B, T, H, d), torch.float32)
    h.gdn2_prefill(q, k, v, ga, gb, gw, chunk_init=init, want_state=False, o=o)
    g.check("gated deltanet-2 maps and routed outputs")


@pytest.mark.parametrize("window", [32, 64])
def test_chunk_reps_guards(window):
    B, H, T, d = 1, 4, 7 * C - 9, 128
    note(f"guards: learned representatives, window {window}")
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=155)
    _, k, _, _, _ = token_tensors(x)
    Wd = {n: dev(a, "bf16") for n, a in inputs.gen_pooler_weights(H, d, dtype="bf16", seed=156).items()}
    h = hla()
    N = math.ceil(T / C)
    g = Guarded()
    out = g((B, N * (C // window), H, d), torch.bfloat16)
    dims = h.make_dims(B, T, H, T, d, d, 1, C)
    ws = g((h.workspace_bytes(h.FN_CHUNK_REPS, dims, C // window),), torch.uint8, output=False)
    h.chunk_reps(k, Wd, window=window, out=out, ws=ws)
    g.check(f"learned representatives, window {window}")
