"""The no-allocation entry point hla_chunk_reps_noalloc against hla_chunk_reps, through the
C ABI: the same kernels on the same inputs, with the window means in the library's fixed
device array instead of a caller workspace, so the representatives must agree bit for bit.
Two calls in a row, the second on a smaller problem, so the array's leftovers from the
first call cannot leak into the second."""
import math

import numpy as np
import pytest
import torch

from gated_deltanet_hybrid_amd import inputs
from gpu_util import dev, note, token_tensors

pytestmark = pytest.mark.gpu


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_reps_noalloc_matches_workspace_call(dtype):
    h = hla()
    cases = [  # (B, T, H, dk, C, window): the second is smaller
        (2, 7 * 64 - 9, 4, 128, 64, 32),
        (1, 3 * 64 - 40, 2, 128 if dtype == "bf16" else 64, 64, 16),
    ]
    for i, (B, T, H, dk, C, window) in enumerate(cases):
        note(f"no-alloc reps {dtype} case {i}: B={B} T={T} H={H} dk={dk} window={window}")
        x = inputs.gen_tokens(B, T, H, dk, dk, dtype=dtype, seed=90 + i, with_q=False)
        _, k, _, _, _ = token_tensors(x)
        Wd = {n: dev(a, dtype) for n, a in inputs.gen_pooler_weights(H, dk, dtype=dtype, seed=91 + i).items()}
        ref = h.chunk_reps(k, Wd, window=window, C=C)
        N = math.ceil(T / C)
        out = torch.full((B, N * (C // window), H, dk), float("nan"), dtype=k.dtype, device="cuda")
        got = h.chunk_reps_noalloc(k, Wd, window=window, C=C, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        bits = torch.int16 if k.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(got.view(bits), ref.view(bits)), f"case {i}: representatives differ"
        assert not torch.isnan(got.float()).any()


def test_chunk_reps_noalloc_rejects_beyond_its_scratch():
    h = hla()
    B, T, H, dk = 8, 32768, 16, 128  # 64 MiB of window means at window 32
    k = torch.zeros((B, T, H, dk), dtype=torch.bfloat16, device="cuda")
    Wd = {n: torch.zeros((1, dk, dk), dtype=torch.bfloat16, device="cuda") for n in ("Wq", "Wk", "Wv", "Wp")}
    with pytest.raises(h.HlaError) as e:
        h.chunk_reps_noalloc(k, Wd, window=32)
    assert e.value.status == h.ERR_SCRATCH_LIMIT
