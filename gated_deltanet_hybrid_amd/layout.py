"""Host-side size arithmetic for the tensors that cross the C ABI.

Layouts (row-major, element strides in brackets):
* per-token inputs q, k [B, ld_T, H, dk], v [B, ld_T, H, dv]; beta, alpha [B, ld_T, H];
* chunk transitions in state orientation: At [B, H, N, dk, dk], Bc [B, H, N, dk, dv],
  with M_end = At @ M_start + Bc for the stored state M = S^T [dk, dv];
* states [B, H, dk, dv] float32; routed states [B, H, N, dk, dv] float32.
"""
import math

DTYPE_BYTES = {"bf16": 2, "f32": 4}


def n_chunks(T: int, C: int) -> int:
    return math.ceil(T / C)


def transition_cache_bytes(n_chunks: int, dk: int, dv: int, dtype: str) -> int:
    """Bytes of the per-chunk affine summaries (At: dk x dk, Bc: dk x dv) of one head."""
    return n_chunks * (dk * dk + dk * dv) * DTYPE_BYTES[dtype]
