"""CPU oracle for the Gated DeltaNet + HLA hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, sequential float64 numpy that states what the hot path computes.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it; the product
path (the HIP library and its Python binding) never does, and this package imports
nothing from the product.  It shares no code with the HIP kernels: it never uses the
chunkwise UT/WY form, it builds chunk transitions token by token, and it composes gated
transitions one chunk at a time.

Sources (cited by page title and section):

* [HLA] "HLA: Expressive Hybrid Linear Attention via Chunk-Wise Dynamic Mixing", the
  ai.info AI-summary page: Overview, Key Contributions, Methodology in Plain English
  (paragraphs 1-4), Authors' abstract.
* [TR] the Tail-Replay abstract (second abstract on the thelatestinai.com page listed
  under the same HLA title).
* The per-token update is the gated delta rule of Gated DeltaNet, the affine recurrence
  that [HLA] Methodology paragraph 1 describes in words (decay and edit the old state,
  then add a key-value write).

Orientation: the math state S has shape [dv, dk] and acts on keys (o = S q).  Chunk
transitions act on the right: S_end = S_start @ A + B with A [dk, dk], B [dv, dk].

Gradients (``oracle.grad``, ``oracle.grad_gdn2`` for the Gated DeltaNet-2 recurrence and
``oracle.grad_reps`` for the learned representatives) are those of the same forward, taken
by torch.autograd on a float64 CPU restatement of it.

Parity status: every function is pinned by tests/test_oracle_pins.py (gradients by
tests/test_oracle_grad_pins.py, tests/test_oracle_grad_gdn2_pins.py and
tests/test_oracle_grad_reps_pins.py) except the readings listed in ``PARITY_UNPINNED`` (no
printed number can confirm them).
"""
from .gdn import (  # noqa: F401
    gdn_recurrent,
    chunk_bounds,
    chunk_transition,
    chunk_transitions,
    log_mean_exp,
    window_rep,
    window_reps,
    router_gates,
    routed_states,
    routed_states_by_replay,
    routed_outputs,
    hla_prefill,
    decode_step,
    tail_replay,
    tail_replay_bound_log10,
    n_eff,
    PARITY_UNPINNED,
)
from .grad import (  # noqa: F401
    routed_states_backward,
    chunk_outputs_backward,
    chunk_transitions_backward,
    router_backward,
    hla_prefill_backward,
)
from .gdn2 import (  # noqa: F401
    gdn2_recurrent,
    gdn2_chunk_transition,
    gdn2_chunk_transitions,
    gdn2_routed_outputs,
    gdn2_hla_prefill,
    gdn2_decode_step,
)
from .grad_reps import window_reps_backward  # noqa: F401
from .grad_gdn2 import (  # noqa: F401
    gdn2_chunk_outputs_backward,
    gdn2_chunk_transitions_backward,
    gdn2_hla_prefill_backward,
)
