/*
 * hla.h -- C ABI of libhla.so: the Gated DeltaNet + HLA hot path on MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [HLA]  "HLA: Expressive Hybrid Linear Attention via Chunk-Wise Dynamic Mixing"
 *          (ai.info AI-summary page): Overview, Key Contributions, Methodology in Plain
 *          English paragraphs 1-4, Authors' abstract.
 *   [TR]   Tail-Replay abstract (second abstract on the thelatestinai.com page listed
 *          under the same HLA title).
 *   The per-token update is the gated delta rule of Gated DeltaNet, the affine update
 *   [HLA] Methodology paragraph 1 describes in words:
 *       S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
 *
 * Orientation and layouts (all tensors dense, row-major, no hidden padding):
 *   - The math state S is [dv, dk]; the library stores M = S^T as [dk, dv] float32.
 *   - A chunk's exact affine map ([HLA] Methodology paragraph 1) S -> S A_c + B_c is
 *     stored in the state orientation as the pair (At, Bc) with
 *         M_end = At @ M_start + Bc,   At = A_c^T [dk, dk],   Bc = B_c^T [dk, dv].
 *   - Per-token inputs: q, k [B, ld_T, H, dk]; v [B, ld_T, H, dv]; beta, alpha
 *     [B, ld_T, H] float32, with beta in [0, 1] and alpha in [0, 1] (alpha = 0 clears the
 *     state: the chunk kernels take log alpha clamped at float32's smallest normal).  Only tokens [0, T) of each batch row are read, so a suffix
 *     view (Tail-Replay) passes base pointers offset to the suffix start and ld_T = the
 *     allocated row length.
 *   - Chunk c covers tokens [c C, min((c + 1) C, T)); N = ceil(T / C); the last chunk may
 *     be partial and its transition is the product over its own tokens.
 *   - q, k, v, reps and the transitions use the call's dtype (float32 or bfloat16);
 *     states, outputs, gates and every accumulation are float32.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked "host".  Base pointers of tensors moved in
 *     16-byte vectors (q, k, v and reps of the prefill calls, transitions, states, chunk
 *     inits, caches and the workspace) must be 16-byte aligned; per-token scalars (beta,
 *     alpha), gates, counts, element-wise outputs (o) and the decode token vectors need
 *     4-byte alignment (2 bytes for bf16 decode tokens).  The caller allocates and owns
 *     every buffer, including the workspace; the library never allocates or frees device
 *     memory and keeps no pointer after return.
 *   - Calls only enqueue work on `stream`; nothing synchronises.  Calls that overlap on
 *     the same buffers race; calls on separate buffers are independent and reentrant.
 *   - Arguments are validated before anything is enqueued.  On an error the call returns a
 *     non-zero status and enqueues nothing.  A failed launch returns HLA_ERR_HIP.
 *     Asynchronous device faults surface at the caller's next synchronisation.
 *   - Every output element is overwritten, so results never depend on prior contents.
 */
#ifndef HLA_H_
#define HLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HLA_ABI_VERSION 7

typedef enum { HLA_F32 = 0, HLA_BF16 = 1 } hla_dtype_t;

typedef enum {
  HLA_OK = 0,
  HLA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                              */
  HLA_ERR_BAD_SHAPE = 2,    /* a size is out of range or inconsistent                  */
  HLA_ERR_BAD_DTYPE = 3,    /* dtype is not HLA_F32 / HLA_BF16                         */
  HLA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than hla_workspace_bytes() */
  HLA_ERR_HIP = 5,          /* a kernel launch failed                                  */
  HLA_ERR_UNSUPPORTED = 6,  /* a valid but unsupported combination of arguments        */
  HLA_ERR_ALIGN = 7,        /* a base pointer is not 16-byte aligned                   */
  HLA_ERR_INTERNAL = 8,     /* an unexpected host-side failure                         */
  HLA_ERR_SCRATCH_LIMIT = 9 /* a no-allocation call exceeds its fixed device scratch    */
} hla_status_t;

/* Problem sizes.  B batch rows, T tokens processed per row, H heads, ld_T >= T tokens
 * allocated per row; dk, dv in {64, 128}; C in {64, 128, 256} tokens per chunk (C > 64
 * needs dtype HLA_BF16, else HLA_ERR_UNSUPPORTED).  The kernels work on 64-token pieces;
 * a chunk of C tokens is C / 64 consecutive pieces, and its map is their composition. */
typedef struct {
  int64_t B, T, H, ld_T;
  int32_t dk, dv, C;
  int32_t dtype; /* hla_dtype_t */
} hla_dims_t;

/* Which entry point a workspace size is asked for (hla_workspace_bytes). */
typedef enum {
  HLA_FN_CHUNK_TRANSITIONS = 0,
  HLA_FN_GDN_PREFILL = 1,
  HLA_FN_ROUTE_MIX = 2,
  HLA_FN_WU_HANDOFF = 3, /* size of the optional wu buffer of hla_chunk_transitions and
                            hla_gdn_prefill: B H ceil(T / 64) 64 (dk + dv) bf16 values;
                            0 for float32, which takes no hand-off */
  HLA_FN_CHUNK_REPS = 4, /* workspace of hla_chunk_reps; n_rep = C / window */
  HLA_FN_COMPOSE_BACKWARD = 5, /* workspace of hla_compose_backward (one pass) */
  HLA_FN_PREFILL_BACKWARD = 6, /* workspace of hla_prefill_backward (one pass) */
  HLA_FN_CHUNK_BACKWARD = 7,   /* workspace of hla_chunk_backward */
  HLA_FN_COMPOSE_BACKWARD_MIN = 8, /* smallest workspace hla_compose_backward accepts */
  HLA_FN_PREFILL_BACKWARD_MIN = 9, /* smallest workspace hla_prefill_backward accepts */
  HLA_FN_GDN2_CHUNK_BACKWARD = 10, /* workspace of hla_gdn2_chunk_backward */
  HLA_FN_GDN2_PREFILL_BACKWARD = 11, /* workspace of hla_gdn2_prefill_backward (one pass) */
  HLA_FN_GDN2_PREFILL_BACKWARD_MIN = 12, /* smallest workspace hla_gdn2_prefill_backward accepts */
  HLA_FN_ROUTER_BACKWARD = 13,   /* workspace of hla_router_backward */
  HLA_FN_CHUNK_REPS_BACKWARD = 14 /* workspace of hla_chunk_reps_backward; n_rep says whether Wr
                                     is given (0: no, 1: yes) */
} hla_fn_t;

/*
 * hla_chunk_transitions -- the exact affine map of every chunk.
 * [HLA] Methodology paragraph 1 (affine maps compose, so a chunk is summarised exactly by
 * one affine map) and Key Contributions 2 (exact chunk-wise affine transitions).
 * Computed per (b, h, chunk) through the UT form of the chunk: the strictly lower matrix
 * diag(beta)(K K^T o decay) is inverted per chunk instead of running the token loop.
 *   k, v, beta, alpha : inputs as in the header notes (q is not needed).
 *   At [B, H, N, dk, dk], Bc [B, H, N, dk, dv] (out, dtype): M_end = At M_start + Bc.
 *   wu     (out, optional, bf16 only): a buffer of at least
 *           hla_workspace_bytes(HLA_FN_WU_HANDOFF) bytes (B H ceil(T / 64) 64 (dk + dv)
 *           bf16 values; the call has no size argument for it, so a smaller buffer is
 *           written past its end), or NULL.  Receives, for every 64-token piece, the
 *           UT-transformed keys and values W = X diag(beta gamma) K and U = X diag(beta) V
 *           (X the inverted strictly lower part plus identity) in the library's own
 *           fragment order, so that hla_gdn_prefill on the same inputs can take them
 *           instead of recomputing the inverse.  The layout is private to this library version.  A non-NULL wu
 *           with float32 inputs is HLA_ERR_UNSUPPORTED.
 *   ws, ws_bytes: workspace of at least hla_workspace_bytes(HLA_FN_CHUNK_TRANSITIONS)
 *           bytes (zero for C = 64; for C > 64 it holds the maps of the 64-token pieces,
 *           which are then composed C / 64 at a time: [HLA] Methodology paragraph 1).
 * Errors: HLA_ERR_NULL_ARG, HLA_ERR_BAD_SHAPE, HLA_ERR_BAD_DTYPE, HLA_ERR_ALIGN,
 *         HLA_ERR_WORKSPACE, HLA_ERR_UNSUPPORTED, HLA_ERR_HIP.
 */
hla_status_t hla_chunk_transitions(const hla_dims_t* d, const void* k, const void* v,
                                   const float* beta, const float* alpha, void* At, void* Bc,
                                   void* wu, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_gdn_prefill -- chunkwise Gated DeltaNet prefill.
 * [HLA] Methodology paragraph 1 (the per-token affine recurrence and its chunk form);
 * [TR] (state rebuild by replaying a suffix from a zero state: pass o = NULL).
 * Modes:
 *   native  (chunk_init == NULL): states run through the chunks in order starting from S0
 *           (NULL = zero state); o_t = S_t q_t; S_final = state after token T-1.
 *   routed  (chunk_init != NULL): chunk c starts from chunk_init[b, h, c] (the routed
 *           states of hla_route_mix; the current chunk has weight one, [HLA]
 *           Methodology paragraph 3); no state is carried between chunks.  S0 and S_final
 *           must be NULL.
 *   state-only (o == NULL): only S_final is produced; q may be NULL (Tail-Replay).
 *   q, k, v, beta, alpha : per-token inputs.
 *   S0         [B, H, dk, dv] float32 or NULL.
 *   chunk_init [B, H, N, dk, dv] float32 or NULL.
 *   wu         (optional, bf16 only): a buffer of hla_workspace_bytes(HLA_FN_WU_HANDOFF)
 *           bytes that hla_chunk_transitions filled from the same k, v, beta, alpha and
 *           dims, or NULL.  Given, the routed output pass reads W and U from it instead
 *           of recomputing them; results are identical.  The native bf16 prefill forms
 *           W and U inside its single pass and does not read it.
 *   o          [B, T, H, dv] float32 (out) or NULL.
 *   S_final    [B, H, dk, dv] float32 (out) or NULL.  At least one of o, S_final.
 *   ws, ws_bytes: workspace of at least hla_workspace_bytes(HLA_FN_GDN_PREFILL) bytes
 *           (none in routed mode with C = 64; in routed mode with C > 64 every chunk's
 *           64-token pieces start from states scanned from its routed state).  The
 *           native outputs do not depend on C: the prefill runs on 64-token pieces.
 * Native mode with bf16 inputs and outputs runs in two passes and never forms the chunk
 * maps (a state-only call scans the chunk maps instead): a parallel pass writes every
 * piece's UT products (-W, U^T, the log decays and (Q K^T) o decay: B H ceil(T / 64)
 * (128 (dk + dv) + 8448) bytes of the workspace), then one workgroup per (b, h, 32 state
 * columns) carries the state through the pieces in order, forming each piece's outputs
 * and next state on the way; no state goes through HBM.
 * Errors: as hla_chunk_transitions, plus HLA_ERR_WORKSPACE, HLA_ERR_UNSUPPORTED.
 */
hla_status_t hla_gdn_prefill(const hla_dims_t* d, const void* q, const void* k, const void* v,
                             const float* beta, const float* alpha, const float* S0,
                             const float* chunk_init, const void* wu, float* o, float* S_final,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_gdn2_chunk_transitions, hla_gdn2_prefill -- the same two calls for the Gated
 * DeltaNet-2 recurrence.
 * [GDN2] the Gated DeltaNet-2 abstract (thelatestinai.com pages): channel-wise decay, a
 * channel-wise erase gate on the key side and a channel-wise write gate on the value side;
 * with one scalar for both gates it is Kimi Delta Attention, and with a scalar decay too,
 * Gated DeltaNet.  The formula taken here (the pages print none): with the math state S
 * [dv, dk], each token does
 *     S' = S diag(a_t),   S = S' - (S' k_t)(b_t o k_t)^T + (w_t o v_t) k_t^T,   o_t = S q_t.
 * Each token is affine in S, so each chunk is one exact affine map and hla_route_mix
 * composes these maps exactly as it composes Gated DeltaNet's ([HLA] Methodology
 * paragraph 1).
 *   a_decay [B, ld_T, H, dk], b_erase [B, ld_T, H, dk], w_write [B, ld_T, H, dv]: float32
 *           per-token gates (4-byte aligned) in place of beta and alpha.
 *   Every other argument, output, mode, workspace size and error is as for
 *           hla_chunk_transitions and hla_gdn_prefill, which have no wu argument here (the
 *           W | U hand-off belongs to Gated DeltaNet's UT form).
 * With bf16 inputs the chunk pass runs the chunkwise WY form on the matrix cores (every
 * per-channel decay factor it forms is taken against a reference token of its 16 x 16
 * block, and log a_t is floored at -11 per token); with float32 inputs it runs each
 * 64-token piece's tokens in float32 on the vector units.
 */
hla_status_t hla_gdn2_chunk_transitions(const hla_dims_t* d, const void* k, const void* v,
                                        const float* a_decay, const float* b_erase,
                                        const float* w_write, void* At, void* Bc, void* ws,
                                        size_t ws_bytes, hipStream_t stream);
hla_status_t hla_gdn2_prefill(const hla_dims_t* d, const void* q, const void* k, const void* v,
                              const float* a_decay, const float* b_erase, const float* w_write,
                              const float* S0, const float* chunk_init, float* o, float* S_final,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_chunk_reps -- learned representatives of every chunk.
 * [HLA] Methodology paragraph 2: each chunk is cut into pooling windows of `window`
 * consecutive tokens; one-head self-attention runs inside every window over its keys
 * (scores scaled by 1/sqrt(dk), every token sees the whole window), the token outputs are
 * mean-pooled and a learned projection gives one representative per window.  The router's
 * learned query projection Wr is folded in: the output row is r' = Wr^T Wp pooled, so
 * hla_route_mix and hla_gdn_decode, which score the plain query q against r', compute
 * (Wr q) . (Wp pooled).  A window cut by the end of the sequence pools the tokens it has;
 * a window with no tokens gets a zero row.
 *   k      : [B, ld_T, H, dk] keys (dims d; dv is not used).
 *   window : 8, 16, 32 or 64 tokens (C / window representatives per chunk).
 *   Wq, Wk, Wv, Wp : [dk, dk] weights in the dims' dtype, row-major [out, in] (a row
 *           vector x maps to W x); head h's matrices start w_hstride elements after head
 *           h-1's (w_hstride = 0: one set shared by all heads; else >= dk*dk).
 *   Wr     : [dk, dk] query projection [out, in], same head stride, or NULL (identity).
 *   reps   : [B, N * (C / window), H, dk] (out, dtype): chunk j's representatives are rows
 *           [j n_rep, (j + 1) n_rep) with n_rep = C / window -- the reps argument of
 *           hla_route_mix with that n_rep and ld_R = N n_rep.
 *   ws, ws_bytes: workspace of at least hla_workspace_bytes(HLA_FN_CHUNK_REPS, d,
 *           C / window) bytes (float32 window means).
 * Errors: HLA_ERR_NULL_ARG, HLA_ERR_BAD_SHAPE (window, w_hstride), HLA_ERR_BAD_DTYPE,
 *         HLA_ERR_ALIGN (every pointer 16-byte aligned, head strides 16-byte multiples),
 *         HLA_ERR_WORKSPACE, HLA_ERR_UNSUPPORTED, HLA_ERR_HIP.
 */
hla_status_t hla_chunk_reps(const hla_dims_t* d, const void* k, int32_t window, const void* Wq,
                            const void* Wk, const void* Wv, const void* Wp, const void* Wr,
                            int64_t w_hstride, void* reps, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * hla_chunk_reps_noalloc -- hla_chunk_reps for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, kernels and results as hla_chunk_reps, without ws and ws_bytes: the
 * float32 window means live in a fixed device array of 32 MiB (HLA_REPS_SCRATCH_BYTES)
 * that the library holds on every GPU it runs on until the process ends; the call itself
 * allocates nothing.  It holds B H ceil(T / C) (C / window) dk float32 values, so at
 * dk = 128 up to 65536 (batch row, head, representative) rows.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * Errors: as hla_chunk_reps, and HLA_ERR_SCRATCH_LIMIT (returned before anything reaches
 * the GPU) when the problem needs more than the fixed array.
 */
#define HLA_REPS_SCRATCH_BYTES ((size_t)32 << 20)
hla_status_t hla_chunk_reps_noalloc(const hla_dims_t* d, const void* k, int32_t window, const void* Wq,
                                    const void* Wk, const void* Wv, const void* Wp, const void* Wr,
                                    int64_t w_hstride, void* reps, hipStream_t stream);

/*
 * hla_route_mix -- HLA router gates and the gated composition of chunk transitions.
 * [HLA] Overview (log-mean-exp pooled routing gates), Methodology paragraphs 2-4,
 * Key Contributions 3 and the abstract (effective support):
 *   qbar_i   = mean of q over query chunk i's tokens;
 *   l_ij     = log( (1/n_rep) sum_r exp(qbar_i . r / sqrt(dk)) ) over chunk j's
 *              representatives r;  g_ij = sigmoid(l_ij) for j < i (independent gates);
 *   g_ii = 1 (current chunk), g_ij = 0 for j > i (future masked);
 *   mask_ij  = (j < i) and (g_ij >= tau)   [skip below tau without renormalisation,
 *              decided in float32];  ghat = g * mask;
 *   n_eff_i  = (sum_j ghat_ij)^2 / sum_j ghat_ij^2 over j < i (0 when all are skipped);
 *   S~_i     = chronological composition over j < i with mask_ij of
 *              M -> M + ghat_ij (At_j M + Bc_j - M), starting from S0 (NULL = zero).
 *   q          per-token queries (read only when gates_in == NULL).
 *   reps       [B, ld_R, H, dk] (dtype): chunk j's representatives are rows
 *              [j n_rep, (j + 1) n_rep); rows are read for j < N - 1 only, so
 *              ld_R >= (N - 1) n_rep.  Passing k with n_rep = C, ld_R = ld_T uses the
 *              chunk's raw keys.
 *   At, Bc     [B, H, N, dk, dk] / [B, H, N, dk, dv] (dtype), from hla_chunk_transitions.
 *   gates_in   [B, H, N, N] float32 caller gates (entries j < i are read) or NULL.
 *   gates      [B, H, N, N] float32 out (full matrix, diagonal 1, upper 0).
 *   mask       [B, H, N, N] uint8 out (1 = composed).
 *   active_idx [B, H, N, N] int32 out: ascending j with mask_ij, then -1.
 *   active_cnt [B, H, N] int32 out.   n_eff [B, H, N] float32 out or NULL.
 *   S_routed   [B, H, N, dk, dv] float32 out.
 *   ws, ws_bytes: workspace of at least hla_workspace_bytes(HLA_FN_ROUTE_MIX) bytes (the
 *              query-chunk means and, for bf16, reordered copies of At - I and of Bc for
 *              the composition).
 * Errors: as hla_gdn_prefill.
 */
hla_status_t hla_route_mix(const hla_dims_t* d, const void* q, const void* reps, int32_t n_rep,
                           int64_t ld_R, const void* At, const void* Bc, const float* S0,
                           const float* gates_in, float tau, float* gates, uint8_t* mask,
                           int32_t* active_idx, int32_t* active_cnt, float* n_eff,
                           float* S_routed, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_gdn_decode -- one single-token decode step for Bs sequences x H heads.
 * [HLA] Key Contributions 3 (dynamic autoregressive decoding) with Methodology
 * paragraphs 2-4.  Per (sequence b, head h):
 *   live chunk : S_cur (= M of the tokens since the last cached chunk) and its
 *                transition At_cur are extended by this token:
 *                M <- alpha (I - beta k k^T) M + beta k v^T,  At <- alpha (I - beta k k^T) At.
 *   gates      : g_j = sigmoid(log-mean-exp_r (q . r / sqrt(dk))) over cached chunk j's
 *                representatives, using the token's own q (or gates_in);
 *                ghat_j = g_j if g_j >= tau else 0.
 *   output     : o = (S~ A_cur + B_cur) q in math orientation, where S~ composes the
 *                gated cached chunks j < n_cache[b] from zero in time order.
 *   native     : At_cur == NULL: S_cur is the full-prefix state and o = S_cur^T q.
 *   q, k [Bs, H, dk], v [Bs, H, dv] (dtype); beta, alpha [Bs, H] float32.
 *   S_cur   [Bs, H, dk, dv] float32 in/out.   At_cur [Bs, H, dk, dk] float32 in/out or NULL.
 *   At_cache [Bs, H, n_cap, dk, dk], Bc_cache [Bs, H, n_cap, dk, dv] (dtype) in/out.
 *   reps_cache [Bs, H, n_cap, n_rep, dk] (dtype); may be NULL when gates_in is given.
 *   n_cache [Bs] int32 in/out (device): cached chunks per sequence; values above n_cap
 *           are clamped to n_cap.
 *   gates_in [Bs, H, n_cap] float32 or NULL;  gates_out [Bs, H, n_cap] float32 or NULL
 *           (entries j >= n_cache[b] are written as 0).
 *   o [Bs, H, dv] float32 out.
 *   commit: 1 = after the step append (At_cur, S_cur), cast to dtype, at slot n_cache[b],
 *           reset At_cur = I, S_cur = 0 and increment n_cache[b].  A full cache
 *           (n_cache[b] == n_cap) is left unchanged.  The caller writes that chunk's
 *           representatives.
 * Errors: HLA_ERR_NULL_ARG, HLA_ERR_BAD_SHAPE, HLA_ERR_BAD_DTYPE, HLA_ERR_ALIGN, HLA_ERR_HIP.
 */
hla_status_t hla_gdn_decode(int64_t Bs, int64_t H, int32_t dk, int32_t dv, int32_t dtype,
                            const void* q, const void* k, const void* v, const float* beta,
                            const float* alpha, float* S_cur, float* At_cur, void* At_cache,
                            void* Bc_cache, const void* reps_cache, int32_t n_rep,
                            int32_t* n_cache, int32_t n_cap, const float* gates_in, float tau,
                            float* o, float* gates_out, int32_t commit, hipStream_t stream);

/*
 * hla_gdn2_decode -- hla_gdn_decode for the Gated DeltaNet-2 recurrence ([GDN2] abstract):
 * a_decay, b_erase [Bs, H, dk] and w_write [Bs, H, dv] (float32, 4-byte aligned) replace
 * beta and alpha; the live chunk takes the token as in hla_gdn2_prefill,
 *     S_cur <- S_cur diag(a) (I - k (b o k)^T) + (w o v) k^T,   A_cur likewise with no write,
 * and the gates, the routed read over the cache and commit are hla_gdn_decode's.  Every
 * other argument and error is as for hla_gdn_decode.
 */
hla_status_t hla_gdn2_decode(int64_t Bs, int64_t H, int32_t dk, int32_t dv, int32_t dtype,
                             const void* q, const void* k, const void* v, const float* a_decay,
                             const float* b_erase, const float* w_write, float* S_cur,
                             float* At_cur, void* At_cache, void* Bc_cache, const void* reps_cache,
                             int32_t n_rep, int32_t* n_cache, int32_t n_cap, const float* gates_in,
                             float tau, float* o, float* gates_out, int32_t commit,
                             hipStream_t stream);

/*
 * hla_compose_backward -- reverse of the gated composition of hla_route_mix.
 * [HLA] Methodology paragraphs 1, 3 and 4.  Query chunk i's routed state is the chain
 *     M_j = M_{j-1} + g_ij (At_j - I) M_{j-1} + g_ij Bc_j    over active j < i, M = S0 first,
 * and given lambda = dL/dS~_i (stored orientation) the reverse of every step is
 *     dBc_j += g lambda_j,  dAt_j += g lambda_j M_{j-1}^T,
 *     dg_ij = <lambda_j, (At_j - I) M_{j-1} + Bc_j>,  lambda_{j-1} = lambda_j + g (At_j - I)^T lambda_j.
 * Skipped pairs (mask 0) pass lambda unchanged and get dg = 0 (the skip is a step function
 * of g with zero derivative).
 *   At, Bc     [B, H, N, dk, dk] / [B, H, N, dk, dv] (dtype), as given to hla_route_mix.
 *   gates, mask [B, H, N, N] float32 / uint8, as hla_route_mix wrote them (entries j < i
 *              are read).
 *   S0         [B, H, dk, dv] float32 or NULL (zero).
 *   dS_routed  [B, H, N, dk, dv] float32: upstream gradient of S_routed.
 *   dAt, dBc   out [B, H, N, dk, dk] / [B, H, N, dk, dv] float32.
 *   dgates     out [B, H, N, N] float32: dL/dg_ij for active j < i, 0 elsewhere.
 *   dS0        out [B, H, dk, dv] float32, or NULL.
 *   S_routed   out [B, H, N, dk, dv] float32 (the routed states, recomputed), or NULL.
 *   ws, ws_bytes: workspace: (At - I), its transpose and Bc reordered for the matrix
 *              cores, and slots for the state in front of an active step, (At_j - I) M
 *              + Bc_j and g lambda (dtype, dk x dv each) of the pairs whose step j lies in
 *              one segment of K consecutive history steps, plus float32 checkpoints of
 *              every chain's state at each segment boundary it crosses.  The call takes
 *              the longest segments the workspace holds and runs them last to first, each
 *              chain's steps of a segment replayed from its checkpoint.  With
 *              hla_workspace_bytes(HLA_FN_COMPOSE_BACKWARD) bytes K = N: one segment,
 *              every pair j < i has its slots (N (N - 1) / 2 per (b, h), so it grows as
 *              N^2) and there is no checkpoint.  Any size down to
 *              hla_workspace_bytes(HLA_FN_COMPOSE_BACKWARD_MIN) (the segment length that
 *              needs least, about K (N - 1) slots and N^2 / (2 K) checkpoints per (b, h))
 *              works too.  float32 maps: the checkpoints come from the call's own replay
 *              and results are bit-identical to one segment's; bf16 maps: they come from
 *              the bf16 composition of hla_route_mix (several chains share each staged
 *              map), whose rounding differs, and results agree to bf16 rounding.
 * Computation: bf16 (or float32) matrix-core products with float32 accumulation; sums in a
 * fixed order (deterministic).
 * Errors: HLA_ERR_NULL_ARG, HLA_ERR_BAD_SHAPE, HLA_ERR_BAD_DTYPE, HLA_ERR_ALIGN,
 * HLA_ERR_WORKSPACE, HLA_ERR_HIP.
 */
hla_status_t hla_compose_backward(const hla_dims_t* d, const void* At, const void* Bc,
                                  const float* gates, const uint8_t* mask, const float* S0,
                                  const float* dS_routed, float* dAt, float* dBc, float* dgates,
                                  float* dS0, float* S_routed, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * hla_chunk_backward -- reverse of the per-chunk work (64-token chunks, C = 64):
 *   outputs part: the routed outputs of hla_gdn_prefill with chunk_init (every chunk's
 *     tokens run by the gated delta rule from its own start state, o_t = S_t q_t);
 *   map part: the chunk maps (At, Bc) of hla_chunk_transitions ([HLA] Methodology
 *     paragraph 1: the product of the per-token linear parts, and the state from zero).
 * Every state column follows x <- alpha (x - beta k (k . x)) + beta k u on its own; the
 * reverse of one token with dx = dL/dx after it is b = k . dx, dv[col] += beta b,
 * dbeta += b (u - alpha k . x_prev), dalpha += dx . x_prev - beta (k . x_prev) b,
 * dk += beta u dx - alpha beta ((k . x_prev) dx + b x_prev), dx <- alpha (dx - beta k b).
 *   q, k, v, beta, alpha: as for hla_gdn_prefill (q is read by the outputs part only).
 *   chunk_init [B, H, N, dk, dv] float32 and dO [B, T, H, dv] float32: both or neither
 *              (outputs part).
 *   dAt [B, H, N, dk, dk], dBc [B, H, N, dk, dv] float32: both or neither (map part).
 *   dq, dk [B, T, H, dk], dv [B, T, H, dv], dbeta, dalpha [B, T, H]: float32 outputs, the
 *              sum of both parts (dq is zero without the outputs part).
 *   dchunk_init [B, H, N, dk, dv] float32 out (required with the outputs part).
 *   ws, ws_bytes: workspace of at least hla_workspace_bytes(HLA_FN_CHUNK_BACKWARD) bytes
 *              (per-workgroup partial sums).
 * Arithmetic is float32 throughout; partial sums are added in a fixed order.
 * Errors: HLA_ERR_NULL_ARG (no part, or a missing output), HLA_ERR_UNSUPPORTED (C != 64),
 * and as hla_gdn_prefill.
 */
hla_status_t hla_chunk_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                const float* beta, const float* alpha, const float* chunk_init,
                                const float* dO, const float* dAt, const float* dBc, float* dq,
                                float* dk, float* dv, float* dbeta, float* dalpha,
                                float* dchunk_init, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_prefill_backward -- gradients of the routed prefill (raw-key representatives, C = 64).
 * Given dO = dL/do for the outputs of hla_chunk_transitions + hla_route_mix (reps = k,
 * n_rep = 64) + hla_gdn_prefill with chunk_init = S_routed, the call recomputes that
 * forward and returns dL/d(q, k, v, beta, alpha), dL/dS0 and dL/dg for the history gates:
 *   the outputs part of hla_chunk_backward (dS~ and the chunk-local gradients);
 *   hla_compose_backward (dAt, dBc, dgates, dS0);
 *   the maps part of hla_chunk_backward;
 *   the router ([HLA] Overview, Methodology paragraph 2): dl_ij = dg_ij g_ij (1 - g_ij),
 *     p_ijr = softmax over chunk j's keys of qbar_i . k_r / sqrt(dk),
 *     dqbar_i = sum_j dl_ij sum_r p_ijr k_r / sqrt(dk) (spread as dqbar_i / n_i over chunk
 *     i's tokens), dk_r += sum_i dl_ij p_ijr qbar_i / sqrt(dk);
 * then the per-token sums.  The skip mask is a step function of g: a skipped pair passes
 * no gradient.  With gates_in the gates are the caller's: dgates is the gradient w.r.t.
 * them and the router takes no part.
 *   q, k, v, beta, alpha, S0, gates_in, tau: as for the forward calls.
 *   dO [B, T, H, dv] float32.
 *   dq, dk [B, T, H, dk], dv [B, T, H, dv], dbeta, dalpha [B, T, H]: float32 out.
 *   dS0 [B, H, dk, dv] float32 out or NULL;  dgates [B, H, N, N] float32 out or NULL.
 *   ws, ws_bytes: workspace; it holds the composition backward's per-pair states.  With
 *              hla_workspace_bytes(HLA_FN_PREFILL_BACKWARD) bytes (growing as N^2 dk dv
 *              per (b, h)) every chunk pair has its slots; any size down to
 *              hla_workspace_bytes(HLA_FN_PREFILL_BACKWARD_MIN) runs the composition's
 *              history steps in segments replayed from checkpoints, as for
 *              hla_compose_backward.
 * Errors: HLA_ERR_UNSUPPORTED (C != 64) and as hla_gdn_prefill.
 */
hla_status_t hla_prefill_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                  const float* beta, const float* alpha, const float* S0,
                                  const float* gates_in, float tau, const float* dO, float* dq,
                                  float* dk, float* dv, float* dbeta, float* dalpha, float* dS0,
                                  float* dgates, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_gdn2_chunk_backward, hla_gdn2_prefill_backward -- hla_chunk_backward and
 * hla_prefill_backward for the Gated DeltaNet-2 recurrence (the formula of
 * hla_gdn2_chunk_transitions: S' = S diag(a_t), S = S' - (S' k_t)(b_t o k_t)^T +
 * (w_t o v_t) k_t^T, o_t = S q_t; [GDN2] the Gated DeltaNet-2 abstract).  The per-token
 * gates a_decay, b_erase [B, ld_T, H, dk] and w_write [B, ld_T, H, dv] (float32) take the
 * place of alpha and beta, and their gradients da, db [B, T, H, dk] and dw [B, T, H, dv]
 * (float32 out) the place of dalpha and dbeta.  The reverse of a chunk runs token by token
 * per state column in float32, from the state in front of every 8-token block: per token
 *     du = k . dx,  dp = -(b o k) . dx,  dv[col] += w[col] du,  dw[col] += v[col] du,
 *     dk += dx o (u - b p) + dp x',  db += -p k o dx,  dx' = dx + dp k,  da += dx' o x,
 *     dx <- a o dx'
 * (x the column before the token, x' = a o x, p = k . x', u = w[col] v[col]).  The
 * routed prefill's router, composition and their reverses are those of
 * hla_prefill_backward, unchanged.  Every other argument, output, mode, workspace rule
 * (HLA_FN_GDN2_CHUNK_BACKWARD, HLA_FN_GDN2_PREFILL_BACKWARD, down to
 * HLA_FN_GDN2_PREFILL_BACKWARD_MIN with history segments) and error is as for the Gated
 * DeltaNet calls.
 */
hla_status_t hla_gdn2_chunk_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                     const float* a_decay, const float* b_erase, const float* w_write,
                                     const float* chunk_init, const float* dO, const float* dAt,
                                     const float* dBc, float* dq, float* dk, float* dv, float* da,
                                     float* db, float* dw, float* dchunk_init, void* ws,
                                     size_t ws_bytes, hipStream_t stream);
hla_status_t hla_gdn2_prefill_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                       const float* a_decay, const float* b_erase,
                                       const float* w_write, const float* S0, const float* gates_in,
                                       float tau, const float* dO, float* dq, float* dk, float* dv,
                                       float* da, float* db, float* dw, float* dS0, float* dgates,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_router_backward -- gradients of the history gates to the queries and to the
 * representatives (learned ones, or the raw keys), for callers that compose the learned-
 * representative backward themselves: hla_prefill_backward with the forward's gates as
 * gates_in returns dgates; this call takes them on to dq and dreps, and
 * hla_chunk_reps_backward takes dreps on to the keys and the pooler's weights.
 * [HLA] Overview, Methodology paragraph 2: with qbar_i the mean of q over chunk i,
 * s_ijr = qbar_i . r_{j n_rep + r} / sqrt(dk), g_ij = sigmoid(log-mean-exp_r s_ijr):
 *     dl_ij = dg_ij g_ij (1 - g_ij),  p_ijr = softmax_r s_ijr,
 *     dq_t = (1 / n_i) sum_{j<i} dl_ij sum_r p_ijr r_{j n_rep + r} / sqrt(dk)  (t in chunk i),
 *     dr_{j n_rep + r} = sum_{i>j} dl_ij p_ijr qbar_i / sqrt(dk).
 *   d      : dims (C = 64).
 *   q      : [B, ld_T, H, dk] (dtype);  reps: [B, ld_R, H, dk] (dtype), chunk j's rows
 *           [j n_rep, (j + 1) n_rep), 1 <= n_rep <= 64, ld_R >= (N - 1) n_rep.
 *   gates, dgates : [B, H, N, N] float32: the gates hla_route_mix wrote and their gradient
 *           (entries j < i are read; a skipped pair's gradient is zero).
 *   dq     : [B, T, H, dk] float32 out (the router's part of the query gradient).
 *   dreps  : [B, N n_rep, H, dk] float32 out (the last chunk's rows are zero).
 *   ws, ws_bytes : hla_workspace_bytes(HLA_FN_ROUTER_BACKWARD) bytes.
 * Errors: HLA_ERR_NULL_ARG, HLA_ERR_BAD_SHAPE (n_rep, ld_R), HLA_ERR_ALIGN (q, reps, ws
 *         16 bytes; the float32 arrays 4), HLA_ERR_WORKSPACE, HLA_ERR_UNSUPPORTED (C != 64),
 *         HLA_ERR_HIP.
 */
hla_status_t hla_router_backward(const hla_dims_t* d, const void* q, const void* reps, int32_t n_rep,
                                 int64_t ld_R, const float* gates, const float* dgates, float* dq,
                                 float* dreps, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hla_chunk_reps_backward -- reverse of hla_chunk_reps: from dreps, the gradient of every
 * representative row, the gradients of the keys and of the weights.
 * [HLA] Methodology paragraph 2 (the forward of hla_chunk_reps).  Per window of n >= 1
 * tokens X, with P the window's attention, c_s its column sums, m = (1/n) sum_s c_s V_s
 * and z = Wp m:
 *     dz = Wr dr (dr without Wr),  dWr += z dr^T,  dm = Wp^T dz,  dWp += dz m^T,
 *     dV_s = c_s dm / n,  e_s = V_s . dm / n,  dS_ts = P_ts (e_s - sum_s' P_ts' e_s'),
 *     dQ = dS K / sqrt(dk),  dK = dS^T Q / sqrt(dk),
 *     dX = dQ Wq + dK Wk + dV Wv,  dWq += dQ^T X,  dWk += dK^T X,  dWv += dV^T X;
 * an empty window passes nothing.  The weight gradients sum over every window of every
 * batch row (and head, with shared weights) in a fixed order.
 *   k, window, Wq, Wk, Wv, Wp, Wr, w_hstride : as for hla_chunk_reps (C a multiple of 64).
 *   dreps  : [B, N (C / window), H, dk] float32, rows as hla_chunk_reps writes them.
 *   dk     : [B, T, H, dk] float32 out.
 *   dWq, dWk, dWv, dWp : [Hw, dk, dk] float32 out, Hw = H (w_hstride != 0) or 1 (shared),
 *           each head's matrix dk * dk elements after the previous one.
 *   dWr    : same, out; required exactly when Wr is given.
 *   ws, ws_bytes : hla_workspace_bytes(HLA_FN_CHUNK_REPS_BACKWARD, d, Wr ? 1 : 0) bytes
 *           (dWq, dWk and dWv of every 8 consecutive 64-token tiles, and four dk-vectors per
 *           window).
 * Errors: as hla_chunk_reps, and HLA_ERR_UNSUPPORTED (C not a multiple of 64).
 */
hla_status_t hla_chunk_reps_backward(const hla_dims_t* d, const void* k, int32_t window, const void* Wq,
                                     const void* Wk, const void* Wv, const void* Wp, const void* Wr,
                                     int64_t w_hstride, const float* dreps, float* dk, float* dWq,
                                     float* dWk, float* dWv, float* dWp, float* dWr, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* Workspace bytes that entry point `fn` needs for dims `d`; n_rep is the number of
 * representatives per chunk for HLA_FN_CHUNK_REPS (C / window; it must divide C), whether
 * Wr is given (0 or 1) for HLA_FN_CHUNK_REPS_BACKWARD, and ignored otherwise.  `out` is a
 * host pointer. */
hla_status_t hla_workspace_bytes(int32_t fn, const hla_dims_t* d, int32_t n_rep, size_t* out);

/* Kernel kinds that hla_timing_read() reports. */
typedef enum {
  HLA_KERNEL_CHUNK = 0,    /* per-chunk UT kernel (transitions, chunk outputs)        */
  HLA_KERNEL_SCAN = 1,     /* sequential chunk scan of the native prefill             */
  HLA_KERNEL_GATES = 2,    /* router: query-chunk means, gate scores, mask and lists  */
  HLA_KERNEL_COMPOSE = 3,  /* gated composition of chunk transitions                  */
  HLA_KERNEL_DECODE = 4,   /* single-token decode step                                */
  HLA_KERNEL_REPS = 5,     /* learned representatives: window attention and mean-pool */
  HLA_KERNEL_BWD_SAVE = 6,    /* backward: composition replay that keeps the step states */
  HLA_KERNEL_BWD_ADJOINT = 7, /* backward: adjoint sweep of every composition chain     */
  HLA_KERNEL_BWD_REDUCE = 8,  /* backward: per-history-chunk sums (dAt, dBc, gates, dS0)  */
  HLA_KERNEL_BWD_CHUNK = 9,   /* backward: per-chunk reverse token recurrence            */
  HLA_KERNEL_BWD_ROUTER = 10, /* backward: router gates to queries and keys              */
  HLA_KERNEL_PREFILL = 11,    /* one-pass native prefill (bf16): UT, outputs, state scan */
  HLA_KERNEL_BWD_REPS = 12,   /* backward: learned representatives (tiles and reduction)  */
  HLA_KERNEL_COUNT = 13
} hla_kernel_t;

/*
 * Optional per-kernel timing (profiling aid; off by default).  hla_timing_enable(1) clears
 * earlier records and starts bracketing every launch of the kernels above with two HIP
 * events recorded on that launch's own stream; hla_timing_enable(0) stops and clears.
 * hla_timing_read() waits for the recorded events of one kernel kind and returns the
 * summed elapsed milliseconds and the number of launches (host pointers).  These two
 * calls are the one exception to the no-global-state convention above: the switch and the
 * event records are process-global (host memory and HIP events, never device buffers), so
 * enable timing only while one thread issues work.  With timing off no entry point reads
 * or writes that state.
 */
hla_status_t hla_timing_enable(int32_t on);
hla_status_t hla_timing_read(int32_t which, double* total_ms, int64_t* launches);

/* Static description of a status code (never NULL). */
const char* hla_status_string(int32_t status);

/* HLA_ABI_VERSION of the loaded library. */
int32_t hla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H_ */
