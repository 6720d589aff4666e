// Internal launchers of libhla.so (host side).  Arguments are validated by abi.cpp before
// any of these is called; every launcher only enqueues work on the given stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla {

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* alpha;
  int64_t B, T, H, ld_T;
  int32_t N;
  void* At;                // out [B,H,N,dk,dk] (dtype) when transitions are wanted
  void* Bc;                // out [B,H,N,dk,dv]
  const float* chunk_init; // [B,H,N,dk,dv] start state of every chunk (outputs wanted)
  const void* chunk_init_t;  // or (bf16) the same states as bf16 [B,H,N,dv,dk], from the scan
  int32_t lanes;           // transitions: write Bc in the scan's lane order (bf16)
  float* o;                // out [B,T,H,dv]
  // W | U of every chunk in the output pass's B-operand fragment order (bf16 only):
  // written by the transitions pass when aux_out is set, read by the output pass (which
  // then skips the UT transform) when aux_in is set.  [B,H,N, (dk+dv)/32, 4, 64 lanes, 8].
  void* aux_out;
  const void* aux_in;
  // Gated DeltaNet-2 (variant 2): per-token channel-wise decay ga [B,ld_T,H,dk], erase gate
  // gb [B,ld_T,H,dk] and write gate gw [B,ld_T,H,dv] (float32) replace beta and alpha.
  const float* ga;
  const float* gb;
  const float* gw;
  int32_t variant;  // 0: Gated DeltaNet, 2: Gated DeltaNet-2
};

// Either the transitions (want_ab) or the outputs from chunk_init (want_o).
hipError_t launch_chunk(const ChunkArgs& a, int dtype, int dk, int dv, bool want_ab, bool want_o,
                        hipStream_t s);
// Gated DeltaNet-2 chunk pass: maps (At, Bc) of every 64-token piece, or (want_o) the
// outputs from chunk_init.
hipError_t launch_gdn2_chunk(const ChunkArgs& a, int dtype, int dk, int dv, bool want_o, hipStream_t s);
// bytes of the W | U fragment image of one chunk
constexpr int64_t aux_chunk_bytes(int dk, int dv) { return (int64_t)64 * (dk + dv) * 2; }

struct ScanArgs {
  const void* At;     // [B,H,N,dk,dk]
  const void* Bc;     // [B,H,N,dk,dv]
  const float* S0;    // [B,H,dk,dv] or null
  float* states;      // out [B,H,N,dk,dv]: state at the start of every chunk, or null
  float* S_final;     // out [B,H,dk,dv] or null
  int64_t B, H;
  int32_t N;
  // Segmented forms (bf16 only): segments of `seg` consecutive chunks, NS = ceil(N / seg).
  int32_t seg;
  const float* seg_init;  // [B,H,NS,dk,dv]: start state of every segment (states are written)
  void* seg_At;           // out [B,H,NS,dk,dk] (bf16): composite map of every segment
  void* seg_Bc;           // out [B,H,NS,dk,dv] (bf16)
  // bf16 maps from the library's own transitions pass (lanes != 0): Bc in the
  // accumulator's lane order [B,H,N, dv/32, dk/32, 64, 16], and the start states written
  // to states_t as bf16 [B,H,N,dv,dk] instead of to states
  int32_t lanes;
  void* states_t;
};
// Sequential chunk scan M_{c+1} = At_c M_c + Bc_c (S0, states, S_final).
hipError_t launch_scan(const ScanArgs& a, int dtype, int dk, int dv, hipStream_t s);
// Per segment, the start state of every chunk from seg_init (states; bf16).
hipError_t launch_scan_segments(const ScanArgs& a, int dk, int dv, hipStream_t s);
// Per segment, the composite map (seg_At, seg_Bc) of its chunks (bf16).
hipError_t launch_combine_segments(const ScanArgs& a, int dk, int dv, hipStream_t s);

struct RouteArgs {
  const void* q;        // [B,ld_T,H,dk]
  const void* reps;     // [B,ld_R,H,dk]
  int32_t n_rep;
  int64_t ld_R;
  const void* At;       // [B,H,N,dk,dk]
  const void* Bc;       // [B,H,N,dk,dv]
  const float* S0;      // [B,H,dk,dv] or null
  const float* gates_in;// [B,H,N,N] or null
  float tau;
  float* gates;         // [B,H,N,N]
  uint8_t* mask;        // [B,H,N,N]
  int32_t* active_idx;  // [B,H,N,N]
  int32_t* active_cnt;  // [B,H,N]
  float* n_eff;         // [B,H,N] or null
  float* S_routed;      // [B,H,N,dk,dv]; null: gates, mask and lists only (internal use)
  int32_t C;            // tokens per chunk
  float* qbar;          // workspace [B,H,N,dk] float32
  void* At_prep;        // workspace [B,H,N,dk,dk] bf16: (At - I) reordered for the composition
  int64_t B, T, H, ld_T;
  int32_t N;
};
hipError_t launch_route(const RouteArgs& a, int dtype, int dk, int dv, hipStream_t s);
// bf16 gated composition (the routed prefill's hot loop); gates and mask must be final.
hipError_t launch_compose_bf16(const RouteArgs& a, int dk, int dv, hipStream_t s);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* alpha;
  float* S_cur;
  float* At_cur;
  void* At_cache;
  void* Bc_cache;
  const void* reps_cache;
  int32_t n_rep;
  int32_t* n_cache;
  int32_t n_cap;
  const float* gates_in;
  float tau;
  float* o;
  float* gates_out;
  int32_t commit;
  int64_t Bs, H;
  // Gated DeltaNet-2 (variant 2): ga, gb [Bs,H,dk] and gw [Bs,H,dv] replace alpha and beta
  const float* ga;
  const float* gb;
  const float* gw;
  int32_t variant;
};
hipError_t launch_decode(const DecodeArgs& a, int dtype, int dk, int dv, hipStream_t s);

struct RepsArgs {
  const void* k;          // [B,ld_T,H,dk]
  int64_t B, T, H, ld_T;
  int32_t C, window, N;   // N chunks of C tokens, C / window representatives each
  const void* Wq;         // [*, dk, dk] (out, in) in dtype; head h at + h * w_hstride
  const void* Wk;
  const void* Wv;
  const void* Wp;
  const void* Wr;         // query projection folded into the representatives, or null
  int64_t w_hstride;      // elements between the heads' weights (0: shared)
  float* pooled;          // workspace [B,H,N*C/window,dk] float32: window means
  void* reps;             // out [B,N*C/window,H,dk] (dtype)
  int32_t groups;         // set by the launcher: workgroups per (b, h) of the pooling pass
};
// Learned chunk representatives: window self-attention, mean-pool, projections.
hipError_t launch_reps(const RepsArgs& a, int dtype, int dk, hipStream_t s);

struct ComposeBwdArgs {
  const void* At;        // [B,H,N,dk,dk] (dtype)
  const void* Bc;        // [B,H,N,dk,dv]
  const float* gates;    // [B,H,N,N]
  const uint8_t* mask;   // [B,H,N,N]
  const float* S0;       // [B,H,dk,dv] or null
  const float* dS;       // [B,H,N,dk,dv] upstream gradient of the routed states
  float* dAt;            // out [B,H,N,dk,dk]
  float* dBc;            // out [B,H,N,dk,dv]
  float* dgates;         // out [B,H,N,N]
  float* dS0;            // out [B,H,dk,dv] or null
  float* S_routed;       // out [B,H,N,dk,dv] or null
  void* Ap;              // workspace [B,H,N,dk,dk] (dtype): At - I in the fragment order
  void* ApT;             // workspace [B,H,N,dk,dk] (dtype): (At - I)^T in the fragment order
  void* Bl;              // workspace [B,H,N,dk,dv] (dtype): Bc in the accumulator's lane order
  // per-pair slots of the chain group's pairs ([B,H,slots,dk,dv], dtype each):
  void* Msave;           // M_{j-1} of pair (i, j)
  void* Dsave;           // D_j of pair (i, j), lane order
  void* Lsave;           // g lambda_j of pair (i, j)
  float* dgp;            // workspace [B,H,N,N,dv/32]: per-wave gate-gradient parts
  float* lam_end;        // workspace [B,H,N,dk,dv]: final lambda of every chain
  int64_t B, H;
  int32_t N;
  // the group of chains (query chunks) i0 <= i < i1 this launch takes; its pairs fill the
  // slots of Msave, Dsave and Lsave.  accumulate: add to dAt, dBc (a group after the first)
  int32_t i0, i1, accumulate;
};
// Backward of the gated composition (see compose_bwd.hip).  `stages`: 1 the forward replay
// that keeps the step states (and writes S_routed when asked), 2 the adjoint sweep and the
// sums (dAt, dBc, dgates, dS0).
constexpr int kComposeBwdSave = 1, kComposeBwdReverse = 2;
hipError_t launch_compose_backward(const ComposeBwdArgs& a, int dtype, int dk, int dv, int stages, hipStream_t s);

struct ChunkBwdArgs {
  const void* q;            // [B,ld_T,H,dk] (dtype)
  const void* k;
  const void* v;
  const float* beta;        // [B,ld_T,H]
  const float* alpha;
  int64_t B, T, H, ld_T;
  int32_t N;                // 64-token chunks
  int32_t c0, c1;           // the chunks c0 <= c < c1 that the outputs and maps parts take
  int32_t have_out;         // reverse of the outputs from chunk_init
  int32_t have_map;         // reverse of the chunk maps
  const float* chunk_init;  // [B,H,N,dk,dv] start state of every chunk (have_out)
  const float* dO;          // [B,T,H,dv] upstream gradient of the outputs (have_out)
  const float* dAt;         // [B,H,N,dk,dk] upstream gradient of At (have_map)
  const float* dBc;         // [B,H,N,dk,dv]
  float* dchunk_init;       // out [B,H,N,dk,dv] (have_out)
  // workspace: per-workgroup partial sums
  float* part_k;            // [B,H,N,(dv + dk + dv)/32,64,dk]
  float* part_q;            // [B,H,N,dv/32,64,dk]
  float* part_s;            // [B,H,N,(dv + dk + dv)/32,64,2]: dbeta, dalpha
  float* part_v;            // [B,H,N,2,64,dv]
  // router parts added by the finalize pass, or null
  const float* dqbar;       // [B,H,N,dk] gradient of each chunk's query mean
  const float* dk_router;   // [B,T,H,dk]
  float* dq;                // out [B,T,H,dk]
  float* dk;                // out [B,T,H,dk]
  float* dv;                // out [B,T,H,dv]
  float* dbeta;             // out [B,T,H]
  float* dalpha;            // out [B,T,H]
};
// Backward of the chunk outputs and / or the chunk maps, then the per-token sums.  `stages`
// picks what is launched: 1 the outputs part, 2 the maps part, 4 the finalize pass.
constexpr int kChunkBwdOut = 1, kChunkBwdMap = 2, kChunkBwdFinalize = 4;
hipError_t launch_chunk_backward(const ChunkBwdArgs& a, int dtype, int dk, int dv, int stages, hipStream_t s);

struct RouterBwdArgs {
  const void* q;         // [B,ld_T,H,dk] (dtype)
  const void* k;         // [B,ld_T,H,dk]: the representatives (raw keys, n_rep = 64)
  const float* gates;    // [B,H,N,N]
  const float* dgates;   // [B,H,N,N] gradient of the gates (zero for skipped pairs)
  float* qbar;           // workspace [B,H,N,dk]
  float* dqbar;          // out [B,H,N,dk]
  float* dk_router;      // out [B,T,H,dk]
  int64_t B, T, H, ld_T;
  int32_t N;
};
// Backward of the router gates to the query-chunk means and the keys.
hipError_t launch_router_backward(const RouterBwdArgs& a, int dtype, int dk, hipStream_t s);

}  // namespace hla
