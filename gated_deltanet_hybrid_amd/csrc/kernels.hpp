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

struct UtArgs {
  const void* q;        // [B,ld_T,H,dk] bf16 (read when o is set)
  const void* k;        // [B,ld_T,H,dk] bf16
  const void* v;        // [B,ld_T,H,dv] bf16
  const float* beta;    // [B,ld_T,H]
  const float* alpha;   // [B,ld_T,H]
  const float* S0;      // [B,H,dk,dv] or null (zero)
  float* o;             // [B,T,H,dv] or null (state only)
  float* S_final;       // [B,H,dk,dv] or null
  void* rec;            // workspace: one record of ut_record_bytes per (b, h, piece)
  int64_t B, T, H, ld_T;
  int32_t N;            // 64-token pieces
};
// One piece's record in the native prefill's workspace.  Every matrix operand of the state
// pass is stored as MFMA fragments (32 x 32 x 16 bf16): a fragment is 1 KiB, lane L's 16
// bytes at 16 L, lane L = 32 h + m holding row m and the 8 k values
// 16 ks + {4 h .. 4 h + 3, 8 + 4 h .. 8 + 4 h + 3} of its k-step ks -- the k order in which
// a 32 x 32 accumulator tile (row r of element e = 8 (r / 8) ... ) turns into a B operand
// in place.  Byte offsets:
//   -W  fragments [tt 2][ks dk/16], rows t = 32 tt + m, k = key channel;
//   K^T fragments [rt dk/32][ks 4], rows dk = 32 rt + m, k = token;
//   U   in the accumulator order of the state pass's E tiles [dv/32][tt 2][64][16] bf16;
//   gamma_t = exp(g_t) [64] then D_t = exp(g_63 - g_t) [64], float32 (1 KiB reserved);
//   Q   fragments [tt 2][ks dk/16] (outputs only);
//   P = (Q K^T) o Gamma fragments [tt 2][ks 4], rows t, k = token s (outputs only).
constexpr int64_t ut_off_kt(int dk) { return (int64_t)2 * (dk / 16) * 1024; }
constexpr int64_t ut_off_u(int dk) { return ut_off_kt(dk) + (int64_t)(dk / 32) * 4 * 1024; }
constexpr int64_t ut_off_gd(int dk, int dv) { return ut_off_u(dk) + (int64_t)(dv / 32) * 4 * 1024; }
constexpr int64_t ut_off_q(int dk, int dv) { return ut_off_gd(dk, dv) + 1024; }
constexpr int64_t ut_off_p(int dk, int dv) { return ut_off_q(dk, dv) + (int64_t)2 * (dk / 16) * 1024; }
// The record is padded to a whole number of 1 KiB blocks per state-pass wave (dv / 32), so
// that every wave copies the same number of blocks of it.
constexpr int64_t ut_record_bytes(int dk, int dv) {
  return (ut_off_p(dk, dv) + 8 * 1024 + (dv / 32) * 1024 - 1) / ((dv / 32) * 1024) * ((dv / 32) * 1024);
}
// Native bf16 prefill: the per-piece UT pass, then the state pass that carries the state
// through the pieces (prefill.hip).
hipError_t launch_prefill_native(const UtArgs& a, int dk, int dv, hipStream_t s);

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
  void* Bc_prep;        // workspace [B,H,N,dk,dv] bf16: Bc in the composition's accumulator order
  int64_t B, T, H, ld_T;
  int32_t N;
  // optional (bf16 composition): every chain's state in front of each history step b ckpt_K
  // (b >= 1) that it crosses, float32 in the accumulator's lane order, at ckpt_slot() of
  // [B,H,ckpt_nck,dk,dv] (the composition backward's checkpoints)
  float* ckpt;
  int32_t ckpt_K;
  int64_t ckpt_nck;
};
// Checkpoint slot (per (b, h)) of chain i at history-segment boundary b K (b >= 1, i > b K):
// the boundaries before b hold the chains above them, N - 1 - b' K each.
__host__ __device__ inline int64_t ckpt_slot(int32_t N, int32_t K, int b, int i) {
  const int64_t bm = b - 1;
  return bm * (N - 1) - (int64_t)K * bm * (bm + 1) / 2 + ((int64_t)i - (int64_t)b * K - 1);
}
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
// Backward of the learned representatives: from the gradient of every representative row,
// the gradient of the keys the windows pooled and of the weights.
struct RepsBwdArgs {
  const void* k;          // [B,ld_T,H,dk]
  int64_t B, T, H, ld_T;
  int32_t window;         // 8, 16, 32 or 64 (windows never cross a 64-token tile)
  const void* Wq;         // [*, dk, dk] (out, in) in dtype; head h at + h * w_hstride
  const void* Wk;
  const void* Wv;
  const void* Wp;
  const void* Wr;         // folded query projection, or null
  int64_t w_hstride;      // 0: one set shared by all heads
  const float* dreps;     // [B,R,H,dk]: row t0 / window is the window starting at token t0
  int64_t R;              // rows per batch of dreps
  float* dk;              // out [B,T,H,dk]
  float* part;            // workspace [B,H,ceil(ceil(T/64)/8),3,dk,dk]: dWq, dWk, dWv of each
                          // workgroup of the tile kernel (8 tiles of 64 tokens)
  float* wvec;            // workspace [4,B,RW,H,dk]: each window's dz, m, z and dr', row
                          // t0 / window for the window starting at token t0
  int64_t RW;             // rows per batch of wvec: ceil(T/64) 8 (the most, at window 8)
  float* part2;           // workspace: dWp (and dWr) of every chunk of 256 windows of a (b, h)
  float* dW[5];           // out [Hw,dk,dk] float32: dWq, dWk, dWv, dWp, dWr (Hw = H, or 1
                          // when shared)
};
hipError_t launch_reps_backward(const RepsBwdArgs& a, int dtype, int dk, hipStream_t s);

// Bytes of the fixed device scratch that hla_chunk_reps_noalloc keeps its window means in.
constexpr int64_t kRepsScratchBytes = (int64_t)32 << 20;
// That scratch on the current device (its address looked up once per device, then cached).
hipError_t reps_scratch(float** out);

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
  // per-pair slots of the pairs (i, j) whose step j lies in the current segment
  // ([B,H,slots,dk,dv], dtype each):
  void* Msave;           // M_{j-1} of pair (i, j)
  void* Dsave;           // D_j of pair (i, j), lane order
  void* Lsave;           // g lambda_j of pair (i, j)
  float* Ckpt;           // workspace [B,H,nck,dk,dv] float32, lane order: every chain's state in
                         // front of each segment boundary it crosses
  float* dgp;            // workspace [B,H,N,N,dv/32]: per-wave gate-gradient parts
  float* lam_end;        // workspace [B,H,N,dk,dv]: lambda of every chain, carried from one
                         // segment to the one before it (the final lambda at the end)
  int64_t B, H;
  int32_t N;
  // the history steps j are cut into segments of K ([j0, j1) the current one), run last to
  // first; slots and nck are the per-(b, h) counts of pair slots and checkpoints
  int32_t K, j0, j1;
  int64_t slots, nck;
  // the checkpoints were written by the bf16 composition (ckpt of RouteArgs), so the prep
  // stage does not replay the chains for them
  int32_t ckpt_done;
};
// Backward of the gated composition (see compose_bwd.hip), in stages the caller sequences:
//   kComposeBwdPrep     the reordered maps, and with more than one segment the checkpoint
//                       replay (which also writes S_routed when asked);
//   kComposeBwdSave     the current segment's replay that keeps its step states (and with a
//                       single segment writes S_routed when asked);
//   kComposeBwdReverse  the current segment's adjoint sweep and its steps' sums (dAt, dBc,
//                       dgates);
//   kComposeBwdFinish   dS0.
constexpr int kComposeBwdPrep = 1, kComposeBwdSave = 2, kComposeBwdReverse = 4, kComposeBwdFinish = 8;
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
  int32_t ut;               // both parts run through the UT form (one partial-sum slot per
                            // piece and part) rather than by state columns (set by the launcher)
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

// Backward of the Gated DeltaNet-2 per-chunk work: the outputs from chunk_init and the
// chunk maps, token by token per state column (channel-wise decay ga, erase gate gb and
// write gate gw in place of alpha and beta), then the per-token sums.  Stages as for
// launch_chunk_backward.
struct Gdn2BwdArgs {
  const void* q;            // [B,ld_T,H,dk] (dtype)
  const void* k;
  const void* v;            // [B,ld_T,H,dv]
  const float* ga;          // [B,ld_T,H,dk] decay
  const float* gb;          // [B,ld_T,H,dk] erase gate
  const float* gw;          // [B,ld_T,H,dv] write gate
  int64_t B, T, H, ld_T;
  int32_t N;                // 64-token chunks
  int32_t c0, c1;           // the chunks c0 <= c < c1 that the outputs and maps parts take
  int32_t have_out, have_map;
  const float* chunk_init;  // [B,H,N,dk,dv] (have_out)
  const float* dO;          // [B,T,H,dv] (have_out)
  const float* dAt;         // [B,H,N,dk,dk] (have_map)
  const float* dBc;         // [B,H,N,dk,dv]
  float* dchunk_init;       // out [B,H,N,dk,dv] (have_out)
  // workspace: per-workgroup column sums (NC = gdn2_bwd_cols(dtype) state columns per
  // workgroup)
  float* part_k;            // [B,H,N,(dv + dk + dv)/NC,64,dk]
  float* part_a;            // same
  float* part_b;            // same
  float* part_q;            // [B,H,N,dv/NC,64,dk]
  float* part_v;            // [B,H,N,2,64,dv]: outputs part, maps part
  float* part_w;            // same
  const float* dqbar;       // [B,H,N,dk] router parts added by the finalize pass, or null
  const float* dk_router;   // [B,T,H,dk]
  float* dq;                // out [B,T,H,dk]
  float* dk;                // out [B,T,H,dk]
  float* dv;                // out [B,T,H,dv]
  float* da;                // out [B,T,H,dk]
  float* db;                // out [B,T,H,dk]
  float* dw;                // out [B,T,H,dv]
};
// State columns per workgroup of the Gated DeltaNet-2 reverse: 32 for bf16 inputs (dtype 1),
// 16 for float32 ones (their keys and queries take twice the LDS).
constexpr int gdn2_bwd_cols(int dtype) { return dtype == 1 ? 32 : 16; }
hipError_t launch_gdn2_chunk_backward(const Gdn2BwdArgs& a, int dtype, int dk, int dv, int stages, hipStream_t s);

struct RouterBwdArgs {
  const void* q;         // [B,ld_T,H,dk] (dtype)
  const void* reps;      // [B,ld_R,H,dk] (dtype): chunk j's representatives are rows
                         // [j n_rep, (j + 1) n_rep) (the raw keys: n_rep = 64, ld_R = ld_T)
  const float* gates;    // [B,H,N,N]
  const float* dgates;   // [B,H,N,N] gradient of the gates (zero for skipped pairs)
  float* qbar;           // workspace [B,H,N,dk]
  float* dqbar;          // out [B,H,N,dk]
  float* dreps;          // out [B,R_out,H,dk]: gradient of every representative row below R_out
  float* dq_tok;         // out [B,T,H,dk] dqbar of each token's chunk over its token count, or null
  int64_t B, T, H, ld_T;
  int32_t N;
  int32_t n_rep;         // 1 .. 64
  int64_t ld_R, R_out;
  float* part;           // workspace of router_bwd_part_bytes: dqbar per history segment
};
// History chunks per workgroup of the router backward's query-side pass: about 1024
// workgroups over (b, h, group of 128 query chunks, segment), between 4 and 32 chunks.
__host__ __device__ inline int router_bwd_seg(int64_t BH, int64_t N) {
  const int64_t nqg = ((N + 31) / 32 + 3) / 4;
  const int64_t s = (N * BH * nqg + 1023) / 1024;
  return (int)(s < 4 ? 4 : (s > 32 ? 32 : s));
}
// Workspace bytes of the router backward's parts: dqbar per history segment.
inline int64_t router_bwd_part_bytes(int64_t B, int64_t H, int64_t N, int dk) {
  const int64_t seg = router_bwd_seg(B * H, N), njs = (N + seg - 1) / seg;
  return (njs * B * H * N * dk * 4 + 255) / 256 * 256;
}
// Backward of the router gates to the query-chunk means and the representatives.
hipError_t launch_router_backward(const RouterBwdArgs& a, int dtype, int dk, hipStream_t s);

}  // namespace hla
