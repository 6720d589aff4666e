// C ABI of libhla.so: argument validation, workspace layout and dispatch.
// Every check runs before anything is enqueued, so an invalid call returns its status
// with the stream untouched (and without touching the GPU at all).
#include "../../include/hla.h"

#include <cmath>
#include <cstdint>
#include <utility>
#include <vector>

#include "kernels.hpp"

namespace {

constexpr int64_t kMaxGrid = 0x7fffffffLL;
constexpr int32_t kMaxCacheSlots = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t n_chunks(const hla_dims_t* d) { return (d->T + d->C - 1) / d->C; }
// the kernels work on 64-token pieces; a chunk of C tokens is C / 64 consecutive pieces
constexpr int32_t kPiece = 64;
int64_t n_pieces(const hla_dims_t* d) { return (d->T + kPiece - 1) / kPiece; }

int64_t dtype_bytes(int32_t dt) { return dt == HLA_BF16 ? 2 : 4; }

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

hla_status_t check_dims(const hla_dims_t* d) {
  if (!d) return HLA_ERR_NULL_ARG;
  if (d->dtype != HLA_F32 && d->dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (d->B < 1 || d->H < 1 || d->T < 1 || d->ld_T < d->T) return HLA_ERR_BAD_SHAPE;
  if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return HLA_ERR_BAD_SHAPE;
  if (d->C != 64 && d->C != 128 && d->C != 256) return HLA_ERR_BAD_SHAPE;
  if (d->C != kPiece && d->dtype != HLA_BF16) return HLA_ERR_UNSUPPORTED;
  // element counts must stay far from int64 overflow, grids within 2^31 blocks
  const double elems = (double)d->B * (double)d->ld_T * (double)d->H * 128.0;
  if (elems > 4.0e18) return HLA_ERR_BAD_SHAPE;
  const int64_t N = n_pieces(d);
  if ((double)d->B * (double)d->H * (double)N > (double)kMaxGrid) return HLA_ERR_BAD_SHAPE;
  if ((double)d->B * d->H * (double)N * (double)N > 4.0e18) return HLA_ERR_BAD_SHAPE;
  return HLA_OK;
}

// Tensors read or written in 16-byte vectors need 16-byte alignment; per-token scalars,
// gates and element-wise outputs need only 4-byte alignment.
template <class... P>
bool all_aligned(P... p) {
  return (aligned16(p) && ...);
}
template <class... P>
bool all_aligned4(P... p) {
  return (aligned4(p) && ...);
}

// Bytes of the W | U image of every 64-token piece (bf16; float32 takes no hand-off).
int64_t wu_bytes(const hla_dims_t* d) {
  return d->dtype == HLA_BF16 ? d->B * d->H * n_pieces(d) * hla::aux_chunk_bytes(d->dk, d->dv) : 0;
}

// Workspace of the prefill: transitions of the 64-token pieces (dtype), then, when outputs
// are wanted, the W | U hand-off (bf16) and the float32 state at the start of every piece.
// The native prefill uses it; a routed prefill with C > 64 uses it to run each chunk's
// pieces from its routed state.
struct PrefillWs {
  int64_t at_off, bc_off, wu_off, st_off, total_ab, total;
};
PrefillWs prefill_ws(const hla_dims_t* d) {
  const int64_t N = n_pieces(d), BHN = d->B * d->H * N, e = dtype_bytes(d->dtype);
  PrefillWs w;
  w.at_off = 0;
  w.bc_off = round_up(BHN * d->dk * d->dk * e, 256);
  w.total_ab = w.bc_off + round_up(BHN * d->dk * d->dv * e, 256);
  w.wu_off = w.total_ab;
  w.st_off = w.wu_off + round_up(wu_bytes(d), 256);
  w.total = w.st_off + round_up(BHN * d->dk * d->dv * 4, 256);
  return w;
}

// Workspace of the native bf16 Gated DeltaNet prefill: one UT record per (b, h, piece).
int64_t native_ws(const hla_dims_t* d) { return d->B * d->H * n_pieces(d) * hla::ut_record_bytes(d->dk, d->dv); }

// Workspace of hla_route_mix: float32 query-chunk means, then (bf16 only) the reordered
// copies of At - I and of Bc that the composition streams.
int64_t route_qbar_bytes(const hla_dims_t* d) { return round_up(d->B * d->H * n_chunks(d) * d->dk * 4, 256); }
int64_t route_atp_bytes(const hla_dims_t* d) {
  return d->dtype == HLA_BF16 ? round_up(d->B * d->H * n_chunks(d) * d->dk * d->dk * 2, 256) : 0;
}
int64_t route_ws(const hla_dims_t* d) {
  const int64_t bcp = d->dtype == HLA_BF16 ? round_up(d->B * d->H * n_chunks(d) * d->dk * d->dv * 2, 256) : 0;
  return route_qbar_bytes(d) + route_atp_bytes(d) + bcp;
}

// Workspace of hla_chunk_reps: float32 window means [B,H,N*n_rep,dk].
int64_t reps_ws(const hla_dims_t* d, int32_t n_rep) {
  return round_up(d->B * d->H * n_chunks(d) * n_rep * d->dk * 4, 256);
}

// Workspace of hla_router_backward: the query-chunk means, their gradients, then the
// per-segment parts of those gradients.
int64_t router_bwd_means(const hla_dims_t* d) { return round_up(d->B * d->H * n_chunks(d) * d->dk * 4, 256); }
int64_t router_bwd_ws(const hla_dims_t* d) {
  return 2 * router_bwd_means(d) + hla::router_bwd_part_bytes(d->B, d->H, n_chunks(d), d->dk);
}
// Workspace of hla_chunk_reps_backward: dWq, dWk, dWv of every workgroup of the tile kernel
// (8 consecutive 64-token tiles of a (b, h) row), then four vectors (dz, m, z, dr') per
// window, sized for the smallest window (8 per tile).
int64_t reps_bwd_rows(const hla_dims_t* d) { return (d->T + 63) / 64 * 8; }
int64_t reps_bwd_part_bytes(const hla_dims_t* d) {
  const int64_t groups = ((d->T + 63) / 64 + 7) / 8;
  return round_up(d->B * d->H * groups * 3 * (int64_t)d->dk * d->dk * 4, 256);
}
int64_t reps_bwd_vec_bytes(const hla_dims_t* d) {
  return round_up(4 * d->B * reps_bwd_rows(d) * d->H * d->dk * 4, 256);
}
// then dWp and dWr of every chunk of 256 windows of one (b, h)
int64_t reps_bwd_ws(const hla_dims_t* d, bool) {
  const int64_t chunks = d->B * d->H * ((reps_bwd_rows(d) + 255) / 256);
  return reps_bwd_part_bytes(d) + reps_bwd_vec_bytes(d) + round_up(2 * chunks * (int64_t)d->dk * d->dk * 4, 256);
}

// Workspace of hla_compose_backward with history segments of K steps: (At - I) and its
// transpose in the fragment order, Bc in the lane order, per-wave gate-gradient parts and
// every chain's lambda, the float32 checkpoints of every chain at each segment boundary it
// crosses, then per (b, h) the pair slots of the largest segment (the first: chain i holds
// min(K, i) pairs) for each of the state in front of a step, D_j and lambda (dtype).  With
// K = N there is one segment, every pair has its slot and there is no checkpoint.
struct ComposeBwdWs {
  int64_t ap_off, apt_off, bl_off, dgp_off, le_off, ck_off, ms_off, ds_off, ls_off, total;
  int32_t K;
  int64_t slots, nck;
};
int64_t pair_bytes(const hla_dims_t* d) { return d->B * d->H * d->dk * d->dv * dtype_bytes(d->dtype); }
// pair slots per (b, h) of the first segment, and checkpoints per (b, h)
int64_t seg_slots(int64_t N, int64_t K) {
  return K >= N - 1 ? N * (N - 1) / 2 : K * (K + 1) / 2 + (N - 1 - K) * K;
}
int64_t seg_ckpts(int64_t N, int64_t K) {
  int64_t n = 0;
  for (int64_t b = 1; b * K < N; ++b) n += N - 1 - b * K;
  return n;
}
ComposeBwdWs compose_bwd_ws(const hla_dims_t* d, int64_t K) {
  const int64_t N = n_chunks(d), BH = d->B * d->H, e = dtype_bytes(d->dtype);
  ComposeBwdWs w;
  w.K = (int32_t)K;
  w.slots = seg_slots(N, K);
  w.nck = seg_ckpts(N, K);
  const int64_t at = round_up(BH * N * d->dk * d->dk * e, 256), pr = round_up(w.slots * pair_bytes(d), 256);
  w.ap_off = 0;
  w.apt_off = at;
  w.bl_off = 2 * at;
  w.dgp_off = w.bl_off + round_up(BH * N * d->dk * d->dv * e, 256);
  w.le_off = w.dgp_off + round_up(BH * N * N * (d->dv / 32) * 4, 256);
  w.ck_off = w.le_off + round_up(BH * N * d->dk * d->dv * 4, 256);
  w.ms_off = w.ck_off + round_up(BH * w.nck * d->dk * d->dv * 4, 256);
  w.ds_off = w.ms_off + pr;
  w.ls_off = w.ds_off + pr;
  w.total = w.ls_off + pr;
  return w;
}
// The smallest composition workspace over the segment lengths.
int64_t compose_bwd_min(const hla_dims_t* d) {
  const int64_t N = n_chunks(d);
  int64_t best = compose_bwd_ws(d, N).total;
  for (int64_t K = 1; K < N; ++K) best = std::min(best, compose_bwd_ws(d, K).total);
  return best;
}
// The longest segment whose workspace fits `bytes` (fewest segments), or -1.
int64_t seg_len_for(const hla_dims_t* d, int64_t bytes) {
  for (int64_t K = n_chunks(d); K >= 1; --K)
    if (compose_bwd_ws(d, K).total <= bytes) return K;
  return -1;
}

void set_compose_bwd_ws(hla::ComposeBwdArgs& a, const ComposeBwdWs& w, void* ws) {
  char* base = static_cast<char*>(ws);
  a.Ap = base + w.ap_off; a.ApT = base + w.apt_off; a.Bl = base + w.bl_off;
  a.Msave = base + w.ms_off; a.Dsave = base + w.ds_off; a.Lsave = base + w.ls_off;
  a.Ckpt = reinterpret_cast<float*>(base + w.ck_off);
  a.dgp = reinterpret_cast<float*>(base + w.dgp_off); a.lam_end = reinterpret_cast<float*>(base + w.le_off);
  a.K = w.K; a.slots = w.slots; a.nck = w.nck;
}

// Workspace of hla_chunk_backward: per-workgroup partial sums of the per-token gradients.
struct ChunkBwdWs {
  int64_t k_off, q_off, s_off, v_off, total;
};
ChunkBwdWs chunk_bwd_ws(const hla_dims_t* d) {
  const int64_t BHN = d->B * d->H * n_pieces(d), C = kPiece;
  const int64_t nb_out = d->dv / 32, nb_all = nb_out + (d->dk + d->dv) / 32;
  ChunkBwdWs w;
  w.k_off = 0;
  w.q_off = round_up(BHN * nb_all * C * d->dk * 4, 256);
  w.s_off = w.q_off + round_up(BHN * nb_out * C * d->dk * 4, 256);
  w.v_off = w.s_off + round_up(BHN * nb_all * C * 2 * 4, 256);
  w.total = w.v_off + round_up(BHN * 2 * C * d->dv * 4, 256);
  return w;
}

void set_chunk_bwd_ws(hla::ChunkBwdArgs& a, const ChunkBwdWs& w, void* ws) {
  char* base = static_cast<char*>(ws);
  a.part_k = reinterpret_cast<float*>(base + w.k_off);
  a.part_q = reinterpret_cast<float*>(base + w.q_off);
  a.part_s = reinterpret_cast<float*>(base + w.s_off);
  a.part_v = reinterpret_cast<float*>(base + w.v_off);
}

// Workspace of hla_gdn2_chunk_backward: per-workgroup column sums of the per-token
// gradients (gdn2_bwd_cols state columns per workgroup).
struct Gdn2ChunkBwdWs {
  int64_t k_off, a_off, b_off, q_off, v_off, w_off, total;
};
Gdn2ChunkBwdWs gdn2_chunk_bwd_ws(const hla_dims_t* d) {
  const int64_t BHN = d->B * d->H * n_pieces(d), C = kPiece, NC = hla::gdn2_bwd_cols(d->dtype);
  const int64_t nb_out = d->dv / NC, nb_all = nb_out + (d->dk + d->dv) / NC;
  const int64_t vec = round_up(BHN * nb_all * C * d->dk * 4, 256), per_v = round_up(BHN * 2 * C * d->dv * 4, 256);
  Gdn2ChunkBwdWs w;
  w.k_off = 0;
  w.a_off = vec;
  w.b_off = 2 * vec;
  w.q_off = 3 * vec;
  w.v_off = w.q_off + round_up(BHN * nb_out * C * d->dk * 4, 256);
  w.w_off = w.v_off + per_v;
  w.total = w.w_off + per_v;
  return w;
}

void set_gdn2_chunk_bwd_ws(hla::Gdn2BwdArgs& a, const Gdn2ChunkBwdWs& w, void* ws) {
  char* base = static_cast<char*>(ws);
  a.part_k = reinterpret_cast<float*>(base + w.k_off);
  a.part_a = reinterpret_cast<float*>(base + w.a_off);
  a.part_b = reinterpret_cast<float*>(base + w.b_off);
  a.part_q = reinterpret_cast<float*>(base + w.q_off);
  a.part_v = reinterpret_cast<float*>(base + w.v_off);
  a.part_w = reinterpret_cast<float*>(base + w.w_off);
}

// Workspace of hla_prefill_backward: the forward's transitions, route outputs and routed
// states, the gradients handed between the passes, then the workspaces of the route, the
// chunk backward and the composition backward (with history segments of K steps, last, so
// that what a caller's workspace holds beyond the rest sets the segment length).
struct PrefillBwdWs {
  int64_t at_off, bc_off, gates_off, mask_off, aidx_off, acnt_off, sr_off, dsr_off, dat_off, dbc_off, dg_off,
      qbar_off, dqbar_off, dkr_off, rpart_off, route_off, chunk_off, comp_off, total;
};
// (hla_gdn2_prefill_backward: the same with the Gated DeltaNet-2 chunk backward's region)
PrefillBwdWs prefill_bwd_ws(const hla_dims_t* d, int64_t K, int variant = 0) {
  const int64_t N = n_chunks(d), BH = d->B * d->H, BHN = BH * N, e = dtype_bytes(d->dtype);
  PrefillBwdWs w;
  int64_t o = 0;
  auto take = [&](int64_t bytes) {
    const int64_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  w.at_off = take(BHN * d->dk * d->dk * e);
  w.bc_off = take(BHN * d->dk * d->dv * e);
  w.gates_off = take(BH * N * N * 4);
  w.mask_off = take(BH * N * N);
  w.aidx_off = take(BH * N * N * 4);
  w.acnt_off = take(BHN * 4);
  w.sr_off = take(BHN * d->dk * d->dv * 4);
  w.dsr_off = take(BHN * d->dk * d->dv * 4);
  w.dat_off = take(BHN * d->dk * d->dk * 4);
  w.dbc_off = take(BHN * d->dk * d->dv * 4);
  w.dg_off = take(BH * N * N * 4);
  w.qbar_off = take(BHN * d->dk * 4);
  w.dqbar_off = take(BHN * d->dk * 4);
  w.dkr_off = take(d->B * d->T * d->H * d->dk * 4);
  w.rpart_off = take(hla::router_bwd_part_bytes(d->B, d->H, N, d->dk));
  w.route_off = take(route_ws(d));
  w.chunk_off = take(variant == 2 ? gdn2_chunk_bwd_ws(d).total : chunk_bwd_ws(d).total);
  w.comp_off = take(compose_bwd_ws(d, K).total);
  w.total = o;
  return w;
}

hla_status_t hip_status(hipError_t e) { return e == hipSuccess ? HLA_OK : HLA_ERR_HIP; }

// One chunk pass of either recurrence: transitions (want_ab) or outputs from chunk_init.
hipError_t chunk_pass(const hla::ChunkArgs& a, const hla_dims_t* d, bool want_ab, bool want_o, hipStream_t s) {
  if (a.variant == 2) return hla::launch_gdn2_chunk(a, d->dtype, d->dk, d->dv, want_o, s);
  return hla::launch_chunk(a, d->dtype, d->dk, d->dv, want_ab, want_o, s);
}

// Where a prefill's own transitions pass writes W | U: nowhere when the caller supplies
// them, for float32 or for the Gated DeltaNet-2 pass (which has no UT form), else the
// workspace region.
void* wu_internal(const hla_dims_t* d, const hla::ChunkArgs& a, const void* wu, void* region) {
  return (wu || d->dtype != HLA_BF16 || a.variant != 0) ? nullptr : region;
}

// Maps that the library writes for its own scans (never a caller's buffer) carry Bc in the
// scan's lane order, and the scan then hands the chunk start states on as the bf16 image the
// output pass multiplies with (bf16 Gated DeltaNet; the Gated DeltaNet-2 pass and float32
// keep the row-major forms).
int32_t own_lanes(const hla_dims_t* d, const hla::ChunkArgs& a) { return d->dtype == HLA_BF16 && a.variant != 2; }
void set_states(hla::ScanArgs& s, char* region) {
  if (s.lanes) s.states_t = region;
  else s.states = reinterpret_cast<float*>(region);
}

// Shared body of the transitions entry points (arguments validated by the caller; `a`
// carries the token inputs of either recurrence).
hla_status_t transitions_body(const hla_dims_t* d, hla::ChunkArgs a, void* At, void* Bc, void* wu, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  const PrefillWs w = prefill_ws(d);
  if (d->C != kPiece && (!ws || (int64_t)ws_bytes < w.total_ab)) return HLA_ERR_WORKSPACE;
  a.aux_out = wu;
  a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.N = (int32_t)n_pieces(d);
  if (d->C == kPiece) {
    a.At = At; a.Bc = Bc;
    return hip_status(chunk_pass(a, d, true, false, stream));
  }
  // pieces of 64 tokens, then the composite map of every C / 64 consecutive pieces
  char* base = static_cast<char*>(ws);
  a.At = base + w.at_off;
  a.Bc = base + w.bc_off;
  a.lanes = own_lanes(d, a);
  hipError_t e = chunk_pass(a, d, true, false, stream);
  if (e != hipSuccess) return HLA_ERR_HIP;
  hla::ScanArgs s{};
  s.At = a.At; s.Bc = a.Bc; s.B = d->B; s.H = d->H; s.N = a.N; s.lanes = a.lanes;
  s.seg = d->C / kPiece; s.seg_At = At; s.seg_Bc = Bc;
  return hip_status(hla::launch_combine_segments(s, d->dk, d->dv, stream));
}

// Shared body of the prefill entry points.
hla_status_t prefill_body(const hla_dims_t* d, hla::ChunkArgs a, const float* S0, const float* chunk_init,
                          const void* wu, float* o, float* S_final, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int32_t N = (int32_t)n_pieces(d);
  a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.N = N;
  const PrefillWs w = prefill_ws(d);
  if (chunk_init) {
    // routed: every chunk starts from its own given state
    if (S0 || S_final || !o) return HLA_ERR_UNSUPPORTED;
    a.o = o;
    if (d->C == kPiece) {
      a.chunk_init = chunk_init;
      a.aux_in = wu;
      return hip_status(chunk_pass(a, d, false, true, stream));
    }
    // C > 64: the start state of every 64-token piece from its chunk's routed state
    if (!ws || (int64_t)ws_bytes < w.total) return HLA_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws);
    a.At = base + w.at_off;
    a.Bc = base + w.bc_off;
    a.aux_out = wu_internal(d, a, wu, base + w.wu_off);
    a.lanes = own_lanes(d, a);
    hipError_t e = chunk_pass(a, d, true, false, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
    hla::ScanArgs s{};
    s.At = a.At; s.Bc = a.Bc; s.B = d->B; s.H = d->H; s.N = N; s.lanes = a.lanes;
    s.seg = d->C / kPiece; s.seg_init = chunk_init;
    set_states(s, base + w.st_off);
    e = hla::launch_scan_segments(s, d->dk, d->dv, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
    hla::ChunkArgs b = a;
    b.At = nullptr; b.Bc = nullptr; b.aux_out = nullptr; b.lanes = 0;
    b.aux_in = wu ? wu : a.aux_out;
    b.chunk_init = s.states;
    b.chunk_init_t = s.states_t;
    return hip_status(chunk_pass(b, d, false, true, stream));
  }
  if (d->dtype == HLA_BF16 && a.variant == 0) {
    // bf16 Gated DeltaNet: the per-piece UT records, then one state pass per (b, h) that
    // carries the state through the pieces and writes the outputs on the way (wu is not
    // read).
    if (!ws || (int64_t)ws_bytes < native_ws(d)) return HLA_ERR_WORKSPACE;
    hla::UtArgs f{};
    f.q = o ? a.q : nullptr; f.k = a.k; f.v = a.v; f.beta = a.beta; f.alpha = a.alpha;
    f.S0 = S0; f.o = o; f.S_final = S_final; f.rec = ws;
    f.B = d->B; f.T = d->T; f.H = d->H; f.ld_T = d->ld_T; f.N = N;
    return hip_status(hla::launch_prefill_native(f, d->dk, d->dv, stream));
  }
  const int64_t need = o ? w.total : w.total_ab;
  if (!ws || (int64_t)ws_bytes < need) return HLA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  a.At = base + w.at_off;
  a.Bc = base + w.bc_off;
  if (o) a.aux_out = wu_internal(d, a, wu, base + w.wu_off);
  a.lanes = own_lanes(d, a);
  hipError_t e = chunk_pass(a, d, true, false, stream);
  if (e != hipSuccess) return HLA_ERR_HIP;
  hla::ScanArgs s{};
  s.At = a.At; s.Bc = a.Bc; s.S0 = S0; s.lanes = a.lanes;
  if (o) set_states(s, base + w.st_off);
  s.S_final = S_final;
  s.B = d->B; s.H = d->H; s.N = N;
  e = hla::launch_scan(s, d->dtype, d->dk, d->dv, stream);
  if (e != hipSuccess || !o) return hip_status(e);
  hla::ChunkArgs b = a;
  b.At = nullptr; b.Bc = nullptr; b.aux_out = nullptr; b.lanes = 0;
  b.aux_in = wu ? wu : a.aux_out;
  b.chunk_init = s.states;
  b.chunk_init_t = s.states_t;
  b.o = o;
  return hip_status(chunk_pass(b, d, false, true, stream));
}

}  // namespace

extern "C" {

int32_t hla_abi_version(void) { return HLA_ABI_VERSION; }

const char* hla_status_string(int32_t s) {
  switch (s) {
    case HLA_OK: return "ok";
    case HLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case HLA_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case HLA_ERR_BAD_DTYPE: return "dtype must be HLA_F32 or HLA_BF16";
    case HLA_ERR_WORKSPACE: return "workspace missing or too small";
    case HLA_ERR_HIP: return "a HIP kernel launch failed";
    case HLA_ERR_UNSUPPORTED: return "unsupported combination of arguments";
    case HLA_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case HLA_ERR_INTERNAL: return "internal error";
    case HLA_ERR_SCRATCH_LIMIT: return "the problem needs more scratch than the fixed device buffer holds";
    default: return "unknown status";
  }
}

hla_status_t hla_workspace_bytes(int32_t fn, const hla_dims_t* d, int32_t n_rep, size_t* out) {
  if (!out) return HLA_ERR_NULL_ARG;
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  switch (fn) {
    case HLA_FN_CHUNK_TRANSITIONS: *out = d->C == kPiece ? 0 : (size_t)prefill_ws(d).total_ab; return HLA_OK;
    case HLA_FN_GDN_PREFILL: *out = (size_t)prefill_ws(d).total; return HLA_OK;
    case HLA_FN_ROUTE_MIX: *out = (size_t)route_ws(d); return HLA_OK;
    case HLA_FN_WU_HANDOFF: *out = (size_t)wu_bytes(d); return HLA_OK;
    case HLA_FN_CHUNK_REPS:
      if (n_rep < 1 || d->C % n_rep != 0) return HLA_ERR_BAD_SHAPE;
      *out = (size_t)reps_ws(d, n_rep);
      return HLA_OK;
    case HLA_FN_COMPOSE_BACKWARD: *out = (size_t)compose_bwd_ws(d, n_chunks(d)).total; return HLA_OK;
    case HLA_FN_COMPOSE_BACKWARD_MIN: *out = (size_t)compose_bwd_min(d); return HLA_OK;
    case HLA_FN_CHUNK_BACKWARD:
      if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
      *out = (size_t)chunk_bwd_ws(d).total;
      return HLA_OK;
    case HLA_FN_PREFILL_BACKWARD:
    case HLA_FN_PREFILL_BACKWARD_MIN:
    case HLA_FN_GDN2_PREFILL_BACKWARD:
    case HLA_FN_GDN2_PREFILL_BACKWARD_MIN: {
      if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
      const int variant = (fn == HLA_FN_GDN2_PREFILL_BACKWARD || fn == HLA_FN_GDN2_PREFILL_BACKWARD_MIN) ? 2 : 0;
      const bool one_pass = fn == HLA_FN_PREFILL_BACKWARD || fn == HLA_FN_GDN2_PREFILL_BACKWARD;
      *out = one_pass ? (size_t)prefill_bwd_ws(d, n_chunks(d), variant).total
                      : (size_t)(prefill_bwd_ws(d, 1, variant).comp_off + compose_bwd_min(d));
      return HLA_OK;
    }
    case HLA_FN_ROUTER_BACKWARD:
      if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
      *out = (size_t)router_bwd_ws(d);
      return HLA_OK;
    case HLA_FN_CHUNK_REPS_BACKWARD:
      if (d->C % kPiece != 0) return HLA_ERR_UNSUPPORTED;
      *out = (size_t)reps_bwd_ws(d, n_rep != 0);
      return HLA_OK;
    case HLA_FN_GDN2_CHUNK_BACKWARD:
      if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
      *out = (size_t)gdn2_chunk_bwd_ws(d).total;
      return HLA_OK;
    default: return HLA_ERR_UNSUPPORTED;
  }
}

hla_status_t hla_chunk_transitions(const hla_dims_t* d, const void* k, const void* v, const float* beta,
                                   const float* alpha, void* At, void* Bc, void* wu, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!k || !v || !beta || !alpha || !At || !Bc) return HLA_ERR_NULL_ARG;
  if (!all_aligned(k, v, At, Bc, wu, ws) || !all_aligned4(beta, alpha)) return HLA_ERR_ALIGN;
  if (wu && d->dtype != HLA_BF16) return HLA_ERR_UNSUPPORTED;
  hla::ChunkArgs a{};
  a.k = k; a.v = v; a.beta = beta; a.alpha = alpha;
  return transitions_body(d, a, At, Bc, wu, ws, ws_bytes, stream);
}

hla_status_t hla_gdn2_chunk_transitions(const hla_dims_t* d, const void* k, const void* v, const float* a_decay,
                                        const float* b_erase, const float* w_write, void* At, void* Bc, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!k || !v || !a_decay || !b_erase || !w_write || !At || !Bc) return HLA_ERR_NULL_ARG;
  if (!all_aligned(k, v, At, Bc, ws) || !all_aligned4(a_decay, b_erase, w_write)) return HLA_ERR_ALIGN;
  hla::ChunkArgs a{};
  a.k = k; a.v = v; a.ga = a_decay; a.gb = b_erase; a.gw = w_write; a.variant = 2;
  return transitions_body(d, a, At, Bc, nullptr, ws, ws_bytes, stream);
}

hla_status_t hla_gdn_prefill(const hla_dims_t* d, const void* q, const void* k, const void* v,
                             const float* beta, const float* alpha, const float* S0, const float* chunk_init,
                             const void* wu, float* o, float* S_final, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!k || !v || !beta || !alpha) return HLA_ERR_NULL_ARG;
  if (!o && !S_final) return HLA_ERR_NULL_ARG;
  if (o && !q) return HLA_ERR_NULL_ARG;
  if (!all_aligned(q, k, v, S0, chunk_init, wu, S_final, ws) || !all_aligned4(beta, alpha, o)) return HLA_ERR_ALIGN;
  if (wu && d->dtype != HLA_BF16) return HLA_ERR_UNSUPPORTED;
  hla::ChunkArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.alpha = alpha;
  return prefill_body(d, a, S0, chunk_init, wu, o, S_final, ws, ws_bytes, stream);
}

hla_status_t hla_gdn2_prefill(const hla_dims_t* d, const void* q, const void* k, const void* v, const float* a_decay,
                              const float* b_erase, const float* w_write, const float* S0, const float* chunk_init,
                              float* o, float* S_final, void* ws, size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!k || !v || !a_decay || !b_erase || !w_write) return HLA_ERR_NULL_ARG;
  if (!o && !S_final) return HLA_ERR_NULL_ARG;
  if (o && !q) return HLA_ERR_NULL_ARG;
  if (!all_aligned(q, k, v, S0, chunk_init, S_final, ws) || !all_aligned4(a_decay, b_erase, w_write, o))
    return HLA_ERR_ALIGN;
  hla::ChunkArgs a{};
  a.q = q; a.k = k; a.v = v; a.ga = a_decay; a.gb = b_erase; a.gw = w_write; a.variant = 2;
  return prefill_body(d, a, S0, chunk_init, nullptr, o, S_final, ws, ws_bytes, stream);
}

// Shared checks and arguments of the two representative entry points (all but the scratch).
static hla_status_t reps_args(const hla_dims_t* d, const void* k, int32_t window, const void* Wq, const void* Wk,
                              const void* Wv, const void* Wp, const void* Wr, int64_t w_hstride, void* reps,
                              hla::RepsArgs* a) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!k || !Wq || !Wk || !Wv || !Wp || !reps) return HLA_ERR_NULL_ARG;
  if (window != 8 && window != 16 && window != 32 && window != 64) return HLA_ERR_BAD_SHAPE;
  const int64_t wsz = (int64_t)d->dk * d->dk;
  if (w_hstride != 0 && w_hstride < wsz) return HLA_ERR_BAD_SHAPE;
  if ((w_hstride * dtype_bytes(d->dtype)) % 16 != 0) return HLA_ERR_ALIGN;
  if (!all_aligned(k, Wq, Wk, Wv, Wp, Wr, reps)) return HLA_ERR_ALIGN;
  *a = hla::RepsArgs{};
  a->k = k; a->B = d->B; a->T = d->T; a->H = d->H; a->ld_T = d->ld_T;
  a->C = d->C; a->window = window; a->N = (int32_t)n_chunks(d);
  a->Wq = Wq; a->Wk = Wk; a->Wv = Wv; a->Wp = Wp; a->Wr = Wr; a->w_hstride = w_hstride;
  a->reps = reps;
  return HLA_OK;
}

hla_status_t hla_chunk_reps(const hla_dims_t* d, const void* k, int32_t window, const void* Wq, const void* Wk,
                            const void* Wv, const void* Wp, const void* Wr, int64_t w_hstride, void* reps, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  hla::RepsArgs a;
  const hla_status_t st = reps_args(d, k, window, Wq, Wk, Wv, Wp, Wr, w_hstride, reps, &a);
  if (st != HLA_OK) return st;
  if (!aligned16(ws)) return HLA_ERR_ALIGN;
  if (!ws || (int64_t)ws_bytes < reps_ws(d, d->C / window)) return HLA_ERR_WORKSPACE;
  a.pooled = static_cast<float*>(ws);
  return hip_status(hla::launch_reps(a, d->dtype, d->dk, stream));
}

hla_status_t hla_chunk_reps_noalloc(const hla_dims_t* d, const void* k, int32_t window, const void* Wq,
                                    const void* Wk, const void* Wv, const void* Wp, const void* Wr,
                                    int64_t w_hstride, void* reps, hipStream_t stream) {
  hla::RepsArgs a;
  const hla_status_t st = reps_args(d, k, window, Wq, Wk, Wv, Wp, Wr, w_hstride, reps, &a);
  if (st != HLA_OK) return st;
  // the size limit is checked before anything touches the GPU
  if (reps_ws(d, d->C / window) > hla::kRepsScratchBytes) return HLA_ERR_SCRATCH_LIMIT;
  float* scratch = nullptr;
  if (hla::reps_scratch(&scratch) != hipSuccess) return HLA_ERR_HIP;
  a.pooled = scratch;
  return hip_status(hla::launch_reps(a, d->dtype, d->dk, stream));
}

hla_status_t hla_chunk_reps_backward(const hla_dims_t* d, const void* k, int32_t window, const void* Wq,
                                     const void* Wk, const void* Wv, const void* Wp, const void* Wr, int64_t w_hstride,
                                     const float* dreps, float* dk, float* dWq, float* dWk, float* dWv, float* dWp,
                                     float* dWr, void* ws, size_t ws_bytes, hipStream_t stream) {
  hla::RepsArgs f;
  hla_status_t st = reps_args(d, k, window, Wq, Wk, Wv, Wp, Wr, w_hstride, const_cast<float*>(dreps), &f);
  if (st != HLA_OK) return st;
  if (d->C % kPiece != 0) return HLA_ERR_UNSUPPORTED;
  if (!dk || !dWq || !dWk || !dWv || !dWp || (Wr && !dWr)) return HLA_ERR_NULL_ARG;
  if (!all_aligned(ws) || !all_aligned4(dk, dWq, dWk, dWv, dWp, dWr)) return HLA_ERR_ALIGN;
  if (!ws || (int64_t)ws_bytes < reps_bwd_ws(d, Wr != nullptr)) return HLA_ERR_WORKSPACE;
  hla::RepsBwdArgs a{};
  a.k = k; a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.window = window;
  a.Wq = Wq; a.Wk = Wk; a.Wv = Wv; a.Wp = Wp; a.Wr = Wr; a.w_hstride = w_hstride;
  a.dreps = dreps; a.R = n_chunks(d) * (d->C / window); a.dk = dk;
  a.part = static_cast<float*>(ws);
  a.wvec = reinterpret_cast<float*>(static_cast<char*>(ws) + reps_bwd_part_bytes(d));
  a.part2 = reinterpret_cast<float*>(static_cast<char*>(ws) + reps_bwd_part_bytes(d) + reps_bwd_vec_bytes(d));
  a.RW = reps_bwd_rows(d);
  a.dW[0] = dWq; a.dW[1] = dWk; a.dW[2] = dWv; a.dW[3] = dWp; a.dW[4] = Wr ? dWr : nullptr;
  return hip_status(hla::launch_reps_backward(a, d->dtype, d->dk, stream));
}

hla_status_t hla_router_backward(const hla_dims_t* d, const void* q, const void* reps, int32_t n_rep, int64_t ld_R,
                                 const float* gates, const float* dgates, float* dq, float* dreps, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
  if (!q || !reps || !gates || !dgates || !dq || !dreps) return HLA_ERR_NULL_ARG;
  const int64_t N = n_chunks(d);
  if (n_rep < 1 || n_rep > kPiece || ld_R < (N - 1) * (int64_t)n_rep) return HLA_ERR_BAD_SHAPE;
  if (!all_aligned(q, reps, ws) || !all_aligned4(gates, dgates, dq, dreps)) return HLA_ERR_ALIGN;
  if (!ws || (int64_t)ws_bytes < router_bwd_ws(d)) return HLA_ERR_WORKSPACE;
  hla::RouterBwdArgs rb{};
  rb.q = q; rb.reps = reps; rb.gates = gates; rb.dgates = dgates;
  rb.qbar = static_cast<float*>(ws);
  rb.dqbar = reinterpret_cast<float*>(static_cast<char*>(ws) + router_bwd_means(d));
  rb.part = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * router_bwd_means(d));
  rb.dreps = dreps; rb.dq_tok = dq;
  rb.B = d->B; rb.T = d->T; rb.H = d->H; rb.ld_T = d->ld_T; rb.N = (int32_t)N;
  rb.n_rep = n_rep; rb.ld_R = ld_R; rb.R_out = N * n_rep;
  return hip_status(hla::launch_router_backward(rb, d->dtype, d->dk, stream));
}

hla_status_t hla_route_mix(const hla_dims_t* d, const void* q, const void* reps, int32_t n_rep, int64_t ld_R,
                           const void* At, const void* Bc, const float* S0, const float* gates_in, float tau,
                           float* gates, uint8_t* mask, int32_t* active_idx, int32_t* active_cnt, float* n_eff,
                           float* S_routed, void* ws, size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  const int64_t N = n_chunks(d);
  if (!At || !Bc || !gates || !mask || !active_idx || !active_cnt || !S_routed) return HLA_ERR_NULL_ARG;
  const bool computed = !gates_in && N > 1;
  if (computed && (!q || !reps)) return HLA_ERR_NULL_ARG;
  if (computed && (n_rep < 1 || ld_R < (N - 1) * (int64_t)n_rep)) return HLA_ERR_BAD_SHAPE;
  if (std::isnan(tau)) return HLA_ERR_BAD_SHAPE;
  if (!all_aligned(q, reps, At, Bc, S0, S_routed, ws) || !all_aligned4(gates_in, gates, active_idx, active_cnt, n_eff))
    return HLA_ERR_ALIGN;
  if (!ws || (int64_t)ws_bytes < route_ws(d)) return HLA_ERR_WORKSPACE;
  hla::RouteArgs a{};
  a.q = q; a.reps = reps; a.n_rep = n_rep; a.ld_R = ld_R; a.At = At; a.Bc = Bc; a.S0 = S0;
  a.gates_in = gates_in; a.tau = tau; a.gates = gates; a.mask = mask; a.active_idx = active_idx;
  a.active_cnt = active_cnt; a.n_eff = n_eff; a.S_routed = S_routed; a.qbar = static_cast<float*>(ws);
  a.At_prep = static_cast<char*>(ws) + route_qbar_bytes(d);
  a.Bc_prep = static_cast<char*>(a.At_prep) + route_atp_bytes(d);
  a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.N = (int32_t)N; a.C = d->C;
  return hip_status(hla::launch_route(a, d->dtype, d->dk, d->dv, stream));
}

// The composition backward's checkpoints from the bf16 composition of the forward: it runs
// every chain (sharing each staged map among several chains) and keeps each chain's state at
// the segment boundaries it crosses; its reordered maps go to the backward's Ap and Bl
// regions, which the backward's prep stage overwrites afterwards.
static hipError_t compose_checkpoints(hla::ComposeBwdArgs& a, const hla_dims_t* d, hipStream_t stream) {
  hla::RouteArgs r{};
  r.At = a.At; r.Bc = a.Bc; r.S0 = a.S0; r.gates = const_cast<float*>(a.gates);
  r.mask = const_cast<uint8_t*>(a.mask);
  r.S_routed = a.S_routed ? a.S_routed : a.lam_end;
  r.At_prep = a.Ap; r.Bc_prep = a.Bl;
  r.B = d->B; r.T = d->T; r.H = d->H; r.ld_T = d->ld_T; r.N = a.N; r.C = d->C;
  r.ckpt = a.Ckpt; r.ckpt_K = a.K; r.ckpt_nck = a.nck;
  a.ckpt_done = 1;
  return hla::launch_compose_bf16(r, d->dk, d->dv, stream);
}

hla_status_t hla_compose_backward(const hla_dims_t* d, const void* At, const void* Bc, const float* gates,
                                  const uint8_t* mask, const float* S0, const float* dS_routed, float* dAt,
                                  float* dBc, float* dgates, float* dS0, float* S_routed, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (!At || !Bc || !gates || !mask || !dS_routed || !dAt || !dBc || !dgates) return HLA_ERR_NULL_ARG;
  if (!all_aligned(At, Bc, S0, dS_routed, dAt, dBc, dS0, S_routed, ws) || !all_aligned4(gates, dgates))
    return HLA_ERR_ALIGN;
  const int64_t K = ws ? seg_len_for(d, (int64_t)ws_bytes) : -1;
  if (K < 0) return HLA_ERR_WORKSPACE;
  hla::ComposeBwdArgs a{};
  a.At = At; a.Bc = Bc; a.gates = gates; a.mask = mask; a.S0 = S0; a.dS = dS_routed;
  a.dAt = dAt; a.dBc = dBc; a.dgates = dgates; a.dS0 = dS0; a.S_routed = S_routed;
  set_compose_bwd_ws(a, compose_bwd_ws(d, K), ws);
  a.B = d->B; a.H = d->H; a.N = (int32_t)n_chunks(d);
  hipError_t e = hipSuccess;
  if (a.K < a.N && d->dtype == HLA_BF16) {
    // checkpoints (and the routed states) from the bf16 composition, with its reordered
    // maps in the regions the backward's own take over afterwards; without a caller's
    // S_routed the states land in the lambda buffer, which is free until the adjoint
    e = compose_checkpoints(a, d, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
  }
  // the reordered maps (and the checkpoints, if not yet taken), then the segments last to
  // first
  e = hla::launch_compose_backward(a, d->dtype, d->dk, d->dv, hla::kComposeBwdPrep, stream);
  if (e != hipSuccess) return HLA_ERR_HIP;
  if (a.K < a.N) a.S_routed = nullptr;  // written with the checkpoints
  for (int32_t j0 = (a.N - 1) / a.K * a.K; j0 >= 0; j0 -= a.K) {
    a.j0 = j0; a.j1 = std::min(j0 + a.K, a.N);
    e = hla::launch_compose_backward(a, d->dtype, d->dk, d->dv, hla::kComposeBwdSave | hla::kComposeBwdReverse, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
  }
  return hip_status(hla::launch_compose_backward(a, d->dtype, d->dk, d->dv, hla::kComposeBwdFinish, stream));
}

hla_status_t hla_chunk_backward(const hla_dims_t* d, const void* q, const void* k, const void* v, const float* beta,
                                const float* alpha, const float* chunk_init, const float* dO, const float* dAt,
                                const float* dBc, float* dq, float* dk, float* dv, float* dbeta, float* dalpha,
                                float* dchunk_init, void* ws, size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
  const bool have_out = chunk_init || dO, have_map = dAt || dBc;
  if (!have_out && !have_map) return HLA_ERR_NULL_ARG;
  if (have_out && (!chunk_init || !dO || !q || !dchunk_init)) return HLA_ERR_NULL_ARG;
  if (have_map && (!dAt || !dBc)) return HLA_ERR_NULL_ARG;
  if (!k || !v || !beta || !alpha || !dq || !dk || !dv || !dbeta || !dalpha) return HLA_ERR_NULL_ARG;
  if (!all_aligned(q, k, v, chunk_init, dAt, dBc, dchunk_init, ws) ||
      !all_aligned4(beta, alpha, dO, dq, dk, dv, dbeta, dalpha))
    return HLA_ERR_ALIGN;
  const ChunkBwdWs w = chunk_bwd_ws(d);
  if (!ws || (int64_t)ws_bytes < w.total) return HLA_ERR_WORKSPACE;
  hla::ChunkBwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.alpha = alpha;
  a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.N = (int32_t)n_pieces(d);
  a.c0 = 0; a.c1 = a.N;
  a.have_out = have_out; a.have_map = have_map;
  a.chunk_init = chunk_init; a.dO = dO; a.dAt = dAt; a.dBc = dBc; a.dchunk_init = dchunk_init;
  set_chunk_bwd_ws(a, w, ws);
  a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta; a.dalpha = dalpha;
  const int stages = (have_out ? hla::kChunkBwdOut : 0) | (have_map ? hla::kChunkBwdMap : 0) | hla::kChunkBwdFinalize;
  return hip_status(hla::launch_chunk_backward(a, d->dtype, d->dk, d->dv, stages, stream));
}

}  // extern "C"

// What the routed-prefill backward hands the per-chunk reverse of its recurrence.
struct ChunkBwdBufs {
  const float* S_routed;  // [B,H,N,dk,dv] each chunk's routed start state (the forward's)
  float* dS_routed;       // out: its gradient (outputs part)
  const float* dAt;       // gradients of the chunk maps (maps part)
  const float* dBc;
  void* ws;               // the chunk reverse's own workspace region
  const float* dqbar;     // router parts for the per-token sums, or null
  const float* dk_router;
};

// The routed-prefill backward of either recurrence (C = 64, raw-key representatives):
// `maps(At, Bc)` recomputes the forward's chunk maps, `chunk_bwd(bufs, stages)` runs the
// per-chunk reverse (stages kChunkBwdOut, kChunkBwdMap, kChunkBwdFinalize).  The router, the
// composition and their reverses are the same for both ([HLA] Methodology paragraphs 2-4).
template <class Maps, class ChunkBwd>
static hla_status_t prefill_backward_body(const hla_dims_t* d, int variant, const void* q, const void* k,
                                          const float* S0, const float* gates_in, float tau, float* dS0, float* dgates,
                                          void* ws, size_t ws_bytes, hipStream_t stream, Maps maps,
                                          ChunkBwd chunk_bwd) {
  const PrefillBwdWs w0 = prefill_bwd_ws(d, 1, variant);
  const int64_t K = ws ? seg_len_for(d, (int64_t)ws_bytes - w0.comp_off) : -1;
  if (K < 0) return HLA_ERR_WORKSPACE;
  const PrefillBwdWs w = prefill_bwd_ws(d, K, variant);
  char* base = static_cast<char*>(ws);
  const int32_t N = (int32_t)n_chunks(d);
  auto at = [&](int64_t off) { return static_cast<void*>(base + off); };
  auto fat = [&](int64_t off) { return reinterpret_cast<float*>(base + off); };
  // 1. forward: chunk maps, then gates, mask and lists (the routed states come from the
  //    composition backward's forward replay)
  hipError_t e = maps(at(w.at_off), at(w.bc_off));
  if (e != hipSuccess) return HLA_ERR_HIP;
  hla::RouteArgs r{};
  r.q = q; r.reps = k; r.n_rep = kPiece; r.ld_R = d->ld_T; r.At = at(w.at_off); r.Bc = at(w.bc_off); r.S0 = S0;
  r.gates_in = gates_in; r.tau = tau; r.gates = fat(w.gates_off);
  r.mask = reinterpret_cast<uint8_t*>(base + w.mask_off);
  r.active_idx = reinterpret_cast<int32_t*>(base + w.aidx_off);
  r.active_cnt = reinterpret_cast<int32_t*>(base + w.acnt_off);
  r.n_eff = nullptr; r.S_routed = nullptr;
  r.qbar = fat(w.route_off); r.At_prep = base + w.route_off + route_qbar_bytes(d);
  r.Bc_prep = static_cast<char*>(r.At_prep) + route_atp_bytes(d);
  r.B = d->B; r.T = d->T; r.H = d->H; r.ld_T = d->ld_T; r.N = N; r.C = d->C;
  e = hla::launch_route(r, d->dtype, d->dk, d->dv, stream);
  if (e != hipSuccess) return HLA_ERR_HIP;
  float* dg = dgates ? dgates : fat(w.dg_off);
  hla::ComposeBwdArgs m{};
  m.At = r.At; m.Bc = r.Bc; m.gates = r.gates; m.mask = r.mask; m.S0 = S0; m.dS = fat(w.dsr_off);
  m.dAt = fat(w.dat_off); m.dBc = fat(w.dbc_off); m.dgates = dg; m.dS0 = dS0; m.S_routed = fat(w.sr_off);
  set_compose_bwd_ws(m, compose_bwd_ws(d, K), at(w.comp_off));
  m.B = d->B; m.H = d->H; m.N = N;
  ChunkBwdBufs cb{fat(w.sr_off), fat(w.dsr_off), m.dAt, m.dBc, at(w.chunk_off), nullptr, nullptr};
  // 2. composition backward, forward replay: with more than one history segment the
  //    checkpoints and the routed states (from the bf16 composition, or the backward's own
  //    replay), then the reordered maps; with one segment the routed states come from the
  //    segment's replay
  if (m.K < N && d->dtype == HLA_BF16) {
    e = compose_checkpoints(m, d, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
  }
  e = hla::launch_compose_backward(m, d->dtype, d->dk, d->dv, hla::kComposeBwdPrep, stream);
  if (e != hipSuccess) return HLA_ERR_HIP;
  const int32_t j_last = (N - 1) / m.K * m.K;
  m.j0 = j_last; m.j1 = N;
  if (m.K >= N) {
    e = hla::launch_compose_backward(m, d->dtype, d->dk, d->dv, hla::kComposeBwdSave, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
  }
  m.S_routed = nullptr;
  // 3. outputs part of the chunk backward: dS~ and the chunk-local partial sums
  e = chunk_bwd(cb, hla::kChunkBwdOut);
  if (e != hipSuccess) return HLA_ERR_HIP;
  // 4. composition backward per history segment, last to first: replay the segment's steps
  //    keeping their states (already done for a single segment), then the adjoint and the
  //    segment's parts of dAt, dBc, dgates; dS0 at the end
  for (int32_t j0 = j_last; j0 >= 0; j0 -= m.K) {
    m.j0 = j0; m.j1 = std::min(j0 + m.K, N);
    const int stages = (m.K >= N ? 0 : hla::kComposeBwdSave) | hla::kComposeBwdReverse;
    e = hla::launch_compose_backward(m, d->dtype, d->dk, d->dv, stages, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
  }
  e = hla::launch_compose_backward(m, d->dtype, d->dk, d->dv, hla::kComposeBwdFinish, stream);
  if (e != hipSuccess) return HLA_ERR_HIP;
  // then the maps part of the chunk backward
  e = chunk_bwd(cb, hla::kChunkBwdMap);
  if (e != hipSuccess) return HLA_ERR_HIP;
  // 5. router (computed gates only), then the per-token sums
  if (!gates_in && N > 1) {
    hla::RouterBwdArgs rb{};
    rb.q = q; rb.reps = k; rb.gates = r.gates; rb.dgates = dg;
    rb.qbar = fat(w.qbar_off); rb.dqbar = fat(w.dqbar_off); rb.dreps = fat(w.dkr_off); rb.part = fat(w.rpart_off);
    rb.B = d->B; rb.T = d->T; rb.H = d->H; rb.ld_T = d->ld_T; rb.N = N;
    rb.n_rep = kPiece; rb.ld_R = d->ld_T; rb.R_out = d->T;  // the raw keys, rows = tokens
    e = hla::launch_router_backward(rb, d->dtype, d->dk, stream);
    if (e != hipSuccess) return HLA_ERR_HIP;
    cb.dqbar = rb.dqbar;
    cb.dk_router = rb.dreps;
  }
  return hip_status(chunk_bwd(cb, hla::kChunkBwdFinalize));
}

extern "C" {

hla_status_t hla_prefill_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                  const float* beta, const float* alpha, const float* S0, const float* gates_in,
                                  float tau, const float* dO, float* dq, float* dk, float* dv, float* dbeta,
                                  float* dalpha, float* dS0, float* dgates, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !beta || !alpha || !dO || !dq || !dk || !dv || !dbeta || !dalpha) return HLA_ERR_NULL_ARG;
  if (std::isnan(tau)) return HLA_ERR_BAD_SHAPE;
  if (!all_aligned(q, k, v, S0, dS0, ws) || !all_aligned4(beta, alpha, gates_in, dO, dq, dk, dv, dbeta, dalpha, dgates))
    return HLA_ERR_ALIGN;
  const int32_t N = (int32_t)n_chunks(d);
  auto maps = [&](void* At, void* Bc) {
    hla::ChunkArgs c{};
    c.q = q; c.k = k; c.v = v; c.beta = beta; c.alpha = alpha;
    c.B = d->B; c.T = d->T; c.H = d->H; c.ld_T = d->ld_T; c.N = N;
    c.At = At; c.Bc = Bc;
    return hla::launch_chunk(c, d->dtype, d->dk, d->dv, true, false, stream);
  };
  auto chunk_bwd = [&](const ChunkBwdBufs& p, int stages) {
    hla::ChunkBwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.alpha = alpha;
    a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.N = N;
    a.c0 = 0; a.c1 = N;
    a.have_out = 1; a.have_map = 1;
    a.chunk_init = p.S_routed; a.dO = dO; a.dchunk_init = p.dS_routed; a.dAt = p.dAt; a.dBc = p.dBc;
    set_chunk_bwd_ws(a, chunk_bwd_ws(d), p.ws);
    a.dqbar = p.dqbar; a.dk_router = p.dk_router;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta; a.dalpha = dalpha;
    return hla::launch_chunk_backward(a, d->dtype, d->dk, d->dv, stages, stream);
  };
  return prefill_backward_body(d, 0, q, k, S0, gates_in, tau, dS0, dgates, ws, ws_bytes, stream, maps, chunk_bwd);
}

}  // extern "C"

static hla::Gdn2BwdArgs gdn2_bwd_args(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                      const float* a_decay, const float* b_erase, const float* w_write, float* dq,
                                      float* dk, float* dv, float* da, float* db, float* dw) {
  hla::Gdn2BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.ga = a_decay; a.gb = b_erase; a.gw = w_write;
  a.B = d->B; a.T = d->T; a.H = d->H; a.ld_T = d->ld_T; a.N = (int32_t)n_pieces(d);
  a.c0 = 0; a.c1 = a.N;
  a.dq = dq; a.dk = dk; a.dv = dv; a.da = da; a.db = db; a.dw = dw;
  return a;
}

extern "C" {

hla_status_t hla_gdn2_chunk_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                     const float* a_decay, const float* b_erase, const float* w_write,
                                     const float* chunk_init, const float* dO, const float* dAt, const float* dBc,
                                     float* dq, float* dk, float* dv, float* da, float* db, float* dw,
                                     float* dchunk_init, void* ws, size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
  const bool have_out = chunk_init || dO, have_map = dAt || dBc;
  if (!have_out && !have_map) return HLA_ERR_NULL_ARG;
  if (have_out && (!chunk_init || !dO || !q || !dchunk_init)) return HLA_ERR_NULL_ARG;
  if (have_map && (!dAt || !dBc)) return HLA_ERR_NULL_ARG;
  if (!k || !v || !a_decay || !b_erase || !w_write || !dq || !dk || !dv || !da || !db || !dw) return HLA_ERR_NULL_ARG;
  if (!all_aligned(q, k, v, chunk_init, dAt, dBc, dchunk_init, ws) ||
      !all_aligned4(a_decay, b_erase, w_write, dO, dq, dk, dv, da, db, dw))
    return HLA_ERR_ALIGN;
  const Gdn2ChunkBwdWs w = gdn2_chunk_bwd_ws(d);
  if (!ws || (int64_t)ws_bytes < w.total) return HLA_ERR_WORKSPACE;
  hla::Gdn2BwdArgs a = gdn2_bwd_args(d, q, k, v, a_decay, b_erase, w_write, dq, dk, dv, da, db, dw);
  a.have_out = have_out; a.have_map = have_map;
  a.chunk_init = chunk_init; a.dO = dO; a.dAt = dAt; a.dBc = dBc; a.dchunk_init = dchunk_init;
  set_gdn2_chunk_bwd_ws(a, w, ws);
  const int stages = (have_out ? hla::kChunkBwdOut : 0) | (have_map ? hla::kChunkBwdMap : 0) | hla::kChunkBwdFinalize;
  return hip_status(hla::launch_gdn2_chunk_backward(a, d->dtype, d->dk, d->dv, stages, stream));
}

hla_status_t hla_gdn2_prefill_backward(const hla_dims_t* d, const void* q, const void* k, const void* v,
                                       const float* a_decay, const float* b_erase, const float* w_write,
                                       const float* S0, const float* gates_in, float tau, const float* dO, float* dq,
                                       float* dk, float* dv, float* da, float* db, float* dw, float* dS0,
                                       float* dgates, void* ws, size_t ws_bytes, hipStream_t stream) {
  hla_status_t st = check_dims(d);
  if (st != HLA_OK) return st;
  if (d->C != kPiece) return HLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !a_decay || !b_erase || !w_write || !dO || !dq || !dk || !dv || !da || !db || !dw)
    return HLA_ERR_NULL_ARG;
  if (std::isnan(tau)) return HLA_ERR_BAD_SHAPE;
  if (!all_aligned(q, k, v, S0, dS0, ws) ||
      !all_aligned4(a_decay, b_erase, w_write, gates_in, dO, dq, dk, dv, da, db, dw, dgates))
    return HLA_ERR_ALIGN;
  const int32_t N = (int32_t)n_chunks(d);
  auto maps = [&](void* At, void* Bc) {
    hla::ChunkArgs c{};
    c.k = k; c.v = v; c.ga = a_decay; c.gb = b_erase; c.gw = w_write; c.variant = 2;
    c.B = d->B; c.T = d->T; c.H = d->H; c.ld_T = d->ld_T; c.N = N;
    c.At = At; c.Bc = Bc;
    return hla::launch_gdn2_chunk(c, d->dtype, d->dk, d->dv, false, stream);
  };
  auto chunk_bwd = [&](const ChunkBwdBufs& p, int stages) {
    hla::Gdn2BwdArgs a = gdn2_bwd_args(d, q, k, v, a_decay, b_erase, w_write, dq, dk, dv, da, db, dw);
    a.have_out = 1; a.have_map = 1;
    a.chunk_init = p.S_routed; a.dO = dO; a.dchunk_init = p.dS_routed; a.dAt = p.dAt; a.dBc = p.dBc;
    set_gdn2_chunk_bwd_ws(a, gdn2_chunk_bwd_ws(d), p.ws);
    a.dqbar = p.dqbar; a.dk_router = p.dk_router;
    return hla::launch_gdn2_chunk_backward(a, d->dtype, d->dk, d->dv, stages, stream);
  };
  return prefill_backward_body(d, 2, q, k, S0, gates_in, tau, dS0, dgates, ws, ws_bytes, stream, maps, chunk_bwd);
}

// Shared checks of the two decode entry points (everything but the per-token gates).
static hla_status_t decode_checks(int64_t Bs, int64_t H, int32_t dk, int32_t dv, int32_t dtype, const void* q, const void* k,
                           const void* v, float* S_cur, float* At_cur, void* At_cache, void* Bc_cache,
                           const void* reps_cache, int32_t n_rep, int32_t* n_cache, int32_t n_cap,
                           const float* gates_in, float tau, float* o, float* gates_out, int32_t commit) {
  if (dtype != HLA_F32 && dtype != HLA_BF16) return HLA_ERR_BAD_DTYPE;
  if (Bs < 1 || H < 1 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return HLA_ERR_BAD_SHAPE;
  if ((double)Bs * (double)H > (double)kMaxGrid) return HLA_ERR_BAD_SHAPE;
  if (!q || !k || !v || !S_cur || !o) return HLA_ERR_NULL_ARG;
  if (commit != 0 && commit != 1) return HLA_ERR_BAD_SHAPE;
  if (!At_cur) {
    if (commit) return HLA_ERR_UNSUPPORTED;
  } else {
    if (!n_cache || !At_cache || !Bc_cache) return HLA_ERR_NULL_ARG;
    if (n_cap < 0 || n_cap > kMaxCacheSlots) return HLA_ERR_BAD_SHAPE;
    if (!gates_in && n_cap > 0) {
      if (!reps_cache) return HLA_ERR_NULL_ARG;
      if (n_rep < 1) return HLA_ERR_BAD_SHAPE;
    }
    if (std::isnan(tau)) return HLA_ERR_BAD_SHAPE;
  }
  if (!all_aligned(S_cur, At_cur, At_cache, Bc_cache, reps_cache) || !all_aligned4(q, k, v, gates_in, o, gates_out))
    return HLA_ERR_ALIGN;
  return HLA_OK;
}

hla_status_t hla_gdn_decode(int64_t Bs, int64_t H, int32_t dk, int32_t dv, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* beta, const float* alpha, float* S_cur,
                            float* At_cur, void* At_cache, void* Bc_cache, const void* reps_cache, int32_t n_rep,
                            int32_t* n_cache, int32_t n_cap, const float* gates_in, float tau, float* o,
                            float* gates_out, int32_t commit, hipStream_t stream) {
  hla_status_t st = decode_checks(Bs, H, dk, dv, dtype, q, k, v, S_cur, At_cur, At_cache, Bc_cache, reps_cache, n_rep,
                                  n_cache, n_cap, gates_in, tau, o, gates_out, commit);
  if (st != HLA_OK) return st;
  if (!beta || !alpha) return HLA_ERR_NULL_ARG;
  if (!all_aligned4(beta, alpha)) return HLA_ERR_ALIGN;
  hla::DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.alpha = alpha; a.S_cur = S_cur; a.At_cur = At_cur;
  a.At_cache = At_cache; a.Bc_cache = Bc_cache; a.reps_cache = reps_cache; a.n_rep = n_rep; a.n_cache = n_cache;
  a.n_cap = n_cap; a.gates_in = gates_in; a.tau = tau; a.o = o; a.gates_out = gates_out; a.commit = commit;
  a.Bs = Bs; a.H = H;
  return hip_status(hla::launch_decode(a, dtype, dk, dv, stream));
}

hla_status_t hla_gdn2_decode(int64_t Bs, int64_t H, int32_t dk, int32_t dv, int32_t dtype, const void* q,
                             const void* k, const void* v, const float* a_decay, const float* b_erase,
                             const float* w_write, float* S_cur, float* At_cur, void* At_cache, void* Bc_cache,
                             const void* reps_cache, int32_t n_rep, int32_t* n_cache, int32_t n_cap,
                             const float* gates_in, float tau, float* o, float* gates_out, int32_t commit,
                             hipStream_t stream) {
  hla_status_t st = decode_checks(Bs, H, dk, dv, dtype, q, k, v, S_cur, At_cur, At_cache, Bc_cache, reps_cache, n_rep,
                                  n_cache, n_cap, gates_in, tau, o, gates_out, commit);
  if (st != HLA_OK) return st;
  if (!a_decay || !b_erase || !w_write) return HLA_ERR_NULL_ARG;
  if (!all_aligned4(a_decay, b_erase, w_write)) return HLA_ERR_ALIGN;
  hla::DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.ga = a_decay; a.gb = b_erase; a.gw = w_write; a.variant = 2;
  a.S_cur = S_cur; a.At_cur = At_cur;
  a.At_cache = At_cache; a.Bc_cache = Bc_cache; a.reps_cache = reps_cache; a.n_rep = n_rep; a.n_cache = n_cache;
  a.n_cap = n_cap; a.gates_in = gates_in; a.tau = tau; a.o = o; a.gates_out = gates_out; a.commit = commit;
  a.Bs = Bs; a.H = H;
  return hip_status(hla::launch_decode(a, dtype, dk, dv, stream));
}

}  // extern "C"
