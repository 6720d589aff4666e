// Backward of the gated composition: gradients of the routed states w.r.t. the chunk maps,
// the gates and the initial state.
//
// [HLA] Methodology paragraphs 1, 3 and 4: query chunk i starts from S0 and applies, in
// time order, each active history chunk j < i interpolated with the identity.  In the
// stored orientation (M = S^T [dk, dv], At = A^T, Bc = B^T) one step is
//     M_j = M_{j-1} + g (At_j - I) M_{j-1} + g Bc_j,     g = g_ij.
// With lambda_j = dL/dM_j (lambda of the last step = the upstream gradient of S~_i), the
// reverse of one step is
//     dBc_j += g lambda_j,   dAt_j += g lambda_j M_{j-1}^T,
//     dg_ij  = <lambda_j, (At_j - I) M_{j-1} + Bc_j>,
//     lambda_{j-1} = lambda_j + g (At_j - I)^T lambda_j,
// and dS0 sums the final lambda of every chain.  Skipped pairs pass lambda through.
//
// Memory: the sums over the query chunks in pass 3 need, per pair (i, j), the state in front
// of the step and g lambda_j, so the history steps are cut into segments of K consecutive
// steps and run one segment at a time, last to first.  A segment's pairs are at most
// K (N - 1) per (b, h) instead of N (N - 1) / 2; every chain's state at each segment start
// comes from a checkpoint kept by one forward replay, and each chain's lambda is carried from
// one segment to the one before it.  With K = N there is one segment and no checkpoint.
//
// Passes (one chain per workgroup in 1 and 2, one wave per 32 state columns):
//   0. prep_bwd_kernel writes (At_j - I) and its transpose with every 16-wide k block in the
//      order the MFMA fragments read it (one 16-byte load per fragment), and Bc_j in the
//      accumulator's lane order; with more than one segment compose_replay_kernel<.., true>
//      then runs every chain forward and keeps its state at each segment boundary it crosses;
//   per segment [j0, j1), last first:
//   1. compose_replay_kernel<.., false> runs each chain's steps of the segment from its
//      checkpoint (one chain per workgroup; the step's (At_j - I) staged in LDS and shared by
//      the column waves, the next one loaded while the current one is multiplied): per
//      active step it forms D_j = (At_j - I) M_{j-1} + Bc_j on the matrix cores, stores
//      M_{j-1} (row-major, for pass 3) and D_j (in the accumulator's lane order, for pass 2),
//      and sets M += g D_j;
//   2. compose_adjoint_kernel runs each chain's steps of the segment backward: per active
//      step it stores g lambda_j, takes the gate gradient <lambda_j, D_j> (per wave, summed
//      over its 32 columns) and updates lambda += (At_j - I)^T (g lambda) on the matrix cores;
//   3. compose_grad_reduce_kernel, one workgroup per step j of the segment, sums over the
//      query chunks i > j: dAt_j = sum_i (g lambda)_i M_i^T on the matrix cores, dBc_j =
//      sum_i (g lambda)_i, and the gate gradients of column j;
//   4. chain_sum_kernel: dS0 = sum over chains of the final lambda.
// Every reduction runs in a fixed order (no atomics): results are deterministic.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Slot of pair (i, j), j in the segment [j0, j1) (per (b, h)): the pairs of the chains before
// chain i come first, chain i' > j0 having min(j1, i') - j0 of them.
__device__ __forceinline__ int64_t pair_slot(const ComposeBwdArgs& a, int i, int j) {
  const int64_t m = (int64_t)i - 1 - a.j0, L = a.j1 - a.j0;
  const int64_t base = m <= 0 ? 0 : (i - 1 <= a.j1 ? m * (m + 1) / 2 : L * (L + 1) / 2 + ((int64_t)i - 1 - a.j1) * L);
  return base + (j - a.j0);
}

__device__ __forceinline__ int64_t ckpt_index(const ComposeBwdArgs& a, int b, int i) { return ckpt_slot(a.N, a.K, b, i); }

// Offset of element e of lane `lane` in the accumulator-lane-order image of one dk x dv
// matrix: [dv/32 column tiles][dk/32 row tiles][64 lanes][16].
template <int DK>
__device__ __forceinline__ int64_t lane_off(int ct, int rt, int lane) {
  return ((int64_t)(ct * (DK / 32) + rt) * 64 + lane) * 16;
}

// 16 values of one accumulator tile in the lane's order, in T.  bf16 pieces go out as
// non-temporal stores: whole 16-byte pieces of a stream far larger than the caches.
template <class T>
__device__ __forceinline__ void store16(T* dst, const f32x16& v, float scale) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = (bf16)(v[e] * scale);
      hi[e] = (bf16)(v[e + 8] * scale);
    }
    __builtin_nontemporal_store(lo, reinterpret_cast<bf16x8*>(dst));
    __builtin_nontemporal_store(hi, reinterpret_cast<bf16x8*>(dst + 8));
  } else {
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(v[e] * scale, v[e + 1] * scale, v[e + 2] * scale, v[e + 3] * scale);
  }
}
template <class T>
__device__ __forceinline__ f32x16 load16(const T* src) {
  f32x16 v;
  if constexpr (sizeof(T) == 2) {
    const bf16x8 lo = *reinterpret_cast<const bf16x8*>(src), hi = *reinterpret_cast<const bf16x8*>(src + 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)lo[e];
      v[e + 8] = (float)hi[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 f = *reinterpret_cast<const float4*>(src + e);
      v[e] = f.x; v[e + 1] = f.y; v[e + 2] = f.z; v[e + 3] = f.w;
    }
  }
  return v;
}

// Position of k within its 16-wide block in the prepared bf16 image: slots 0-3 hold k 0-3,
// 4-7 hold k 8-11, 8-11 hold k 4-7 and 12-15 hold k 12-15 (the clayout order of the two
// lane halves).
__device__ __forceinline__ int prep_pos(int k) {
  const int b = k & ~15, r = k & 15;
  const int q = r >> 2;
  const int qp = q == 1 ? 2 : q == 2 ? 1 : q;
  return b + qp * 4 + (r & 3);
}

}  // namespace

// Pass 0: (At - I) and (At - I)^T in the fragment order, and Bc in the lane order.  One
// thread per (chunk, row m, 16-wide k block) for the two At images; consecutive threads
// take consecutive m, so the transposed reads are coalesced.
template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void prep_bwd_kernel(ComposeBwdArgs a, int64_t n_chunks) {
  const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
  constexpr int KB = DK / 16;
  const int64_t n_at = n_chunks * KB * DK;
  if (t < n_at) {
    const int m = (int)(t % DK);
    const int kb = (int)((t / DK) % KB);
    const int64_t chunk = t / ((int64_t)DK * KB);
    const T* X = reinterpret_cast<const T*>(a.At) + chunk * DK * DK;
    // the 16 values of this block, row m of (At - I) and of its transpose, placed in the
    // fragment order in registers, then written as whole 16-byte pieces
    alignas(16) T vp[16];
    alignas(16) T vt[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = kb * 16 + r;
      const int pos = sizeof(T) == 2 ? prep_pos(k) - kb * 16 : r;
      const float d = (k == m) ? 1.f : 0.f;
      vp[pos] = from_f<T>(to_f<T>(X[(int64_t)m * DK + k]) - d);
      vt[pos] = from_f<T>(to_f<T>(X[(int64_t)k * DK + m]) - d);
    }
    u32x4* P = reinterpret_cast<u32x4*>(reinterpret_cast<T*>(a.Ap) + chunk * DK * DK + (int64_t)m * DK + kb * 16);
    u32x4* PT = reinterpret_cast<u32x4*>(reinterpret_cast<T*>(a.ApT) + chunk * DK * DK + (int64_t)m * DK + kb * 16);
    constexpr int NP = 16 * (int)sizeof(T) / 16;
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      P[c] = reinterpret_cast<const u32x4*>(vp)[c];
      PT[c] = reinterpret_cast<const u32x4*>(vt)[c];
    }
    return;
  }
  const int64_t u = t - n_at;  // Bc: one thread per (chunk, column tile, row tile, lane)
  constexpr int NRT = DK / 32, NCT = DV / 32;
  if (u >= n_chunks * NCT * NRT * 64) return;
  const int lane = (int)(u % 64), rt = (int)((u / 64) % NRT), ct = (int)((u / (64 * NRT)) % NCT);
  const int64_t chunk = u / (64 * NRT * NCT);
  const int hh = lane >> 5, c32 = lane & 31;
  const T* B = reinterpret_cast<const T*>(a.Bc) + chunk * DK * DV;
  f32x16 v;
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = to_f<T>(B[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + ct * 32 + c32]);
  store16<T>(reinterpret_cast<T*>(a.Bl) + chunk * DK * DV + lane_off<DK>(ct, rt, lane), v, 1.f);
}

// (At - I) images of one history chunk staged in LDS, shared by the workgroup's waves: rows
// padded by 16 bytes so that a 16-lane read phase of fragment rows hits distinct banks.
template <class T, int DK>
struct StagedA {
  static constexpr int PAD = 16 / (int)sizeof(T), PP = DK + PAD;  // row pitch (elements)
  static constexpr int BYTES = DK * PP * (int)sizeof(T);
};

template <class T, int DK>
__device__ __forceinline__ typename Mma<T>::Frag lds_frag(const T* sA, int rt, int ks, int hh, int c32) {
  const T* row = sA + (rt * 32 + c32) * StagedA<T, DK>::PP;
  if constexpr (sizeof(T) == 2)
    return *reinterpret_cast<const bf16x8*>(row + ks * 16 + hh * 8);
  else
    return Mma<T>::load_clayout(row, ks, hh);
}

// Copy of one prepared (At - I) image (global, rows of DK elements) into registers, then into
// padded LDS rows: NCP 16-byte pieces per thread.
template <class T, int DK, int NTH>
struct AStage {
  static constexpr int EPP = 16 / (int)sizeof(T);  // elements per 16-byte piece
  static constexpr int NCP = DK * DK / EPP / NTH;
  static_assert(NCP * EPP * NTH == DK * DK, "pieces split evenly");
};
template <class T, int DK, int NTH, int NC>
__device__ __forceinline__ void stage_load(u32x4 (&r)[NC], const T* src, int tid) {
  static_assert(NC == AStage<T, DK, NTH>::NCP, "piece count");
#pragma unroll
  for (int c = 0; c < NC; ++c) r[c] = reinterpret_cast<const u32x4*>(src)[tid + c * NTH];
}
template <class T, int DK, int NTH, int NC>
__device__ __forceinline__ void stage_store(const u32x4 (&r)[NC], T* sA, int tid) {
  constexpr int EPP = AStage<T, DK, NTH>::EPP;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e0 = (tid + c * NTH) * EPP;
    *reinterpret_cast<u32x4*>(sA + (e0 / DK) * StagedA<T, DK>::PP + e0 % DK) = r[c];
  }
}

// Passes 0 and 1: forward over each chain.  CK: every step of the chain, keeping the state in
// front of each segment boundary it crosses; else the steps of the current segment, from the
// chain's checkpoint, storing M_{j-1} and D_j of each active step.  One chain per workgroup:
// (At_j - I) of the next active step is loaded into registers while the current one is
// multiplied from LDS, then written to the other LDS buffer.
template <class T, int DK, int DV, bool CK>
__global__ __launch_bounds__(DV / 32 * 64) void compose_replay_kernel(ComposeBwdArgs a) {
  using MM = Mma<T>;
  constexpr int NRT = DK / 32, NKS = DK / MM::KS, KPT = 32 / MM::KS, NTH = DV / 32 * 64;
  __shared__ __attribute__((aligned(16))) char smem[2 * StagedA<T, DK>::BYTES];
  auto sbuf = [&](int b) { return reinterpret_cast<T*>(smem + b * StagedA<T, DK>::BYTES); };
  const int tid = threadIdx.x, lane = tid & 63, ct = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int N = a.N;
  const int i = N - 1 - (int)(blockIdx.x / BH);  // longest chains first
  const int jb = CK ? 0 : a.j0, je = CK ? i : (a.j1 < i ? a.j1 : i);  // the steps [jb, je)
  const int col = ct * 32 + c32;
  T* Ms = reinterpret_cast<T*>(a.Msave) + bh * a.slots * DK * DV;
  T* Ds = reinterpret_cast<T*>(a.Dsave) + bh * a.slots * DK * DV;
  float* Ck = a.Ckpt + bh * a.nck * DK * DV;
  const T* Apb = reinterpret_cast<const T*>(a.Ap) + bh * N * (int64_t)DK * DK;
  const T* Blb = reinterpret_cast<const T*>(a.Bl) + bh * N * (int64_t)DK * DV;
  const uint8_t* mrow = a.mask + (bh * N + i) * (int64_t)N;
  const float* grow = a.gates + (bh * N + i) * (int64_t)N;

  f32x16 M[NRT];
  if (jb > 0) {  // from the chain's checkpoint at the segment start
    const float* ck = Ck + ckpt_index(a, jb / a.K, i) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) M[rt] = load16<float>(ck + lane_off<DK>(ct, rt, lane));
  } else {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        M[rt][e] = a.S0 ? a.S0[bh * DK * DV + (int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] : 0.f;
  }
  // CK: the state in front of boundaries nb K .. up to step `upto` (boundaries below i only)
  int nb = 1;
  auto keep = [&](int upto) {
    for (; nb * a.K <= upto && nb * a.K < i; ++nb) {
      float* ck = Ck + ckpt_index(a, nb, i) * DK * DV;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) store16<float>(ck + lane_off<DK>(ct, rt, lane), M[rt], 1.f);
    }
  };

  auto next_active = [&](int j) {
    while (j < je && !mrow[j]) ++j;
    return j;
  };
  u32x4 pre[AStage<T, DK, NTH>::NCP];
  int j = next_active(jb);
  int buf = 0;
  if (j < je) {
    stage_load<T, DK, NTH>(pre, Apb + (int64_t)j * DK * DK, tid);
    stage_store<T, DK, NTH>(pre, sbuf(0), tid);
    __syncthreads();
  }
  while (j < je) {
    const int jn = next_active(j + 1);
    if (jn < je) stage_load<T, DK, NTH>(pre, Apb + (int64_t)jn * DK * DK, tid);
    const float g = grow[j];
    if constexpr (CK) {
      keep(j);
    } else {
      // the opaque lane offset keeps the compiler from holding 64 store addresses in
      // registers across the whole chain
      int lofs = hh * 4 * DV + col;
      asm volatile("" : "+v"(lofs));
      T* dst = Ms + pair_slot(a, i, j) * DK * DV + lofs;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[(rt * 32 + (e >> 2) * 8 + (e & 3)) * DV] = from_f<T>(M[rt][e]);
    }
    typename MM::Frag bf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bf[ks] = MM::from_acc(M[ks / KPT], ks, 1.f);
    const T* sA = sbuf(buf);
    const T* Bl = Blb + (int64_t)j * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x16 D = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) D = MM::mma(lds_frag<T, DK>(sA, rt, ks, hh, c32), bf[ks], D);
      const f32x16 b = load16<T>(Bl + lane_off<DK>(ct, rt, lane));
#pragma unroll
      for (int e = 0; e < 16; ++e) D[e] += b[e];
      if constexpr (!CK) store16<T>(Ds + pair_slot(a, i, j) * DK * DV + lane_off<DK>(ct, rt, lane), D, 1.f);
#pragma unroll
      for (int e = 0; e < 16; ++e) M[rt][e] = fmaf(g, D[e], M[rt][e]);
    }
    if (jn < je) stage_store<T, DK, NTH>(pre, sbuf(buf ^ 1), tid);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }
  if constexpr (CK) keep(i - 1);
  if (a.S_routed && je == i) {
    float* so = a.S_routed + (bh * N + i) * (int64_t)DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) so[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] = M[rt][e];
  }
}

// Pass 2: backward over each chain's steps of the segment, staged like pass 1 with
// (At_j - I)^T.  D_j of the next active step is loaded into registers (raw, in the storage
// type) during the current one, so the gate gradient <lambda_j, D_j> can be taken before the
// products and lambda can be updated in place.
template <class T, int DK, int DV>
__global__ __launch_bounds__(DV / 32 * 64) void compose_adjoint_kernel(ComposeBwdArgs a) {
  using MM = Mma<T>;
  constexpr int NRT = DK / 32, NKS = DK / MM::KS, KPT = 32 / MM::KS, NCT = DV / 32, NTH = NCT * 64;
  constexpr int DPC = 16 * (int)sizeof(T) / 16;  // 16-byte pieces of one lane's tile values
  __shared__ __attribute__((aligned(16))) char smem[2 * StagedA<T, DK>::BYTES];
  auto sbuf = [&](int b) { return reinterpret_cast<T*>(smem + b * StagedA<T, DK>::BYTES); };
  const int tid = threadIdx.x, lane = tid & 63, ct = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int N = a.N;
  const int i = N - 1 - (int)(blockIdx.x / BH);
  const int jt = a.j1 < i ? a.j1 : i;  // the chain's steps [j0, jt) in this segment
  const int col = ct * 32 + c32;
  const T* ATb = reinterpret_cast<const T*>(a.ApT) + bh * N * (int64_t)DK * DK;
  const T* Ds = reinterpret_cast<const T*>(a.Dsave) + bh * a.slots * DK * DV;
  T* Ls = reinterpret_cast<T*>(a.Lsave) + bh * a.slots * DK * DV;
  const uint8_t* mrow = a.mask + (bh * N + i) * (int64_t)N;
  const float* grow = a.gates + (bh * N + i) * (int64_t)N;

  // lambda after the segment's last step of the chain: the upstream gradient in the segment
  // that holds the chain's last step, else as the later segment left it
  f32x16 lam[NRT];
  float* le = a.lam_end + (bh * N + i) * (int64_t)DK * DV;
  const float* l0 = i <= a.j1 ? a.dS + (bh * N + i) * (int64_t)DK * DV : le;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) lam[rt][e] = l0[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col];

  auto prev_active = [&](int j) {
    while (j >= a.j0 && !mrow[j]) --j;
    return j;
  };
  u32x4 pre[AStage<T, DK, NTH>::NCP];
  u32x4 dcur[NRT][DPC], dnext[NRT][DPC];
  auto load_d = [&](u32x4 (&dst)[NRT][DPC], int j) {
    const T* dd = Ds + pair_slot(a, i, j) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int c = 0; c < DPC; ++c) dst[rt][c] = reinterpret_cast<const u32x4*>(dd + lane_off<DK>(ct, rt, lane))[c];
  };
  int j = prev_active(jt - 1);
  int buf = 0;
  if (j >= a.j0) {
    stage_load<T, DK, NTH>(pre, ATb + (int64_t)j * DK * DK, tid);
    load_d(dcur, j);
    stage_store<T, DK, NTH>(pre, sbuf(0), tid);
    __syncthreads();
  }
  while (j >= a.j0) {
    const int jn = prev_active(j - 1);
    if (jn >= a.j0) {
      stage_load<T, DK, NTH>(pre, ATb + (int64_t)jn * DK * DK, tid);
      load_d(dnext, jn);
    }
    const float g = grow[j];
    // gate gradient <lambda_j, D_j>, this wave's 32 columns
    float part = 0.f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const T* dv = reinterpret_cast<const T*>(dcur[rt]);
#pragma unroll
      for (int e = 0; e < 16; ++e) part = fmaf(lam[rt][e], to_f<T>(dv[e]), part);
    }
    int lofs = hh * 4 * DV + col;  // opaque: see compose_save_kernel
    asm volatile("" : "+v"(lofs));
    T* ld = Ls + pair_slot(a, i, j) * DK * DV + lofs;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) ld[(rt * 32 + (e >> 2) * 8 + (e & 3)) * DV] = from_f<T>(g * lam[rt][e]);
    // lambda += (At_j - I)^T (g lambda), accumulated in place
    typename MM::Frag bf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bf[ks] = MM::from_acc(lam[ks / KPT], ks, g);
    const T* sA = sbuf(buf);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) lam[rt] = MM::mma(lds_frag<T, DK>(sA, rt, ks, hh, c32), bf[ks], lam[rt]);
    part = wave_sum(part);
    if (lane == 0) a.dgp[((bh * N + i) * N + j) * NCT + ct] = part;
    if (jn >= a.j0) {
      stage_store<T, DK, NTH>(pre, sbuf(buf ^ 1), tid);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int c = 0; c < DPC; ++c) dcur[rt][c] = dnext[rt][c];
    }
    __syncthreads();
    buf ^= 1;
    j = jn;
  }
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) le[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] = lam[rt][e];
}

// Pass 3: per history chunk j of the segment, the sums over the query chunks that keep it.  Each active
// chain's g lambda and M (row-major) are staged in padded LDS rows shared by the four
// waves; the next active chain's are loaded into registers while the current ones are
// multiplied, and dBc_j accumulates straight from those registers.
template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void compose_grad_reduce_kernel(ComposeBwdArgs a) {
  using MM = Mma<T>;
  constexpr int NRT = DK / 32, NTILE = NRT * NRT, TPW = NTILE / 4, NKS = DV / MM::KS, NCT = DV / 32;
  static_assert(NTILE % 4 == 0, "four waves share the dAt tiles");
  constexpr int EPP = 16 / (int)sizeof(T), PP = DV + EPP;  // elements per piece, LDS row pitch
  constexpr int NPC = DK * DV / EPP / 256;                  // 16-byte pieces per thread and matrix
  static_assert(NPC * EPP * 256 == DK * DV, "pieces split evenly");
  __shared__ __attribute__((aligned(16))) T sL[DK * PP];
  __shared__ __attribute__((aligned(16))) T sM[DK * PP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int j = a.j0 + (int)(blockIdx.x / BH);  // most query chunks first
  const int N = a.N;
  const T* Ms = reinterpret_cast<const T*>(a.Msave) + bh * a.slots * DK * DV;
  const T* Ls = reinterpret_cast<const T*>(a.Lsave) + bh * a.slots * DK * DV;
  auto active = [&](int i) { return a.mask[(bh * N + i) * (int64_t)N + j] != 0; };
  auto next_active = [&](int i) {
    while (i < N && !active(i)) ++i;
    return i;
  };

  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero16();
  float sb[NPC][EPP];
#pragma unroll
  for (int c = 0; c < NPC; ++c)
#pragma unroll
    for (int e = 0; e < EPP; ++e) sb[c][e] = 0.f;
  u32x4 preL[NPC], preM[NPC];
  auto prefetch = [&](int i) {
    const int64_t p = pair_slot(a, i, j);
    const u32x4* L = reinterpret_cast<const u32x4*>(Ls + p * DK * DV);
    const u32x4* Mi = reinterpret_cast<const u32x4*>(Ms + p * DK * DV);
    // the last read of a pair's states: non-temporal loads, which leave the caches to data read again
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
      preL[c] = __builtin_nontemporal_load(L + tid + c * 256);
      preM[c] = __builtin_nontemporal_load(Mi + tid + c * 256);
    }
  };

  int i = next_active(j + 1);
  if (i < N) prefetch(i);
  while (i < N) {
    __syncthreads();  // the previous chain's LDS reads are done
#pragma unroll
    for (int c = 0; c < NPC; ++c) {
      const int e0 = (tid + c * 256) * EPP;
      *reinterpret_cast<u32x4*>(sL + (e0 / DV) * PP + e0 % DV) = preL[c];
      *reinterpret_cast<u32x4*>(sM + (e0 / DV) * PP + e0 % DV) = preM[c];
      const T* v = reinterpret_cast<const T*>(&preL[c]);
#pragma unroll
      for (int e = 0; e < EPP; ++e) sb[c][e] += to_f<T>(v[e]);
    }
    __syncthreads();
    const int in = next_active(i + 1);
    if (in < N) prefetch(in);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = w * TPW + u, rt = t / NRT, st = t % NRT;
      const T* ar = sL + (rt * 32 + c32) * PP;
      const T* br = sM + (st * 32 + c32) * PP;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[u] = MM::mma(MM::load_plain(ar, ks, hh), MM::load_plain(br, ks, hh), acc[u]);
    }
    i = in;
  }
  float* dA = a.dAt + (bh * N + j) * (int64_t)DK * DK;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = w * TPW + u, rt = t / NRT, st = t % NRT;
#pragma unroll
    for (int e = 0; e < 16; ++e) dA[(int64_t)(rt * 32 + acc_row(e, hh)) * DK + st * 32 + c32] = acc[u][e];
  }
  float* dB = a.dBc + (bh * N + j) * (int64_t)DK * DV;
#pragma unroll
  for (int c = 0; c < NPC; ++c) {
    const int64_t e0 = (int64_t)(tid + c * 256) * EPP;
#pragma unroll
    for (int e = 0; e < EPP; ++e) dB[e0 + e] = sb[c][e];
  }
  // gate gradients of column j (zero for skipped, diagonal and future pairs)
  for (int ii = tid; ii < N; ii += 256) {
    const int64_t o = (bh * N + ii) * N + j;
    float sg = 0.f;
    if (ii > j && a.mask[o]) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) sg += a.dgp[o * NCT + c];
    }
    a.dgates[o] = sg;
  }
}

// Pass 4: dS0 = sum over the chains of their final lambda.
__global__ __launch_bounds__(256) void chain_sum_kernel(const float* __restrict__ lam_end, float* __restrict__ dS0,
                                                        int32_t N, int64_t per_bh, int64_t total) {
  const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (t >= total) return;
  const int64_t bh = t / per_bh, e = t % per_bh;
  const float* src = lam_end + bh * N * per_bh + e;
  float s = 0.f;
  for (int i = 0; i < N; ++i) s += src[(int64_t)i * per_bh];
  dS0[t] = s;
}

template <class T, int DK, int DV>
static hipError_t launch_compose_bwd_t(const ComposeBwdArgs& a, int stages, hipStream_t s) {
  const int64_t BH = a.B * a.H, BHN = BH * a.N;
  const int lo = a.j0 == 0 ? 0 : a.j0 + 1;  // the segment's chains: i > j0 (and chain 0 in the first)
  const int64_t BHC = BH * (a.N - lo), BHJ = BH * (a.j1 - a.j0);
  if (stages & kComposeBwdPrep) {
    TimedLaunch tl(HLA_KERNEL_BWD_SAVE, s);
    const int64_t nt = BHN * (DK / 16) * DK + BHN * (DV / 32) * (DK / 32) * 64;
    hipLaunchKernelGGL((prep_bwd_kernel<T, DK, DV>), dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, a, BHN);
    if (a.K < a.N && !a.ckpt_done)  // the checkpoints of more than one segment
      hipLaunchKernelGGL((compose_replay_kernel<T, DK, DV, true>), dim3((unsigned)BHN), dim3(DV / 32 * 64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (stages & kComposeBwdSave) {
    TimedLaunch tl(HLA_KERNEL_BWD_SAVE, s);
    if (BHC > 0)
      hipLaunchKernelGGL((compose_replay_kernel<T, DK, DV, false>), dim3((unsigned)BHC), dim3(DV / 32 * 64), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (stages & kComposeBwdReverse) {
    {
      TimedLaunch tl(HLA_KERNEL_BWD_ADJOINT, s);
      if (BHC > 0)
        hipLaunchKernelGGL((compose_adjoint_kernel<T, DK, DV>), dim3((unsigned)BHC), dim3(DV / 32 * 64), 0, s, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    TimedLaunch tl(HLA_KERNEL_BWD_REDUCE, s);
    if (BHJ > 0)
      hipLaunchKernelGGL((compose_grad_reduce_kernel<T, DK, DV>), dim3((unsigned)BHJ), dim3(256), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((stages & kComposeBwdFinish) && a.dS0) {
    TimedLaunch tl(HLA_KERNEL_BWD_REDUCE, s);
    const int64_t per = (int64_t)DK * DV, total = BH * per;
    hipLaunchKernelGGL(chain_sum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a.lam_end, a.dS0,
                       a.N, per, total);
  }
  return hipGetLastError();
}

template <class T>
static hipError_t launch_compose_bwd_d(const ComposeBwdArgs& a, int dk, int dv, int stages, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_compose_bwd_t<T, 64, 64>(a, stages, s);
  if (dk == 64 && dv == 128) return launch_compose_bwd_t<T, 64, 128>(a, stages, s);
  if (dk == 128 && dv == 64) return launch_compose_bwd_t<T, 128, 64>(a, stages, s);
  return launch_compose_bwd_t<T, 128, 128>(a, stages, s);
}

hipError_t launch_compose_backward(const ComposeBwdArgs& a, int dtype, int dk, int dv, int stages, hipStream_t s) {
  return dtype == 1 ? launch_compose_bwd_d<bf16>(a, dk, dv, stages, s)
                    : launch_compose_bwd_d<float>(a, dk, dv, stages, s);
}

}  // namespace hla
