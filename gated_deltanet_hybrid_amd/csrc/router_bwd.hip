// Backward of the HLA router gates (C = 64; the raw keys, n_rep = 64, or learned
// representatives, n_rep of them per chunk).
//
// [HLA] Overview and Methodology paragraph 2: qbar_i = mean of q over query chunk i,
// s_ijr = qbar_i . r_{j n_rep + r} / sqrt(dk) over history chunk j's representatives,
// l_ij = log-mean-exp over r of s_ijr, g_ij = sigmoid(l_ij).  Given dg_ij (zero for skipped
// pairs):
//     dl_ij = dg_ij g_ij (1 - g_ij),   p_ijr = softmax over r of s_ijr,
//     dqbar_i  = sum_{j<i} dl_ij sum_r p_ijr r_{j n_rep + r} / sqrt(dk),
//     dr_{j n_rep + r} = sum_{i>j} dl_ij p_ijr qbar_i / sqrt(dk),
// and every token of chunk i receives dqbar_i / n_i (added by the chunk backward's
// finalize pass, or written per token here).
//
// Lane r owns representative r of a history chunk (lanes r >= n_rep take no part), so the
// softmax over a chunk's representatives is a wave reduction.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

// Query-chunk side: qbar_i, then dqbar_i.  A workgroup takes 4 consecutive query chunks,
// one per wave; the keys of each history chunk j are staged once in LDS rows padded by 16
// bytes (row r read by lane r in 16-byte pieces, so each 16-lane phase hits distinct
// banks) and the next chunk's keys are loaded into registers while the current ones are
// used.
constexpr int kRouterQG = 4;

// q . k over DK with eight independent partial sums (no long dependent chain); k is a
// 16-byte aligned LDS row, q a per-wave (LDS) or wave-uniform (global) vector.
template <int DK>
__device__ __forceinline__ float dot_rows(const float* q, const float* k) {
  float p[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) p[u] = 0.f;
#pragma unroll
  for (int e = 0; e < DK; e += 8) {
    const float4 k0 = *reinterpret_cast<const float4*>(k + e), k1 = *reinterpret_cast<const float4*>(k + e + 4);
    p[0] = fmaf(q[e], k0.x, p[0]);
    p[1] = fmaf(q[e + 1], k0.y, p[1]);
    p[2] = fmaf(q[e + 2], k0.z, p[2]);
    p[3] = fmaf(q[e + 3], k0.w, p[3]);
    p[4] = fmaf(q[e + 4], k1.x, p[4]);
    p[5] = fmaf(q[e + 5], k1.y, p[5]);
    p[6] = fmaf(q[e + 6], k1.z, p[6]);
    p[7] = fmaf(q[e + 7], k1.w, p[7]);
  }
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

template <class T, int DK>
__global__ __launch_bounds__(64 * kRouterQG) void router_dq_kernel(RouterBwdArgs a) {
  constexpr int C = kChunk, QG = kRouterQG, NTH = 64 * QG, PK = DK + 4;
  constexpr int EPP = 16 / (int)sizeof(T), UPR = DK / EPP, NU = C * UPR / NTH;  // 16-byte units
  static_assert(NU * NTH == C * UPR, "key staging split");
  __shared__ __attribute__((aligned(16))) float s_key[C * PK];
  __shared__ __attribute__((aligned(16))) float s_qb[QG][DK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ng = (a.N + QG - 1) / QG;
  const int64_t bh = blockIdx.x / ng;
  const int i0 = (ng - 1 - (int)(blockIdx.x % ng)) * QG;  // longest histories first
  const int i = i0 + w;
  const int64_t h = bh % a.H, b = bh / a.H;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.reps);
  const float rs = 1.f / sqrtf((float)DK);
  if (i < a.N) {
    const int64_t t0 = (int64_t)i * C;
    const int ni = (int)((a.T - t0) < C ? (a.T - t0) : C);
    for (int e = lane; e < DK; e += 64) {
      float sq = 0.f;
      for (int t = 0; t < ni; ++t) sq += to_f<T>(q[((b * a.ld_T + t0 + t) * a.H + h) * DK + e]);
      sq /= (float)ni;
      s_qb[w][e] = sq;
      a.qbar[(bh * a.N + i) * DK + e] = sq;
    }
  }
  const int jmax = (i0 + QG - 1 < a.N - 1 ? i0 + QG - 1 : a.N - 1);  // history chunks 0 .. jmax-1
  float acc[DK];
#pragma unroll
  for (int e = 0; e < DK; ++e) acc[e] = 0.f;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 pre[NU];
  // history chunk j's representative rows (every one exists: j < N - 1); rows r >= n_rep
  // are zero and take no part
  auto load_keys = [&](int j) {
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int u = tid + m * NTH, r = u / UPR, cu = u % UPR;
      pre[m] = u32x4{0u, 0u, 0u, 0u};
      if (r < a.n_rep)
        pre[m] = *reinterpret_cast<const u32x4*>(
            k + ((b * a.ld_R + (int64_t)j * a.n_rep + r) * a.H + h) * DK + cu * EPP);
    }
  };
  if (jmax > 0) load_keys(0);
  for (int j = 0; j < jmax; ++j) {
    __syncthreads();  // earlier reads of s_key (and the s_qb writes) are done
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int u = tid + m * NTH, r = u / UPR, cu = u % UPR;
      const T* v = reinterpret_cast<const T*>(&pre[m]);
#pragma unroll
      for (int e = 0; e < EPP; ++e) s_key[r * PK + cu * EPP + e] = to_f<T>(v[e]);
    }
    __syncthreads();
    if (j + 1 < jmax) load_keys(j + 1);
    if (i < a.N && j < i) {
      const int64_t o = (bh * a.N + i) * (int64_t)a.N + j;
      const float g = a.gates[o], dl = a.dgates[o] * g * (1.f - g);
      if (dl != 0.f) {  // uniform over the wave
        const float* kr = s_key + lane * PK;
        const float sc = lane < a.n_rep ? dot_rows<DK>(s_qb[w], kr) * rs : -INFINITY;
        const float mx = wave_max_valu(sc);
        const float p = __expf(sc - mx);
        const float cr = dl * (p / wave_sum_valu(p)) * rs;
#pragma unroll
        for (int e = 0; e < DK; e += 4) {
          const float4 kv = *reinterpret_cast<const float4*>(kr + e);
          acc[e] = fmaf(cr, kv.x, acc[e]);
          acc[e + 1] = fmaf(cr, kv.y, acc[e + 1]);
          acc[e + 2] = fmaf(cr, kv.z, acc[e + 2]);
          acc[e + 3] = fmaf(cr, kv.w, acc[e + 3]);
        }
      }
    }
  }
  if (i < a.N) {
    float* out = a.dqbar + (bh * a.N + i) * DK;
#pragma unroll
    for (int e = 0; e < DK; ++e) {
      const float v = wave_sum_valu(acc[e]);
      if (lane == (e & 63)) out[e] = v;
    }
  }
}

// Representative side: the gradient of every representative row of chunk j (zero for the
// last chunk, which no query chunk reads).  Lane r keeps row r's gradient; the query means
// (from router_dq_kernel) are wave-uniform loads, so a pair needs no barrier.
template <class T, int DK>
__global__ __launch_bounds__(64) void router_dk_kernel(RouterBwdArgs a) {
  constexpr int C = kChunk, PK = DK + 4;
  __shared__ __attribute__((aligned(16))) float s_key[C * PK];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / a.N;
  const int j = (int)(blockIdx.x % a.N);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t r0 = (int64_t)j * a.n_rep;  // first row of chunk j
  const int nj = (int)((a.R_out - r0) < a.n_rep ? (a.R_out - r0) : a.n_rep);  // its rows below R_out
  const T* k = reinterpret_cast<const T*>(a.reps);
  const float rs = 1.f / sqrtf((float)DK);
  const bool read = j + 1 < a.N;  // a history chunk: all n_rep rows exist
  for (int idx = lane; idx < C * DK; idx += 64) {
    const int r = idx / DK, e = idx % DK;
    s_key[r * PK + e] = (read && r < a.n_rep) ? to_f<T>(k[((b * a.ld_R + r0 + r) * a.H + h) * DK + e]) : 0.f;
  }
  __syncthreads();
  const float* kr = s_key + lane * PK;
  float acc[DK];
#pragma unroll
  for (int e = 0; e < DK; ++e) acc[e] = 0.f;
  for (int i = j + 1; i < a.N; ++i) {
    const int64_t o = (bh * a.N + i) * (int64_t)a.N + j;
    const float g = a.gates[o], dl = a.dgates[o] * g * (1.f - g);
    if (dl == 0.f) continue;  // uniform over the wave
    const float* qb = a.qbar + (bh * a.N + i) * DK;
    const float sc = lane < a.n_rep ? dot_rows<DK>(qb, kr) * rs : -INFINITY;
    const float mx = wave_max_valu(sc);
    const float p = __expf(sc - mx);
    const float cr = dl * (p / wave_sum_valu(p)) * rs;
#pragma unroll
    for (int e = 0; e < DK; ++e) acc[e] = fmaf(cr, qb[e], acc[e]);
  }
  if (lane < nj) {
    float* out = a.dreps + ((b * a.R_out + r0 + lane) * a.H + h) * DK;
#pragma unroll
    for (int e = 0; e < DK; ++e) out[e] = acc[e];
  }
}

// dqbar of each token's chunk over the chunk's token count, per token.
template <int DK>
__global__ __launch_bounds__(256) void router_spread_kernel(RouterBwdArgs a) {
  constexpr int C = kChunk;
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (id >= a.B * a.T * a.H * DK) return;
  const int e = (int)(id % DK);
  const int64_t bth = id / DK;
  const int64_t h = bth % a.H, bt = bth / a.H;
  const int64_t t = bt % a.T, b = bt / a.T;
  const int c = (int)(t / C);
  const int64_t t0 = (int64_t)c * C;
  const int nc = (int)((a.T - t0) < C ? (a.T - t0) : C);
  a.dq_tok[id] = a.dqbar[((b * a.H + h) * a.N + c) * DK + e] / (float)nc;
}

template <class T, int DK>
static hipError_t launch_router_bwd_t(const RouterBwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const unsigned nq = (unsigned)(BH * ((a.N + kRouterQG - 1) / kRouterQG)), nk = (unsigned)(BH * a.N);
  TimedLaunch tl(HLA_KERNEL_BWD_ROUTER, s);
  hipLaunchKernelGGL((router_dq_kernel<T, DK>), dim3(nq), dim3(64 * kRouterQG), 0, s, a);
  hipLaunchKernelGGL((router_dk_kernel<T, DK>), dim3(nk), dim3(64), 0, s, a);
  if (a.dq_tok) {
    const int64_t total = a.B * a.T * a.H * DK;
    hipLaunchKernelGGL((router_spread_kernel<DK>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_router_backward(const RouterBwdArgs& a, int dtype, int dk, hipStream_t s) {
  if (dtype == 1) return dk == 64 ? launch_router_bwd_t<bf16, 64>(a, s) : launch_router_bwd_t<bf16, 128>(a, s);
  return dk == 64 ? launch_router_bwd_t<float, 64>(a, s) : launch_router_bwd_t<float, 128>(a, s);
}

}  // namespace hla
