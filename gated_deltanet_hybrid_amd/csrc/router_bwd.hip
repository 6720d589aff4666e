// Backward of the HLA router gates (raw-key representatives, n_rep = C = 64).
//
// [HLA] Overview and Methodology paragraph 2: qbar_i = mean of q over query chunk i,
// s_ijr = qbar_i . k_{jC+r} / sqrt(dk) over history chunk j's keys, l_ij = log-mean-exp
// over r of s_ijr, g_ij = sigmoid(l_ij).  Given dg_ij (zero for skipped pairs):
//     dl_ij = dg_ij g_ij (1 - g_ij),   p_ijr = softmax over r of s_ijr,
//     dqbar_i  = sum_{j<i} dl_ij sum_r p_ijr k_{jC+r} / sqrt(dk),
//     dk_{jC+r} = sum_{i>j} dl_ij p_ijr qbar_i / sqrt(dk),
// and every token of chunk i receives dqbar_i / n_i (added by the chunk backward's
// finalize pass).
//
// One wavefront per (b, h, chunk); lane r owns key r of a history chunk, so the softmax
// over a chunk's 64 keys is a wave reduction.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

// Query-chunk side: qbar_i, then dqbar_i.
template <class T, int DK>
__global__ __launch_bounds__(64) void router_dq_kernel(RouterBwdArgs a) {
  constexpr int C = kChunk;
  __shared__ float s_qb[DK];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / a.N;
  const int i = (int)(blockIdx.x % a.N);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)i * C;
  const int ni = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const float rs = 1.f / sqrtf((float)DK);
  for (int e = lane; e < DK; e += 64) {
    float s = 0.f;
    for (int t = 0; t < ni; ++t) s += to_f<T>(q[((b * a.ld_T + t0 + t) * a.H + h) * DK + e]);
    s /= (float)ni;
    s_qb[e] = s;
    a.qbar[(bh * a.N + i) * DK + e] = s;
  }
  __syncthreads();
  float acc[DK];
#pragma unroll
  for (int e = 0; e < DK; ++e) acc[e] = 0.f;
  const float* gts = a.gates + (bh * a.N + i) * (int64_t)a.N;
  const float* dgs = a.dgates + (bh * a.N + i) * (int64_t)a.N;
  for (int j = 0; j < i; ++j) {
    const float g = gts[j], dg = dgs[j];
    const float dl = dg * g * (1.f - g);
    if (dl == 0.f) continue;  // uniform over the wave
    const T* kr = k + ((b * a.ld_T + (int64_t)j * C + lane) * a.H + h) * DK;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < DK; ++e) s = fmaf(s_qb[e], to_f<T>(kr[e]), s);
    s *= rs;
    const float m = wave_max(s);
    const float p = __expf(s - m);
    const float cr = dl * (p / wave_sum(p)) * rs;
#pragma unroll
    for (int e = 0; e < DK; ++e) acc[e] = fmaf(cr, to_f<T>(kr[e]), acc[e]);
  }
  float* out = a.dqbar + (bh * a.N + i) * DK;
#pragma unroll
  for (int e = 0; e < DK; ++e) {
    const float v = wave_sum(acc[e]);
    if (lane == (e & 63)) out[e] = v;
  }
}

// Key side: dk of every token of history chunk j (zero for the last chunk, which no query
// chunk reads).  Needs qbar from router_dq_kernel.
template <class T, int DK>
__global__ __launch_bounds__(64) void router_dk_kernel(RouterBwdArgs a) {
  constexpr int C = kChunk;
  __shared__ float s_key[C][DK + 1];
  __shared__ float s_qb[DK];
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x / a.N;
  const int j = (int)(blockIdx.x % a.N);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)j * C;
  const int nj = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const T* k = reinterpret_cast<const T*>(a.k);
  const float rs = 1.f / sqrtf((float)DK);
  for (int idx = lane; idx < C * DK; idx += 64) {
    const int r = idx / DK, e = idx % DK;
    s_key[r][e] = r < nj ? to_f<T>(k[((b * a.ld_T + t0 + r) * a.H + h) * DK + e]) : 0.f;
  }
  float acc[DK];
#pragma unroll
  for (int e = 0; e < DK; ++e) acc[e] = 0.f;
  for (int i = j + 1; i < a.N; ++i) {
    const int64_t o = (bh * a.N + i) * (int64_t)a.N + j;
    const float g = a.gates[o], dg = a.dgates[o];
    const float dl = dg * g * (1.f - g);
    if (dl == 0.f) continue;  // uniform over the wave
    __syncthreads();          // earlier reads of s_qb are done
    for (int e = lane; e < DK; e += 64) s_qb[e] = a.qbar[(bh * a.N + i) * DK + e];
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < DK; ++e) s = fmaf(s_qb[e], s_key[lane][e], s);
    s *= rs;
    const float m = wave_max(s);
    const float p = __expf(s - m);
    const float cr = dl * (p / wave_sum(p)) * rs;
#pragma unroll
    for (int e = 0; e < DK; ++e) acc[e] = fmaf(cr, s_qb[e], acc[e]);
  }
  if (lane < nj) {
    float* out = a.dk_router + ((b * a.T + t0 + lane) * a.H + h) * DK;
#pragma unroll
    for (int e = 0; e < DK; ++e) out[e] = acc[e];
  }
}

template <class T, int DK>
static hipError_t launch_router_bwd_t(const RouterBwdArgs& a, hipStream_t s) {
  const unsigned nb = (unsigned)(a.B * a.H * (int64_t)a.N);
  TimedLaunch tl(HLA_KERNEL_BWD_ROUTER, s);
  hipLaunchKernelGGL((router_dq_kernel<T, DK>), dim3(nb), dim3(64), 0, s, a);
  hipLaunchKernelGGL((router_dk_kernel<T, DK>), dim3(nb), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_router_backward(const RouterBwdArgs& a, int dtype, int dk, hipStream_t s) {
  if (dtype == 1) return dk == 64 ? launch_router_bwd_t<bf16, 64>(a, s) : launch_router_bwd_t<bf16, 128>(a, s);
  return dk == 64 ? launch_router_bwd_t<float, 64>(a, s) : launch_router_bwd_t<float, 128>(a, s);
}

}  // namespace hla
