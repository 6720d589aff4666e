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
// Passes (one chain per workgroup in the first two, one wave per 32 state columns):
//   1. compose_save_kernel runs every chain forward and stores the state in front of each
//      active step (M_{j-1}) in the workspace;
//   2. compose_adjoint_kernel runs every chain backward: per active step it stores
//      g lambda_j, forms Y = (At_j - I)^T lambda_j on the matrix cores, takes the gate
//      gradient as <Y, M_{j-1}> + <lambda_j, Bc_j> (per wave, summed over its 32 columns),
//      and updates lambda += g Y;
//   3. compose_grad_reduce_kernel, one workgroup per history chunk j, sums over the query
//      chunks i > j: dAt_j = sum_i (g lambda)_i M_i^T on the matrix cores, dBc_j = sum_i
//      (g lambda)_i, and the gate gradients of column j;
//   4. chain_sum_kernel: dS0 = sum over chains of the final lambda.
// Every reduction runs in a fixed order (no atomics): results are deterministic.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {

__device__ __forceinline__ int64_t pair_index(int i, int j) { return (int64_t)i * (i - 1) / 2 + j; }

// A fragment of (X - I) for row tile rt and k-step ks, X row-major [DK][DK], in the
// clayout k order that matches from_acc B fragments.
template <class T, int DK>
__device__ __forceinline__ typename Mma<T>::Frag minus_eye_frag(const T* X, int rt, int ks, int hh, int c32) {
  const int m = rt * 32 + c32;
  typename Mma<T>::Frag f = Mma<T>::load_clayout(X + (int64_t)m * DK, ks, hh);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (clayout_k<T>(ks, hh, e) == m) f[e] = (T)((float)f[e] - 1.f);
  } else {
    if (clayout_k<T>(ks, hh, 0) == m) f -= 1.f;
  }
  return f;
}

}  // namespace

// At^T of every chunk (plain transpose through LDS, 32 x 32 tiles).
template <class T, int DK>
__global__ __launch_bounds__(256) void transpose_at_kernel(const T* __restrict__ At, T* __restrict__ AtT) {
  __shared__ T tile[32][33];
  constexpr int NT = DK / 32;
  const int64_t chunk = blockIdx.x / (NT * NT);
  const int tr = (int)(blockIdx.x % (NT * NT)) / NT, tc = (int)(blockIdx.x % NT);
  const T* src = At + chunk * DK * DK;
  T* dst = AtT + chunk * DK * DK;
  const int x = threadIdx.x & 31, y0 = threadIdx.x >> 5;
  for (int y = y0; y < 32; y += 8) tile[y][x] = src[(int64_t)(tr * 32 + y) * DK + tc * 32 + x];
  __syncthreads();
  for (int y = y0; y < 32; y += 8) dst[(int64_t)(tc * 32 + y) * DK + tr * 32 + x] = tile[x][y];
}

// Pass 1: forward over every chain, storing M_{j-1} of each active step.
template <class T, int DK, int DV>
__global__ __launch_bounds__(DV / 32 * 64) void compose_save_kernel(ComposeBwdArgs a) {
  using MM = Mma<T>;
  constexpr int NRT = DK / 32, NKS = DK / MM::KS, KPT = 32 / MM::KS;
  const int lane = threadIdx.x & 63, ct = threadIdx.x >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int i = a.N - 1 - (int)(blockIdx.x / BH);  // longest chains first
  const int N = a.N;
  const int col = ct * 32 + c32;
  const int64_t P = (int64_t)N * (N - 1) / 2;
  const T* Ab = reinterpret_cast<const T*>(a.At) + bh * N * (int64_t)DK * DK;
  const T* Bb = reinterpret_cast<const T*>(a.Bc) + bh * N * (int64_t)DK * DV;
  T* Ms = reinterpret_cast<T*>(a.Msave) + bh * P * DK * DV;

  f32x16 M[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      M[rt][e] = a.S0 ? a.S0[bh * DK * DV + (int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] : 0.f;

  for (int j = 0; j < i; ++j) {
    const int64_t o = (bh * N + i) * N + j;
    if (!a.mask[o]) continue;
    const float g = a.gates[o];
    T* dst = Ms + pair_index(i, j) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] = from_f<T>(M[rt][e]);
    typename MM::Frag bf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bf[ks] = MM::from_acc(M[ks / KPT], ks, g);
    const T* X = Ab + (int64_t)j * DK * DK;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) M[rt] = MM::mma(minus_eye_frag<T, DK>(X, rt, ks, hh, c32), bf[ks], M[rt]);
    const T* Bj = Bb + (int64_t)j * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) M[rt][e] = fmaf(g, to_f<T>(Bj[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col]), M[rt][e]);
  }
  if (a.S_routed) {
    float* so = a.S_routed + (bh * N + i) * (int64_t)DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) so[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] = M[rt][e];
  }
}

// Pass 2: backward over every chain.
template <class T, int DK, int DV>
__global__ __launch_bounds__(DV / 32 * 64) void compose_adjoint_kernel(ComposeBwdArgs a) {
  using MM = Mma<T>;
  constexpr int NRT = DK / 32, NKS = DK / MM::KS, KPT = 32 / MM::KS, NCT = DV / 32;
  const int lane = threadIdx.x & 63, ct = threadIdx.x >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int i = a.N - 1 - (int)(blockIdx.x / BH);
  const int N = a.N;
  const int col = ct * 32 + c32;
  const int64_t P = (int64_t)N * (N - 1) / 2;
  const T* ATb = reinterpret_cast<const T*>(a.AtT) + bh * N * (int64_t)DK * DK;
  const T* Bb = reinterpret_cast<const T*>(a.Bc) + bh * N * (int64_t)DK * DV;
  const T* Ms = reinterpret_cast<const T*>(a.Msave) + bh * P * DK * DV;
  T* Ls = reinterpret_cast<T*>(a.Lsave) + bh * P * DK * DV;

  f32x16 lam[NRT];
  const float* dS = a.dS + (bh * N + i) * (int64_t)DK * DV;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) lam[rt][e] = dS[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col];

  for (int j = i - 1; j >= 0; --j) {
    const int64_t o = (bh * N + i) * N + j;
    if (!a.mask[o]) continue;
    const float g = a.gates[o];
    const int64_t p = pair_index(i, j);
    T* ld = Ls + p * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) ld[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] = from_f<T>(g * lam[rt][e]);
    typename MM::Frag bf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bf[ks] = MM::from_acc(lam[ks / KPT], ks, 1.f);
    const T* XT = ATb + (int64_t)j * DK * DK;
    f32x16 Y[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      Y[rt] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) Y[rt] = MM::mma(minus_eye_frag<T, DK>(XT, rt, ks, hh, c32), bf[ks], Y[rt]);
    }
    const T* Mj = Ms + p * DK * DV;
    const T* Bj = Bb + (int64_t)j * DK * DV;
    float part = 0.f;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t off = (int64_t)(rt * 32 + acc_row(e, hh)) * DV + col;
        part = fmaf(Y[rt][e], to_f<T>(Mj[off]), part);
        part = fmaf(lam[rt][e], to_f<T>(Bj[off]), part);
      }
    part = wave_sum(part);
    if (lane == 0) a.dgp[o * NCT + ct] = part;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) lam[rt][e] = fmaf(g, Y[rt][e], lam[rt][e]);
  }
  float* le = a.lam_end + (bh * N + i) * (int64_t)DK * DV;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) le[(int64_t)(rt * 32 + acc_row(e, hh)) * DV + col] = lam[rt][e];
}

// Pass 3: per history chunk j, the sums over the query chunks that keep it.
template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void compose_grad_reduce_kernel(ComposeBwdArgs a) {
  using MM = Mma<T>;
  constexpr int NRT = DK / 32, NTILE = NRT * NRT, TPW = NTILE / 4, NKS = DV / MM::KS, NCT = DV / 32;
  static_assert(NTILE % 4 == 0, "four waves share the dAt tiles");
  constexpr int NV8 = DK * DV / 8 / 256;  // 8-element groups of dBc per thread
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int64_t bh = blockIdx.x % BH;
  const int j = (int)(blockIdx.x / BH);  // most query chunks first
  const int N = a.N;
  const int64_t P = (int64_t)N * (N - 1) / 2;
  const T* Ms = reinterpret_cast<const T*>(a.Msave) + bh * P * DK * DV;
  const T* Ls = reinterpret_cast<const T*>(a.Lsave) + bh * P * DK * DV;

  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = zero16();
  float sb[NV8][8];
#pragma unroll
  for (int v = 0; v < NV8; ++v)
#pragma unroll
    for (int e = 0; e < 8; ++e) sb[v][e] = 0.f;

  for (int i = j + 1; i < N; ++i) {
    const int64_t o = (bh * N + i) * N + j;
    if (!a.mask[o]) continue;
    const int64_t p = pair_index(i, j);
    const T* L = Ls + p * DK * DV;
    const T* Mi = Ms + p * DK * DV;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = w * TPW + u, rt = t / NRT, st = t % NRT;
      const T* ar = L + (int64_t)(rt * 32 + c32) * DV;
      const T* br = Mi + (int64_t)(st * 32 + c32) * DV;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[u] = MM::mma(MM::load_plain(ar, ks, hh), MM::load_plain(br, ks, hh), acc[u]);
    }
#pragma unroll
    for (int v = 0; v < NV8; ++v) {
      const int64_t base = (int64_t)(v * 256 + tid) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sb[v][e] += to_f<T>(L[base + e]);
    }
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
  for (int v = 0; v < NV8; ++v) {
    const int64_t base = (int64_t)(v * 256 + tid) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dB[base + e] = sb[v][e];
  }
  // gate gradients of column j (zero for skipped, diagonal and future pairs)
  for (int i = tid; i < N; i += 256) {
    const int64_t o = (bh * N + i) * N + j;
    float s = 0.f;
    if (i > j && a.mask[o]) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) s += a.dgp[o * NCT + c];
    }
    a.dgates[o] = s;
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
static hipError_t launch_compose_bwd_t(const ComposeBwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H, BHN = BH * a.N;
  {
    TimedLaunch tl(HLA_KERNEL_BWD_SAVE, s);
    hipLaunchKernelGGL((compose_save_kernel<T, DK, DV>), dim3((unsigned)BHN), dim3(DV / 32 * 64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedLaunch tl(HLA_KERNEL_BWD_ADJOINT, s);
    hipLaunchKernelGGL((transpose_at_kernel<T, DK>), dim3((unsigned)(BHN * (DK / 32) * (DK / 32))), dim3(256), 0, s,
                       reinterpret_cast<const T*>(a.At), reinterpret_cast<T*>(a.AtT));
    hipLaunchKernelGGL((compose_adjoint_kernel<T, DK, DV>), dim3((unsigned)BHN), dim3(DV / 32 * 64), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedLaunch tl(HLA_KERNEL_BWD_REDUCE, s);
    hipLaunchKernelGGL((compose_grad_reduce_kernel<T, DK, DV>), dim3((unsigned)BHN), dim3(256), 0, s, a);
    if (a.dS0) {
      const int64_t per = (int64_t)DK * DV, total = BH * per;
      hipLaunchKernelGGL(chain_sum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a.lam_end, a.dS0,
                         a.N, per, total);
    }
  }
  return hipGetLastError();
}

template <class T>
static hipError_t launch_compose_bwd_d(const ComposeBwdArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_compose_bwd_t<T, 64, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_compose_bwd_t<T, 64, 128>(a, s);
  if (dk == 128 && dv == 64) return launch_compose_bwd_t<T, 128, 64>(a, s);
  return launch_compose_bwd_t<T, 128, 128>(a, s);
}

hipError_t launch_compose_backward(const ComposeBwdArgs& a, int dtype, int dk, int dv, hipStream_t s) {
  return dtype == 1 ? launch_compose_bwd_d<bf16>(a, dk, dv, s) : launch_compose_bwd_d<float>(a, dk, dv, s);
}

}  // namespace hla
