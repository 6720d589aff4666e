// Sequential chunk scan for native prefill: M_{c+1} = At_c M_c + Bc_c.
//
// [HLA] Methodology paragraph 1: the per-chunk affine maps compose in time order, so the
// state at every chunk boundary follows from the chunk summaries alone.
//
// One wavefront per (b, h, 32-column block of dv).  The 32 state columns are independent
// (M -> At M acts on each column separately), so no data moves between wavefronts.  The
// state tile lives in the accumulator layout: its bf16 copy is the B operand of the next
// product without leaving the lane, and At is read in the matching k order.  Bc is added
// by one more MFMA against the identity (Bc as the A operand, k = dv).  The next chunk's
// At and Bc are prefetched into registers while the current chunk computes.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

template <class T, int DK, int DV, bool PREFETCH>
__global__ __launch_bounds__(64) void scan_kernel(ScanArgs a) {
  using MM = Mma<T>;
  constexpr int E = sizeof(T), PAD = 16 / E;
  constexpr int PA = DK + PAD;       // LDS pitch of At rows
  constexpr int PB = 32 + PAD;       // LDS pitch of the Bc column block
  constexpr int NRT = DK / 32;
  constexpr int UA = DK / PAD;       // 16-byte units per At row
  constexpr int UB = 32 / PAD;       // 16-byte units per Bc block row
  constexpr int NA = DK * UA / 64;   // units per lane
  constexpr int NB = DK * UB / 64;
  constexpr int NVT = DV / 32;
  __shared__ __attribute__((aligned(16))) T sA[DK * PA];
  __shared__ __attribute__((aligned(16))) T sB[DK * PB];

  const int lane = threadIdx.x, hh = lane >> 5, c32 = lane & 31;
  const int64_t id = blockIdx.x;
  const int dvt = (int)(id % NVT);
  const int64_t bh = id / NVT;
  const int dv0 = dvt * 32;
  const int N = a.N;
  const T* Ag = reinterpret_cast<const T*>(a.At) + bh * N * (int64_t)DK * DK;
  const T* Bg = reinterpret_cast<const T*>(a.Bc) + bh * N * (int64_t)DK * DV;

  f32x16 M[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    M[rt] = zero16();
    if (a.S0) {
      const float* s0 = a.S0 + bh * (int64_t)DK * DV;
#pragma unroll
      for (int e = 0; e < 16; ++e) M[rt][e] = s0[(rt * 32 + acc_row(e, hh)) * DV + dv0 + c32];
    }
  }

  uint4 pa[PREFETCH ? NA : 1], pb[PREFETCH ? NB : 1];
  auto load_regs = [&](int c) {
    const uint4* src = reinterpret_cast<const uint4*>(Ag + (int64_t)c * DK * DK);
#pragma unroll
    for (int i = 0; i < NA; ++i) pa[i] = src[lane + 64 * i];
    const T* bsrc = Bg + (int64_t)c * DK * DV + dv0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int idx = lane + 64 * i, row = idx / UB, u = idx % UB;
      pb[i] = *reinterpret_cast<const uint4*>(bsrc + row * DV + u * PAD);
    }
  };
  auto store_regs = [&]() {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int idx = lane + 64 * i, row = idx / UA, u = idx % UA;
      *reinterpret_cast<uint4*>(sA + row * PA + u * PAD) = pa[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int idx = lane + 64 * i, row = idx / UB, u = idx % UB;
      *reinterpret_cast<uint4*>(sB + row * PB + u * PAD) = pb[i];
    }
  };
  auto load_direct = [&](int c) {
    const uint4* src = reinterpret_cast<const uint4*>(Ag + (int64_t)c * DK * DK);
    for (int i = lane; i < DK * UA; i += 64) {
      const int row = i / UA, u = i % UA;
      *reinterpret_cast<uint4*>(sA + row * PA + u * PAD) = src[i];
    }
    const T* bsrc = Bg + (int64_t)c * DK * DV + dv0;
    for (int i = lane; i < DK * UB; i += 64) {
      const int row = i / UB, u = i % UB;
      *reinterpret_cast<uint4*>(sB + row * PB + u * PAD) = *reinterpret_cast<const uint4*>(bsrc + row * DV + u * PAD);
    }
  };

  if constexpr (PREFETCH) {
    if (N > 0) load_regs(0);
  }
  for (int c = 0; c < N; ++c) {
    if constexpr (PREFETCH) {
      store_regs();
      if (c + 1 < N) load_regs(c + 1);
    } else {
      load_direct(c);
    }
    __syncthreads();
    if (a.states) {
      float* st = a.states + (bh * N + c) * (int64_t)DK * DV;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) st[(rt * 32 + acc_row(e, hh)) * DV + dv0 + c32] = M[rt][e];
    }
    typename MM::Frag bfr[DK / MM::KS];
#pragma unroll
    for (int ks = 0; ks < DK / MM::KS; ++ks) bfr[ks] = MM::from_acc(M[ks / (32 / MM::KS)], ks, 1.f);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x16 acc = zero16();
      const T* arow = sA + (rt * 32 + c32) * PA;
#pragma unroll
      for (int ks = 0; ks < DK / MM::KS; ++ks) acc = MM::mma(MM::load_clayout(arow, ks, hh), bfr[ks], acc);
      const T* brow = sB + (rt * 32 + c32) * PB;
#pragma unroll
      for (int kd = 0; kd < 32 / MM::KS; ++kd) acc = MM::mma(MM::load_plain(brow, kd, hh), diag_frag<T>(kd, lane, 1.f), acc);
      M[rt] = acc;
    }
    __syncthreads();
  }
  if (a.S_final) {
    float* sf = a.S_final + bh * (int64_t)DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sf[(rt * 32 + acc_row(e, hh)) * DV + dv0 + c32] = M[rt][e];
  }
}

template <class T, int DK, int DV>
static hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  constexpr int E = sizeof(T), PAD = 16 / E;
  constexpr int NA = DK * (DK / PAD) / 64, NB = DK * (32 / PAD) / 64;
  constexpr bool PF = (NA + NB) <= 48;
  const int64_t nb = a.B * a.H * (DV / 32);
  if (nb == 0) return hipSuccess;
  TimedLaunch tl(HLA_KERNEL_SCAN, s);
  hipLaunchKernelGGL((scan_kernel<T, DK, DV, PF>), dim3((unsigned)nb), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_scan_d(const ScanArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_scan_t<T, 64, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_scan_t<T, 64, 128>(a, s);
  if (dk == 128 && dv == 64) return launch_scan_t<T, 128, 64>(a, s);
  return launch_scan_t<T, 128, 128>(a, s);
}

hipError_t launch_scan(const ScanArgs& a, int dtype, int dk, int dv, hipStream_t s) {
  return dtype == 1 ? launch_scan_d<bf16>(a, dk, dv, s) : launch_scan_d<float>(a, dk, dv, s);
}

}  // namespace hla
