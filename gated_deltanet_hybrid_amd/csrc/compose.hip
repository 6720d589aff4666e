// Gated composition of chunk transitions, bf16 MFMA path (the hot loop of the routed
// prefill).
//
// [HLA] Methodology paragraphs 1 and 3: every query chunk i starts from S0 and applies, in
// time order, each history chunk j < i that its gate keeps, interpolated with the identity:
//     M <- M + g_ij (At_j M + Bc_j - M)  =  M + (At_j - I) (g_ij M) + g_ij Bc_j.
// Skipped pairs (mask 0) leave M untouched ([HLA] Methodology paragraph 4).
//
// Work decomposition (MI355X, 256 CUs x 4 SIMDs):
//   * workgroup = (b, h, QG consecutive query chunks); NW wavefronts (two per SIMD); wave w
//     owns the 32 state columns [32 ct, 32 ct + 32) of SPW of the group's query chunks;
//   * the state slice (dk x 32 float32 per query chunk) lives in the MFMA accumulators for
//     the whole chain; its bf16 copy (scaled by g) is the B operand of the next product
//     without leaving the lane (the k order of the accumulator rows is matched by how At
//     is read);
//   * g Bc_j is one more pair of MFMAs per row tile: Bc_j as the A operand against g I;
//   * (At_j, Bc_j) of the next history chunk are copied global -> LDS asynchronously
//     (global_load_lds, 16 bytes per lane) while the current one is multiplied; the LDS
//     rows are XOR-swizzled in 16-byte units so fragment reads are bank-conflict free;
//   * a prep pass writes (At_j - I) with each 16-wide k block reordered so that one lane's
//     8 k values of a k-step are 16 contiguous bytes: every A fragment is a single
//     conflict-free 16-byte LDS read;
//   * gates sit in one register per query chunk (64 history chunks per refill) and are
//     broadcast with readlane, so the loop touches no other memory;
//   * groups are dispatched longest chain first, head-fastest, so the workgroups running
//     together sweep the same history chunks of the same heads (L2 reuse of At_j, Bc_j).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

typedef __attribute__((address_space(3))) void lds_void_t;

// (At_j - I) in the k order the composition reads: within every 16-wide k block the two
// middle groups of four are swapped, so the 8 k values one lane needs for a k-step
// (ks*16 + {h*4 .. h*4+3, 8 + h*4 .. 8 + h*4+3}) are 16 contiguous bytes at unit 2 ks + h.
template <int DK>
__global__ __launch_bounds__(256) void prep_at_kernel(const bf16* __restrict__ At, bf16* __restrict__ Ap, int64_t n_units) {
  const int64_t u = blockIdx.x * (int64_t)256 + threadIdx.x;  // output 16-byte unit
  if (u >= n_units) return;
  constexpr int UPR = DK / 8;
  const int64_t row_all = u / UPR;  // row over all (b, h, j, r)
  const int U = (int)(u % UPR), r = (int)(row_all % DK);
  const bf16* src = At + row_all * DK;
  const int q0 = 4 * (U >> 1) + (U & 1), q1 = q0 + 2;  // source groups of four
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(src + q0 * 4);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(src + q1 * 4);
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = (q0 * 4 + e == r) ? (bf16)((float)a[e] - 1.f) : a[e];
    o[e + 4] = (q1 * 4 + e == r) ? (bf16)((float)b[e] - 1.f) : b[e];
  }
  *reinterpret_cast<bf16x8*>(Ap + u * 8) = o;
}

template <int DK, int DV, int NW, int SPW, int NBUF, bool BCG>
__global__ __launch_bounds__(NW * 64, (NBUF == 1 || BCG) ? 2 : 1) void compose_bf16_kernel(RouteArgs a) {
  constexpr int NCTV = DV / 32;
  constexpr int QG = NW * SPW / NCTV;
  constexpr int NRT = DK / 32, NKS = DK / 16;
  constexpr int UA = DK / 8, UB = DV / 8;  // 16-byte units per LDS row
  constexpr int NIA = DK * UA / 64, NIB = DK * UB / 64;
  // Two separate LDS variables (not one array indexed by the step parity): the copy into
  // one buffer can then be proven not to alias reads of the other, so the compiler does
  // not wait for the copy before the multiplications that overlap it.
  // BCG: Bc fragments come from global memory into registers (prefetched one history
  // chunk ahead) and only At is staged in LDS, halving the LDS of a workgroup.
  __shared__ __attribute__((aligned(16))) bf16 sA0[DK * DK];
  __shared__ __attribute__((aligned(16))) bf16 sB0[BCG ? 8 : DK * DV];
  __shared__ __attribute__((aligned(16))) bf16 sA1[NBUF == 2 ? DK * DK : 8];
  __shared__ __attribute__((aligned(16))) bf16 sB1[(NBUF == 2 && !BCG) ? DK * DV : 8];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.N;
  const int64_t BH = a.B * a.H;
  const int ng = (N + QG - 1) / QG;
  const int64_t id = blockIdx.x;
  const int64_t bh = id % BH;
  const int grp = ng - 1 - (int)(id / BH);
  const int i0 = grp * QG;
  const int nsteps = (i0 + QG < N ? i0 + QG : N) - 1;  // history chunks 0 .. nsteps-1
  const int ct = w % NCTV;
  int qi[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) qi[s] = i0 + w / NCTV + s * (NW / NCTV);

  const bf16* Ag = reinterpret_cast<const bf16*>(a.At_prep) + bh * N * (int64_t)DK * DK;
  const bf16* Bg = reinterpret_cast<const bf16*>(a.Bc) + bh * N * (int64_t)DK * DV;
  const float* gts = a.gates + bh * (int64_t)N * N;
  const uint8_t* msk = a.mask + bh * (int64_t)N * N;
  static_assert((DK * UA / 64) % NW == 0 && (DK * UB / 64) % NW == 0, "copy blocks split evenly");
  float* Sout = a.S_routed + bh * (int64_t)N * DK * DV;

  // async copy of (At_j, Bc_j) into LDS buffer `buf`; LDS unit p of row r holds global
  // unit p ^ (r mod units-per-row).  Wave w copies 1 KiB blocks w, w + NW, ...; because NW
  // is a multiple of 4 the swizzle of a lane is the same in all of its blocks, so one
  // offset per lane serves every block.
  static_assert(NW % 4 == 0, "one swizzle per lane needs NW % 4 == 0");
  const int offA = [&] {
    const int u = w * 64 + lane, r = u / UA, p = u % UA;
    return r * DK + ((p ^ (r & (UA - 1))) * 8);
  }();
  const int offB = [&] {
    const int u = w * 64 + lane, r = u / UB, p = u % UB;
    return r * DV + ((p ^ (r & (UB - 1))) * 8);
  }();
  auto issue = [&](int j, bf16* dA, bf16* dB) {
    const char* as = reinterpret_cast<const char*>(Ag + (int64_t)j * DK * DK);  // uniform base
    const char* bs = reinterpret_cast<const char*>(Bg + (int64_t)j * DK * DV);
#pragma unroll
    for (int m = 0; m < NIA / NW; ++m)
      __builtin_amdgcn_global_load_lds(as + (uint32_t)((offA + m * NW * 512) * 2), (lds_void_t*)&dA[(w + m * NW) * 512],
                                       16, 0, 0);
    if constexpr (!BCG) {
#pragma unroll
      for (int m = 0; m < NIB / NW; ++m)
        __builtin_amdgcn_global_load_lds(bs + (uint32_t)((offB + m * NW * 512) * 2),
                                         (lds_void_t*)&dB[(w + m * NW) * 512], 16, 0, 0);
    }
  };
  // Bc A fragments of history chunk j straight from global memory: row rt*32 + c32,
  // the 8 columns ct*32 + kd*16 + hh*8 ..
  bf16x8 bcf[NRT][2];
  auto load_bc = [&](int j) {
    const bf16* bs = Bg + (int64_t)j * DK * DV + c32 * DV + ct * 32 + hh * 8;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int kd = 0; kd < 2; ++kd) bcf[rt][kd] = *reinterpret_cast<const bf16x8*>(bs + rt * 32 * DV + kd * 16);
  };
  auto wait_copies = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 M[SPW][NRT];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      M[s][rt] = zero16();
      if (a.S0) {
        int lofs = hh * 4 * DV + ct * 32 + c32;
        asm volatile("" : "+v"(lofs));
        const float* s0 = a.S0 + bh * (int64_t)DK * DV + lofs;
#pragma unroll
        for (int e = 0; e < 16; ++e) M[s][rt][e] = s0[(rt * 32 + (e >> 2) * 8 + (e & 3)) * DV];
      }
    }
  // Store a finished state slice.  The opaque lane offset keeps the compiler from holding
  // 64 precomputed store addresses across the whole chain.
  auto write_state = [&](int s) {
    int lofs = hh * 4 * DV + ct * 32 + c32;
    asm volatile("" : "+v"(lofs));
    float* dst = Sout + (int64_t)qi[s] * DK * DV + lofs;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(rt * 32 + (e >> 2) * 8 + (e & 3)) * DV] = M[s][rt][e];
  };
#pragma unroll
  for (int s = 0; s < SPW; ++s)
    if (qi[s] == 0) write_state(s);

  // gates of 64 consecutive history chunks, lane j holds chunk jb*64 + j (0 when skipped)
  float greg[SPW];
  auto load_gates = [&](int jb) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int j = jb * 64 + lane;
      float v = 0.f;
      if (qi[s] < N && j < qi[s]) {
        const int64_t o = (int64_t)qi[s] * N + j;
        if (msk[o]) v = gts[o];
      }
      greg[s] = v;
    }
  };

  // diagonal B fragments for g Bc: slot k (plain order) of k-step kd equals the lane's
  // column in exactly one lane-half; the pattern keeps g's bf16 bits there
  uint32_t pat[2][4];
#pragma unroll
  for (int kd = 0; kd < 2; ++kd)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t m = 0;
      const int k0 = kd * 16 + hh * 8 + 2 * d;
      if (k0 == c32) m |= 0x0000ffffu;
      if (k0 + 1 == c32) m |= 0xffff0000u;
      pat[kd][d] = m;
    }

  // one history chunk: multiply with the (At_j - I, Bc_j) in (cA, cB) while the copy of
  // chunk j + 1 lands in (nA, nB)
  auto step = [&](int j, const bf16* cA, const bf16* cB, bf16* nA, bf16* nB) {
    if ((j & 63) == 0) load_gates(j >> 6);
    // read the gates before issuing the next copies, so waiting for the gate loads never
    // waits for the copies
    float g[SPW];
    bool any = false;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      g[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(greg[s]), j & 63));
      any |= (g[s] != 0.f);
    }
    if (NBUF == 2 && j + 1 < nsteps) issue(j + 1, nA, nB);
    if (BCG && !any && j + 1 < nsteps) load_bc(j + 1);
    if (any) {
      // B operand bf16(g M) straight from the accumulator rows this lane holds
      bf16x8 bfr[SPW][NKS];
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) bfr[s][ks] = Mma<bf16>::from_acc(M[s][ks >> 1], ks, g[s]);
      if constexpr (BCG) {
#pragma unroll
        for (int kd = 0; kd < 2; ++kd) {
          bf16x8 dg[SPW];
#pragma unroll
          for (int s = 0; s < SPW; ++s) {
            const uint32_t gb = (uint32_t)__builtin_bit_cast(unsigned short, (bf16)g[s]);
            const uint32_t g2 = gb | (gb << 16);
            uint32_t d4[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) d4[d] = pat[kd][d] & g2;
            dg[s] = __builtin_bit_cast(bf16x8, d4);
          }
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int s = 0; s < SPW; ++s) M[s][rt] = Mma<bf16>::mma(bcf[rt][kd], dg[s], M[s][rt]);
        }
      }
      if (BCG && j + 1 < nsteps) load_bc(j + 1);  // bcf was consumed at issue above
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const int r = rt * 32 + c32;
          const bf16x8 af =
              *reinterpret_cast<const bf16x8*>(cA + r * DK + (((2 * ks + hh) ^ (r & (UA - 1))) * 8));
#pragma unroll
          for (int s = 0; s < SPW; ++s) M[s][rt] = Mma<bf16>::mma(af, bfr[s][ks], M[s][rt]);
        }
      }
if constexpr (!BCG) {
#pragma unroll
      for (int kd = 0; kd < 2; ++kd) {
        bf16x8 dg[SPW];
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
          const uint32_t gb = (uint32_t)__builtin_bit_cast(unsigned short, (bf16)g[s]);
          const uint32_t g2 = gb | (gb << 16);
          uint32_t d4[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) d4[d] = pat[kd][d] & g2;
          dg[s] = __builtin_bit_cast(bf16x8, d4);
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const int r = rt * 32 + c32;
          const int unit = 4 * ct + 2 * kd + hh;
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(cB + r * DV + ((unit ^ (r & (UB - 1))) * 8));
#pragma unroll
          for (int s = 0; s < SPW; ++s) M[s][rt] = Mma<bf16>::mma(af, dg[s], M[s][rt]);
        }
      }
}
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s)
      if (qi[s] == j + 1 && qi[s] < N) write_state(s);
    if (j + 1 < nsteps) {
      if (NBUF == 1) {
        __syncthreads();  // every wave is done reading the single buffer
        issue(j + 1, nA, nB);
      }
      wait_copies();
      __syncthreads();
    }
  };

  if (nsteps > 0) {
    issue(0, sA0, sB0);
    if constexpr (BCG) load_bc(0);
    wait_copies();
    __syncthreads();
  }
  if constexpr (NBUF == 2) {
    for (int j = 0; j < nsteps; j += 2) {
      step(j, sA0, sB0, sA1, sB1);
      if (j + 1 < nsteps) step(j + 1, sA1, sB1, sA0, sB0);
    }
  } else {
    for (int j = 0; j < nsteps; ++j) step(j, sA0, sB0, sA0, sB0);
  }
}

template <int DK, int DV, int NW, int SPW, int NBUF, bool BCG>
static hipError_t launch_compose_bf16_t(const RouteArgs& a, hipStream_t s) {
  constexpr int QG = NW * SPW / (DV / 32);
  const int64_t ng = (a.N + QG - 1) / QG;
  const int64_t nb = ng * a.B * a.H;
  TimedLaunch tl(HLA_KERNEL_COMPOSE, s);
  hipLaunchKernelGGL((compose_bf16_kernel<DK, DV, NW, SPW, NBUF, BCG>), dim3((unsigned)nb), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compose_bf16(const RouteArgs& a, int dk, int dv, hipStream_t s) {
  const int64_t n_units = a.B * a.H * (int64_t)a.N * dk * (dk / 8);
  if (n_units > 0) {
    const unsigned nb = (unsigned)((n_units + 255) / 256);
    if (dk == 64)
      hipLaunchKernelGGL(prep_at_kernel<64>, dim3(nb), dim3(256), 0, s, reinterpret_cast<const bf16*>(a.At),
                         reinterpret_cast<bf16*>(a.At_prep), n_units);
    else
      hipLaunchKernelGGL(prep_at_kernel<128>, dim3(nb), dim3(256), 0, s, reinterpret_cast<const bf16*>(a.At),
                         reinterpret_cast<bf16*>(a.At_prep), n_units);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#ifndef HLA_COMPOSE_SHAPE
#define HLA_COMPOSE_SHAPE 8, 2, 2, false
#endif
  if (dk == 64 && dv == 64) return launch_compose_bf16_t<64, 64, HLA_COMPOSE_SHAPE>(a, s);
  if (dk == 64 && dv == 128) return launch_compose_bf16_t<64, 128, HLA_COMPOSE_SHAPE>(a, s);
  if (dk == 128 && dv == 64) return launch_compose_bf16_t<128, 64, HLA_COMPOSE_SHAPE>(a, s);
  return launch_compose_bf16_t<128, 128, HLA_COMPOSE_SHAPE>(a, s);
}

}  // namespace hla
