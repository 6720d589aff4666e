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

// bf16 transitions: one workgroup per (b, h, 32-column block) with one wave per 32-row
// tile.  Wave rt keeps rows [32 rt, 32 rt + 32) of the state block in its accumulators and
// needs only those rows of At: its A fragments (row 32 rt + lane%32, 8 consecutive k) come
// straight from global memory into registers.  The B operand is the whole 128 x 32 state
// block in bf16; every wave writes its tile into an LDS image laid out [column][k] (so a B
// fragment is one 16-byte read) and one barrier per chunk publishes it.  The image is
// double-buffered: buffer c % 2 is rewritten only after the next barrier, when every wave
// has read it.  Bc seeds the accumulator (fp32), so no extra products are needed.
//
// LANES (maps written by the library's own transitions pass): Bc comes in the accumulator's
// lane order, [chunk][dv/32 column tile][dk/32 row tile][64 lanes][16], two 16-byte loads
// per lane, and the At rows and Bc of the next kScanDepth chunks are in flight in a
// register ring (a step is a few products and one barrier, far shorter than a load from
// HBM).  The start state of every chunk is written as the bf16 image [dv][dk] that the
// output pass multiplies with (it rounds the state to bf16 there in any case): the LDS
// image of the step is that state already, and one more wave copies it out.  That wave
// issues every global store of the loop, so the product waves issue only loads and their
// waits for the ring never also wait for stores.  Without LANES, Bc is row-major, one
// chunk is loaded ahead and the product waves store the float32 states [dk][dv].
//
// MODE 0: one scan over all N chunks from S0 (states, S_final).
// MODE 1: independent segments of `seg` chunks, each starting from its seg_init state; the
//         start state of every chunk is written (a chunk of C = 64 seg tokens seen as seg
//         chunks of 64).
// MODE 2: the composite map of every segment: the scan runs over the augmented state
//         [At_seg | Bc_seg] (dk x (dk + dv)) from [I | 0], the additive term being [0 | Bc]
//         ([HLA] Methodology paragraph 1: affine maps compose; the map of a chunk of C tokens
//         is the composition of the maps of its 64-token pieces).
constexpr int kScanDepth = 3;

template <int DK, int DV, int MODE, bool LANES>
__global__ __launch_bounds__(DK / 32 * 64 + (LANES ? 64 : 0)) void scan_bf16_kernel(ScanArgs a) {
  constexpr int NCT = (MODE == 2 ? DK + DV : DV) / 32, NKS = DK / 16, NRT = DK / 32;
  constexpr int DEPTH = LANES ? kScanDepth : 1;
  constexpr int PB = DK + 8;  // bf16 pitch of an image row (one row per state column)
  __shared__ __attribute__((aligned(16))) bf16 sB0[32 * PB];
  __shared__ __attribute__((aligned(16))) bf16 sB1[32 * PB];

  const int lane = threadIdx.x & 63, hh = lane >> 5, c32 = lane & 31;
  const int rt = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block -> (column tile, scan): consecutive blocks go to the 8 XCDs in turn, and the NCT
  // column tiles of one scan all read its At, so when the scans come in multiples of 8 the
  // tiles of a scan take block indices equal mod 8: one XCD, one L2 for its At
  const int64_t id = blockIdx.x, nscan = gridDim.x / NCT;
  int ct;
  int64_t rest;
  if (nscan % 8 == 0) {
    const int64_t r = id >> 3;
    ct = (int)(r % NCT);
    rest = (r / NCT) * 8 + (id & 7);
  } else {
    ct = (int)(id % NCT);
    rest = id / NCT;
  }
  const int N = a.N;
  int64_t bh = rest;
  int NS = 1, g = 0, c0 = 0, nsub = N;
  if (MODE != 0) {
    NS = (N + a.seg - 1) / a.seg;
    g = (int)(rest % NS);
    bh = rest / NS;
    c0 = g * a.seg;
    nsub = N - c0 < a.seg ? N - c0 : a.seg;
  }
  // MODE 1 never needs the end state of a segment's last piece
  const int nmul = MODE == 1 ? nsub - 1 : nsub;
  const bool want_states = MODE != 2 && (LANES ? a.states_t != nullptr : a.states != nullptr);
  if (LANES && rt == NRT) {
    // the writer wave: after each step's barrier, the image of the chunk's start state goes
    // out to states_t (row ct * 32 + r of the [dv][dk] image is image row r); the barrier
    // sequence is the product waves'
    const int nstep = want_states ? nsub : nmul;
    for (int c = (MODE == 2 && nsub > 0) ? 1 : 0; c < nstep; ++c) {
      __syncthreads();
      if (want_states) {
        const bf16* img = (c & 1) ? sB1 : sB0;
        bf16* dst = reinterpret_cast<bf16*>(a.states_t) + ((bh * N + c0 + c) * (int64_t)DV + ct * 32) * DK;
#pragma unroll
        for (int i = lane; i < 32 * (DK / 8); i += 64) {
          const int r = i / (DK / 8), u = i % (DK / 8);
          *reinterpret_cast<uint4*>(dst + r * DK + u * 8) = *reinterpret_cast<const uint4*>(img + r * PB + u * 8);
        }
      }
    }
    return;
  }
  // MODE 2: column blocks [0, DK/32) are the At part (additive term 0), the rest the Bc part
  const bool apart = MODE == 2 && ct < DK / 32;
  const int ctv = MODE == 2 ? (apart ? 0 : ct - DK / 32) : ct;  // column tile of Bc
  const bf16* arow = reinterpret_cast<const bf16*>(a.At) + (bh * N + c0) * (int64_t)DK * DK + (rt * 32 + c32) * DK +
                     hh * 8;
  // this lane's Bc values of chunk c: 16 rows (row_of) of one column, row-major or lane order
  const bf16* bbase = reinterpret_cast<const bf16*>(a.Bc) + (bh * N + c0) * (int64_t)DK * DV;
  auto bc_ptr = [&](int c) {
    return LANES ? bbase + (int64_t)c * DK * DV + (((int64_t)ctv * NRT + rt) * 64 + lane) * 16
                 : bbase + (int64_t)c * DK * DV + rt * 32 * DV + ctv * 32 + c32;
  };
  // accumulator element e of this lane: row 32 rt + (e / 4) 8 + 4 hh + e % 4, column 32 ct + c32
  auto row_of = [&](int e) { return (e >> 2) * 8 + hh * 4 + (e & 3); };

  f32x16 M = zero16();
  if (MODE == 0 && a.S0) {
    const float* s0 = a.S0 + bh * (int64_t)DK * DV + rt * 32 * DV + ct * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) M[e] = s0[row_of(e) * DV];
  }
  if (MODE == 1) {
    const float* s0 = a.seg_init + (bh * NS + g) * (int64_t)DK * DV + rt * 32 * DV + ct * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) M[e] = s0[row_of(e) * DV];
  }
  // MODE 2 starts from the first piece's own map ([I | 0] through piece 0 is [At_0 | Bc_0])
  int cstart = 0;
  if (MODE == 2 && nsub > 0) {
    cstart = 1;
    if (apart) {
      const bf16* p0 = reinterpret_cast<const bf16*>(a.At) + (bh * N + c0) * (int64_t)DK * DK + rt * 32 * DK + ct * 32 + c32;
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = (float)p0[row_of(e) * DK];
    } else if (LANES) {
      const bf16x8* p = reinterpret_cast<const bf16x8*>(bc_ptr(0));
      const bf16x8 lo = p[0], hi = p[1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        M[e] = (float)lo[e];
        M[e + 8] = (float)hi[e];
      }
    } else {
      const bf16* p = bc_ptr(0);
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = (float)p[row_of(e) * DV];
    }
  }
  bf16x8 af[DEPTH][NKS];
  bf16x8 bl[DEPTH][2];   // LANES: 16 Bc values in lane order
  bf16 bcv[DEPTH][16];   // otherwise: 16 Bc values, one load each
  // the loads of one ring slot; the At part of MODE 2 has no additive term (its Bc loads
  // read the first column tile and are not used, so every slot's loads are unconditional)
  auto load = [&](int slot, int c) __attribute__((always_inline)) {
    const bf16* ap = arow + (int64_t)c * DK * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) af[slot][ks] = *reinterpret_cast<const bf16x8*>(ap + ks * 16);
    if constexpr (LANES) {
      const bf16x8* p = reinterpret_cast<const bf16x8*>(bc_ptr(c));
      bl[slot][0] = p[0];
      bl[slot][1] = p[1];
    } else {
      const bf16* p = bc_ptr(c);
#pragma unroll
      for (int e = 0; e < 16; ++e) bcv[slot][e] = p[row_of(e) * DV];
    }
  };
  auto store_state = [&](int c) __attribute__((always_inline)) {  // float32 states (not LANES)
    float* p = a.states + (bh * N + c0 + c) * (int64_t)DK * DV + rt * 32 * DV + ct * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) p[row_of(e) * DV] = M[e];
  };
#pragma unroll
  for (int sl = 0; sl < DEPTH; ++sl)
    if (cstart + sl < nmul) load(sl, cstart + sl);
  for (int cb = cstart; cb < nsub; cb += DEPTH) {
#pragma unroll
    for (int sl = 0; sl < DEPTH; ++sl) {  // unrolled: every ring slot index is static
      const int c = cb + sl;
      if (c >= nsub) break;
      if (!LANES && want_states) store_state(c);
      // the last piece of a MODE 1 segment needs no product: only (LANES) its image, for
      // the writer wave
      if (c >= nmul && !(LANES && want_states)) break;
      bf16* img = (c & 1) ? sB1 : sB0;
      // this wave's rows of bf16(M) into the image: 4 runs of 4 consecutive k per lane
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)M[gq * 4 + e];
        *reinterpret_cast<bf16x4*>(img + c32 * PB + rt * 32 + gq * 8 + hh * 4) = v;
      }
      __syncthreads();
      if (c >= nmul) break;
      f32x16 acc0, acc1 = zero16();
      if constexpr (LANES) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc0[e] = apart ? 0.f : (float)bl[sl][0][e];
          acc0[e + 8] = apart ? 0.f : (float)bl[sl][1][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc0[e] = apart ? 0.f : (float)bcv[sl][e];
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(img + c32 * PB + ks * 16 + hh * 8);
        if (ks & 1)
          acc1 = Mma<bf16>::mma(af[sl][ks], bfr, acc1);
        else
          acc0 = Mma<bf16>::mma(af[sl][ks], bfr, acc0);
      }
      if (c + DEPTH < nmul) load(sl, c + DEPTH);
#pragma unroll
      for (int e = 0; e < 16; ++e) M[e] = acc0[e] + acc1[e];
    }
  }
  if (MODE == 0 && a.S_final) {
    float* p = a.S_final + bh * (int64_t)DK * DV + rt * 32 * DV + ct * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) p[row_of(e) * DV] = M[e];
  }
  if (MODE == 2) {
    const int64_t sidx = bh * NS + g;
    if (apart) {
      bf16* p = reinterpret_cast<bf16*>(a.seg_At) + sidx * DK * DK + rt * 32 * DK + ct * 32 + c32;
#pragma unroll
      for (int e = 0; e < 16; ++e) p[row_of(e) * DK] = (bf16)M[e];
    } else {
      bf16* p = reinterpret_cast<bf16*>(a.seg_Bc) + sidx * DK * DV + rt * 32 * DV + ctv * 32 + c32;
#pragma unroll
      for (int e = 0; e < 16; ++e) p[row_of(e) * DV] = (bf16)M[e];
    }
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

template <int DK, int DV, int MODE>
static hipError_t launch_scan_bf16_t(const ScanArgs& a, hipStream_t s) {
  constexpr int NCT = (MODE == 2 ? DK + DV : DV) / 32;
  const int64_t ns = MODE == 0 ? 1 : (a.N + a.seg - 1) / a.seg;
  const int64_t nb = a.B * a.H * ns * NCT;
  if (nb == 0) return hipSuccess;
  TimedLaunch tl(HLA_KERNEL_SCAN, s);
  if (a.lanes)
    hipLaunchKernelGGL((scan_bf16_kernel<DK, DV, MODE, true>), dim3((unsigned)nb), dim3(DK / 32 * 64 + 64), 0, s, a);
  else
    hipLaunchKernelGGL((scan_bf16_kernel<DK, DV, MODE, false>), dim3((unsigned)nb), dim3(DK / 32 * 64), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_scan_bf16(const ScanArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_scan_bf16_t<64, 64, MODE>(a, s);
  if (dk == 64 && dv == 128) return launch_scan_bf16_t<64, 128, MODE>(a, s);
  if (dk == 128 && dv == 64) return launch_scan_bf16_t<128, 64, MODE>(a, s);
  return launch_scan_bf16_t<128, 128, MODE>(a, s);
}

hipError_t launch_scan(const ScanArgs& a, int dtype, int dk, int dv, hipStream_t s) {
  if (dtype == 1) return launch_scan_bf16<0>(a, dk, dv, s);
  return launch_scan_d<float>(a, dk, dv, s);
}

hipError_t launch_scan_segments(const ScanArgs& a, int dk, int dv, hipStream_t s) {
  return launch_scan_bf16<1>(a, dk, dv, s);
}

hipError_t launch_combine_segments(const ScanArgs& a, int dk, int dv, hipStream_t s) {
  return launch_scan_bf16<2>(a, dk, dv, s);
}

}  // namespace hla
