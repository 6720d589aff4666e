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
//   * (At_j - I, Bc_j) of the next history chunk are copied global -> LDS asynchronously
//     (global_load_lds, 16 bytes per lane, every instruction a contiguous 1 KiB source)
//     while the current one is multiplied;
//   * a prep pass writes (At_j - I) in the exact byte order of its LDS image: every A
//     fragment is one conflict-free 16-byte LDS read at a lane-constant address plus a
//     compile-time offset, which leaves registers for a ring of fragment reads in flight;
//   * gates sit in one register per query chunk (64 history chunks per refill) and are
//     broadcast with readlane, so the loop touches no other memory;
//   * each XCD works through its heads one at a time, longest chain first, so the 32
//     workgroups running on an XCD sweep the same head's history (L2 reuse of At_j, Bc_j).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

typedef __attribute__((address_space(3))) void lds_void_t;

// (At_j - I) written in the exact byte order of the composition's LDS image of it, so the
// copy into LDS is a plain contiguous 1 KiB block per instruction.  The image: the columns
// are cut into 16-wide k blocks stored one after the other (DK rows x 32 bytes each);
// within a block the 16 columns are reordered so that the 8 k values one lane needs for a
// k-step (ks*16 + {h*4 .. h*4+3, 8 + h*4 .. 8 + h*4+3}) form the 16-byte half h, and the
// two halves of row r are swapped when bits 2 and 3 of r differ, so that rows r, r + 4,
// r + 8 and r + 12 start on distinct bank groups and a read phase of 8 or of 16 lanes is
// conflict free.  Copy block m (1 KiB) holds k block m / (DK/32) for rows
// 32 (m % (DK/32)) .. + 31, two 16-byte units per row.
template <int DK>
__global__ __launch_bounds__(256) void prep_at_kernel(const bf16* __restrict__ At, bf16* __restrict__ Ap, int64_t n_pairs) {
  // one thread per (row, k block): reads the row's 32 contiguous bytes of the block
  // (consecutive threads walk along a row, so the reads are fully coalesced) and writes
  // the two 16-byte halves to their adjacent places in the image.
  const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (t >= n_pairs) return;
  constexpr int KB = DK / 16, NRT = DK / 32;
  const int kb = (int)(t % KB);
  const int64_t row_all = t / KB;  // row over all (b, h, j, r)
  const int r = (int)(row_all % DK);
  const int64_t chunk = row_all / DK;
  const bf16* src = At + row_all * DK + kb * 16;
  const bf16x8 lo = *reinterpret_cast<const bf16x8*>(src);      // groups of four 0, 1
  const bf16x8 hi = *reinterpret_cast<const bf16x8*>(src + 8);  // groups 2, 3
  bf16x8 h0, h1;  // logical halves: groups (0, 2) and (1, 3)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h0[e] = lo[e];
    h0[e + 4] = hi[e];
    h1[e] = lo[e + 4];
    h1[e + 4] = hi[e + 4];
  }
  const int d = r - kb * 16;  // the diagonal entry of this row, if it falls in the block
  if (d >= 0 && d < 16) {
    const int half = (d >> 2) & 1, e = (d & 3) + ((d >> 3) << 2);
    if (half == 0)
      h0[e] = (bf16)((float)h0[e] - 1.f);
    else
      h1[e] = (bf16)((float)h1[e] - 1.f);
  }
  const int m = kb * NRT + (r >> 5);
  bf16* dst = Ap + chunk * DK * DK + m * 512 + (r & 31) * 16;
  const bool swap = ((r >> 2) ^ (r >> 3)) & 1;
  *reinterpret_cast<bf16x8*>(dst) = swap ? h1 : h0;
  *reinterpret_cast<bf16x8*>(dst + 8) = swap ? h0 : h1;
}

template <int DK, int DV, int NW, int SPW, int PF>
__global__ __launch_bounds__(NW * 64, 1) void compose_bf16_kernel(RouteArgs a) {
  constexpr int NCTV = DV / 32;
  constexpr int NRT = DK / 32, NKS = DK / 16;
  constexpr int BLK = DK * 32;                     // bytes of one 16-wide k block in LDS
  constexpr int NDA = (DK / 16) * NRT, NDB = (DV / 16) * NRT;  // 1 KiB copy blocks
  static_assert(NDA % NW == 0 && NDB % NW == 0, "copy blocks split evenly");
  static_assert(NDA / NW + NDB / NW <= NKS * NRT, "at most one copy per A fragment");
  // LDS images: (At_j - I) as the prep pass laid it out (k blocks of DK rows x 32 bytes,
  // every fragment read is one lane-constant address plus a compile-time offset); Bc_j row
  // by row, 16-byte unit p of row r holding unit p ^ (r mod units-per-row), so both the
  // copy (whole rows) and the column-block reads are bank-conflict free.  Two separate LDS
  // variables per operand (not one array indexed by the step parity): the copy into one
  // buffer can then be proven not to alias reads of the other, so the compiler does not
  // wait for the copy before the multiplications that overlap it.
  __shared__ __attribute__((aligned(16))) bf16 sA0[DK * DK];
  __shared__ __attribute__((aligned(16))) bf16 sB0[DK * DV];
  __shared__ __attribute__((aligned(16))) bf16 sA1[DK * DK];
  __shared__ __attribute__((aligned(16))) bf16 sB1[DK * DV];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.N;
  const int64_t BH = a.B * a.H;
  constexpr int QG = NW * SPW / NCTV;
  const int ng = (N + QG - 1) / QG;
  const int64_t id = blockIdx.x;
  // Workgroup ids go to XCDs round-robin (id % 8).  When the heads split evenly over the 8
  // XCDs, the k-th workgroup of an XCD takes the XCD's heads one at a time, each longest
  // chain first: all 32 CUs of an XCD then sweep the history of one head and share its
  // chunks in that XCD's L2.  Otherwise heads run fastest, longest chains first.
  int64_t bh;
  int grp;
  if (BH % 8 == 0) {
    const int64_t xcd = id % 8, k = id / 8;
    bh = xcd + 8 * (k / ng);
    grp = ng - 1 - (int)(k % ng);
  } else {
    bh = id % BH;
    grp = ng - 1 - (int)(id / BH);
  }
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
  float* Sout = a.S_routed + bh * (int64_t)N * DK * DV;

  // Async copy of (At_j, Bc_j) into LDS, 1 KiB blocks m = w, w + NW, ... per wave.  Bc
  // block m is UPB = 1024 / (2 DV) whole rows; its lane -> source unit permutation depends
  // on m only through m mod (units-per-row / UPB), which is fixed per wave because NW is a
  // multiple of it, so one offset per lane serves every block.
  constexpr int UB = DV / 8, RPB = 1024 / (2 * DV);  // units per Bc row, rows per block
  static_assert(NW % (UB / RPB) == 0, "Bc swizzle fixed per wave");
  const int srcB = [&] {
    const int r = w * RPB + lane / UB, p = lane % UB;
    return (lane / UB) * DV * 2 + ((p ^ (r & (UB - 1))) << 4);
  }();
  // copy instruction d (0 .. NDW-1) of this wave for history chunk j
  constexpr int NDW = NDA / NW + NDB / NW;
  auto issue_one = [&](int j, int d, bf16* dA, bf16* dB) {
    if (d < NDA / NW) {
      const int m = w + d * NW;
      const char* as = reinterpret_cast<const char*>(Ag + (int64_t)j * DK * DK);  // uniform base
      __builtin_amdgcn_global_load_lds(as + m * 1024 + lane * 16,
                                       (lds_void_t*)(reinterpret_cast<char*>(dA) + m * 1024), 16, 0, 0);
    } else {
      const int m = w + (d - NDA / NW) * NW;
      const char* bs = reinterpret_cast<const char*>(Bg + (int64_t)j * DK * DV);
      __builtin_amdgcn_global_load_lds(bs + m * 1024 + srcB,
                                       (lds_void_t*)(reinterpret_cast<char*>(dB) + m * 1024), 16, 0, 0);
    }
  };
  auto issue = [&](int j, bf16* dA, bf16* dB) {
#pragma unroll
    for (int d = 0; d < NDW; ++d) issue_one(j, d, dA, dB);
  };
  auto wait_copies = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // fragment reads: row rt*32 + c32, logical half hh of k block kb (At); Bc columns
  // 32 ct + 16 kd + 8 hh .. (unit 4 ct + 2 kd + hh of the row)
  const int rd = c32 * 32 + ((hh ^ (((c32 >> 2) ^ (c32 >> 3)) & 1)) << 4);
  const int rdB0 = c32 * DV * 2 + (((4 * ct + hh) ^ (c32 & (UB - 1))) << 4);
  const int rdB1 = c32 * DV * 2 + (((4 * ct + 2 + hh) ^ (c32 & (UB - 1))) << 4);
  constexpr int NFA = NKS * NRT, NF = NFA + 2 * NRT;
  auto frag = [&](const bf16* cA, const bf16* cB, int f) -> bf16x8 {
    if (f < NFA)
      return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(cA) + rd + (f / NRT) * BLK + (f % NRT) * 1024);
    const int fb = f - NFA;
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(cB) + (fb / NRT ? rdB1 : rdB0) +
                                            (fb % NRT) * 32 * DV * 2);
  };

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
  // 64 precomputed store addresses across the whole chain.  The stores are non-temporal:
  // the routed states are read once, later, and the L2 is better left to the transitions
  // that other workgroups still read.
  auto write_state = [&](int s) {
    int lofs = hh * 4 * DV + ct * 32 + c32;
    asm volatile("" : "+v"(lofs));
    float* dst = Sout + (int64_t)qi[s] * DK * DV + lofs;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) __builtin_nontemporal_store(M[s][rt][e], &dst[(rt * 32 + (e >> 2) * 8 + (e & 3)) * DV]);
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
    const bool more = j + 1 < nsteps;
    if (any) {
      // the first PF fragment reads are in flight while the B operands are converted
      bf16x8 ring[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) ring[p] = frag(cA, cB, p);
      // B operand bf16(g M) straight from the accumulator rows this lane holds
      bf16x8 bfr[SPW][NKS];
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) bfr[s][ks] = Mma<bf16>::from_acc(M[s][ks >> 1], ks, g[s]);
      bf16x8 dg[SPW];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        // the copies of chunk j + 1 are spread over the products, so the address unit
        // drains them in the background instead of stalling every wave at once (after
        // the last step this copies chunk nsteps <= N - 1 into the idle buffer: in
        // bounds, never read, and waited for before the kernel ends)
#pragma unroll
        for (int d = 0; d < NDW; ++d)
          if (f == d * NFA / NDW) {
#ifdef HLA_SPREAD_MASK
            __builtin_amdgcn_sched_barrier(HLA_SPREAD_MASK);
#endif
            issue_one(j + 1, d, nA, nB);
#ifdef HLA_SPREAD_MASK
            __builtin_amdgcn_sched_barrier(HLA_SPREAD_MASK);
#endif
          }
        const bf16x8 af = ring[f % PF];
        if (f + PF < NF) ring[f % PF] = frag(cA, cB, f + PF);
        const int rt = (f < NFA ? f : f - NFA) % NRT;
        if (f >= NFA && (f - NFA) % NRT == 0) {
          const int kd = (f - NFA) / NRT;
#pragma unroll
          for (int s = 0; s < SPW; ++s) {
            const uint32_t gb = (uint32_t)__builtin_bit_cast(unsigned short, (bf16)g[s]);
            const uint32_t g2 = gb | (gb << 16);
            uint32_t d4[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) d4[d] = pat[kd][d] & g2;
            dg[s] = __builtin_bit_cast(bf16x8, d4);
          }
        }
#pragma unroll
        for (int s = 0; s < SPW; ++s)
          M[s][rt] = Mma<bf16>::mma(af, f < NFA ? bfr[s][f / NRT] : dg[s], M[s][rt]);
      }
#ifdef HLA_SGB
      // instruction order of the block: the ring prologue, then per fragment its SPW
      // products followed by the refill of its ring slot, with the copy instructions
      // spread evenly in front of the fragments they were placed at
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int d = 0; d < NDW; ++d)
          if (f == d * NFA / NDW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, SPW, 0);
        if (f + PF < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#endif
    } else if (more) {
      issue(j + 1, nA, nB);
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s)
      if (qi[s] == j + 1 && qi[s] < N) write_state(s);
    if (more) {
      wait_copies();
      __syncthreads();
    }
  };

  if (nsteps > 0) {
    issue(0, sA0, sB0);
    wait_copies();
    __syncthreads();
  }
  for (int j = 0; j < nsteps; j += 2) {
    step(j, sA0, sB0, sA1, sB1);
    if (j + 1 < nsteps) step(j + 1, sA1, sB1, sA0, sB0);
  }
  wait_copies();
}

template <int DK, int DV, int NW, int SPW, int PF>
static hipError_t launch_compose_bf16_t(const RouteArgs& a, hipStream_t s) {
  constexpr int QG = NW * SPW / (DV / 32);
  const int64_t ng = (a.N + QG - 1) / QG;
  const int64_t nb = ng * a.B * a.H;
  TimedLaunch tl(HLA_KERNEL_COMPOSE, s);
  hipLaunchKernelGGL((compose_bf16_kernel<DK, DV, NW, SPW, PF>), dim3((unsigned)nb), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compose_bf16(const RouteArgs& a, int dk, int dv, hipStream_t s) {
  const int64_t n_pairs = a.B * a.H * (int64_t)a.N * dk * (dk / 16);
  if (n_pairs > 0) {
    const unsigned nb = (unsigned)((n_pairs + 255) / 256);
    if (dk == 64)
      hipLaunchKernelGGL(prep_at_kernel<64>, dim3(nb), dim3(256), 0, s, reinterpret_cast<const bf16*>(a.At),
                         reinterpret_cast<bf16*>(a.At_prep), n_pairs);
    else
      hipLaunchKernelGGL(prep_at_kernel<128>, dim3(nb), dim3(256), 0, s, reinterpret_cast<const bf16*>(a.At),
                         reinterpret_cast<bf16*>(a.At_prep), n_pairs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#ifndef HLA_COMPOSE_SHAPE
#define HLA_COMPOSE_SHAPE 8, 2, 4
#endif
  if (dk == 64 && dv == 64) return launch_compose_bf16_t<64, 64, HLA_COMPOSE_SHAPE>(a, s);
  if (dk == 64 && dv == 128) return launch_compose_bf16_t<64, 128, HLA_COMPOSE_SHAPE>(a, s);
  if (dk == 128 && dv == 64) return launch_compose_bf16_t<128, 64, HLA_COMPOSE_SHAPE>(a, s);
  return launch_compose_bf16_t<128, 128, HLA_COMPOSE_SHAPE>(a, s);
}

}  // namespace hla
