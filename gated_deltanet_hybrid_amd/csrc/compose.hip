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
//   * g Bc_j is added on the vector ALU, not the matrix cores: Bc_j is stored in the order
//     of the accumulator elements, so a lane reads the 16 values of one row tile as two
//     16-byte units and adds g times each with a packed bf16 dot product (v_dot2 of the
//     pair with (g, 0) or (0, g)) straight into the float32 accumulator;
//   * (At_j - I, Bc_j) of the next history chunk are copied global -> LDS asynchronously
//     (global_load_lds, 16 bytes per lane, every instruction a contiguous 1 KiB source)
//     while the current one is multiplied;
//   * a prep pass writes (At_j - I) and Bc_j in the exact byte order of their LDS images:
//     every fragment is one conflict-free 16-byte LDS read at a lane-constant address plus
//     a compile-time offset, which leaves registers for a ring of fragment reads in flight;
//   * gates sit in one register per query chunk (64 history chunks per refill) and are
//     broadcast with readlane, so the loop touches no other memory;
//   * each XCD works through its heads one at a time, longest chain first, so the 32
//     workgroups running on an XCD sweep the same head's history (L2 reuse of At_j, Bc_j).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef float f32x4v __attribute__((ext_vector_type(4)));

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

// Bc_j in the order of the composition's accumulators.  A lane (column c32 of column tile
// ct, half hh = lane / 32) holds in row tile rt the rows rt*32 + 8 g + 4 hh + i (g, i =
// 0..3) as its accumulator elements e = 4 g + i.  Unit (ct, rt, p) of the image is 1 KiB:
// lane L = 32 hh + c32 at bytes 16 L .. 16 L + 15, holding elements e = 8 p .. 8 p + 7
// of that lane, so the composition reads them with one conflict-free 16-byte LDS read.
template <int DK, int DV>
__global__ __launch_bounds__(256) void prep_bc_kernel(const bf16* __restrict__ Bc, bf16* __restrict__ Bp, int64_t n_units) {
  // one thread per 16-byte unit; consecutive threads take consecutive columns, so each of
  // the 8 rows a unit gathers is read as one 64-byte run per half wave
  const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (t >= n_units) return;
  constexpr int NRT = DK / 32;
  const int L = (int)(t & 63), c32 = L & 31, hh = L >> 5;
  const int64_t u = t >> 6;  // unit over all (b, h, j, ct, rt, p)
  const int p = (int)(u & 1), rt = (int)((u >> 1) % NRT);
  const int64_t cu = (u >> 1) / NRT;
  const int ct = (int)(cu % (DV / 32));
  const int64_t chunk = cu / (DV / 32);
  const bf16* src = Bc + chunk * DK * DV + ct * 32 + c32;
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int el = 8 * p + e;
    out[e] = src[(rt * 32 + (el >> 2) * 8 + hh * 4 + (el & 3)) * DV];
  }
  *reinterpret_cast<bf16x8*>(Bp + t * 8) = out;
}

// Order of the A fragments within one composition step: position q -> fragment index
// kb * NRT + rt.  Four blocks (R0,K0) (R0,K1) (R1,K0) (R1,K1), R0 / R1 the row tiles
// [0, NRT/2) and [NRT/2, NRT), K0 / K1 the k-steps [0, NRT) and [NRT, 2 NRT); k-step
// outer, row tile inner.
template <int NRT>
__host__ __device__ constexpr int compose_seq(int q) {
  constexpr int RH = NRT / 2, HALF = 2 * NRT * RH;
  const int rbase = q >= HALF ? RH : 0;
  q %= HALF;
  return (q / RH) * NRT + rbase + q % RH;
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
  const bf16* Bg = reinterpret_cast<const bf16*>(a.Bc_prep) + bh * N * (int64_t)DK * DV;
  const float* gts = a.gates + bh * (int64_t)N * N;
  const uint8_t* msk = a.mask + bh * (int64_t)N * N;
  float* Sout = a.S_routed + bh * (int64_t)N * DK * DV;

  // Async copy of (At_j, Bc_j) into LDS, 1 KiB blocks m = w, w + NW, ... per wave, each a
  // contiguous block of the prepared images.
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
      __builtin_amdgcn_global_load_lds(bs + m * 1024 + lane * 16,
                                       (lds_void_t*)(reinterpret_cast<char*>(dB) + m * 1024), 16, 0, 0);
    }
  };
  auto issue = [&](int j, bf16* dA, bf16* dB) {
#pragma unroll
    for (int d = 0; d < NDW; ++d) issue_one(j, d, dA, dB);
  };
  auto wait_copies = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // fragment reads: row rt*32 + c32, logical half hh of k block kb (At); the lane's own
  // unit of Bc image block (ct, rt, p)
  const int rd = c32 * 32 + ((hh ^ (((c32 >> 2) ^ (c32 >> 3)) & 1)) << 4);
  constexpr int NFA = NKS * NRT;
  auto frag = [&](const bf16* cA, int f) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(cA) + rd + (f / NRT) * BLK + (f % NRT) * 1024);
  };
  auto bc_unit = [&](const bf16* cB, int rt, int p) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(cB) + ((ct * NRT + rt) * 2 + p) * 1024 +
                                            lane * 16);
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
  // Checkpoint of the chains that cross history step jb = b K (taken before that step), in
  // the accumulator's lane order: 16 floats per lane and row tile, stored non-temporally.
  auto keep_state = [&](int jb) {
    const int b = jb / a.ckpt_K;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (qi[s] <= jb || qi[s] >= N) continue;
      float* ck = a.ckpt + (bh * a.ckpt_nck + ckpt_slot(N, a.ckpt_K, b, qi[s])) * (int64_t)DK * DV;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f32x4v* dst = reinterpret_cast<f32x4v*>(ck + ((int64_t)(ct * NRT + rt) * 64 + lane) * 16);
#pragma unroll
        for (int e = 0; e < 16; e += 4)
          __builtin_nontemporal_store(f32x4v{M[s][rt][e], M[s][rt][e + 1], M[s][rt][e + 2], M[s][rt][e + 3]}, &dst[e / 4]);
      }
    }
  };

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

  // One history chunk: multiply with the (At_j - I, Bc_j) in (cA, cB) while the copy of
  // chunk j + 1 lands in (nA, nB).  The products of a step run in four blocks
  //   (R0,K0) (R0,K1) (R1,K0) (R1,K1)
  // (R0 / R1 the upper and lower row tiles of the state slice, K0 / K1 the matching halves
  // of the k range), and the vector work of the step is spread over them so that it runs
  // while the matrix cores work on other accumulators:
  //   (R0,K0): the K1 half of this step's B operand (scale by the gate, round to bf16),
  //            from rows R1, which the previous step finished and this step has not
  //            touched yet;
  //   (R0,K1): g Bc_j added to rows R1, which no product of this step has touched yet;
  //   (R1,K0): g Bc_j added to rows R0, whose products for this step are issued;
  //   (R1,K1): the K0 half of the next step's B operand, from rows R0 (now final), into
  //            registers whose last reader was (R1,K0).
  constexpr int RH = NRT / 2, KH = NKS / 2, BLK_Q = KH * RH;
  bf16x8 bfr[SPW][NKS];
  auto convert = [&](int s, int ks, float gs) { bfr[s][ks] = Mma<bf16>::from_acc(M[s][ks >> 1], ks, gs); };
  float gnext[SPW];
  auto read_gates = [&](int j, float* out) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) out[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(greg[s]), j & 63));
  };

  auto step = [&](int j, const bf16* cA, const bf16* cB, bf16* nA, bf16* nB) {
    float g[SPW];
    bool any = false;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      g[s] = gnext[s];
      any |= (g[s] != 0.f);
    }
    // gates of the next step (a new block of 64 is loaded when it starts)
    if (((j + 1) & 63) == 0) load_gates((j + 1) >> 6);
    read_gates(j + 1, gnext);
    const bool more = j + 1 < nsteps;
    if (any) {
      // (g, 0) and (0, g) as bf16 pairs: the dot product of a Bc pair with one of them is
      // g times its first or its second element
      bf16x2 gp[SPW][2];
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        const bf16 gb = (bf16)g[s], z = (bf16)0.f;
        gp[s][0] = bf16x2{gb, z};
        gp[s][1] = bf16x2{z, gb};
      }
      bf16x8 ring[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) ring[p] = frag(cA, compose_seq<NRT>(p));
      bf16x8 bcv[RH][2];  // Bc units of the half being added
      constexpr int NC = SPW * KH;          // conversions per half
      constexpr int NB = SPW * RH * 16;     // Bc elements per half
      static_for<0, NFA>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        constexpr int f = compose_seq<NRT>(q);
        constexpr int blk = q / BLK_Q, qb = q % BLK_Q;
        static_for<0, NDW>([&](auto dc) {
          constexpr int d = decltype(dc)::value;
          if constexpr (q == d * NFA / NDW) issue_one(j + 1, d, nA, nB);
        });
        // Bc units: rows R1 at the start of (R0,K0); unit r of rows R0 at the first position
        // of (R0,K1) after its R1 unit was last used there, or at the start of (R1,K0)
        if constexpr (q == 0) {
#pragma unroll
          for (int r = 0; r < RH; ++r)
#pragma unroll
            for (int p = 0; p < 2; ++p) bcv[r][p] = bc_unit(cB, RH + r, p);
        }
        static_for<0, RH>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          constexpr int last = ((r + 1) * SPW * 16 - 1) * BLK_Q / NB;  // last position using unit r
          if constexpr (q == BLK_Q + last + 1) {
#pragma unroll
            for (int p = 0; p < 2; ++p) bcv[r][p] = bc_unit(cB, r, p);
          }
        });
        const bf16x8 af = ring[q % PF];
        if constexpr (q + PF < NFA) ring[q % PF] = frag(cA, compose_seq<NRT>(q + PF));
        if constexpr (blk == 0 || blk == 3) {
          static_for<0, NC>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            if constexpr (c * BLK_Q / NC == qb) {
              if constexpr (blk == 0)
                convert(c % SPW, KH + c / SPW, g[c % SPW]);
              else
                convert(c % SPW, c / SPW, gnext[c % SPW]);
            }
          });
        } else {
          // g Bc_j into rows R1 (block 1) or R0 (block 2): element x of the half is slice
          // x % SPW, row tile x / SPW / 16, accumulator element x / SPW % 16
          constexpr int r0 = blk == 1 ? RH : 0;
          static_for<0, NB>([&](auto xc) {
            constexpr int x = decltype(xc)::value;
            if constexpr (x * BLK_Q / NB == qb) {
              constexpr int s = x % SPW, e = (x / SPW) % 16, r = x / SPW / 16;
              const bf16x8 u = bcv[r][e >> 3];
              const bf16x2 pr = __builtin_shufflevector(u, u, (e & 7) & ~1, ((e & 7) & ~1) + 1);
              M[s][r0 + r][e] = __builtin_amdgcn_fdot2_f32_bf16(pr, gp[s][e & 1], M[s][r0 + r][e], false);
            }
          });
        }
        constexpr int rt = f % NRT;
#pragma unroll
        for (int s = 0; s < SPW; ++s) M[s][rt] = Mma<bf16>::mma(af, bfr[s][f / NRT], M[s][rt]);
      });
    } else {
      if (more) issue(j + 1, nA, nB);
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int ks = 0; ks < KH; ++ks) convert(s, ks, gnext[s]);
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s)
      if (qi[s] == j + 1 && qi[s] < N) write_state(s);
    if (a.ckpt && (j + 1) % a.ckpt_K == 0) keep_state(j + 1);
    if (more) {
      wait_copies();
      __syncthreads();
    }
  };

  if (nsteps > 0) {
    issue(0, sA0, sB0);
    load_gates(0);
    read_gates(0, gnext);
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int ks = 0; ks < KH; ++ks) convert(s, ks, gnext[s]);
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
    const int64_t n_units = a.B * a.H * (int64_t)a.N * dk * dv / 8;
    const unsigned nu = (unsigned)((n_units + 255) / 256);
    const bf16* bc = reinterpret_cast<const bf16*>(a.Bc);
    bf16* bp = reinterpret_cast<bf16*>(a.Bc_prep);
    if (dk == 64 && dv == 64)
      hipLaunchKernelGGL((prep_bc_kernel<64, 64>), dim3(nu), dim3(256), 0, s, bc, bp, n_units);
    else if (dk == 64 && dv == 128)
      hipLaunchKernelGGL((prep_bc_kernel<64, 128>), dim3(nu), dim3(256), 0, s, bc, bp, n_units);
    else if (dk == 128 && dv == 64)
      hipLaunchKernelGGL((prep_bc_kernel<128, 64>), dim3(nu), dim3(256), 0, s, bc, bp, n_units);
    else
      hipLaunchKernelGGL((prep_bc_kernel<128, 128>), dim3(nu), dim3(256), 0, s, bc, bp, n_units);
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
  }
  // 8 waves of 2 state slices each, a 4-deep ring of fragment reads
  if (dk == 64 && dv == 64) return launch_compose_bf16_t<64, 64, 8, 2, 4>(a, s);
  if (dk == 64 && dv == 128) return launch_compose_bf16_t<64, 128, 8, 2, 4>(a, s);
  if (dk == 128 && dv == 64) return launch_compose_bf16_t<128, 64, 8, 2, 4>(a, s);
  return launch_compose_bf16_t<128, 128, 8, 2, 4>(a, s);
}

}  // namespace hla
