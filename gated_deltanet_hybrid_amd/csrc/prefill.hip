// Native chunkwise prefill (bf16 inputs, float32 state) in two passes that never form the
// chunk maps (At, Bc) nor write any state to HBM.
//
// [HLA] Methodology paragraph 1: within a piece of n <= 64 tokens (padded to 64 with
// beta = 0, alpha = 1, the identity map) that starts from state M (stored orientation,
// M = S^T [dk, dv]),
//   g_t = sum_{s<=t} log alpha_s,  gamma_t = exp(g_t),  Gamma_ts = exp(g_t - g_s) (s <= t),
//   L = strictly_lower(diag(beta) (K K^T) o Gamma),  X = (I + L)^-1,
//   W = X diag(beta gamma) K,  U = X diag(beta) V,  E = U - W M  (the deltas actually written),
//   O = diag(gamma) Q M + ((Q K^T) o Gamma) E,
//   M_next = gamma_63 M + K^T diag(D) E,  D_s = exp(g_63 - g_s).
// Every decay is the exp (or exp2) of a difference of log-decays, never exp(-g).
//
// Pass 1, ut_kernel (one workgroup per (b, h, piece), all pieces at once): everything that
// does not depend on the state -- the decays, the blocked inverse X, W and U, P -- into a
// per-piece record whose matrices are stored as the second pass's MFMA fragments.  The
// inverse is a chain of dependent LDS phases, so it runs here, many pieces per CU at once,
// instead of on the sequential path.
//
// Pass 2, state_kernel (one workgroup per (b, h), one wave per 32 state columns): the state
// runs through the pieces in order, its 32 columns held by one wave in MFMA accumulators
// (M [dk x 32], four 32 x 32 tiles) for the whole pass.  Per piece:
//   E = U + (-W) M            (U seeds the accumulators, M's bf16 copy is the B operand)
//   O = gamma (Q M) + P E     (E's bf16 copy is the B operand)
//   M <- gamma_63 M + K^T (D E)
// Every B operand is an accumulator tile rounded to bf16 in place, because the A operands
// (-W, Q, K^T, P) were stored with their k values in the accumulator's row order; so a
// wave never exchanges state with another, and the only barrier per piece guards the
// double-buffered LDS copy of the records (global_load_lds, issued one piece ahead).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTiny = 1.17549435e-38f;  // log alpha is clamped here: alpha = 0 (a reset) stays finite
}  // namespace

template <int DK, int DV>
__global__ __launch_bounds__(512, 4) void ut_kernel(UtArgs a) {
  constexpr int C = kChunk;
  constexpr int NT = 512;
  constexpr int PT = C + 8;   // bf16 pitch of [d][t] rows
  constexpr int PX = C + 4;   // fp32 pitch of L and X
  constexpr int NDT = DK / 32, NVT = DV / 32;
  constexpr int KPT = DK * C / 8 / NT, VPT = DV * C / 8 / NT;  // 16-byte units per thread
  static_assert(KPT >= 1 && VPT >= 1, "units per thread");
  static_assert(2 * NDT <= 8 && 2 * NVT <= 8, "one W and one U tile per wave at most");

  __shared__ __attribute__((aligned(16))) bf16 KT[DK * PT];
  __shared__ __attribute__((aligned(16))) bf16 VT[DV * PT];
  // L and X, and before them (phase A) the row-major staging copies of K and V
  __shared__ __attribute__((aligned(16))) float LX[2 * C * PX];
  float* const Lb = LX;
  float* const Xb = LX + C * PX;
  __shared__ __attribute__((aligned(16))) float s_beta[C], s_g2[C], s_bg[C];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t id = blockIdx.x;
  const int c = (int)(id % a.N);
  const int64_t bh = id / a.N;
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)c * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;
  const bf16* kg = reinterpret_cast<const bf16*>(a.k);
  const bf16* vg = reinterpret_cast<const bf16*>(a.v);
  char* rec = static_cast<char*>(a.rec) + id * ut_record_bytes(DK, DV);

  // ---- A. keys, values and queries: rows loaded whole (a wave reads 4 tokens' rows, 8
  // cache lines per instruction, instead of one 16-byte column unit of 64 tokens), staged
  // row-major in LDS (K and V in the space of L and X, Q in that of K^T), then K and V turned
  // into the [d][t] images KT and VT inside LDS; the K K^T and Q K^T operands and the
  // record's Q fragments from the staged rows; per-token decays (wave 0)
  constexpr int RK = DK + 8, RV = DV + 8;  // bf16 pitch of the staged rows
  static_assert(C * (RK + RV) * 2 <= 2 * C * PX * 4, "staging fits in L and X");
  bf16* const Ks = reinterpret_cast<bf16*>(LX);
  bf16* const Vs = Ks + C * RK;
  // K K^T lower tiles (0,0), (1,0), (1,1) on waves 0-2 and, when outputs are wanted, the
  // same tiles of Q K^T on waves 3-5: both operands are rows (8 consecutive dk per lane),
  // read from the staged copies (K zero past the end)
  const bool want_p = a.q != nullptr;
  const int job = w < 3 ? w : w - 3;
  const int tm = job == 0 ? 0 : 1, tn = job == 2 ? 1 : 0;
  bf16x8 fa[DK / 16], fb[DK / 16];
  constexpr int NQ = 2 * (DK / 16), NQW = (NQ + 7) / 8;
  // Q rows (outputs only) are staged row-major in the space of the K^T image, which is
  // free until K is transposed at the end of phase A
  static_assert(C * RK <= DK * PT, "Q staging fits in K^T");
  bf16* const Qs = KT;
  {
    // every load first (rows past the end of a partial piece read its last row, in bounds),
    // then the zero padding where the values are stored, so no load waits for another
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // (not uint4: kept in registers)
    u32x4 rk[KPT], rv[VPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + NT * j, t = i / (DK / 8), u = i % (DK / 8);
      rk[j] = *reinterpret_cast<const u32x4*>(kg + (row0 + (t < n ? t : n - 1) * a.H) * DK + u * 8);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = tid + NT * j, t = i / (DV / 8), u = i % (DV / 8);
      rv[j] = *reinterpret_cast<const u32x4*>(vg + (row0 + (t < n ? t : n - 1) * a.H) * DV + u * 8);
    }
    u32x4 rq[KPT];
    if (want_p) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int i = tid + NT * j, t = i / (DK / 8), u = i % (DK / 8);
        rq[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(a.q) + (row0 + (t < n ? t : n - 1) * a.H) * DK + u * 8);
      }
    }
    float bt = 0.f, ra = 1.f;
    if (tid < C) {
      const int64_t r = row0 + (int64_t)(tid < n ? tid : n - 1) * a.H;
      bt = a.beta[r];
      ra = a.alpha[r];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + NT * j, t = i / (DK / 8), u = i % (DK / 8);
      *reinterpret_cast<u32x4*>(Ks + t * RK + u * 8) = t < n ? rk[j] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = tid + NT * j, t = i / (DV / 8), u = i % (DV / 8);
      *reinterpret_cast<u32x4*>(Vs + t * RV + u * 8) = t < n ? rv[j] : u32x4{0u, 0u, 0u, 0u};
    }
    if (want_p) {
      // (rows past the end hold the last row: their results are never used)
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int i = tid + NT * j, t = i / (DK / 8), u = i % (DK / 8);
        *reinterpret_cast<u32x4*>(Qs + t * RK + u * 8) = rq[j];
      }
    }
    if (tid < C) {
      float x = 0.f;
      if (tid < n) {
        x = logf(fmaxf(ra, kTiny));
      } else {
        bt = 0.f;
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {  // inclusive prefix sum over wave 0
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      s_beta[tid] = bt;
      s_g2[tid] = x * kLog2e;
      s_bg[tid] = bt * expf(x);
      const float x_end = __shfl(x, 63, 64);
      float* gd = reinterpret_cast<float*>(rec + ut_off_gd(DK, DV));
      gd[tid] = expf(x);
      gd[C + tid] = expf(x_end - x);
    }
  }
  __syncthreads();
  // the [d][t] images: unit (channel d, tokens 8 g .. 8 g + 7), lanes along d, so that the
  // eight 2-byte reads of a unit are consecutive across the wave; V's first, and the Q
  // operands read from their staging before K's image overwrites it
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int i = tid + NT * j, d = i % DV, g = i / DV;
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = Vs[(g * 8 + e) * RV + d];
    *reinterpret_cast<bf16x8*>(VT + d * PT + g * 8) = x;
  }
  if (want_p) {
    if (w >= 3 && w < 6) {
      const bf16* pa = Qs + (tm * 32 + c32) * RK + hh * 8;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) fa[ks] = *reinterpret_cast<const bf16x8*>(pa + ks * 16);
    }
    // the record's Q fragments, stored here (fragment min(w + 8 j, NQ - 1) of each wave)
#pragma unroll
    for (int j = 0; j < NQW; ++j) {
      const int fq = min(w + 8 * j, NQ - 1), tt = fq / (DK / 16), ks = fq % (DK / 16);
      reinterpret_cast<bf16x8*>(rec + ut_off_q(DK, DV))[fq * 64 + lane] =
          Mma<bf16>::load_clayout(Qs + (tt * 32 + c32) * RK, ks, hh);
    }
  }
  // the K operands of the K K^T (waves 0-2) and Q K^T (waves 3-5) tiles from the staged rows
  if (w < 3 || (want_p && w < 6)) {
    const bf16* pb = Ks + (tn * 32 + c32) * RK + hh * 8;
    if (w < 3) {
      const bf16* pa = Ks + (tm * 32 + c32) * RK + hh * 8;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) fa[ks] = *reinterpret_cast<const bf16x8*>(pa + ks * 16);
    }
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) fb[ks] = *reinterpret_cast<const bf16x8*>(pb + ks * 16);
  }
  if (want_p) __syncthreads();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + NT * j, d = i % DK, g = i / DK;
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = Ks[(g * 8 + e) * RK + d];
    *reinterpret_cast<bf16x8*>(KT + d * PT + g * 8) = x;
  }
  __syncthreads();

  // ---- B. L = strictly_lower(diag(beta) (K K^T) o Gamma); P = (Q K^T) o Gamma into the
  // record as fragments (wave 6 writes the zero upper tile's two); X = 0
  if (want_p && w >= 3 && w < 6) {
    // tile (t block tm, s block tn) of P computed as K Q^T: the accumulator holds, for the
    // lane's token t, the tokens s in the k order of P's fragments
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) acc = Mma<bf16>::mma(fb[ks], fa[ks], acc);
    const float gt = s_g2[tm * 32 + c32];
    const int t = tm * 32 + c32;
    float gsv[16];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<float4*>(gsv + 4 * r) = *reinterpret_cast<const float4*>(s_g2 + tn * 32 + r * 8 + hh * 4);
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int sx = tn * 32 + acc_row(e, hh);
      const bf16 v = (bf16)((sx <= t) ? __builtin_amdgcn_exp2f(gt - gsv[e]) * acc[e] : 0.f);
      if (e < 8) lo[e] = v; else hi[e - 8] = v;
    }
    bf16x8* po = reinterpret_cast<bf16x8*>(rec + ut_off_p(DK, DV));
    po[(tm * 4 + 2 * tn) * 64 + lane] = lo;
    po[(tm * 4 + 2 * tn + 1) * 64 + lane] = hi;
  } else if (want_p && w == 6) {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
    bf16x8* po = reinterpret_cast<bf16x8*>(rec + ut_off_p(DK, DV));
    po[2 * 64 + lane] = z;
    po[3 * 64 + lane] = z;
  }
  if (w < 3) {
    // a padded row's product is zeroed below: its beta is 0 (row t) or the row is past the
    // end (column s >= n only meets rows t > s >= n)
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) acc = Mma<bf16>::mma(fa[ks], fb[ks], acc);
    const int s = tn * 32 + c32;
    const float gs = s_g2[s];
    float gt[16], bt[16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4*>(gt + 4 * r) = *reinterpret_cast<const float4*>(s_g2 + tm * 32 + r * 8 + hh * 4);
      *reinterpret_cast<float4*>(bt + 4 * r) = *reinterpret_cast<const float4*>(s_beta + tm * 32 + r * 8 + hh * 4);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      Lb[t * PX + s] = (s < t) ? bt[e] * __builtin_amdgcn_exp2f(gt[e] - gs) * acc[e] : 0.f;
    }
  }
  for (int i = tid; i < C * PX; i += NT) Xb[i] = 0.f;
  __syncthreads();

  // ---- C. X = (I + L)^-1, blocked by 16: the diagonal blocks by substitution (wave 0);
  // meanwhile waves 1-7 store the K^T fragments (from K^T in LDS; padded tokens are zero)
  if (w > 0) {
    constexpr int NKT = (DK / 32) * 4;
    for (int f = w - 1; f < NKT; f += 7) {
      const int rt = f >> 2, ks = f & 3;
      reinterpret_cast<bf16x8*>(rec + ut_off_kt(DK))[f * 64 + lane] =
          Mma<bf16>::load_clayout(KT + (rt * 32 + c32) * PT, ks, hh);
    }
  }
  if (tid < 64) {
    const int bi = tid >> 4, cc = tid & 15, base = bi * 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int q2 = 0; q2 < r; ++q2) s -= Lb[(base + r) * PX + base + q2] * x[q2];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Xb[(base + r) * PX + base + cc] = x[r];
  }
  __syncthreads();
  // the blocks below the diagonal, from (I + L) X = I: X_ik = sum_m Z_im X_mk with
  // Z_im = -X_ii L_im (m < i), kept in L's unused block (m, i) above the diagonal; then X by
  // sub-diagonal d = i - k
  for (int e = tid; e < 6 * 256; e += NT) {
    const int bz = e >> 8, r = (e >> 4) & 15, cc = e & 15;
    const int i = bz < 1 ? 1 : (bz < 3 ? 2 : 3), m = bz - i * (i - 1) / 2;
    float z = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 16; ++q2) z -= Xb[(i * 16 + r) * PX + i * 16 + q2] * Lb[(i * 16 + q2) * PX + m * 16 + cc];
    Lb[(m * 16 + r) * PX + i * 16 + cc] = z;
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    for (int e = tid; e < (4 - d) * 256; e += NT) {
      const int k = e >> 8, i = k + d, r = (e >> 4) & 15, cc = e & 15;
      float x = 0.f;
      for (int m = k; m < i; ++m)
#pragma unroll
        for (int q2 = 0; q2 < 16; ++q2) x += Lb[(m * 16 + r) * PX + i * 16 + q2] * Xb[(m * 16 + q2) * PX + k * 16 + cc];
      Xb[(i * 16 + r) * PX + k * 16 + cc] = x;
    }
    __syncthreads();
  }

  // ---- F. W^T tile (dk block db, token block tt) on wave 2 db + tt -> -W fragments (tt,
  // 2 db) and (tt, 2 db + 1);  U tile (token block tt, column block ct) on wave 2 ct + tt
  // -> the E accumulator order.  X enters as hi + lo bf16 parts (about 16 mantissa bits).
  // A wave's W tile and U tile share the token block tt, so X's rows are read once per
  // k-step for both, and the two accumulator chains interleave on the matrix cores.
  const bool do_w = w < 2 * NDT, do_u = w < 2 * NVT;
  if (do_w || do_u) {
    // W^T = K^T diag(beta gamma) X^T: A = K^T rows (dk block jb), B = X rows (token t), k = s;
    // U = X diag(beta) V: A = X rows (token t), B = V^T rows (column block jb), k = s
    const int tt = w & 1, jb = w >> 1;
    const float* xrow = Xb + (tt * 32 + c32) * PX;
    const bf16* arow = KT + (jb * 32 + c32) * PT;  // (read only by W's waves)
    const bf16* brow = VT + (jb * 32 + c32) * PT;  // (read only by U's waves)
    f32x16 acc_w = zero16(), acc_u = zero16();
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const int s0 = ks * 16 + hh * 8;
      float xv[8], gv[8], bv[8];
      *reinterpret_cast<float4*>(xv) = *reinterpret_cast<const float4*>(xrow + s0);
      *reinterpret_cast<float4*>(xv + 4) = *reinterpret_cast<const float4*>(xrow + s0 + 4);
      *reinterpret_cast<float4*>(gv) = *reinterpret_cast<const float4*>(s_bg + s0);
      *reinterpret_cast<float4*>(gv + 4) = *reinterpret_cast<const float4*>(s_bg + s0 + 4);
      *reinterpret_cast<float4*>(bv) = *reinterpret_cast<const float4*>(s_beta + s0);
      *reinterpret_cast<float4*>(bv + 4) = *reinterpret_cast<const float4*>(s_beta + s0 + 4);
      // X enters as hi + lo bf16 parts (about 16 mantissa bits)
      bf16x8 hw, lw, hu, lu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x_w = xv[e] * gv[e], x_u = xv[e] * bv[e];
        hw[e] = (bf16)x_w;
        lw[e] = (bf16)(x_w - (float)hw[e]);
        hu[e] = (bf16)x_u;
        lu[e] = (bf16)(x_u - (float)hu[e]);
      }
      bf16x8 af, bf;
      if (do_w) {
        af = Mma<bf16>::load_plain(arow, ks, hh);
        acc_w = Mma<bf16>::mma(af, hw, acc_w);
      }
      if (do_u) {
        bf = Mma<bf16>::load_plain(brow, ks, hh);
        acc_u = Mma<bf16>::mma(hu, bf, acc_u);
      }
      if (do_w) acc_w = Mma<bf16>::mma(af, lw, acc_w);
      if (do_u) acc_u = Mma<bf16>::mma(lu, bf, acc_u);
    }
    if (do_w) {
      bf16x8 lo8, hi8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo8[e] = (bf16)(-acc_w[e]);
        hi8[e] = (bf16)(-acc_w[e + 8]);
      }
      bf16x8* wo = reinterpret_cast<bf16x8*>(rec);
      wo[(tt * (DK / 16) + 2 * jb) * 64 + lane] = lo8;
      wo[(tt * (DK / 16) + 2 * jb + 1) * 64 + lane] = hi8;
    }
    if (do_u) {
      bf16x8 lo8, hi8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo8[e] = (bf16)acc_u[e];
        hi8[e] = (bf16)acc_u[e + 8];
      }
      bf16x8* uo = reinterpret_cast<bf16x8*>(rec + ut_off_u(DK)) + ((jb * 2 + tt) * 64 + lane) * 2;
      uo[0] = lo8;
      uo[1] = hi8;
    }
  }
}


template <int DK, int DV, int NWB, bool WANT_O>
__global__ __launch_bounds__(256, 1) void state_kernel(UtArgs a) {
  constexpr int C = kChunk;
  constexpr int NCB = DV / 32;        // 32-column slices of the state
  constexpr int NG = NCB / NWB;       // workgroups per (b, h): NWB slices (waves) each
  // Four waves per workgroup: the NWB that compute and, when NWB < 4, NH helpers that only
  // move records into LDS (plain 16-byte loads into registers, then LDS writes: the
  // asynchronous global -> LDS copy moves fewer bytes per clock and CU than the products
  // of a piece need).  Without helpers the compute waves copy with global_load_lds.
  constexpr int NTW = 4, NH = NTW - NWB;
  constexpr int NRT = DK / 32, NKS = DK / 16;
  // The part of a piece's record this workgroup stages in LDS, as 1 KiB blocks: -W and K^T
  // fragments, the U of its own slices, the decays, and (outputs) the Q and P fragments.
  constexpr int B_WK = (int)(ut_off_u(DK) / 1024), B_U = 4 * NWB, B_GD = 1;
  constexpr int B_QP = WANT_O ? (int)((ut_record_bytes(DK, DV) - ut_off_q(DK, DV)) / 1024) : 0;
  constexpr int B_QP_REAL = WANT_O ? 2 * NKS + 8 : 0;
  constexpr int NB_REAL = B_WK + B_U + B_GD + B_QP_REAL;
  constexpr int ND = (NB_REAL + NTW - 1) / NTW;  // copy instructions per wave and piece
  constexpr int NB = ND * NTW;                   // blocks per buffer (the extra ones repeat the decays)
  constexpr int RB = NB * 1024;
  static_assert(B_QP >= B_QP_REAL, "record layout");
  // LDS offsets within a buffer
  constexpr int L_KT = (int)ut_off_kt(DK), L_U = B_WK * 1024, L_GD = L_U + B_U * 1024, L_Q = L_GD + 1024,
                L_P = L_Q + 2 * NKS * 1024;
  // LDS buffers for the records of consecutive pieces: three when they fit and no outputs
  // are stored (the copy of a piece is issued NBUF - 1 pieces ahead), else two; separate
  // variables, so the copy into one is not taken to alias reads of another
  constexpr int NBUF = (NH == 0 && !WANT_O && 3 * RB <= 160 * 1024) ? 3 : 2;
  static_assert(NBUF * RB <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char buf0[RB];
  __shared__ __attribute__((aligned(16))) char buf1[RB];
  __shared__ __attribute__((aligned(16))) char buf2[NBUF == 3 ? RB : 16];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (b, h, slice group); with B H a multiple of 8 the groups of one (b, h) go to
  // the same XCD (workgroups go to the 8 XCDs round robin) and share its records in its L2
  const int64_t id = blockIdx.x;
  int64_t bh;
  int sg;
  if ((a.B * a.H) % 8 == 0) {
    const int64_t j = id >> 3;
    sg = (int)(j % NG);
    bh = (j / NG) * 8 + (id & 7);
  } else {
    sg = (int)(id % NG);
    bh = id / NG;
  }
  const int64_t h = bh % a.H, b = bh / a.H;
  const int cb = sg * NWB + (w < NWB ? w : 0);  // this wave's slice (helpers: unused)
  const int col0 = cb * 32;
  const int N = a.N;
  const int64_t RS = ut_record_bytes(DK, DV);
  const char* recs = static_cast<const char*>(a.rec) + bh * (int64_t)N * RS;

  // The copy of a record into LDS, ND instructions per wave, written out rather than through
  // the builtin: the compiler would otherwise place a wait for every copy in flight before
  // the first LDS read of each piece (it cannot tell the buffers apart), which serialises
  // the copy of the next piece with the current one.  The waits the copies need are the
  // explicit ones before each barrier below.
  auto src_block = [&](int m) -> int64_t {  // record offset of LDS block m
    if (m < B_WK) return (int64_t)m * 1024;
    if (m < B_WK + B_U) return ut_off_u(DK) + (int64_t)sg * NWB * 4096 + (int64_t)(m - B_WK) * 1024;
    if (m < B_WK + B_U + B_GD || m >= NB_REAL) return ut_off_gd(DK, DV);
    return ut_off_q(DK, DV) + (int64_t)(m - B_WK - B_U - B_GD) * 1024;
  };
  auto issue_one = [&](int c, char* dst, int i) __attribute__((always_inline)) {
    const char* src = recs + (int64_t)c * RS + lane * 16;
    const uint32_t ldst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst;
    const int m = w + i * NTW;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_nop 0"
                 :: "s"(ldst + m * 1024), "v"(src + src_block(m)) : "memory", "m0");
  };
  auto issue = [&](int c, char* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ND; ++i) issue_one(c, dst, i);
  };
  auto frag = [&](const char* base, int off, int f) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(base + off + f * 1024 + lane * 16);
  };

  // the state's 32 columns: M [dk x 32] as NRT accumulator tiles (dk = 32 rt + acc_row)
  f32x16 M[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    M[rt] = zero16();
    if (a.S0) {
      const float* s0 = a.S0 + bh * (int64_t)DK * DV + col0 + c32;
#pragma unroll
      for (int e = 0; e < 16; ++e) M[rt][e] = s0[(rt * 32 + acc_row(e, hh)) * DV];
    }
  }
  bf16x8 bM[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) bM[ks] = Mma<bf16>::from_acc(M[ks >> 1], ks, 1.f);

  // outputs as O^T tiles: lane c32 holds token 32 tt + c32, element e column
  // col0 + acc_row(e), so each group of four elements is one 16-byte store
  f32x16 OT[2];
  auto store_o = [&](int c) {
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = tt * 32 + c32;
      if (t < n) {
        float* ob = a.o + ((b * a.T + t0 + t) * a.H + h) * DV + col0 + hh * 4;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typedef float f4 __attribute__((ext_vector_type(4)));
          const f4 v = {OT[tt][4 * g], OT[tt][4 * g + 1], OT[tt][4 * g + 2], OT[tt][4 * g + 3]};
          __builtin_nontemporal_store(v, reinterpret_cast<f4*>(ob + g * 8));
        }
      }
    }
  };

  // The copy of a later piece is spread over the products of this one (copy instruction i
  // after product slot i NMF / ND), so the wave never stalls on a burst of memory
  // instructions while the matrix cores wait.
  constexpr int NMF = WANT_O ? 2 * NKS + 4 * (NRT + 2) : NKS + 4 * NRT;  // product slots per piece
  auto piece = [&](const char* cur, int c_ahead, char* ahead) __attribute__((always_inline)) {
    auto slot = [&](int k) __attribute__((always_inline)) {
      if (NH == 0 && c_ahead < N) {
#pragma unroll
        for (int i = 0; i < ND; ++i)
          if (i * NMF / ND == k) issue_one(c_ahead, ahead, i);
      }
    };
    // E = U + (-W) M and O^T = M^T Q^T, k-step by k-step: four independent accumulator
    // chains (E and O^T of both token tiles; without outputs, E's k range in two halves
    // instead), with the A fragments of the next PF k-steps read ahead from LDS.  The
    // B operand bf16(M) of E serves as the A operand of O^T (its lane holds a column of M),
    // and the Q fragments (lane = token) as its B operand.
    constexpr int PF = 3;
    bf16x8 fu[4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const bf16x8* u = reinterpret_cast<const bf16x8*>(cur + L_U) + ((w * 2 + tt) * 64 + lane) * 2;
      fu[2 * tt] = u[0];
      fu[2 * tt + 1] = u[1];
    }
    f32x16 E[2], E2[2];
    if constexpr (WANT_O) {
      bf16x8 rw[2][PF], rq[2][PF];
#pragma unroll
      for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          rw[tt][p] = frag(cur, 0, tt * NKS + p);
          rq[tt][p] = frag(cur, L_Q, tt * NKS + p);
        }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          E[tt][e] = (float)fu[2 * tt][e];
          E[tt][e + 8] = (float)fu[2 * tt + 1][e];
        }
        OT[tt] = zero16();
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          E[tt] = Mma<bf16>::mma(rw[tt][ks % PF], bM[ks], E[tt]);
          OT[tt] = Mma<bf16>::mma(bM[ks], rq[tt][ks % PF], OT[tt]);
          slot(ks * 2 + tt);
          if (ks + PF < NKS) {
            rw[tt][ks % PF] = frag(cur, 0, tt * NKS + ks + PF);
            rq[tt][ks % PF] = frag(cur, L_Q, tt * NKS + ks + PF);
          }
        }
      }
    } else {
      constexpr int KH = NKS / 2;
      bf16x8 rw[2][2][PF];  // [k half][tt][slot]
#pragma unroll
      for (int p = 0; p < PF; ++p)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) rw[hf][tt][p] = frag(cur, 0, tt * NKS + hf * KH + p);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          E[tt][e] = (float)fu[2 * tt][e];
          E[tt][e + 8] = (float)fu[2 * tt + 1][e];
        }
        E2[tt] = zero16();
      }
#pragma unroll
      for (int k2 = 0; k2 < KH; ++k2) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          E[tt] = Mma<bf16>::mma(rw[0][tt][k2 % PF], bM[k2], E[tt]);
          E2[tt] = Mma<bf16>::mma(rw[1][tt][k2 % PF], bM[KH + k2], E2[tt]);
          slot(k2 * 2 + tt);
          if (k2 + PF < KH) {
            rw[0][tt][k2 % PF] = frag(cur, 0, tt * NKS + k2 + PF);
            rw[1][tt][k2 % PF] = frag(cur, 0, tt * NKS + KH + k2 + PF);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) E[tt][e] += E2[tt][e];
    }
    const float* gam = reinterpret_cast<const float*>(cur + L_GD);
    const float* dec = gam + C;
    const float g_end = gam[C - 1];
    // B operands from E: bf16(E) (the A operand of E^T P^T) and bf16(D E) for the state
    // update (D_t per token)
    bf16x8 bE[4], bDE[4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float dv_[16];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4*>(dv_ + 4 * r) = *reinterpret_cast<const float4*>(dec + tt * 32 + r * 8 + hh * 4);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = E[tt][p * 8 + e];
          if constexpr (WANT_O) bE[tt * 2 + p][e] = (bf16)x;
          bDE[tt * 2 + p][e] = (bf16)(x * dv_[p * 8 + e]);
        }
      }
    }
    if constexpr (WANT_O) {
      // O = gamma (Q M): gamma of the lane's token
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float gt = gam[tt * 32 + c32];
#pragma unroll
        for (int e = 0; e < 16; ++e) OT[tt][e] *= gt;
      }
    }
    // M <- gamma_63 M + K^T (D E);  O^T += E^T P^T: per k-step (token block of 16) NRT + 2
    // products, fragments two k-steps ahead
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) M[rt][e] *= g_end;
    bf16x8 rk[2][NRT], rp[2][2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) rk[p][rt] = frag(cur, L_KT, rt * 4 + p);
      if constexpr (WANT_O) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) rp[p][tt] = frag(cur, L_P, tt * 4 + p);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        M[rt] = Mma<bf16>::mma(rk[ks & 1][rt], bDE[ks], M[rt]);
        slot((WANT_O ? 2 * NKS : NKS) + ks * (WANT_O ? NRT + 2 : NRT) + rt);
        if (ks + 2 < 4) rk[ks & 1][rt] = frag(cur, L_KT, rt * 4 + ks + 2);
      }
      if constexpr (WANT_O) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          OT[tt] = Mma<bf16>::mma(bE[ks], rp[ks & 1][tt], OT[tt]);
          slot(2 * NKS + ks * (NRT + 2) + NRT + tt);
          if (ks + 2 < 4) rp[ks & 1][tt] = frag(cur, L_P, tt * 4 + ks + 2);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bM[ks] = Mma<bf16>::from_acc(M[ks >> 1], ks, 1.f);
  };

  // Helper waves (NH > 0): blocks m = hlp, hlp + NH, ... of a piece's part, all loaded
  // unconditionally (blocks past the record's part repeat the decays into spare slots, so no
  // load waits behind a branch).  A piece's blocks are loaded into registers two pieces
  // ahead and written into LDS one piece ahead, so each load has a whole piece step to
  // arrive before its LDS write waits for it.
  constexpr int NDH = NH > 0 ? (NB_REAL + NH - 1) / NH : 1;
  static_assert(NH == 0 || NDH * NH <= NB, "helper slots within the buffer");
  const int hlp = w - NWB;

  // Per piece c: the stores of piece c - 1's outputs are issued, then piece c is computed
  // from its buffer; the copy of piece c + 1 into the other buffer is either spread over the
  // products by the computing waves (no helpers: global_load_lds, issued NBUF - 1 pieces
  // ahead) or made by the helpers.  Then every wave waits for its LDS operations (and,
  // without helpers, for its copies up to piece c + 1: with two buffers all of them, with
  // three all but the ND just issued, since the counter retires operations in issue order),
  // and a barrier makes that true for all waves before piece c + 1 reads its buffer or a
  // copy overwrites the buffer piece c read.  With helpers the computing waves issue no
  // loads and the helpers' loads of piece c + 2 stay in flight across the barrier.
  static_assert(ND < 64, "vmcnt range");
  auto barrier_after = [&](int c) __attribute__((always_inline)) {
    // (a plain s_barrier: __syncthreads' release fence would also wait for the loads
    // issued ahead)
    if constexpr (NH > 0)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (NBUF == 3 && c + NBUF - 1 < N)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(ND) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  auto step = [&](int c, const char* cur, char* ahead) __attribute__((always_inline)) {
    if constexpr (WANT_O) {
      if (c > 0) store_o(c - 1);
    }
    piece(cur, c + NBUF - 1, ahead);
    barrier_after(c);
  };
  if (N > 0) {
    issue(0, buf0);  // (every wave, global_load_lds)
    if (NBUF == 3 && N > 1) issue(1, buf1);

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  if constexpr (NH > 0) {
    if (w >= NWB) {
      // (a vector type, not uint4: the loop-carried array must stay in registers)
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
      u32x4 hreg[NDH];
      if (N > 1) {
        const char* src = recs + RS + lane * 16;
#pragma unroll
        for (int i = 0; i < NDH; ++i) hreg[i] = *reinterpret_cast<const u32x4*>(src + src_block(hlp + i * NH));
      }
      for (int c = 0; c < N; ++c) {
        char* ahead = (c & 1) ? buf0 : buf1;
        if (c + 1 < N) {
#pragma unroll
          for (int i = 0; i < NDH; ++i) *reinterpret_cast<u32x4*>(ahead + (hlp + i * NH) * 1024 + lane * 16) = hreg[i];
        }
        if (c + 2 < N) {
          const char* src = recs + (int64_t)(c + 2) * RS + lane * 16;
#pragma unroll
          for (int i = 0; i < NDH; ++i) hreg[i] = *reinterpret_cast<const u32x4*>(src + src_block(hlp + i * NH));
        }
        barrier_after(c);
      }
      return;
    }
  }
  static_assert(NH == 0 || NBUF == 2, "helpers fill two buffers");
  if constexpr (NBUF == 3) {
    for (int c = 0; c < N; c += 3) {
      step(c, buf0, buf2);
      if (c + 1 < N) step(c + 1, buf1, buf0);
      if (c + 2 < N) step(c + 2, buf2, buf1);
    }
  } else {
    for (int c = 0; c < N; c += 2) {
      step(c, buf0, buf1);
      if (c + 1 < N) step(c + 1, buf1, buf0);
    }
  }
  if (w >= NWB) return;
  if constexpr (WANT_O) {
    if (N > 0) store_o(N - 1);
  }
  if (a.S_final) {
    float* sf = a.S_final + bh * (int64_t)DK * DV + col0 + c32;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sf[(rt * 32 + acc_row(e, hh)) * DV] = M[rt][e];
  }
}

template <int DK, int DV>
static hipError_t launch_native_t(const UtArgs& a, hipStream_t s) {
  {
    TimedLaunch tl(HLA_KERNEL_CHUNK, s);
    hipLaunchKernelGGL((ut_kernel<DK, DV>), dim3((unsigned)(a.B * a.H * a.N)), dim3(512), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // state pass: the chains' 32-column slices spread over about one workgroup per CU (a
  // CU streams its piece records at its share of HBM bandwidth, so more CUs per chain
  // means less time per piece; the slices of a chain share the records through L2)
  constexpr int NCB = DV / 32;
  const int64_t chains = a.B * a.H;
  TimedLaunch tl(HLA_KERNEL_PREFILL, s);
  auto go = [&](auto nwb_c) {
    constexpr int NWB = decltype(nwb_c)::value;
    const unsigned nb = (unsigned)(chains * (NCB / NWB));
    if (a.o)
      hipLaunchKernelGGL((state_kernel<DK, DV, NWB, true>), dim3(nb), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((state_kernel<DK, DV, NWB, false>), dim3(nb), dim3(256), 0, s, a);
  };
  if (chains * NCB <= 256)
    go(std::integral_constant<int, 1>{});
  else if (chains * NCB <= 512)
    go(std::integral_constant<int, 2>{});
  else
    go(std::integral_constant<int, NCB>{});
  return hipGetLastError();
}

hipError_t launch_prefill_native(const UtArgs& a, int dk, int dv, hipStream_t s) {
  if (a.B * a.H == 0 || a.N == 0) return hipSuccess;
  if (dk == 64 && dv == 64) return launch_native_t<64, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_native_t<64, 128>(a, s);
  if (dk == 128 && dv == 64) return launch_native_t<128, 64>(a, s);
  return launch_native_t<128, 128>(a, s);
}

}  // namespace hla
