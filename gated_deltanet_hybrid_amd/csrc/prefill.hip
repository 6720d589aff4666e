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
// does not depend on the state -- g, the blocked inverse X, W and U -- into a per-piece
// record: -W row-major [t][dk] bf16, U^T in the accumulator lane order of the second pass's
// E^T tiles (bf16), g (float32) and, when outputs are wanted, P = (Q K^T) o Gamma (bf16).  The inverse is a chain of dependent LDS phases, so it
// runs here, many pieces per CU at once, instead of on the sequential path.
//
// Pass 2, state_kernel (one workgroup per (b, h, 32 state columns)): the state runs through
// the pieces in order.  Per piece, in the transposed forms whose operands sit in rows of
// contiguous k:
//   E^T = U^T - M^T W^T          (U^T seeds the accumulator, -W rows are the B operand)
//   O   = gamma (Q M) + P E      (P = (Q K^T) o Gamma from the record)
//   M^T <- gamma_63 M^T + (E^T D) K
// with the state kept in MFMA accumulators (one 32 x 32 tile of M^T per wave) and exchanged
// as a bf16 image MT [col][dk] in LDS.  Three barriers per piece; the next piece's operands
// are loaded into registers while the current one computes, and each output tile is stored
// at the start of the next piece.
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
  __shared__ __attribute__((aligned(16))) float Lb[C * PX];
  __shared__ __attribute__((aligned(16))) float Xb[C * PX];
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

  // ---- A. keys and values transposed into LDS; the K K^T operands of waves 0-2 into
  // registers; per-token decays (wave 0)
  {
    // every load first (rows past the end of a partial piece read its last row, in bounds),
    // then the zero padding where the values are used, so no load waits for another
    uint4 rk[KPT], rv[VPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + NT * j, t = i & (C - 1), u = i / C;
      rk[j] = *reinterpret_cast<const uint4*>(kg + (row0 + (t < n ? t : n - 1) * a.H) * DK + u * 8);
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = tid + NT * j, t = i & (C - 1), u = i / C;
      rv[j] = *reinterpret_cast<const uint4*>(vg + (row0 + (t < n ? t : n - 1) * a.H) * DV + u * 8);
    }
    float bt = 0.f, ra = 1.f;
    if (tid < C) {
      const int64_t r = row0 + (int64_t)(tid < n ? tid : n - 1) * a.H;
      bt = a.beta[r];
      ra = a.alpha[r];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + NT * j, t = i & (C - 1), u = i / C;
      const uint4 kv = t < n ? rk[j] : make_uint4(0u, 0u, 0u, 0u);
      const bf16* e8 = reinterpret_cast<const bf16*>(&kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) KT[(u * 8 + e) * PT + t] = e8[e];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = tid + NT * j, t = i & (C - 1), u = i / C;
      const uint4 vv = t < n ? rv[j] : make_uint4(0u, 0u, 0u, 0u);
      const bf16* e8 = reinterpret_cast<const bf16*>(&vv);
#pragma unroll
      for (int e = 0; e < 8; ++e) VT[(u * 8 + e) * PT + t] = e8[e];
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
      reinterpret_cast<float*>(rec + ut_off_g(DK, DV))[tid] = x;
    }
  }
  // K K^T lower tiles (0,0), (1,0), (1,1) on waves 0-2 and, when outputs are wanted, the
  // same tiles of Q K^T on waves 3-5: both operands are rows (8 consecutive dk per lane)
  // straight from global memory
  const bool want_p = a.q != nullptr;
  const int job = w < 3 ? w : w - 3;
  const int tm = job == 0 ? 0 : 1, tn = job == 2 ? 1 : 0;
  bf16x8 fa[DK / 16], fb[DK / 16];
  if (w < 3 || (want_p && w < 6)) {
    const int ta = tm * 32 + c32, tb = tn * 32 + c32;
    const bf16* ag = w < 3 ? kg : reinterpret_cast<const bf16*>(a.q);
    const bf16* pa = ag + (row0 + (ta < n ? ta : n - 1) * a.H) * DK + hh * 8;
    const bf16* pb = kg + (row0 + (tb < n ? tb : n - 1) * a.H) * DK + hh * 8;
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
      fa[ks] = *reinterpret_cast<const bf16x8*>(pa + ks * 16);
      fb[ks] = *reinterpret_cast<const bf16x8*>(pb + ks * 16);
    }
  }
  __syncthreads();

  // ---- B. L = strictly_lower(diag(beta) (K K^T) o Gamma); P = (Q K^T) o Gamma into the
  // record (wave 6 writes its zero upper tile); X = 0
  if (want_p && w >= 3 && w < 6) {
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) acc = Mma<bf16>::mma(fa[ks], fb[ks], acc);
    const int s = tn * 32 + c32;
    const float gs = s_g2[s];
    float gt[16];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<float4*>(gt + 4 * r) = *reinterpret_cast<const float4*>(s_g2 + tm * 32 + r * 8 + hh * 4);
    bf16* po = reinterpret_cast<bf16*>(rec + ut_off_p(DK, DV)) + (tm * 32 + hh * 4) * C + s;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      po[((e >> 2) * 8 + (e & 3)) * C] = (bf16)((s <= t) ? __builtin_amdgcn_exp2f(gt[e] - gs) * acc[e] : 0.f);
    }
  } else if (want_p && w == 6) {
    bf16* po = reinterpret_cast<bf16*>(rec + ut_off_p(DK, DV)) + (hh * 4) * C + 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) po[((e >> 2) * 8 + (e & 3)) * C] = (bf16)0.f;
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

  // ---- C. X = (I + L)^-1, blocked by 16: the diagonal blocks by substitution
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

  // ---- F. W tile (tt, db) on wave 2 db + tt -> -W [t][dk];  U^T tile (ct, tt) on wave
  // 2 ct + tt -> lane order.  X enters as hi + lo bf16 parts (about 16 mantissa bits).
  auto xfrag = [&](const float* xrow, const float* fac, int ks, bf16x8& hi, bf16x8& lo) {
    const int s0 = ks * 16 + hh * 8;
    float xv[8], fv[8];
    *reinterpret_cast<float4*>(xv) = *reinterpret_cast<const float4*>(xrow + s0);
    *reinterpret_cast<float4*>(xv + 4) = *reinterpret_cast<const float4*>(xrow + s0 + 4);
    *reinterpret_cast<float4*>(fv) = *reinterpret_cast<const float4*>(fac + s0);
    *reinterpret_cast<float4*>(fv + 4) = *reinterpret_cast<const float4*>(fac + s0 + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = xv[e] * fv[e];
      const bf16 hv = (bf16)x;
      hi[e] = hv;
      lo[e] = (bf16)(x - (float)hv);
    }
  };
  if (w < 2 * NDT) {
    const int tt = w & 1, db = w >> 1;
    const float* xrow = Xb + (tt * 32 + c32) * PX;
    const bf16* brow = KT + (db * 32 + c32) * PT;
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      bf16x8 hi, lo;
      xfrag(xrow, s_bg, ks, hi, lo);
      const bf16x8 bf = Mma<bf16>::load_plain(brow, ks, hh);
      acc = Mma<bf16>::mma(hi, bf, acc);
      acc = Mma<bf16>::mma(lo, bf, acc);
    }
    // element (token tt 32 + acc_row(e), key channel db 32 + c32)
    bf16* wo = reinterpret_cast<bf16*>(rec) + (tt * 32 + hh * 4) * DK + db * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) wo[((e >> 2) * 8 + (e & 3)) * DK] = (bf16)(-acc[e]);
  }
  if (w < 2 * NVT) {
    const int tt = w & 1, ct = w >> 1;
    const bf16* arow = VT + (ct * 32 + c32) * PT;
    const float* xrow = Xb + (tt * 32 + c32) * PX;
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      bf16x8 hi, lo;
      xfrag(xrow, s_beta, ks, hi, lo);
      const bf16x8 af = Mma<bf16>::load_plain(arow, ks, hh);
      acc = Mma<bf16>::mma(af, hi, acc);
      acc = Mma<bf16>::mma(af, lo, acc);
    }
    bf16x8 lo8, hi8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo8[e] = (bf16)acc[e];
      hi8[e] = (bf16)acc[e + 8];
    }
    bf16* uo = reinterpret_cast<bf16*>(rec + ut_off_u(DK)) + ((ct * 2 + tt) * 64 + lane) * 16;
    *reinterpret_cast<bf16x8*>(uo) = lo8;
    *reinterpret_cast<bf16x8*>(uo + 8) = hi8;
  }
}

template <int DK, int DV, bool WANT_O>
__global__ __launch_bounds__(512, WANT_O ? 2 : 4) void state_kernel(UtArgs a) {
  constexpr int C = kChunk;
  constexpr int NT = 512;
  constexpr int PK = DK + 8;   // bf16 pitch of [t][dk] and [col][dk] rows
  constexpr int PT = C + 8;    // bf16 pitch of [d][t] rows
  constexpr int NDT = DK / 32;
  constexpr int NCB = DV / 32;
  constexpr int KU = DK / 8;           // 16-byte units per key row
  constexpr int KPT = C * KU / NT;     // units of K, Q and -W each thread moves per piece
  constexpr int NKS = DK / 16;
  static_assert(KPT >= 1 && C * KU % NT == 0, "units per thread");

  __shared__ __attribute__((aligned(16))) bf16 KT[DK * PT];
  __shared__ __attribute__((aligned(16))) bf16 Wn[C * PK];
  __shared__ __attribute__((aligned(16))) bf16 Qp[WANT_O ? C * PK : 8];
  __shared__ __attribute__((aligned(16))) bf16 MT[2][32 * PK];
  __shared__ __attribute__((aligned(16))) bf16 ET[32 * PT];
  __shared__ __attribute__((aligned(16))) bf16 DET[32 * PT];
  __shared__ __attribute__((aligned(16))) float s_gam[C], s_d[C];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup -> (b, h, 32-column block); with B H a multiple of 8 the blocks of one (b, h)
  // share an XCD (workgroups go to the 8 XCDs round robin) and meet its inputs in its L2
  const int64_t id = blockIdx.x;
  int64_t bh;
  int cb;
  if ((a.B * a.H) % 8 == 0) {
    const int64_t j = id >> 3;
    cb = (int)(j % NCB);
    bh = (j / NCB) * 8 + (id & 7);
  } else {
    cb = (int)(id % NCB);
    bh = id / NCB;
  }
  const int64_t h = bh % a.H, b = bh / a.H;
  const int col0 = cb * 32;
  const int N = a.N;
  const bf16* kg = reinterpret_cast<const bf16*>(a.k);
  const bf16* qg = reinterpret_cast<const bf16*>(a.q);
  const int64_t RB = ut_record_bytes(DK, DV);
  const char* recs = static_cast<const char*>(a.rec) + bh * (int64_t)N * RB;

  // ---- roles: E^T tile tt on waves 0, 1; output tile tt on waves 2, 3; M^T tile db (the
  // block's 32 columns x dk 32 db ..) on wave 4 + db
  const bool has_e = w < 2;
  const bool has_o = WANT_O && (w == 2 || w == 3);
  const bool has_m = w >= 4 && w < 4 + NDT;
  const int e_tt = w & 1, o_tt = w & 1;
  const int m_db = w - 4;

  // ---- the start state (S0 or zero) and its bf16 image; P's upper tile is zero
  f32x16 Macc = zero16();
  if (has_m) {
    if (a.S0) {
      const float* s0 = a.S0 + bh * (int64_t)DK * DV;
      const int dk = m_db * 32 + c32;
#pragma unroll
      for (int e = 0; e < 16; ++e) Macc[e] = s0[dk * DV + col0 + acc_row(e, hh)];
    }
    bf16* img = MT[0] + m_db * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) img[acc_row(e, hh) * PK] = (bf16)Macc[e];
  }

  // ---- the next piece's operands, in registers: K units (lane = token, so the transposed
  // copy is written without bank conflicts), Q and -W units (consecutive threads along a
  // row), g (threads < 64), the U^T tile in lane order (E waves) and the output tile's rows
  // of P (output waves, A operand)
  uint4 rk[KPT], rq[WANT_O ? KPT : 1], rw[KPT], ru[2], rp[WANT_O ? 4 : 1];
  float rg = 0.f;
  auto load_piece = [&](int c) {
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
    const int64_t row0 = (b * a.ld_T + t0) * a.H + h;
    const char* rec = recs + (int64_t)c * RB;
    // rows past the end of a partial piece load its last row (in bounds, never waited for
    // here) and are replaced by zeros where they are staged
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + NT * j;
      const int t = i & (C - 1), u = i / C;
      rk[j] = *reinterpret_cast<const uint4*>(kg + (row0 + (t < n ? t : n - 1) * a.H) * DK + u * 8);
      const int tr = i / KU, ur = i % KU;
      rw[j] = reinterpret_cast<const uint4*>(rec)[i];
      if constexpr (WANT_O)
        rq[j] = *reinterpret_cast<const uint4*>(qg + (row0 + (tr < n ? tr : n - 1) * a.H) * DK + ur * 8);
    }
    if (tid < C) rg = reinterpret_cast<const float*>(rec + ut_off_g(DK, DV))[tid];
    if (has_e) {
      const uint4* ur = reinterpret_cast<const uint4*>(rec + ut_off_u(DK)) + ((cb * 2 + e_tt) * 64 + lane) * 2;
      ru[0] = ur[0];
      ru[1] = ur[1];
    }
    if constexpr (WANT_O) {
      if (has_o) {
        const bf16* pr = reinterpret_cast<const bf16*>(rec + ut_off_p(DK, DV)) + (o_tt * 32 + c32) * C + hh * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) rp[ks] = *reinterpret_cast<const uint4*>(pr + ks * 16);
      }
    }
  };

  f32x16 Oacc = zero16();
  auto store_o = [&](int c) {
    // output tile of piece c: token t = 32 o_tt + acc_row(e), column col0 + c32
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
    float* ob = a.o + ((b * a.T + t0 + o_tt * 32 + hh * 4) * a.H + h) * DV + col0 + c32;
    const int64_t ostride = a.H * DV;
    if (n == C) {
#pragma unroll
      for (int e = 0; e < 16; ++e) __builtin_nontemporal_store(Oacc[e], &ob[((e >> 2) * 8 + (e & 3)) * ostride]);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (o_tt * 32 + acc_row(e, hh) < n) __builtin_nontemporal_store(Oacc[e], &ob[((e >> 2) * 8 + (e & 3)) * ostride]);
    }
  };

  if (N > 0) load_piece(0);
  for (int c = 0; c < N; ++c) {
    const int cur = c & 1;
    const int64_t tc0 = (int64_t)c * C;
    const int n = (int)((a.T - tc0) < C ? (a.T - tc0) : C);
    // ---- A. piece c's operands into LDS (K^T, K, Q, -W, decays) and U^T into the E
    // accumulators; the previous piece's outputs; then piece c + 1's loads
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + NT * j;
      const int t = i & (C - 1), u = i / C;
      const uint4 kv = t < n ? rk[j] : make_uint4(0u, 0u, 0u, 0u);
      const bf16* e8 = reinterpret_cast<const bf16*>(&kv);
#pragma unroll
      for (int e = 0; e < 8; ++e) KT[(u * 8 + e) * PT + t] = e8[e];
      const int tr = i / KU, ur = i % KU;
      *reinterpret_cast<uint4*>(Wn + tr * PK + ur * 8) = rw[j];
      if constexpr (WANT_O) *reinterpret_cast<uint4*>(Qp + tr * PK + ur * 8) = tr < n ? rq[j] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid < C) {
      const float g_end = __shfl(rg, 63, 64);
      s_gam[tid] = expf(rg);
      s_d[tid] = expf(g_end - rg);
    }
    uint4 cp[WANT_O ? 4 : 1];
    if constexpr (WANT_O) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) cp[ks] = rp[ks];
    }
    f32x16 Eacc;
    if (has_e) {
      const bf16* u16 = reinterpret_cast<const bf16*>(ru);
#pragma unroll
      for (int e = 0; e < 16; ++e) Eacc[e] = (float)u16[e];
    }
    if constexpr (WANT_O) {
      if (has_o && c > 0) store_o(c - 1);
    }
    if (c + 1 < N) load_piece(c + 1);
    __syncthreads();

    // ---- G. E^T = U^T - M^T W^T -> ET, DET;  outputs: gamma (Q M);  P = (Q K^T) o Gamma
    const bf16* Mimg = MT[cur];
    if (has_e) {
      const bf16* arow = Mimg + c32 * PK;
      const bf16* brow = Wn + (e_tt * 32 + c32) * PK;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        Eacc = Mma<bf16>::mma(Mma<bf16>::load_plain(arow, ks, hh), Mma<bf16>::load_plain(brow, ks, hh), Eacc);
      // element (column acc_row(e), token t = 32 e_tt + c32)
      const int t = e_tt * 32 + c32;
      const float dt = s_d[t];
      bf16* eo = ET + t;
      bf16* deo = DET + t;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        eo[acc_row(e, hh) * PT] = (bf16)Eacc[e];
        deo[acc_row(e, hh) * PT] = (bf16)(Eacc[e] * dt);
      }
    }
    if constexpr (WANT_O) {
      if (has_o) {
        const bf16* arow = Qp + (o_tt * 32 + c32) * PK;
        const bf16* brow = Mimg + c32 * PK;
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          acc = Mma<bf16>::mma(Mma<bf16>::load_plain(arow, ks, hh), Mma<bf16>::load_plain(brow, ks, hh), acc);
        float gm[16];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float4*>(gm + 4 * r) = *reinterpret_cast<const float4*>(s_gam + o_tt * 32 + r * 8 + hh * 4);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] *= gm[e];
        Oacc = acc;
      }
    }
    __syncthreads();

    // ---- H. outputs: + P E;  state: M^T <- gamma_63 M^T + (E^T D) K
    if constexpr (WANT_O) {
      if (has_o) {
        const bf16* brow = ET + c32 * PT;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks)
          Oacc = Mma<bf16>::mma(__builtin_bit_cast(bf16x8, cp[ks]), Mma<bf16>::load_plain(brow, ks, hh), Oacc);
      }
    }
    if (has_m) {
      const float g_end = s_gam[C - 1];
#pragma unroll
      for (int e = 0; e < 16; ++e) Macc[e] *= g_end;
      const bf16* arow = DET + c32 * PT;
      const bf16* brow = KT + (m_db * 32 + c32) * PT;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks)
        Macc = Mma<bf16>::mma(Mma<bf16>::load_plain(arow, ks, hh), Mma<bf16>::load_plain(brow, ks, hh), Macc);
      bf16* img = MT[cur ^ 1] + m_db * 32 + c32;
#pragma unroll
      for (int e = 0; e < 16; ++e) img[acc_row(e, hh) * PK] = (bf16)Macc[e];
    }
    __syncthreads();
  }
  if constexpr (WANT_O) {
    if (has_o && N > 0) store_o(N - 1);
  }
  if (has_m && a.S_final) {
    float* sf = a.S_final + bh * (int64_t)DK * DV;
    const int dk = m_db * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) sf[dk * DV + col0 + acc_row(e, hh)] = Macc[e];
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
  const unsigned nb = (unsigned)(a.B * a.H * (DV / 32));
  TimedLaunch tl(HLA_KERNEL_PREFILL, s);
  if (a.o)
    hipLaunchKernelGGL((state_kernel<DK, DV, true>), dim3(nb), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((state_kernel<DK, DV, false>), dim3(nb), dim3(512), 0, s, a);
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
