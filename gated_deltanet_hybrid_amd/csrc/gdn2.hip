// Gated DeltaNet-2 chunk pass: exact chunk maps, and chunk outputs from given start
// states, by running the chunk's tokens in float32.
//
// [GDN2] the Gated DeltaNet-2 abstract: channel-wise decay alpha_t in (0,1)^dk, a
// channel-wise erase gate b_t on the key side and a channel-wise write gate w_t on the
// value side.  In the stored orientation M = S^T [dk, dv] one token is
//     M <- (I - e_t k_t^T) D_t M + k_t u_t^T,    D_t = diag(alpha_t), e_t = b_t o k_t,
//                                                u_t = w_t o v_t,
// and o_t = M^T q_t.  Every column x of M evolves on its own:
//     x <- D_t x - e_t (k_t . D_t x) + k_t u_t[col],
// and so does every column of a chunk map [P | Q] (M_end = P M_start + Q): P starts at I
// and takes no write, Q starts at 0.  [HLA] Methodology paragraph 1: the chunk is one
// exact affine map, which the HLA router and composition consume unchanged.
//
// Layout: one workgroup per (b, h, 64-token piece).  A thread holds 2 columns over a
// quarter of the rows (2 x dk/4 floats); the 4 threads of a column group are adjacent
// lanes, so the read k . D x is a sum over the thread's rows plus two DPP quad moves.
// Token vectors (k o alpha, alpha, e, k, u, and q for outputs) are staged 8 tokens at a
// time in LDS and read as broadcasts.  The work is float32 VALU: per token and column
// about 4 dk fused multiply-adds (5 dk with the output read).  The layout was chosen by
// timing: 2 columns x 4 row groups x 8 staged tokens ran the routed step's two passes at
// 3.6 ms against 5.3 ms for 4 x 4 x 16 (more waves in flight, smaller LDS).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {
template <int CPT_, int RQ_, int TB_>
struct G2Shape {
  static constexpr int CPT = CPT_, RQ = RQ_, TB = TB_;
};
using G2 = G2Shape<2, 4, 8>;  // columns per thread, row groups, tokens per staged block
constexpr int kTB = G2::TB;
}

// threads of one workgroup: one per (group of CPT columns, row group)
template <int DK, int DV, bool OUT>
constexpr int gdn2_threads() {
  return (OUT ? DV : DK + DV) / G2::CPT * G2::RQ;
}

template <class T, int DK, int DV, bool OUT>
__global__ __launch_bounds__((gdn2_threads<DK, DV, OUT>())) void gdn2_chunk_kernel(ChunkArgs a) {
  constexpr int C = kChunk;
  constexpr int NCOL = OUT ? DV : DK + DV;
  constexpr int CPT = G2::CPT, RQ = G2::RQ, RPT = DK / RQ;
  constexpr int NT = NCOL / CPT * RQ;
  constexpr int PR = DK + 4;  // LDS row pitch
  static_assert(NT <= 1024 && RPT % 4 == 0 && (RQ & (RQ - 1)) == 0, "thread layout");
  __shared__ __attribute__((aligned(16))) float s_ka[kTB][PR];
  __shared__ __attribute__((aligned(16))) float s_al[kTB][PR];
  __shared__ __attribute__((aligned(16))) float s_e[kTB][PR];
  __shared__ __attribute__((aligned(16))) float s_k[kTB][PR];
  __shared__ __attribute__((aligned(16))) float s_q[OUT ? kTB : 1][PR];
  __shared__ __attribute__((aligned(16))) float s_u[kTB][DV];

  const int tid = threadIdx.x;
  const int rq = tid % RQ, grp = tid / RQ;  // row group, column group
  const int64_t id = blockIdx.x;
  const int c = (int)(id % a.N);
  const int64_t bh = id / a.N;
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)c * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
  const int r0 = rq * RPT;
  const bool active = tid < NT;

  float x[CPT][RPT];
  if (active) {
    if constexpr (OUT) {
      const float* M0 = a.chunk_init + ((b * a.H + h) * a.N + c) * (int64_t)DK * DV;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int j = 0; j < CPT; ++j) x[j][i] = M0[(int64_t)(r0 + i) * DV + grp * CPT + j];
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int i = 0; i < RPT; ++i) x[j][i] = (grp * CPT + j == r0 + i) ? 1.f : 0.f;
    }
  }
  // column j's write input: u[col] for state / Q columns, none for P columns
  const bool writes = OUT || grp * CPT >= DK;
  const int ucol0 = OUT ? grp * CPT : (writes ? grp * CPT - DK : 0);

  for (int tb = 0; tb < n; tb += kTB) {
    const int nb = n - tb < kTB ? n - tb : kTB;
    __syncthreads();  // the previous block's reads are done
    for (int i = tid; i < nb * DK; i += blockDim.x) {
      const int t = i / DK, r = i % DK;
      const int64_t row = row0 + (int64_t)(tb + t) * a.H;
      const float kv = to_f<T>(reinterpret_cast<const T*>(a.k)[row * DK + r]);
      const float al = a.ga[row * DK + r];
      s_k[t][r] = kv;
      s_al[t][r] = al;
      s_ka[t][r] = kv * al;
      s_e[t][r] = a.gb[row * DK + r] * kv;
      if constexpr (OUT) s_q[t][r] = to_f<T>(reinterpret_cast<const T*>(a.q)[row * DK + r]);
    }
    for (int i = tid; i < nb * DV; i += blockDim.x) {
      const int t = i / DV, r = i % DV;
      const int64_t row = row0 + (int64_t)(tb + t) * a.H;
      s_u[t][r] = a.gw[row * DV + r] * to_f<T>(reinterpret_cast<const T*>(a.v)[row * DV + r]);
    }
    __syncthreads();
    if (!active) continue;
    for (int t = 0; t < nb; ++t) {
      // read of every column: k . D x over this thread's rows, then over the row quarters
      float s[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) s[j] = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; i += 4) {
        const float4 ka = *reinterpret_cast<const float4*>(&s_ka[t][r0 + i]);
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          s[j] = fmaf(ka.x, x[j][i], s[j]);
          s[j] = fmaf(ka.y, x[j][i + 1], s[j]);
          s[j] = fmaf(ka.z, x[j][i + 2], s[j]);
          s[j] = fmaf(ka.w, x[j][i + 3], s[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) s[j] = group_sum<RQ>(s[j]);  // the RQ row groups are adjacent lanes
      float u[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) u[j] = writes ? s_u[t][ucol0 + j] : 0.f;
#pragma unroll
      for (int i = 0; i < RPT; i += 4) {
        const float4 al = *reinterpret_cast<const float4*>(&s_al[t][r0 + i]);
        const float4 e = *reinterpret_cast<const float4*>(&s_e[t][r0 + i]);
        const float4 kv = *reinterpret_cast<const float4*>(&s_k[t][r0 + i]);
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          x[j][i] = fmaf(kv.x, u[j], fmaf(-e.x, s[j], al.x * x[j][i]));
          x[j][i + 1] = fmaf(kv.y, u[j], fmaf(-e.y, s[j], al.y * x[j][i + 1]));
          x[j][i + 2] = fmaf(kv.z, u[j], fmaf(-e.z, s[j], al.z * x[j][i + 2]));
          x[j][i + 3] = fmaf(kv.w, u[j], fmaf(-e.w, s[j], al.w * x[j][i + 3]));
        }
      }
      if constexpr (OUT) {
        float o[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) o[j] = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; i += 4) {
          const float4 qv = *reinterpret_cast<const float4*>(&s_q[t][r0 + i]);
#pragma unroll
          for (int j = 0; j < CPT; ++j) {
            o[j] = fmaf(qv.x, x[j][i], o[j]);
            o[j] = fmaf(qv.y, x[j][i + 1], o[j]);
            o[j] = fmaf(qv.z, x[j][i + 2], o[j]);
            o[j] = fmaf(qv.w, x[j][i + 3], o[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) o[j] = group_sum<RQ>(o[j]);
        if (rq == 0) {
          float* orow = a.o + ((b * a.T + t0 + tb + t) * a.H + h) * DV + grp * CPT;
#pragma unroll
          for (int j = 0; j < CPT; ++j) orow[j] = o[j];
        }
      }
    }
  }
  if constexpr (!OUT) {
    if (active) {
      // column grp*CPT + j of [P | Q]: P is At [dk, dk], Q is Bc [dk, dv]
      const bool isq = grp * CPT >= DK;
      T* out = isq ? reinterpret_cast<T*>(a.Bc) + ((b * a.H + h) * a.N + c) * (int64_t)DK * DV
                   : reinterpret_cast<T*>(a.At) + ((b * a.H + h) * a.N + c) * (int64_t)DK * DK;
      const int ld = isq ? DV : DK, col = isq ? grp * CPT - DK : grp * CPT;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int j = 0; j < CPT; ++j) out[(int64_t)(r0 + i) * ld + col + j] = from_f<T>(x[j][i]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// The chunk maps in the WY (UT) form on the matrix cores, bf16 inputs.
//
// [GDN2] abstract: the chunkwise algorithm absorbs the channel-wise decay into asymmetric
// erase factors.  With G_t = sum_{s<=t} log alpha_s per key channel, Gamma_t = diag(exp G_t)
// and M~_t = Gamma_t^-1 M_t, one token is
//     M~ <- M~ - e^_t (k^_t . M~) + k-_t u_t^T,   e^_t = e_t / Gamma_t, k^_t = Gamma_t k_t,
//                                                  k-_t = k_t / Gamma_t,
// a delta step whose erase and read vectors differ.  Over a piece of 64 tokens (rows t):
//     R   = X (K^ M_0 + B U),  X = (I + A)^-1,  with, for s < t,
//     A_ts = sum_c k_tc e_sc exp(G_tc - G_sc),   B_ts = sum_c k_tc k_sc exp(G_tc - G_sc);
//     M_63 = Gamma_63 M_0 - E~^T R + K~^T U,  E~_t = e_t exp(G_63 - G_t), K~_t = k_t exp(G_63 - G_t),
// so At = Gamma_63 - E~^T X K^ and Bc = K~^T U - E~^T X (B U).  Every factor above is the
// exp of a difference of log-decays that is at most zero, except in A and B, whose 16 x 16
// blocks take a reference token: below the diagonal blocks the last token of the s block
// (both factors at most one), on them the block's eighth token (factors at most the decay
// over eight tokens, which the per-token floor log alpha >= -11 keeps below 2^127).
//
// The outputs of a piece that starts from M_0: o_t = M_t^T q_t with M_t = Gamma_t M~_t, so
//     O = (Q^ - Pe W) M_0 + (Pk U - Pe Z),  W = X K^, Z = X (B U),  Q^_t = Gamma_t q_t,
//     Pe_ts = sum_c q_tc e_sc exp(G_tc - G_sc),  Pk_ts = sum_c q_tc k_sc exp(G_tc - G_sc)  (s <= t).
//
// One workgroup of 8 waves per (b, h, piece).  A, B (and Pe, Pk) come from 16 x 16 x 32
// MFMAs, ten blocks each; the inverse is the blocked one of the Gated DeltaNet pass.  For
// the maps, wave ct then owns column tile ct of [At | Bc]: W = X K^ or B U and Z = X (B U)
// stay in its accumulators and feed the last products as B operands in place.  For the
// outputs, the waves of the key columns form Q^ - Pe W (staged in LDS), those of the value
// columns B U, Z and then their columns of O.  X and B enter as hi + lo bf16 parts.
namespace {
constexpr float kG2Floor = -11.f * 1.4426950408889634f;  // log2 of the per-token decay floor
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
}  // namespace

// A workgroup barrier that orders LDS only: __syncthreads' release fence would also wait for
// the next piece's loads in flight and for the output stores.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int DK, int DV, bool OUT>
__global__ __launch_bounds__(512, 1) void gdn2_wy_kernel(ChunkArgs a, int64_t npieces) {
  constexpr int C = kChunk, NT = 512;
  constexpr int PG = DK + 4;   // fp32 pitch of log2-decay rows [t][c]
  constexpr int PX = C + 4;    // fp32 pitch of A, B, X rows
  constexpr int PT = C + 8;    // bf16 pitch of [c][t] rows
  constexpr int NRT = DK / 32, NKQ = DK / 32;
  constexpr int PK = DK + 8;   // bf16 pitch of [t][c] rows
  static_assert((DK + DV) / 32 <= 8, "one column tile of [At | Bc] per wave");
  // LDS.  Region R0 first holds G2 (fp32 [t][c]) and the raw rows of k, b (and q) (bf16
  // [t][c]); from step 4 on, K^ T and E~ T, K~ T, U T (maps) or K^ T, U T and Q^ (outputs).
  constexpr int RA = C * PG * 4 + (OUT ? 3 : 2) * C * PK * 2;
  constexpr int RB = OUT ? 2 * DK * PT * 2 + DV * PT * 2 : 0;  // (K^ T, U T, Q^ rows)
  constexpr int RB2 = OUT ? DK * PT * 2 + DV * PT * 2 + C * PK * 2 : (3 * DK + DV) * PT * 2;
  constexpr int R0 = RA > RB2 ? RA : RB2;
  (void)RB;
  __shared__ __attribute__((aligned(16))) char r0[R0];
  __shared__ __attribute__((aligned(16))) float Lb[C * PX];
  __shared__ __attribute__((aligned(16))) float Xb[C * PX];
  __shared__ __attribute__((aligned(16))) float Bb[C * PX];
  __shared__ __attribute__((aligned(16))) float s_gend[DK];
  // outputs: Pe, Pk (bf16 [t][s])
  __shared__ __attribute__((aligned(16))) bf16 PeB[OUT ? C * PT : 8];
  __shared__ __attribute__((aligned(16))) bf16 PkB[OUT ? C * PT : 8];
  float* sG2 = reinterpret_cast<float*>(r0);
  bf16* rK = reinterpret_cast<bf16*>(r0 + C * PG * 4);
  bf16* rB = rK + C * PK;
  bf16* rQ = rB + C * PK;
  bf16* KhT = reinterpret_cast<bf16*>(r0);
  bf16* UT = KhT + DK * PT;
  bf16* EtT = UT + DV * PT;   // (maps)
  bf16* KtT = EtT + DK * PT;  // (maps)
  bf16* QpB = UT + DV * PT;   // (outputs: Q^, then Q^ - Pe W)

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bf16* kg = reinterpret_cast<const bf16*>(a.k);
  const bf16* vg = reinterpret_cast<const bf16*>(a.v);
  const bf16* qg = reinterpret_cast<const bf16*>(a.q);

  // The global reads of one piece, all unconditional (rows past the end read the last row):
  // alpha and b in float4 units, k (and q) in 16-byte units, v and w per step-4 value task
  // (token fastest).  They are issued for the next piece while this one computes.
  constexpr int A4 = C * DK / 4 / NT;  // float4 units of alpha and b per thread
  constexpr int K8 = C * DK / 8 / NT;  // 16-byte units of k (and q) per thread
  constexpr int NVB = DV / 8, NVTASK = C * NVB / NT;
  static_assert(A4 * NT * 4 == C * DK && K8 * NT * 8 == C * DK, "units per thread");
  static_assert(NVTASK * NT == C * NVB, "value tasks per thread");
  float4 al[A4], bv[A4];
  bf16x8 kv[K8], qv[K8], vreg[NVTASK];
  float wreg[NVTASK][8];
  // where a piece's token rows start, and how many of its tokens exist
  struct Piece {
    int64_t row0;  // token-row of (b, t0, h)
    int n;
  };
  auto piece_of = [&](int64_t id) -> Piece {
    const int c = (int)(id % a.N);
    const int64_t bh = id / a.N, h = bh % a.H, b = bh / a.H, t0 = (int64_t)c * C;
    return Piece{(b * a.ld_T + t0) * a.H + h, (int)((a.T - t0) < C ? (a.T - t0) : C)};
  };
  // Load li of the thread's list (alpha, b, k, q, v, w lo / hi) is issued in part
  // li * NPART / NLOAD: the parts go out between the steps of the current piece, so that
  // the CU's memory pipeline is never handed the whole piece at once.
  constexpr int NLOAD = 2 * A4 + (OUT ? 2 : 1) * K8 + 3 * NVTASK, NPART = 6;
  auto fetch = [&](const Piece& pc, int tid, int part) {
    auto row = [&](int t) -> int64_t { return pc.row0 + (int64_t)(t < pc.n ? t : pc.n - 1) * a.H; };
    auto mine = [&](int li) { return li * NPART / NLOAD == part; };
#pragma unroll
    for (int jj = 0; jj < A4; ++jj) {
      const int u = tid + NT * jj, t = u / (DK / 4), c4 = (u % (DK / 4)) * 4;
      if (mine(jj)) al[jj] = *reinterpret_cast<const float4*>(a.ga + row(t) * DK + c4);
      if (mine(A4 + jj)) bv[jj] = *reinterpret_cast<const float4*>(a.gb + row(t) * DK + c4);
    }
#pragma unroll
    for (int jj = 0; jj < K8; ++jj) {
      const int u = tid + NT * jj, t = u / (DK / 8), c8 = (u % (DK / 8)) * 8;
      if (mine(2 * A4 + jj)) kv[jj] = *reinterpret_cast<const bf16x8*>(kg + row(t) * DK + c8);
      if constexpr (OUT)
        if (mine(2 * A4 + K8 + jj)) qv[jj] = *reinterpret_cast<const bf16x8*>(qg + row(t) * DK + c8);
    }
    constexpr int LV = 2 * A4 + (OUT ? 2 : 1) * K8;
#pragma unroll
    for (int jj = 0; jj < NVTASK; ++jj) {
      const int task = tid + NT * jj, t = task & (C - 1), c0 = (task / C) * 8;
      const float* wr = a.gw + row(t) * DV + c0;
      if (mine(LV + 3 * jj)) vreg[jj] = *reinterpret_cast<const bf16x8*>(vg + row(t) * DV + c0);
      if (mine(LV + 3 * jj + 1)) *reinterpret_cast<float4*>(wreg[jj]) = *reinterpret_cast<const float4*>(wr);
      if (mine(LV + 3 * jj + 2)) *reinterpret_cast<float4*>(wreg[jj] + 4) = *reinterpret_cast<const float4*>(wr + 4);
    }
  };

  // Blocks that stay zero for every piece, written once: B's, Pe's and Pk's blocks above
  // the diagonal (B is a full A operand later) and X above its diagonal blocks.
  for (int i = threadIdx.x; i < 6 * 256; i += NT) {
    const int bz = i >> 8, r = (i >> 4) & 15, cc = i & 15;
    const int bt = bz < 3 ? 0 : (bz < 5 ? 1 : 2), bs = bz < 3 ? bz + 1 : (bz < 5 ? bz - 1 : 3);  // bs > bt
    Bb[(bt * 16 + r) * PX + bs * 16 + cc] = 0.f;
    Xb[(bt * 16 + r) * PX + bs * 16 + cc] = 0.f;
    if constexpr (OUT) {
      PeB[(bt * 16 + r) * PT + bs * 16 + cc] = (bf16)0.f;
      PkB[(bt * 16 + r) * PT + bs * 16 + cc] = (bf16)0.f;
    }
  }
  {
    const Piece p0 = piece_of(blockIdx.x);
#pragma unroll
    for (int part = 0; part < NPART; ++part) fetch(p0, threadIdx.x, part);
  }

  // pieces blockIdx.x, + gridDim.x, ... (one workgroup per CU)
  for (int64_t id = blockIdx.x; id < npieces; id += gridDim.x) {
    // the thread index, opaque to the compiler, so that the LDS addresses derived from it are
    // formed in each piece rather than held in registers across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
    const int c = (int)(id % a.N);
    const int64_t bh = id / a.N;
    const int64_t h = bh % a.H, b = bh / a.H;
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
    const int64_t cidx = (b * a.H + h) * a.N + c;

    // ---- 0. the fetched piece into LDS: per-token log2 decays (floored; 0 past the end), b,
    // k and q (0 past the end); u = w o v (0 past the end) stays in registers
    lds_barrier();  // the previous piece is done with LDS
    bf16x8 uu[NVTASK];
    {
#pragma unroll
      for (int jj = 0; jj < A4; ++jj) {
        const int u = tid + NT * jj, t = u / (DK / 4), c4 = (u % (DK / 4)) * 4;
        float4 l;
        l.x = t < n ? fmaxf(log2f(al[jj].x), kG2Floor) : 0.f;
        l.y = t < n ? fmaxf(log2f(al[jj].y), kG2Floor) : 0.f;
        l.z = t < n ? fmaxf(log2f(al[jj].z), kG2Floor) : 0.f;
        l.w = t < n ? fmaxf(log2f(al[jj].w), kG2Floor) : 0.f;
        *reinterpret_cast<float4*>(sG2 + t * PG + c4) = l;
        bf16 b4[4] = {(bf16)bv[jj].x, (bf16)bv[jj].y, (bf16)bv[jj].z, (bf16)bv[jj].w};
        *reinterpret_cast<uint2*>(rB + t * PK + c4) = *reinterpret_cast<const uint2*>(b4);
      }
#pragma unroll
      for (int jj = 0; jj < K8; ++jj) {
        const int u = tid + NT * jj, t = u / (DK / 8), c8 = (u % (DK / 8)) * 8;
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
        *reinterpret_cast<bf16x8*>(rK + t * PK + c8) = t < n ? kv[jj] : z;
        if constexpr (OUT) *reinterpret_cast<bf16x8*>(rQ + t * PK + c8) = t < n ? qv[jj] : z;
      }
#pragma unroll
      for (int jj = 0; jj < NVTASK; ++jj) {
        const int task = tid + NT * jj, t = task & (C - 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) uu[jj][e] = (bf16)(t < n ? (float)vreg[jj][e] * wreg[jj][e] : 0.f);
      }
    }
    lds_barrier();
    const Piece nx = piece_of(id + gridDim.x < npieces ? id + gridDim.x : id);
    fetch(nx, tid, 0);

    // ---- 1. G2 = running sum over tokens, in place: NQ adjacent lanes per channel, C / NQ
    // tokens each, joined through the lane totals
    {
      constexpr int NQ = NT / DK;  // lanes per channel
      constexpr int TQ = C / NQ;   // tokens per lane
      static_assert(NQ * DK == NT && (NQ & (NQ - 1)) == 0 && NQ <= 64, "cumsum layout");
      const int ch = tid / NQ, q = tid % NQ;
      float l[TQ];
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < TQ; ++jj) {
        acc += sG2[(q * TQ + jj) * PG + ch];
        l[jj] = acc;
      }
      float pre = 0.f;
      {
        float tot[NQ];
#pragma unroll
        for (int r = 0; r < NQ; ++r) tot[r] = __shfl(acc, (lane & ~(NQ - 1)) + r, 64);
#pragma unroll
        for (int r = 0; r < NQ; ++r) pre += r < q ? tot[r] : 0.f;
        if (q == NQ - 1) s_gend[ch] = pre + acc;
      }
#pragma unroll
      for (int jj = 0; jj < TQ; ++jj) sG2[(q * TQ + jj) * PG + ch] = pre + l[jj];
    }
    lds_barrier();
    fetch(nx, tid, 1);

    // ---- 2. A and B (and Pe, Pk) by 16 x 16 blocks (s block bs <= t block bt), 16 x 16 x 32
    // MFMAs: lane (m = lane % 16, g = lane / 16) holds row m and channels 32 kq + 8 g .. 8 g + 7
    // of k-step kq for both operands; the result holds rows 4 g + i, column m.
    {
      const int m = lane & 15, g = lane >> 4;
      for (int bi = w; bi < 10; bi += 8) {
        // blocks: the four diagonal ones, then (1,0) (2,0) (3,0) (2,1) (3,1) (3,2)
        const int bt = bi < 4 ? bi : (bi < 7 ? bi - 3 : (bi < 9 ? bi - 5 : 3));
        const int bs = bi < 4 ? bi : (bi < 7 ? 0 : (bi < 9 ? 1 : 2));
        const bool diag = bt == bs;
        const int rt = diag ? 16 * bt + 7 : 16 * bs + 15;  // reference token
        const int t = 16 * bt + m, sx = 16 * bs + m;       // this lane's x row and y row
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
        f32x4 accPe = {0.f, 0.f, 0.f, 0.f}, accPk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < NKQ; ++kq) {
          const int c0 = 32 * kq + 8 * g;
          const bf16x8 kt8 = *reinterpret_cast<const bf16x8*>(rK + t * PK + c0);
          const bf16x8 ks8 = *reinterpret_cast<const bf16x8*>(rK + sx * PK + c0);
          const bf16x8 b8 = *reinterpret_cast<const bf16x8*>(rB + sx * PK + c0);
          bf16x8 q8;
          if constexpr (OUT) q8 = *reinterpret_cast<const bf16x8*>(rQ + t * PK + c0);
          float gt[8], gs[8], gr[8];
          *reinterpret_cast<float4*>(gt) = *reinterpret_cast<const float4*>(sG2 + t * PG + c0);
          *reinterpret_cast<float4*>(gt + 4) = *reinterpret_cast<const float4*>(sG2 + t * PG + c0 + 4);
          *reinterpret_cast<float4*>(gs) = *reinterpret_cast<const float4*>(sG2 + sx * PG + c0);
          *reinterpret_cast<float4*>(gs + 4) = *reinterpret_cast<const float4*>(sG2 + sx * PG + c0 + 4);
          *reinterpret_cast<float4*>(gr) = *reinterpret_cast<const float4*>(sG2 + rt * PG + c0);
          *reinterpret_cast<float4*>(gr + 4) = *reinterpret_cast<const float4*>(sG2 + rt * PG + c0 + 4);
          bf16x8 xa, xq, ye, yk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float fy = __builtin_amdgcn_exp2f(gr[e] - gs[e]);
            const float fx = __builtin_amdgcn_exp2f(gt[e] - gr[e]);
            const float ky = (float)ks8[e];
            xa[e] = (bf16)((float)kt8[e] * fx);
            if constexpr (OUT) xq[e] = (bf16)((float)q8[e] * fx);
            yk[e] = (bf16)(ky * fy);
            ye[e] = (bf16)(ky * (float)b8[e] * fy);
          }
          accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ye, accA, 0, 0, 0);
          accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, yk, accB, 0, 0, 0);
          if constexpr (OUT) {
            accPe = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xq, ye, accPe, 0, 0, 0);
            accPk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xq, yk, accPk, 0, 0, 0);
          }
        }
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int tr = 16 * bt + 4 * g + i2, sc = 16 * bs + m;
          const bool keep = !diag || sc < tr;  // (entries on and above the diagonal may be inf: selected away)
          Lb[tr * PX + sc] = keep ? accA[i2] : 0.f;
          Bb[tr * PX + sc] = keep ? accB[i2] : 0.f;
          if constexpr (OUT) {
            const bool keepd = !diag || sc <= tr;  // (with the diagonal)
            PeB[tr * PT + sc] = (bf16)(keepd ? accPe[i2] : 0.f);
            PkB[tr * PT + sc] = (bf16)(keepd ? accPk[i2] : 0.f);
          }
        }
      }
    }
    lds_barrier();
    // outputs: this piece's start state M_0, column c32 of the wave's value tile, 8 rows per
    // lane (coalesced over lanes), loaded here and turned into B operand fragments two steps
    // later
    float mv[DK / 16][8];
    bf16x8 bm[DK / 16];
    if constexpr (OUT) {
      if (w >= DK / 32 && w < (DK + DV) / 32) {
        const float* m0 = a.chunk_init + cidx * (int64_t)DK * DV + (w - DK / 32) * 32 + c32;
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) mv[ks][e] = m0[(int64_t)(ks * 16 + hh * 8 + e) * DV];
      }
    }
    fetch(nx, tid, 2);

    // ---- 3. X = (I + A)^-1, blocked by 16: diagonal blocks by substitution, then the blocks
    // below them by sub-diagonal from Z = -X_ii A_im (kept in A's unused blocks above)
    if (tid < 64) {
      const int bi = tid >> 4, cc = tid & 15, base = bi * 16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sacc = (r == cc) ? 1.f : 0.f;
#pragma unroll
        for (int q2 = 0; q2 < r; ++q2) sacc -= Lb[(base + r) * PX + base + q2] * x[q2];
        x[r] = sacc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Xb[(base + r) * PX + base + cc] = x[r];
    }
    lds_barrier();
    fetch(nx, tid, 3);
    for (int e = tid; e < 6 * 256; e += NT) {
      const int bz = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int i = bz < 1 ? 1 : (bz < 3 ? 2 : 3), mm = bz - i * (i - 1) / 2;  // block (i, mm), mm < i
      float z = 0.f;
#pragma unroll
      for (int q2 = 0; q2 < 16; ++q2) z -= Xb[(i * 16 + r) * PX + i * 16 + q2] * Lb[(i * 16 + q2) * PX + mm * 16 + cc];
      Lb[(mm * 16 + r) * PX + i * 16 + cc] = z;
    }
    lds_barrier();
    if constexpr (OUT) {
      if (w >= DK / 32 && w < (DK + DV) / 32) {
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) bm[ks][e] = (bf16)mv[ks][e];
      }
    }
    fetch(nx, tid, 4);
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      for (int e = tid; e < (4 - d) * 256; e += NT) {
        const int k = e >> 8, i = k + d, r = (e >> 4) & 15, cc = e & 15;
        float x = 0.f;
        for (int mm = k; mm < i; ++mm)
#pragma unroll
          for (int q2 = 0; q2 < 16; ++q2) x += Lb[(mm * 16 + r) * PX + i * 16 + q2] * Xb[(mm * 16 + q2) * PX + k * 16 + cc];
        Xb[(i * 16 + r) * PX + k * 16 + cc] = x;
      }
      lds_barrier();
    }
    fetch(nx, tid, 5);

    // ---- 4. K^ T, U T and E~ T, K~ T (maps) or Q^ (outputs): computed into registers from
    // the raw rows and G2, written over them after a barrier.  Task (token t, 8-channel block),
    // t fastest, so the 2-byte column writes of consecutive threads are contiguous.
    {
      constexpr int NKB = DK / 8;
      constexpr int NKTASK = C * NKB / NT;
      static_assert(NKTASK * NT == C * NKB, "tasks per thread");
      bf16x8 kh[NKTASK], et[NKTASK], kw[NKTASK];  // (outputs: et holds Q^)
#pragma unroll
      for (int jj = 0; jj < NKTASK; ++jj) {
        const int task = tid + NT * jj, t = task & (C - 1), c0 = (task / C) * 8;
        const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(rK + t * PK + c0);
        const bf16x8 b8 = *reinterpret_cast<const bf16x8*>(rB + t * PK + c0);
        bf16x8 q8;
        if constexpr (OUT) q8 = *reinterpret_cast<const bf16x8*>(rQ + t * PK + c0);
        float g8[8], ge[8];
        *reinterpret_cast<float4*>(g8) = *reinterpret_cast<const float4*>(sG2 + t * PG + c0);
        *reinterpret_cast<float4*>(g8 + 4) = *reinterpret_cast<const float4*>(sG2 + t * PG + c0 + 4);
        *reinterpret_cast<float4*>(ge) = *reinterpret_cast<const float4*>(s_gend + c0);
        *reinterpret_cast<float4*>(ge + 4) = *reinterpret_cast<const float4*>(s_gend + c0 + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kv = (float)k8[e];
          const float dtl = __builtin_amdgcn_exp2f(ge[e] - g8[e]);
          const float gm = __builtin_amdgcn_exp2f(g8[e]);
          kh[jj][e] = (bf16)(kv * gm);
          kw[jj][e] = (bf16)(kv * dtl);
          if constexpr (OUT)
            et[jj][e] = (bf16)((float)q8[e] * gm);
          else
            et[jj][e] = (bf16)(kv * (float)b8[e] * dtl);
        }
      }
      lds_barrier();  // G2 and the raw rows are dead
#pragma unroll
      for (int jj = 0; jj < NKTASK; ++jj) {
        const int task = tid + NT * jj, t = task & (C - 1), c0 = (task / C) * 8;
        if constexpr (OUT) *reinterpret_cast<bf16x8*>(QpB + t * PK + c0) = et[jj];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          KhT[(c0 + e) * PT + t] = kh[jj][e];
          if constexpr (!OUT) {
            EtT[(c0 + e) * PT + t] = et[jj][e];
            KtT[(c0 + e) * PT + t] = kw[jj][e];
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < NVTASK; ++jj) {
        const int task = tid + NT * jj, t = task & (C - 1), c0 = (task / C) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) UT[(c0 + e) * PT + t] = uu[jj][e];
      }
    }
    lds_barrier();

    // ---- 5. wave w owns column tile w of [At | Bc]
    // X (or B) row r as an A fragment of k-step ks, hi + lo bf16 parts, k in plain order or
    // in the accumulator's row order (two runs of four)
    auto xhl = [&](const float* xr, int ks, bool cl, bf16x8& hi, bf16x8& lo) {
      float xv[8];
      if (cl) {
        *reinterpret_cast<float4*>(xv) = *reinterpret_cast<const float4*>(xr + ks * 16 + hh * 4);
        *reinterpret_cast<float4*>(xv + 4) = *reinterpret_cast<const float4*>(xr + ks * 16 + 8 + hh * 4);
      } else {
        *reinterpret_cast<float4*>(xv) = *reinterpret_cast<const float4*>(xr + ks * 16 + hh * 8);
        *reinterpret_cast<float4*>(xv + 4) = *reinterpret_cast<const float4*>(xr + ks * 16 + hh * 8 + 4);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16 hv = (bf16)xv[e];
        hi[e] = hv;
        lo[e] = (bf16)(xv[e] - (float)hv);
      }
    };
    // W = X K^, columns 32 ct .. (both token tiles)
    auto w_tiles = [&](int ct, f32x16* wt) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x16 acc = zero16();
        const float* xr = Xb + (tt * 32 + c32) * PX;
        const bf16* br = KhT + (ct * 32 + c32) * PT;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          bf16x8 hi, lo;
          xhl(xr, ks, false, hi, lo);
          const bf16x8 bf = Mma<bf16>::load_plain(br, ks, hh);
          acc = Mma<bf16>::mma(hi, bf, acc);
          acc = Mma<bf16>::mma(lo, bf, acc);
        }
        wt[tt] = acc;
      }
    };
    // B U and Z = X (B U), value columns 32 cv .. (both token tiles); returns -Z as B operands
    auto z_tiles = [&](int cv, bf16x8* bz) {
      const bf16* ur = UT + (cv * 32 + c32) * PT;
      f32x16 bu[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x16 acc = zero16();
        const float* brw = Bb + (tt * 32 + c32) * PX;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          bf16x8 hi, lo;
          xhl(brw, ks, false, hi, lo);
          const bf16x8 bf = Mma<bf16>::load_plain(ur, ks, hh);
          acc = Mma<bf16>::mma(hi, bf, acc);
          acc = Mma<bf16>::mma(lo, bf, acc);
        }
        bu[tt] = acc;
      }
      bf16x8 bb[C / 16];
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) bb[ks] = Mma<bf16>::from_acc(bu[ks >> 1], ks, 1.f);
      f32x16 zt[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x16 acc = zero16();
        const float* xr = Xb + (tt * 32 + c32) * PX;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          bf16x8 hi, lo;
          xhl(xr, ks, true, hi, lo);
          acc = Mma<bf16>::mma(hi, bb[ks], acc);
          acc = Mma<bf16>::mma(lo, bb[ks], acc);
        }
        zt[tt] = acc;
      }
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) bz[ks] = Mma<bf16>::from_acc(zt[ks >> 1], ks, -1.f);
    };
    if constexpr (OUT) {
      bf16x8 bz[C / 16];
      if (w < DK / 32) {
        // Q^ - Pe W over the columns 32 w .. of Q^ (staged in QpB), in place
        f32x16 wt[2];
        w_tiles(w, wt);
        bf16x8 bw[C / 16];
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) bw[ks] = Mma<bf16>::from_acc(wt[ks >> 1], ks, -1.f);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          bf16* qp = QpB + (tt * 32 + hh * 4) * PK + w * 32 + c32;
          f32x16 acc;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = (float)qp[((e >> 2) * 8 + (e & 3)) * PK];
          const bf16* pr = PeB + (tt * 32 + c32) * PT;
#pragma unroll
          for (int ks = 0; ks < C / 16; ++ks) acc = Mma<bf16>::mma(Mma<bf16>::load_clayout(pr, ks, hh), bw[ks], acc);
#pragma unroll
          for (int e = 0; e < 16; ++e) qp[((e >> 2) * 8 + (e & 3)) * PK] = (bf16)acc[e];
        }
      } else if (w < (DK + DV) / 32) {
        z_tiles(w - DK / 32, bz);
      }
      lds_barrier();  // Q^ - Pe W complete
      if (w >= DK / 32 && w < (DK + DV) / 32) {
        // O columns 32 cv ..: (Q^ - Pe W) M_0 + Pk U - Pe Z
        const int cv = w - DK / 32;
        const bf16* ur = UT + (cv * 32 + c32) * PT;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          f32x16 acc = zero16();
          const bf16* qr = QpB + (tt * 32 + c32) * PK;
#pragma unroll
          for (int ks = 0; ks < DK / 16; ++ks) acc = Mma<bf16>::mma(Mma<bf16>::load_plain(qr, ks, hh), bm[ks], acc);
          const bf16* kr = PkB + (tt * 32 + c32) * PT;
          const bf16* er = PeB + (tt * 32 + c32) * PT;
#pragma unroll
          for (int ks = 0; ks < C / 16; ++ks) {
            acc = Mma<bf16>::mma(Mma<bf16>::load_plain(kr, ks, hh), Mma<bf16>::load_plain(ur, ks, hh), acc);
            acc = Mma<bf16>::mma(Mma<bf16>::load_clayout(er, ks, hh), bz[ks], acc);
          }
          float* ob = a.o + ((b * a.T + t0 + tt * 32 + hh * 4) * a.H + h) * DV + cv * 32 + c32;
          const int64_t ostride = a.H * DV;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (tt * 32 + acc_row(e, hh) < n) __builtin_nontemporal_store(acc[e], &ob[((e >> 2) * 8 + (e & 3)) * ostride]);
        }
      }
    } else if (w < DK / 32) {
      // W = X K^ (tile columns 32 w ..), then At = Gamma_63 - E~^T W
      const int col0 = w * 32;
      f32x16 wt[2];
      w_tiles(w, wt);
      bf16x8 bw[C / 16];
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) bw[ks] = Mma<bf16>::from_acc(wt[ks >> 1], ks, -1.f);
      bf16* ob = reinterpret_cast<bf16*>(a.At) + cidx * DK * DK + (hh * 4) * DK + col0 + c32;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f32x16 acc = zero16();
        if (rt * 32 == col0) {
          const float gd = __builtin_amdgcn_exp2f(s_gend[col0 + c32]);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = acc_row(e, hh) == c32 ? gd : 0.f;
        }
        const bf16* ar = EtT + (rt * 32 + c32) * PT;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) acc = Mma<bf16>::mma(Mma<bf16>::load_clayout(ar, ks, hh), bw[ks], acc);
        bf16* o = ob + rt * 32 * DK;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[((e >> 2) * 8 + (e & 3)) * DK] = (bf16)acc[e];
      }
    } else if (w < (DK + DV) / 32) {
      // B U and Z = X (B U) (tile columns 32 (w - dk/32) .. of the values), then
      // Bc = K~^T U - E~^T Z
      const int col0 = (w - DK / 32) * 32;
      const bf16* ur = UT + (col0 + c32) * PT;
      bf16x8 bz[C / 16];
      z_tiles(w - DK / 32, bz);
      bf16* ob = reinterpret_cast<bf16*>(a.Bc) + cidx * DK * DV + (hh * 4) * DV + col0 + c32;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f32x16 acc = zero16();
        const bf16* ak = KtT + (rt * 32 + c32) * PT;
        const bf16* ae = EtT + (rt * 32 + c32) * PT;
#pragma unroll
        for (int ks = 0; ks < C / 16; ++ks) {
          acc = Mma<bf16>::mma(Mma<bf16>::load_plain(ak, ks, hh), Mma<bf16>::load_plain(ur, ks, hh), acc);
          acc = Mma<bf16>::mma(Mma<bf16>::load_clayout(ae, ks, hh), bz[ks], acc);
        }
        bf16* o = ob + rt * 32 * DV;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[((e >> 2) * 8 + (e & 3)) * DV] = (bf16)acc[e];
      }
    }
  }  // pieces
}

template <class T, int DK, int DV, bool OUT>
static hipError_t launch_gdn2_t(const ChunkArgs& a, hipStream_t s) {
  constexpr int NT = gdn2_threads<DK, DV, OUT>();
  const int64_t nb = a.B * a.H * (int64_t)a.N;
  TimedLaunch tl(HLA_KERNEL_CHUNK, s);
  hipLaunchKernelGGL((gdn2_chunk_kernel<T, DK, DV, OUT>), dim3((unsigned)nb), dim3(NT < 64 ? 64 : NT), 0, s, a);
  return hipGetLastError();
}

template <class T, bool OUT>
static hipError_t launch_gdn2_d(const ChunkArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_gdn2_t<T, 64, 64, OUT>(a, s);
  if (dk == 64 && dv == 128) return launch_gdn2_t<T, 64, 128, OUT>(a, s);
  if (dk == 128 && dv == 64) return launch_gdn2_t<T, 128, 64, OUT>(a, s);
  return launch_gdn2_t<T, 128, 128, OUT>(a, s);
}

template <int DK, int DV, bool OUT>
static hipError_t launch_gdn2_wy_t(const ChunkArgs& a, hipStream_t s) {
  const int64_t nb = a.B * a.H * (int64_t)a.N;
  // one workgroup per CU (its LDS fills the CU), each looping over pieces
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidDevice;
  const int64_t grid = nb < cus ? nb : cus;
  TimedLaunch tl(HLA_KERNEL_CHUNK, s);
  hipLaunchKernelGGL((gdn2_wy_kernel<DK, DV, OUT>), dim3((unsigned)grid), dim3(512), 0, s, a, nb);
  return hipGetLastError();
}

template <bool OUT>
static hipError_t launch_gdn2_wy_d(const ChunkArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_gdn2_wy_t<64, 64, OUT>(a, s);
  if (dk == 64 && dv == 128) return launch_gdn2_wy_t<64, 128, OUT>(a, s);
  if (dk == 128 && dv == 64) return launch_gdn2_wy_t<128, 64, OUT>(a, s);
  return launch_gdn2_wy_t<128, 128, OUT>(a, s);
}

hipError_t launch_gdn2_chunk(const ChunkArgs& a, int dtype, int dk, int dv, bool want_o, hipStream_t s) {
  // bf16: the WY form on the matrix cores (outputs from float32 start states)
  if (dtype == 1 && (!want_o || a.chunk_init)) return want_o ? launch_gdn2_wy_d<true>(a, dk, dv, s) : launch_gdn2_wy_d<false>(a, dk, dv, s);
  if (dtype == 1) return want_o ? launch_gdn2_d<bf16, true>(a, dk, dv, s) : launch_gdn2_d<bf16, false>(a, dk, dv, s);
  return want_o ? launch_gdn2_d<float, true>(a, dk, dv, s) : launch_gdn2_d<float, false>(a, dk, dv, s);
}

}  // namespace hla
