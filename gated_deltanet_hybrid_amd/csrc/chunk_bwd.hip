// Backward of the per-chunk work: the routed outputs of a chunk from its start state, and
// the chunk's exact affine map.
//
// Every column x of the stored state M = S^T [dk, dv] follows the token recurrence on its
// own ([HLA] Methodology paragraph 1, the gated delta rule):
//     a_t = k_t . x,   x <- alpha_t (x - beta_t k_t a_t) + beta_t k_t u_t,
// with u_t = v_t[col] for a state column and o_t[col] = q_t . x after the token.  The chunk
// map M_end = At M_start + Bc is the same recurrence on dk + dv columns: the columns of At
// start at the identity and take no write (u = 0), those of Bc start at zero and write v.
// The reverse of one token, with dx = dL/dx after it (plus q_t dO_t[col] for outputs):
//     b = k_t . dx,   dv_t[col] += beta b,   dbeta_t += b (u - alpha a),
//     dalpha_t += dx . x_prev - beta a b,
//     dk_t += beta u dx - alpha beta (a dx + b x_prev),   dq_t += dO_t[col] x_after,
//     dx <- alpha (dx - beta k_t b).
// dk, dq, dbeta and dalpha sum over every column; dv_t[col] comes from one column.
//
// Layout: one workgroup per (b, h, chunk, block of 32 columns); a thread holds 8 rows of one
// column (the dk / 8 threads of a column are adjacent lanes, so a dot product is a sum over
// 8 rows plus log2(dk / 8) DPP lane moves, which keeps the token recurrence's critical path
// short).  The reverse needs the state in front of every
// token: a forward pass keeps the state in front of every 8-token block in registers (8
// checkpoints x 8 rows per thread), and each block is replayed from its checkpoint before
// it is reversed.
// Sums over columns run through DPP row moves and gfx950's permlane swaps inside a wave
// (no LDS traffic) and through LDS across waves, once per block of 8 tokens; every workgroup writes its own partial sums, which
// chunk_bwd_finalize_kernel adds in a fixed order (no atomics: deterministic).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {
constexpr int kRPT = 8;  // rows per thread
constexpr int kTB = 8;   // tokens per checkpoint block
}  // namespace

template <int DK>
constexpr int chunk_bwd_threads() {
  return 32 * (DK / kRPT);
}

template <class T, int DK, int DV, bool OUT>
__global__ __launch_bounds__(chunk_bwd_threads<DK>()) void chunk_bwd_kernel(ChunkBwdArgs a) {
  constexpr int C = kChunk, RG = DK / kRPT, NTH = 32 * RG, NWV = NTH / 64;
  constexpr int NB_OUT = DV / 32, NB_MAP = (DK + DV) / 32, NB = OUT ? NB_OUT : NB_MAP, NB_ALL = NB_OUT + NB_MAP;
  constexpr int NRED = DK + 2;  // per wave and token: dk partial, then dbeta, dalpha
  __shared__ __attribute__((aligned(16))) float s_k[C][DK];
  __shared__ __attribute__((aligned(16))) float s_q[OUT ? C : 1][DK];
  __shared__ float s_u[C][32];
  __shared__ float s_do[OUT ? C : 1][32];
  __shared__ float s_beta[C], s_alpha[C];
  __shared__ float s_red[kTB][NWV][NRED];
  __shared__ float s_redq[OUT ? kTB : 1][NWV][DK];

  const int tid = threadIdx.x, rg = tid % RG, cl = tid / RG, lane = tid & 63, wv = tid >> 6;
  const int64_t id = blockIdx.x;
  const int cb = (int)(id % NB);
  const int64_t rest = id / NB;
  const int c = a.c0 + (int)(rest % (a.c1 - a.c0));
  const int64_t bh = rest / (a.c1 - a.c0);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)c * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
  const int r0 = rg * kRPT;
  // this thread's column: a state column (outputs), or a column of [At | Bc] (map)
  const int colall = cb * 32 + cl;
  const bool isP = !OUT && colall < DK;
  const bool writes = !isP;
  const int vcol = OUT ? colall : colall - DK;  // column of v / Bc (when writes)
  const int blk = OUT ? cb : NB_OUT + cb;       // partial-sum slot of this workgroup

  // ---- stage the chunk's tokens
  const T* kg = reinterpret_cast<const T*>(a.k);
  const T* qg = reinterpret_cast<const T*>(a.q);
  const T* vg = reinterpret_cast<const T*>(a.v);
  for (int i = tid; i < C * DK; i += NTH) {
    const int t = i / DK, r = i % DK;
    const int64_t row = row0 + (int64_t)t * a.H;
    s_k[t][r] = t < n ? to_f<T>(kg[row * DK + r]) : 0.f;
    if constexpr (OUT) s_q[t][r] = t < n ? to_f<T>(qg[row * DK + r]) : 0.f;
  }
  for (int i = tid; i < C * 32; i += NTH) {
    const int t = i / 32, cc = i % 32;
    const int64_t row = row0 + (int64_t)t * a.H;
    const int vc = OUT ? cb * 32 + cc : cb * 32 + cc - DK;
    const bool w = OUT || cb * 32 >= DK;
    s_u[t][cc] = (t < n && w) ? to_f<T>(vg[row * DV + vc]) : 0.f;
    if constexpr (OUT) s_do[t][cc] = t < n ? a.dO[((b * a.T + t0 + t) * a.H + h) * DV + vc] : 0.f;
  }
  if (tid < C) {
    const int64_t row = row0 + (int64_t)tid * a.H;
    s_beta[tid] = tid < n ? a.beta[row] : 0.f;
    s_alpha[tid] = tid < n ? a.alpha[row] : 1.f;
  }
  __syncthreads();

  auto rowdot = [&](const float* vec, const float* x) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kRPT; ++i) s = fmaf(vec[r0 + i], x[i], s);
    return group_sum<RG>(s);  // the column's RG threads are one aligned lane group
  };

  // ---- forward, keeping the state in front of every 8-token block
  float x[kRPT];
  if constexpr (OUT) {
    const float* M0 = a.chunk_init + ((bh * a.N + c) * (int64_t)DK) * DV;
#pragma unroll
    for (int i = 0; i < kRPT; ++i) x[i] = M0[(int64_t)(r0 + i) * DV + colall];
  } else {
#pragma unroll
    for (int i = 0; i < kRPT; ++i) x[i] = (isP && r0 + i == colall) ? 1.f : 0.f;
  }
  // x <- alpha (x - beta k a) + beta k u  =  alpha x + c k  with  c = beta (u - alpha a)
  auto step = [&](int t, float* xx) {
    const float at = rowdot(s_k[t], xx);
    const float be = s_beta[t], al = s_alpha[t], u = s_u[t][cl];
    const float cc = be * fmaf(-al, at, u);
#pragma unroll
    for (int i = 0; i < kRPT; ++i) xx[i] = fmaf(cc, s_k[t][r0 + i], al * xx[i]);
    return at;
  };
  float ck[C / kTB][kRPT];
  // Tokens past the end of a partial chunk are staged as k = 0, beta = 0, alpha = 1, u = 0
  // and dO = 0: exact identity steps both ways, so every loop runs all 64 tokens without
  // branches (their partial sums land in slots the finalize pass never reads).
#pragma unroll
  for (int s = 0; s < C / kTB; ++s) {
#pragma unroll
    for (int i = 0; i < kRPT; ++i) ck[s][i] = x[i];
#pragma unroll
    for (int u = 0; u < kTB; ++u) step(s * kTB + u, x);
  }

  // ---- reverse, one 8-token block at a time
  float dx[kRPT];
  if constexpr (OUT) {
#pragma unroll
    for (int i = 0; i < kRPT; ++i) dx[i] = 0.f;
  } else {
    const int64_t cc = bh * a.N + c;
#pragma unroll
    for (int i = 0; i < kRPT; ++i)
      dx[i] = isP ? a.dAt[(cc * DK + r0 + i) * DK + colall] : a.dBc[(cc * DK + r0 + i) * DV + vcol];
  }
  float* pv = a.part_v + ((bh * a.N + c) * 2 + (OUT ? 0 : 1)) * (int64_t)C * DV;
  const int nblk = (n + kTB - 1) / kTB;
  for (int s = nblk - 1; s >= 0; --s) {
    const int tb = s * kTB;
    {
      float xs[kTB][kRPT], av[kTB];
      // the block's checkpoint, picked with compile-time register indices
#pragma unroll
      for (int ss = 0; ss < C / kTB; ++ss)
#pragma unroll
        for (int i = 0; i < kRPT; ++i) x[i] = ss == s ? ck[ss][i] : x[i];
#pragma unroll
      for (int u = 0; u < kTB; ++u) {
#pragma unroll
        for (int i = 0; i < kRPT; ++i) xs[u][i] = x[i];
        av[u] = step(tb + u, x);
      }
#pragma unroll
      for (int u = kTB - 1; u >= 0; --u) {
        {
          const int t = tb + u;
          const float be = s_beta[t], al = s_alpha[t], uu = s_u[t][cl], at = av[u];
          float pq[kRPT];
          if constexpr (OUT) {
            const float go = s_do[t][cl];
#pragma unroll
            for (int i = 0; i < kRPT; ++i) {
              const float xa = u + 1 < kTB ? xs[u + 1 < kTB ? u + 1 : u][i] : x[i];  // state after token t
              dx[i] = fmaf(s_q[t][r0 + i], go, dx[i]);
              pq[i] = xa * go;
            }
          }
          const float bd = rowdot(s_k[t], dx);
          if (writes && rg == 0) pv[(int64_t)t * DV + vcol] = be * bd;
          float pa = rg == 0 ? -be * at * bd : 0.f;
          const float pb = rg == 0 ? bd * (uu - al * at) : 0.f;
          // dk partial = beta (u - alpha a) dx - alpha beta b x_prev;  dx <- alpha dx - alpha beta b k
          const float c1 = be * fmaf(-al, at, uu), c2 = -al * be * bd;
          float pk[kRPT];
#pragma unroll
          for (int i = 0; i < kRPT; ++i) {
            const float xp = xs[u][i];
            pa = fmaf(dx[i], xp, pa);
            pk[i] = fmaf(c2, xp, c1 * dx[i]);
            dx[i] = fmaf(c2, s_k[t][r0 + i], al * dx[i]);
          }
          // sums over the wave's columns (lanes with the same row group), in the VALU: with
          // 8-lane row groups the two columns of a 16-lane row are added first; then
          // rows_sum8 leaves row rho with the totals of rows r0 + rho and r0 + 4 + rho
          static_assert(kRPT == 8, "rows_sum8 takes the thread's 8 rows");
          if constexpr (RG == 8) {
#pragma unroll
            for (int i = 0; i < kRPT; ++i) {
              pk[i] += dpp_f<0x128>(pk[i]);  // row_ror 8: the other column of the row
              if constexpr (OUT) pq[i] += dpp_f<0x128>(pq[i]);
            }
          }
          float ka, kb2, qa = 0.f, qb2 = 0.f;
          rows_sum8(pk, ka, kb2);
          if constexpr (OUT) rows_sum8(pq, qa, qb2);
          const float pab = wave_sum_valu(pa), pbb = wave_sum_valu(pb);
          const int rho = lane >> 4;
          if (RG == 16 || ((lane >> 3) & 1) == 0) {
            s_red[u][wv][r0 + rho] = ka;
            s_red[u][wv][r0 + 4 + rho] = kb2;
            if constexpr (OUT) {
              s_redq[u][wv][r0 + rho] = qa;
              s_redq[u][wv][r0 + 4 + rho] = qb2;
            }
          }
          if (lane == 0) {
            s_red[u][wv][DK] = pbb;
            s_red[u][wv][DK + 1] = pab;
          }
        }
      }
      __syncthreads();
      // sums over the waves, written as this workgroup's partial sums
      const int64_t slot = ((bh * a.N + c) * NB_ALL + blk) * (int64_t)C;
      for (int i = tid; i < kTB * NRED; i += NTH) {
        const int u = i / NRED, e = i % NRED;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) sum += s_red[u][w][e];
        if (e < DK)
          a.part_k[(slot + tb + u) * DK + e] = sum;
        else
          a.part_s[(slot + tb + u) * 2 + (e - DK)] = sum;
      }
      if constexpr (OUT) {
        const int64_t qslot = ((bh * a.N + c) * NB_OUT + cb) * (int64_t)C;
        for (int i = tid; i < kTB * DK; i += NTH) {
          const int u = i / DK, e = i % DK;
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < NWV; ++w) sum += s_redq[u][w][e];
          a.part_q[(qslot + tb + u) * DK + e] = sum;
        }
      }
      __syncthreads();  // s_red is reused by the next block
    }
  }
  if constexpr (OUT) {
    float* dM0 = a.dchunk_init + ((bh * a.N + c) * (int64_t)DK) * DV;
#pragma unroll
    for (int i = 0; i < kRPT; ++i) dM0[(int64_t)(r0 + i) * DV + colall] = dx[i];
  }
}

// ---------------------------------------------------------------------------------------
// The chunk-map part of the reverse through the UT form, on the matrix cores (bf16 inputs,
// float32 arithmetic).
//
// [HLA] Methodology paragraph 1: a piece's map is At = gamma_63 I - K^T D W and
// Bc = K^T D U, with (for the piece's tokens t, s)
//     A0 = strictly_lower((K K^T) o Gamma),  L = diag(beta) A0,  X = (I + L)^-1,
//     W = X diag(beta gamma) K,  U = X diag(beta) V,  D = diag(exp(g_63 - g_s)).
// Given dAt and dBc (float32) the reverse is, in this order,
//     dY = -K dAt,  dKB = K dBc,  dD_s = dY_s . W_s + dKB_s . U_s,  dW = D dY,  dU = D dKB,
//     dK  = D (-W dAt^T + U dBc^T),                                (K in K^T D W, K^T D U)
//     F = X^T dU,  G = X^T dW,  dV = diag(beta) F,  dK += diag(beta gamma) G,
//     T1 = X^T dX = F (diag(beta) V)^T + G (diag(beta gamma) K)^T,  H = -T1 X^T (s < t),
//     dK += H' K + H'^T K,  H'_ts = beta_t Gamma_ts H_ts,
//     dbeta_t = F_t . v_t + gamma_t G_t . k_t + sum_s H_ts A0_ts,
//     dg_t = beta_t gamma_t G_t . k_t + sum_s Psi_ts - sum_s Psi_st - dD_t D_t
//            (+ sum_s dD_s D_s + tr(dAt) gamma_63 at t = 63),   Psi_ts = beta_t H_ts A0_ts,
//     dlog alpha_s = sum_{t >= s} dg_t,  dalpha = dlog alpha / alpha.
// One workgroup of 8 waves per (b, h, piece); every product is a 32 x 32 tile of
// v_mfma_f32_32x32x2_f32 with its operands read from LDS (dAt, dBc from global memory), and
// wave w owns tile w of the 64 x dk and of the 64 x dv results.  The workgroup writes its
// per-token sums into the first chunk-map slot of the partial sums.
namespace {
// C (32 x 32) += A B over KD k values: fa(k) = A[m0 + lane % 32][k], fb(k) = B[k][n0 + lane % 32]
template <int KD, class FA, class FB>
__device__ __forceinline__ f32x16 mm32(f32x16 acc, int hh, FA fa, FB fb) {
#pragma unroll 8
  for (int ks = 0; ks < KD / 2; ++ks) {
    const int k = 2 * ks + hh;
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa(k), fb(k), acc, 0, 0, 0);
  }
  return acc;
}
}  // namespace

template <int DK, int DV>
__global__ __launch_bounds__(512, 1) void chunk_bwd_map_ut_kernel(ChunkBwdArgs a) {
  constexpr int C = kChunk, NT = 512;
  constexpr int PX = C + 4;                // float32 pitch of the 64 x 64 matrices
  constexpr int PK = DK + 8, PV = DV + 8;  // bf16 pitch of the k and v rows
  constexpr int PW = DK + 4, PU = DV + 4;  // float32 pitch of W (dW, G) and U (dU, F)
  constexpr int NKT = 2 * (DK / 32), NVT = 2 * (DV / 32);  // 32 x 32 tiles of 64 x dk, 64 x dv
  constexpr int NB_OUT = DV / 32, NB_ALL = NB_OUT + (DK + DV) / 32;
  static_assert(NKT <= 8 && NVT <= 8, "one tile of each kind per wave");
  __shared__ __attribute__((aligned(16))) float A0[C * PX];  // lower: Gamma o K K^T; upper blocks: scratch
  __shared__ __attribute__((aligned(16))) float Xb[C * PX];
  __shared__ __attribute__((aligned(16))) float Tb[C * PX];  // T1, then H
  __shared__ __attribute__((aligned(16))) bf16 Ks[C * PK];
  __shared__ __attribute__((aligned(16))) bf16 Vs[C * PV];
  __shared__ __attribute__((aligned(16))) float Wb[C * PW];  // W, then dW, then G
  __shared__ __attribute__((aligned(16))) float Ub[C * PU];  // U, then dU, then F
  __shared__ float s_beta[C], s_alpha[C], s_g2[C], s_gam[C], s_D[C], s_dD[C];
  __shared__ float s_red[C][8];
  __shared__ float s_row[3][C];  // sum_s Psi_ts, sum_t Psi_ts (by s), sum_s H_ts A0_ts
  __shared__ float s_tr;

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t id = blockIdx.x;
  const int c = a.c0 + (int)(id % (a.c1 - a.c0));
  const int64_t bh = id / (a.c1 - a.c0);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)c * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
  const int64_t cc = bh * a.N + c;
  const float* dAt = a.dAt + cc * (int64_t)DK * DK;
  const float* dBc = a.dBc + cc * (int64_t)DK * DV;

  // ---- 0. k, v rows (zero past the end), per-token gates and decays
  {
    const bf16* kg = reinterpret_cast<const bf16*>(a.k);
    const bf16* vg = reinterpret_cast<const bf16*>(a.v);
    for (int i = tid; i < C * (DK / 8); i += NT) {
      const int t = i / (DK / 8), u = i % (DK / 8);
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (t < n) x = *reinterpret_cast<const uint4*>(kg + (row0 + (int64_t)t * a.H) * DK + u * 8);
      *reinterpret_cast<uint4*>(Ks + t * PK + u * 8) = x;
    }
    for (int i = tid; i < C * (DV / 8); i += NT) {
      const int t = i / (DV / 8), u = i % (DV / 8);
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (t < n) x = *reinterpret_cast<const uint4*>(vg + (row0 + (int64_t)t * a.H) * DV + u * 8);
      *reinterpret_cast<uint4*>(Vs + t * PV + u * 8) = x;
    }
    for (int i = tid; i < C * PX; i += NT) Xb[i] = 0.f;
    if (tid < C) {
      const int64_t r = row0 + (int64_t)tid * a.H;
      const float be = tid < n ? a.beta[r] : 0.f, al = tid < n ? a.alpha[r] : 1.f;
      float x = logf(fmaxf(al, 1.17549435e-38f));  // alpha = 0 (a reset) stays finite
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {  // inclusive prefix sum over wave 0
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float x_end = __shfl(x, 63, 64);
      s_beta[tid] = be;
      s_alpha[tid] = al;
      s_g2[tid] = x * 1.4426950408889634f;
      s_gam[tid] = expf(x);
      s_D[tid] = expf(x_end - x);
    }
    if (w == 2) {  // tr(dAt)
      float tr = 0.f;
      for (int i = lane; i < DK; i += 64) tr += dAt[(int64_t)i * DK + i];
      tr = wave_sum(tr);
      if (lane == 0) s_tr = tr;
    }
  }
  __syncthreads();

  // ---- 1. A0 = strictly_lower(Gamma o K K^T): tiles (0,0), (1,0), (1,1) on waves 0-2
  // (bf16 products of the bf16 keys, float32 sums); wave 3 zeroes tile (0,1)
  if (w < 3) {
    const int tm = w == 0 ? 0 : 1, tn = w == 2 ? 1 : 0;
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      acc = Mma<bf16>::mma(Mma<bf16>::load_plain(Ks + (tm * 32 + c32) * PK, ks, hh),
                           Mma<bf16>::load_plain(Ks + (tn * 32 + c32) * PK, ks, hh), acc);
    const int s = tn * 32 + c32;
    const float gs = s_g2[s];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      A0[t * PX + s] = s < t ? __builtin_amdgcn_exp2f(s_g2[t] - gs) * acc[e] : 0.f;
    }
  } else if (w == 3) {
    for (int i = lane; i < 32 * 32; i += 64) A0[(i >> 5) * PX + 32 + (i & 31)] = 0.f;
  }
  __syncthreads();

  // ---- 2. X = (I + L)^-1 with L = diag(beta) A0, blocked by 16: the diagonal blocks by
  // substitution, then the blocks below them by sub-diagonal from Z = -X_ii L_im (kept in
  // A0's unused blocks above the diagonal)
  if (tid < 64) {
    const int bi = tid >> 4, cl = tid & 15, base = bi * 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cl) ? 1.f : 0.f;
      const float br = s_beta[base + r];
#pragma unroll
      for (int q2 = 0; q2 < r; ++q2) s -= br * A0[(base + r) * PX + base + q2] * x[q2];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Xb[(base + r) * PX + base + cl] = x[r];
  }
  __syncthreads();
  for (int e = tid; e < 6 * 256; e += NT) {
    const int bz = e >> 8, r = (e >> 4) & 15, cl = e & 15;
    const int i = bz < 1 ? 1 : (bz < 3 ? 2 : 3), m = bz - i * (i - 1) / 2;
    float z = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 16; ++q2)
      z -= Xb[(i * 16 + r) * PX + i * 16 + q2] * s_beta[i * 16 + q2] * A0[(i * 16 + q2) * PX + m * 16 + cl];
    A0[(m * 16 + r) * PX + i * 16 + cl] = z;
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    for (int e = tid; e < (4 - d) * 256; e += NT) {
      const int k = e >> 8, i = k + d, r = (e >> 4) & 15, cl = e & 15;
      float x = 0.f;
      for (int m = k; m < i; ++m)
#pragma unroll
        for (int q2 = 0; q2 < 16; ++q2) x += A0[(m * 16 + r) * PX + i * 16 + q2] * Xb[(m * 16 + q2) * PX + k * 16 + cl];
      Xb[(i * 16 + r) * PX + k * 16 + cl] = x;
    }
    __syncthreads();
  }

  // wave w's tiles: (rows tk * 32, columns ck * 32) of the 64 x dk results and (tv, cv) of
  // the 64 x dv ones
  const bool hk = w < NKT, hv = w < NVT;
  const int tk = w & 1, ck = w >> 1, tv = w & 1, cv = w >> 1;
  const int rk0 = tk * 32, rv0 = tv * 32;  // first row of the tiles
  auto tok = [&](int r0, int e) { return r0 + acc_row(e, hh); };

  // ---- 3. W = X diag(beta gamma) K and U = X diag(beta) V
  if (hk) {
    const float* xr = Xb + (rk0 + c32) * PX;
    const bf16* kc = Ks + ck * 32 + c32;
    const f32x16 acc = mm32<C>(zero16(), hh, [&](int k) { return xr[k] * s_beta[k] * s_gam[k]; },
                               [&](int k) { return (float)kc[k * PK]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) Wb[tok(rk0, e) * PW + ck * 32 + c32] = acc[e];
  }
  if (hv) {
    const float* xr = Xb + (rv0 + c32) * PX;
    const bf16* vc = Vs + cv * 32 + c32;
    const f32x16 acc = mm32<C>(zero16(), hh, [&](int k) { return xr[k] * s_beta[k]; },
                               [&](int k) { return (float)vc[k * PV]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) Ub[tok(rv0, e) * PU + cv * 32 + c32] = acc[e];
  }
  __syncthreads();

  // ---- 4. dY = -K dAt, dKB = K dBc, dK_ab = D (-W dAt^T + U dBc^T), dD
  f32x16 dkab = zero16(), dy = zero16(), dkb = zero16();
  if (hk) {
    const bf16* kr = Ks + (rk0 + c32) * PK;
    const float* wr = Wb + (rk0 + c32) * PW;
    const float* ur = Ub + (rk0 + c32) * PU;
    const int nc = ck * 32 + c32;
    dy = mm32<DK>(dy, hh, [&](int k) { return -(float)kr[k]; }, [&](int k) { return dAt[(int64_t)k * DK + nc]; });
    dkab = mm32<DK>(dkab, hh, [&](int k) { return -wr[k]; }, [&](int k) { return dAt[(int64_t)nc * DK + k]; });
    dkab = mm32<DV>(dkab, hh, [&](int k) { return ur[k]; }, [&](int k) { return dBc[(int64_t)nc * DV + k]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) dkab[e] *= s_D[tok(rk0, e)];
  }
  if (hv) {
    const bf16* kr = Ks + (rv0 + c32) * PK;
    const int nc = cv * 32 + c32;
    dkb = mm32<DK>(dkb, hh, [&](int k) { return (float)kr[k]; }, [&](int k) { return dBc[(int64_t)k * DV + nc]; });
  }
  // dD_t = dY_t . W_t + dKB_t . U_t: each tile's 32 columns summed over the lanes of a half
  if (hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = lane_group_sum<32>(dy[e] * Wb[tok(rk0, e) * PW + ck * 32 + c32]);
      if (c32 == 0) s_red[tok(rk0, e)][ck] = p;
    }
  }
  if (hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = lane_group_sum<32>(dkb[e] * Ub[tok(rv0, e) * PU + cv * 32 + c32]);
      if (c32 == 0) s_red[tok(rv0, e)][DK / 32 + cv] = p;
    }
  }
  __syncthreads();  // W, U and the partial sums are complete
  if (tid < C) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < DK / 32 + DV / 32; ++j) s += s_red[tid][j];
    s_dD[tid] = s;
  }
  if (hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Wb[tok(rk0, e) * PW + ck * 32 + c32] = s_D[tok(rk0, e)] * dy[e];  // dW
  }
  if (hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Ub[tok(rv0, e) * PU + cv * 32 + c32] = s_D[tok(rv0, e)] * dkb[e];  // dU
  }
  __syncthreads();

  // ---- 5. G = X^T dW, F = X^T dU
  f32x16 gt = zero16(), ft = zero16();
  if (hk) {
    const float* xc = Xb + rk0 + c32;
    const float* dw = Wb + ck * 32 + c32;
    gt = mm32<C>(gt, hh, [&](int k) { return xc[k * PX]; }, [&](int k) { return dw[k * PW]; });
  }
  if (hv) {
    const float* xc = Xb + rv0 + c32;
    const float* du = Ub + cv * 32 + c32;
    ft = mm32<C>(ft, hh, [&](int k) { return xc[k * PX]; }, [&](int k) { return du[k * PU]; });
  }
  __syncthreads();  // dW, dU are dead
  if (hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Wb[tok(rk0, e) * PW + ck * 32 + c32] = gt[e];
  }
  if (hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) Ub[tok(rv0, e) * PU + cv * 32 + c32] = ft[e];
  }
  __syncthreads();

  // ---- 6. T1 = F (diag(beta) V)^T + G (diag(beta gamma) K)^T: tile (tm, tn) on wave tm + 2 tn
  if (w < 4) {
    const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
    const float* fr = Ub + (tm * 32 + c32) * PU;
    const float* gr = Wb + (tm * 32 + c32) * PW;
    const bf16* vr = Vs + s * PV;
    const bf16* kr = Ks + s * PK;
    const f32x16 a1 = mm32<DV>(zero16(), hh, [&](int k) { return fr[k]; }, [&](int k) { return (float)vr[k]; });
    const f32x16 a2 = mm32<DK>(zero16(), hh, [&](int k) { return gr[k]; }, [&](int k) { return (float)kr[k]; });
    const float bs = s_beta[s], gs = s_gam[s];
#pragma unroll
    for (int e = 0; e < 16; ++e) Tb[(tm * 32 + acc_row(e, hh)) * PX + s] = bs * (a1[e] + gs * a2[e]);
  }
  __syncthreads();
  // ---- 7. H = -T1 X^T, kept below the diagonal
  f32x16 ht = zero16();
  if (w < 4) {
    const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
    const float* tr = Tb + (tm * 32 + c32) * PX;
    const float* xr = Xb + s * PX;
    ht = mm32<C>(ht, hh, [&](int k) { return tr[k]; }, [&](int k) { return xr[k]; });
  }
  __syncthreads();
  if (w < 4) {
    const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      Tb[t * PX + s] = s < t ? -ht[e] : 0.f;
    }
  }
  __syncthreads();

  // ---- 8. dK = dK_ab + diag(beta gamma) G + H' K + H'^T K;  dV = diag(beta) F
  const int64_t pslot = (cc * NB_ALL + NB_OUT) * (int64_t)C;  // first chunk-map slot
  if (hk) {
    const int t = rk0 + c32;
    const float* hr = Tb + t * PX;  // row t of H
    const float* hc = Tb + t;       // column t of H
    const bf16* kc = Ks + ck * 32 + c32;
    const float bt = s_beta[t], g2t = s_g2[t];
    f32x16 acc = mm32<C>(zero16(), hh,
                         [&](int k) { return k < t ? hr[k] * bt * __builtin_amdgcn_exp2f(g2t - s_g2[k]) : 0.f; },
                         [&](int k) { return (float)kc[k * PK]; });
    acc = mm32<C>(acc, hh,
                  [&](int k) { return k > t ? hc[k * PX] * s_beta[k] * __builtin_amdgcn_exp2f(s_g2[k] - g2t) : 0.f; },
                  [&](int k) { return (float)kc[k * PK]; });
    float* pk = a.part_k + pslot * DK + ck * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = tok(rk0, e);
      if (te < n) pk[(int64_t)te * DK] = acc[e] + dkab[e] + s_beta[te] * s_gam[te] * gt[e];
    }
  }
  if (hv) {
    float* pv = a.part_v + (cc * 2 + 1) * (int64_t)C * DV + cv * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = tok(rv0, e);
      if (te < n) pv[(int64_t)te * DV] = s_beta[te] * ft[e];
    }
  }
  // ---- 9. the per-token dots: F_t . v_t, G_t . k_t (by tiles), the sums of Psi and of
  // H o A0 (threads 0-127), then dbeta, dg and the reverse cumulative sum for dalpha
  if (hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = tok(rv0, e);
      const float p = lane_group_sum<32>(ft[e] * (float)Vs[te * PV + cv * 32 + c32]);
      if (c32 == 0) s_red[te][cv] = p;
    }
  }
  if (hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = tok(rk0, e);
      const float p = lane_group_sum<32>(gt[e] * (float)Ks[te * PK + ck * 32 + c32]);
      if (c32 == 0) s_red[te][4 + ck] = p;
    }
  }
  if (tid < C) {
    const int t = tid;
    float ps = 0.f, ha = 0.f;
    for (int s = 0; s < t; ++s) {
      const float x = Tb[t * PX + s] * A0[t * PX + s];
      ha += x;
    }
    ps = s_beta[t] * ha;
    s_row[0][t] = ps;
    s_row[2][t] = ha;
  } else if (tid < 2 * C) {
    const int s = tid - C;
    float pc = 0.f;
    for (int t = s + 1; t < C; ++t) pc += s_beta[t] * Tb[t * PX + s] * A0[t * PX + s];
    s_row[1][s] = pc;
  }
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    float fv = 0.f, gk = 0.f;
#pragma unroll
    for (int j = 0; j < DV / 32; ++j) fv += s_red[t][j];
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) gk += s_red[t][4 + j];
    const float be = s_beta[t], ga = s_gam[t], dd = s_dD[t] * s_D[t];
    const float dbeta = fv + ga * gk + s_row[2][t];
    float dg = be * ga * gk + s_row[0][t] - s_row[1][t] - dd;
    const float ddsum = wave_sum(dd);
    if (t == C - 1) dg += ddsum + s_tr * ga;
    // dlog alpha_t = sum_{u >= t} dg_u: inclusive suffix sum over the wave
    float x = dg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (lane + off < 64) x += y;
    }
    if (t < n) {
      float* ps = a.part_s + (pslot + t) * 2;
      ps[0] = dbeta;
      ps[1] = x / fmaxf(s_alpha[t], 1.17549435e-38f);
    }
  }
}

// dq, dk, dv, dbeta, dalpha of every token: the workgroups' partial sums in a fixed order,
// plus the router's parts (dqbar of the token's chunk divided by its token count, and the
// per-token key gradient) when given.  One thread per (b, t, h, row).
template <int DK, int DV>
__global__ __launch_bounds__(256) void chunk_bwd_finalize_kernel(ChunkBwdArgs a) {
  constexpr int C = kChunk, NB_OUT = DV / 32, NB_MAP = (DK + DV) / 32, NB_ALL = NB_OUT + NB_MAP;
  constexpr int W = DK > DV ? DK : DV;
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  const int64_t total = a.B * a.T * a.H * W;
  if (id >= total) return;
  const int e = (int)(id % W);
  const int64_t bth = id / W;
  const int64_t h = bth % a.H, bt = bth / a.H;
  const int64_t t = bt % a.T, b = bt / a.T;
  const int c = (int)(t / C), u = (int)(t % C);
  const int64_t bh = b * a.H + h;
  const int64_t base = (bh * a.N + c) * NB_ALL;
  const int b0 = a.have_out ? 0 : NB_OUT, b1 = a.have_map ? (a.map_ut ? NB_OUT + 1 : NB_ALL) : NB_OUT;
  // every partial sum is read once, here: non-temporal loads, all of a thread's in flight
  if (e < DK) {
    float sk = 0.f;
#pragma unroll
    for (int k = 0; k < NB_ALL; ++k)
      if (k >= b0 && k < b1) sk += __builtin_nontemporal_load(a.part_k + ((base + k) * C + u) * DK + e);
    if (a.dk_router) sk += a.dk_router[bth * DK + e];
    a.dk[bth * DK + e] = sk;
    float sq = 0.f;
    if (a.have_out) {
      const int64_t qb = (bh * a.N + c) * NB_OUT;
#pragma unroll
      for (int k = 0; k < NB_OUT; ++k) sq += __builtin_nontemporal_load(a.part_q + ((qb + k) * C + u) * DK + e);
    }
    if (a.dqbar) {
      const int64_t t0 = (int64_t)c * C;
      const int nc = (int)((a.T - t0) < C ? (a.T - t0) : C);
      sq += a.dqbar[(bh * a.N + c) * DK + e] / (float)nc;
    }
    a.dq[bth * DK + e] = sq;
  }
  if (e < DV) {
    float sv = 0.f;
    if (a.have_out) sv += a.part_v[((bh * a.N + c) * 2 + 0) * (int64_t)C * DV + (int64_t)u * DV + e];
    if (a.have_map) sv += a.part_v[((bh * a.N + c) * 2 + 1) * (int64_t)C * DV + (int64_t)u * DV + e];
    a.dv[bth * DV + e] = sv;
  }
  if (e < 2) {
    float ss = 0.f;
    for (int k = b0; k < b1; ++k) ss += a.part_s[((base + k) * C + u) * 2 + e];
    (e == 0 ? a.dbeta : a.dalpha)[bth] = ss;
  }
}

template <class T, int DK, int DV>
static hipError_t launch_chunk_bwd_t(const ChunkBwdArgs& a, int stages, hipStream_t s) {
  const int64_t BHN = a.B * a.H * (int64_t)(a.c1 - a.c0);
  constexpr int NT = chunk_bwd_threads<DK>();
  if ((stages & (kChunkBwdOut | kChunkBwdMap)) && BHN > 0) {
    TimedLaunch tl(HLA_KERNEL_BWD_CHUNK, s);
    if (stages & kChunkBwdOut)
      hipLaunchKernelGGL((chunk_bwd_kernel<T, DK, DV, true>), dim3((unsigned)(BHN * (DV / 32))), dim3(NT), 0, s, a);
    if (stages & kChunkBwdMap) {
      if (a.map_ut)
        hipLaunchKernelGGL((chunk_bwd_map_ut_kernel<DK, DV>), dim3((unsigned)BHN), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((chunk_bwd_kernel<T, DK, DV, false>), dim3((unsigned)(BHN * ((DK + DV) / 32))), dim3(NT),
                           0, s, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(stages & kChunkBwdFinalize)) return e;
  constexpr int W = DK > DV ? DK : DV;
  const int64_t total = a.B * a.T * a.H * W;
  hipLaunchKernelGGL((chunk_bwd_finalize_kernel<DK, DV>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_chunk_bwd_d(const ChunkBwdArgs& a, int dk, int dv, int stages, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_chunk_bwd_t<T, 64, 64>(a, stages, s);
  if (dk == 64 && dv == 128) return launch_chunk_bwd_t<T, 64, 128>(a, stages, s);
  if (dk == 128 && dv == 64) return launch_chunk_bwd_t<T, 128, 64>(a, stages, s);
  return launch_chunk_bwd_t<T, 128, 128>(a, stages, s);
}

hipError_t launch_chunk_backward(const ChunkBwdArgs& a, int dtype, int dk, int dv, int stages, hipStream_t s) {
  // bf16: the chunk-map part through the UT form on the matrix cores
  ChunkBwdArgs b = a;
  b.map_ut = dtype == 1;
  return dtype == 1 ? launch_chunk_bwd_d<bf16>(b, dk, dv, stages, s) : launch_chunk_bwd_d<float>(b, dk, dv, stages, s);
}

}  // namespace hla
