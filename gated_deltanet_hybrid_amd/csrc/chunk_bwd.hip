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
// The reverse of the per-piece work through the UT form, on the matrix cores (bf16 inputs,
// float32 arithmetic): chunk maps and chunk outputs.
//
// [HLA] Methodology paragraph 1: within a piece (tokens t, s; g the running sum of log alpha,
// gamma_t = exp g_t, Gamma_ts = exp(g_t - g_s), D_s = exp(g_63 - g_s))
//     A0 = strictly_lower((K K^T) o Gamma),  L = diag(beta) A0,  X = (I + L)^-1,
//     W = X diag(beta gamma) K,  U = X diag(beta) V,
//     maps:    At = gamma_63 I - K^T D W,  Bc = K^T D U,
//     outputs: E = U - W M_0,  P = (Q K^T) o Gamma (s <= t),  O = diag(gamma) Q M_0 + P E.
// Both parts end in gradients dU and dW, which a common tail takes back through the
// transform:
//     F = X^T dU,  G = X^T dW,  dV = diag(beta) F,  dK += diag(beta gamma) G,
//     T1 = X^T dX = F (diag(beta) V)^T + G (diag(beta gamma) K)^T,  H = -T1 X^T (s < t),
//     dK += H' K + H'^T K,  H'_ts = beta_t Gamma_ts H_ts,
//     dbeta_t = F_t . v_t + gamma_t G_t . k_t + sum_s H_ts A0_ts,
//     dg_t += beta_t gamma_t G_t . k_t + sum_s Psi_ts - sum_s Psi_st,  Psi_ts = beta_t H_ts A0_ts,
//     dlog alpha_s = sum_{t >= s} dg_t,  dalpha = dlog alpha / alpha.
// The chunk-map part first forms, from dAt and dBc,
//     dY = -K dAt,  dKB = K dBc,  dD_s = dY_s . W_s + dKB_s . U_s,  dW = D dY,  dU = D dKB,
//     dK = D (-W dAt^T + U dBc^T),
//     dg_t = -dD_t D_t (+ sum_s dD_s D_s + tr(dAt) gamma_63 at t = 63);
// the outputs part, from dO and the start state M_0,
//     dE = P^T dO,  dP = (dO E^T) o mask (s <= t),  dQ = diag(gamma) dO M_0^T + (dP o Gamma) K,
//     dK = (dP o Gamma)^T Q,  dM_0 = Q^T diag(gamma) dO - W^T dE,  dU = dE,  dW = -dE M_0^T,
//     dg_t = gamma_t q_t . (M_0 do_t) + sum_s PsiP_ts - sum_s PsiP_st,  PsiP_ts = dP_ts P_ts (s < t).
// One workgroup of 8 waves per (b, h, piece).  Every product is a 32 x 32 tile of
// v_mfma_f32_32x32x2_f32 (K K^T and Q K^T: bf16 products of the bf16 inputs), its operands
// read from LDS, or from global memory for dAt, dBc, dO, M_0 and q; wave w owns tile w of the
// 64 x dk and of the 64 x dv results.  Each workgroup writes its per-token sums into one
// partial-sum slot of its part.
namespace {
// The workgroup's LDS for the UT reverse, and the lane's coordinates.
template <int DK, int DV>
struct UtRev {
  static constexpr int C = kChunk, NT = 512;
  static constexpr int PX = C + 4;                // float32 pitch of the 64 x 64 matrices
  static constexpr int PK = DK + 8, PV = DV + 8;  // bf16 pitch of the k and v rows
  static constexpr int PW = DK + 4, PU = DV + 4;  // float32 pitch of W (dW, G) and U (E, dU, F)
  static constexpr int NKT = 2 * (DK / 32), NVT = 2 * (DV / 32);
  static_assert(NKT <= 8 && NVT <= 8, "one tile of each kind per wave");
  float* A0;        // [C][PX] lower: Gamma o K K^T; upper blocks: the inverse's scratch
  float* Xb;        // [C][PX] X
  float* Tb;        // [C][PX] P (outputs), dP o Gamma, T1, then H
  bf16* Ks;         // [C][PK]
  bf16* Vs;         // [C][PV]
  float* Wb;        // [C][PW] W, dW, G
  float* Ub;        // [C][PU] U (E), dU, F
  float* beta;      // [C] per token: beta, alpha, log2-unit g, gamma, D
  float* alpha;
  float* g2;
  float* gam;
  float* D;
  float (*red)[8];  // [C][8] per-row partial sums of the column tiles
  float (*row)[C];  // [4][C] sums of Psi by rows and by columns, of H o A0, and the part's dg
  int tid, lane, hh, c32, w;
  int tk, ck, tv, cv;  // the wave's tiles (row block, column block) of 64 x dk and 64 x dv
  bool hk, hv;
  __device__ int tok(int r0, int e) const { return r0 + acc_row(e, hh); }
};

// Steps common to both parts: k and v rows (zero past the end), gates and decays, A0 (and P
// into Tb when asked, q rows from global memory), X, then W into Wb and U into Ub.
template <int DK, int DV, bool WANT_P>
__device__ __forceinline__ void ut_prologue(const UtRev<DK, DV>& L, const ChunkBwdArgs& a, int64_t row0, int n) {
  using R = UtRev<DK, DV>;
  constexpr int C = R::C, NT = R::NT, PX = R::PX, PK = R::PK, PV = R::PV, PW = R::PW, PU = R::PU;
  const int tid = L.tid, lane = L.lane, hh = L.hh, c32 = L.c32, w = L.w;
  const bf16* kg = reinterpret_cast<const bf16*>(a.k);
  const bf16* vg = reinterpret_cast<const bf16*>(a.v);
  for (int i = tid; i < C * (DK / 8); i += NT) {
    const int t = i / (DK / 8), u = i % (DK / 8);
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (t < n) x = *reinterpret_cast<const uint4*>(kg + (row0 + (int64_t)t * a.H) * DK + u * 8);
    *reinterpret_cast<uint4*>(L.Ks + t * PK + u * 8) = x;
  }
  for (int i = tid; i < C * (DV / 8); i += NT) {
    const int t = i / (DV / 8), u = i % (DV / 8);
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (t < n) x = *reinterpret_cast<const uint4*>(vg + (row0 + (int64_t)t * a.H) * DV + u * 8);
    *reinterpret_cast<uint4*>(L.Vs + t * PV + u * 8) = x;
  }
  for (int i = tid; i < C * PX; i += NT) L.Xb[i] = 0.f;
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
    L.beta[tid] = be;
    L.alpha[tid] = al;
    L.g2[tid] = x * 1.4426950408889634f;
    L.gam[tid] = expf(x);
    L.D[tid] = expf(x_end - x);
  }
  __syncthreads();

  // A0 tiles (0,0), (1,0), (1,1) on waves 0-2, zero tile (0,1) on wave 3; P the same on
  // waves 4-6 and 7 (with the diagonal), from q rows read straight from global memory
  if (w < 3 || (WANT_P && w >= 4 && w < 7)) {
    const int j = w < 3 ? w : w - 4;
    const int tm = j == 0 ? 0 : 1, tn = j == 2 ? 1 : 0;
    f32x16 acc = zero16();
    if (w < 3) {
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks)
        acc = Mma<bf16>::mma(Mma<bf16>::load_plain(L.Ks + (tm * 32 + c32) * PK, ks, hh),
                             Mma<bf16>::load_plain(L.Ks + (tn * 32 + c32) * PK, ks, hh), acc);
    } else {
      const int tq = tm * 32 + c32;
      const bf16* qr = reinterpret_cast<const bf16*>(a.q) + (row0 + (int64_t)(tq < n ? tq : 0) * a.H) * DK;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) {
        bf16x8 qf = Mma<bf16>::load_plain(qr, ks, hh);
        if (tq >= n) qf = bf16x8{};
        acc = Mma<bf16>::mma(qf, Mma<bf16>::load_plain(L.Ks + (tn * 32 + c32) * PK, ks, hh), acc);
      }
    }
    float* dst = w < 3 ? L.A0 : L.Tb;
    const int s = tn * 32 + c32;
    const float gs = L.g2[s];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      const bool keep = w < 3 ? s < t : s <= t;
      dst[t * PX + s] = keep ? __builtin_amdgcn_exp2f(L.g2[t] - gs) * acc[e] : 0.f;
    }
  } else if (w == 3 || (WANT_P && w == 7)) {
    float* dst = w == 3 ? L.A0 : L.Tb;
    for (int i = lane; i < 32 * 32; i += 64) dst[(i >> 5) * PX + 32 + (i & 31)] = 0.f;
  }
  __syncthreads();

  // X = (I + L)^-1 with L = diag(beta) A0, blocked by 16: the diagonal blocks by
  // substitution, then the blocks below them by sub-diagonal from Z = -X_ii L_im (kept in
  // A0's unused blocks above the diagonal)
  if (tid < 64) {
    const int bi = tid >> 4, cl = tid & 15, base = bi * 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cl) ? 1.f : 0.f;
      const float br = L.beta[base + r];
#pragma unroll
      for (int q2 = 0; q2 < r; ++q2) s -= br * L.A0[(base + r) * PX + base + q2] * x[q2];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) L.Xb[(base + r) * PX + base + cl] = x[r];
  }
  __syncthreads();
  for (int e = tid; e < 6 * 256; e += NT) {
    const int bz = e >> 8, r = (e >> 4) & 15, cl = e & 15;
    const int i = bz < 1 ? 1 : (bz < 3 ? 2 : 3), m = bz - i * (i - 1) / 2;
    float z = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 16; ++q2)
      z -= L.Xb[(i * 16 + r) * PX + i * 16 + q2] * L.beta[i * 16 + q2] * L.A0[(i * 16 + q2) * PX + m * 16 + cl];
    L.A0[(m * 16 + r) * PX + i * 16 + cl] = z;
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    for (int e = tid; e < (4 - d) * 256; e += NT) {
      const int k = e >> 8, i = k + d, r = (e >> 4) & 15, cl = e & 15;
      float x = 0.f;
      for (int m = k; m < i; ++m)
#pragma unroll
        for (int q2 = 0; q2 < 16; ++q2)
          x += L.A0[(m * 16 + r) * PX + i * 16 + q2] * L.Xb[(m * 16 + q2) * PX + k * 16 + cl];
      L.Xb[(i * 16 + r) * PX + k * 16 + cl] = x;
    }
    __syncthreads();
  }

  // W = X diag(beta gamma) K and U = X diag(beta) V
  if (L.hk) {
    const int rk0 = L.tk * 32;
    const float* xr = L.Xb + (rk0 + c32) * PX;
    const bf16* kc = L.Ks + L.ck * 32 + c32;
    const f32x16 acc = mm32<C>(zero16(), hh, [&](int k) { return xr[k] * L.beta[k] * L.gam[k]; },
                               [&](int k) { return (float)kc[k * PK]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Wb[L.tok(rk0, e) * PW + L.ck * 32 + c32] = acc[e];
  }
  if (L.hv) {
    const int rv0 = L.tv * 32;
    const float* xr = L.Xb + (rv0 + c32) * PX;
    const bf16* vc = L.Vs + L.cv * 32 + c32;
    const f32x16 acc = mm32<C>(zero16(), hh, [&](int k) { return xr[k] * L.beta[k]; },
                               [&](int k) { return (float)vc[k * PV]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Ub[L.tok(rv0, e) * PU + L.cv * 32 + c32] = acc[e];
  }
  __syncthreads();
}

// The common tail, from dU in Ub and dW in Wb, the part's own dK tile `dk_part` (the wave's
// 64 x dk tile) and its dg in row[3]: writes dK, dV, dbeta and dalpha of the piece's tokens
// t < n at pk + t * dk, pv + t * dv and ps + 2 t.
template <int DK, int DV>
__device__ __forceinline__ void ut_tail(const UtRev<DK, DV>& L, int n, const f32x16& dk_part, float* pk, float* pv,
                                        float* ps) {
  using R = UtRev<DK, DV>;
  constexpr int C = R::C, PX = R::PX, PK = R::PK, PV = R::PV, PW = R::PW, PU = R::PU;
  const int tid = L.tid, lane = L.lane, hh = L.hh, c32 = L.c32, w = L.w;
  const int rk0 = L.tk * 32, rv0 = L.tv * 32, ck = L.ck, cv = L.cv;

  // G = X^T dW, F = X^T dU
  f32x16 gt = zero16(), ft = zero16();
  if (L.hk) {
    const float* xc = L.Xb + rk0 + c32;
    const float* dw = L.Wb + ck * 32 + c32;
    gt = mm32<C>(gt, hh, [&](int k) { return xc[k * PX]; }, [&](int k) { return dw[k * PW]; });
  }
  if (L.hv) {
    const float* xc = L.Xb + rv0 + c32;
    const float* du = L.Ub + cv * 32 + c32;
    ft = mm32<C>(ft, hh, [&](int k) { return xc[k * PX]; }, [&](int k) { return du[k * PU]; });
  }
  __syncthreads();  // dW, dU are dead
  if (L.hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Wb[L.tok(rk0, e) * PW + ck * 32 + c32] = gt[e];
  }
  if (L.hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Ub[L.tok(rv0, e) * PU + cv * 32 + c32] = ft[e];
  }
  __syncthreads();

  // T1 = F (diag(beta) V)^T + G (diag(beta gamma) K)^T: tile (tm, tn) on wave tm + 2 tn
  if (w < 4) {
    const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
    const float* fr = L.Ub + (tm * 32 + c32) * PU;
    const float* gr = L.Wb + (tm * 32 + c32) * PW;
    const bf16* vr = L.Vs + s * PV;
    const bf16* kr = L.Ks + s * PK;
    const f32x16 a1 = mm32<DV>(zero16(), hh, [&](int k) { return fr[k]; }, [&](int k) { return (float)vr[k]; });
    const f32x16 a2 = mm32<DK>(zero16(), hh, [&](int k) { return gr[k]; }, [&](int k) { return (float)kr[k]; });
    const float bs = L.beta[s], gs = L.gam[s];
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Tb[(tm * 32 + acc_row(e, hh)) * PX + s] = bs * (a1[e] + gs * a2[e]);
  }
  __syncthreads();
  // H = -T1 X^T, kept below the diagonal
  f32x16 ht = zero16();
  if (w < 4) {
    const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
    const float* tr = L.Tb + (tm * 32 + c32) * PX;
    const float* xr = L.Xb + s * PX;
    ht = mm32<C>(ht, hh, [&](int k) { return tr[k]; }, [&](int k) { return xr[k]; });
  }
  __syncthreads();
  if (w < 4) {
    const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      L.Tb[t * PX + s] = s < t ? -ht[e] : 0.f;
    }
  }
  __syncthreads();

  // dK = dk_part + diag(beta gamma) G + H' K + H'^T K;  dV = diag(beta) F
  if (L.hk) {
    const int t = rk0 + c32;
    const float* hr = L.Tb + t * PX;  // row t of H
    const float* hc = L.Tb + t;       // column t of H
    const bf16* kc = L.Ks + ck * 32 + c32;
    const float bt = L.beta[t], g2t = L.g2[t];
    f32x16 acc = mm32<C>(zero16(), hh,
                         [&](int k) { return k < t ? hr[k] * bt * __builtin_amdgcn_exp2f(g2t - L.g2[k]) : 0.f; },
                         [&](int k) { return (float)kc[k * PK]; });
    acc = mm32<C>(acc, hh,
                  [&](int k) { return k > t ? hc[k * PX] * L.beta[k] * __builtin_amdgcn_exp2f(L.g2[k] - g2t) : 0.f; },
                  [&](int k) { return (float)kc[k * PK]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = L.tok(rk0, e);
      if (te < n) pk[(int64_t)te * DK + ck * 32 + c32] = acc[e] + dk_part[e] + L.beta[te] * L.gam[te] * gt[e];
    }
  }
  if (L.hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = L.tok(rv0, e);
      if (te < n) pv[(int64_t)te * DV + cv * 32 + c32] = L.beta[te] * ft[e];
    }
  }
  // per-token dots F_t . v_t and G_t . k_t (by tiles); the sums of Psi and of H o A0
  if (L.hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = L.tok(rv0, e);
      const float p = lane_group_sum<32>(ft[e] * (float)L.Vs[te * PV + cv * 32 + c32]);
      if (c32 == 0) L.red[te][cv] = p;
    }
  }
  if (L.hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = L.tok(rk0, e);
      const float p = lane_group_sum<32>(gt[e] * (float)L.Ks[te * PK + ck * 32 + c32]);
      if (c32 == 0) L.red[te][4 + ck] = p;
    }
  }
  if (tid < C) {
    const int t = tid;
    float ha = 0.f;
    for (int s = 0; s < t; ++s) ha += L.Tb[t * PX + s] * L.A0[t * PX + s];
    L.row[0][t] = L.beta[t] * ha;
    L.row[2][t] = ha;
  } else if (tid < 2 * C) {
    const int s = tid - C;
    float pc = 0.f;
    for (int t = s + 1; t < C; ++t) pc += L.beta[t] * L.Tb[t * PX + s] * L.A0[t * PX + s];
    L.row[1][s] = pc;
  }
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    float fv = 0.f, gk = 0.f;
#pragma unroll
    for (int j = 0; j < DV / 32; ++j) fv += L.red[t][j];
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) gk += L.red[t][4 + j];
    const float be = L.beta[t], ga = L.gam[t];
    const float dbeta = fv + ga * gk + L.row[2][t];
    // dlog alpha_t = sum_{u >= t} dg_u: inclusive suffix sum over the wave
    float x = be * ga * gk + L.row[0][t] - L.row[1][t] + L.row[3][t];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (lane + off < 64) x += y;
    }
    if (t < n) {
      ps[2 * t] = dbeta;
      ps[2 * t + 1] = x / fmaxf(L.alpha[t], 1.17549435e-38f);
    }
  }
}
}  // namespace

#define HLA_UT_REV_LDS(DK, DV)                                                                  \
  using R = UtRev<DK, DV>;                                                                      \
  __shared__ __attribute__((aligned(16))) float s_A0[R::C * R::PX];                             \
  __shared__ __attribute__((aligned(16))) float s_X[R::C * R::PX];                              \
  __shared__ __attribute__((aligned(16))) float s_T[R::C * R::PX];                              \
  __shared__ __attribute__((aligned(16))) bf16 s_K[R::C * R::PK];                               \
  __shared__ __attribute__((aligned(16))) bf16 s_V[R::C * R::PV];                               \
  __shared__ __attribute__((aligned(16))) float s_W[R::C * R::PW];                              \
  __shared__ __attribute__((aligned(16))) float s_U[R::C * R::PU];                              \
  __shared__ float s_vec[5][R::C];                                                              \
  __shared__ float s_red[R::C][8];                                                              \
  __shared__ float s_row[4][R::C];                                                              \
  R L;                                                                                          \
  L.A0 = s_A0; L.Xb = s_X; L.Tb = s_T; L.Ks = s_K; L.Vs = s_V; L.Wb = s_W; L.Ub = s_U;          \
  L.beta = s_vec[0]; L.alpha = s_vec[1]; L.g2 = s_vec[2]; L.gam = s_vec[3]; L.D = s_vec[4];     \
  L.red = s_red; L.row = s_row;                                                                 \
  L.tid = threadIdx.x; L.lane = L.tid & 63; L.hh = L.lane >> 5; L.c32 = L.lane & 31;            \
  L.w = __builtin_amdgcn_readfirstlane(L.tid >> 6);                                             \
  L.tk = L.w & 1; L.ck = L.w >> 1; L.tv = L.w & 1; L.cv = L.w >> 1;                             \
  L.hk = L.w < R::NKT; L.hv = L.w < R::NVT

template <int DK, int DV>
__global__ __launch_bounds__(512, 1) void chunk_bwd_map_ut_kernel(ChunkBwdArgs a) {
  HLA_UT_REV_LDS(DK, DV);
  __shared__ float s_tr;
  constexpr int C = R::C, PW = R::PW, PU = R::PU;
  constexpr int NB_OUT = DV / 32, NB_ALL = NB_OUT + (DK + DV) / 32;
  const int tid = L.tid, lane = L.lane, hh = L.hh, c32 = L.c32, w = L.w;
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
  if (w == 0) {  // tr(dAt)
    float tr = 0.f;
    for (int i = lane; i < DK; i += 64) tr += dAt[(int64_t)i * DK + i];
    tr = wave_sum(tr);
    if (lane == 0) s_tr = tr;
  }
  ut_prologue<DK, DV, false>(L, a, row0, n);
  const int rk0 = L.tk * 32, rv0 = L.tv * 32, ck = L.ck, cv = L.cv;

  // dY = -K dAt, dKB = K dBc, dK_ab = D (-W dAt^T + U dBc^T), dD
  f32x16 dkab = zero16(), dy = zero16(), dkb = zero16();
  if (L.hk) {
    const bf16* kr = L.Ks + (rk0 + c32) * R::PK;
    const float* wr = L.Wb + (rk0 + c32) * PW;
    const float* ur = L.Ub + (rk0 + c32) * PU;
    const int nc = ck * 32 + c32;
    dy = mm32<DK>(dy, hh, [&](int k) { return -(float)kr[k]; }, [&](int k) { return dAt[(int64_t)k * DK + nc]; });
    dkab = mm32<DK>(dkab, hh, [&](int k) { return -wr[k]; }, [&](int k) { return dAt[(int64_t)nc * DK + k]; });
    dkab = mm32<DV>(dkab, hh, [&](int k) { return ur[k]; }, [&](int k) { return dBc[(int64_t)nc * DV + k]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) dkab[e] *= L.D[L.tok(rk0, e)];
  }
  if (L.hv) {
    const bf16* kr = L.Ks + (rv0 + c32) * R::PK;
    const int nc = cv * 32 + c32;
    dkb = mm32<DK>(dkb, hh, [&](int k) { return (float)kr[k]; }, [&](int k) { return dBc[(int64_t)k * DV + nc]; });
  }
  // dD_t = dY_t . W_t + dKB_t . U_t: each tile's 32 columns summed over the lanes of a half
  if (L.hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = lane_group_sum<32>(dy[e] * L.Wb[L.tok(rk0, e) * PW + ck * 32 + c32]);
      if (c32 == 0) L.red[L.tok(rk0, e)][ck] = p;
    }
  }
  if (L.hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = lane_group_sum<32>(dkb[e] * L.Ub[L.tok(rv0, e) * PU + cv * 32 + c32]);
      if (c32 == 0) L.red[L.tok(rv0, e)][DK / 32 + cv] = p;
    }
  }
  __syncthreads();  // W, U and the partial sums are complete
  // the map part's dg: -dD_t D_t, plus sum_s dD_s D_s + tr(dAt) gamma_63 at t = 63
  if (tid < C) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < DK / 32 + DV / 32; ++j) s += L.red[tid][j];
    const float dd = s * L.D[tid];
    const float ddsum = wave_sum(dd);
    L.row[3][tid] = tid == C - 1 ? ddsum + s_tr * L.gam[tid] - dd : -dd;
  }
  if (L.hk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Wb[L.tok(rk0, e) * PW + ck * 32 + c32] = L.D[L.tok(rk0, e)] * dy[e];  // dW
  }
  if (L.hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Ub[L.tok(rv0, e) * PU + cv * 32 + c32] = L.D[L.tok(rv0, e)] * dkb[e];  // dU
  }
  __syncthreads();
  const int64_t pslot = (cc * NB_ALL + NB_OUT) * (int64_t)C;  // first chunk-map slot
  ut_tail<DK, DV>(L, n, dkab, a.part_k + pslot * DK, a.part_v + (cc * 2 + 1) * (int64_t)C * DV, a.part_s + pslot * 2);
}

template <int DK, int DV>
__global__ __launch_bounds__(512, 1) void chunk_bwd_out_ut_kernel(ChunkBwdArgs a) {
  HLA_UT_REV_LDS(DK, DV);
  constexpr int C = R::C, PX = R::PX, PW = R::PW, PU = R::PU;
  constexpr int NB_OUT = DV / 32, NB_ALL = NB_OUT + (DK + DV) / 32;
  const int tid = L.tid, hh = L.hh, c32 = L.c32, w = L.w;
  const int64_t id = blockIdx.x;
  const int c = a.c0 + (int)(id % (a.c1 - a.c0));
  const int64_t bh = id / (a.c1 - a.c0);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)c * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
  const int64_t cc = bh * a.N + c;
  const float* M0 = a.chunk_init + cc * (int64_t)DK * DV;
  // token t's rows of dO and q (t < n; callers clamp t)
  const int64_t ldo = a.H * (int64_t)DV, ldq = a.H * (int64_t)DK;
  const float* dOg = a.dO + ((b * a.T + t0) * a.H + h) * DV;
  const bf16* qg = reinterpret_cast<const bf16*>(a.q) + row0 * DK;
  auto dO_at = [&](int t, int v) { return t < n ? dOg[(int64_t)(t < n ? t : 0) * ldo + v] : 0.f; };
  auto q_at = [&](int t, int i) { return t < n ? (float)qg[(int64_t)(t < n ? t : 0) * ldq + i] : 0.f; };

  ut_prologue<DK, DV, true>(L, a, row0, n);  // P in Tb, W in Wb, U in Ub
  const int rk0 = L.tk * 32, rv0 = L.tv * 32, ck = L.ck, cv = L.cv;

  // E = U - W M0, in place (each wave updates its own tile)
  if (L.hv) {
    const float* wr = L.Wb + (rv0 + c32) * PW;
    const float* mc = M0 + cv * 32 + c32;
    const f32x16 acc = mm32<DK>(zero16(), hh, [&](int k) { return wr[k]; }, [&](int k) { return mc[(int64_t)k * DV]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Ub[L.tok(rv0, e) * PU + cv * 32 + c32] -= acc[e];
  }
  __syncthreads();

  // dE = P^T dO;  dP = (dO E^T) o mask (s <= t) on waves 0-2 (tiles (0,0), (1,0), (1,1));
  // the sums of PsiP_ts = dP_ts P_ts (s < t) by rows (red[t][tn]) and by columns (red[s][2 + tm])
  f32x16 de = zero16(), dp = zero16();
  if (L.hv) {
    const float* pc = L.Tb + rv0 + c32;  // column s of P
    de = mm32<C>(de, hh, [&](int k) { return pc[k * PX]; }, [&](int k) { return dO_at(k, cv * 32 + c32); });
  }
  if (w < 3) {
    const int tm = w == 0 ? 0 : 1, tn = w == 2 ? 1 : 0, s = tn * 32 + c32;
    const int tr = tm * 32 + c32;
    const float* er = L.Ub + s * PU;
    dp = mm32<DV>(dp, hh, [&](int k) { return dO_at(tr, k); }, [&](int k) { return er[k]; });
    float colp = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      if (s > t) dp[e] = 0.f;
      const float psi = s < t ? dp[e] * L.Tb[t * PX + s] : 0.f;
      colp += psi;
      const float rp = lane_group_sum<32>(psi);
      if (c32 == 0) L.red[t][tn] = rp;
    }
    colp += __shfl_xor(colp, 32, 64);
    if (hh == 0) L.red[s][2 + tm] = colp;
  } else if (w == 3) {  // the sums no tile gives
    const int t = L.lane;
    if (t < 32) L.red[t][1] = 0.f;
    else L.red[t][2] = 0.f;
  }
  __syncthreads();  // P and E are dead
  if (L.hv) {
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Ub[L.tok(rv0, e) * PU + cv * 32 + c32] = de[e];  // dE = dU
  }
  if (w < 3) {  // dP o Gamma (tile (0,1) stays zero)
    const int tm = w == 0 ? 0 : 1, tn = w == 2 ? 1 : 0, s = tn * 32 + c32;
    const float gs = L.g2[s];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh);
      L.Tb[t * PX + s] = __builtin_amdgcn_exp2f(L.g2[t] - gs) * dp[e];
    }
  }
  if (tid < C) L.row[3][tid] = L.red[tid][0] + L.red[tid][1] - L.red[tid][2] - L.red[tid][3];
  __syncthreads();

  // dQ = diag(gamma) dO M0^T + (dP o Gamma) K, with dgamma_t = q_t . (dO M0^T)_t;
  // dK_P = (dP o Gamma)^T Q
  f32x16 dkp = zero16();
  if (L.hk) {
    const int tr = rk0 + c32, ic = ck * 32 + c32;
    const float* mr = M0 + (int64_t)ic * DV;  // row i of M0
    f32x16 q0 = mm32<DV>(zero16(), hh, [&](int k) { return dO_at(tr, k); }, [&](int k) { return mr[k]; });
    const float* pr = L.Tb + tr * PX;
    const bf16* kc = L.Ks + ic;
    const f32x16 q1 = mm32<C>(zero16(), hh, [&](int k) { return pr[k]; }, [&](int k) { return (float)kc[k * R::PK]; });
    const float* pc = L.Tb + tr;  // column s = tr of dP o Gamma
    dkp = mm32<C>(dkp, hh, [&](int k) { return pc[k * PX]; }, [&](int k) { return q_at(k, ic); });
    float* pq = a.part_q + cc * NB_OUT * (int64_t)C * DK + ic;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int te = L.tok(rk0, e);
      const float dg = lane_group_sum<32>(q0[e] * q_at(te, ic));
      if (c32 == 0) L.red[te][4 + ck] = dg;
      if (te < n) pq[(int64_t)te * DK] = L.gam[te] * q0[e] + q1[e];
    }
  }
  // dM0 = Q^T diag(gamma) dO - W^T dE, tiles (ti, tj) of dk x dv
  {
    constexpr int NMI = DK / 32, NM = NMI * (DV / 32);
    float* dM0 = a.dchunk_init + cc * (int64_t)DK * DV;
    for (int j = w; j < NM; j += 8) {
      const int ic = (j % NMI) * 32 + c32, vc = (j / NMI) * 32 + c32;
      f32x16 acc = mm32<C>(zero16(), hh, [&](int k) { return q_at(k, ic) * L.gam[k]; },
                           [&](int k) { return dO_at(k, vc); });
      acc = mm32<C>(acc, hh, [&](int k) { return -L.Wb[k * PW + ic]; }, [&](int k) { return L.Ub[k * PU + vc]; });
#pragma unroll
      for (int e = 0; e < 16; ++e) dM0[(int64_t)((j % NMI) * 32 + acc_row(e, hh)) * DV + vc] = acc[e];
    }
  }
  __syncthreads();  // W is dead
  // dW = -dE M0^T; the part's dg: gamma_t dgamma_t + sum_s PsiP_ts - sum_s PsiP_st
  if (L.hk) {
    const float* er = L.Ub + (rk0 + c32) * PU;
    const float* mr = M0 + (int64_t)(ck * 32 + c32) * DV;
    const f32x16 acc = mm32<DV>(zero16(), hh, [&](int k) { return -er[k]; }, [&](int k) { return mr[k]; });
#pragma unroll
    for (int e = 0; e < 16; ++e) L.Wb[L.tok(rk0, e) * PW + ck * 32 + c32] = acc[e];
  }
  if (tid < C) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) s += L.red[tid][4 + j];
    L.row[3][tid] += L.gam[tid] * s;
  }
  __syncthreads();
  const int64_t pslot = cc * NB_ALL * (int64_t)C;  // first outputs slot
  ut_tail<DK, DV>(L, n, dkp, a.part_k + pslot * DK, a.part_v + cc * 2 * (int64_t)C * DV, a.part_s + pslot * 2);
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
  // the slots each part wrote: one per piece through the UT form, else one per column block
  auto used = [&](int k) {
    return k < NB_OUT ? a.have_out && (!a.ut || k == 0) : a.have_map && (!a.ut || k == NB_OUT);
  };
  // every partial sum is read once, here: non-temporal loads, all of a thread's in flight
  if (e < DK) {
    float sk = 0.f;
#pragma unroll
    for (int k = 0; k < NB_ALL; ++k)
      if (used(k)) sk += __builtin_nontemporal_load(a.part_k + ((base + k) * C + u) * DK + e);
    if (a.dk_router) sk += a.dk_router[bth * DK + e];
    a.dk[bth * DK + e] = sk;
    float sq = 0.f;
    if (a.have_out) {
      const int64_t qb = (bh * a.N + c) * NB_OUT;
#pragma unroll
      for (int k = 0; k < NB_OUT; ++k)
        if (!a.ut || k == 0) sq += __builtin_nontemporal_load(a.part_q + ((qb + k) * C + u) * DK + e);
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
    for (int k = 0; k < NB_ALL; ++k)
      if (used(k)) ss += a.part_s[((base + k) * C + u) * 2 + e];
    (e == 0 ? a.dbeta : a.dalpha)[bth] = ss;
  }
}

template <class T, int DK, int DV>
static hipError_t launch_chunk_bwd_t(const ChunkBwdArgs& a, int stages, hipStream_t s) {
  const int64_t BHN = a.B * a.H * (int64_t)(a.c1 - a.c0);
  constexpr int NT = chunk_bwd_threads<DK>();
  if ((stages & (kChunkBwdOut | kChunkBwdMap)) && BHN > 0) {
    TimedLaunch tl(HLA_KERNEL_BWD_CHUNK, s);
    if (stages & kChunkBwdOut) {
      if (a.ut)
        hipLaunchKernelGGL((chunk_bwd_out_ut_kernel<DK, DV>), dim3((unsigned)BHN), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((chunk_bwd_kernel<T, DK, DV, true>), dim3((unsigned)(BHN * (DV / 32))), dim3(NT), 0, s, a);
    }
    if (stages & kChunkBwdMap) {
      if (a.ut)
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
  // bf16: both parts through the UT form on the matrix cores
  ChunkBwdArgs b = a;
  b.ut = dtype == 1;
  return dtype == 1 ? launch_chunk_bwd_d<bf16>(b, dk, dv, stages, s) : launch_chunk_bwd_d<float>(b, dk, dv, stages, s);
}

}  // namespace hla
