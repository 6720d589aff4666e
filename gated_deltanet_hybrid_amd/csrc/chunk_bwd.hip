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
  const int b0 = a.have_out ? 0 : NB_OUT, b1 = a.have_map ? NB_ALL : NB_OUT;
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
    if (stages & kChunkBwdMap)
      hipLaunchKernelGGL((chunk_bwd_kernel<T, DK, DV, false>), dim3((unsigned)(BHN * ((DK + DV) / 32))), dim3(NT), 0,
                         s, a);
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
  return dtype == 1 ? launch_chunk_bwd_d<bf16>(a, dk, dv, stages, s) : launch_chunk_bwd_d<float>(a, dk, dv, stages, s);
}

}  // namespace hla
