// Backward of the Gated DeltaNet-2 per-chunk work: the routed outputs of a chunk from its
// start state, and the chunk's exact affine map.
//
// [GDN2] the Gated DeltaNet-2 abstract: per key channel decay a_t, a channel-wise erase gate
// b_t on the key side and a channel-wise write gate w_t on the value side.  With the math
// state S [dv, dk] a token does S' = S diag(a_t), S = S' - (S' k_t)(b_t o k_t)^T +
// (w_t o v_t) k_t^T and o_t = S q_t (the formula this library takes; the pages print none).
// Every column x of the stored state M = S^T [dk, dv] follows it on its own:
//     x' = a_t o x,   p = k_t . x',   x <- x' + k_t o (u - b_t p),
// with u = w_t[col] v_t[col] for a state column, and o_t[col] = q_t . x after the token.
// The chunk map M_end = At M_start + Bc is the same recurrence on dk + dv columns: the
// columns of At start at the identity and take no write (u = 0), those of Bc start at zero.
// The reverse of one token, with dx = dL/dx after it (plus q_t dO_t[col] for outputs):
//     du = k_t . dx,   dp = -(b_t o k_t) . dx,
//     dv_t[col] += w_t[col] du,   dw_t[col] += v_t[col] du,
//     dk_t += dx o (u - b_t p) + dp x',   db_t += -p k_t o dx,
//     dx' = dx + dp k_t,   da_t += dx' o x,   dq_t += dO_t[col] x_after,   dx <- a_t o dx'.
// dk, da, db and dq are sums over every column; dv_t[col] and dw_t[col] come from one.
//
// Layout: one workgroup per (b, h, chunk, block of 32 columns, 16 for float32 inputs, whose
// keys and queries take twice the LDS); a thread holds 8 rows of one
// column, the column's dk / 8 threads adjacent lanes (a dot product is a sum over 8 rows
// plus log2(dk / 8) DPP lane moves).  A forward pass keeps the state in front of every
// 8-token block in registers, and each block is replayed from its checkpoint before it is
// reversed.  The column sums run through DPP row moves and permlane swaps inside a wave and
// through LDS across waves, every second token; each workgroup writes its own partial sums,
// which the finalize pass adds in a fixed order (no atomics: deterministic).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {
constexpr int kRows = 8;  // rows per thread
constexpr int kTB = 8;    // tokens per checkpoint block
constexpr int kKF = 2;    // tokens per flush of the column sums
}  // namespace

template <class T, int DK>
constexpr int gdn2_bwd_threads() {
  return gdn2_bwd_cols(sizeof(T) == 2 ? 1 : 0) * (DK / kRows);
}

template <class T, int DK, int DV, bool OUT>
__global__ __launch_bounds__((gdn2_bwd_threads<T, DK>())) void gdn2_chunk_bwd_kernel(Gdn2BwdArgs a) {
  constexpr int C = kChunk, R = kRows, RG = DK / R, NCOL = gdn2_bwd_cols(sizeof(T) == 2 ? 1 : 0);
  constexpr int NTH = NCOL * RG, NWV = NTH / 64;
  constexpr int NB_OUT = DV / NCOL, NB_MAP = (DK + DV) / NCOL, NB = OUT ? NB_OUT : NB_MAP, NB_ALL = NB_OUT + NB_MAP;
  constexpr int NV = OUT ? 4 : 3;  // column sums per token: dk, da, db (, dq)
  static_assert(RG == 8 || RG == 16, "dk of 64 or 128");
  __shared__ __attribute__((aligned(16))) T s_k[C][DK];
  __shared__ __attribute__((aligned(16))) T s_q[OUT ? C : 1][DK];
  __shared__ __attribute__((aligned(16))) float s_a[C][DK];
  __shared__ __attribute__((aligned(16))) float s_b[C][DK];
  __shared__ float s_v[C][NCOL], s_w[C][NCOL];
  __shared__ float s_do[OUT ? C : 1][NCOL];
  __shared__ float s_red[kKF][NWV][NV][DK];

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
  const int r0 = rg * R;
  // this thread's column: a state column (outputs), or a column of [At | Bc] (maps)
  const int colall = cb * NCOL + cl;
  const bool isP = !OUT && colall < DK;
  const bool writes = !isP;
  const int vcol = OUT ? colall : colall - DK;  // column of v / Bc (when writes)
  const int blk = OUT ? cb : NB_OUT + cb;       // partial-sum slot of this workgroup

  // ---- stage the chunk's tokens; past the end: k = q = 0, a = 1, b = 0, v = w = dO = 0,
  // exact identity steps both ways (their partial sums land in slots never read)
  const T* kg = reinterpret_cast<const T*>(a.k);
  const T* qg = reinterpret_cast<const T*>(a.q);
  const T* vg = reinterpret_cast<const T*>(a.v);
  for (int i = tid; i < C * DK; i += NTH) {
    const int t = i / DK, r = i % DK;
    const int64_t row = row0 + (int64_t)t * a.H;
    const bool in = t < n;
    s_k[t][r] = in ? kg[row * DK + r] : (T)0.f;
    if constexpr (OUT) s_q[t][r] = in ? qg[row * DK + r] : (T)0.f;
    s_a[t][r] = in ? a.ga[row * DK + r] : 1.f;
    s_b[t][r] = in ? a.gb[row * DK + r] : 0.f;
  }
  for (int i = tid; i < C * NCOL; i += NTH) {
    const int t = i / NCOL, cc = i % NCOL;
    const int64_t row = row0 + (int64_t)t * a.H;
    const int col = cb * NCOL + cc;
    const bool w = t < n && (OUT || col >= DK);
    const int vc = OUT ? col : col - DK;
    s_v[t][cc] = w ? to_f<T>(vg[row * DV + vc]) : 0.f;
    s_w[t][cc] = w ? a.gw[row * DV + vc] : 0.f;
    if constexpr (OUT) s_do[t][cc] = t < n ? a.dO[((b * a.T + t0 + t) * a.H + h) * DV + vc] : 0.f;
  }
  __syncthreads();

  auto load_rows = [&](int t, float (&kk)[R], float (&aa)[R], float (&bb)[R]) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      kk[i] = to_f<T>(s_k[t][r0 + i]);
      aa[i] = s_a[t][r0 + i];
      bb[i] = s_b[t][r0 + i];
    }
  };
  // x <- x' + k o (u - b p) with x' = a o x and p = k . x'; returns p
  auto step = [&](int t, float* xx) {
    float kk[R], aa[R], bb[R];
    load_rows(t, kk, aa, bb);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      xx[i] *= aa[i];
      s = fmaf(kk[i], xx[i], s);
    }
    const float p = group_sum<RG>(s);  // the column's RG threads are one aligned lane group
    const float u = s_w[t][cl] * s_v[t][cl];
#pragma unroll
    for (int i = 0; i < R; ++i) xx[i] = fmaf(kk[i], fmaf(-bb[i], p, u), xx[i]);
    return p;
  };

  // ---- forward, keeping the state in front of every 8-token block
  float x[R];
  if constexpr (OUT) {
    const float* M0 = a.chunk_init + ((bh * a.N + c) * (int64_t)DK) * DV;
#pragma unroll
    for (int i = 0; i < R; ++i) x[i] = M0[(int64_t)(r0 + i) * DV + colall];
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) x[i] = (isP && r0 + i == colall) ? 1.f : 0.f;
  }
  float ck[C / kTB][R];
#pragma unroll
  for (int s = 0; s < C / kTB; ++s) {
#pragma unroll
    for (int i = 0; i < R; ++i) ck[s][i] = x[i];
#pragma unroll
    for (int u = 0; u < kTB; ++u) step(s * kTB + u, x);
  }

  // ---- reverse, one 8-token block at a time
  float dx[R];
  if constexpr (OUT) {
#pragma unroll
    for (int i = 0; i < R; ++i) dx[i] = 0.f;
  } else {
    const int64_t cc = bh * a.N + c;
#pragma unroll
    for (int i = 0; i < R; ++i)
      dx[i] = isP ? a.dAt[(cc * DK + r0 + i) * DK + colall] : a.dBc[(cc * DK + r0 + i) * DV + vcol];
  }
  const int64_t vbase = ((bh * a.N + c) * 2 + (OUT ? 0 : 1)) * (int64_t)C * DV;
  const int64_t slot = ((bh * a.N + c) * NB_ALL + blk) * (int64_t)C;
  const int64_t qslot = ((bh * a.N + c) * NB_OUT + cb) * (int64_t)C;
  const int nblk = (n + kTB - 1) / kTB;
  for (int s = nblk - 1; s >= 0; --s) {
    const int tb = s * kTB;
    float xs[kTB][R], pv[kTB];
    // the block's checkpoint, picked with compile-time register indices
#pragma unroll
    for (int ss = 0; ss < C / kTB; ++ss)
#pragma unroll
      for (int i = 0; i < R; ++i) x[i] = ss == s ? ck[ss][i] : x[i];
#pragma unroll
    for (int u = 0; u < kTB; ++u) {
#pragma unroll
      for (int i = 0; i < R; ++i) xs[u][i] = x[i];
      pv[u] = step(tb + u, x);
    }
#pragma unroll
    for (int u = kTB - 1; u >= 0; --u) {
      const int t = tb + u;
      float kk[R], aa[R], bb[R];
      load_rows(t, kk, aa, bb);
      float vec[NV][R];  // this column's parts of dk, da, db (, dq)
      if constexpr (OUT) {
        const float go = s_do[t][cl];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const float xa = u + 1 < kTB ? xs[u + 1 < kTB ? u + 1 : u][i] : x[i];  // state after token t
          dx[i] = fmaf(to_f<T>(s_q[t][r0 + i]), go, dx[i]);
          vec[NV - 1][i] = xa * go;
        }
      }
      float su = 0.f, se = 0.f;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        su = fmaf(kk[i], dx[i], su);
        se = fmaf(bb[i] * kk[i], dx[i], se);
      }
      const float du = group_sum<RG>(su), dp = -group_sum<RG>(se);
      const float p = pv[u], uu = s_w[t][cl] * s_v[t][cl];
      if (writes && rg == 0) {
        a.part_v[vbase + (int64_t)t * DV + vcol] = s_w[t][cl] * du;
        a.part_w[vbase + (int64_t)t * DV + vcol] = s_v[t][cl] * du;
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float xp = aa[i] * xs[u][i];
        vec[0][i] = fmaf(dx[i], fmaf(-bb[i], p, uu), dp * xp);  // dk
        vec[2][i] = -p * kk[i] * dx[i];                         // db
        const float dxp = fmaf(dp, kk[i], dx[i]);
        vec[1][i] = dxp * xs[u][i];                             // da
        dx[i] = aa[i] * dxp;
      }
      // sums over the wave's columns: with 8-lane row groups the two columns of a 16-lane
      // row are added first; rows_sum8 then leaves row rho with the totals of rows r0 + rho
      // and r0 + 4 + rho
      const int rho = lane >> 4;
#pragma unroll
      for (int m = 0; m < NV; ++m) {
        if constexpr (RG == 8) {
#pragma unroll
          for (int i = 0; i < R; ++i) vec[m][i] += dpp_f<0x128>(vec[m][i]);  // row_ror 8: the row's other column
        }
        float ra, rb;
        rows_sum8(vec[m], ra, rb);
        if (RG == 16 || ((lane >> 3) & 1) == 0) {
          s_red[u % kKF][wv][m][r0 + rho] = ra;
          s_red[u % kKF][wv][m][r0 + 4 + rho] = rb;
        }
      }
      if (u % kKF == 0) {
        // sums over the waves of tokens t .. t + kKF - 1, written as this workgroup's partials
        __syncthreads();
        for (int i = tid; i < kKF * NV * DK; i += NTH) {
          const int j = i / (NV * DK), m = (i / DK) % NV, e = i % DK;
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < NWV; ++w) sum += s_red[j][w][m][e];
          const int64_t tt = t + j;
          if (OUT && m == NV - 1)
            a.part_q[(qslot + tt) * DK + e] = sum;
          else
            (m == 0 ? a.part_k : m == 1 ? a.part_a : a.part_b)[(slot + tt) * DK + e] = sum;
        }
        __syncthreads();  // s_red is reused by the next tokens
      }
    }
  }
  if constexpr (OUT) {
    float* dM0 = a.dchunk_init + ((bh * a.N + c) * (int64_t)DK) * DV;
#pragma unroll
    for (int i = 0; i < R; ++i) dM0[(int64_t)(r0 + i) * DV + colall] = dx[i];
  }
}

// dq, dk, dv, da, db, dw of every token: the workgroups' partial sums in a fixed order, plus
// the router's parts (dqbar of the token's chunk divided by its token count, and the
// per-token key gradient) when given.  One thread per (b, t, h, row).
template <int DK, int DV, int NCOL>
__global__ __launch_bounds__(256) void gdn2_chunk_bwd_finalize_kernel(Gdn2BwdArgs a) {
  constexpr int C = kChunk, NB_OUT = DV / NCOL, NB_ALL = NB_OUT + (DK + DV) / NCOL;
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
  if (e < DK) {
    float sk = 0.f, sa = 0.f, sb = 0.f;
#pragma unroll
    for (int k = 0; k < NB_ALL; ++k) {
      if (k < NB_OUT ? !a.have_out : !a.have_map) continue;
      const int64_t o = ((base + k) * C + u) * DK + e;
      sk += __builtin_nontemporal_load(a.part_k + o);
      sa += __builtin_nontemporal_load(a.part_a + o);
      sb += __builtin_nontemporal_load(a.part_b + o);
    }
    if (a.dk_router) sk += a.dk_router[bth * DK + e];
    a.dk[bth * DK + e] = sk;
    a.da[bth * DK + e] = sa;
    a.db[bth * DK + e] = sb;
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
    float sv = 0.f, sw = 0.f;
    const int64_t o0 = ((bh * a.N + c) * 2 + 0) * (int64_t)C * DV + (int64_t)u * DV + e;
    const int64_t o1 = o0 + (int64_t)C * DV;
    if (a.have_out) {
      sv += a.part_v[o0];
      sw += a.part_w[o0];
    }
    if (a.have_map) {
      sv += a.part_v[o1];
      sw += a.part_w[o1];
    }
    a.dv[bth * DV + e] = sv;
    a.dw[bth * DV + e] = sw;
  }
}

template <class T, int DK, int DV>
static hipError_t launch_gdn2_bwd_t(const Gdn2BwdArgs& a, int stages, hipStream_t s) {
  const int64_t BHN = a.B * a.H * (int64_t)(a.c1 - a.c0);
  constexpr int NT = gdn2_bwd_threads<T, DK>(), NCOL = gdn2_bwd_cols(sizeof(T) == 2 ? 1 : 0);
  if ((stages & (kChunkBwdOut | kChunkBwdMap)) && BHN > 0) {
    TimedLaunch tl(HLA_KERNEL_BWD_CHUNK, s);
    if (stages & kChunkBwdOut)
      hipLaunchKernelGGL((gdn2_chunk_bwd_kernel<T, DK, DV, true>), dim3((unsigned)(BHN * (DV / NCOL))), dim3(NT), 0, s,
                         a);
    if (stages & kChunkBwdMap)
      hipLaunchKernelGGL((gdn2_chunk_bwd_kernel<T, DK, DV, false>), dim3((unsigned)(BHN * ((DK + DV) / NCOL))),
                         dim3(NT), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(stages & kChunkBwdFinalize)) return e;
  constexpr int W = DK > DV ? DK : DV;
  const int64_t total = a.B * a.T * a.H * W;
  hipLaunchKernelGGL((gdn2_chunk_bwd_finalize_kernel<DK, DV, NCOL>), dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_gdn2_bwd_d(const Gdn2BwdArgs& a, int dk, int dv, int stages, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_gdn2_bwd_t<T, 64, 64>(a, stages, s);
  if (dk == 64 && dv == 128) return launch_gdn2_bwd_t<T, 64, 128>(a, stages, s);
  if (dk == 128 && dv == 64) return launch_gdn2_bwd_t<T, 128, 64>(a, stages, s);
  return launch_gdn2_bwd_t<T, 128, 128>(a, stages, s);
}

hipError_t launch_gdn2_chunk_backward(const Gdn2BwdArgs& a, int dtype, int dk, int dv, int stages, hipStream_t s) {
  return dtype == 1 ? launch_gdn2_bwd_d<bf16>(a, dk, dv, stages, s) : launch_gdn2_bwd_d<float>(a, dk, dv, stages, s);
}

}  // namespace hla
