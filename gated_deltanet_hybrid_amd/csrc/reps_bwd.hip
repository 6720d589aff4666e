// Backward of the learned chunk representatives (float32 matrix cores).
//
// [HLA] Methodology paragraph 2: inside a pooling window the keys X [n, dk] attend to one
// another, Q = X Wq^T, K = X Wk^T, V = X Wv^T, P = row-softmax(Q K^T / sqrt(dk)), O = P V;
// the rows of O are mean-pooled, m = (1/n) sum_t O_t = (1/n) sum_s c_s V_s with c_s the
// column sums of P, and projected, z = Wp m; with the router's query projection folded in
// the representative is r' = Wr^T z.  Given dr' for every representative row:
//     dz = Wr dr' (dr' without Wr),  dWr += z dr'^T,  dm = Wp^T dz,  dWp += dz m^T,
//     dO_t = dm / n,  dV_s = c_s dm / n,  dP_ts = e_s = V_s . dm / n (the same for every t),
//     dS_ts = P_ts (e_s - sum_s' P_ts' e_s'),  dQ = dS K / sqrt(dk),  dK = dS^T Q / sqrt(dk),
//     dX = dQ Wq + dK Wk + dV Wv,  dWq += dQ^T X,  dWk += dK^T X,  dWv += dV^T X.
// A window with no tokens has a constant zero row and passes nothing.
//
// Three kernels:
//   tile    one workgroup of 8 waves per 8 consecutive 64-token tiles of a (b, h) row
//           (windows divide 64, so none crosses a tile), one tile after another: the
//           projections, the window-block scores, dQ, dK, dX and the weight gradients are
//           32 x 32 tiles of v_mfma_f32_32x32x2_f32, the softmax and the per-window vectors
//           run on the VALU; dX goes straight to dk, dWq, dWk and dWv add up in registers
//           over the workgroup's tiles and go to its own slot, and each window's dz, m, z
//           and dr' go to the workspace;
//   outer   dWp = sum_w dz_w m_w^T and dWr = sum_w z_w dr'_w^T over chunks of 256 windows of
//           one (b, h), on the matrix cores, each chunk's part to its own slot;
//   reduce  the parts of every head (of every head, for shared weights) summed in a fixed
//           order: deterministic, no atomics.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

constexpr int kRepsBwdTiles = 8;     // 64-token tiles per workgroup of the tile kernel
constexpr int kRepsOuterRows = 256;  // windows per workgroup of the outer kernel

template <class T, int DK, int WN>
__global__ __launch_bounds__(512, 1) void reps_bwd_tile_kernel(RepsBwdArgs a) {
  constexpr int C = 64, NT = 512, P = DK + 4, PX = C + 4, NW = C / WN;
  constexpr int NKT = 2 * (DK / 32);           // 32 x 32 tiles of a 64 x dk matrix
  constexpr int NDT = (DK / 32) * (DK / 32);   // 32 x 32 tiles of a dk x dk matrix
  constexpr int NJ = (2 * NKT + 7) / 8;        // dQ and dK tiles per wave
  constexpr int NWJ = (3 * NDT + 7) / 8;       // weight-gradient tiles per wave
  __shared__ __attribute__((aligned(16))) float s_x[C * P];   // X, then V, then X again
  __shared__ __attribute__((aligned(16))) float s_q[C * P];   // Q, then dQ
  __shared__ __attribute__((aligned(16))) float s_k[C * P];   // K, then dK
  __shared__ __attribute__((aligned(16))) float s_p[C * PX];  // scores, P, then dS
  __shared__ float s_m[NW][DK], s_z[NW][DK], s_dz[NW][DK], s_dm[NW][DK], s_dr[NW][DK];
  __shared__ float s_c[C], s_e[C];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t NTL = (a.T + C - 1) / C, NG = (NTL + kRepsBwdTiles - 1) / kRepsBwdTiles;
  const int64_t id = blockIdx.x;
  const int64_t grp = id % NG, bh = id / NG;
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t wo = a.w_hstride * h;
  const T* Wq = reinterpret_cast<const T*>(a.Wq) + wo;
  const T* Wk = reinterpret_cast<const T*>(a.Wk) + wo;
  const T* Wv = reinterpret_cast<const T*>(a.Wv) + wo;
  const T* Wp = reinterpret_cast<const T*>(a.Wp) + wo;
  const T* Wr = a.Wr ? reinterpret_cast<const T*>(a.Wr) + wo : nullptr;
  const float rs = 1.f / sqrtf((float)DK);
  // the workgroup's dWq, dWk, dWv, summed over its tiles
  f32x16 accw[NWJ];
#pragma unroll
  for (int jj = 0; jj < NWJ; ++jj) accw[jj] = zero16();
  const int64_t tl1 = (grp + 1) * kRepsBwdTiles < NTL ? (grp + 1) * kRepsBwdTiles : NTL;
  for (int64_t tile = grp * kRepsBwdTiles; tile < tl1; ++tile) {
    if (tile > grp * kRepsBwdTiles) __syncthreads();  // the previous tile's reads of LDS are done
    const int64_t t0 = tile * C;
    const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
    const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
    auto nwin = [&](int wi) {  // tokens of window wi of the tile
      const int v = n - wi * WN;
      return v < 0 ? 0 : (v > WN ? WN : v);
    };
    const T* kg = reinterpret_cast<const T*>(a.k);
    auto stage_x = [&]() {
      for (int i = tid; i < C * DK; i += NT) {
        const int t = i / DK, e = i % DK;
        s_x[t * P + e] = t < n ? to_f<T>(kg[(row0 + (int64_t)t * a.H) * DK + e]) : 0.f;
      }
    };

    // ---- 0. X (zero past n) and each window's upstream row (zero for an empty window)
    stage_x();
    for (int i = tid; i < NW * DK; i += NT) {
      const int wi = i / DK, e = i % DK;
      const int64_t r = (t0 + wi * WN) / WN;  // the window's representative row
      s_dr[wi][e] = nwin(wi) > 0 ? a.dreps[((b * a.R + r) * a.H + h) * DK + e] : 0.f;
    }
    __syncthreads();

    // ---- 1. Q = X Wq^T and K = X Wk^T into LDS, V = X Wv^T in registers (tile (w & 1, w >> 1))
    for (int j = w; j < 2 * NKT; j += 8) {
      const int tl = j % NKT, tm = tl & 1, tn = tl >> 1;
      const T* wr = (j < NKT ? Wq : Wk) + (int64_t)(tn * 32 + c32) * DK;
      const float* xr = s_x + (tm * 32 + c32) * P;
      const f32x16 acc = mm32<DK>(zero16(), hh, [&](int k) { return xr[k]; }, [&](int k) { return to_f<T>(wr[k]); });
      float* dst = j < NKT ? s_q : s_k;
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(tm * 32 + acc_row(e, hh)) * P + tn * 32 + c32] = acc[e];
    }
    const bool hv = w < NKT;
    const int tv = w & 1, cv = w >> 1;
    f32x16 vt = zero16();
    if (hv) {
      const T* wr = Wv + (int64_t)(cv * 32 + c32) * DK;
      const float* xr = s_x + (tv * 32 + c32) * P;
      vt = mm32<DK>(vt, hh, [&](int k) { return xr[k]; }, [&](int k) { return to_f<T>(wr[k]); });
    }
    __syncthreads();  // X is dead until it is staged again
    if (hv) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_x[(tv * 32 + acc_row(e, hh)) * P + cv * 32 + c32] = vt[e];  // V
    }

    // ---- 2. scores on the window blocks (tile (tm, tn) on wave tm + 2 tn): -inf outside the
    // token's window and past n
    if (w < 4) {
      const int tm = w & 1, tn = w >> 1, s = tn * 32 + c32;
      f32x16 acc = zero16();
      if (WN == 64 || tm == tn) {
        const float* qr = s_q + (tm * 32 + c32) * P;
        const float* kr = s_k + s * P;
        acc = mm32<DK>(acc, hh, [&](int k) { return qr[k]; }, [&](int k) { return kr[k]; });
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = tm * 32 + acc_row(e, hh);
        const bool in = t / WN == s / WN && t < n && s < n;
        s_p[t * PX + s] = in ? acc[e] * rs : -INFINITY;
      }
    }
    __syncthreads();

    // ---- 3. P = softmax over each row's window (rows past n and entries outside: zero)
    if (tid < C) {
      const int t = tid, w0 = (t / WN) * WN;
      float* pr = s_p + t * PX;
      if (t < n) {
        float mx = -INFINITY;
#pragma unroll 4
        for (int s = w0; s < w0 + WN; ++s) mx = fmaxf(mx, pr[s]);
        float sum = 0.f;
#pragma unroll 4
        for (int s = w0; s < w0 + WN; ++s) {
          const float p = __expf(pr[s] - mx);  // exp(-inf) = 0 past n
          pr[s] = p;
          sum += p;
        }
        const float inv = 1.f / sum;
#pragma unroll 4
        for (int s = w0; s < w0 + WN; ++s) pr[s] *= inv;
      } else {
#pragma unroll 4
        for (int s = w0; s < w0 + WN; ++s) pr[s] = 0.f;
      }
#pragma unroll 4
      for (int s = 0; s < C; ++s)
        if (s < w0 || s >= w0 + WN) pr[s] = 0.f;
    }
    __syncthreads();

    // ---- 4. column sums of P within the window
    if (tid < C) {
      const int s = tid, w0 = (s / WN) * WN;
      float c = 0.f;
#pragma unroll 4
      for (int t = w0; t < w0 + WN; ++t) c += s_p[t * PX + s];
      s_c[s] = c;
    }
    __syncthreads();

    // ---- 5. m = (1/n) sum_s c_s V_s per window
    for (int i = tid; i < NW * DK; i += NT) {
      const int wi = i / DK, e = i % DK, nw = nwin(wi);
      float m = 0.f;
#pragma unroll 4
      for (int s = wi * WN; s < wi * WN + nw; ++s) m = fmaf(s_c[s], s_x[s * P + e], m);
      s_m[wi][e] = nw > 0 ? m / (float)nw : 0.f;
    }
    __syncthreads();

    // ---- 6. z = Wp m;  dz = Wr dr' (or dr');  then dm = Wp^T dz
    for (int i = tid; i < NW * DK; i += NT) {
      const int wi = i / DK, e = i % DK;
      const T* wp = Wp + (int64_t)e * DK;
      float z = 0.f;
#pragma unroll 4
      for (int k = 0; k < DK; ++k) z = fmaf(to_f<T>(wp[k]), s_m[wi][k], z);
      s_z[wi][e] = z;
      float dz = s_dr[wi][e];
      if (Wr) {
        const T* wr = Wr + (int64_t)e * DK;
        dz = 0.f;
#pragma unroll 4
        for (int k = 0; k < DK; ++k) dz = fmaf(to_f<T>(wr[k]), s_dr[wi][k], dz);
      }
      s_dz[wi][e] = nwin(wi) > 0 ? dz : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < NW * DK; i += NT) {
      const int wi = i / DK, e = i % DK;
      float dm = 0.f;
#pragma unroll 4
      for (int k = 0; k < DK; ++k) dm = fmaf(to_f<T>(Wp[(int64_t)k * DK + e]), s_dz[wi][k], dm);
      s_dm[wi][e] = dm;
    }
    __syncthreads();

    // ---- 7. e_s = V_s . dm / n (the upstream of P_ts for every t of s's window)
    if (tid < C) {
      const int s = tid, wi = s / WN;
      float e = 0.f;
      if (s < n) {
#pragma unroll 4
        for (int k = 0; k < DK; ++k) e = fmaf(s_dm[wi][k], s_x[s * P + k], e);
        e /= (float)nwin(wi);
      }
      s_e[s] = e;
    }
    __syncthreads();

    // ---- 8. dS_ts = P_ts (e_s - sum_s' P_ts' e_s'), row by row
    if (tid < C) {
      const int t = tid, w0 = (t / WN) * WN;
      float* pr = s_p + t * PX;
      float rho = 0.f;
#pragma unroll 4
      for (int s = w0; s < w0 + WN; ++s) rho = fmaf(pr[s], s_e[s], rho);
#pragma unroll 4
      for (int s = w0; s < w0 + WN; ++s) pr[s] *= s_e[s] - rho;
    }
    __syncthreads();

    // ---- 9. dQ = dS K / sqrt(dk) and dK = dS^T Q / sqrt(dk)
    f32x16 g[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      g[jj] = zero16();
      const int j = w + 8 * jj;
      if (j < 2 * NKT) {
        const int tl = j % NKT, tm = tl & 1, tn = tl >> 1, col = tn * 32 + c32;
        if (j < NKT) {
          const float* dr = s_p + (tm * 32 + c32) * PX;
          g[jj] = mm32<C>(g[jj], hh, [&](int k) { return dr[k]; }, [&](int k) { return s_k[k * P + col]; });
        } else {
          const float* dc = s_p + tm * 32 + c32;
          g[jj] = mm32<C>(g[jj], hh, [&](int k) { return dc[k * PX]; }, [&](int k) { return s_q[k * P + col]; });
        }
      }
    }
    __syncthreads();  // Q, K and dS are read; V is dead
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + 8 * jj;
      if (j < 2 * NKT) {
        const int tl = j % NKT, tm = tl & 1, tn = tl >> 1;
        float* dst = j < NKT ? s_q : s_k;
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[(tm * 32 + acc_row(e, hh)) * P + tn * 32 + c32] = g[jj][e] * rs;
      }
    }
    stage_x();
    __syncthreads();

    // ---- 10. dX = dQ Wq + dK Wk + dV Wv -> dk  (dV_t = c_t dm_w(t) / n_w(t))
    if (w < NKT) {
      const int tm = w & 1, tn = w >> 1, col = tn * 32 + c32, tr = tm * 32 + c32;
      const float* qr = s_q + tr * P;
      const float* kr = s_k + tr * P;
      const float cvt = tr < n ? s_c[tr] / (float)nwin(tr / WN) : 0.f;
      const float* dmr = s_dm[tr / WN];
      f32x16 acc = mm32<DK>(zero16(), hh, [&](int k) { return qr[k]; }, [&](int k) { return to_f<T>(Wq[(int64_t)k * DK + col]); });
      acc = mm32<DK>(acc, hh, [&](int k) { return kr[k]; }, [&](int k) { return to_f<T>(Wk[(int64_t)k * DK + col]); });
      acc = mm32<DK>(acc, hh, [&](int k) { return cvt * dmr[k]; }, [&](int k) { return to_f<T>(Wv[(int64_t)k * DK + col]); });
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = tm * 32 + acc_row(e, hh);
        if (t < n) a.dk[((b * a.T + t0 + t) * a.H + h) * DK + col] = acc[e];
      }
    }

    // ---- 11. the tile's dWq = dQ^T X, dWk = dK^T X, dWv = dV^T X on the matrix cores, and
    // each window's dz, m, z and dr' for dWp and dWr (zero for an empty window)
#pragma unroll
    for (int jj = 0; jj < NWJ; ++jj) {
      const int j = w + 8 * jj;
      if (j < 3 * NDT) {
        const int mat = j / NDT, tl = j % NDT, ti = tl % (DK / 32), tj = tl / (DK / 32);
        const int ia = ti * 32 + c32, jb = tj * 32 + c32;
        auto fb = [&](int k) { return s_x[k * P + jb]; };
        if (mat == 0) {
          accw[jj] = mm32<C>(accw[jj], hh, [&](int k) { return s_q[k * P + ia]; }, fb);
        } else if (mat == 1) {
          accw[jj] = mm32<C>(accw[jj], hh, [&](int k) { return s_k[k * P + ia]; }, fb);
        } else {
          accw[jj] = mm32<C>(accw[jj], hh,
                             [&](int k) { return k < n ? s_c[k] / (float)nwin(k / WN) * s_dm[k / WN][ia] : 0.f; },
                             fb);
        }
      }
    }
    for (int i = tid; i < 4 * NW * DK; i += NT) {
      const int v = i / (NW * DK), wi = (i / DK) % NW, e = i % DK;
      const float x = v == 0 ? s_dz[wi][e] : v == 1 ? s_m[wi][e] : v == 2 ? s_z[wi][e] : s_dr[wi][e];
      const int64_t r = (t0 + wi * WN) / WN;  // the window's representative row
      a.wvec[(((int64_t)v * a.B + b) * a.RW + r) * a.H * DK + h * DK + e] = x;
    }
  }  // tiles

  // the workgroup's dWq, dWk, dWv into its slot
  float* part = a.part + (bh * NG + grp) * 3 * (int64_t)DK * DK;
#pragma unroll
  for (int jj = 0; jj < NWJ; ++jj) {
    const int j = w + 8 * jj;
    if (j < 3 * NDT) {
      const int mat = j / NDT, tl = j % NDT, ti = tl % (DK / 32), tj = tl / (DK / 32);
      float* dst = part + (int64_t)mat * DK * DK;
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(ti * 32 + acc_row(e, hh)) * DK + tj * 32 + c32] = accw[jj][e];
    }
  }
}

// dWp = sum dz m^T (vectors 0, 1) and dWr = sum z dr'^T (vectors 2, 3) over the windows of
// one weight set (every b and head that uses it), in chunks of kRepsOuterRows rows of one
// (b, h): one workgroup of 8 waves per (hw, matrix, b, head of the set, chunk), 32 x 32 output
// tiles, k over the chunk's windows.
template <int DK>
__global__ __launch_bounds__(512) void reps_bwd_outer_kernel(RepsBwdArgs a) {
  constexpr int KR = kRepsOuterRows, NDT = (DK / 32) * (DK / 32);
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NMO = a.Wr ? 2 : 1;
  const int64_t rows = (a.T + 63) / 64 * (64 / a.window);  // representative rows the tiles wrote
  const int64_t nh = a.w_hstride ? 1 : a.H, NKR = (rows + KR - 1) / KR, NP = a.B * nh * NKR;
  const int64_t id = blockIdx.x;
  const int64_t p = id % NP, mo = (id / NP) % NMO, hw = id / (NP * NMO);
  const int64_t kr = p % NKR, hs = (p / NKR) % nh, b = p / (NKR * nh);
  const int64_t h = a.w_hstride ? hw : hs;
  const int64_t r0 = kr * KR, nr = rows - r0 < KR ? rows - r0 : KR;  // this chunk's rows
  const int64_t vs = a.B * a.RW * a.H * DK, ld = a.H * DK;  // elements per vector kind; row stride
  const float* base = a.wvec + ((b * a.RW + r0) * a.H + h) * DK;
  const float* va = base + (mo * 2) * vs;
  const float* vb = base + (mo * 2 + 1) * vs;
  float* dst = a.part2 + ((hw * NMO + mo) * NP + p) * (int64_t)DK * DK;
  for (int j = w; j < NDT; j += 8) {
    const int ti = j % (DK / 32), tj = j / (DK / 32), ia = ti * 32 + c32, jb = tj * 32 + c32;
    const f32x16 acc = mm32<KR>(zero16(), hh, [&](int k) { return k < nr ? va[k * ld + ia] : 0.f; },
                                [&](int k) { return k < nr ? vb[k * ld + jb] : 0.f; });
#pragma unroll
    for (int e = 0; e < 16; ++e) dst[(ti * 32 + acc_row(e, hh)) * DK + jb] = acc[e];
  }
}

// dWq, dWk, dWv: the sum over b, the workgroups and (shared weights) the heads of the tile
// kernel's parts; dWp, dWr: the sum over the outer kernel's parts (b, head, chunk); in that
// fixed order.
// One thread per (hw, matrix, element).
template <int DK>
__global__ __launch_bounds__(256) void reps_bwd_reduce_kernel(RepsBwdArgs a) {
  const int NM = a.Wr ? 5 : 4, NMO = NM - 3;
  const int64_t Hw = a.w_hstride ? a.H : 1, DD = (int64_t)DK * DK;
  const int64_t NG = ((a.T + 63) / 64 + kRepsBwdTiles - 1) / kRepsBwdTiles;
  const int64_t rows = (a.T + 63) / 64 * (64 / a.window);
  const int64_t nh = a.w_hstride ? 1 : a.H, NP = a.B * nh * ((rows + kRepsOuterRows - 1) / kRepsOuterRows);
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (id >= Hw * NM * DD) return;
  const int64_t e = id % DD, m = (id / DD) % NM, hw = id / (DD * NM);
  const int64_t h0 = a.w_hstride ? hw : 0, h1 = a.w_hstride ? hw + 1 : a.H;
  float s = 0.f;
  if (m < 3) {
    for (int64_t b = 0; b < a.B; ++b)
      for (int64_t h = h0; h < h1; ++h)
        for (int64_t g = 0; g < NG; ++g) s += a.part[(((b * a.H + h) * NG + g) * 3 + m) * DD + e];
  } else {
    for (int64_t p = 0; p < NP; ++p) s += a.part2[((hw * NMO + (m - 3)) * NP + p) * DD + e];
  }
  a.dW[m][hw * DD + e] = s;
}

template <class T, int DK, int WN>
static void launch_tiles(const RepsBwdArgs& a, hipStream_t s) {
  const int64_t groups = a.B * a.H * (((a.T + 63) / 64 + kRepsBwdTiles - 1) / kRepsBwdTiles);
  hipLaunchKernelGGL((reps_bwd_tile_kernel<T, DK, WN>), dim3((unsigned)groups), dim3(512), 0, s, a);
}

template <class T, int DK>
static hipError_t launch_reps_bwd_t(const RepsBwdArgs& a, hipStream_t s) {
  TimedLaunch tl(HLA_KERNEL_BWD_REPS, s);
  switch (a.window) {
    case 8: launch_tiles<T, DK, 8>(a, s); break;
    case 16: launch_tiles<T, DK, 16>(a, s); break;
    case 32: launch_tiles<T, DK, 32>(a, s); break;
    default: launch_tiles<T, DK, 64>(a, s); break;
  }
  const int64_t Hw = a.w_hstride ? a.H : 1, NMO = a.Wr ? 2 : 1;
  const int64_t rows = (a.T + 63) / 64 * (64 / a.window), nh = a.w_hstride ? 1 : a.H;
  const int64_t NP = a.B * nh * ((rows + kRepsOuterRows - 1) / kRepsOuterRows);
  hipLaunchKernelGGL((reps_bwd_outer_kernel<DK>), dim3((unsigned)(Hw * NMO * NP)), dim3(512), 0, s, a);
  const int64_t total = Hw * (3 + NMO) * (int64_t)DK * DK;
  hipLaunchKernelGGL((reps_bwd_reduce_kernel<DK>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reps_backward(const RepsBwdArgs& a, int dtype, int dk, hipStream_t s) {
  if (dtype == 1) return dk == 64 ? launch_reps_bwd_t<bf16, 64>(a, s) : launch_reps_bwd_t<bf16, 128>(a, s);
  return dk == 64 ? launch_reps_bwd_t<float, 64>(a, s) : launch_reps_bwd_t<float, 128>(a, s);
}

}  // namespace hla
