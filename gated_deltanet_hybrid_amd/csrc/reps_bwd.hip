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
// Two kernels:
//   tile    one workgroup of 8 waves per 64-token tile of a (b, h) row (windows divide 64,
//           so none crosses a tile): the projections, the window-block scores, dQ, dK, dX
//           and the tile's weight gradients are 32 x 32 tiles of v_mfma_f32_32x32x2_f32,
//           the softmax and the per-window vectors run on the VALU; dX goes straight to
//           dk, the tile's weight gradients to its own workspace slot;
//   reduce  the weight gradients of every tile of a head (of every head, for shared
//           weights) summed in a fixed order: deterministic, no atomics.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

template <class T, int DK, int WN>
__global__ __launch_bounds__(512, 1) void reps_bwd_tile_kernel(RepsBwdArgs a) {
  constexpr int C = 64, NT = 512, P = DK + 4, PX = C + 4, NW = C / WN;
  constexpr int NKT = 2 * (DK / 32);           // 32 x 32 tiles of a 64 x dk matrix
  constexpr int NDT = (DK / 32) * (DK / 32);   // 32 x 32 tiles of a dk x dk matrix
  constexpr int NJ = (2 * NKT + 7) / 8;        // dQ and dK tiles per wave
  __shared__ __attribute__((aligned(16))) float s_x[C * P];   // X, then V, then X again
  __shared__ __attribute__((aligned(16))) float s_q[C * P];   // Q, then dQ
  __shared__ __attribute__((aligned(16))) float s_k[C * P];   // K, then dK
  __shared__ __attribute__((aligned(16))) float s_p[C * PX];  // scores, P, then dS
  __shared__ float s_m[NW][DK], s_z[NW][DK], s_dz[NW][DK], s_dm[NW][DK], s_dr[NW][DK];
  __shared__ float s_c[C], s_e[C];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t NTL = (a.T + C - 1) / C;
  const int64_t id = blockIdx.x;
  const int64_t tile = id % NTL, bh = id / NTL;
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = tile * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
  const int64_t wo = a.w_hstride * h;
  const T* Wq = reinterpret_cast<const T*>(a.Wq) + wo;
  const T* Wk = reinterpret_cast<const T*>(a.Wk) + wo;
  const T* Wv = reinterpret_cast<const T*>(a.Wv) + wo;
  const T* Wp = reinterpret_cast<const T*>(a.Wp) + wo;
  const T* Wr = a.Wr ? reinterpret_cast<const T*>(a.Wr) + wo : nullptr;
  const float rs = 1.f / sqrtf((float)DK);
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

  // ---- 11. the tile's weight gradients: dWq = dQ^T X, dWk = dK^T X, dWv = dV^T X on the
  // matrix cores; dWp = sum_w dz_w m_w^T and dWr = sum_w z_w dr'_w^T on the VALU
  const int NM = Wr ? 5 : 4;
  float* part = a.part + ((bh * NTL + tile) * NM) * (int64_t)DK * DK;
  for (int j = w; j < 3 * NDT; j += 8) {
    const int mat = j / NDT, tl = j % NDT, ti = tl % (DK / 32), tj = tl / (DK / 32);
    const int ia = ti * 32 + c32, jb = tj * 32 + c32;
    auto fb = [&](int k) { return s_x[k * P + jb]; };
    f32x16 acc = zero16();
    if (mat == 0) {
      acc = mm32<C>(acc, hh, [&](int k) { return s_q[k * P + ia]; }, fb);
    } else if (mat == 1) {
      acc = mm32<C>(acc, hh, [&](int k) { return s_k[k * P + ia]; }, fb);
    } else {
      acc = mm32<C>(acc, hh, [&](int k) { return k < n ? s_c[k] / (float)nwin(k / WN) * s_dm[k / WN][ia] : 0.f; }, fb);
    }
    float* dst = part + (int64_t)mat * DK * DK;
#pragma unroll
    for (int e = 0; e < 16; ++e) dst[(ti * 32 + acc_row(e, hh)) * DK + jb] = acc[e];
  }
  for (int i = tid; i < DK * DK; i += NT) {
    const int r = i / DK, c = i % DK;
    float sp = 0.f, sr = 0.f;
#pragma unroll
    for (int wi = 0; wi < NW; ++wi) {
      sp = fmaf(s_dz[wi][r], s_m[wi][c], sp);
      sr = fmaf(s_z[wi][r], s_dr[wi][c], sr);
    }
    part[3 * DK * DK + i] = sp;
    if (Wr) part[4 * DK * DK + i] = sr;
  }
}

// dW[m][hw] = the sum over b, the tiles and (shared weights) the heads of the tiles' parts,
// in that fixed order.  One thread per (hw, m, element).
template <int DK>
__global__ __launch_bounds__(256) void reps_bwd_reduce_kernel(RepsBwdArgs a) {
  const int NM = a.Wr ? 5 : 4;
  const int64_t Hw = a.w_hstride ? a.H : 1, NTL = (a.T + 63) / 64, DD = (int64_t)DK * DK;
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (id >= Hw * NM * DD) return;
  const int64_t e = id % DD, m = (id / DD) % NM, hw = id / (DD * NM);
  const int64_t h0 = a.w_hstride ? hw : 0, h1 = a.w_hstride ? hw + 1 : a.H;
  float s = 0.f;
  for (int64_t b = 0; b < a.B; ++b)
    for (int64_t h = h0; h < h1; ++h)
      for (int64_t tl = 0; tl < NTL; ++tl) s += a.part[((((b * a.H + h) * NTL + tl) * NM + m) * DD) + e];
  a.dW[m][hw * DD + e] = s;
}

template <class T, int DK, int WN>
static void launch_tiles(const RepsBwdArgs& a, hipStream_t s) {
  const int64_t tiles = a.B * a.H * ((a.T + 63) / 64);
  hipLaunchKernelGGL((reps_bwd_tile_kernel<T, DK, WN>), dim3((unsigned)tiles), dim3(512), 0, s, a);
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
  const int64_t total = (a.w_hstride ? a.H : 1) * (a.Wr ? 5 : 4) * (int64_t)DK * DK;
  hipLaunchKernelGGL((reps_bwd_reduce_kernel<DK>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_reps_backward(const RepsBwdArgs& a, int dtype, int dk, hipStream_t s) {
  if (dtype == 1) return dk == 64 ? launch_reps_bwd_t<bf16, 64>(a, s) : launch_reps_bwd_t<bf16, 128>(a, s);
  return dk == 64 ? launch_reps_bwd_t<float, 64>(a, s) : launch_reps_bwd_t<float, 128>(a, s);
}

}  // namespace hla
