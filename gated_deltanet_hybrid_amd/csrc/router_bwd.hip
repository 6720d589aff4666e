// Backward of the HLA router gates (C = 64; the raw keys, n_rep = 64, or learned
// representatives, n_rep of them per chunk).
//
// [HLA] Overview and Methodology paragraph 2: qbar_i = mean of q over query chunk i,
// s_ijr = qbar_i . r_{j n_rep + r} / sqrt(dk) over history chunk j's representatives,
// l_ij = log-mean-exp over r of s_ijr, g_ij = sigmoid(l_ij).  Given dg_ij (zero for skipped
// pairs):
//     dl_ij = dg_ij g_ij (1 - g_ij),   p_ijr = softmax over r of s_ijr,
//     dqbar_i  = sum_{j<i} dl_ij sum_r p_ijr r_{j n_rep + r} / sqrt(dk),
//     dr_{j n_rep + r} = sum_{i>j} dl_ij p_ijr qbar_i / sqrt(dk),
// and every token of chunk i receives dqbar_i / n_i (added by the chunk backward's
// finalize pass, or written per token here).
//
// Both sums run on the matrix cores in the forward gate pass's orientation: S^T (a history
// chunk's representatives x 32 query chunks, one query per lane column) from representative
// rows and query means (float32 split into bf16 high and low parts on the bf16 path, so the
// scores keep float32 accuracy), the softmax down each lane's column, and
// Z^T = (dl p / sqrt(dk))^T in the accumulators.  Then
//   query side (router_dq_kernel): dqbar (32 queries x dk per wave) += Z R_j, with Z^T taken
//     straight from the accumulators (their row order serves as the k order of the next
//     product) and R_j staged feature-major in LDS; one workgroup per (b, h, 128 query
//     chunks, segment of history chunks), each segment's sum a part that
//     router_dq_sum_kernel adds in a fixed order;
//   representative side (router_dr_kernel): one wave per history chunk j, dR_j (n_rep x dk)
//     += Z Qbar over tiles of 32 query chunks i > j, Z transposed through LDS, written once.
// No atomics: the results are bitwise reproducible.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {
constexpr int kRT = 64;  // representative rows of a history chunk, padded (n_rep <= 64)

// x ~= hi + lo with both parts in bf16 (about 16 significant bits together): element e of
// the fragments fh (high parts) and fl (low parts)
__device__ __forceinline__ void split_bf16(float x, bf16x8& fh, bf16x8& fl, int e) {
  const bf16 hi = (bf16)x;
  fh[e] = hi;
  fl[e] = (bf16)(x - (float)hi);
}

// softmax over a history chunk's representatives of the scores in sc (rows = representatives
// rt * 32 + acc_row(e, hh), this lane's column = one query), scaled by w: sc <- w p.
__device__ __forceinline__ void column_softmax(f32x16 (&sc)[2], int n_rep, int hh, float scale, float w) {
  float mx = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float v = rt * 32 + acc_row(e, hh) < n_rep ? sc[rt][e] * scale : -INFINITY;
      sc[rt][e] = v;
      mx = fmaxf(mx, v);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float sum = 0.f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sc[rt][e] = __expf(sc[rt][e] - mx);  // 0 past n_rep
      sum += sc[rt][e];
    }
  sum += __shfl_xor(sum, 32, 64);
  const float z = w / sum;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[rt][e] *= z;
}

// dl_ij = dg_ij g_ij (1 - g_ij) of one (query chunk, history chunk) pair
__device__ __forceinline__ float pair_weight(const RouterBwdArgs& a, int64_t bh, int i, int j) {
  const int64_t o = (bh * a.N + i) * (int64_t)a.N + j;
  const float g = a.gates[o];
  return a.dgates[o] * g * (1.f - g);
}
}  // namespace

// qbar_i, the mean of q over query chunk i: one thread per (b, h, i, feature).
template <class T, int DK>
__global__ __launch_bounds__(256) void router_qbar_kernel(RouterBwdArgs a) {
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (id >= a.B * a.H * a.N * DK) return;
  const int e = (int)(id % DK);
  const int64_t bhi = id / DK;
  const int i = (int)(bhi % a.N);
  const int64_t bh = bhi / a.N, h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)i * kChunk;
  const int ni = (int)((a.T - t0) < kChunk ? (a.T - t0) : kChunk);
  const T* q = reinterpret_cast<const T*>(a.q) + ((b * a.ld_T + t0) * a.H + h) * DK + e;
  // all 64 loads issued together (rows past the chunk's end re-read its last row and count
  // zero), summed in token order
  float v[kChunk];
#pragma unroll
  for (int t = 0; t < kChunk; ++t) v[t] = to_f<T>(q[(int64_t)(t < ni ? t : ni - 1) * a.H * DK]);
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < kChunk; ++t) s += t < ni ? v[t] : 0.f;
  a.qbar[id] = s / (float)ni;
}

// Query side.  Wave w of workgroup (b, h, qg, js) owns query chunks (4 qg + w) 32 + lane % 32
// and sums over history chunks j in [js seg, (js + 1) seg) below the group's last query
// chunk.  Chunk j + 1's rows are prefetched into registers while chunk j is used.
template <class T, int DK>
__global__ __launch_bounds__(256) void router_dq_kernel(RouterBwdArgs a) {
  using MM = Mma<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int EPP = 16 / (int)sizeof(T), PR = DK + EPP, UPR = DK / EPP, NU = kRT * UPR / 256;
  constexpr int PRT = kRT + 8;  // feature-major rows of the bf16 copy
  constexpr int NKS = DK / MM::KS, NDT = DK / 32, NZK = BF ? 2 : 16;  // k-steps per 32 representatives
  static_assert(NU * 256 == kRT * UPR, "staging split");
  __shared__ __attribute__((aligned(16))) T sR[2][kRT * PR];
  __shared__ __attribute__((aligned(16))) T sRT[2][BF ? DK * PRT : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int seg = router_bwd_seg(a.B * a.H, a.N);
  const int nqg = ((a.N + 31) / 32 + 3) / 4, njs = (a.N + seg - 1) / seg;
  int64_t id = blockIdx.x;
  const int js = (int)(id % njs);
  id /= njs;
  const int qg = (int)(id % nqg);
  const int64_t bh = id / nqg, h = bh % a.H, b = bh / a.H;
  const int imax = ((qg + 1) * 128 < a.N ? (qg + 1) * 128 : a.N) - 1;  // the group's last query chunk
  const int j_lo = js * seg, j_hi = j_lo + seg < imax ? j_lo + seg : imax;  // pairs j < i <= imax
  if (j_lo >= j_hi) return;  // no pair here; router_dq_sum_kernel reads no part of it
  const int qi = (qg * 4 + w) * 32 + c32;
  const float scale = 1.f / sqrtf((float)DK);

  // B operand of the scores: this lane's query mean
  typename MM::Frag bhi[NKS], blo[BF ? NKS : 1];
  {
    const float* qb = a.qbar + (bh * a.N + (qi < a.N ? qi : 0)) * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF) {
        bf16x8 fh, fl;
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(qi < a.N ? qb[ks * 16 + hh * 8 + e] : 0.f, fh, fl, e);
        bhi[ks] = fh;
        blo[ks] = fl;
      } else {
        bhi[ks] = qi < a.N ? qb[ks * 2 + hh] : 0.f;
      }
    }
  }
  const T* reps = reinterpret_cast<const T*>(a.reps);
  uint4 pf[NU];
  auto load_chunk = [&](int j) {
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int u = tid + 256 * m, r = u / UPR, cu = u % UPR;
      pf[m] = make_uint4(0u, 0u, 0u, 0u);
      if (r < a.n_rep)
        pf[m] = *reinterpret_cast<const uint4*>(reps + ((b * a.ld_R + (int64_t)j * a.n_rep + r) * a.H + h) * DK +
                                                cu * EPP);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int u = tid + 256 * m, r = u / UPR, cu = u % UPR;
      *reinterpret_cast<uint4*>(&sR[buf][r * PR + cu * EPP]) = pf[m];
      if constexpr (BF) {
        const bf16* v = reinterpret_cast<const bf16*>(&pf[m]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sRT[buf][(cu * 8 + e) * PRT + r] = v[e];
      }
    }
  };

  f32x16 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dq[dt] = zero16();
  // dl of this lane's pair with history chunk j (zero unless j < qi < N); every load in bounds
  auto weight = [&](int j) {
    const float v = pair_weight(a, bh, qi < a.N ? qi : a.N - 1, j);
    return (qi < a.N && j < qi) ? v : 0.f;
  };
  // One history chunk: scores, softmax, dqbar += Z R_j.  TWO: a second tile of 32
  // representatives (n_rep > 32).  Fragments are loaded in blocks ahead of their products,
  // and the high and low parts of the query means feed separate accumulators, so that
  // independent products are in flight while the LDS loads return.
  auto round = [&](int buf, float dl, auto TWO) {
    constexpr bool two = decltype(TWO)::value;
    constexpr int KB = BF ? NKS : 16;
    f32x16 sc[2], sl[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sc[rt] = sl[rt] = zero16();
    const T* r0 = &sR[buf][c32 * PR];
    const T* r1 = &sR[buf][(32 + c32) * PR];
#pragma unroll
    for (int k0 = 0; k0 < NKS; k0 += KB) {
      typename MM::Frag a0[KB], a1[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        a0[u] = MM::load_plain(r0, k0 + u, hh);
        if constexpr (two) a1[u] = MM::load_plain(r1, k0 + u, hh);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        sc[0] = MM::mma(a0[u], bhi[k0 + u], sc[0]);
        if constexpr (two) sc[1] = MM::mma(a1[u], bhi[k0 + u], sc[1]);
        if constexpr (BF) {
          sl[0] = MM::mma(a0[u], blo[k0 + u], sl[0]);
          if constexpr (two) sl[1] = MM::mma(a1[u], blo[k0 + u], sl[1]);
        }
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[rt][e] += sl[rt][e];
    }
    column_softmax(sc, a.n_rep, hh, scale, dl * scale);
    // dqbar += Z R_j: A = Z (lane = query; slot k = accumulator row), B = R_j in that k order
    constexpr int KK = BF ? NZK : 4;
#pragma unroll
    for (int rt = 0; rt < (two ? 2 : 1); ++rt) {
#pragma unroll
      for (int k0 = 0; k0 < NZK; k0 += KK) {
        typename MM::Frag rb[KK][NDT];
#pragma unroll
        for (int u = 0; u < KK; ++u)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            if constexpr (BF)
              rb[u][dt] = MM::load_clayout(&sRT[buf][(dt * 32 + c32) * PRT + rt * 32], k0 + u, hh);
            else
              rb[u][dt] = sR[buf][(rt * 32 + Mma<float>::clayout_k(k0 + u, hh)) * PR + dt * 32 + c32];
          }
#pragma unroll
        for (int u = 0; u < KK; ++u) {
          typename MM::Frag zh, zl;
          if constexpr (BF) {
#pragma unroll
            for (int e = 0; e < 8; ++e) split_bf16(sc[rt][(k0 + u) * 8 + e], zh, zl, e);
          } else {
            zh = sc[rt][k0 + u];
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) dq[dt] = MM::mma(zh, rb[u][dt], dq[dt]);
          if constexpr (BF) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) dq[dt] = MM::mma(zl, rb[u][dt], dq[dt]);
          }
        }
      }
    }
  };
  load_chunk(j_lo);
  float dl_next = weight(j_lo);
  store_chunk(0);
  __syncthreads();
  for (int j = j_lo; j < j_hi; ++j) {
    const int buf = (j - j_lo) & 1;
    const float dl = dl_next;
    if (j + 1 < j_hi) {  // chunk j + 1 and its weights: in flight during this round
      load_chunk(j + 1);
      dl_next = weight(j + 1);
    }
    if (a.n_rep > 32)
      round(buf, dl, std::true_type{});
    else
      round(buf, dl, std::false_type{});
    if (j + 1 < j_hi) store_chunk(buf ^ 1);  // buf ^ 1 was last read before the previous barrier
    __syncthreads();
  }
  // this segment's part of dqbar for the wave's 32 query chunks (rows = queries)
  float* pdq = a.part + ((int64_t)js * a.B * a.H + bh) * a.N * DK;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = (qg * 4 + w) * 32 + acc_row(e, hh);
      if (q < a.N) pdq[(int64_t)q * DK + dt * 32 + c32] = dq[dt][e];
    }
}

// dqbar_i = the sum of the parts of the segments that start below i, in segment order.
template <int DK>
__global__ __launch_bounds__(256) void router_dq_sum_kernel(RouterBwdArgs a) {
  const int64_t nq = a.B * a.H * a.N * DK;
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (id >= nq) return;
  const int seg = router_bwd_seg(a.B * a.H, a.N);
  const int i = (int)((id / DK) % a.N);
  const int nseg = (i + seg - 1) / seg;
  float s = 0.f;
  for (int g = 0; g < nseg; ++g) s += a.part[g * nq + id];
  a.dqbar[id] = s;
}

// Representative side.  Wave w of workgroup (b, h, g) owns history chunk j = 4 g + w; the
// workgroup walks the tiles of 32 query chunks that hold an i > 4 g, staging each tile's
// means in LDS in both orientations.  Rows of the last chunk (no query reads it) are zero.
template <class T, int DK>
__global__ __launch_bounds__(256) void router_dr_kernel(RouterBwdArgs a) {
  using MM = Mma<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int PQ = DK + 16 / (int)sizeof(T), PQT = 32 + 16 / (int)sizeof(T), PZ = 32 + 4;
  constexpr int NKS = DK / MM::KS, NDT = DK / 32, NQK = 32 / MM::KS;
  __shared__ __attribute__((aligned(16))) T sQh[32 * PQ];
  __shared__ __attribute__((aligned(16))) T sQl[BF ? 32 * PQ : 1];
  __shared__ __attribute__((aligned(16))) T sQTh[DK * PQT];
  __shared__ __attribute__((aligned(16))) T sQTl[BF ? DK * PQT : 1];
  __shared__ __attribute__((aligned(16))) float sZ[4][kRT * PZ];
  __shared__ __attribute__((aligned(16))) T sRw[4][BF ? kRT * (DK + 8) : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int ng = (a.N + 3) / 4;
  const int64_t bh = blockIdx.x / ng, h = bh % a.H, b = bh / a.H;
  const int g = (int)(blockIdx.x % ng);
  const int j = g * 4 + w;
  const bool hist = j < a.N - 1;  // some query chunk i > j reads chunk j
  const int nrt = (a.n_rep + 31) / 32;
  const float scale = 1.f / sqrtf((float)DK);
  const T* reps = reinterpret_cast<const T*>(a.reps);
  auto rep_row = [&](int rt) -> const T* {  // this lane's representative row of tile rt, or null
    const int r = rt * 32 + c32;
    return (hist && r < a.n_rep) ? reps + ((b * a.ld_R + (int64_t)j * a.n_rep + r) * a.H + h) * DK : nullptr;
  };
  // A operand of the scores on the bf16 path: the wave's own chunk rows, staged in LDS once
  // (zero past n_rep, and for a chunk no query reads)
  constexpr int UPR = DK / 8, PR = DK + 8;
  if constexpr (BF) {
    for (int u = lane; u < kRT * UPR; u += 64) {
      const int r = u / UPR, cu = u % UPR;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (hist && r < a.n_rep)
        v = *reinterpret_cast<const uint4*>(reps + ((b * a.ld_R + (int64_t)j * a.n_rep + r) * a.H + h) * DK + cu * 8);
      *reinterpret_cast<uint4*>(&sRw[w][r * PR + cu * 8]) = v;
    }
  }
  f32x16 dr[2][NDT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dr[rt][dt] = zero16();
  // the next tile's query means (one slice per thread) and this lane's pair weight, loaded
  // a tile ahead; every load in bounds
  constexpr int NQV = 32 * DK / 256;
  const int nqt = (a.N + 31) / 32, jc = j < a.N - 1 ? j : a.N - 1;
  float qv[NQV], dl_next = 0.f;
  auto load_tile = [&](int t) {
#pragma unroll
    for (int m = 0; m < NQV; ++m) {
      const int x = tid + 256 * m, r = x / DK, d = x % DK, i = t * 32 + r;
      const float v = a.qbar[(bh * a.N + (i < a.N ? i : a.N - 1)) * DK + d];
      qv[m] = i < a.N ? v : 0.f;
    }
    const int qi = t * 32 + c32;
    const float v = pair_weight(a, bh, qi < a.N ? qi : a.N - 1, jc);
    dl_next = (hist && qi < a.N && qi > j) ? v : 0.f;
  };
  // One tile: scores, softmax, Z^T to LDS, dR_j += Z Qbar (TWO: n_rep > 32).  As in the
  // query-side pass, fragments are loaded in blocks ahead of their products and the two
  // parts of the means feed separate accumulators.
  auto tile = [&](float dl, auto TWO) {
    constexpr bool two = decltype(TWO)::value;
    constexpr int KB = BF ? 4 : 16;
    f32x16 sc[2], sl[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) sc[rt] = sl[rt] = zero16();
    const T* row0 = rep_row(0);
    const T* row1 = rep_row(1);
#pragma unroll
    for (int k0 = 0; k0 < NKS; k0 += KB) {
      typename MM::Frag qh[KB], ql[KB];
      typename MM::Frag ra0[BF ? KB : 1], ra1[BF ? KB : 1];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        qh[u] = MM::load_plain(&sQh[c32 * PQ], k0 + u, hh);
        if constexpr (BF) {
          ql[u] = MM::load_plain(&sQl[c32 * PQ], k0 + u, hh);
          ra0[u] = MM::load_plain(&sRw[w][c32 * PR], k0 + u, hh);
          if constexpr (two) ra1[u] = MM::load_plain(&sRw[w][(32 + c32) * PR], k0 + u, hh);
        }
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        typename MM::Frag a0, a1;
        if constexpr (BF) {
          a0 = ra0[u];
          if constexpr (two) a1 = ra1[u];
        } else {
          a0 = row0 ? MM::load_plain(row0, k0 + u, hh) : 0.f;
          if constexpr (two) a1 = row1 ? MM::load_plain(row1, k0 + u, hh) : 0.f;
        }
        sc[0] = MM::mma(a0, qh[u], sc[0]);
        if constexpr (two) sc[1] = MM::mma(a1, qh[u], sc[1]);
        if constexpr (BF) {
          sl[0] = MM::mma(a0, ql[u], sl[0]);
          if constexpr (two) sl[1] = MM::mma(a1, ql[u], sl[1]);
        }
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[rt][e] += sl[rt][e];
    }
    column_softmax(sc, a.n_rep, hh, scale, dl * scale);
#pragma unroll
    for (int rt = 0; rt < (two ? 2 : 1); ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sZ[w][(rt * 32 + acc_row(e, hh)) * PZ + c32] = sc[rt][e];
    __syncthreads();
    // dR_j += Z Qbar: A = Z (lane = representative, k = query), B = Qbar (k = query, lane = feature)
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) {
      typename MM::Frag bh_[NDT], bl_[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bh_[dt] = MM::load_plain(&sQTh[(dt * 32 + c32) * PQT], ks, hh);
        if constexpr (BF) bl_[dt] = MM::load_plain(&sQTl[(dt * 32 + c32) * PQT], ks, hh);
      }
#pragma unroll
      for (int rt = 0; rt < (two ? 2 : 1); ++rt) {
        const float* zrow = &sZ[w][(rt * 32 + c32) * PZ];
        typename MM::Frag zh, zl;
        if constexpr (BF) {
#pragma unroll
          for (int e = 0; e < 8; ++e) split_bf16(zrow[ks * 16 + hh * 8 + e], zh, zl, e);
        } else {
          zh = zrow[ks * 2 + hh];
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) dr[rt][dt] = MM::mma(zh, bh_[dt], dr[rt][dt]);
        if constexpr (BF) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) dr[rt][dt] = MM::mma(zh, bl_[dt], dr[rt][dt]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) dr[rt][dt] = MM::mma(zl, bh_[dt], dr[rt][dt]);
        }
      }
    }
  };
  const int t_lo = (g * 4 + 1) / 32;
  if (t_lo < nqt) load_tile(t_lo);
  for (int t = t_lo; t < nqt; ++t) {
    __syncthreads();  // the previous tile's reads of sQ*, sZ are done
#pragma unroll
    for (int m = 0; m < NQV; ++m) {
      const int x = tid + 256 * m, r = x / DK, d = x % DK;
      const float v = qv[m];
      if constexpr (BF) {
        const bf16 vh = (bf16)v, vl = (bf16)(v - (float)vh);
        sQh[r * PQ + d] = vh;
        sQl[r * PQ + d] = vl;
        sQTh[d * PQT + r] = vh;
        sQTl[d * PQT + r] = vl;
      } else {
        sQh[r * PQ + d] = v;
        sQTh[d * PQT + r] = v;
      }
    }
    const float dl = dl_next;
    if (t + 1 < nqt) load_tile(t + 1);  // in flight during this tile
    __syncthreads();
    if (nrt > 1)
      tile(dl, std::true_type{});
    else
      tile(dl, std::false_type{});
  }
  if (j >= a.N) return;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = rt * 32 + acc_row(e, hh);
        const int64_t row = (int64_t)j * a.n_rep + r;
        if (r < a.n_rep && row < a.R_out)
          a.dreps[((b * a.R_out + row) * a.H + h) * DK + dt * 32 + c32] = dr[rt][dt][e];
      }
}

// dqbar of each token's chunk over the chunk's token count, per token.
template <int DK>
__global__ __launch_bounds__(256) void router_spread_kernel(RouterBwdArgs a) {
  constexpr int C = kChunk;
  const int64_t id = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (id >= a.B * a.T * a.H * DK) return;
  const int e = (int)(id % DK);
  const int64_t bth = id / DK;
  const int64_t h = bth % a.H, bt = bth / a.H;
  const int64_t t = bt % a.T, b = bt / a.T;
  const int c = (int)(t / C);
  const int64_t t0 = (int64_t)c * C;
  const int nc = (int)((a.T - t0) < C ? (a.T - t0) : C);
  a.dq_tok[id] = a.dqbar[((b * a.H + h) * a.N + c) * DK + e] / (float)nc;
}

template <class T, int DK>
static hipError_t launch_router_bwd_t(const RouterBwdArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H, nq = BH * a.N * DK;
  const int seg = router_bwd_seg(BH, a.N);
  const int64_t nqg = ((a.N + 31) / 32 + 3) / 4, njs = (a.N + seg - 1) / seg, ng = (a.N + 3) / 4;
  const unsigned gq = (unsigned)((nq + 255) / 256);
  TimedLaunch tl(HLA_KERNEL_BWD_ROUTER, s);
  hipLaunchKernelGGL((router_qbar_kernel<T, DK>), dim3(gq), dim3(256), 0, s, a);
  hipLaunchKernelGGL((router_dq_kernel<T, DK>), dim3((unsigned)(BH * nqg * njs)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((router_dr_kernel<T, DK>), dim3((unsigned)(BH * ng)), dim3(256), 0, s, a);
  hipLaunchKernelGGL((router_dq_sum_kernel<DK>), dim3(gq), dim3(256), 0, s, a);
  if (a.dq_tok) {
    const int64_t total = a.B * a.T * a.H * DK;
    hipLaunchKernelGGL((router_spread_kernel<DK>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_router_backward(const RouterBwdArgs& a, int dtype, int dk, hipStream_t s) {
  if (dtype == 1) return dk == 64 ? launch_router_bwd_t<bf16, 64>(a, s) : launch_router_bwd_t<bf16, 128>(a, s);
  return dk == 64 ? launch_router_bwd_t<float, 64>(a, s) : launch_router_bwd_t<float, 128>(a, s);
}

}  // namespace hla
