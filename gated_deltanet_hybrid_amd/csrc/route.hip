// HLA router and gated composition.
//
// [HLA] Overview (log-mean-exp pooled routing gates) and Methodology paragraphs 2-4:
//   qbar_i = mean of q over query chunk i
//   l_ij   = log((1/n_rep) sum_r exp(qbar_i . r / sqrt(dk)))  over chunk j's representatives
//   g_ij   = sigmoid(l_ij) for j < i, g_ii = 1, g_ij = 0 for j > i (independent gates)
//   mask   = (j < i) and g_ij >= tau (skip below tau, no renormalisation)
//   n_eff  = (sum ghat)^2 / sum ghat^2            ([HLA] Key Contributions 3)
//   S~_i   = fold over j < i in time order of  M -> M + g_ij (At_j M + Bc_j - M)
// The composition is written as M <- M + (At_j - I) (g M) + g Bc_j: the identity part of
// the blend stays in fp32 (the state is the MFMA accumulator), only g M enters the matrix
// core as a bf16 operand, and g Bc_j is one more MFMA against g I.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

// ---------------------------------------------------------------- query-chunk means
// One 256-thread workgroup per (b, h, chunk i): 16 token groups x 16 lanes of 16 bytes.
template <class T, int DK>
__global__ __launch_bounds__(256) void qbar_kernel(RouteArgs a) {
  constexpr int PAD = 16 / sizeof(T), UPR = DK / PAD;  // 16-byte units per token row
  constexpr int TG = 256 / UPR;                        // token groups
  __shared__ float part[TG][DK];
  const int64_t id = blockIdx.x;  // (b, h, i)
  const int i = (int)(id % a.N);
  const int64_t bh = id / a.N, h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)i * a.C;
  const int n = (int)((a.T - t0) < a.C ? (a.T - t0) : a.C);
  const int u = threadIdx.x % UPR, tg = threadIdx.x / UPR;
  const T* q = reinterpret_cast<const T*>(a.q) + ((b * a.ld_T + t0) * a.H + h) * DK + u * PAD;
  float acc[PAD];
#pragma unroll
  for (int e = 0; e < PAD; ++e) acc[e] = 0.f;
  for (int t = tg; t < n; t += TG) {
    const uint4 raw = *reinterpret_cast<const uint4*>(q + (int64_t)t * a.H * DK);
    const T* ev = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < PAD; ++e) acc[e] += to_f<T>(ev[e]);
  }
#pragma unroll
  for (int e = 0; e < PAD; ++e) part[tg][u * PAD + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < DK) {
    float s = 0.f;
    for (int g = 0; g < TG; ++g) s += part[g][threadIdx.x];
    a.qbar[id * DK + threadIdx.x] = s / (float)n;
  }
}

// ---------------------------------------------------------------- gate scores
// Workgroup = (b, h, segment of 32 history chunks, group of 4 query tiles of 32 chunks);
// wave w scores query tile 4 g + w.  Each history chunk's representatives (the MFMA rows)
// are staged once in LDS with coalesced loads and shared by the four waves; the next
// chunk's rows are prefetched into registers while the current one is scored.  Queries
// are the columns, so pooling over representatives is lane-local plus one exchange
// between the lane halves.
// History chunks per workgroup of gate_kernel: about 64 rounds of 32 representatives each
// (32 chunks of the raw 64 keys; 8 chunks of 256 keys, so that C = 256, with 4x fewer
// chunks, still fills the GPU), and at most 32 chunks.
__host__ __device__ inline int gate_seg(int n_rep) {
  const int nkt = (n_rep + 31) / 32;
  const int s = 64 / nkt;
  return s < 1 ? 1 : (s > 32 ? 32 : s);
}
template <class T, int DK>
__global__ __launch_bounds__(256) void gate_kernel(RouteArgs a) {
  using MM = Mma<T>;
  const int JSEG = gate_seg(a.n_rep);
  constexpr int PAD = 16 / sizeof(T), UPR = DK / PAD;
  constexpr int RT = 32;                  // representatives staged per round
  constexpr int PR = DK + PAD;            // LDS row pitch (elements)
  constexpr int NU = RT * UPR / 256;      // 16-byte units per thread per round
  static_assert(NU >= 1 && (RT * UPR) % 256 == 0, "staging split");
  __shared__ __attribute__((aligned(16))) T sR[2][RT * PR];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int nqt = (a.N + 31) / 32, nqg = (nqt + 3) / 4, njs = (a.N + JSEG - 1) / JSEG;
  int64_t id = blockIdx.x;
  const int js = (int)(id % njs);
  id /= njs;
  const int qg = (int)(id % nqg);
  const int64_t bh = id / nqg, h = bh % a.H, b = bh / a.H;
  const int qt = qg * 4 + w;
  const int qi = qt * 32 + c32;
  const int grp_imax = (qg * 4 + 3) * 32 + 31 < a.N - 1 ? (qg * 4 + 3) * 32 + 31 : a.N - 1;
  const int wave_imax = qt * 32 + 31 < a.N - 1 ? qt * 32 + 31 : a.N - 1;
  const int j_lo = js * JSEG;
  const int j_hi = (j_lo + JSEG < grp_imax ? j_lo + JSEG : grp_imax);  // exclusive; j < i <= grp_imax
  if (j_lo >= j_hi) return;

  // B operand: query-chunk means (fp32 split into bf16 hi + lo on the bf16 path)
  const float* qb = a.qbar + (bh * a.N + (qi < a.N ? qi : 0)) * DK;
  constexpr int NKS = DK / MM::KS;
  typename MM::Frag bhi[NKS], blo[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if constexpr (sizeof(T) == 2) {
      bf16x8 fh, fl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = qi < a.N ? qb[ks * 16 + hh * 8 + e] : 0.f;
        const bf16 xh = (bf16)x;
        fh[e] = xh;
        fl[e] = (bf16)(x - (float)xh);
      }
      bhi[ks] = fh;
      blo[ks] = fl;
    } else {
      bhi[ks] = qi < a.N ? qb[ks * 2 + hh] : 0.f;
      blo[ks] = 0.f;
    }
  }
  const float scale = 1.f / sqrtf((float)DK);
  const T* reps = reinterpret_cast<const T*>(a.reps);
  const int nkt = (a.n_rep + RT - 1) / RT;
  // rounds = (history chunk, key tile of 32 representatives), staged in order
  const int nrounds = (j_hi - j_lo) * nkt;
  uint4 pf[NU];
  auto load_round = [&](int rd) {
    const int j = j_lo + rd / nkt, kt = rd % nkt;
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int uu = tid + 256 * m, r = uu / UPR, cu = uu % UPR;
      const int rr = kt * RT + r;
      pf[m] = make_uint4(0u, 0u, 0u, 0u);
      if (rr < a.n_rep)
        pf[m] = *reinterpret_cast<const uint4*>(reps + ((b * a.ld_R + (int64_t)j * a.n_rep + rr) * a.H + h) * DK +
                                                cu * PAD);
    }
  };
  auto store_round = [&](int buf) {
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int uu = tid + 256 * m, r = uu / UPR, cu = uu % UPR;
      *reinterpret_cast<uint4*>(&sR[buf][r * PR + cu * PAD]) = pf[m];
    }
  };
  load_round(0);
  store_round(0);
  __syncthreads();
  float m = -INFINITY, ssum = 0.f;
  for (int rd = 0; rd < nrounds; ++rd) {
    const int buf = rd & 1;
    const int j = j_lo + rd / nkt, kt = rd % nkt;
    if (rd + 1 < nrounds) load_round(rd + 1);
    if (j < wave_imax) {
      const T* arow = &sR[buf][c32 * PR];
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const auto af = MM::load_plain(arow, ks, hh);
        acc = MM::mma(af, bhi[ks], acc);
        if constexpr (sizeof(T) == 2) acc = MM::mma(af, blo[ks], acc);
      }
      // streaming log-mean-exp over the representatives this lane holds
      float sv[16], tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = kt * RT + acc_row(e, hh);
        sv[e] = rr < a.n_rep ? acc[e] * scale : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      const float mn = fmaxf(m, tmax);
      if (mn > -INFINITY) {
        float add = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) add += sv[e] > -INFINITY ? __expf(sv[e] - mn) : 0.f;
        ssum = (m > -INFINITY ? ssum * __expf(m - mn) : 0.f) + add;
        m = mn;
      }
      if (kt == nkt - 1) {
        // the other lane half holds the remaining rows of the same query column
        const float mo = __shfl_xor(m, 32, 64), so = __shfl_xor(ssum, 32, 64);
        const float mall = fmaxf(m, mo);
        const float stot = (m > -INFINITY ? ssum * __expf(m - mall) : 0.f) + (mo > -INFINITY ? so * __expf(mo - mall) : 0.f);
        const float l = mall + logf(stot / (float)a.n_rep);
        const float g = 1.f / (1.f + expf(-l));
        if (hh == 0 && qi < a.N && j < qi) a.gates[(bh * a.N + qi) * a.N + j] = g;
        m = -INFINITY;
        ssum = 0.f;
      }
    }
    if (rd + 1 < nrounds) {
      store_round(buf ^ 1);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- mask, lists, n_eff
// One wavefront per (b, h, query chunk i).
__global__ __launch_bounds__(64) void lists_kernel(RouteArgs a) {
  const int64_t row = blockIdx.x;  // (b, h, i)
  const int i = (int)(row % a.N);
  const int lane = threadIdx.x;
  const float* gsrc = a.gates_in ? a.gates_in : a.gates;
  float* grow = a.gates + row * a.N;
  uint8_t* mrow = a.mask + row * a.N;
  int32_t* arow = a.active_idx + row * a.N;
  int cnt = 0;
  float s1 = 0.f, s2 = 0.f;
  for (int j0 = 0; j0 < a.N; j0 += 64) {
    const int j = j0 + lane;
    float g = 0.f;
    bool keep = false;
    if (j < a.N) {
      if (j < i) {
        g = gsrc[row * a.N + j];
        keep = g >= a.tau;
      } else {
        g = (j == i) ? 1.f : 0.f;
      }
      grow[j] = g;
      mrow[j] = keep ? 1 : 0;
    }
    const uint64_t bal = __ballot(keep);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (keep) arow[cnt + pre] = j;
    cnt += __popcll(bal);
    const float gh = keep ? g : 0.f;
    s1 += gh;
    s2 += gh * gh;
  }
  for (int j = cnt + lane; j < a.N; j += 64) arow[j] = -1;
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) {
    a.active_cnt[row] = cnt;
    if (a.n_eff) a.n_eff[row] = s2 > 0.f ? (s1 * s1) / s2 : 0.f;
  }
}

// ---------------------------------------------------------------- gated composition
// Workgroup = (b, h, group of QG consecutive query chunks); 4 waves, wave w owns the dv
// column tile w % (DV/32) of two query chunks of the group.  Groups are dispatched longest
// chain first; the state of each query chunk stays in registers for the whole chain, and
// every history chunk's (At_j - I, Bc_j) is staged once in LDS for all chains of the group.
template <class T, int DK, int DV, int NBUF>
__global__ __launch_bounds__(256) void compose_kernel(RouteArgs a) {
  using MM = Mma<T>;
  constexpr int E = sizeof(T), PAD = 16 / E;
  constexpr int PA = DK + PAD, PB = DV + PAD;
  constexpr int NCTV = DV / 32;
  constexpr int SPW = 2;                 // query chunks per wave
  constexpr int QG = 4 * SPW / NCTV;     // query chunks per workgroup
  constexpr int NRT = DK / 32;
  constexpr int NKS = DK / MM::KS;
  constexpr int UA = DK / PAD, UB = DV / PAD;
  constexpr int NU = (DK * UA + DK * UB) / 256;  // 16-byte units per thread per step
  __shared__ __attribute__((aligned(16))) T sA[NBUF][DK * PA];
  __shared__ __attribute__((aligned(16))) T sB[NBUF][DK * PB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t BH = a.B * a.H;
  const int ng = (a.N + QG - 1) / QG;
  const int64_t id = blockIdx.x;
  const int64_t bh = id % BH;
  const int grp = ng - 1 - (int)(id / BH);
  const int i0 = grp * QG;
  const int i_hi = (i0 + QG < a.N ? i0 + QG : a.N) - 1;
  const int ct = w % NCTV;
  int qi[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) qi[s] = i0 + w / NCTV + s * (4 / NCTV);

  const T* Ag = reinterpret_cast<const T*>(a.At) + bh * a.N * (int64_t)DK * DK;
  const T* Bg = reinterpret_cast<const T*>(a.Bc) + bh * a.N * (int64_t)DK * DV;
  const float* grow_base = a.gates + bh * a.N * (int64_t)a.N;
  const uint8_t* mrow_base = a.mask + bh * a.N * (int64_t)a.N;
  float* Sout = a.S_routed + bh * a.N * (int64_t)DK * DV;

  f32x16 M[SPW][NRT];
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      M[s][rt] = zero16();
      if (a.S0) {
        const float* s0 = a.S0 + bh * (int64_t)DK * DV;
#pragma unroll
        for (int e = 0; e < 16; ++e) M[s][rt][e] = s0[(rt * 32 + acc_row(e, hh)) * DV + ct * 32 + c32];
      }
    }
  auto write_state = [&](int s) __attribute__((always_inline)) {
    float* dst = Sout + (int64_t)qi[s] * DK * DV;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[(rt * 32 + acc_row(e, hh)) * DV + ct * 32 + c32] = M[s][rt][e];
  };
#pragma unroll
  for (int s = 0; s < SPW; ++s)
    if (qi[s] == 0) write_state(s);
  const int nsteps = i_hi;  // history chunks j = 0 .. i_hi - 1

  uint4 pf[NU];
  auto load_step = [&](int j) __attribute__((always_inline)) {
    const uint4* asrc = reinterpret_cast<const uint4*>(Ag + (int64_t)j * DK * DK);
    const uint4* bsrc = reinterpret_cast<const uint4*>(Bg + (int64_t)j * DK * DV);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int idx = tid + 256 * u;
      pf[u] = idx < DK * UA ? asrc[idx] : bsrc[idx - DK * UA];
    }
  };
  auto store_step = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int idx = tid + 256 * u;
      if (idx < DK * UA) {
        const int row = idx / UA, cu = idx % UA;
        uint4 val = pf[u];
        if (cu == row / PAD) {  // this unit holds the diagonal element: store At - I
          T* ev = reinterpret_cast<T*>(&val);
          ev[row % PAD] = from_f<T>(to_f<T>(ev[row % PAD]) - 1.f);
        }
        *reinterpret_cast<uint4*>(&sA[buf][row * PA + cu * PAD]) = val;
      } else {
        const int i2 = idx - DK * UA, row = i2 / UB, cu = i2 % UB;
        *reinterpret_cast<uint4*>(&sB[buf][row * PB + cu * PAD]) = pf[u];
      }
    }
  };

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
    __syncthreads();
  }
  for (int j = 0; j < nsteps; ++j) {
    const int buf = NBUF == 2 ? (j & 1) : 0;
    if (NBUF == 2 && j + 1 < nsteps) load_step(j + 1);
    bool act[SPW];
    float g[SPW];
    bool any = false;
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      act[s] = qi[s] < a.N && j < qi[s] && mrow_base[(int64_t)qi[s] * a.N + j] != 0;
      g[s] = act[s] ? grow_base[(int64_t)qi[s] * a.N + j] : 0.f;
      any |= act[s];
    }
    if (any) {
      typename MM::Frag bfr[SPW][NKS];
#pragma unroll
      for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) bfr[s][ks] = MM::from_acc(M[s][ks / (32 / MM::KS)], ks, g[s]);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const T* arow = &sA[buf][(rt * 32 + c32) * PA];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const auto af = MM::load_clayout(arow, ks, hh);
#pragma unroll
          for (int s = 0; s < SPW; ++s)
            if (act[s]) M[s][rt] = MM::mma(af, bfr[s][ks], M[s][rt]);
        }
        const T* brow = &sB[buf][(rt * 32 + c32) * PB + ct * 32];
#pragma unroll
        for (int kd = 0; kd < 32 / MM::KS; ++kd) {
          const auto af = MM::load_plain(brow, kd, hh);
#pragma unroll
          for (int s = 0; s < SPW; ++s)
            if (act[s]) M[s][rt] = MM::mma(af, diag_frag<T>(kd, lane, g[s]), M[s][rt]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s)
      if (qi[s] == j + 1 && qi[s] < a.N) write_state(s);
    if (j + 1 < nsteps) {
      if (NBUF == 1) {
        __syncthreads();
        load_step(j + 1);
        store_step(0);
      } else {
        store_step((j + 1) & 1);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- launchers
template <class T, int DK, int DV>
static hipError_t launch_compose_t(const RouteArgs& a, hipStream_t s) {
  constexpr int E = sizeof(T), PAD = 16 / E;
  constexpr int bytes2 = 2 * (DK * (DK + PAD) + DK * (DV + PAD)) * E;
  constexpr int NBUF = bytes2 <= 150 * 1024 ? 2 : 1;
  constexpr int QG = 8 / (DV / 32);
  const int64_t ng = (a.N + QG - 1) / QG;
  const int64_t nb = ng * a.B * a.H;
  TimedLaunch tl(HLA_KERNEL_COMPOSE, s);
  hipLaunchKernelGGL((compose_kernel<T, DK, DV, NBUF>), dim3((unsigned)nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <class T, int DK, int DV>
static hipError_t launch_route_t(const RouteArgs& a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  if (BH == 0 || a.N == 0) return hipSuccess;
  {
    TimedLaunch tl(HLA_KERNEL_GATES, s);
    if (!a.gates_in && a.N > 1) {
      hipLaunchKernelGGL((qbar_kernel<T, DK>), dim3((unsigned)(BH * a.N)), dim3(256), 0, s, a);
      const int64_t nqt = (a.N + 31) / 32, nqg = (nqt + 3) / 4, seg = gate_seg(a.n_rep);
      const int64_t njs = (a.N + seg - 1) / seg;
      hipLaunchKernelGGL((gate_kernel<T, DK>), dim3((unsigned)(BH * nqg * njs)), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(lists_kernel, dim3((unsigned)(BH * a.N)), dim3(64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.S_routed) return e;  // no S_routed: gates, mask and lists only
  if constexpr (sizeof(T) == 2) return launch_compose_bf16(a, DK, DV, s);
  return launch_compose_t<T, DK, DV>(a, s);
}

template <class T>
static hipError_t launch_route_d(const RouteArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_route_t<T, 64, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_route_t<T, 64, 128>(a, s);
  if (dk == 128 && dv == 64) return launch_route_t<T, 128, 64>(a, s);
  return launch_route_t<T, 128, 128>(a, s);
}

hipError_t launch_route(const RouteArgs& a, int dtype, int dk, int dv, hipStream_t s) {
  return dtype == 1 ? launch_route_d<bf16>(a, dk, dv, s) : launch_route_d<float>(a, dk, dv, s);
}

}  // namespace hla
