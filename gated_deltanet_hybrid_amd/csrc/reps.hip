// Learned chunk representatives (bf16 / fp32 MFMA).
//
// [HLA] Methodology paragraph 2: a completed chunk is cut into pooling windows of `window`
// consecutive tokens; self-attention runs inside each window over the window's keys, the
// token outputs are mean-pooled and a learned projection turns the pooled vector into one
// representative per window.  The router compares a projected query with them; that
// projection is folded in here, r' = Wr^T Wp pooled, so the router's plain query mean
// against r' gives (Wr qbar) . (Wp pooled).
//
// Two kernels:
//   pool    one wavefront per 32-token tile (every window of the tile; windows never cross
//           a tile since window divides 32, and tiles never cross a chunk since 32 divides
//           C).  Q^T, K^T = Wq X^T, Wk X^T and V = X Wv^T are MFMA products whose
//           accumulators feed the next products without leaving the lane: S^T = K Q^T, the
//           window softmax runs down each lane's column, O = P V, and the mean over a
//           window's rows is a sum inside the lane plus one exchange between lane halves.
//           bf16 weights are staged once per workgroup in LDS (rows padded by 16 bytes so
//           a 16-lane read phase hits distinct banks); every wave then works through its
//           tiles of the same head.  Output: pooled means, float32.
//   project one wavefront per 32 windows: Wp pooled, then Wr^T of that, both as MFMA
//           products with the float32 operand split into bf16 high and low parts; the
//           result goes through LDS so rows are stored as 16-byte runs.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

namespace {

constexpr int kPoolWaves = 8;
constexpr int kProjWaves = 4;

template <class T>
struct Split;  // float32 -> (hi, lo) operand fragments of one k-step
template <>
struct Split<bf16> {
  __device__ __forceinline__ static void from8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16 h = (bf16)x[e];
      hi[e] = h;
      lo[e] = (bf16)(x[e] - (float)h);
    }
  }
};

}  // namespace

template <class T, int DK, int WIN>
__global__ __launch_bounds__(kPoolWaves * 64) void reps_pool_kernel(RepsArgs a) {
  using MM = Mma<T>;
  constexpr bool STAGE = sizeof(T) == 2;   // bf16 weights live in LDS; fp32 ones are read from L2
  constexpr int PW = DK + 16 / sizeof(T);  // LDS row pitch (elements)
  constexpr int NFT = DK / 32;             // 32-row feature tiles
  constexpr int NKS = DK / MM::KS;         // k-steps over the features
  constexpr int NKT = 32 / MM::KS;         // k-steps over the 32 tokens of a tile
  constexpr int TPK = 32 / MM::KS;         // k-steps per 32-row accumulator tile
  constexpr int NWT = WIN <= 32 ? 32 / WIN : 1;  // windows per 32-token tile
  static_assert(32 % WIN == 0 || WIN == 64, "window divides the 32-token tile, or spans two");
  __shared__ __attribute__((aligned(16))) T sW[STAGE ? 3 * DK * PW : 8];

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / a.groups;
  const int grp = (int)(blockIdx.x % a.groups);
  const int64_t h = bh % a.H, b = bh / a.H;
  const int nrep = a.C / WIN;
  const int64_t nrows = (int64_t)a.N * nrep;              // windows of this head
  const int64_t ntiles = (int64_t)a.N * (a.C / 32);

  // matrix m: 0 = Wq, 1 = Wk, 2 = Wv, each [out, in]
  auto wsrc = [&](int m) {
    return reinterpret_cast<const T*>(m == 0 ? a.Wq : m == 1 ? a.Wk : a.Wv) + h * a.w_hstride;
  };
  if constexpr (STAGE) {
    constexpr int UPR = DK * (int)sizeof(T) / 16;  // 16-byte units per row
    for (int i = tid; i < 3 * DK * UPR; i += kPoolWaves * 64) {
      const int m = i / (DK * UPR), r = (i / UPR) % DK, u = i % UPR;
      *reinterpret_cast<uint4*>(&sW[(m * DK + r) * PW + u * (16 / sizeof(T))]) =
          *reinterpret_cast<const uint4*>(wsrc(m) + (int64_t)r * DK + u * (16 / sizeof(T)));
    }
    __syncthreads();
  }
  // weight fragment: row `row` of matrix m, k-step ks, plain order
  auto wfrag = [&](int m, int row, int ks) -> typename MM::Frag {
    if constexpr (STAGE) return MM::load_plain(&sW[(m * DK + row) * PW], ks, hh);
    else return MM::load_plain(wsrc(m) + (int64_t)row * DK, ks, hh);
  };
  const float qscale = 1.f / sqrtf((float)DK);

  if constexpr (WIN == 64) {
    // One wavefront per 64-token window: two 32-token tiles a (keys) and b (queries).
    // S^T_ab = K_a Q_b^T; the softmax of query column t runs over the rows of S^T_0b and
    // S^T_1b (and the partner lane half); O_b = sum_a P_ab V_a, and the window mean is the
    // sum over the rows of O_0 and O_1 over the valid tokens.
    const int64_t nwin = (int64_t)a.N * (a.C / 64);
    for (int64_t tw = (int64_t)grp * kPoolWaves + w; tw < nwin; tw += (int64_t)a.groups * kPoolWaves) {
      const int64_t t0 = tw * 64;
      const int64_t cend = ((t0 / a.C) + 1) * a.C < a.T ? ((t0 / a.C) + 1) * a.C : a.T;
      const int nv = (int)(cend - t0 < 0 ? 0 : (cend - t0 < 64 ? cend - t0 : 64));  // valid tokens
      float* prow = a.pooled + (bh * nrows + tw) * DK;
      if (nv == 0) {
        for (int i = lane; i < DK; i += 64) prow[i] = 0.f;
        continue;
      }
      // X fragments of tile a: lane column = token 32 a + c32 (zero beyond the valid tokens).
      // Each use loads them again (from L1 / L2): the opaque token keeps the compiler from
      // holding both tiles in registers across the whole window.
      auto load_x = [&](int at, typename MM::Frag (&xf)[NKS]) {
        int tok = 32 * at + c32;
        asm volatile("" : "+v"(tok));
        const T* xr = reinterpret_cast<const T*>(a.k) + ((b * a.ld_T + t0 + (tok < nv ? tok : 0)) * a.H + h) * DK;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          xf[ks] = MM::load_plain(xr, ks, hh);
          if (tok >= nv) xf[ks] = typename MM::Frag{};
        }
      };
      // W X_a^T [feature][token] as operand fragments over the features (m: 0 = Wq, 1 = Wk)
      auto proj = [&](int m, const typename MM::Frag (&xf)[NKS], typename MM::Frag (&out)[NKS], float scale) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          f32x16 acc = zero16();
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc = MM::mma(wfrag(m, ft * 32 + c32, ks), xf[ks], acc);
#pragma unroll
          for (int j = 0; j < TPK; ++j) out[ft * TPK + j] = MM::from_acc(acc, ft * TPK + j, scale);
        }
      };
      typename MM::Frag pf[2][2][NKT];  // [a][b]: P_ab as A fragments over the keys of tile a
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        // S^T_ab for both key tiles (K_a formed again for each query tile: fewer registers)
        f32x16 p[2];
        {
          typename MM::Frag qf[NKS];
          {
            typename MM::Frag xf[NKS];
            load_x(bt, xf);
            proj(0, xf, qf, qscale);
          }
#pragma unroll
          for (int at = 0; at < 2; ++at) {
            typename MM::Frag xf[NKS], kf[NKS];
            load_x(at, xf);
            proj(1, xf, kf, 1.f);
            p[at] = zero16();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) p[at] = MM::mma(kf[ks], qf[ks], p[at]);
          }
        }
        // softmax of query column t over the valid keys s of both key tiles
        float mx = -INFINITY;
#pragma unroll
        for (int at = 0; at < 2; ++at)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * at + acc_row(e, hh) < nv) mx = fmaxf(mx, p[at][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        float sum = 0.f;
#pragma unroll
        for (int at = 0; at < 2; ++at)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            p[at][e] = 32 * at + acc_row(e, hh) < nv ? __expf(p[at][e] - mx) : 0.f;
            sum += p[at][e];
          }
        sum += __shfl_xor(sum, 32, 64);
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
        for (int at = 0; at < 2; ++at) {
#pragma unroll
          for (int e = 0; e < 16; ++e) p[at][e] *= inv;
#pragma unroll
          for (int ks = 0; ks < NKT; ++ks) pf[at][bt][ks] = MM::from_acc(p[at], ks, 1.f);
        }
      }
      // V_a per feature tile, O_b = sum_a P_ab V_a, then the mean over the valid query rows
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        f32x16 o[2] = {zero16(), zero16()};
#pragma unroll
        for (int at = 0; at < 2; ++at) {
          typename MM::Frag xf[NKS];
          load_x(at, xf);
          f32x16 v = zero16();
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) v = MM::mma(xf[ks], wfrag(2, ft * 32 + c32, ks), v);
#pragma unroll
          for (int bt = 0; bt < 2; ++bt)
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) o[bt] = MM::mma(pf[at][bt][ks], MM::from_acc(v, ks, 1.f), o[bt]);
        }
        float sacc = 0.f;
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * bt + acc_row(e, hh) < nv) sacc += o[bt][e];
        sacc += __shfl_xor(sacc, 32, 64);
        if (hh == 0) prow[ft * 32 + c32] = sacc / (float)nv;
      }
    }
    return;
  }

  for (int64_t tt = (int64_t)grp * kPoolWaves + w; tt < ntiles; tt += (int64_t)a.groups * kPoolWaves) {
    const int64_t t0 = tt * 32;
    const int64_t cend = ((t0 / a.C) + 1) * a.C < a.T ? ((t0 / a.C) + 1) * a.C : a.T;
    const int nv = (int)(cend - t0 < 0 ? 0 : (cend - t0 < 32 ? cend - t0 : 32));  // valid tokens
    float* prow = a.pooled + (bh * nrows + t0 / WIN) * DK;
    if (nv == 0) {
      for (int i = lane; i < NWT * DK; i += 64) prow[i] = 0.f;
      continue;
    }
    // X fragments: lane column = token c32 (zero beyond the valid tokens)
    typename MM::Frag xf[NKS];
    {
      const T* xr = reinterpret_cast<const T*>(a.k) + ((b * a.ld_T + t0 + (c32 < nv ? c32 : 0)) * a.H + h) * DK;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        xf[ks] = MM::load_plain(xr, ks, hh);
        if (c32 >= nv) xf[ks] = typename MM::Frag{};
      }
    }
    // K^T and Q^T tiles [feature][token] -> operand fragments over the features
    typename MM::Frag kf[NKS], qf[NKS];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = MM::mma(wfrag(which == 0 ? 1 : 0, ft * 32 + c32, ks), xf[ks], acc);
#pragma unroll
        for (int j = 0; j < TPK; ++j) {
          if (which == 0) kf[ft * TPK + j] = MM::from_acc(acc, ft * TPK + j, 1.f);
          else qf[ft * TPK + j] = MM::from_acc(acc, ft * TPK + j, qscale);
        }
      }
    }
    // S^T [key token s][query token t]: lane column t, rows s
    f32x16 p = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) p = MM::mma(kf[ks], qf[ks], p);
    // softmax over s inside t's window; the other 16 rows sit in the partner lane half
    {
      const int wt = c32 / WIN;
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = acc_row(e, hh);
        if (s / WIN == wt && s < nv) mx = fmaxf(mx, p[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = acc_row(e, hh);
        p[e] = (s / WIN == wt && s < nv) ? __expf(p[e] - mx) : 0.f;
        sum += p[e];
      }
      sum += __shfl_xor(sum, 32, 64);
      const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] *= inv;
    }
    typename MM::Frag pf[NKT];
#pragma unroll
    for (int ks = 0; ks < NKT; ++ks) pf[ks] = MM::from_acc(p, ks, 1.f);
    // V [token][feature] per feature tile, then O = P V and the window means of O's rows
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      f32x16 v = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) v = MM::mma(xf[ks], wfrag(2, ft * 32 + c32, ks), v);
      f32x16 o = zero16();
#pragma unroll
      for (int ks = 0; ks < NKT; ++ks) o = MM::mma(pf[ks], MM::from_acc(v, ks, 1.f), o);
      // lane column = feature ft*32 + c32, element e is token row acc_row(e, hh); the
      // partner lane half holds the tile's other 16 rows
#pragma unroll
      for (int wl = 0; wl < NWT; ++wl) {
        float sacc = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = acc_row(e, hh);
          if (t / WIN == wl && t < nv) sacc += o[e];
        }
        sacc += __shfl_xor(sacc, 32, 64);
        const int nw = nv - wl * WIN < 0 ? 0 : (nv - wl * WIN < WIN ? nv - wl * WIN : WIN);
        if (hh == 0) prow[wl * DK + ft * 32 + c32] = nw > 0 ? sacc / (float)nw : 0.f;
      }
    }
  }
}

// rows r0 .. r0+31 of one head: out = Wr^T (Wp pooled) (or Wp pooled without Wr)
template <class T, int DK>
__global__ __launch_bounds__(kProjWaves * 64) void reps_project_kernel(RepsArgs a) {
  using MM = Mma<T>;
  constexpr int NFT = DK / 32, NKS = DK / MM::KS, TPK = 32 / MM::KS;
  constexpr int PO = DK + 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) T sO[kProjWaves][32 * PO];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nrows = (int64_t)a.N * (a.C / a.window);
  const int64_t blocks_per_head = (nrows + 32 * kProjWaves - 1) / (32 * kProjWaves);
  const int64_t bh = blockIdx.x / blocks_per_head;
  const int64_t r0 = (blockIdx.x % blocks_per_head) * (32 * kProjWaves) + w * 32;
  const int64_t h = bh % a.H, b = bh / a.H;
  if (r0 >= nrows) return;
  const int nr = (int)(nrows - r0 < 32 ? nrows - r0 : 32);
  const T* Wp = reinterpret_cast<const T*>(a.Wp) + h * a.w_hstride;
  const T* Wr = a.Wr ? reinterpret_cast<const T*>(a.Wr) + h * a.w_hstride : nullptr;

  // B operand: pooled row c32 (features, plain order), float32 split into hi + lo
  const float* prow = a.pooled + (bh * nrows + r0 + (c32 < nr ? c32 : 0)) * DK;
  f32x16 d1[NFT];
#pragma unroll
  for (int mt = 0; mt < NFT; ++mt) d1[mt] = zero16();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    typename MM::Frag bh_, bl_;
    if constexpr (sizeof(T) == 2) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = c32 < nr ? prow[ks * 16 + hh * 8 + e] : 0.f;
      Split<bf16>::from8(x, bh_, bl_);
    } else {
      bh_ = c32 < nr ? prow[ks * 2 + hh] : 0.f;
    }
#pragma unroll
    for (int mt = 0; mt < NFT; ++mt) {
      const typename MM::Frag af = MM::load_plain(Wp + (int64_t)(mt * 32 + c32) * DK, ks, hh);
      d1[mt] = MM::mma(af, bh_, d1[mt]);
      if constexpr (sizeof(T) == 2) d1[mt] = MM::mma(af, bl_, d1[mt]);
    }
  }
  if (Wr) {
    f32x16 d2[NFT];
    // A operand Wr^T: lane row k = kt*32 + c32, slots in the accumulator's k order over m
#pragma unroll
    for (int kt = 0; kt < NFT; ++kt) d2[kt] = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f32x16& src = d1[ks / TPK];
      typename MM::Frag bhi, blo;
      if constexpr (sizeof(T) == 2) {
        float x[8];
        const int base = (ks & 1) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = src[base + e];
        Split<bf16>::from8(x, bhi, blo);
      } else {
        bhi = src[ks & 15];
      }
#pragma unroll
      for (int kt = 0; kt < NFT; ++kt) {
        typename MM::Frag af;
        const int kcol = kt * 32 + c32;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) af[e] = Wr[(int64_t)clayout_k<bf16>(ks, hh, e) * DK + kcol];
        } else {
          af = Wr[(int64_t)clayout_k<float>(ks, hh, 0) * DK + kcol];
        }
        d2[kt] = MM::mma(af, bhi, d2[kt]);
        if constexpr (sizeof(T) == 2) d2[kt] = MM::mma(af, blo, d2[kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < NFT; ++kt) d1[kt] = d2[kt];
  }
  // rows (features) of d1 are the output's columns; lane column c32 = window row
  T* so = sO[w];
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
    for (int e = 0; e < 16; ++e) so[c32 * PO + ft * 32 + acc_row(e, hh)] = from_f<T>(d1[ft][e]);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  constexpr int UPR = DK * (int)sizeof(T) / 16;
  T* out = reinterpret_cast<T*>(a.reps);
  for (int i = lane; i < nr * UPR; i += 64) {
    const int r = i / UPR, u = i % UPR;
    *reinterpret_cast<uint4*>(out + ((b * nrows + r0 + r) * a.H + h) * DK + u * (16 / sizeof(T))) =
        *reinterpret_cast<const uint4*>(so + r * PO + u * (16 / sizeof(T)));
  }
}

template <class T, int DK>
static hipError_t launch_reps_t(RepsArgs a, hipStream_t s) {
  const int64_t BH = a.B * a.H;
  const int64_t ntiles = (int64_t)a.N * (a.C / 32);
  // about one workgroup per CU in all, each wave with several tiles of one head
  int64_t g = (256 + BH - 1) / BH;
  const int64_t gmax = (ntiles + kPoolWaves - 1) / kPoolWaves;
  a.groups = (int32_t)(g < gmax ? g : gmax);
  {
    TimedLaunch tl(HLA_KERNEL_REPS, s);
    const dim3 grid((unsigned)(BH * a.groups)), block(kPoolWaves * 64);
    switch (a.window) {
      case 8: hipLaunchKernelGGL((reps_pool_kernel<T, DK, 8>), grid, block, 0, s, a); break;
      case 16: hipLaunchKernelGGL((reps_pool_kernel<T, DK, 16>), grid, block, 0, s, a); break;
      case 64: hipLaunchKernelGGL((reps_pool_kernel<T, DK, 64>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((reps_pool_kernel<T, DK, 32>), grid, block, 0, s, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrows = (int64_t)a.N * (a.C / a.window);
  const int64_t bph = (nrows + 32 * kProjWaves - 1) / (32 * kProjWaves);
  hipLaunchKernelGGL((reps_project_kernel<T, DK>), dim3((unsigned)(BH * bph)), dim3(kProjWaves * 64), 0, s, a);
  return hipGetLastError();
}

// The window means of hla_chunk_reps_noalloc, for callers that cannot allocate: a fixed
// array in device memory, one per GPU the library runs on, held until the process ends.
// Every call on a GPU shares that GPU's copy (calls that overlap on one GPU race); the
// pooling kernel writes every row of it before the projection reads any, so nothing needs
// clearing between calls.
static __device__ __align__(256) float scratch[kRepsScratchBytes / 4];

hipError_t reps_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the host-side name of the array is no device address: ask the runtime for this
    // device's copy, with the device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

hipError_t launch_reps(const RepsArgs& a, int dtype, int dk, hipStream_t s) {
  if (dtype == 1) return dk == 64 ? launch_reps_t<bf16, 64>(a, s) : launch_reps_t<bf16, 128>(a, s);
  return dk == 64 ? launch_reps_t<float, 64>(a, s) : launch_reps_t<float, 128>(a, s);
}

}  // namespace hla
