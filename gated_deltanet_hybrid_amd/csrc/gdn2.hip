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

hipError_t launch_gdn2_chunk(const ChunkArgs& a, int dtype, int dk, int dv, bool want_o, hipStream_t s) {
  if (dtype == 1) return want_o ? launch_gdn2_d<bf16, true>(a, dk, dv, s) : launch_gdn2_d<bf16, false>(a, dk, dv, s);
  return want_o ? launch_gdn2_d<float, true>(a, dk, dv, s) : launch_gdn2_d<float, false>(a, dk, dv, s);
}

}  // namespace hla
