// Single-token HLA decode step.
//
// [HLA] Key Contributions 3 (dynamic autoregressive decoding) and Methodology paragraphs
// 2-4.  Per (sequence b, head h), with the live chunk (At_cur, M_cur) of the tokens since
// the last cached chunk and Nc cached chunk summaries (At_j, Bc_j, representatives):
//   M_cur  <- alpha (I - beta k k^T) M_cur + beta k v^T           (gated delta rule)
//   At_cur <- alpha (I - beta k k^T) At_cur
//   g_j    = sigmoid(log-mean-exp_r(q . r / sqrt(dk))),  ghat_j = g_j [g_j >= tau]
//   y      = A_cur q = At_cur^T q
//   o      = M_cur^T q + S~ y  with S~ y evaluated backwards over the cache:
//            z <- y; for j = Nc-1 .. 0: o += ghat_j Bc_j^T z;  z <- z + ghat_j (At_j^T z - z)
// Everything is HBM-bound streaming: the live state and transition are read and written
// once (float4, coalesced); representatives and the cached (At_j, Bc_j) are read once with
// 16-byte loads, the next active chunk prefetched into registers during the current
// chunk's reduction.  Chunks with ghat_j = 0 are never read (the skip cuts memory traffic,
// [HLA] Methodology paragraph 4).
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

constexpr int kMaxCache = 1024;  // largest n_cap a decode call accepts

// A 16-byte non-temporal load.  The cached chunk maps are read once per step and the whole
// cache is far larger than L2 and the MALL, so the stream is kept from allocating there.
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The live state and transition of every (sequence, head) are read and written once per
// step, 1 GiB in all at the decode workload: non-temporal too.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
  const nt_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float* p, const float4& x) {
  const nt_f32x4 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4*>(p));
}

// Per-row token vectors of the Gated DeltaNet-2 live update (LDS): ka = k o a, qa = q o a,
// a, e = b o k; the write vector (w o v) is passed as s_v and qe = q . e.
struct G2Rows {
  const float* ka;
  const float* qa;
  const float* a;
  const float* e;
  float qe;
};

// One read + write pass over a live [DK][W] matrix `mat` (float32, row-major):
//   u = k^T mat, z0 = q^T mat
//   state      (IS_STATE): mat' = alpha mat + beta k (v - alpha u)^T,  out = q^T mat'
//   transition (else)    : mat' = alpha mat - alpha beta k u^T,        out = q^T mat'
// Gated DeltaNet-2 (G2): u = (k o a)^T mat, z0 = (q o a)^T mat and
//   mat' = diag(a) mat - e u^T (+ k (w o v)^T for the state),  out = z0 - qe u (+ qk (w o v)).
// With `commit`, mat' goes to the cache slot (cast to T) and mat is reset (0, or I).
template <class T, int DK, int W, bool IS_STATE, int NT, bool G2>
__device__ __forceinline__ void live_pass(float* mat, T* cache_out, bool commit, float alpha, float beta, float qk,
                          const float* s_q, const float* s_k, const float* s_v, float* red0, float* red1,
                          int red_size, float* s_u, float* out, const G2Rows& g2) {
  constexpr int CPR = W / 4, RPP = NT / CPR, NP = DK / RPP;
  const int tid = threadIdx.x;
  const int col = (tid % CPR) * 4, r0 = tid / CPR;
  float4 m[NP];
  float4 pu = make_float4(0.f, 0.f, 0.f, 0.f), pz = pu;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = p * RPP + r0;
    m[p] = load_stream(mat + r * W + col);
    const float kr = G2 ? g2.ka[r] : s_k[r], qr = G2 ? g2.qa[r] : s_q[r];
    pu.x += kr * m[p].x; pu.y += kr * m[p].y; pu.z += kr * m[p].z; pu.w += kr * m[p].w;
    pz.x += qr * m[p].x; pz.y += qr * m[p].y; pz.z += qr * m[p].z; pz.w += qr * m[p].w;
  }
  (void)red_size;
  *reinterpret_cast<float4*>(red0 + r0 * W + col) = pu;
  *reinterpret_cast<float4*>(red1 + r0 * W + col) = pz;
  __syncthreads();
  if (tid < W) {
    float u = 0.f, z = 0.f;
    for (int g2 = 0; g2 < RPP; ++g2) { u += red0[g2 * W + tid]; z += red1[g2 * W + tid]; }
    s_u[tid] = u;
    if constexpr (G2) out[tid] = z - g2.qe * u + (IS_STATE ? qk * s_v[tid] : 0.f);
    else if (IS_STATE) out[tid] = alpha * z + beta * qk * (s_v[tid] - alpha * u);
    else out[tid] = alpha * z - alpha * beta * qk * u;
  }
  __syncthreads();
  const float4 uu = *reinterpret_cast<const float4*>(&s_u[col]);
  float4 dd;
  if constexpr (G2) dd = IS_STATE ? *reinterpret_cast<const float4*>(&s_v[col]) : make_float4(0.f, 0.f, 0.f, 0.f);
  else if (IS_STATE) dd = make_float4(s_v[col] - alpha * uu.x, s_v[col + 1] - alpha * uu.y, s_v[col + 2] - alpha * uu.z, s_v[col + 3] - alpha * uu.w);
  else dd = make_float4(-alpha * uu.x, -alpha * uu.y, -alpha * uu.z, -alpha * uu.w);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = p * RPP + r0;
    float4 nm;
    if constexpr (G2) {
      const float ar = g2.a[r], er = g2.e[r], kr = s_k[r];
      nm.x = ar * m[p].x - er * uu.x + kr * dd.x;
      nm.y = ar * m[p].y - er * uu.y + kr * dd.y;
      nm.z = ar * m[p].z - er * uu.z + kr * dd.z;
      nm.w = ar * m[p].w - er * uu.w + kr * dd.w;
    } else {
      const float bk = beta * s_k[r];
      nm.x = alpha * m[p].x + bk * dd.x;
      nm.y = alpha * m[p].y + bk * dd.y;
      nm.z = alpha * m[p].z + bk * dd.z;
      nm.w = alpha * m[p].w + bk * dd.w;
    }
    if (commit) {
      T* cdst = cache_out + r * W + col;
      cdst[0] = from_f<T>(nm.x); cdst[1] = from_f<T>(nm.y); cdst[2] = from_f<T>(nm.z); cdst[3] = from_f<T>(nm.w);
      float4 rs = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!IS_STATE) {
        if (r == col) rs.x = 1.f;
        if (r == col + 1) rs.y = 1.f;
        if (r == col + 2) rs.z = 1.f;
        if (r == col + 3) rs.w = 1.f;
      }
      nm = rs;
    }
    store_stream(mat + r * W + col, nm);
  }
  __syncthreads();
}

// 512 threads per (sequence, head) and a two-deep register prefetch of the cached chunks
// fit in ~121 VGPRs, so two workgroups share a CU; every phase is a short dependent chain
// of loads and reductions, and the second workgroup keeps HBM busy meanwhile.
template <class T, int DK, int DV, int NT, int WPC, bool G2>
__global__ __launch_bounds__(NT, WPC) void decode_kernel(DecodeArgs a) {
  constexpr int E = sizeof(T), PAD = 16 / E;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / a.H;

  __shared__ float s_q[DK], s_k[DK], s_v[DV];
  __shared__ float s_u[DV > DK ? DV : DK], s_z[DK], s_o[DV], s_y[DK];
  constexpr int WMAX = DV > DK ? DV : DK;
  constexpr int R1_ = NT / ((DV < DK ? DV : DK) / 4), R2_ = NT / (DK / PAD), R3_ = NT / (DV / PAD);
  constexpr int RMAX = R1_ > R2_ ? (R1_ > R3_ ? R1_ : R3_) : (R2_ > R3_ ? R2_ : R3_);
  __shared__ float s_red[2][RMAX][WMAX];
  __shared__ float s_qk;
  __shared__ int s_nc;

  const T* qg = reinterpret_cast<const T*>(a.q) + bh * DK;
  const T* kg = reinterpret_cast<const T*>(a.k) + bh * DK;
  const T* vg = reinterpret_cast<const T*>(a.v) + bh * DV;
  if (tid < DK) {
    s_q[tid] = to_f<T>(qg[tid]);
    s_k[tid] = to_f<T>(kg[tid]);
  }
  if (tid < DV) s_v[tid] = to_f<T>(vg[tid]);
  // Gated DeltaNet-2 rows: ka = k o a, qa = q o a, a, e = b o k; s_v becomes w o v
  __shared__ float s_ka[G2 ? DK : 1], s_qa[G2 ? DK : 1], s_a[G2 ? DK : 1], s_e[G2 ? DK : 1];
  __shared__ float s_qe;
  if constexpr (G2) {
    if (tid < DK) {
      const float av = a.ga[bh * DK + tid], kv = s_k[tid];
      s_a[tid] = av;
      s_ka[tid] = kv * av;
      s_qa[tid] = s_q[tid] * av;
      s_e[tid] = a.gb[bh * DK + tid] * kv;
    }
    if (tid < DV) s_v[tid] *= a.gw[bh * DV + tid];
  }
  if (tid == 0) {
    int nc = 0;
    if (a.At_cur) {
      nc = a.n_cache[b];
      nc = nc < 0 ? 0 : (nc > a.n_cap ? a.n_cap : nc);
    }
    s_nc = nc;
  }
  __syncthreads();
  if (w == 0) {
    float x = 0.f;
    for (int i = lane; i < DK; i += 64) x += s_q[i] * s_k[i];
    x = wave_sum(x);
    if (lane == 0) s_qk = x;
  }
  if constexpr (G2) {
    if (w == 1) {
      float x = 0.f;
      for (int i = lane; i < DK; i += 64) x += s_q[i] * s_e[i];
      x = wave_sum(x);
      if (lane == 0) s_qe = x;
    }
  }
  const float alpha = G2 ? 0.f : a.alpha[bh], beta = G2 ? 0.f : a.beta[bh];
  const int nc = s_nc;
  const bool commit = a.commit && a.At_cur && nc < a.n_cap;
  __syncthreads();

  T* Acache = reinterpret_cast<T*>(a.At_cache);
  T* Bcache = reinterpret_cast<T*>(a.Bc_cache);
  const int64_t slot = bh * a.n_cap + nc;
  const G2Rows g2{s_ka, s_qa, s_a, s_e, G2 ? s_qe : 0.f};
  live_pass<T, DK, DV, true, NT, G2>(a.S_cur + bh * (int64_t)DK * DV, commit ? Bcache + slot * DK * DV : nullptr,
                                     commit, alpha, beta, s_qk, s_q, s_k, s_v, &s_red[0][0][0], &s_red[1][0][0],
                                     RMAX * WMAX, s_u, s_o, g2);
  if (!a.At_cur) {
    if (tid < DV) a.o[bh * DV + tid] = s_o[tid];
    return;
  }
  live_pass<T, DK, DK, false, NT, G2>(a.At_cur + bh * (int64_t)DK * DK, commit ? Acache + slot * DK * DK : nullptr,
                                      commit, alpha, beta, s_qk, s_q, s_k, s_v, &s_red[0][0][0], &s_red[1][0][0],
                                      RMAX * WMAX, s_u, s_y, g2);

  // ---- gates over the cached chunks (wave w takes chunks j = w, w + 4, ...)
  __shared__ float s_g[kMaxCache];
  __shared__ int s_keep[kMaxCache];
  const int ncap = a.n_cap;
  for (int j = w; j < nc; j += NT / 64) {
    float g;
    if (a.gates_in) {
      g = a.gates_in[bh * ncap + j];
    } else {
      constexpr int TPR = DK / PAD;      // lanes per representative row
      constexpr int RPI = 64 / TPR;      // rows per wave instruction
      const int grp = lane / TPR, sub = lane % TPR;
      const T* rep = reinterpret_cast<const T*>(a.reps_cache) + (bh * ncap + j) * (int64_t)a.n_rep * DK;
      float m = -INFINITY, ssum = 0.f;
      const float scale = 1.f / sqrtf((float)DK);
#pragma unroll 4
      for (int r0 = 0; r0 < a.n_rep; r0 += RPI) {
        const int r = r0 + grp;
        float part = 0.f;
        if (r < a.n_rep) {
          const uint4 raw = *reinterpret_cast<const uint4*>(rep + (int64_t)r * DK + sub * PAD);
          const T* ev = reinterpret_cast<const T*>(&raw);
#pragma unroll
          for (int e = 0; e < PAD; ++e) part += to_f<T>(ev[e]) * s_q[sub * PAD + e];
        }
        part = lane_group_sum<TPR>(part);  // the TPR lanes of a row are an aligned group
        if (r < a.n_rep) {
          const float s = part * scale;
          const float mn = fmaxf(m, s);
          ssum = (m > -INFINITY ? ssum * __expf(m - mn) : 0.f) + __expf(s - mn);
          m = mn;
        }
      }
      // combine the row groups of the wave (lanes with equal sub hold the same values); the
      // combine is symmetric, so each level takes the two values a lane move delivers
      auto combine = [&](float m1, float s1, float m2, float s2) {
        const float mn = fmaxf(m1, m2);
        ssum = (m1 > -INFINITY ? s1 * __expf(m1 - mn) : 0.f) + (m2 > -INFINITY ? s2 * __expf(m2 - mn) : 0.f);
        m = mn;
      };
      if constexpr (TPR <= 8) combine(m, ssum, dpp_f<0x128>(m), dpp_f<0x128>(ssum));  // 8 lanes apart
      if constexpr (TPR <= 16) {
        const auto rm = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, m), __builtin_bit_cast(unsigned, m), false, false);
        const auto rs = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, ssum), __builtin_bit_cast(unsigned, ssum), false, false);
        combine(__builtin_bit_cast(float, (unsigned)rm[0]), __builtin_bit_cast(float, (unsigned)rs[0]),
                __builtin_bit_cast(float, (unsigned)rm[1]), __builtin_bit_cast(float, (unsigned)rs[1]));
      }
      {
        const auto rm = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, m), __builtin_bit_cast(unsigned, m), false, false);
        const auto rs = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, ssum), __builtin_bit_cast(unsigned, ssum), false, false);
        combine(__builtin_bit_cast(float, (unsigned)rm[0]), __builtin_bit_cast(float, (unsigned)rs[0]),
                __builtin_bit_cast(float, (unsigned)rm[1]), __builtin_bit_cast(float, (unsigned)rs[1]));
      }
      g = 1.f / (1.f + expf(-(m + logf(ssum / (float)a.n_rep))));
    }
    if (lane == 0) {
      const bool keep = g >= a.tau;
      s_g[j] = keep ? g : 0.f;
      s_keep[j] = keep ? 1 : 0;
      if (a.gates_out) a.gates_out[bh * ncap + j] = g;
    }
  }
  if (a.gates_out)
    for (int j = nc + tid; j < ncap; j += NT) a.gates_out[bh * ncap + j] = 0.f;
  if (tid < DK) s_z[tid] = s_y[tid];
  __syncthreads();

  // ---- backward chain over the active cached chunks
  constexpr int TA = DK / PAD, RA = NT / TA, NPA = DK / RA;  // At: threads/row, rows/pass, passes
  constexpr int TB = DV / PAD, RB = NT / TB, NPB = DK / RB;
  uint4 ra0[NPA], rb0[NPB], ra1[NPA], rb1[NPB];
  auto load_chunk = [&](int j, uint4 (&ra)[NPA], uint4 (&rb)[NPB]) {
    const uint4* ap = reinterpret_cast<const uint4*>(Acache + (bh * ncap + j) * (int64_t)DK * DK);
    const uint4* bp = reinterpret_cast<const uint4*>(Bcache + (bh * ncap + j) * (int64_t)DK * DV);
#pragma unroll
    for (int p = 0; p < NPA; ++p) ra[p] = load_stream(ap + p * NT + tid);
#pragma unroll
    for (int p = 0; p < NPB; ++p) rb[p] = load_stream(bp + p * NT + tid);
  };
  auto next_active = [&](int j) {
    --j;
    while (j >= 0 && !s_keep[j]) --j;
    return j;
  };
  // o += ghat_j Bc_j^T z;  z <- z + ghat_j (At_j^T z - z)
  auto process = [&](int j, const uint4 (&ra)[NPA], const uint4 (&rb)[NPB]) {
    const float gj = s_g[j];
    const int ca = (tid % TA) * PAD, r0a = tid / TA;
    float pa[PAD];
#pragma unroll
    for (int e = 0; e < PAD; ++e) pa[e] = 0.f;
#pragma unroll
    for (int p = 0; p < NPA; ++p) {
      const float zr = s_z[p * RA + r0a];
      const T* ev = reinterpret_cast<const T*>(&ra[p]);
#pragma unroll
      for (int e = 0; e < PAD; ++e) pa[e] += zr * to_f<T>(ev[e]);
    }
#pragma unroll
    for (int e = 0; e < PAD; ++e) s_red[0][r0a][ca + e] = pa[e];
    const int cb = (tid % TB) * PAD, r0b = tid / TB;
    float pb[PAD];
#pragma unroll
    for (int e = 0; e < PAD; ++e) pb[e] = 0.f;
#pragma unroll
    for (int p = 0; p < NPB; ++p) {
      const float zr = s_z[p * RB + r0b];
      const T* ev = reinterpret_cast<const T*>(&rb[p]);
#pragma unroll
      for (int e = 0; e < PAD; ++e) pb[e] += zr * to_f<T>(ev[e]);
    }
#pragma unroll
    for (int e = 0; e < PAD; ++e) s_red[1][r0b][cb + e] = pb[e];
    __syncthreads();
    if (tid < DK) {
      float s = 0.f;
      for (int g2 = 0; g2 < RA; ++g2) s += s_red[0][g2][tid];
      s_z[tid] = s_z[tid] + gj * (s - s_z[tid]);
    } else if (tid - DK < DV) {
      const int c = tid - DK;
      float s = 0.f;
      for (int g2 = 0; g2 < RB; ++g2) s += s_red[1][g2][c];
      s_o[c] += gj * s;
    }
    __syncthreads();
  };
  int j = next_active(nc);
  if (j >= 0) load_chunk(j, ra0, rb0);
  while (j >= 0) {
    int jn = next_active(j);
    if (jn >= 0) load_chunk(jn, ra1, rb1);
    process(j, ra0, rb0);
    j = jn;
    if (j < 0) break;
    jn = next_active(j);
    if (jn >= 0) load_chunk(jn, ra0, rb0);
    process(j, ra1, rb1);
    j = jn;
  }
  if (tid < DV) a.o[bh * DV + tid] = s_o[tid];
}

__global__ void advance_cache_kernel(int32_t* n_cache, int32_t n_cap, int64_t Bs) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b < Bs) {
    const int n = n_cache[b];
    if (n >= 0 && n < n_cap) n_cache[b] = n + 1;
  }
}

template <class T, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int64_t nb = a.Bs * a.H;
  if (nb == 0) return hipSuccess;
  {
    TimedLaunch tl(HLA_KERNEL_DECODE, s);
    if (a.variant == 2)
      hipLaunchKernelGGL((decode_kernel<T, DK, DV, 512, 1, true>), dim3((unsigned)nb),
                         dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<T, DK, DV, 512, 1, false>), dim3((unsigned)nb),
                         dim3(512), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(a.commit && a.At_cur)) return e;
  hipLaunchKernelGGL(advance_cache_kernel, dim3((unsigned)((a.Bs + 255) / 256)), dim3(256), 0, s, a.n_cache,
                     a.n_cap, a.Bs);
  return hipGetLastError();
}

template <class T>
static hipError_t launch_decode_d(const DecodeArgs& a, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_decode_t<T, 64, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_decode_t<T, 64, 128>(a, s);
  if (dk == 128 && dv == 64) return launch_decode_t<T, 128, 64>(a, s);
  return launch_decode_t<T, 128, 128>(a, s);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int dk, int dv, hipStream_t s) {
  return dtype == 1 ? launch_decode_d<bf16>(a, dk, dv, s) : launch_decode_d<float>(a, dk, dv, s);
}

}  // namespace hla
