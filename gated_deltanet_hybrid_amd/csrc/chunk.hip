// Per-chunk kernel: the UT form of one chunk of the gated delta rule.
//
// [HLA] Methodology paragraph 1 / Key Contributions 2: a chunk is summarised exactly by the
// affine map M -> At M + Bc (state orientation M = S^T [dk, dv]).  Within a chunk of n <= 64
// tokens (local t, padded to 64 with beta = 0, alpha = 1, which is the identity map):
//   g_t = sum_{s<=t} log alpha_s,  gamma_t = exp(g_t),  Gamma_ts = exp(g_t - g_s) (s <= t)
//   L   = strictly_lower(diag(beta) (K K^T) o Gamma),  X = (I + L)^-1
//   W   = X diag(beta gamma) K,  U = X diag(beta) V,  D_s = exp(g_63 - g_s)
//   At  = gamma_63 I - K^T diag(D) W,   Bc = K^T diag(D) U
//   P   = (Q K^T) o Gamma (lower, with diagonal),  Qp = diag(gamma) Q - P W,  O_intra = P U
//   O   = O_intra + Qp M0 for a chunk that starts from state M0.
// Every decay is the exp of a difference of per-chunk log-decays (never exp(-g)), so nothing
// overflows when the product of alphas underflows.
//
// One 256/512-thread workgroup per (b, h, chunk).  Products run on MFMA (bf16 inputs with
// fp32 accumulation, or fp32 MFMA for fp32 inputs).  The inverse is blocked (16 x 16
// diagonal blocks by substitution, then the blocks below them by sub-diagonal) in fp32; its
// bf16 use is split into hi + lo parts so W and U keep ~16 mantissa bits.
#include "common.hpp"
#include "kernels.hpp"
#include "timing.hpp"

namespace hla {

template <class T, int DK, int DV, int NW, bool WANT_AB, bool WANT_O, bool AUXIN>
__global__ __launch_bounds__(NW * 64) void chunk_kernel(ChunkArgs a) {
  // AUXIN: the output pass takes W | U from a.aux_in and skips the UT transform
  static_assert(!AUXIN || (WANT_O && !WANT_AB && sizeof(T) == 2), "W | U hand-off is an output-pass, bf16 option");
  using MM = Mma<T>;
  constexpr int C = kChunk;
  constexpr int E = sizeof(T);
  constexpr int PAD = 16 / E;
  constexpr int PK = DK + PAD;  // pitch of [t][dk] rows (elements)
  constexpr int PT = C + PAD;   // pitch of [d][t] rows
  constexpr int PX = C + 4;     // fp32 pitch of L and X
  constexpr int NCT = (DK + DV) / 32;
  constexpr int NT = NW * 64;
  constexpr int R1a = (WANT_O ? 2 : 1) * C * PK * E;
  constexpr int R1b = 2 * C * PX * 4;
  constexpr int R1 = R1a > R1b ? R1a : R1b;
  // R2 holds K^T, V^T for the UT transform, then S~^T; an output pass that takes W | U
  // from the hand-off needs only the latter (two workgroups fit in one CU's LDS)
  constexpr int R2 = AUXIN ? DV * PK * E : (DK + DV) * PT * E;
  constexpr int R3 = WANT_O ? C * PT * E : 16;
  static_assert(!WANT_O || DV * PK * E <= R2, "S~^T staging must fit in R2");
  static_assert(!WANT_O || C * PK * E <= R1, "Qp staging must fit in R1");
  static_assert(NCT <= 2 * NW, "at most two column tiles per wave");

  __shared__ __attribute__((aligned(16))) char sm1[R1];
  __shared__ __attribute__((aligned(16))) char sm2[R2];
  __shared__ __attribute__((aligned(16))) char sm3[R3];
  // per token: beta, cumulative log decay g (in log2 units: pairwise decays are one exp2),
  // gamma = exp(g), beta gamma, D = exp(g_63 - g)
  __shared__ __attribute__((aligned(16))) float s_beta[C], s_g[C], s_gam[C], s_bg[C];
  __shared__ float s_d[WANT_AB ? C : 1];  // (an output pass keeps two workgroups per CU)

  T* Kp = reinterpret_cast<T*>(sm1);
  T* Qp = Kp + C * PK;
  float* Lb = reinterpret_cast<float*>(sm1);
  float* Xb = Lb + C * PX;
  T* KT = reinterpret_cast<T*>(sm2);
  T* VT = KT + DK * PT;
  T* Pb = reinterpret_cast<T*>(sm3);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, c32 = lane & 31;
  const int64_t id = blockIdx.x;
  const int c = (int)(id % a.N);
  const int64_t bh = id / a.N;
  const int64_t h = bh % a.H, b = bh / a.H;
  const int64_t t0 = (int64_t)c * C;
  const int n = (int)((a.T - t0) < C ? (a.T - t0) : C);
  const int64_t row0 = (b * a.ld_T + t0) * a.H + h;  // token-row of (b, t0, h)
  const T* kg = reinterpret_cast<const T*>(a.k) + row0 * DK;
  const T* vg = reinterpret_cast<const T*>(a.v) + row0 * DV;
  const T* qg = WANT_O ? reinterpret_cast<const T*>(a.q) + row0 * DK : nullptr;
  const int64_t kstride = a.H * DK, vstride = a.H * DV;

  // ---- 1. stage K (row-major and transposed), V (transposed), Q (row-major)
  {
    constexpr int VK = DK / PAD;
    for (int i = tid; i < C * VK; i += NT) {
      const int t = i / VK, cc = i % VK;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (t < n) val = *reinterpret_cast<const uint4*>(kg + t * kstride + cc * PAD);
      *reinterpret_cast<uint4*>(Kp + t * PK + cc * PAD) = val;
      if constexpr (sizeof(T) == 4) {
        const T* ev = reinterpret_cast<const T*>(&val);
#pragma unroll
        for (int e = 0; e < PAD; ++e) KT[(cc * PAD + e) * PT + t] = ev[e];
      }
      if constexpr (WANT_O) {
        uint4 qv = make_uint4(0u, 0u, 0u, 0u);
        if (t < n) qv = *reinterpret_cast<const uint4*>(qg + t * kstride + cc * PAD);
        *reinterpret_cast<uint4*>(Qp + t * PK + cc * PAD) = qv;
      }
    }
    if constexpr (sizeof(T) == 4) {
      constexpr int VV = DV / PAD;
      for (int i = tid; i < C * VV; i += NT) {
        const int t = i / VV, cc = i % VV;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (t < n) val = *reinterpret_cast<const uint4*>(vg + t * vstride + cc * PAD);
        const T* ev = reinterpret_cast<const T*>(&val);
#pragma unroll
        for (int e = 0; e < PAD; ++e) VT[(cc * PAD + e) * PT + t] = ev[e];
      }
    } else if constexpr (!AUXIN) {
      // K^T and V^T by 8 x 8 register transposes: task (token block tb, column block db)
      // loads 8 tokens x 8 columns and writes 8 rows of 8 tokens.  tb runs fastest, so the
      // 8 lanes of a write phase hit rows (8 db + e) at token blocks 0..7: 16-byte units
      // e * (PT / 8) + tb, distinct modulo 8 because PT / 8 is odd.
      static_assert((PT / 8) % 2 == 1, "odd row pitch in 16-byte units");
      constexpr int NTB = C / 8, NDK = DK / 8, NDV = DV / 8;
      for (int i = tid; i < NTB * (NDK + NDV); i += NT) {
        const int tb = i % NTB, dball = i / NTB;
        const bool isk = dball < NDK;
        const int db = isk ? dball : dball - NDK;
        const T* src = (isk ? kg + db * 8 : vg + db * 8);
        const int64_t stride = isk ? kstride : vstride;
        uint4 in[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = tb * 8 + r;
          in[r] = t < n ? *reinterpret_cast<const uint4*>(src + t * stride) : make_uint4(0u, 0u, 0u, 0u);
        }
        T* dst = (isk ? KT : VT) + db * 8 * PT + tb * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // tokens (2m, 2m + 1) of column e: the 16-bit half e & 1 of word e / 2
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const int wd = e >> 1;
          auto word = [&](const uint4& u) { return wd == 0 ? u.x : wd == 1 ? u.y : wd == 2 ? u.z : u.w; };
          uint4 o;
          o.x = __builtin_amdgcn_perm(word(in[1]), word(in[0]), sel);
          o.y = __builtin_amdgcn_perm(word(in[3]), word(in[2]), sel);
          o.z = __builtin_amdgcn_perm(word(in[5]), word(in[4]), sel);
          o.w = __builtin_amdgcn_perm(word(in[7]), word(in[6]), sel);
          *reinterpret_cast<uint4*>(dst + e * PT) = o;
        }
      }
    }
    if (tid < C) {
      float bt = 0.f, la = 0.f;
      if (tid < n) {
        const int64_t idx = row0 + (int64_t)tid * a.H;
        bt = a.beta[idx];
        la = logf(fmaxf(a.alpha[idx], 1.17549435e-38f));  // alpha = 0 (a reset) stays finite
      }
      float x = la;  // inclusive prefix sum over the 64 lanes of wave 0
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float gam = expf(x), g_end = __shfl(x, 63, 64);
      s_beta[tid] = bt;
      s_g[tid] = x * 1.4426950408889634f;  // log2(e)
      s_gam[tid] = gam;
      s_bg[tid] = bt * gam;
      if constexpr (WANT_AB) s_d[tid] = expf(g_end - x);
    }
  }
  __syncthreads();

  // ---- 2. K K^T and Q K^T tiles (64 x 64 each, 32 x 32 tiles)
  f32x16 kk = zero16(), qk = zero16();
  int kk_tile = -1, qk_tile = -1;
  if (AUXIN) {
    qk_tile = w < 4 ? w : -1;
  } else if (NW == 8) {
    if (w < 4) kk_tile = w; else qk_tile = WANT_O ? w - 4 : -1;
  } else {
    kk_tile = w;
    qk_tile = WANT_O ? w : -1;
  }
  if (kk_tile >= 0 && (kk_tile & 1) <= (kk_tile >> 1)) {
    const T* ar = Kp + ((kk_tile >> 1) * 32 + c32) * PK;
    const T* br = Kp + ((kk_tile & 1) * 32 + c32) * PK;
#pragma unroll
    for (int ks = 0; ks < DK / MM::KS; ++ks) kk = MM::mma(MM::load_plain(ar, ks, hh), MM::load_plain(br, ks, hh), kk);
  }
  if constexpr (WANT_O) {
    if (qk_tile >= 0 && (qk_tile & 1) <= (qk_tile >> 1)) {
      const T* ar = Qp + ((qk_tile >> 1) * 32 + c32) * PK;
      const T* br = Kp + ((qk_tile & 1) * 32 + c32) * PK;
#pragma unroll
      for (int ks = 0; ks < DK / MM::KS; ++ks) qk = MM::mma(MM::load_plain(ar, ks, hh), MM::load_plain(br, ks, hh), qk);
    }
  }
  __syncthreads();  // Kp and Qp are dead: R1 now holds L and X
  if (kk_tile >= 0) {
    const int tm = kk_tile >> 1, tn = kk_tile & 1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = tm * 32 + acc_row(e, hh), s = tn * 32 + c32;
      Lb[t * PX + s] = (s < t) ? s_beta[t] * __builtin_amdgcn_exp2f(s_g[t] - s_g[s]) * kk[e] : 0.f;
    }
  }
  if constexpr (WANT_O) {
    if (qk_tile >= 0) {
      const int tm = qk_tile >> 1, tn = qk_tile & 1;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = tm * 32 + acc_row(e, hh), s = tn * 32 + c32;
        Pb[t * PT + s] = from_f<T>((s <= t) ? __builtin_amdgcn_exp2f(s_g[t] - s_g[s]) * qk[e] : 0.f);
      }
    }
  }
  if constexpr (!AUXIN)
    for (int i = tid; i < C * PX; i += NT) Xb[i] = 0.f;
  __syncthreads();

  // ---- 3. X = (I + L)^-1, blocked by 16
  if constexpr (!AUXIN) {
  if (tid < 64) {
    const int bi = tid >> 4, cc = tid & 15, base = bi * 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int q2 = 0; q2 < r; ++q2) s -= Lb[(base + r) * PX + base + q2] * x[q2];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Xb[(base + r) * PX + base + cc] = x[r];
  }
  __syncthreads();
  // Off-diagonal blocks, from (I + L) X = I by blocks: X_ik = -X_ii sum_{m=k}^{i-1} L_im X_mk
  // = sum_m Z_im X_mk with Z_im = -X_ii L_im.  Z of the six blocks below the diagonal comes
  // first (all at once), into L's block (m, i) above the diagonal, which nothing reads;
  // then X by sub-diagonal d = i - k, each from the ones before it.
#pragma unroll
  for (int e = tid; e < 6 * 256; e += NT) {
    const int bz = e >> 8, r = (e >> 4) & 15, cc = e & 15;
    const int i = bz < 1 ? 1 : (bz < 3 ? 2 : 3), m = bz - i * (i - 1) / 2;  // block (i, m), m < i
    float z = 0.f;
#pragma unroll
    for (int q2 = 0; q2 < 16; ++q2) z -= Xb[(i * 16 + r) * PX + i * 16 + q2] * Lb[(i * 16 + q2) * PX + m * 16 + cc];
    Lb[(m * 16 + r) * PX + i * 16 + cc] = z;
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
#pragma unroll
    for (int e = tid; e < (4 - d) * 256; e += NT) {
      const int k = e >> 8, i = k + d, r = (e >> 4) & 15, cc = e & 15;
      float x = 0.f;
      for (int m = k; m < i; ++m)
#pragma unroll
        for (int q2 = 0; q2 < 16; ++q2) x += Lb[(m * 16 + r) * PX + i * 16 + q2] * Xb[(m * 16 + q2) * PX + k * 16 + cc];
      Xb[(i * 16 + r) * PX + k * 16 + cc] = x;
    }
    __syncthreads();
  }
  }  // !AUXIN

  // ---- 4. [W | U] = X diag(beta gamma | beta) [K | V]; wave w owns column tiles w, w + NW
  f32x16 wu[2][2];
  int my_ct[2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int ct = w + NW * sl;
    my_ct[sl] = ct < NCT ? ct : -1;
    wu[sl][0] = zero16();
    wu[sl][1] = zero16();
    if (AUXIN || ct >= NCT) continue;
    const bool isw = ct * 32 < DK;
    const int col0 = isw ? ct * 32 : ct * 32 - DK;
    const T* brow = (isw ? KT : VT) + (col0 + c32) * PT;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x16 acc = zero16();
      const float* xrow = Xb + (tt * 32 + c32) * PX;
      const float* fac = isw ? s_bg : s_beta;  // column factor: beta gamma for W, beta for U
#pragma unroll
      for (int ks = 0; ks < C / MM::KS; ++ks) {
        const auto bf = MM::load_plain(brow, ks, hh);
        if constexpr (sizeof(T) == 2) {
          // 8 consecutive entries of this lane's X row and their factors, 16-byte reads
          const int s0 = ks * 16 + hh * 8;
          float xv[8], fv[8];
          *reinterpret_cast<float4*>(xv) = *reinterpret_cast<const float4*>(xrow + s0);
          *reinterpret_cast<float4*>(xv + 4) = *reinterpret_cast<const float4*>(xrow + s0 + 4);
          *reinterpret_cast<float4*>(fv) = *reinterpret_cast<const float4*>(fac + s0);
          *reinterpret_cast<float4*>(fv + 4) = *reinterpret_cast<const float4*>(fac + s0 + 4);
          bf16x8 ahi, alo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = xv[e] * fv[e];
            const bf16 hv = (bf16)x;
            ahi[e] = hv;
            alo[e] = (bf16)(x - (float)hv);
          }
          acc = MM::mma(ahi, bf, acc);
          acc = MM::mma(alo, bf, acc);
        } else {
          const int s = ks * 2 + hh;
          acc = MM::mma(xrow[s] * fac[s], bf, acc);
        }
      }
      wu[sl][tt] = acc;
    }
  }

  // W | U fragment image of this chunk for a later output pass: fragment (ct, ks) is the
  // B operand bf16 rows 16 ks .. of columns 32 ct .., 16 bytes per lane, lanes in order
  constexpr int NKC = C / 16;
  if constexpr (WANT_AB && sizeof(T) == 2) {
    if (a.aux_out) {
      bf16* ax = reinterpret_cast<bf16*>(a.aux_out) + ((b * a.H + h) * a.N + c) * (int64_t)C * (DK + DV);
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int ct = my_ct[sl];
        if (ct < 0) continue;
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks)
          *reinterpret_cast<bf16x8*>(ax + ((ct * NKC + ks) * 64 + lane) * 8) = MM::from_acc(wu[sl][ks >> 1], ks, 1.f);
      }
    }
  }

  // ---- 5. transitions: At = gamma_63 I - K^T D W,  Bc = K^T D U
  if constexpr (WANT_AB) {
    const float gam_n = s_gam[C - 1];
    const int64_t cidx = (b * a.H + h) * a.N + c;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ct = my_ct[sl];
      if (ct < 0) continue;
      const bool isw = ct * 32 < DK;
      const int col0 = isw ? ct * 32 : ct * 32 - DK;
      typename MM::Frag bfr[C / MM::KS];
#pragma unroll
      for (int ks = 0; ks < C / MM::KS; ++ks) {
        const int tt = (MM::KS == 16) ? (ks >> 1) : (ks >> 4);
        if constexpr (sizeof(T) == 2) {
          bf16x8 f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ai = (ks & 1) * 8 + e;
            f[e] = (bf16)(wu[sl][tt][ai] * s_d[tt * 32 + acc_row(ai, hh)]);
          }
          bfr[ks] = f;
        } else {
          const int ai = ks & 15;
          bfr[ks] = wu[sl][tt][ai] * s_d[tt * 32 + acc_row(ai, hh)];
        }
      }
      // row-major stores: one base address per lane (row 32 rt + 4 hh, column col0 + c32)
      // and compile-time strides, so the 16 stores of a tile differ only in their offsets;
      // gamma_63 is added on the diagonal of At's diagonal tiles only
      T* const base = isw ? reinterpret_cast<T*>(a.At) + cidx * DK * DK + (hh * 4) * DK + col0 + c32
                          : reinterpret_cast<T*>(a.Bc) + cidx * DK * DV + (hh * 4) * DV + col0 + c32;
#pragma unroll
      for (int rt = 0; rt < DK / 32; ++rt) {
        f32x16 acc = zero16();
        const T* arow = KT + (rt * 32 + c32) * PT;
#pragma unroll
        for (int ks = 0; ks < C / MM::KS; ++ks) acc = MM::mma(MM::load_clayout(arow, ks, hh), bfr[ks], acc);
        if constexpr (sizeof(T) == 2) {
          if (!isw && a.lanes) {
            // the scan's lane order: [chunk][dv/32 column tile][dk/32 row tile][64 lanes][16]
            bf16* bl = reinterpret_cast<bf16*>(a.Bc) + (((cidx * (DV / 32) + col0 / 32) * (DK / 32) + rt) * 64 + lane) * 16;
            bf16x8 lo, hi;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              lo[e] = (bf16)acc[e];
              hi[e] = (bf16)acc[e + 8];
            }
            *reinterpret_cast<bf16x8*>(bl) = lo;
            *reinterpret_cast<bf16x8*>(bl + 8) = hi;
            continue;
          }
        }
        if (isw) {
          if (rt * 32 == col0) {  // diagonal tile: row == column where acc_row(e) == c32
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = (acc_row(e, hh) == c32 ? gam_n : 0.f) - acc[e];
          } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = -acc[e];
          }
          T* o = base + rt * 32 * DK;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[((e >> 2) * 8 + (e & 3)) * DK] = from_f<T>(acc[e]);
        } else {
          T* o = base + rt * 32 * DV;
#pragma unroll
          for (int e = 0; e < 16; ++e) o[((e >> 2) * 8 + (e & 3)) * DV] = from_f<T>(acc[e]);
        }
      }
    }
  }

  // ---- 6. outputs: Qp = diag(gamma) Q - P W, O_intra = P U, O = O_intra + Qp M0
  if constexpr (WANT_O) {
    f32x16 res[2][2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ct = my_ct[sl];
      res[sl][0] = zero16();
      res[sl][1] = zero16();
      if (ct < 0) continue;
      typename MM::Frag bfr[C / MM::KS];
      if constexpr (AUXIN) {
        const bf16* ax = reinterpret_cast<const bf16*>(a.aux_in) + ((b * a.H + h) * a.N + c) * (int64_t)C * (DK + DV);
#pragma unroll
        for (int ks = 0; ks < C / MM::KS; ++ks)
          bfr[ks] = *reinterpret_cast<const bf16x8*>(ax + ((ct * (C / 16) + ks) * 64 + lane) * 8);
      } else {
#pragma unroll
        for (int ks = 0; ks < C / MM::KS; ++ks) {
          const int tt = (MM::KS == 16) ? (ks >> 1) : (ks >> 4);
          bfr[ks] = MM::from_acc(wu[sl][tt], ks, 1.f);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x16 acc = zero16();
        const T* arow = Pb + (tt * 32 + c32) * PT;
#pragma unroll
        for (int ks = 0; ks < C / MM::KS; ++ks) acc = MM::mma(MM::load_clayout(arow, ks, hh), bfr[ks], acc);
        res[sl][tt] = acc;
      }
    }
    __syncthreads();  // every wave is past its reads of X, KT, VT and P
    T* Qb = reinterpret_cast<T*>(sm1);   // [C][PK]
    T* STb = reinterpret_cast<T*>(sm2);  // [DV][PK]: S~ transposed
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ct = my_ct[sl];
      if (ct < 0 || ct * 32 >= DK) continue;
      const int col0 = ct * 32;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = tt * 32 + acc_row(e, hh);
          // with the hand-off nothing overwrote the staged Q (zero past n); otherwise L and X
          // did, and q is read again
          const float qv = AUXIN ? to_f<T>(Qp[t * PK + col0 + c32]) : (t < n ? to_f<T>(qg[t * kstride + col0 + c32]) : 0.f);
          Qb[t * PK + col0 + c32] = from_f<T>(s_gam[t] * qv - res[sl][tt][e]);
        }
    }
    const float* S0 = a.chunk_init ? a.chunk_init + ((b * a.H + h) * a.N + c) * (int64_t)DK * DV : nullptr;
    if (sizeof(T) == 2 && a.chunk_init_t) {
      // the scan's bf16 image [dv][dk] of the start state: straight copies into padded rows
      const bf16* src = reinterpret_cast<const bf16*>(a.chunk_init_t) + ((b * a.H + h) * a.N + c) * (int64_t)DV * DK;
      for (int i = tid; i < DV * DK / 8; i += NT) {
        const int r = i / (DK / 8), u = i % (DK / 8);
        *reinterpret_cast<uint4*>(STb + r * PK + u * 8) = *reinterpret_cast<const uint4*>(src + r * DK + u * 8);
      }
    } else if constexpr (sizeof(T) == 4) {
      for (int i = tid; i < DK * DV / 4; i += NT) {
        const int dk = i / (DV / 4), dv = (i % (DV / 4)) * 4;
        const float4 val = *reinterpret_cast<const float4*>(S0 + dk * DV + dv);
        STb[(dv + 0) * PK + dk] = from_f<T>(val.x);
        STb[(dv + 1) * PK + dk] = from_f<T>(val.y);
        STb[(dv + 2) * PK + dk] = from_f<T>(val.z);
        STb[(dv + 3) * PK + dk] = from_f<T>(val.w);
      }
    } else {
      // S~ transposed to bf16 by register blocks: task (row block rb of 8 dk, column group
      // cg of 4 dv) loads 8 float4 and writes 4 rows of 8 dk.  rb runs fastest, so the 8
      // lanes of a write phase hit 16-byte units (4 cg + j) (PK / 8) + rb, distinct modulo
      // 8 because PK / 8 is odd.
      static_assert((PK / 8) % 2 == 1, "odd row pitch in 16-byte units");
      constexpr int NRB = DK / 8, NCG = DV / 4;
      for (int i = tid; i < NRB * NCG; i += NT) {
        const int rb = i % NRB, cg = i / NRB;
        const float* src = S0 + rb * 8 * DV + cg * 4;
        float4 in[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) in[r] = *reinterpret_cast<const float4*>(src + r * DV);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x8 o;
#pragma unroll
          for (int r = 0; r < 8; ++r) o[r] = (bf16)(j == 0 ? in[r].x : j == 1 ? in[r].y : j == 2 ? in[r].z : in[r].w);
          *reinterpret_cast<bf16x8*>(STb + (cg * 4 + j) * PK + rb * 8) = o;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ct = my_ct[sl];
      if (ct < 0 || ct * 32 < DK) continue;
      const int col0 = ct * 32 - DK;
      const T* brow = STb + (col0 + c32) * PK;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x16 acc = res[sl][tt];
        const T* arow = Qb + (tt * 32 + c32) * PK;
#pragma unroll
        for (int ks = 0; ks < DK / MM::KS; ++ks) acc = MM::mma(MM::load_plain(arow, ks, hh), MM::load_plain(brow, ks, hh), acc);
        // token t = 32 tt + acc_row(e): rows of o are H DV floats apart.  o is the pass's
        // final output, written in whole 128-byte rows of 32 lanes: non-temporal stores
        const int64_t ostride = a.H * DV;
        float* ob = a.o + ((b * a.T + t0 + tt * 32 + hh * 4) * a.H + h) * DV + col0 + c32;
        if (n == C) {
#pragma unroll
          for (int e = 0; e < 16; ++e) __builtin_nontemporal_store(acc[e], &ob[((e >> 2) * 8 + (e & 3)) * ostride]);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (tt * 32 + acc_row(e, hh) < n) __builtin_nontemporal_store(acc[e], &ob[((e >> 2) * 8 + (e & 3)) * ostride]);
        }
      }
    }
  }
}

template <class T, int DK, int DV, bool WANT_AB, bool WANT_O>
static hipError_t launch_chunk_t(const ChunkArgs& a, int64_t nblocks, hipStream_t s) {
  constexpr int NCT = (DK + DV) / 32;
  constexpr int NW = NCT >= 8 ? 8 : 4;
  TimedLaunch tl(HLA_KERNEL_CHUNK, s);
  if constexpr (WANT_O && !WANT_AB && sizeof(T) == 2) {
    if (a.aux_in) {
      hipLaunchKernelGGL((chunk_kernel<T, DK, DV, NW, WANT_AB, WANT_O, true>), dim3((unsigned)nblocks), dim3(NW * 64), 0,
                         s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((chunk_kernel<T, DK, DV, NW, WANT_AB, WANT_O, false>), dim3((unsigned)nblocks), dim3(NW * 64), 0, s,
                     a);
  return hipGetLastError();
}

template <class T, bool WANT_AB, bool WANT_O>
static hipError_t launch_chunk_d(const ChunkArgs& a, int dk, int dv, int64_t nb, hipStream_t s) {
  if (dk == 64 && dv == 64) return launch_chunk_t<T, 64, 64, WANT_AB, WANT_O>(a, nb, s);
  if (dk == 64 && dv == 128) return launch_chunk_t<T, 64, 128, WANT_AB, WANT_O>(a, nb, s);
  if (dk == 128 && dv == 64) return launch_chunk_t<T, 128, 64, WANT_AB, WANT_O>(a, nb, s);
  return launch_chunk_t<T, 128, 128, WANT_AB, WANT_O>(a, nb, s);
}

hipError_t launch_chunk(const ChunkArgs& a, int dtype, int dk, int dv, bool want_ab, bool want_o, hipStream_t s) {
  const int64_t nb = a.B * a.H * (int64_t)a.N;
  if (nb == 0) return hipSuccess;
  if (dtype == 1) {
    if (want_ab && !want_o) return launch_chunk_d<bf16, true, false>(a, dk, dv, nb, s);
    if (!want_ab && want_o) return launch_chunk_d<bf16, false, true>(a, dk, dv, nb, s);
    return hipErrorInvalidValue;
  }
  if (want_ab && !want_o) return launch_chunk_d<float, true, false>(a, dk, dv, nb, s);
  if (!want_ab && want_o) return launch_chunk_d<float, false, true>(a, dk, dv, nb, s);
  return hipErrorInvalidValue;
}

}  // namespace hla
