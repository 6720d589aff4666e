// Device helpers shared by the gfx950 kernels: MFMA traits, fragment loaders that match
// the 32x32 accumulator layout, bf16 packing and wave reductions.
//
// 32x32 MFMA lane layout (64-wide wavefront, lane l, half h = l / 32, c = l % 32):
//   accumulator (16 floats)   : acc[a] is element (row (a/4)*8 + h*4 + a%4, col c)
//   A operand (rows x K)      : row c; bf16 32x32x16 gives 8 k-slots h*8 + e,
//                               f32 32x32x2 gives 1 k-slot h
//   B operand (K x cols)      : col c; same k-slots as A.
// A contraction only needs the two operands to agree on which k each slot holds.  Two
// slot->k maps are used:
//   plain   : bf16 slot s of k-step ks is k = ks*16 + s;  f32 slot h is k = ks*2 + h.
//   clayout : the k order in which an accumulator tile already sits in a lane, so the
//             result of one product feeds the next as its B operand without leaving the
//             lane.  bf16 k-step ks, slot h*8 + e is k = ks*16 + (e/4)*8 + h*4 + e%4, and
//             the B fragment is acc[8*(ks%2) .. 8*(ks%2)+7] of the tile holding rows
//             32*(ks/2) ...;  f32 k-step ks, slot h is k = (ks/16)*32 + ((ks%16)/4)*8 +
//             h*4 + ks%4 and the B fragment is acc[ks%16].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kChunk = 64;  // tokens per chunk

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, so that every
// index inside the body is a constant (register arrays stay in registers).
template <int B, int E, class F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of accumulator element a for lane half h.
__device__ __forceinline__ int acc_row(int a, int h) { return (a >> 2) * 8 + h * 4 + (a & 3); }

// One 32 x 32 float32 tile on the matrix cores (v_mfma_f32_32x32x2_f32): C += A B over KD
// k values, with fa(k) = A[m0 + lane % 32][k] and fb(k) = B[k][n0 + lane % 32] for the lane's
// k = 2 ks + lane / 32; the result is in the accumulator layout (row acc_row(e, lane / 32)).
template <int KD, class FA, class FB>
__device__ __forceinline__ f32x16 mm32(f32x16 acc, int hh, FA fa, FB fb) {
#pragma unroll 8
  for (int ks = 0; ks < KD / 2; ++ks) {
    const int k = 2 * ks + hh;
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa(k), fb(k), acc, 0, 0, 0);
  }
  return acc;
}

template <class T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KS = 16;
  using Frag = bf16x8;
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // plain k order: 8 contiguous elements
  __device__ __forceinline__ static Frag load_plain(const bf16* row, int ks, int h) {
    return *reinterpret_cast<const bf16x8*>(row + ks * 16 + h * 8);
  }
  // clayout k order: two runs of 4
  __device__ __forceinline__ static Frag load_clayout(const bf16* row, int ks, int h) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + ks * 16 + h * 4);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + ks * 16 + 8 + h * 4);
    Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[e] = lo[e]; f[e + 4] = hi[e]; }
    return f;
  }
  // B fragment for k-step ks from an accumulator tile that holds rows 32*(ks/2)..
  __device__ __forceinline__ static Frag from_acc(const f32x16& acc, int ks, float scale) {
    Frag f;
    const int b = (ks & 1) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)(acc[b + e] * scale);
    return f;
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 2;
  using Frag = float;
  __device__ __forceinline__ static f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static Frag load_plain(const float* row, int ks, int h) { return row[ks * 2 + h]; }
  __device__ __forceinline__ static int clayout_k(int ks, int h) {
    const int kl = ks & 15;
    return (ks >> 4) * 32 + (kl >> 2) * 8 + h * 4 + (kl & 3);
  }
  __device__ __forceinline__ static Frag load_clayout(const float* row, int ks, int h) {
    return row[clayout_k(ks, h)];
  }
  __device__ __forceinline__ static Frag from_acc(const f32x16& acc, int ks, float scale) {
    return acc[ks & 15] * scale;
  }
};

// k index of plain slot (ks, h, e) -- used to build elementwise-scaled A fragments.
template <class T> __device__ __forceinline__ int plain_k(int ks, int h, int e);
template <> __device__ __forceinline__ int plain_k<bf16>(int ks, int h, int e) { return ks * 16 + h * 8 + e; }
template <> __device__ __forceinline__ int plain_k<float>(int ks, int h, int) { return ks * 2 + h; }

// k index of clayout slot (ks, h, e).
template <class T> __device__ __forceinline__ int clayout_k(int ks, int h, int e);
template <> __device__ __forceinline__ int clayout_k<bf16>(int ks, int h, int e) {
  return ks * 16 + (e >> 2) * 8 + h * 4 + (e & 3);
}
template <> __device__ __forceinline__ int clayout_k<float>(int ks, int h, int) { return Mma<float>::clayout_k(ks, h); }

// Number of elements a fragment holds per lane.
template <class T> struct FragLen;
template <> struct FragLen<bf16> { static constexpr int n = 8; };
template <> struct FragLen<float> { static constexpr int n = 1; };

template <class T> __device__ __forceinline__ float to_f(T x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f(float x) { return (T)x; }

// Diagonal B fragment: value g where the slot's k (plain order) equals the lane's column.
template <class T> __device__ __forceinline__ typename Mma<T>::Frag diag_frag(int ks, int lane, float g);
template <> __device__ __forceinline__ bf16x8 diag_frag<bf16>(int ks, int lane, float g) {
  bf16x8 f;
  const int col = lane & 31, h = lane >> 5;
  const bf16 gb = (bf16)g, z = (bf16)0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (ks * 16 + h * 8 + e == col) ? gb : z;
  return f;
}
template <> __device__ __forceinline__ float diag_frag<float>(int ks, int lane, float g) {
  const int col = lane & 31, h = lane >> 5;
  return (ks * 2 + h == col) ? g : 0.f;
}

// Sum over the 64 lanes of a wavefront (fixed order: deterministic).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Cross-lane move inside a 16-lane row (DPP), for sums over small lane groups.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Sum over aligned groups of G consecutive lanes (G = 2, 4, 8 or 16), every lane of the group
// receiving it: quad permutations swap lanes 1 and 2 apart, a half-row mirror pairs the two
// quads of an 8-lane half, and row rotations by 4 and 8 add the other quads of a 16-lane row.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2, 4, 8 or 16 lanes");
  x += dpp_f<0xB1>(x);  // quad_perm [1, 0, 3, 2]
  if constexpr (G >= 4) x += dpp_f<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  if constexpr (G == 8) x += dpp_f<0x141>(x);  // row_half_mirror
  if constexpr (G == 16) {
    x += dpp_f<0x124>(x);  // row_ror 4
    x += dpp_f<0x128>(x);  // row_ror 8
  }
  return x;
}

// x plus the value of the lane 16 (swap16) or 32 (swap32) apart, every lane receiving the
// sum: gfx950's permlane swaps exchange 16-lane rows between two registers in the VALU,
// with no LDS traffic.  Both registers hold x, so the two halves of the result are the
// lane's own value and its partner's.
__device__ __forceinline__ float swap16_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
// Sum over the lanes that agree with this one in the lane-index bits below G (G = 8, 16 or
// 32): the lanes G, 2G, ... apart.
template <int G>
__device__ __forceinline__ float stride_sum(float x) {
  static_assert(G == 8 || G == 16 || G == 32, "stride of 8, 16 or 32 lanes");
  if constexpr (G == 8) x += dpp_f<0x128>(x);  // row_ror 8: the lane 8 apart in its row
  if constexpr (G <= 16) x = swap16_sum(x);
  return swap32_sum(x);
}
// Sums of 8 values over the four 16-lane rows of a wave, with the result spread over the
// rows instead of replicated: permlane16_swap of two different values adds each to its
// partner row's copy (rows 0 and 2 keep the first value's pair sums, rows 1 and 3 the
// second's), and permlane32_swap of two such results finishes the four-row sums.  On
// return row rho holds the total of v[rho] in `ra` and of v[4 + rho] in `rb`: 12
// instructions instead of a full all-reduce per value.
__device__ __forceinline__ void rows_sum8(const float (&v)[8], float& ra, float& rb) {
  float l1[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v[2 * m]),
                                                    __builtin_bit_cast(unsigned, v[2 * m + 1]), false, false);
    l1[m] = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  }
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, l1[0]), __builtin_bit_cast(unsigned, l1[1]),
                                            false, false);
  ra = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, l1[2]), __builtin_bit_cast(unsigned, l1[3]),
                                       false, false);
  rb = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Sum over all 64 lanes without LDS traffic.
__device__ __forceinline__ float wave_sum_valu(float x) { return stride_sum<16>(group_sum<16>(x)); }
// Sum over aligned groups of G consecutive lanes (G = 2 .. 64), every lane receiving it.
template <int G>
__device__ __forceinline__ float lane_group_sum(float x) {
  if constexpr (G <= 16) return group_sum<G>(x);
  else if constexpr (G == 32) return swap16_sum(group_sum<16>(x));
  else return wave_sum_valu(x);
}
// Maximum over all 64 lanes without LDS traffic (the same lane moves as wave_sum_valu).
__device__ __forceinline__ float wave_max_valu(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x128>(x));
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  u = __builtin_bit_cast(unsigned, x);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + __expf(-x)); }

// 16-byte global -> LDS copy of `bytes` (multiple of 16) by the whole block.
__device__ __forceinline__ void block_copy16(void* lds, const void* g, int bytes, int tid, int nthreads) {
  const uint4* src = reinterpret_cast<const uint4*>(g);
  uint4* dst = reinterpret_cast<uint4*>(lds);
  for (int i = tid; i < bytes / 16; i += nthreads) dst[i] = src[i];
}

}  // namespace hla
