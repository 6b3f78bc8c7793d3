// Device-side building blocks shared by the libgdn kernels (gfx950 only).
//
// MFMA tiles. Every dense product in the library is built from 16x16 output
// tiles with fp32 accumulation:
//   bf16 operands: v_mfma_f32_16x16x32_bf16 (one instruction per 32-deep step)
//   fp32 operands: v_mfma_f32_16x16x4_f32   (eight instructions per step)
// The accumulator of a 16x16 tile holds, in lane l, rows 4*(l/16)+i (i=0..3)
// of column l%16.
//
// Operand fragments ("frag"): for a 32-deep contraction step starting at k0,
// lane l holds 8 values of its row (A operand) or column (B operand) l%16,
// at the contraction indices
//     k0 + 4*(l/16) + e          for e = 0..3
//     k0 + 16 + 4*(l/16) + e-4   for e = 4..7.
// The products only need A and B to agree on this order. It is chosen so
// that two vertically adjacent accumulator tiles (rows k0..k0+15 and
// k0+16..k0+31) ARE a B fragment (and the A fragment of their transpose)
// without any data movement: this is how the state and the delta rows flow
// from one product into the next inside a wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename E> struct FragOf;
template <> struct FragOf<bf16_t> { typedef bf16x8 type; typedef bf16x4 half; };
template <> struct FragOf<float> { typedef f32x8 type; typedef f32x4 half; };
template <typename E> using Frag = typename FragOf<E>::type;
template <typename E> using Half = typename FragOf<E>::half;

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

template <typename E> __device__ __forceinline__ E to_e(float x);
template <> __device__ __forceinline__ float to_e<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t to_e<bf16_t>(float x) { return (bf16_t)x; }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) { return (float)x; }

template <typename E> __device__ __forceinline__ Half<E> zero_half() {
  Half<E> z;
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = to_e<E>(0.f);
  return z;
}

template <typename E> __device__ __forceinline__ Frag<E> join(const Half<E>& lo, const Half<E>& hi) {
  Frag<E> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = lo[e]; f[e + 4] = hi[e]; }
  return f;
}

// Fragment of a row-major matrix: `row` points at element [row][k0] of the
// lane's row; `kext` is the contraction extent remaining from k0 (a multiple
// of 16), so the upper half is present only when kext > 16.
template <typename E>
__device__ __forceinline__ Frag<E> load_frag(const E* row, int quad, int kext) {
  Half<E> lo = *reinterpret_cast<const Half<E>*>(row + 4 * quad);
  Half<E> hi = (kext > 16) ? *reinterpret_cast<const Half<E>*>(row + 16 + 4 * quad) : zero_half<E>();
  return join<E>(lo, hi);
}

// The same fragment with the contraction index in another order: lane quad
// q holds the 8 consecutive elements k0 + 8 q .. k0 + 8 q + 7 (one 16-byte
// access for bf16), zero where 8 q >= kext. For a product whose other
// operand is read the same way: the MFMA sums over k, so the two operands
// need only agree on its order. `row` must be 16-byte aligned (32-byte for
// fp32 elements).
template <typename E>
__device__ __forceinline__ Frag<E> load_frag8(const E* row, int quad, int kext) {
  Frag<E> z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = to_e<E>(0.f);
  return (8 * quad < kext) ? *reinterpret_cast<const Frag<E>*>(row + 8 * quad) : z;
}

// Same, with the whole row zero when `valid` is false (rows past the end of
// a partial chunk).
template <typename E>
__device__ __forceinline__ Frag<E> load_frag_masked(const E* row, int quad, int kext, bool valid) {
  if (!valid) return join<E>(zero_half<E>(), zero_half<E>());
  return load_frag<E>(row, quad, kext);
}

// Two vertically adjacent accumulator tiles -> operand fragment.
template <typename E>
__device__ __forceinline__ Frag<E> acc_to_frag(const f32x4& lo, const f32x4& hi) {
  Frag<E> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = to_e<E>(lo[e]); f[e + 4] = to_e<E>(hi[e]); }
  return f;
}

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Decay and rank-one update of four state entries, each fma(u_e, k, s_e * alpha):
// the contraction is fixed here rather than left to the compiler, so that
// kernels applying the same update agree bit for bit.
__device__ __forceinline__ f32x4 decay_rank1(f32x4 s, float alpha, f32x4 u, float k) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = fmaf(u[e], k, s[e] * alpha);
  return r;
}

// Cross-lane sums without LDS round trips. The accumulator of a 16x16 tile
// holds one row in each 16-lane row of the wave, so a row's sum over its
// columns is a sum over those 16 lanes (DPP: swap neighbours, then pairs,
// then mirror within 8 and within 16 lanes; every lane gets the sum). Sums
// across the four 16-lane rows use the lane-row swaps (v_permlane16_swap
// and v_permlane32_swap: with both operands x, the two results add up to
// x[l] + x[l ^ 16], respectively x[l] + x[l ^ 32]).
__device__ __forceinline__ float sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}
// Reduce-scatter within each 16-lane row of the wave: lane i of a row gets
// the sum over the row's 16 lanes of their values v[i] (NV = 16), or of
// v[i % 4] (NV = 4, in every lane). A butterfly over the lane pairs i ^ 15,
// i ^ 7 (within each half row), i ^ 2 and i ^ 1: at each step a lane keeps
// the half of its values that its pair does not keep and adds the pair's
// partial sums of that half, so each lane ends with one complete sum, added
// in a fixed order (NV = 4 then sums the row's four groups of four lanes).
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int NV>
__device__ __forceinline__ float row_scatter_sum(const float (&v)[NV], int l16) {
  static_assert(NV == 16 || NV == 4, "16 or 4 values per lane");
  float x[4];
  if constexpr (NV == 16) {
    float w[8];
    const bool b3 = (l16 & 8) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = (b3 ? v[8 + k] : v[k]) + dpp_mov<0x140>(b3 ? v[k] : v[8 + k]);      // row_mirror
    const bool b2 = (l16 & 4) != 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (b2 ? w[4 + k] : w[k]) + dpp_mov<0x141>(b2 ? w[k] : w[4 + k]);      // row_half_mirror
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = v[k];
  }
  const bool b1 = (l16 & 2) != 0;
  float y[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) y[k] = (b1 ? x[2 + k] : x[k]) + dpp_mov<0x4E>(b1 ? x[k] : x[2 + k]);         // quad_perm 2,3,0,1
  const bool b0 = (l16 & 1) != 0;
  float z = (b0 ? y[1] : y[0]) + dpp_mov<0xB1>(b0 ? y[0] : y[1]);                                          // quad_perm 1,0,3,2
  if constexpr (NV == 4) {
    z += dpp_mov<0x124>(z);    // row_ror:4
    z += dpp_mov<0x128>(z);    // row_ror:8
  }
  return z;
}

__device__ __forceinline__ float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// Fused input preparation (GDN_FLAG_PREPARE_INPUTS): the gate maps
// log(alpha) = -softplus(a) and beta = sigmoid(b), written so that neither
// overflows for any sign of the logit, and the L2 normalisation of q and k.
__device__ __forceinline__ float neg_softplus(float a) { return -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a)))); }
__device__ __forceinline__ float sigmoid_of(float b) {
  const float e = expf(-fabsf(b));
  return b >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}
__device__ __forceinline__ float inv_norm(float sum_sq) { return rsqrtf(fmaxf(sum_sq, 1e-12f)); }

// Scales one (token, head) vector of length D to unit L2 norm while it is
// in registers: each of D / N consecutive lanes holds N of its elements in
// `v`; the lanes add their squares in fp32 and combine the sums with lane
// exchanges, so every lane of such a group must be active (groups are
// aligned to D / N lanes).
template <typename E, int D, int N, typename V>
__device__ __forceinline__ void normalize_slice(V& v) {
  constexpr int L = D / N;
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lanes per vector: a power of two within a wave");
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float x = to_f(v[e]);
    ss += x * x;
  }
#pragma unroll
  for (int m = 1; m < L; m <<= 1) ss += __shfl_xor(ss, m);
  const float inv = inv_norm(ss);
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = to_e<E>(to_f(v[e]) * inv);
}

}  // namespace gdn
