// Tile configuration and helpers shared by the prefill and backward kernels
// (gfx950 only). Internal; included by gdn_prefill.hip and gdn_backward.hip.
#pragma once

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Token range [x, y) of sequence n (the whole input when cu_seqlens is
// null). The table's contents are a precondition of the entry points (0 =
// c_0 <= ... <= c_N = T; checked on the host only under GDN_DEBUG). The
// kernels clamp each bound into [0, T] with y >= x, so a table that breaks
// it yields unspecified outputs but no access outside the arguments.
__device__ __forceinline__ int2 seq_range(const PrefillArgs& a, int64_t n) {
  const int t = (int)a.total_tokens;
  if (!a.cu_seqlens) return make_int2(0, t);
  const int s0 = min(max(a.cu_seqlens[n], 0), t);
  return make_int2(s0, min(max(a.cu_seqlens[n + 1], s0), t));
}

// Chunk-slot range [x, y) of sequence n from the per-sequence chunk offsets
// (written by the chunk lookup of kernel 2, or of kernel 1 in the backward pass), clamped
// into [0, max_chunks] likewise (with a table that breaks the precondition
// the offsets could pass the workspace's chunk count).
__device__ __forceinline__ int2 chunk_range(const PrefillArgs& a, int64_t n) {
  const int nc = (int)a.max_chunks;
  const int c0 = min(max(a.seq_chunk_offset[n], 0), nc);
  return make_int2(c0, min(max(a.seq_chunk_offset[n + 1], c0), nc));
}

constexpr int kBlock = 256;

template <typename E, int D, int C>
struct Cfg {
  static constexpr int DT = D / 16, CT = C / 16;
  static constexpr int DKS = (DT + 1) / 2, CKS = (CT + 1) / 2;
  static constexpr int NS = DT >= 2 ? 2 : 1;   // 16-column state slices per scan workgroup
  static constexpr int BV = 16 * NS;           // state columns per scan workgroup
  static constexpr int NCB = D / BV;           // scan workgroups per (sequence, V head)
  static constexpr int KT_FR = DT * CKS;       // K^T fragments per chunk
  static constexpr int T_FR = CT * CKS;        // Tinv fragments per chunk
  static constexpr int QK_FR = CT * CKS;       // q.k fragments per chunk
  static constexpr int Q_FR = CT * DKS;        // Q fragments per chunk
  static constexpr int W_FR = CT * DKS;        // W fragments per chunk
};

// Workgroups are dispatched round-robin over the chip's 8 XCDs (each with
// its own L2): workgroup b runs on XCD b % 8. Renumbering so that logical
// ids [k n/8, (k+1) n/8) all run on XCD k keeps workgroups that read the
// same operands (consecutive logical ids) behind one L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_local_id(int64_t b, int64_t n) {
  if (n % kXcds) return b;
  return (b % kXcds) * (n / kXcds) + b / kXcds;
}

// Contraction index of fragment element e at 32-step s for lane quad q.
__device__ __forceinline__ int frag_k(int s, int quad, int e) {
  return 32 * s + (e < 4 ? 4 * quad + e : 16 + 4 * quad + (e - 4));
}

// True when fragment step s of query tile nt holds only keys after every
// query of the tile (the causal mask makes it zero).
__device__ __forceinline__ constexpr bool causal_zero(int nt, int s) { return 32 * s > 16 * nt + 15; }

// acc += X Y for 16 x 16 tiles held in LDS, in fp32 (v_mfma_f32_16x16x4_f32;
// bf16 elements are widened); X(m, k) = X[m xr + k xc] and
// Y(k, m) = Y[k yr + m yc], so strides give either storage order
template <typename TX, typename TY>
__device__ __forceinline__ f32x4 mma16_f32(const TX* X, int xr, int xc, const TY* Y, int yr, int yc,
                                           f32x4 acc, int lane) {
  const int m = lane & 15, k = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(to_f(X[m * xr + (4 * kk + k) * xc]), to_f(Y[(4 * kk + k) * yr + m * yc]),
                                               acc, 0, 0, 0);
  return acc;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier for the scan and Ut waves: it waits only for this
// wave's LDS operations, not for global stores or L2 warm-up loads (nothing
// in the workgroup reads those back).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One direct global-to-LDS copy of up to 1 KB: lane l copies the 16 bytes
// at src + 16 l to dst + 16 l (dst is the same for the whole wave); lanes
// at or past `bytes` copy nothing.
__device__ __forceinline__ void copy_1k(const char* src, char* dst, int bytes, int lane) {
  if (16 * lane < bytes) __builtin_amdgcn_global_load_lds(src + 16 * lane, (lds_ptr_t)dst, 16, 0, 0);
}


// Stores NT 16 x 16 fp32 accumulator tiles of one wave (tile t holds rows
// 16 t .. 16 t + 15 and, in lane l, rows 16 t + 4 (l / 16) + i of column
// l % 16) to a row-major matrix g (row stride ld elements), rounded to E,
// through a wave-private LDS area of stage_elems<E>() elements, up to four
// tiles at a time: lanes write their elements, then read back 16-byte row
// segments, so the global writes are 16-byte stores (two or four lanes per
// 16-column row segment) instead of one 2- or 4-byte store per element. The
// area may be reused once the call returns.
template <typename E> constexpr int stage_elems() { return 64 * (16 + 16 / (int)sizeof(E)); }

// The first half of store_tiles_rows on its own: NT accumulator tiles (rows
// 16 t + 4 q + i, column l) written row-major into `area` with the padded
// row stride 16 + 16 / sizeof(E), for another wave to read back as 16-byte
// row segments (load_staged_rows) once an LDS barrier has passed.
template <typename E> constexpr int staged_ld() { return 16 + 16 / (int)sizeof(E); }
template <typename E, int NT>
__device__ __forceinline__ void stage_tiles_rows(const f32x4 (&acc)[NT], E* area, int lane) {
  constexpr int SLD = staged_ld<E>();
  const int q = lane >> 4, col = lane & 15;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) area[(16 * t + 4 * q + i) * SLD + col] = to_e<E>(acc[t][i]);
  }
}
// Lane `lane`'s 16-byte piece of instruction j over staged rows: row
// j * RPI + lane / LPR, columns (lane % LPR) * VE .. + VE - 1.
template <typename E> struct StagedRows {
  static constexpr int VE = 16 / (int)sizeof(E), LPR = 16 / VE, RPI = 64 / LPR;
};

template <typename E, int NT>
__device__ __forceinline__ void store_tiles_rows(const f32x4 (&acc)[NT], E* area, E* g, int ld, int lane) {
  constexpr int VE = 16 / (int)sizeof(E);     // elements per 16 bytes
  constexpr int SLD = 16 + VE;                // staging row stride (rows stay 16-byte aligned)
  constexpr int LPR = 16 / VE;                // lanes per 16-column row segment
  constexpr int RPI = 64 / LPR;               // rows per store instruction
  constexpr int NG = NT < 4 ? NT : 4;         // tiles per staging round
  static_assert(NT % NG == 0, "whole staging rounds");
  typedef E Vec __attribute__((ext_vector_type(VE)));
  const int q = lane >> 4, col = lane & 15;
#pragma unroll
  for (int t0 = 0; t0 < NT; t0 += NG) {
#pragma unroll
    for (int t = 0; t < NG; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) area[(16 * t + 4 * q + i) * SLD + col] = to_e<E>(acc[t0 + t][i]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int p = 0; p < (NG * 16 + RPI - 1) / RPI; ++p) {
      const int row = lane / LPR + RPI * p, c = (lane % LPR) * VE;
      if (NG * 16 % RPI == 0 || row < NG * 16) {
        const Vec v = *reinterpret_cast<const Vec*>(&area[row * SLD + c]);
        *reinterpret_cast<Vec*>(&g[(int64_t)(16 * t0 + row) * ld + c]) = v;
      }
    }
  }
}

}  // namespace gdn
