// Backward pass (gdn_chunk_bwd): gradients of a scalar loss through the
// chunkwise evaluation of the gated delta rule of page "Qwen3.8-Flash-Next
// 技术总结", section 2.1 (Gated DeltaNet). The section presents the chunkwise
// algorithm as the way to train the layer; it prints no backward pass, so
// the formulas below are the derivative of the forward block formulas
// (gdn_prefill.hip). For one V head and a chunk entering with state S0 and
// leaving with S_L, with dO = dL/dO and dS_L = dL/dS_L (ea_r = exp(g_r),
// ed_r = exp(g_L - g_r), P = Q K^T * Dincl, Gm[r,i] = exp(g_r - g_i)):
//
//   reverse state scan, chunks in reverse order (dS carries dL/dS):
//     dU     = diag(ed) K dS_L + P^T dO
//     dS0    = exp(g_L) dS_L + Q^T diag(ea) dO - W^T dU
//   per chunk and V head (gradient kernel):
//     dQ     = diag(ea) dO S0^T + (dP * Dincl) K,     dP = dO U^T
//     dK     = (dP * Dincl)^T Q + diag(ed) U dS_L^T + diag(b ea) Tinv^T dW
//              + (B + B^T) K,                          dW = -dU S0^T
//     dV     = diag(b) Tinv^T dU
//     dA     = -Tinv^T dT Tinv^T (strictly lower),    dT = dU (diag(b) V)^T + dW (diag(b ea) K)^T
//     B      = dA * b_r Gm,  M = B * (K K^T)
//     db_r   = (Tinv^T dU)_r . v_r + ea_r (Tinv^T dW)_r . k_r + sum_i dA[r,i] (k_r . k_i) Gm[r,i]
//     dg_r   = b_r ea_r (Tinv^T dW)_r . k_r + rowsum(M)_r - colsum(M)_r
//              + q_r . (ea_r (dO S0^T)_r) + rowsum(dP * P)_r - colsum(dP * P)_r
//              - ed_r k_r . (U dS_L^T)_r    (+ at r = L: the sum of those terms
//              and exp(g_L) <S0, dS_L>)
//     dlog a = the suffix sums of dg within the chunk.
// A QK head's dq and dk sum over its V heads.
//
// Launches: kernel 1 (chunk table, g and b, the K^T, K and Q^T fragments
// and the query-indexed q.k products), kernel 2 in its backward form (also
// writing the P^T and W^T fragments and Tinv^T); kernel 3 in its saving form (the state at
// every chunk start and the U rows, no outputs); the reverse state scan
// (gdn_kb_dstate); the gradient kernel (gdn_kb_grad).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

namespace {
// Raw buffer accesses for the gradient kernel's per-element global reads and
// writes: the base sits in a resource descriptor (uniform), the lane offset
// is a 32-bit byte count, so no 64-bit address arithmetic is needed per
// element. Accesses at or past `bytes` are dropped (reads return zero).
// Descriptor word 3 is gfx9's raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
template <typename E>
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, E x) {
  if constexpr (sizeof(E) == 2) __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, (int)byte_off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, (int)byte_off, 0, 0);
}
template <typename E>
__device__ __forceinline__ E buf_load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  if constexpr (sizeof(E) == 2) return __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b16(r, (int)byte_off, 0, 0));
  else return __builtin_bit_cast(E, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}
}  // namespace

namespace {

// --------------------------------------------------------------------------
// Reverse state scan: one workgroup per (sequence, V head, block of BV state
// columns); the NS scan waves hold dS for their 16-column slices in MFMA
// accumulators and walk the chunks from last to first; the other waves
// copy chunk c-1's operands into the idle LDS buffer (direct global-to-LDS
// loads) while chunk c is processed. Per chunk the scan waves leave dS_L
// and dU (rounded to the input dtype, as the gradient kernel's products use
// them) in an LDS staging area, double-buffered by chunk parity, and store
// waves write the previous chunk's as 16-byte row segments after each
// barrier, so that no wave waits for those stores; the store waves also
// warm L2 three chunks ahead. After the first chunk dS is dL/dS0 of the
// sequence.
// --------------------------------------------------------------------------
constexpr int kDScanBlock = 512;

template <typename E, int D, int C>
struct DScanSmem {
  using G = Cfg<E, D, C>;
  Frag<E> kf[2][G::Q_FR * 64];       // K fragments (row r, k = d)
  Frag<E> pt[2][G::QK_FR * 64];      // P^T fragments (row key j, k = query r)
  Frag<E> qt[2][G::KT_FR * 64];      // Q^T fragments (row d, k = token r)
  Frag<E> wt[2][G::KT_FR * 64];      // W^T fragments (row d, k = token r)
  E dor[2][C * G::BV];               // dL/do rows, this block's columns
  float dtab[2][2 * C + 4] __attribute__((aligned(16)));
  // per chunk parity and scan wave: dS_L (D rows) then dU (C rows) of the
  // wave's 16 columns, row-major with stride 16 + VE, for the store waves
  E stage[2][G::NS][(D + C) * (16 + 16 / sizeof(E))] __attribute__((aligned(16)));
  float touch[G::NS][64];            // landing place of the L2 warm-up loads
};

template <typename E, int D, int C>
__global__ __launch_bounds__(kDScanBlock) void gdn_kb_dstate(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  constexpr int DT = G::DT, CT = G::CT, DKS = G::DKS, CKS = G::CKS, NS = G::NS, BV = G::BV;
  constexpr int NLD = kDScanBlock / 64 - 2 * NS;          // loader waves (then NS store waves)
  constexpr int FB = (int)sizeof(Frag<E>) * 64;
  constexpr int ESZ = (int)sizeof(E);
  constexpr int VE = 16 / ESZ, SLD = 16 + VE;          // staging: 16-byte segments, row stride
  typedef E Vec __attribute__((ext_vector_type(VE)));
  __shared__ DScanSmem<E, D, C> sm;
  const int tid = threadIdx.x, lane = tid & 63, quad = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bid = xcd_local_id(blockIdx.x, gridDim.x);
  const int cb = (int)(bid % G::NCB);
  const int hv = (int)((bid / G::NCB) % a.h_v);
  const int64_t n = bid / ((int64_t)G::NCB * a.h_v);
  const int hq = hv / a.group;
  const int2 cr = chunk_range(a, n), sr = seq_range(a, n);
  const int c0 = cr.x, c1 = cr.y;
  const int seq_start = sr.x, seq_end = sr.y;
  auto chunk_start = [&](int x) { return seq_start + (x - c0) * C; };
  auto chunk_len = [&](int x) { return min(C, seq_end - chunk_start(x)); };
  const bool is_scan = wave < NS, is_loader = !is_scan && wave < NS + NLD;
  const int slice = wave, lw = wave - NS, sw = wave - NS - NLD;
  const int col0 = cb * BV;
  const int64_t state_base = (n * a.h_v + hv) * D * D;

  constexpr int B_KF = G::Q_FR * FB, B_PT = G::QK_FR * FB, B_QT = G::KT_FR * FB, B_WT = G::KT_FR * FB;
  constexpr int B_O = C * BV * ESZ, B_D = (2 * C + 4) * 4;
  constexpr int NREG = 6;
  constexpr int JOBS[NREG] = {(B_KF + 1023) / 1024, (B_PT + 1023) / 1024, (B_QT + 1023) / 1024,
                              (B_WT + 1023) / 1024, (B_D + 1023) / 1024,  (B_O + 1023) / 1024};
  constexpr int CUM[NREG] = {0, JOBS[0], JOBS[0] + JOBS[1], JOBS[0] + JOBS[1] + JOBS[2],
                             JOBS[0] + JOBS[1] + JOBS[2] + JOBS[3],
                             JOBS[0] + JOBS[1] + JOBS[2] + JOBS[3] + JOBS[4]};
  auto copy_region = [&](int r, const char* src, char* dst, int bytes) __attribute__((always_inline)) {
    for (int jj = ((lw - CUM[r]) % NLD + NLD) % NLD; jj < JOBS[r]; jj += NLD)
      copy_1k(src + 1024 * jj, dst + 1024 * jj, bytes - 1024 * jj, lane);
  };
  // chunk x's operands into buffer x & 1 (nothing before the sequence's
  // first chunk)
  auto copy_chunk = [&](int x) __attribute__((always_inline)) {
    if (x < c0) return;
    const int b = x & 1;
    copy_region(0, static_cast<const char*>(a.k_frag) + ((int64_t)x * a.h_qk + hq) * B_KF,
                reinterpret_cast<char*>(sm.kf[b]), B_KF);
    copy_region(1, static_cast<const char*>(a.pt) + ((int64_t)x * a.h_v + hv) * B_PT,
                reinterpret_cast<char*>(sm.pt[b]), B_PT);
    copy_region(2, static_cast<const char*>(a.q_t) + ((int64_t)x * a.h_qk + hq) * B_QT,
                reinterpret_cast<char*>(sm.qt[b]), B_QT);
    copy_region(3, static_cast<const char*>(a.wt) + ((int64_t)x * a.h_v + hv) * B_WT,
                reinterpret_cast<char*>(sm.wt[b]), B_WT);
    copy_region(4, reinterpret_cast<const char*>(a.dtab + ((int64_t)x * a.h_v + hv) * (2 * C + 4)),
                reinterpret_cast<char*>(sm.dtab[b]), B_D);
    // dL/do rows of the block's columns, row i at byte i * BV * ESZ; rows
    // past the chunk end repeat its last row (every product that reads
    // them has zero factors there)
    const int p_start = chunk_start(x), p_last = chunk_len(x) - 1;
    char* dst = reinterpret_cast<char*>(sm.dor[b]);
    for (int jj = ((lw - CUM[5]) % NLD + NLD) % NLD; jj < JOBS[5]; jj += NLD) {
      const int o = 1024 * jj + 16 * lane;
      const int i = min(o / (BV * ESZ), p_last);
      const char* src = static_cast<const char*>(a.d_o) +
                        (((int64_t)(p_start + i) * a.h_v + hv) * D + col0) * ESZ + o % (BV * ESZ);
      if (o < B_O) __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(dst + 1024 * jj), 16, 0, 0);
    }
  };

  // store waves: chunk x's staged dS_L and dU rows (all slices) to the
  // row-major workspace matrices, 16-byte stores; nothing in the kernel
  // reads them back, so no wave waits for them
  auto store_staged = [&](int x) __attribute__((always_inline)) {
    if (x < c0 || x >= c1) return;
    constexpr int SEG = NS * (D + C) * (16 / VE);      // 16-byte segments per chunk
    E* dslg = static_cast<E*>(a.dsl) + ((int64_t)x * a.h_v + hv) * D * D + col0;
    E* dug = static_cast<E*>(a.du) + ((int64_t)x * a.h_v + hv) * C * D + col0;
    for (int sgi = 64 * sw + lane; sgi < SEG; sgi += 64 * NS) {
      const int sl = sgi / ((D + C) * (16 / VE)), rem = sgi % ((D + C) * (16 / VE));
      const int row = rem / (16 / VE), cc = (rem % (16 / VE)) * VE;
      const Vec v = *reinterpret_cast<const Vec*>(&sm.stage[x & 1][sl][row * SLD + cc]);
      if (row < D) *reinterpret_cast<Vec*>(&dslg[row * D + 16 * sl + cc]) = v;
      else *reinterpret_cast<Vec*>(&dug[(row - D) * D + 16 * sl + cc]) = v;
    }
  };

  // L2 warm-up, issued by the store waves after their stores (they load
  // nothing into registers, so nothing ever waits on these) three chunks
  // ahead in the reverse walk: one 4-byte load per 128-byte line of the
  // chunk's streamed operands, each line touched by one of the workgroups
  // that read it (per V head: P^T, W^T and the row-factor table, shared by
  // the NCB column blocks; per QK head: K and Q^T, shared by the group's V
  // heads too), plus this workgroup's own dL/do rows
  constexpr int LV = (B_PT + B_WT + B_D + 127) / 128;              // lines per (chunk, V head)
  constexpr int LQ = (B_KF + B_QT + 127) / 128;                    // lines per (chunk, QK head)
  const int gi = hv % a.group;
  const int nv = (LV - cb + G::NCB - 1) / G::NCB;
  const int qs = gi * G::NCB + cb, qstride = a.group * G::NCB;
  const int nq = qs < LQ ? (LQ - qs + qstride - 1) / qstride : 0;
  auto line_addr = [&](int x, int t) -> const char* {
    if (t < nv) {
      const int o = 128 * (cb + G::NCB * t);
      return o < B_PT ? static_cast<const char*>(a.pt) + ((int64_t)x * a.h_v + hv) * B_PT + o
           : o < B_PT + B_WT ? static_cast<const char*>(a.wt) + ((int64_t)x * a.h_v + hv) * B_WT + (o - B_PT)
           : reinterpret_cast<const char*>(a.dtab + ((int64_t)x * a.h_v + hv) * (2 * C + 4)) +
                 min(o - B_PT - B_WT, B_D - 4);
    }
    t -= nv;
    if (t < nq) {
      const int o = 128 * (qs + qstride * t);
      return o < B_KF ? static_cast<const char*>(a.k_frag) + ((int64_t)x * a.h_qk + hq) * B_KF + o
           : static_cast<const char*>(a.q_t) + ((int64_t)x * a.h_qk + hq) * B_QT + min(o - B_KF, B_QT - 4);
    }
    t -= nq;
    const int i = min(t, chunk_len(x) - 1);
    return static_cast<const char*>(a.d_o) + (((int64_t)(chunk_start(x) + i) * a.h_v + hv) * D + col0) * ESZ;
  };
  auto warm = [&](int x) __attribute__((always_inline)) {
    if (x < c0) return;
    const int total = nv + nq + C;
    for (int t = 64 * sw + lane; t < total; t += 64 * NS)
      __builtin_amdgcn_global_load_lds(line_addr(x, t), (lds_ptr_t)sm.touch[sw], 4, 0, 0);
  };

  f32x4 dS[DT];
  auto dscan_chunk = [&](int c) __attribute__((always_inline)) {
    const int par = c & 1;
    // dS is dL/d(state at chunk c's end); it and dU go to the staging area,
    // which the store waves store after the barrier
    E* stg = sm.stage[par][slice];
    auto stage4 = [&](int row0, const f32x4& v) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) stg[(row0 + 4 * quad + i) * SLD + l16] = to_e<E>(v[i]);
    };
    Frag<E> dSf[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) dSf[ks] = acc_to_frag<E>(dS[2 * ks], (2 * ks + 1 < DT) ? dS[2 * ks + 1] : zero4());
    const float* ea = sm.dtab[par];
    const float* ed = sm.dtab[par] + C;
    // Only K dS_L -> dU -> W^T dU lies on the path from one chunk's dS to
    // the previous one's; P^T dO and Q^T diag(ea) dO, which do not read dS,
    // run while K dS_L's results land.
    //   KdS = K dS_L
    f32x4 KdS[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      KdS[t] = zero4();
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) KdS[t] = mma(sm.kf[par][(t * DKS + ks) * 64 + lane], dSf[ks], KdS[t]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) stage4(16 * dt, dS[dt]);
    // dL/do fragments (k = token r, column = state column), plain and
    // scaled by exp(g_r)
    Frag<E> dOf[CKS], gOf[CKS];
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = frag_k(s, quad, e);
        const E x = (r < C) ? sm.dor[par][r * BV + 16 * slice + l16] : to_e<E>(0.f);
        dOf[s][e] = x;
        gOf[s][e] = to_e<E>((r < C) ? to_f(x) * ea[r] : 0.f);
      }
    }
    //   PdO = P^T dO
    f32x4 dU[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      dU[t] = zero4();
#pragma unroll
      for (int s = 0; s < CKS; ++s)
        if (32 * s + 31 >= 16 * t) dU[t] = mma(sm.pt[par][(t * CKS + s) * 64 + lane], dOf[s], dU[t]);
    }
    //   dS0 = exp(g_L) dS_L + Q^T diag(ea) dO - W^T dU: the first two terms
    const float gam = sm.dtab[par][2 * C];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dS[dt] *= gam;
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dS[dt] = mma(sm.qt[par][(dt * CKS + s) * 64 + lane], gOf[s], dS[dt]);
    }
    // dU = diag(ed) K dS_L + P^T dO
#pragma unroll
    for (int t = 0; t < CT; ++t) dU[t] += KdS[t] * *reinterpret_cast<const f32x4*>(&ed[16 * t + 4 * quad]);
    Frag<E> nUf[CKS];
#pragma unroll
    for (int s = 0; s < CKS; ++s) nUf[s] = acc_to_frag<E>(-dU[2 * s], (2 * s + 1 < CT) ? -dU[2 * s + 1] : zero4());
    //   ... - W^T dU
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dS[dt] = mma(sm.wt[par][(dt * CKS + s) * 64 + lane], nUf[s], dS[dt]);
    }
#pragma unroll
    for (int t = 0; t < CT; ++t) stage4(D + 16 * t, dU[t]);
  };

  auto state_index = [&](int dt, int i) {
    return state_base + (int64_t)(16 * dt + 4 * quad + i) * D + col0 + 16 * slice + l16;
  };
  if (c1 > c0) {
    if (is_scan) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[dt][i] = a.d_final ? a.d_final[state_index(dt, i)] : 0.f;
      }
      __syncthreads();
      for (int c = c1 - 1; c >= c0; --c) {
        dscan_chunk(c);
        lds_barrier();
      }
      if (a.d_init) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) a.d_init[state_index(dt, i)] = dS[dt][i];
        }
      }
    } else if (is_loader) {
      copy_chunk(c1 - 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      for (int c = c1 - 1; c >= c0; --c) {
        copy_chunk(c - 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    } else {
      warm(c1 - 2);
      warm(c1 - 3);
      lds_barrier();
      for (int c = c1 - 1; c >= c0; --c) {
        store_staged(c + 1);
        warm(c - 3);
        lds_barrier();
      }
      store_staged(c0);
    }
  } else if (is_scan && a.d_init) {
    // empty sequence: dL/dS0 is dL/d(final state)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a.d_init[state_index(dt, i)] = a.d_final ? a.d_final[state_index(dt, i)] : 0.f;
    }
  }
}

// --------------------------------------------------------------------------
// Gradient kernel: one workgroup per (chunk slot, QK head), 4 waves, 80 KB
// of LDS so that two workgroups share a CU (one's barriers and loads overlap
// the other's products). The V heads of the group are taken in turn; their
// dq, dk contributions stay in registers (wave w owns the C x D output
// tiles t = w, w + 4, ...). Per V head, dL/do, U and dU rows and Tinv^T are
// staged in LDS; the chunk-start state and dS_L are read straight from the
// workspace as fragments of their transposes; K and Q come from the
// fragments kernel 1 wrote: K fragments (row r, k = d) for the products
// that contract over d, K^T and Q^T fragments (row d, k = token) for those
// that contract over tokens and for their elements, since fragment
// (dt, rt/2) of K^T holds, at element i + 4 (rt & 1), exactly the element
// (16 rt + 4 quad + i, 16 dt + l16) of a C x D accumulator tile. Every
// product runs on the input dtype's MFMA with fp32 accumulation; the C x C
// matrices that only feed products (dP * Dincl, dT, Y, B + B^T) are held in
// the input dtype. Row sums of the per-element terms are reduced within
// each 16-lane row by a DPP butterfly that leaves one row's sum in each
// lane, column sums by lane-row swaps; then LDS atomics (one per lane) add
// them into each wave's own row sums, which are added in wave order at the
// end.
// --------------------------------------------------------------------------
constexpr int kGradBlock = 256;

template <typename E, int D, int C>
struct GradSmem {
  static constexpr int KLD = D + 8;    // row stride of the staged D-wide rows
  static constexpr int ELD = C + 8;    // row stride of the C x C matrices
  static constexpr int TLD = C + 8;    // row stride of Tinv^T
  union {
    E r1[C * KLD];                     // dL/do rows, then v rows
    E y[C * ELD];                      // then Y = dT Tinv^T
  } __attribute__((aligned(16))) u1;
  E r2[C * KLD] __attribute__((aligned(16)));   // U rows, then dW rows
  E r3[C * KLD] __attribute__((aligned(16)));   // dU rows
  E tt[C * TLD] __attribute__((aligned(16)));   // Tinv^T rows
  // dP * Dincl, then dT, then B + B^T (each only an MFMA operand, so held
  // in the input dtype)
  E x1[C * ELD] __attribute__((aligned(16)));
  float g[C], b[C], ea[C], ed[C], dg[C], db[C];
  // each wave's own row sums of the dlog a and db terms, and of <S0, dS_L>
  // and the state-term row factors (LDS atomics, which one wave executes in
  // program order); added across waves in wave order once all are in, so
  // the gradients do not depend on which wave got there first
  float dgw[kGradBlock / 64][C], dbw[kGradBlock / 64][C];
  float sumw[kGradBlock / 64][2];
};

template <typename E, int D, int C>
__global__ __launch_bounds__(kGradBlock, 2) void gdn_kb_grad(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  using SM = GradSmem<E, D, C>;
  constexpr int DT = G::DT, CT = G::CT, DKS = G::DKS, CKS = G::CKS;
  constexpr int KLD = SM::KLD, ELD = SM::ELD, TLD = SM::TLD;
  constexpr int NW = kGradBlock / 64;
  // wave w owns the C x D tiles of d-tiles w, w + NW, ... (all row tiles)
  // and the C x C tiles of column tiles w, w + NW, ...: the operand of a
  // column tile is loaded once and used for every row tile
  constexpr int DPW = (DT + NW - 1) / NW, TPW = DPW * CT;     // d-tiles, C x D tiles per wave
  constexpr int JPW = (CT + NW - 1) / NW;                     // C x C column tiles per wave
  static_assert(C <= 64, "a chunk's rows fit one wave (the dlog a scan)");
  constexpr int VE = 16 / (int)sizeof(E);
  typedef E VLoad __attribute__((ext_vector_type(VE)));
  __shared__ SM sm;
  E* ys = sm.u1.y;
  const int64_t c = blockIdx.x;
  const int hq = blockIdx.y;
  const int4 tab = reinterpret_cast<const int4*>(a.chunk_table)[c];
  if (tab.x < 0) return;
  const int start = tab.y, len = tab.z;
  // lane indices are re-made opaque at the top of every V head's pass (see
  // there); the wave index is uniform
  int tid = threadIdx.x, lane = tid & 63, quad = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool has_dt = wave < DT;       // the wave owns at least one d-tile

  // rows [0, C) of a [T][H][D] input into LDS (zero past the chunk end);
  // a uniform base pointer and 32-bit lane offsets. Every load is issued
  // unconditionally (rows past the end read the last row, then select
  // zero), so all of a thread's loads are in flight before the first wait.
  // Loads and LDS stores are separate steps, so that a phase can request
  // all of its global reads before it waits for any of them (the compiler
  // keeps a load that follows an LDS store after it).
  constexpr int SPT = (C * D / VE + kGradBlock - 1) / kGradBlock;   // 16-byte loads per thread
  struct Rows { VLoad x[SPT]; };
  auto load_rows = [&](const void* src, int heads, int head) __attribute__((always_inline)) {
    const E* sg = static_cast<const E*>(src) + ((int64_t)start * heads + head) * D;
    Rows t;
#pragma unroll
    for (int p = 0; p < SPT; ++p) {
      const int idx = tid + p * kGradBlock;
      const int r = min(idx / (D / VE), len - 1), d = (idx % (D / VE)) * VE;
      if (idx < C * D / VE) t.x[p] = *reinterpret_cast<const VLoad*>(sg + r * heads * D + d);
    }
    return t;
  };
  // the rows of a [C][D] workspace matrix
  auto load_ws = [&](const E* src) __attribute__((always_inline)) {
    Rows t;
#pragma unroll
    for (int p = 0; p < SPT; ++p) {
      const int idx = tid + p * kGradBlock;
      if (idx < C * D / VE) t.x[p] = *reinterpret_cast<const VLoad*>(src + idx * VE);
    }
    return t;
  };
  // into LDS rows of stride KLD; rows past the chunk end zero when
  // `zero_tail` is set
  auto store_rows = [&](E* dst, const Rows& t, bool zero_tail) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < SPT; ++p) {
      const int idx = tid + p * kGradBlock;
      const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
      if (idx < C * D / VE) {
        VLoad v = t.x[p];
        if (zero_tail && r >= len) {
#pragma unroll
          for (int e = 0; e < VE; ++e) v[e] = to_e<E>(0.f);
        }
        *reinterpret_cast<VLoad*>(&dst[r * KLD + d]) = v;
      }
    }
  };
  // operand fragments of LDS matrices for 32-step s: along a row (the
  // contraction runs along the row) or down a column
  auto frag_row = [&](const E* m, int ld, int row0, int s, int kext) __attribute__((always_inline)) {
    return load_frag<E>(m + (row0 + l16) * ld + 32 * s, quad, kext - 32 * s);
  };
  // the same with 8 consecutive contraction indices per lane (load_frag8),
  // for the products whose other operand is read that way too
  auto frag_row8 = [&](const E* m, int ld, int row0, int s, int kext) __attribute__((always_inline)) {
    return load_frag8<E>(m + (row0 + l16) * ld + 32 * s, quad, kext - 32 * s);
  };
  // (a bf16 column fragment is two transposing LDS reads, one per half of
  // 16 rows: in each 16-lane row of the wave, lane 4 e + j addresses the 4
  // elements at row k0 + e, columns col0 + 4 j .. + 3, and lane i receives
  // element i % 4 of the pieces that lanes 4 e + i / 4 address, e = 0..3,
  // that is column col0 + i at rows k0 .. k0 + 3; halves at or past kext
  // are zero. Otherwise it is read element by element: through an LDS-space
  // pointer, so its addresses are 32-bit, and unconditionally, with rows
  // past kext clamped and then zeroed, unless the whole step lies inside)
  auto frag_col = [&](const E* m, int ld, int col0, int s, int kext) __attribute__((always_inline)) {
    if constexpr (sizeof(E) == 2) {
      if (kext % 16 == 0) {
        typedef __attribute__((address_space(3))) bf16x4* TrPtr;
        E* mt = const_cast<E*>(m) + (32 * s + 4 * quad + (l16 >> 2)) * ld + col0 + 4 * (l16 & 3);
        Half<E> hv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          hv[h] = (32 * s + 16 * h < kext) ? __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TrPtr)(mt + 16 * h * ld))
                                           : zero_half<E>();
        return join<E>(hv[0], hv[1]);
      }
    }
    typedef const __attribute__((address_space(3))) E* LdsPtr;
    const LdsPtr ml = (LdsPtr)m;
    Frag<E> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = frag_k(s, quad, e);
      if (32 * s + 32 <= kext) {
        f[e] = ml[k * ld + col0 + l16];
      } else {
        const E x = ml[min(k, kext - 1) * ld + col0 + l16];
        f[e] = (k < kext) ? x : to_e<E>(0.f);
      }
    }
    return f;
  };

  // adds a value per row of the chunk to the wave's own row sums: lane
  // (quad, l16) holds v[4 rt + i] for row 16 rt + 4 quad + i; the row's 16
  // lanes are reduced in registers, then each lane adds one row's sum
  auto add_row_sums = [&](float* dst, const float (&v)[4 * CT]) __attribute__((always_inline)) {
    const float z = row_scatter_sum<4 * CT>(v, l16);
    if (CT == 4 || l16 < 4) atomicAdd(&dst[16 * (l16 >> 2) + 4 * quad + (l16 & 3)], z);
  };
  static_assert(CT == 4 || CT == 1, "row sums of one or four row tiles");

  f32x4 dQ[TPW], dK[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) { dQ[u] = zero4(); dK[u] = zero4(); }
  const Frag<E>* ktf = reinterpret_cast<const Frag<E>*>(a.key_t) + (c * a.h_qk + hq) * G::KT_FR * 64;
  const Frag<E>* qtf = reinterpret_cast<const Frag<E>*>(a.q_t) + (c * a.h_qk + hq) * G::KT_FR * 64;
  const Frag<E>* kff = reinterpret_cast<const Frag<E>*>(a.k_frag) + (c * a.h_qk + hq) * G::Q_FR * 64;

  // K K^T tiles (rt, it) of this wave's column tiles it = wave + NW j2:
  // the same for every V head of the group, so formed once
  f32x4 kkh[JPW][CT];
#pragma unroll
  for (int j2 = 0; j2 < JPW; ++j2) {
    const int it = wave + NW * j2;
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) kkh[j2][rt] = zero4();
    if (it >= CT) continue;
    Frag<E> kb[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) kb[ks] = kff[(it * DKS + ks) * 64 + lane];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) {
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) kkh[j2][rt] = mma(kff[(rt * DKS + ks) * 64 + lane], kb[ks], kkh[j2][rt]);
    }
  }

  for (int h = 0; h < a.group; ++h) {
    const int hv = hq * a.group + h;
    const int64_t ch = c * a.h_v + hv;
    // keeps the compiler from hoisting every lane-dependent address out of
    // this loop (they would stay live across it and spill); recomputing
    // them is a few ALU operations
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(quad), "+v"(l16));
    // restore their ranges, so that index products take 24-bit multiplies
    tid &= kGradBlock - 1; lane &= 63; quad &= 3; l16 &= 15;
    __syncthreads();                   // the previous V head's LDS reads are done
    // every global read of this phase and the next is requested before the
    // first wait: the gate tables, the dL/do, U and dU rows, Tinv^T, and the
    // first d-tile's state fragments and K, Q elements
    float gv = 0.f, bv = 0.f, eav = 0.f, edv = 0.f;
    if (tid < C) {
      gv = a.gate_prefix[ch * C + tid];
      bv = a.beta_chunk[ch * C + tid];
      eav = a.dtab[ch * (2 * C + 4) + tid];
      edv = a.dtab[ch * (2 * C + 4) + C + tid];
    }
    const float gl = a.dtab[ch * (2 * C + 4) + 2 * C];
    const Rows xo = load_rows(a.d_o, a.h_v, hv);
    const Rows xu = load_ws(static_cast<const E*>(a.ub) + ch * C * D);
    const Rows xd = load_ws(static_cast<const E*>(a.du) + ch * C * D);
    constexpr int TPT = (C * C / VE + kGradBlock - 1) / kGradBlock;   // Tinv^T rows, 16-byte loads
    VLoad xt[TPT];
    {
      const E* tg = static_cast<const E*>(a.tt) + ch * C * C;
#pragma unroll
      for (int p = 0; p < TPT; ++p) {
        const int idx = tid + p * kGradBlock;
        if (idx < C * C / VE) xt[p] = *reinterpret_cast<const VLoad*>(tg + idx * VE);
      }
    }
    // the state fragments of d-tile dt (chunk-start state S0 and dS_L, as
    // fragments of their transposes) and the K, Q elements of its tiles.
    // The products below contract them with rows staged in LDS, so both
    // operands take 8 consecutive columns per lane: one 16-byte load each
    const E* scg = static_cast<const E*>(a.sc) + ch * D * D;
    const E* dsg = static_cast<const E*>(a.dsl) + ch * D * D;
    Frag<E> bs[DKS], bl[DKS], qe[CKS], ke[CKS];
    auto load_dtile = [&](int dt) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
        bs[ks] = load_frag8<E>(scg + (16 * dt + l16) * D + 32 * ks, quad, D - 32 * ks);
        bl[ks] = load_frag8<E>(dsg + (16 * dt + l16) * D + 32 * ks, quad, D - 32 * ks);
      }
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        qe[s] = qtf[(dt * CKS + s) * 64 + lane];
        ke[s] = ktf[(dt * CKS + s) * 64 + lane];
      }
    };
    if (tid < C) {
      sm.g[tid] = gv;
      sm.b[tid] = bv;
      sm.ea[tid] = eav;
      sm.ed[tid] = edv;
#pragma unroll
      for (int w = 0; w < NW; ++w) { sm.dgw[w][tid] = 0.f; sm.dbw[w][tid] = 0.f; }
    }
    if (tid < 2 * NW) sm.sumw[tid / 2][tid % 2] = 0.f;
    store_rows(sm.u1.r1, xo, true);
    store_rows(sm.r2, xu, false);
    store_rows(sm.r3, xd, false);
#pragma unroll
    for (int p = 0; p < TPT; ++p) {
      const int idx = tid + p * kGradBlock;
      if (idx < C * C / VE) *reinterpret_cast<VLoad*>(&sm.tt[(idx * VE / C) * TLD + (idx * VE) % C]) = xt[p];
    }
    __syncthreads();

    // dO S0^T, U dS_L^T, -dU S0^T and <S0, dS_L>; the row terms of dg are
    // summed over the wave's d-tiles before the lane reductions
    f32x4 dW[TPW], prow[CT];
    float fro = 0.f, pk_all = 0.f;
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) prow[rt] = zero4();
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int dt = wave + NW * j;
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) dW[j * CT + rt] = zero4();
      if (dt >= DT) continue;
      load_dtile(dt);
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) fro += to_f(bs[ks][e]) * to_f(bl[ks][e]);
      }
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        const int u = j * CT + rt;
        f32x4 aq = zero4(), ak = zero4(), aw = zero4();
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) {
          aq = mma(frag_row8(sm.u1.r1, KLD, 16 * rt, ks, D), bs[ks], aq);
          ak = mma(frag_row8(sm.r2, KLD, 16 * rt, ks, D), bl[ks], ak);
          aw = mma(frag_row8(sm.r3, KLD, 16 * rt, ks, D), bs[ks], aw);
        }
        dW[u] = -aw;
        // K and Q elements (16 rt + 4 quad + i, 16 dt + l16): fragment
        // (dt, rt/2) of K^T or Q^T holds them at element i (+4 for an odd rt)
        f32x4 qv, kv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qv[i] = to_f(qe[rt >> 1][i + 4 * (rt & 1)]);
          kv[i] = to_f(ke[rt >> 1][i + 4 * (rt & 1)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * quad + i;
          const float eq = aq[i] * sm.ea[r], ek = ak[i] * sm.ed[r];
          dQ[u][i] += eq;
          dK[u][i] += ek;
          const float pk = ek * kv[i];
          prow[rt][i] += eq * qv[i] - pk;
          pk_all += pk;
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // one d-tile's operands live at a time
    }
    // the dP phase's P^T fragments, requested before the row sums
    const Frag<E>* ptf = reinterpret_cast<const Frag<E>*>(a.pt) + ch * G::QK_FR * 64;
    if (has_dt) {
      float prv[4 * CT];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) prv[4 * rt + i] = prow[rt][i];
      }
      add_row_sums(sm.dgw[wave], prv);
      fro = sum_rows4(sum16(fro));
      pk_all = sum_rows4(sum16(pk_all));
      if (lane == 0) {
        atomicAdd(&sm.sumw[wave][0], fro);
        atomicAdd(&sm.sumw[wave][1], pk_all);
      }
    }

    // dP = dO U^T: dP * P into dg, dPm = dP * Dincl into x1 (input dtype)
#pragma unroll
    for (int j2 = 0; j2 < JPW; ++j2) {
      const int jt = wave + NW * j2;
      if (jt >= CT) continue;
      Frag<E> pvf[CKS], ub[DKS];
#pragma unroll
      for (int s2 = 0; s2 < CKS; ++s2) pvf[s2] = ptf[(jt * CKS + s2) * 64 + lane];
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) ub[ks] = frag_row8(sm.r2, KLD, 16 * jt, ks, D);
      const int j = 16 * jt + l16;
      float colp = 0.f, m2v[4 * CT];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) acc = mma(frag_row8(sm.u1.r1, KLD, 16 * rt, ks, D), ub[ks], acc);
        // P[r][j] for this tile's elements: fragment (jt, rt/2) of P^T holds
        // row 16 rt + 4 quad + i at element i (+4 for an odd rt)
        const Frag<E> pv = pvf[rt >> 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * quad + i;
          const float m2 = acc[i] * to_f(pv[i + 4 * (rt & 1)]);
          m2v[4 * rt + i] = m2;
          colp += m2;
          const float gm = (j <= r && r < len) ? __expf(fminf(sm.g[r] - sm.g[j], 0.f)) : 0.f;
          sm.x1[r * ELD + j] = to_e<E>(acc[i] * gm);
        }
      }
      add_row_sums(sm.dgw[wave], m2v);
      colp = sum_rows4(colp);
      if (quad == 0) atomicAdd(&sm.dgw[wave][j], -colp);
    }
    __syncthreads();                   // x1 complete; dL/do and U rows dead
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int dt = wave + NW * j;
      if (dt >= DT) continue;
      Frag<E> kb[CKS], qb[CKS];
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        kb[s] = ktf[(dt * CKS + s) * 64 + lane];
        qb[s] = qtf[(dt * CKS + s) * 64 + lane];
      }
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        const int u = j * CT + rt;
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.r2[(16 * rt + 4 * quad + i) * KLD + 16 * dt + l16] = to_e<E>(dW[u][i]);
        // dQ += dPm K, dK += dPm^T Q
#pragma unroll
        for (int s = 0; s < CKS; ++s) {
          dQ[u] = mma(frag_row(sm.x1, ELD, 16 * rt, s, C), kb[s], dQ[u]);
          dK[u] = mma(frag_col(sm.x1, ELD, 16 * rt, s, C), qb[s], dK[u]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_rows(sm.u1.r1, load_rows(a.v, a.h_v, hv), true);
    __syncthreads();                   // v rows and dW rows complete; x1 dead

    // dT = (dU V^T) diag(b) + (dW K^T) diag(b ea) into x1
#pragma unroll
    for (int j2 = 0; j2 < JPW; ++j2) {
      const int it = wave + NW * j2;
      if (it >= CT) continue;
      Frag<E> vb[DKS];
      Frag<E> kb[DKS];
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) kb[ks] = kff[(it * DKS + ks) * 64 + lane];
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) vb[ks] = frag_row8(sm.u1.r1, KLD, 16 * it, ks, D);
      const int i = 16 * it + l16;
      const float bi = sm.b[i], bgi = sm.b[i] * sm.ea[i];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        f32x4 a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks) {
          a1 = mma(frag_row8(sm.r3, KLD, 16 * rt, ks, D), vb[ks], a1);
          a2 = mma(frag_row(sm.r2, KLD, 16 * rt, ks, D), kb[ks], a2);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.x1[(16 * rt + 4 * quad + e) * ELD + i] = to_e<E>(a1[e] * bi + a2[e] * bgi);
      }
    }
    __syncthreads();                   // x1 = dT complete; v rows dead
    // Y = dT Tinv^T over the v rows' buffer; Tinv^T (k = m, column i) is
    // read down tt's columns, once per column tile
#pragma unroll
    for (int j2 = 0; j2 < JPW; ++j2) {
      const int it = wave + NW * j2;
      if (it >= CT) continue;
      Frag<E> tb[CKS];
#pragma unroll
      for (int s = 0; s < CKS; ++s) tb[s] = frag_col(sm.tt, TLD, 16 * it, s, C);
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < CKS; ++s) acc = mma(frag_row(sm.x1, ELD, 16 * rt, s, C), tb[s], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) ys[(16 * rt + 4 * quad + e) * ELD + 16 * it + l16] = to_e<E>(acc[e]);
      }
    }
    __syncthreads();
    // dA = -Tinv^T Y (strictly lower), K K^T; b and g terms of A; B is
    // strictly lower, so B + B^T is written as B at (r, i) and at (i, r)
#pragma unroll
    for (int j2 = 0; j2 < JPW; ++j2) {
      const int it = wave + NW * j2;
      if (it >= CT) continue;
      Frag<E> yb[CKS];
#pragma unroll
      for (int s = 0; s < CKS; ++s) yb[s] = frag_col(ys, ELD, 16 * it, s, C);
      const int i = 16 * it + l16;
      float colm = 0.f, rdbv[4 * CT], rdgv[4 * CT];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        f32x4 acc = zero4();
        const f32x4 kk = kkh[j2][rt];
#pragma unroll
        for (int s = 0; s < CKS; ++s) acc = mma(frag_row(sm.tt, TLD, 16 * rt, s, C), yb[s], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * quad + e;
          const bool lower = i < r && r < len;
          const float gm = lower ? __expf(fminf(sm.g[r] - sm.g[i], 0.f)) : 0.f;
          const float da = lower ? -acc[e] : 0.f;
          const float bm = da * sm.b[r] * gm;
          const float mb2 = bm * kk[e];
          rdbv[4 * rt + e] = da * kk[e] * gm;
          rdgv[4 * rt + e] = mb2;
          colm += mb2;
          if (i < r) {
            sm.x1[r * ELD + i] = to_e<E>(bm);
            sm.x1[i * ELD + r] = to_e<E>(bm);
          } else if (i == r) {
            sm.x1[r * ELD + i] = to_e<E>(0.f);
          }
        }
      }
      add_row_sums(sm.dbw[wave], rdbv);
      add_row_sums(sm.dgw[wave], rdgv);
      colm = sum_rows4(colm);
      if (quad == 0) atomicAdd(&sm.dgw[wave][i], -colm);
    }
    __syncthreads();
    // dK += (B + B^T) K; dV = diag(b) Tinv^T dU and its b term (v read from
    // global); Tinv^T dW into dK and the b, g terms of W. dv is staged in
    // the wave's own dU columns (which only this wave reads here, before it
    // writes them) and stored as 16-byte row pieces after the products: the
    // wave's loads wait on its earlier stores as well (one counter for both),
    // so no store goes out between them
    // this chunk's rows of dv and v for this V head, as raw buffers
    const uint32_t v_row = (uint32_t)(a.h_v * D);    // elements between consecutive tokens
    const uint32_t v_bytes = (uint32_t)len * v_row * (uint32_t)sizeof(E);
    const auto dvb = raw_rsrc(static_cast<E*>(a.dv) + ((int64_t)start * a.h_v + hv) * D, v_bytes);
    const auto vb_ = raw_rsrc(static_cast<const E*>(a.v) + ((int64_t)start * a.h_v + hv) * D, v_bytes);
    f32x4 rdb_acc[CT], rdg_acc[CT];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) { rdb_acc[rt] = zero4(); rdg_acc[rt] = zero4(); }
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int dt = wave + NW * j;
      if (dt >= DT) continue;
      Frag<E> kb[CKS], ub[CKS], wb[CKS];
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        kb[s] = ktf[(dt * CKS + s) * 64 + lane];
        ub[s] = frag_col(sm.r3, KLD, 16 * dt, s, C);
        wb[s] = frag_col(sm.r2, KLD, 16 * dt, s, C);
      }
      const int d = 16 * dt + l16;
      // byte offset of (row 4 quad, column d); each row adds the uniform row
      // stride. The d-tile's v elements are requested before its products.
      const uint32_t lane_off = ((uint32_t)(4 * quad) * v_row + (uint32_t)d) * (uint32_t)sizeof(E);
      E vq[CT][4];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vq[rt][e] = buf_load<E>(vb_, lane_off + (uint32_t)(16 * rt + e) * v_row * (uint32_t)sizeof(E));
      }
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
        const int u = j * CT + rt;
        f32x4 au = zero4(), aw = zero4();
#pragma unroll
        for (int s = 0; s < CKS; ++s) {
          dK[u] = mma(frag_row(sm.x1, ELD, 16 * rt, s, C), kb[s], dK[u]);
          const Frag<E> ta = frag_row(sm.tt, TLD, 16 * rt, s, C);
          au = mma(ta, ub[s], au);
          aw = mma(ta, wb[s], aw);
        }
        // K elements (16 rt + 4 quad + e, d): fragment (dt, rt/2) of K^T is kb[rt/2]
        f32x4 kv;
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = to_f(kb[rt >> 1][e + 4 * (rt & 1)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * quad + e;
          const float bgr = sm.b[r] * sm.ea[r];
          // (rows at or past len fall outside the descriptor: v reads as 0)
          const float vv = to_f(vq[rt][e]);
          sm.r3[r * KLD + d] = to_e<E>(sm.b[r] * au[e]);
          dK[u][e] += bgr * aw[e];
          const float rk = aw[e] * kv[e];
          rdb_acc[rt][e] += au[e] * vv + sm.ea[r] * rk;
          rdg_acc[rt][e] += bgr * rk;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      // the wave's dv columns, 16 bytes a lane (rows at or past len fall
      // outside the buffer and are dropped)
      constexpr int PPR = 16 / VE, NPC = (C * PPR + 63) / 64;
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        const int dt = wave + NW * j;
        if (dt >= DT) continue;
#pragma unroll
        for (int p = 0; p < NPC; ++p) {
          const int pc = lane + 64 * p, row = pc / PPR, col = 16 * dt + (pc % PPR) * VE;
          if (pc < C * PPR)
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sm.r3[row * KLD + col]), dvb,
                                                   (int)(((uint32_t)row * v_row + (uint32_t)col) * sizeof(E)), 0, 0);
        }
      }
    }
    if (has_dt) {
      float sbv[4 * CT], sgv[4 * CT];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { sbv[4 * rt + e] = rdb_acc[rt][e]; sgv[4 * rt + e] = rdg_acc[rt][e]; }
      }
      add_row_sums(sm.dbw[wave], sbv);
      add_row_sums(sm.dgw[wave], sgv);
    }
    __syncthreads();
    if (tid < C) {
      // the waves' sums in wave order; the state terms go to the last row
      float tg = 0.f, tb = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) { tg += sm.dgw[w][tid]; tb += sm.dbw[w][tid]; }
      if (tid == len - 1) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) { s0 += sm.sumw[w][0]; s1 += sm.sumw[w][1]; }
        tg += gl * s0 + s1;
      }
      sm.dg[tid] = tg;
      sm.db[tid] = tb;
    }
    __syncthreads();
    if (wave == 0) {
      // dlog a: the suffix sums of dg within the chunk, as a wave-wide scan
      // (lane r holds row r; rows past len hold 0), in a fixed order
      // (lane addresses from this V head's opaque lane index, so that none
      // stays live across the loop)
      float acc = (lane < len) ? sm.dg[lane] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float x = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane + off) & 63) << 2, __float_as_int(acc)));
        if (lane + off < 64) acc += x;
      }
      if (lane < len) {
        a.dlog_alpha[(int64_t)(start + lane) * a.h_v + hv] = acc;
        a.dbeta[(int64_t)(start + lane) * a.h_v + hv] = sm.db[lane];
      }
    }
  }

  // this chunk's rows of dq and dk for this QK head: the tiles rounded to
  // E into the (now free) dL/do and U row buffers, then stored as 16-byte
  // row pieces through raw buffers (rows at or past len fall outside them
  // and are dropped)
  __syncthreads();                     // the last V head's LDS reads are done
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int dt = wave + NW * j;
    if (dt >= DT) continue;
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) {
      const int u = j * CT + rt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * quad + e;
        sm.u1.r1[r * KLD + 16 * dt + l16] = to_e<E>(dQ[u][e]);
        sm.r2[r * KLD + 16 * dt + l16] = to_e<E>(dK[u][e]);
      }
    }
  }
  __syncthreads();
  const uint32_t qk_row = (uint32_t)(a.h_qk * D);
  const uint32_t qk_bytes = (uint32_t)len * qk_row * (uint32_t)sizeof(E);
  const auto dqb = raw_rsrc(static_cast<E*>(a.dq) + ((int64_t)start * a.h_qk + hq) * D, qk_bytes);
  const auto dkb = raw_rsrc(static_cast<E*>(a.dk) + ((int64_t)start * a.h_qk + hq) * D, qk_bytes);
#pragma unroll
  for (int p = 0; p < SPT; ++p) {
    const int idx = tid + p * kGradBlock;
    const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
    if (idx < C * D / VE) {
      const int o = (int)(((uint32_t)r * qk_row + (uint32_t)d) * sizeof(E));
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sm.u1.r1[r * KLD + d]), dqb, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sm.r2[r * KLD + d]), dkb, o, 0, 0);
    }
  }
}

template <typename E, int D, int C>
hipError_t launch_backward_t(const PrefillArgs& a, hipStream_t s, int first, int last) {
  using G = Cfg<E, D, C>;
  for (int stage = first; stage <= last; ++stage) {
    switch (stage) {
      case 4:
        gdn_kb_dstate<E, D, C><<<dim3((unsigned)(a.num_seqs * a.h_v * G::NCB)), dim3(kDScanBlock), 0, s>>>(a);
        break;
      case 5:
        gdn_kb_grad<E, D, C><<<dim3((unsigned)a.max_chunks, (unsigned)a.h_qk), dim3(kGradBlock), 0, s>>>(a);
        break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_backward_e(const PrefillArgs& a, int d, int c, hipStream_t s, int first, int last) {
  if (d == 128 && c == 64) {
    if constexpr (std::is_same<E, float>::value) return hipErrorInvalidValue;
    else return launch_backward_t<E, 128, 64>(a, s, first, last);
  }
  if (d == 128 && c == 16) return launch_backward_t<E, 128, 16>(a, s, first, last);
  if (d == 16 && c == 64) return launch_backward_t<E, 16, 64>(a, s, first, last);
  if (d == 16 && c == 16) return launch_backward_t<E, 16, 16>(a, s, first, last);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward(const PrefillArgs& a, int dtype, int head_dim, int chunk, hipStream_t stream,
                           int first_stage, int last_stage) {
  // stages 1-3: the forward kernels with their backward outputs (the
  // workspace pointers for those are set in `a`)
  if (first_stage <= 3) {
    const hipError_t e = launch_prefill(a, dtype, head_dim, chunk, stream, first_stage, last_stage < 3 ? last_stage : 3);
    if (e != hipSuccess) return e;
  }
  const int f = first_stage > 4 ? first_stage : 4;
  if (last_stage < f) return hipSuccess;
  if (dtype == 1) return launch_backward_e<bf16_t>(a, head_dim, chunk, stream, f, last_stage);
  return launch_backward_e<float>(a, head_dim, chunk, stream, f, last_stage);
}

}  // namespace gdn
