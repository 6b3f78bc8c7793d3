// Prefill (gdn_chunk_fwd): the chunkwise WY-representation evaluation of the
// gated delta rule, page "Qwen3.8-Flash-Next 技术总结", section 2.1 (Gated
// DeltaNet). That section prints the token-serial update and says that the
// GPU algorithm turns the product of Householder-type transitions into block
// matrix products over chunks; the block formulas used here are derived from
// the first form of its update equation. For one V head and a chunk of L <= C
// tokens entering with state S0 (r, i index tokens in the chunk):
//
//   g_r    = sum_{j<=r} log a_j                          kernel 2 (kernel 1 in the backward pass)
//   A[r,i] = b_r (k_r . k_i) exp(g_r - g_i)  (i < r)     kernel 2
//   Tinv   = (I + A)^{-1}                                kernel 2
//   W      = Tinv diag(b exp(g)) K                       kernel 2
//   Ut     = Tinv diag(b) V                              kernel 3 (producer waves)
//   U      = Ut - W S0                                   kernel 3 (scan waves)
//   S_end  = exp(g_L) S0 + (exp(g_L - g) * K)^T U        kernel 3 (scan waves)
//   O      = diag(exp(g)) Q S0 + (Q K^T * Dincl) U       kernel 3 (scan waves)
//            Dincl[r,i] = exp(g_r - g_i) for i <= r, else 0
//
// The rows of U are the delta vectors u_r = b_r (v_r - a_r S_{r-1}^T k_r)
// of the token-serial form, and O is o_r = S_r^T q_r with the post-update
// state. Every column (dv index) of the state evolves independently, so the
// scan splits a head's state into 16-column slices. exp() is only ever taken
// of g_r - g_i with i <= r, a non-positive number.
//
// The forward pass is two launches. Kernel 2 runs once per (chunk, QK head):
// it lays out K^T and Q once for the group's V heads, forms q.k and K K^T
// once, and then each V head's gate prefix, inverse, W and masked q.k.
// Kernel 3 fuses the Ut construction, the inter-chunk state scan and the
// output products: Ut, U and the per-chunk states never leave the chip. The
// backward pass runs kernel 1 first (the chunk table, g, b and the fragments
// both directions need), then kernel 2's per-V-head form and the saving
// form of kernel 3.
//
// Fragment layouts (see gdn_device.h for the lane/element order): a
// "fragment" is 64 lanes x 8 elements; "frag (a, s)" of a matrix X means
// lane l holds row/col a*16 + l%16 and the 8 contraction indices of step s.
//   key_t [c][hq][D/16][C32] : frag (dt, s) of K^T   (row d,     k = token i)
//   tinv  [c][hv][C/16][C32] : frag (rt, s) of Tinv diag(b) (row r, k = token i)
//   w     [c][hv][C/16][D32] : frag (rt, s) of W     (row r,     k = d)
//   q_frag[c][hq][C/16][D32] : frag (nt, s) of Q     (row r,     k = d)
//   pmask [c][hv][C/16][C32] : frag (nt, s) of P = (q_r . k_j) exp(g_r - g_j) masked to
//                              j <= r < L (col r = query, k = key j)
// with C32 = ceil(C/32), D32 = ceil(D/32); entries past the chunk end are zero.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

namespace {

// --------------------------------------------------------------------------
// Kernel 1 (backward pass): per (chunk slot c, QK head hq): the chunk
// table, the in-chunk prefix sums of log a and the per-chunk b of the QK
// head's V heads, and the chunk's K^T, K, Q^T and query-indexed q.k
// fragments (shared by the QK head's V heads).
// Every group scans the per-sequence chunk counts ceil(L_n / C) to find
// which sequence owns slot c (slots past the last chunk are marked
// seq = -1); the groups of QK head 0 publish the table entry, and slot 0's
// the per-sequence first-chunk offsets. One wave per V head forms g with a
// wavefront prefix sum; past a partial chunk's end g repeats the last valid
// prefix (log a taken as 0) and b is 0. Two vertically adjacent accumulator
// tiles are a fragment as they stand, which is how the q.k fragments are
// written.
// --------------------------------------------------------------------------
// Which sequence owns chunk slot c: every thread of the block calls this
// (it synchronises the block) and gets (sequence, index in the sequence),
// or sequence -1 for a slot past the last chunk. It scans the per-sequence
// chunk counts ceil(L_n / C): in one wave for up to 64 sequences, else with
// a block scan in `scan` (kBlock ints). When `publish` is set the block
// writes the slot's chunk table entry, and slot 0's block also the
// per-sequence first-chunk offsets.
template <int C>
__device__ int2 locate_chunk(const PrefillArgs& a, int64_t c, bool publish, int* scan, int* hit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { hit[0] = -1; hit[1] = 0; }
  __syncthreads();
  int carry = 0;
  if (a.num_seqs <= 64) {
    // up to 64 sequences: one wave's prefix sum, lane n holding sequence n
    if (wave == 0) {
      int cnt = 0;
      if (lane < a.num_seqs) {
        const int2 r = seq_range(a, lane);
        cnt = (r.y - r.x + C - 1) / C;
      }
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int x = __shfl_up(incl, off);
        if (lane >= off) incl += x;
      }
      const int excl = incl - cnt;
      if (lane < a.num_seqs) {
        if (c >= excl && c < incl) { hit[0] = lane; hit[1] = (int)(c - excl); }
        if (c == 0 && publish) a.seq_chunk_offset[lane] = excl;
      }
      carry = __shfl(incl, 63);
    }
    __syncthreads();
  }
  for (int64_t base = 0; a.num_seqs > 64 && base < a.num_seqs; base += kBlock) {
    const int64_t n = base + tid;
    int cnt = 0;
    if (n < a.num_seqs) {
      const int2 r = seq_range(a, n);
      cnt = (r.y - r.x + C - 1) / C;
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {
      const int x = (tid >= off) ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    const int incl = carry + scan[tid];
    const int excl = incl - cnt;
    if (n < a.num_seqs) {
      if (c >= excl && c < incl) { hit[0] = (int)n; hit[1] = (int)(c - excl); }
      if (c == 0 && publish) a.seq_chunk_offset[n] = excl;
    }
    carry += scan[kBlock - 1];
    __syncthreads();
  }
  if (c == 0 && publish && tid == 0) a.seq_chunk_offset[a.num_seqs] = carry;
  const int n = hit[0], j = hit[1];
  if (publish && tid == 0) {
    int4* table = reinterpret_cast<int4*>(a.chunk_table);
    if (n < 0) {
      table[c] = make_int4(-1, 0, 0, 0);
    } else {
      const int2 sr = seq_range(a, n);
      const int st = sr.x + j * C;
      table[c] = make_int4(n, st, min(C, sr.y - st), j);
    }
  }
  return make_int2(n, j);
}

template <typename E, int D, int C>
struct PrepSmem {
  static constexpr int KLD = D + 8;    // row stride of the staged keys and queries
  E ks[C * KLD];
  E qs[C * KLD];
  int scan[kBlock];
  int hit[2];
};

template <typename E, int D, int C>
__global__ __launch_bounds__(kBlock) void gdn_k1_chunk_prep(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  using SM = PrepSmem<E, D, C>;
  constexpr int CT = G::CT, CKS = G::CKS, DKS = G::DKS, KLD = SM::KLD;
  constexpr int NW = kBlock / 64;
  constexpr int VE = 16 / (int)sizeof(E);                 // elements per 16-byte load
  typedef E VLoad __attribute__((ext_vector_type(VE)));
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, l16 = lane & 15;
  // the QK heads of one chunk slot, which read the same gate lines, are
  // consecutive logical ids and so share an XCD
  const int64_t lid = xcd_local_id(blockIdx.x, gridDim.x);
  const int64_t c = lid / a.h_qk;
  const int hq = (int)(lid % a.h_qk);
  const int2 loc = locate_chunk<C>(a, c, hq == 0, sm.scan, sm.hit);
  if (loc.x < 0) return;
  const int2 sr = seq_range(a, loc.x);
  const int start = sr.x + loc.y * C;
  const int len = min(C, sr.y - start);

  // the chunk's key and query rows: every load is issued before the first
  // is used (rows past the chunk end read its last row and are zeroed;
  // threads past the C x D block repeat its last load and store nothing)
  const E* kg = static_cast<const E*>(a.k);
  const E* qg = static_cast<const E*>(a.q);
  constexpr int NV = C * D / VE, NL = (NV + kBlock - 1) / kBlock;
  VLoad kv[NL], qv[NL];
#pragma unroll
  for (int p = 0; p < NL; ++p) {
    const int idx = min(tid + p * kBlock, NV - 1);
    const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
    const int64_t gi = ((int64_t)(start + min(r, len - 1)) * a.h_qk + hq) * D + d;
    kv[p] = *reinterpret_cast<const VLoad*>(kg + gi);
    qv[p] = *reinterpret_cast<const VLoad*>(qg + gi);
  }
  // gates: one wave per V head of the group, lane r holding token r
  for (int h = wave; h < a.group; h += NW) {
    const int hv = hq * a.group + h;
    // lanes past the chunk end read its last token and then take the no-op
    // values (a load under a branch would be waited for on its own)
    const int64_t gi = (int64_t)(start + min(lane, len - 1)) * a.h_v + hv;
    float g = a.log_alpha[gi], b = a.beta[gi];
    if (lane >= len) { g = 0.f; b = 0.f; }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float x = __shfl_up(g, off);
      if (lane >= off) g += x;
    }
    if (lane < C) {
      a.gate_prefix[(c * a.h_v + hv) * C + lane] = g;
      a.beta_chunk[(c * a.h_v + hv) * C + lane] = b;
    }
  }

#pragma unroll
  for (int p = 0; p < NL; ++p) {
    const int idx = tid + p * kBlock;
    const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
    if (r >= len) {
#pragma unroll
      for (int e = 0; e < VE; ++e) { kv[p][e] = to_e<E>(0.f); qv[p][e] = to_e<E>(0.f); }
    }
    if (idx < NV) {
      *reinterpret_cast<VLoad*>(&sm.ks[r * KLD + d]) = kv[p];
      *reinterpret_cast<VLoad*>(&sm.qs[r * KLD + d]) = qv[p];
    }
  }
  __syncthreads();

  // K^T fragments: frag (dt, s), lane row d, elements token i
  Frag<E>* ktg = reinterpret_cast<Frag<E>*>(a.key_t) + (c * a.h_qk + hq) * G::KT_FR * 64;
  for (int it = tid; it < G::KT_FR * 64; it += kBlock) {
    const int f = it / 64, ln = it % 64, dt = f / CKS, s = f % CKS, q4 = ln >> 4;
    const int d = 16 * dt + (ln & 15);
    Frag<E> v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = frag_k(s, q4, e);
      v[e] = (i < C) ? sm.ks[i * KLD + d] : to_e<E>(0.f);
    }
    ktg[it] = v;
  }
  {
    // K fragments (row r, k = d), Q^T fragments (row d, k = token r), and
    // the q.k products with the query as contraction index: fragment
    // (jt, s) is the pair of tiles Q_r K_j^T of query tiles 2s and 2s + 1
    // (zero before the key tile)
    Frag<E>* kfg = reinterpret_cast<Frag<E>*>(a.k_frag) + (c * a.h_qk + hq) * G::Q_FR * 64;
    for (int it = tid; it < G::Q_FR * 64; it += kBlock) {
      const int f = it / 64, ln = it % 64, nt = f / DKS, s = f % DKS;
      kfg[it] = load_frag<E>(&sm.ks[(16 * nt + (ln & 15)) * KLD + 32 * s], ln >> 4, D - 32 * s);
    }
    Frag<E>* qtg = reinterpret_cast<Frag<E>*>(a.q_t) + (c * a.h_qk + hq) * G::KT_FR * 64;
    for (int it = tid; it < G::KT_FR * 64; it += kBlock) {
      const int f = it / 64, ln = it % 64, dt = f / CKS, s = f % CKS, q4 = ln >> 4;
      const int d = 16 * dt + (ln & 15);
      Frag<E> v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = frag_k(s, q4, e);
        v[e] = (i < C) ? sm.qs[i * KLD + d] : to_e<E>(0.f);
      }
      qtg[it] = v;
    }
    Frag<E>* kqg = reinterpret_cast<Frag<E>*>(a.kq) + (c * a.h_qk + hq) * G::QK_FR * 64;
    for (int f = wave; f < G::QK_FR; f += NW) {
      const int jt = f / CKS, s = f % CKS;
      f32x4 t2[2] = {zero4(), zero4()};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rt = 2 * s + h;
        if (rt < jt || rt >= CT) continue;
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks)
          t2[h] = mma(load_frag<E>(&sm.qs[(16 * rt + l16) * KLD + 32 * ks], quad, D - 32 * ks),
                      load_frag<E>(&sm.ks[(16 * jt + l16) * KLD + 32 * ks], quad, D - 32 * ks), t2[h]);
      }
      kqg[f * 64 + lane] = acc_to_frag<E>(t2[0], t2[1]);
    }
  }
}

// --------------------------------------------------------------------------
// Kernel 2: A = strict_lower(b_r (k_r . k_i) exp(g_r - g_i)) and
// Tinv = (I + A)^{-1} for each (chunk, V head), and the operands the scan
// takes from them: the fragments of Tinv diag(b) (the right factor of Ut) and of
// W = Tinv diag(b exp(g)) K; also the V head's masked, decayed q.k
// fragments and the scan's row-factor table.
// K K^T is formed with MFMA from the staged keys; A's entries are made from
// the products' accumulators. A and Tinv share one C x C fp32 array in LDS
// (over the keys, which are dead by then): A's blocks below the diagonal
// stay in place, Tinv's diagonal blocks replace A's, and Tinv's blocks below
// the diagonal are stored transposed in the blocks above it, so that
// Tinv[r][i] sits at [i][r] when r's block is below i's. Tinv is assembled
// blockwise in fp32: the 16 x 16 diagonal blocks by forward substitution
// (one lane per column, the four blocks side by side in one wave), then the
// blocks below them in order of distance from the diagonal,
//   Tinv_ij = -Tinv_ii sum_{j<=m<i} A_im Tinv_mj,
// with fp32 16x16x4 MFMAs, one block per wave per distance. W^T = K^T
// (Tinv diag(b exp(g)))^T is contracted over tokens, wave w taking d-tiles
// 2w and 2w + 1, whose accumulator pairs are W's fragments (rt, w).
// One workgroup per (chunk, QK head) does the QK head's work once and then
// takes the group's V heads in turn; the backward pass's form reads kernel
// 1's outputs and also writes the operands of the gradient kernel.
// The fragments for the scan leave as non-temporal stores, each wave
// instruction a whole 1 KB block: the scan reads them much later (from HBM
// either way), and such stores leave alone the lines that the scan's
// warm-up has brought into L2, which matters while kernel 2 forms a later
// window beside the scan. (Partial-line writes, as the scan's outputs,
// measured slower with the same hint.)
// --------------------------------------------------------------------------

template <typename E, int D, int C>
struct InvSmem {
  using G = Cfg<E, D, C>;
  static constexpr int KLD = D + 8;    // row stride of the staged keys
  static constexpr int FLD = C + 4;    // fp32 row stride of the C x C array (spreads rows over banks)
  static constexpr int XLD = 20;       // row stride of the 16 x 16 scratch tiles
  union {
    E ks[C * KLD];                     // keys of the chunk, rows past its end zero
    float at[C * FLD];                 // A and Tinv (see above)
  } u;
  union {
    struct {
      int scan[kBlock];                // the chunk lookup's block scan (forward pass)
      int hit[2];
    } loc;
    float x[4][16 * XLD];              // one 16 x 16 scratch tile per wave (blocks below the diagonal)
    Frag<E> tbg[G::T_FR * 64];         // then the Tinv diag(b exp(g)) fragments
  } v;
  float gb[2][C] __attribute__((aligned(16)));   // g and b of the current V head
  float eg[C] __attribute__((aligned(16)));      // exp(g), zero past the chunk end
};

// Kernel 2's workgroups per CU: `want`, or fewer where its LDS allows
// fewer (fp32 operands at C = 64)
template <typename E, int D, int C>
constexpr int k2_occupancy(int want) {
  return (int)(160 * 1024 / sizeof(InvSmem<E, D, C>)) < want ? (int)(160 * 1024 / sizeof(InvSmem<E, D, C>)) : want;
}

// Lower tile t of a CT x CT tile grid (on and below the diagonal, row by
// row) -> its row and column tile.
__device__ __forceinline__ int2 lower_tile(int t) {
  int mi = 0;
  while ((mi + 1) * (mi + 2) / 2 <= t) ++mi;
  return make_int2(mi, t - mi * (mi + 1) / 2);
}

// The scan's row-factor table of one (chunk, V head): exp(g_r),
// exp(min(g_L - g_r, 0)) (both zero past the chunk end), exp(g_L); from g
// in sm.gb. exp(g_r) is also kept in sm.eg for the Tinv diag(b exp(g))
// fragments.
template <typename E, int D, int C>
__device__ __forceinline__ void write_row_factors(InvSmem<E, D, C>& sm, float* dtg, int len, int tid) {
  const float gl = sm.gb[0][len - 1];
  if (tid < C) {
    const float valid = (float)(tid < len);
    const float eg = __expf(sm.gb[0][tid]) * valid;
    dtg[tid] = eg;
    sm.eg[tid] = eg;
    dtg[C + tid] = __expf(fminf(gl - sm.gb[0][tid], 0.f)) * valid;
  } else if (tid < C + 4) {
    dtg[C + tid] = (tid == C) ? __expf(gl) : 0.f;
  }
}

// A from the K K^T tiles and this V head's g and b (sm.gb), the blocked
// inverse, and the Tinv diag(b) and W fragments of (chunk, V head) ch
// (backward form: also Tinv^T and the W^T fragments). Every thread of the
// block calls it; it synchronises the block. kk holds this wave's lower K K^T
// tiles (wave + NW u); kta, ktb the K^T fragments of its W d-tiles.
template <typename E, int D, int C, bool BW, int TPW>
__device__ __forceinline__ void k2_invert_and_write(InvSmem<E, D, C>& sm, const PrefillArgs& a, int64_t ch,
                                                    const f32x4 (&kk)[TPW], const Frag<E> (&kta)[Cfg<E, D, C>::CKS],
                                                    const Frag<E> (&ktb)[Cfg<E, D, C>::CKS], int tid, int lane,
                                                    int wave, int quad, int l16) {
  using G = Cfg<E, D, C>;
  using SM = InvSmem<E, D, C>;
  constexpr int CT = G::CT, CKS = G::CKS, DT = G::DT, DKS = G::DKS, FLD = SM::FLD, XLD = SM::XLD;
  constexpr int NW = kBlock / 64, NTILE = CT * (CT + 1) / 2;
  float* at = sm.u.at;
  // A = strict_lower(b_r (k_r . k_i) exp(g_r - g_i))
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave + u * NW;
    if (t >= NTILE) continue;
    const int2 tl = lower_tile(t);
    const int i = 16 * tl.y + l16, r0 = 16 * tl.x + 4 * quad;   // rows r0 .. r0 + 3
    const float gi = sm.gb[0][i];
    const f32x4 gr = *reinterpret_cast<const f32x4*>(&sm.gb[0][r0]);
    const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.gb[1][r0]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i < r0 + e) at[(r0 + e) * FLD + i] = br[e] * kk[u][e] * __expf(fminf(gr[e] - gi, 0.f));
    }
  }
  __syncthreads();
  // diagonal blocks: lanes 16b .. 16b + 15 of wave 0 solve block b, lane
  // 16b + j its column j; the block then holds Tinv's diagonal block
  if (wave == 0 && quad < CT) {
    const int j = l16, o = 16 * quad;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) {
        if (i & 1) s1 -= at[(o + r) * FLD + o + i] * x[i];
        else s0 -= at[(o + r) * FLD + o + i] * x[i];
      }
      x[r] = s0 + s1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) at[(o + r) * FLD + o + j] = x[r];
  }
  __syncthreads();
  // blocks below the diagonal, by distance; one block per wave per distance
#pragma unroll
  for (int dist = 1; dist < CT; ++dist) {
    for (int bi = dist + wave; bi < CT; bi += NW) {
      const int bj = bi - dist;
      float* X = sm.v.x[wave];
      f32x4 acc = zero4();
      for (int bm = bj; bm < bi; ++bm) {
        const float* Am = &at[(16 * bi) * FLD + 16 * bm];
        acc = (bm == bj) ? mma16_f32(Am, FLD, 1, &at[(16 * bj) * FLD + 16 * bj], FLD, 1, acc, lane)
                         : mma16_f32(Am, FLD, 1, &at[(16 * bj) * FLD + 16 * bm], 1, FLD, acc, lane);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) X[(4 * quad + e) * XLD + l16] = acc[e];
      acc = mma16_f32(&at[(16 * bi) * FLD + 16 * bi], FLD, 1, X, XLD, 1, zero4(), lane);
      // Tinv_ij, stored transposed: element (4 quad + e, l16) at [16 bj + l16][16 bi + 4 quad + e]
      *reinterpret_cast<f32x4*>(&at[(16 * bj + l16) * FLD + 16 * bi + 4 * quad]) = -acc;
    }
    __syncthreads();
  }
  if constexpr (BW) {
    // backward pass: Tinv^T row-major, tt[i][r] = Tinv[r][i]
    E* ttg = static_cast<E*>(a.tt) + ch * C * C;
    for (int idx = tid; idx < C * C; idx += kBlock) {
      const int i = idx / C, r = idx % C;
      const float t = ((r >> 4) > (i >> 4)) ? at[i * FLD + r] : (((r >> 4) == (i >> 4)) ? at[r * FLD + i] : 0.f);
      ttg[idx] = to_e<E>(t);
    }
  }
  // Tinv diag(b) fragments to the workspace, Tinv diag(b exp(g)) to LDS
  Frag<E>* tg = reinterpret_cast<Frag<E>*>(a.tinv) + ch * G::T_FR * 64;
  for (int it = tid; it < G::T_FR * 64; it += kBlock) {
    const int f = it / 64, ln = it % 64, rt = f / CKS, s = f % CKS, q4 = ln >> 4;
    if (causal_zero(rt, s)) continue;                // all zero; no product reads it
    const int r = 16 * rt + (ln & 15);
    Frag<E> vb, vg;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // elements 4 hh .. 4 hh + 3 of the fragment: tokens i0 .. i0 + 3, in
      // one 16-token block (b and exp(g) are zero past the chunk end, so
      // those tokens give zeros)
      const int i0 = 32 * s + 16 * hh + 4 * q4;
      f32x4 bi = zero4(), ei = zero4();
      if (i0 < C) {
        bi = *reinterpret_cast<const f32x4*>(&sm.gb[1][i0]);
        ei = *reinterpret_cast<const f32x4*>(&sm.eg[i0]);
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int i = i0 + e4;
        float t = 0.f;
        if (i < C) {
          const float tri = ((r >> 4) > (i >> 4)) ? at[i * FLD + r] : (((r >> 4) == (i >> 4)) ? at[r * FLD + i] : 0.f);
          t = tri * bi[e4];
        }
        vb[4 * hh + e4] = to_e<E>(t);
        vg[4 * hh + e4] = to_e<E>(t * ei[e4]);
      }
    }
    __builtin_nontemporal_store(vb, &tg[it]);
    sm.v.tbg[it] = vg;
  }
  __syncthreads();
  const int ksd = wave;
  if (ksd < DKS) {
    Frag<E>* wg = reinterpret_cast<Frag<E>*>(a.w) + ch * G::W_FR * 64;
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) {
      f32x4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        if (causal_zero(rt, s)) continue;              // Tinv is lower triangular
        const Frag<E> tb = sm.v.tbg[(rt * CKS + s) * 64 + lane];
        acc0 = mma(kta[s], tb, acc0);
        if (2 * ksd + 1 < DT) acc1 = mma(ktb[s], tb, acc1);
      }
      __builtin_nontemporal_store(acc_to_frag<E>(acc0, acc1), &wg[(rt * DKS + ksd) * 64 + lane]);
    }
    if constexpr (BW) {
      // backward pass: W^T fragments (dt, s), lane row d, elements token r:
      // the pair of W tiles (r-tiles 2s, 2s + 1; d-tile dt) formed as
      // Tinv diag(b exp(g)) K
      Frag<E>* wtg = reinterpret_cast<Frag<E>*>(a.wt) + ch * G::KT_FR * 64;
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        f32x4 pa[2] = {zero4(), zero4()}, pb[2] = {zero4(), zero4()};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rt = 2 * s + h;
          if (rt >= CT) continue;
#pragma unroll
          for (int s2 = 0; s2 < CKS; ++s2) {
            if (causal_zero(rt, s2)) continue;
            const Frag<E> tb = sm.v.tbg[(rt * CKS + s2) * 64 + lane];
            pa[h] = mma(tb, kta[s2], pa[h]);
            if (2 * ksd + 1 < DT) pb[h] = mma(tb, ktb[s2], pb[h]);
          }
        }
        wtg[((2 * ksd) * CKS + s) * 64 + lane] = acc_to_frag<E>(pa[0], pa[1]);
        if (2 * ksd + 1 < DT) wtg[((2 * ksd + 1) * CKS + s) * 64 + lane] = acc_to_frag<E>(pb[0], pb[1]);
      }
    }
  }
}

// the chunk's keys into sm.u.ks, all loads issued before the first is used
// (rows past the chunk end read its last row and are zeroed; threads past
// the C x D block repeat its last load and store nothing); P: raw keys,
// scaled to unit rows
template <typename E, int D, int C, bool P>
__device__ __forceinline__ void stage_keys(InvSmem<E, D, C>& sm, const PrefillArgs& a, int start, int len, int hq,
                                           int tid) {
  constexpr int VE = 16 / (int)sizeof(E), KLD = InvSmem<E, D, C>::KLD;
  typedef E VLoad __attribute__((ext_vector_type(VE)));
  const E* kg = static_cast<const E*>(a.k);
  constexpr int NV = C * D / VE, NL = (NV + kBlock - 1) / kBlock;
  VLoad kv[NL];
#pragma unroll
  for (int p = 0; p < NL; ++p) {
    const int idx = min(tid + p * kBlock, NV - 1);
    const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
    kv[p] = *reinterpret_cast<const VLoad*>(kg + ((int64_t)(start + min(r, len - 1)) * a.h_qk + hq) * D + d);
  }
#pragma unroll
  for (int p = 0; p < NL; ++p) {
    const int idx = tid + p * kBlock;
    const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
    if (r >= len) {
#pragma unroll
      for (int e = 0; e < VE; ++e) kv[p][e] = to_e<E>(0.f);
    }
    if constexpr (P) normalize_slice<E, D, VE>(kv[p]);
    if (idx < NV) *reinterpret_cast<VLoad*>(&sm.u.ks[r * KLD + d]) = kv[p];
  }
}

// K K^T tiles on and below the diagonal from the staged keys: wave w's
// lower tiles w + NW u
template <typename E, int D, int C, int TPW>
__device__ __forceinline__ void key_products(const InvSmem<E, D, C>& sm, f32x4 (&kk)[TPW], int wave, int quad,
                                             int l16) {
  using G = Cfg<E, D, C>;
  constexpr int DKS = G::DKS, KLD = InvSmem<E, D, C>::KLD, NW = kBlock / 64, NTILE = G::CT * (G::CT + 1) / 2;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave + u * NW;
    kk[u] = zero4();
    if (t < NTILE) {
      const int2 tl = lower_tile(t);
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks)
        kk[u] = mma(load_frag<E>(&sm.u.ks[(16 * tl.x + l16) * KLD + 32 * ks], quad, D - 32 * ks),
                    load_frag<E>(&sm.u.ks[(16 * tl.y + l16) * KLD + 32 * ks], quad, D - 32 * ks), kk[u]);
    }
  }
}

// One workgroup per (chunk, QK head). What depends only on the QK head is
// done once: the keys are staged, the K^T fragments gathered from them, and
// K K^T formed (kept in registers). Forward pass: also the chunk lookup, the
// K^T and Q fragments the scan reads, and the q.k products (kept in
// registers). The group's V heads are then taken in turn: the gate prefix
// (forward) or kernel 1's g and b (backward), the P fragments (forward) or
// the P^T fragments from kernel 1's query-indexed q.k (backward), the
// row-factor table, then A, the inverse, Tinv diag(b) and W. Each V head's
// gates are requested while the previous one is processed. (One workgroup
// per V head, each repeating the QK head's work, took 0.63 ms against
// 0.51 ms for the forward pass on the 64K-token layer.)
// bf16: five workgroups per CU, 26 KB of LDS and at most 96 VGPRs each
// WIN marks the launches of a window beside the scan (the same code under
// another name, so that traces keep them apart from whole launches)
template <typename E, int D, int C, bool P, bool ND, bool BW, bool WIN = false>
__global__ __launch_bounds__(kBlock, (k2_occupancy<E, D, C>(5))) void gdn_k2_inverse_w(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  using SM = InvSmem<E, D, C>;
  constexpr int CT = G::CT, CKS = G::CKS, DT = G::DT, DKS = G::DKS, KLD = SM::KLD;
  constexpr int NW = kBlock / 64, NTILE = CT * (CT + 1) / 2, TPW = (NTILE + NW - 1) / NW;
  constexpr int KQPT = (G::QK_FR * 64 + kBlock - 1) / kBlock;   // backward: q.k fragments per thread
  static_assert(DKS <= NW && CT <= 4, "one W d-step pair per wave, diagonal blocks in one wave");
  static_assert(!BW || (!P && !ND), "the backward pass takes no flags");
  __shared__ SM sm;
  // the QK heads of one chunk, which read the same gate lines, are
  // consecutive logical ids and so share an XCD
  const int64_t lid = xcd_local_id(blockIdx.x, gridDim.x);
  const int64_t c = a.win_lo + lid / a.h_qk;   // this launch's window of chunk slots
  const int hq = (int)(lid % a.h_qk);
  // lane indices are re-made opaque at the top of every V head's pass (see
  // there); the wave index is uniform
  int tid = threadIdx.x, lane = tid & 63, quad = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int start, len;
  if constexpr (BW) {
    const int4 tab = reinterpret_cast<const int4*>(a.chunk_table)[c];
    if (tab.x < 0) return;
    start = tab.y;
    len = tab.z;
  } else {
    const int2 loc = locate_chunk<C>(a, c, hq == 0, sm.v.loc.scan, sm.v.loc.hit);
    if (loc.x < 0) return;
    const int2 sr = seq_range(a, loc.x);
    start = sr.x + loc.y * C;
    len = min(C, sr.y - start);
  }

  // forward pass: wave w's query tile w, its Q fragments straight from q
  // (rows past the chunk end read its last row and are zeroed below)
  Frag<E> qf[DKS];
  if (!BW && wave < CT) {
    const E* row = static_cast<const E*>(a.q) + ((int64_t)(start + min(16 * wave + l16, len - 1)) * a.h_qk + hq) * D;
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) qf[ks] = load_frag<E>(row + 32 * ks, quad, D - 32 * ks);
  }
  // the gates of V head h of the group, wave 0: forward, log a and b with
  // lane r holding token r (lanes past the chunk end read its last token);
  // backward, kernel 1's g and b of chunk row r
  float gw = 0.f, bw = 0.f;
  auto load_gates = [&](int h) __attribute__((always_inline)) {
    if constexpr (BW) {
      const int64_t o = (c * a.h_v + hq * a.group + h) * C + min(lane, C - 1);
      gw = a.gate_prefix[o];
      bw = a.beta_chunk[o];
    } else {
      const int64_t gi = (int64_t)(start + min(lane, len - 1)) * a.h_v + hq * a.group + h;
      gw = a.log_alpha[gi];
      bw = a.beta[gi];
    }
  };
  if (wave == 0) load_gates(0);
  // backward pass: kernel 1's query-indexed q.k fragments, kept for every V head
  Frag<E> kqf[KQPT];
  if constexpr (BW) {
    const Frag<E>* kqg = reinterpret_cast<const Frag<E>*>(a.kq) + (c * a.h_qk + hq) * G::QK_FR * 64;
#pragma unroll
    for (int p = 0; p < KQPT; ++p) kqf[p] = kqg[min(tid + p * kBlock, G::QK_FR * 64 - 1)];
  }
  stage_keys<E, D, C, P>(sm, a, start, len, hq, tid);
  __syncthreads();

  // K^T fragments (row d, k = token) of this wave's W d-tiles, gathered
  // from the staged keys; the forward pass writes them for the scan (the
  // waves' d-tiles cover all of them; kernel 1 wrote them in the backward)
  const int ksd = wave;
  Frag<E> kta[CKS], ktb[CKS];
  if (ksd < DKS) {
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = frag_k(s, quad, e);
        kta[s][e] = (i < C) ? sm.u.ks[i * KLD + 32 * ksd + l16] : to_e<E>(0.f);
        if (2 * ksd + 1 < DT) ktb[s][e] = (i < C) ? sm.u.ks[i * KLD + 32 * ksd + 16 + l16] : to_e<E>(0.f);
      }
    }
    if constexpr (!BW) {
      Frag<E>* ktg = reinterpret_cast<Frag<E>*>(a.key_t) + (c * a.h_qk + hq) * G::KT_FR * 64;
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        __builtin_nontemporal_store(kta[s], &ktg[((2 * ksd) * CKS + s) * 64 + lane]);
        if (2 * ksd + 1 < DT) __builtin_nontemporal_store(ktb[s], &ktg[((2 * ksd + 1) * CKS + s) * 64 + lane]);
      }
    }
  }
  // forward pass: q.k of query tile nt = wave, the pair of accumulator
  // tiles K_j Q_r^T of key tiles 2s and 2s + 1 (a key tile after the query
  // tile stays zero); the Q fragments are written for the scan
  const int nt = wave;
  int rq = 16 * nt + l16;
  f32x4 qk[CKS][2];
#pragma unroll
  for (int s = 0; s < CKS; ++s) { qk[s][0] = zero4(); qk[s][1] = zero4(); }
  if (!BW && wave < CT) {
    if (rq >= len) {
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) qf[ks] = join<E>(zero_half<E>(), zero_half<E>());
    }
    if constexpr (P) {
      // raw queries: the four lanes holding a row (one per quad) add their
      // sums of squares, then scale it to unit length
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += to_f(qf[ks][e]) * to_f(qf[ks][e]);
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float inv = inv_norm(ss);
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = to_e<E>(to_f(qf[ks][e]) * inv);
      }
    }
    Frag<E>* qfg = reinterpret_cast<Frag<E>*>(a.q_frag) + (c * a.h_qk + hq) * G::Q_FR * 64;
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) __builtin_nontemporal_store(qf[ks], &qfg[(nt * DKS + ks) * 64 + lane]);
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
      if (causal_zero(nt, s)) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kt = 2 * s + h;
        if (kt > nt || kt >= CT) continue;
#pragma unroll
        for (int ks = 0; ks < DKS; ++ks)
          qk[s][h] = mma(load_frag<E>(&sm.u.ks[(16 * kt + l16) * KLD + 32 * ks], quad, D - 32 * ks), qf[ks], qk[s][h]);
      }
    }
  }
  f32x4 kk[TPW];
  if constexpr (!ND) key_products<E, D, C, TPW>(sm, kk, wave, quad, l16);
  __syncthreads();     // the keys are dead from here on; their LDS holds A and Tinv

  for (int h = 0; h < a.group; ++h) {
    const int64_t ch = c * a.h_v + hq * a.group + h;
    // keeps the compiler from hoisting every lane-dependent LDS address out
    // of this loop (they would stay live across it and spill); recomputing
    // them is a few ALU operations. The masks restore their ranges.
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(quad), "+v"(l16), "+v"(rq));
    tid &= kBlock - 1; lane &= 63; quad &= 3; l16 &= 15; rq &= 63;
    if (wave == 0) {
      if constexpr (BW) {
        if (lane < C) { sm.gb[0][lane] = gw; sm.gb[1][lane] = bw; }
      } else {
        // in-chunk prefix of log a (past the chunk end: log a = 0, b = 0)
        float g = gw, b = bw;
        if constexpr (P) { g = neg_softplus(g); b = sigmoid_of(b); }
        if (lane >= len) { g = 0.f; b = 0.f; }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float x = __shfl_up(g, off);
          if (lane >= off) g += x;
        }
        if (lane < C) { sm.gb[0][lane] = g; sm.gb[1][lane] = b; }
      }
      if (h + 1 < a.group) load_gates(h + 1);
    }
    // (also: the previous V head's last readers of g, b and the LDS
    // fragments are done)
    __syncthreads();
    if constexpr (BW) {
      // P^T fragments (jt, s), lane row key j, elements query r
      Frag<E>* ptg = reinterpret_cast<Frag<E>*>(a.pt) + ch * G::QK_FR * 64;
#pragma unroll
      for (int p = 0; p < KQPT; ++p) {
        const int it = tid + p * kBlock;
        if (it >= G::QK_FR * 64) continue;
        const int f = it / 64, ln = it % 64, jt = f / CKS, s = f % CKS, q4 = ln >> 4;
        const int j = 16 * jt + (ln & 15);
        const float gj = sm.gb[0][j];
        Frag<E> v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = frag_k(s, q4, e);
          const float m = (float)(j <= r && r < len);
          v[e] = to_e<E>(to_f(kqf[p][e]) * (__expf(fminf(sm.gb[0][min(r, C - 1)] - gj, 0.f)) * m));
        }
        ptg[it] = v;
      }
    } else if (wave < CT) {
      // the scan's P fragments: P[r][j] = (q_r . k_j) exp(g_r - g_j) for
      // j <= r < len, else 0 (the exponent is clamped at 0 so that masked
      // entries cannot overflow before being zeroed)
      Frag<E>* pg = reinterpret_cast<Frag<E>*>(a.pmask) + ch * G::QK_FR * 64;
      const float gr = sm.gb[0][rq], vr = (float)(rq < len);
#pragma unroll
      for (int s = 0; s < CKS; ++s) {
        if (causal_zero(nt, s)) continue;            // all zero; the scan neither copies nor reads it
        Frag<E> v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = frag_k(s, quad, e);
          const float m = (float)(j <= rq) * vr;
          v[e] = to_e<E>(qk[s][e >> 2][e & 3] * (__expf(fminf(gr - sm.gb[0][min(j, C - 1)], 0.f)) * m));
        }
        __builtin_nontemporal_store(v, &pg[(nt * CKS + s) * 64 + lane]);
      }
    }
    write_row_factors(sm, a.dtab + ch * (2 * C + 4), len, tid);
    if constexpr (ND) {
      // gate-only variant: no delta rule, so Tinv = I; the scan's Ut = diag(b) V
      // takes diag(b) in place of Tinv diag(b), and W is not used
      Frag<E>* tg = reinterpret_cast<Frag<E>*>(a.tinv) + ch * G::T_FR * 64;
      for (int it = tid; it < G::T_FR * 64; it += kBlock) {
        const int f = it / 64, ln = it % 64, rt = f / CKS, s = f % CKS, q4 = ln >> 4;
        if (causal_zero(rt, s)) continue;            // all zero; the scan neither copies nor reads it
        const int r = 16 * rt + (ln & 15);
        Frag<E> vb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = frag_k(s, q4, e);
          vb[e] = to_e<E>((i == r) ? sm.gb[1][r] : 0.f);
        }
        tg[it] = vb;
      }
      __syncthreads();   // the next V head's prefix overwrites g and b
    } else {
      k2_invert_and_write<E, D, C, BW, TPW>(sm, a, ch, kk, kta, ktb, tid, lane, wave, quad, l16);
    }
  }
}

// --------------------------------------------------------------------------
// Kernel 3: fused Ut construction, inter-chunk state scan and outputs.
// One workgroup per (sequence, V head, block of BV state columns), twelve
// waves, looping over the sequence's chunks in order with one barrier per
// chunk:
//   scan waves (one per 16-column slice) process chunk c: with the slice of
//     the state S (D x 16 fp32) held in MFMA accumulators for the whole
//     sequence,
//       O^T  = diag(exp(g)) applied to S^T Q^T      (inter-chunk output)
//       U    = Ut - W S                            (S's accumulator tiles are
//                                                   the B fragments here)
//       O^T += U^T P^T, P = (Q K^T * Dincl)         (U's tiles are the A fragments)
//       S    = exp(g_L) S + K^T (exp(g_L - g) * U)
//     and leave the chunk's (bf16) outputs in their slice's Ut slot: the
//     scan waves touch no global memory per chunk;
//   Ut waves (one per slice), meanwhile, read chunk c-1's outputs from their
//     slot, form chunk c+1's Ut tiles Tinv diag(b) V there, store the
//     outputs, and warm L2 for chunk c+3;
//   loader waves copy chunk c+1's K^T, W, Q and P fragments and row-factor
//     table, and chunk c+2's Tinv diag(b) fragments and V columns, from
//     global memory straight into LDS (direct global-to-LDS loads, 1 KB per
//     wave instruction, no register staging) and wait for them before the
//     barrier.
// Every LDS region is double-buffered by chunk parity; between two barriers
// a slot is either only read or only written, except a Ut slot, which its
// one Ut wave reads and then writes, in program order.
// --------------------------------------------------------------------------
constexpr int kScanBlock = 768;

template <typename E, int D, int C>
struct ScanCfg {
  using G = Cfg<E, D, C>;
  // fp32 operands at head dim 128 with 64-token chunks do not fit two slots
  // per region in LDS: there the workgroup takes one 16-column slice, each
  // operand region has one slot, and every iteration has a compute phase and
  // a copy phase separated by a barrier
  static constexpr bool WIDE = sizeof(E) == 4 && D == 128 && C == 64;
  static constexpr int NS = WIDE ? 1 : G::NS;      // 16-column state slices per workgroup
  static constexpr int BV = 16 * NS;               // state columns per workgroup
  static constexpr int NCB = D / BV;               // workgroups per (sequence, V head)
  static constexpr int NB = WIDE ? 1 : 2;          // slots per operand region
};

template <typename E, int D, int C>
struct ScanSmem {
  using G = Cfg<E, D, C>;
  using SC = ScanCfg<E, D, C>;
  static constexpr int NB = SC::NB;
  Frag<E> kt[NB][G::KT_FR * 64];       // K^T fragments
  Frag<E> wf[NB][G::W_FR * 64];        // W fragments
  Frag<E> qf[NB][G::Q_FR * 64];        // Q fragments
  Frag<E> pf[NB][G::QK_FR * 64];       // masked, decayed q.k fragments
  Frag<E> tf[NB][G::T_FR * 64];        // Tinv diag(b) fragments
  f32x4 uf[2][SC::NS * G::CT * 64];    // Ut accumulator tiles
  E vr[NB][C * SC::BV];                // the block's V columns, row-major
  // exp(g_r) [C], exp(min(g_L - g_r, 0)) [C], exp(g_L), 3 pad
  float dtab[NB][2 * C + 4] __attribute__((aligned(16)));
  float touch[kScanBlock / 64][64];    // landing place of the L2 warm-up loads
};

// WIN: as for kernel 2
template <typename E, int D, int C, bool ND, bool SV, bool WIN = false>
__global__ __launch_bounds__(kScanBlock) void gdn_k3_scan(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  using SC = ScanCfg<E, D, C>;
  constexpr int DT = G::DT, CT = G::CT, DKS = G::DKS, CKS = G::CKS, NS = SC::NS, BV = SC::BV, NCB = SC::NCB;
  constexpr int NB = SC::NB;
  static_assert(sizeof(ScanSmem<E, D, C>) <= 160 * 1024, "scan LDS");
  // operand region slot of chunk x (the Ut tiles always alternate)
  auto slot = [](int x) { return NB == 2 ? (x & 1) : 0; };
  // roles: NS scan waves, NS Ut waves, and loader waves (direct copies only,
  // so that their stalls on the memory pipeline hold up nothing else)
  constexpr int NLD = kScanBlock / 64 - 2 * NS;
  // bf16 outputs leave through LDS and the Ut waves (the fp32 ones from the
  // scan waves' registers)
  constexpr bool STAGE_O = std::is_same<E, bf16_t>::value;
  // the saving form's S and U rows: staged in the (here unused) Q and P
  // fragment buffers by the scan waves, double-buffered by chunk parity, and
  // stored by the slice's Ut wave in the next iteration, where they fit
  constexpr int SLD = staged_ld<E>(), SV_AREA = (D + C) * SLD;
  constexpr bool SV_STAGE =
      SV && 2 * NS * SV_AREA * (int)sizeof(E) <= (int)(sizeof(ScanSmem<E, D, C>::qf) + sizeof(ScanSmem<E, D, C>::pf)) &&
      D % StagedRows<E>::RPI == 0 && C % StagedRows<E>::RPI == 0;
  constexpr int FB = (int)sizeof(Frag<E>) * 64;            // bytes per fragment
  constexpr int ESZ = (int)sizeof(E);
  __shared__ ScanSmem<E, D, C> sm;
  const int tid = threadIdx.x, lane = tid & 63, quad = lane >> 4, l16 = lane & 15;
  // the wave index in a scalar register, so that role and job selection
  // compile to scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the column blocks and V heads of one QK head, which read the same K^T
  // and Q fragments, are consecutive logical ids and so share an XCD
  const int64_t bid = xcd_local_id(blockIdx.x, gridDim.x);
  const int cb = (int)(bid % NCB);
  const int hv = (int)((bid / NCB) % a.h_v);
  const int64_t n = bid / ((int64_t)NCB * a.h_v);
  const int hq = hv / a.group;
  const int2 cr = chunk_range(a, n), sr = seq_range(a, n);
  const int c0 = cr.x, c1 = cr.y;
  // the sequence's chunks in this launch's window of chunk slots: where the
  // sequence began in an earlier window its state enters from final_state,
  // and where it continues in a later one its state is left there
  const int lo = max(c0, (int)a.win_lo), hi = min(c1, (int)a.win_hi);
  const bool carried_in = lo > c0;
  // chunk x of this sequence starts at seq_start + (x - c0) * C; computing
  // start and length here keeps table reads off the per-chunk critical path
  const int seq_start = sr.x, seq_end = sr.y;
  auto chunk_start = [&](int x) { return seq_start + (x - c0) * C; };
  auto chunk_len = [&](int x) { return min(C, seq_end - chunk_start(x)); };
  const bool is_scan = wave < NS, is_loader = !is_scan && wave < NS + NLD;
  const int slice = wave;                      // scan waves: slice index
  const int lw = wave - NS;                    // loader waves: index
  const int uw = wave - NS - NLD;              // Ut waves: slice index
  const int col0 = cb * BV;                    // first state column of this workgroup
  const int64_t state_base = (n * a.h_v + hv) * D * D;

  // ---- direct copies into LDS: chunk xs's scan operands, chunk xp's Ut
  // operands; the window's jobs are dealt round-robin to the loader waves ----
  // (the gate-only variant reads no W, and the saving form for the backward
  // pass, which writes no outputs, no Q and P: their regions, copies and
  // warm-up lines have zero size)
  constexpr int B_KT = G::KT_FR * FB, B_W = ND ? 0 : G::W_FR * FB;
  constexpr int B_Q = SV ? 0 : G::Q_FR * FB, B_P = SV ? 0 : G::QK_FR * FB;
  constexpr int B_T = G::T_FR * FB, B_V = C * BV * ESZ, B_D = (2 * C + 4) * 4;
  constexpr int NREG = 7;
  constexpr int JOBS[NREG] = {(B_KT + 1023) / 1024, (B_W + 1023) / 1024, (B_Q + 1023) / 1024,
                              (B_P + 1023) / 1024,  (B_D + 1023) / 1024, (B_T + 1023) / 1024,
                              (B_V + 1023) / 1024};
  constexpr int CUM[NREG] = {0, JOBS[0], JOBS[0] + JOBS[1], JOBS[0] + JOBS[1] + JOBS[2],
                             JOBS[0] + JOBS[1] + JOBS[2] + JOBS[3],
                             JOBS[0] + JOBS[1] + JOBS[2] + JOBS[3] + JOBS[4],
                             JOBS[0] + JOBS[1] + JOBS[2] + JOBS[3] + JOBS[4] + JOBS[5]};
  // loader wave lw takes the jobs whose window-wide index is lw mod NLD; in
  // the causal regions (P, Tinv diag(b)) the jobs of fragments that the mask
  // makes zero copy nothing (the products never read them)
  auto copy_region = [&](int r, const char* src, char* dst, int bytes, bool causal) __attribute__((always_inline)) {
    for (int jj = ((lw - CUM[r]) % NLD + NLD) % NLD; jj < JOBS[r]; jj += NLD) {
      const int f = 1024 * jj / FB;
      if (causal && causal_zero(f / CKS, f % CKS)) continue;
      copy_1k(src + 1024 * jj, dst + 1024 * jj, bytes - 1024 * jj, lane);
    }
  };
  auto copy_window = [&](int xs, int xp) __attribute__((always_inline)) {
    if (xs < hi) {
      copy_region(0, static_cast<const char*>(a.key_t) + ((int64_t)xs * a.h_qk + hq) * B_KT,
                  reinterpret_cast<char*>(sm.kt[slot(xs)]), B_KT, false);
      copy_region(1, static_cast<const char*>(a.w) + ((int64_t)xs * a.h_v + hv) * B_W,
                  reinterpret_cast<char*>(sm.wf[slot(xs)]), B_W, false);
      copy_region(2, static_cast<const char*>(a.q_frag) + ((int64_t)xs * a.h_qk + hq) * B_Q,
                  reinterpret_cast<char*>(sm.qf[slot(xs)]), B_Q, false);
      copy_region(3, static_cast<const char*>(a.pmask) + ((int64_t)xs * a.h_v + hv) * B_P,
                  reinterpret_cast<char*>(sm.pf[slot(xs)]), B_P, true);
      copy_region(4, reinterpret_cast<const char*>(a.dtab + ((int64_t)xs * a.h_v + hv) * (2 * C + 4)),
                  reinterpret_cast<char*>(sm.dtab[slot(xs)]), B_D, false);
    }
    if (xp < hi) {
      copy_region(5, static_cast<const char*>(a.tinv) + ((int64_t)xp * a.h_v + hv) * B_T,
                  reinterpret_cast<char*>(sm.tf[slot(xp)]), B_T, true);
      // the V columns, row i of the chunk at byte 16 l of its job; rows
      // past the chunk end repeat its last row (Tinv diag(b) has zero
      // columns there)
      const int p_start = chunk_start(xp), p_last = chunk_len(xp) - 1;
      char* vdst = reinterpret_cast<char*>(sm.vr[slot(xp)]);
      for (int jj = ((lw - CUM[6]) % NLD + NLD) % NLD; jj < JOBS[6]; jj += NLD) {
        const int o = 1024 * jj + 16 * lane;
        const int i = min(o / (BV * ESZ), p_last);
        const char* vsrc = static_cast<const char*>(a.v) +
                           (((int64_t)(p_start + i) * a.h_v + hv) * D + col0) * ESZ + o % (BV * ESZ);
        if (o < B_V) __builtin_amdgcn_global_load_lds(vsrc, (lds_ptr_t)(vdst + 1024 * jj), 16, 0, 0);
      }
    }
  };

  // L2 warm-up, issued by the Ut waves after their chunk's work (they load
  // nothing into registers, so nothing ever waits on these) three chunks
  // ahead: one 4-byte load per 128-byte line of the chunk's streamed
  // operands, each line touched by one of the workgroups that read it (per V
  // head: W, P, the row-factor table and Tinv diag(b), shared by the NCB
  // column blocks; per QK head: K^T and Q, shared by the group's V heads
  // too), plus this workgroup's own V rows. The loaded words land in a
  // scratch LDS slot.
  constexpr int LV = (B_W + B_P + B_T + B_D + 127) / 128;        // lines per (chunk, V head)
  constexpr int LQ = (B_KT + B_Q + 127) / 128;                   // lines per (chunk, QK head)
  const int gi = hv % a.group;
  const int nv = (LV - cb + NCB - 1) / NCB;
  const int qs = gi * NCB + cb, qstride = a.group * NCB;
  const int nq = qs < LQ ? (LQ - qs + qstride - 1) / qstride : 0;
  auto line_addr = [&](int x, int t) -> const char* {
    if (t < nv) {
      const int o = 128 * (cb + NCB * t);
      // lines of the P and Tinv diag(b) fragments that the causal mask makes
      // zero are not copied; the forward pass does not touch them either
      // (the saving form measured faster touching its Tinv lines all)
      const int fp = (o - B_W) / FB, ft = (o - B_W - B_P) / FB;
      if (o >= B_W && o < B_W + B_P && causal_zero(fp / CKS, fp % CKS)) return nullptr;
      if (!SV && o >= B_W + B_P && o < B_W + B_P + B_T && causal_zero(ft / CKS, ft % CKS)) return nullptr;
      return o < B_W ? static_cast<const char*>(a.w) + ((int64_t)x * a.h_v + hv) * B_W + o
           : o < B_W + B_P ? static_cast<const char*>(a.pmask) + ((int64_t)x * a.h_v + hv) * B_P + (o - B_W)
           : o < B_W + B_P + B_T ? static_cast<const char*>(a.tinv) + ((int64_t)x * a.h_v + hv) * B_T + (o - B_W - B_P)
           : reinterpret_cast<const char*>(a.dtab + ((int64_t)x * a.h_v + hv) * (2 * C + 4)) +
                 min(o - B_W - B_P - B_T, B_D - 4);
    }
    t -= nv;
    if (t < nq) {
      const int o = 128 * (qs + qstride * t);
      return o < B_KT ? static_cast<const char*>(a.key_t) + ((int64_t)x * a.h_qk + hq) * B_KT + o
           : static_cast<const char*>(a.q_frag) + ((int64_t)x * a.h_qk + hq) * B_Q + min(o - B_KT, B_Q - 4);
    }
    t -= nq;
    const int i = min(t, chunk_len(x) - 1);
    return static_cast<const char*>(a.v) + (((int64_t)(chunk_start(x) + i) * a.h_v + hv) * D + col0) * ESZ;
  };
  auto warm = [&](int x) __attribute__((always_inline)) {
    if (x >= hi) return;
    const int total = nv + nq + C;
    for (int t = 64 * uw + lane; t < total; t += 64 * NS) {
      const char* p = line_addr(x, t);
      if (p) __builtin_amdgcn_global_load_lds(p, (lds_ptr_t)sm.touch[wave], 4, 0, 0);
    }
  };

  // the saving form stages its row-major stores in the Q and P fragment
  // buffers, which it does not use
  static_assert(!SV || NS * stage_elems<E>() * (int)sizeof(E) <=
                           (int)(sizeof(sm.qf) + sizeof(sm.pf)), "staging fits the unused buffers");
  auto sv_area = [&](int par, int sl) { return reinterpret_cast<E*>(sm.qf) + (par * NS + sl) * SV_AREA; };
  // scan waves: the slice's D x 16 state columns in accumulator tiles
  f32x4 S[DT];

  auto scan_chunk = [&](int c) __attribute__((always_inline)) {
    const int start = chunk_start(c), len = chunk_len(c), par = slot(c), upar = c & 1;
    if constexpr (SV && !SV_STAGE) {
      // (the same, stored row-major through the unused Q fragment buffers)
      store_tiles_rows<E, DT>(S, reinterpret_cast<E*>(sm.qf) + slice * stage_elems<E>(),
                              static_cast<E*>(a.sc) + ((int64_t)c * a.h_v + hv) * D * D + col0 + 16 * slice, D, lane);
    }
    Frag<E> Sf[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) Sf[ks] = acc_to_frag<E>(S[2 * ks], (2 * ks + 1 < DT) ? S[2 * ks + 1] : zero4());
    // Only W S -> U -> K^T U lies on the recurrence's path from one chunk's
    // state to the next: W S goes first, Q S (inter-chunk output) runs while
    // its results land, and P U (intra-chunk output) after the state update.
    //   WS[r][col]  = sum_d W[r][d] S[d][col]
    f32x4 WS[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) WS[t] = zero4();
    if constexpr (!ND) {
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
        Frag<E> wa[CT];
#pragma unroll
        for (int t = 0; t < CT; ++t) wa[t] = sm.wf[par][(t * DKS + ks) * 64 + lane];
#pragma unroll
        for (int t = 0; t < CT; ++t) WS[t] = mma(wa[t], Sf[ks], WS[t]);
      }
    }
    //   O^T[col][r] = sum_d S[d][col] q_r[d]
    f32x4 O[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) O[t] = zero4();
    if constexpr (!SV) {
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
        Frag<E> qa[CT];
#pragma unroll
        for (int t = 0; t < CT; ++t) qa[t] = sm.qf[par][(t * DKS + ks) * 64 + lane];
#pragma unroll
        for (int t = 0; t < CT; ++t) O[t] = mma(Sf[ks], qa[t], O[t]);
      }
    }
    // U = Ut - W S; the row factors come from the chunk's table (zero past
    // the chunk end)
    const float* ea = sm.dtab[par];
    const float* ed = sm.dtab[par] + C;
    f32x4 U[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t)
      U[t] = ND ? sm.uf[upar][(slice * CT + t) * 64 + lane] : sm.uf[upar][(slice * CT + t) * 64 + lane] - WS[t];
    Frag<E> Uk[CKS];
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) Uk[ks] = acc_to_frag<E>(U[2 * ks], (2 * ks + 1 < CT) ? U[2 * ks + 1] : zero4());
    if constexpr (SV_STAGE) {
      // backward pass: the chunk's U rows, rounded as the products use them
      stage_tiles_rows<E, CT>(U, sv_area(upar, slice) + D * SLD, lane);
    } else if constexpr (SV) {
      store_tiles_rows<E, CT>(U, reinterpret_cast<E*>(sm.qf) + slice * stage_elems<E>(),
                              static_cast<E*>(a.ub) + ((int64_t)c * a.h_v + hv) * C * D + col0 + 16 * slice, D, lane);
    }
    // decayed rows exp(g_L - g_r) U_r
#pragma unroll
    for (int t = 0; t < CT; ++t) U[t] *= *reinterpret_cast<const f32x4*>(&ed[16 * t + 4 * quad]);
    Frag<E> Ud[CKS];
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) Ud[ks] = acc_to_frag<E>(U[2 * ks], (2 * ks + 1 < CT) ? U[2 * ks + 1] : zero4());
    // S <- exp(g_L) S + K^T Ud (DT independent accumulators per step)
    const float gam = sm.dtab[par][2 * C];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S[dt] *= gam;
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) {
      Frag<E> ka[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ka[dt] = sm.kt[par][(dt * CKS + ks) * 64 + lane];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) S[dt] = mma(ka[dt], Ud[ks], S[dt]);
    }
    if constexpr (SV_STAGE) {
      // backward pass: the state at the chunk's start, rounded as the
      // products above used it (the elements of Sf), staged for the slice's
      // Ut wave; written after the step's operand reads have been issued,
      // since one wave's LDS operations complete in order
      __builtin_amdgcn_sched_barrier(0);
      E* ar = sv_area(upar, slice);
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (2 * ks + (e >> 2) < DT) ar[frag_k(ks, quad, e) * SLD + l16] = Sf[ks][e];   // (rows < D only)
      }
    }
    // the inter-chunk output takes exp(g_r); then O^T += U^T P^T,
    // P = (Q K^T * Dincl), while the state update's results land
    if constexpr (!SV) {
#pragma unroll
      for (int t = 0; t < CT; ++t) O[t] *= ea[16 * t + l16];
#pragma unroll
      for (int ks = 0; ks < CKS; ++ks) {
        Frag<E> pa[CT];
#pragma unroll
        for (int nt = 0; nt < CT; ++nt)
          if (!causal_zero(nt, ks)) pa[nt] = sm.pf[par][(nt * CKS + ks) * 64 + lane];
#pragma unroll
        for (int nt = 0; nt < CT; ++nt)
          if (!causal_zero(nt, ks)) O[nt] = mma(Uk[ks], pa[nt], O[nt]);
      }
    }
    if constexpr (!SV && STAGE_O) {
      // bf16 outputs: row-major (16 columns, 32 bytes a row) into this
      // slice's Ut slot, whose tiles this wave has read above; the slice's
      // Ut wave stores them in the next iteration, before it forms new
      // tiles there
      E* ost = reinterpret_cast<E*>(&sm.uf[upar][slice * CT * 64]);
#pragma unroll
      for (int nt = 0; nt < CT; ++nt) {
        Half<E> h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = to_e<E>(O[nt][i]);
        *reinterpret_cast<Half<E>*>(ost + (16 * nt + l16) * 16 + 4 * quad) = h;
      }
    } else if constexpr (!SV) {
      E* og = static_cast<E*>(a.o);
#pragma unroll
      for (int nt = 0; nt < CT; ++nt) {
        const int r = 16 * nt + l16;
        if (r < len) {
          Half<E> h;
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = to_e<E>(O[nt][i]);
          *reinterpret_cast<Half<E>*>(og + ((int64_t)(start + r) * a.h_v + hv) * D + col0 + 16 * slice + 4 * quad) = h;
        }
      }
    }
  };

  // Ut wave uw: chunk x's outputs for slice uw, staged by that slice's scan
  // wave in its Ut slot of parity x (only this wave writes that slot next).
  // They are read out before the slot takes new tiles and stored after
  // those are formed, so the stores do not queue behind the loaders' copies
  // ahead of the tiles: 16 bytes a lane, 32 rows of 16 columns per
  // instruction.
  constexpr int OJ = (C + 31) / 32;
  auto read_outputs = [&](int x, u32x4 (&val)[OJ]) __attribute__((always_inline)) {
    const E* st = reinterpret_cast<const E*>(&sm.uf[x & 1][uw * CT * 64]);
#pragma unroll
    for (int j = 0; j < OJ; ++j) {
      const int r = min(32 * j + lane / 2, C - 1);
      val[j] = *reinterpret_cast<const u32x4*>(st + r * 16 + 8 * (lane & 1));
    }
  };
  auto store_outputs = [&](int x, const u32x4 (&val)[OJ]) __attribute__((always_inline)) {
    const int start = chunk_start(x), len = chunk_len(x);
#pragma unroll
    for (int j = 0; j < OJ; ++j) {
      const int r = 32 * j + lane / 2;
      if (r < C && r < len)
        *reinterpret_cast<u32x4*>(static_cast<E*>(a.o) + ((int64_t)(start + r) * a.h_v + hv) * D + col0 + 16 * uw +
                                  8 * (lane & 1)) = val[j];
    }
  };

  // Ut wave uw, saving form: chunk x's staged S rows (D) and U rows (C) of
  // slice uw, read out in one iteration and stored after the Ut tiles
  using SR = StagedRows<E>;
  constexpr int NSV = (D + C) / SR::RPI;
  auto read_saved = [&](int x, u32x4 (&val)[NSV]) __attribute__((always_inline)) {
    const E* ar = sv_area(x & 1, uw);
#pragma unroll
    for (int j = 0; j < NSV; ++j)
      val[j] = *reinterpret_cast<const u32x4*>(&ar[(j * SR::RPI + lane / SR::LPR) * SLD + (lane % SR::LPR) * SR::VE]);
  };
  auto store_saved = [&](int x, const u32x4 (&val)[NSV]) __attribute__((always_inline)) {
    const int cix = col0 + 16 * uw + (lane % SR::LPR) * SR::VE;
    E* gs = static_cast<E*>(a.sc) + ((int64_t)x * a.h_v + hv) * D * D + cix;
    E* gu = static_cast<E*>(a.ub) + ((int64_t)x * a.h_v + hv) * C * D + cix;
#pragma unroll
    for (int j = 0; j < NSV; ++j) {
      const int row = j * SR::RPI + lane / SR::LPR;
      if (j * SR::RPI < D) *reinterpret_cast<u32x4*>(gs + (int64_t)row * D) = val[j];
      else *reinterpret_cast<u32x4*>(gu + (int64_t)(row - D) * D) = val[j];
    }
  };

  // Ut wave uw: chunk p's Ut tiles Tinv diag(b) V of slice uw; V's
  // fragments (col = state column, k = token) are gathered from the
  // row-major V columns
  auto produce_chunk = [&](int p) __attribute__((always_inline)) {
    const int par = slot(p), upar = p & 1;
    const E* vr = sm.vr[par];
    Frag<E> vf[CKS];
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = frag_k(s, quad, e);
        vf[s][e] = (i < C) ? vr[i * BV + 16 * uw + l16] : to_e<E>(0.f);
      }
    }
    f32x4 acc[CT];
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) acc[rt] = zero4();
#pragma unroll
    for (int s = 0; s < CKS; ++s) {
      Frag<E> tb[CT];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt)
        if (!causal_zero(rt, s)) tb[rt] = sm.tf[par][(rt * CKS + s) * 64 + lane];
#pragma unroll
      for (int rt = 0; rt < CT; ++rt)
        if (!causal_zero(rt, s)) acc[rt] = mma(tb[rt], vf[s], acc[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < CT; ++rt) sm.uf[upar][(uw * CT + rt) * 64 + lane] = acc[rt];
  };

  // The three roles run separate loops with the same barrier sequence (one
  // after the prologue, one per iteration), so each keeps only its own
  // registers live. Iteration c: the scan waves process chunk c; the
  // loaders copy chunk c+1's scan operands and chunk c+2's Ut operands into
  // LDS and wait for them; the Ut waves form chunk c+1's Ut tiles, then
  // warm L2 for chunk c+3.
  if (hi > lo) {
    if (is_scan) {
      const float* s_in = carried_in ? a.final_state : a.init_state;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[dt][i] = s_in ? s_in[state_base + (int64_t)(16 * dt + 4 * quad + i) * D + col0 + 16 * slice + l16] : 0.f;
      }
      __syncthreads();
      for (int c = lo - 1; c < hi; ++c) {
        if (c >= lo) scan_chunk(c);
        if (NB == 1) lds_barrier();    // compute phase ends: the loaders may refill
        lds_barrier();
      }
      if (a.final_state) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a.final_state[state_base + (int64_t)(16 * dt + 4 * quad + i) * D + col0 + 16 * slice + l16] = S[dt][i];
        }
      }
    } else if (is_loader) {
      // prologue: chunk lo's Ut operands (the scan-operand jobs are switched
      // off by passing a chunk past the end)
      copy_window(hi, lo);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      for (int c = lo - 1; c < hi; ++c) {
        if (NB == 1) __syncthreads();  // one slot per region: wait for the compute phase
        copy_window(c + 1, c + 2);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    } else {
      warm(lo + 1);
      warm(lo + 2);
      __syncthreads();
      u32x4 ov[OJ], sv[NSV];
      for (int c = lo - 1; c < hi; ++c) {
        // chunk c - 1's outputs leave the Ut slot that chunk c + 1's tiles
        // take next (saving form: its S and U rows, whose staging area the
        // scan waves write again in the next iteration)
        const bool st = !SV && STAGE_O && c > lo, ss = SV_STAGE && c > lo;
        if (st) read_outputs(c - 1, ov);
        if (ss) read_saved(c - 1, sv);
        if (c + 1 < hi) produce_chunk(c + 1);
        if (st) store_outputs(c - 1, ov);
        if (ss) store_saved(c - 1, sv);
        warm(c + 3);
        if (NB == 1) lds_barrier();
        lds_barrier();
      }
      if (!SV && STAGE_O) {
        read_outputs(hi - 1, ov);
        store_outputs(hi - 1, ov);
      }
      if (SV_STAGE) {
        read_saved(hi - 1, sv);
        store_saved(hi - 1, sv);
      }
    }
  } else if (is_scan && a.final_state && c1 <= c0 && a.win_lo == 0) {
    // empty sequence (written by the first window): the final state is the
    // initial state
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t idx = state_base + (int64_t)(16 * dt + 4 * quad + i) * D + col0 + 16 * slice + l16;
        a.final_state[idx] = a.init_state ? a.init_state[idx] : 0.f;
      }
    }
  }
}

template <typename E, int D, int C, bool WIN>
hipError_t launch_k2_fwd(PrefillArgs a, int64_t lo, int64_t hi, hipStream_t s) {
  if (hi <= lo) return hipSuccess;
  a.win_lo = lo;
  a.win_hi = hi;
  const dim3 g((unsigned)((hi - lo) * a.h_qk)), b(kBlock);
  if (a.prep) {
    if (a.no_delta) gdn_k2_inverse_w<E, D, C, true, true, false, WIN><<<g, b, 0, s>>>(a);
    else gdn_k2_inverse_w<E, D, C, true, false, false, WIN><<<g, b, 0, s>>>(a);
  } else {
    if (a.no_delta) gdn_k2_inverse_w<E, D, C, false, true, false, WIN><<<g, b, 0, s>>>(a);
    else gdn_k2_inverse_w<E, D, C, false, false, false, WIN><<<g, b, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <typename E, int D, int C, bool WIN>
hipError_t launch_scan_fwd(PrefillArgs a, int64_t lo, int64_t hi, hipStream_t s) {
  a.win_lo = lo;
  a.win_hi = hi;
  const dim3 g((unsigned)(a.num_seqs * a.h_v * ScanCfg<E, D, C>::NCB)), b(kScanBlock);
  if (a.no_delta) gdn_k3_scan<E, D, C, true, false, WIN><<<g, b, 0, s>>>(a);
  else gdn_k3_scan<E, D, C, false, false, WIN><<<g, b, 0, s>>>(a);
  return hipGetLastError();
}

// Kernel 2 beside the scan. The scan holds one CU per workgroup (its LDS),
// one workgroup per (sequence, V head, column block); a long sequence with
// few heads leaves CUs idle for its whole length. Then the chunk slots are
// cut in two windows: kernel 2 forms the first on the whole chip; while the
// scan runs it, kernel 2 forms the second on a second stream, on the CUs the
// scan leaves free; a second scan launch waits for it and enters with the
// state the first left in final_state (fp32, so the results are bitwise
// those of one launch). Neither stream's launches read what the other's
// concurrent ones write: kernel 2 writes only its window's slots, and the
// scan copies and prefetches only its own.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t first = nullptr;    // kernel 2's first window formed (caller's stream)
  hipEvent_t rest = nullptr;     // kernel 2's second window formed (side stream)
  int cus = 0;
  int state = 0;                 // 0 not set up, 1 ready, -1 unavailable
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// The side stream, its events and the CU count of the current device, set
// up on first use (default priority, non-blocking); null if unavailable, or
// if `s` belongs to another device (the side stream's launches would then
// run on the wrong GPU; the caller then runs the stages in order on `s`).
// Called with g_side_mu held.
SideStream* side_stream(hipStream_t s) {
  int dev = 0;
  hipDevice_t sdev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (hipStreamGetDevice(s, &sdev) != hipSuccess || (int)sdev != dev) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.state == 0) {
    ss.state = -1;
    if (hipDeviceGetAttribute(&ss.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ss.cus > 0 &&
        hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) == hipSuccess &&
        hipEventCreateWithFlags(&ss.first, hipEventDisableTiming) == hipSuccess &&
        hipEventCreateWithFlags(&ss.rest, hipEventDisableTiming) == hipSuccess)
      ss.state = 1;
  }
  return ss.state == 1 ? &ss : nullptr;
}

// The first window's share x of the chunk slots. With a fraction phi of the
// CUs idle beside the scan, and kernel 2 on the whole chip taking r times
// the scan's time, the second window lands as the scan reaches it when
// (1 - x) r / phi = x, i.e. x = r / (r + phi). r is fitted to timings
// (d = 128, C = 64, bf16; 48 V heads, phi = 1/4: r from 0.20 to 0.34 timed,
// 0.26-0.28 best, x = 0.51-0.53); kernel 2's own ratio, ~0.38, overstates
// it. More than two windows measured slower: at each later boundary the
// next scan's workgroups, each needing an empty CU, wait behind kernel 2's.
constexpr double kK2OverScan = 0.28;
// fewer chunk slots than this, or fewer than a fifth of the CUs idle beside
// the scan: the two launches run one after the other
constexpr int64_t kOverlapMinChunks = 256;

template <typename E, int D, int C>
hipError_t launch_fwd_overlapped(const PrefillArgs& a, hipStream_t s, bool* done) {
  *done = false;
  const int64_t nc = a.max_chunks;
  const int64_t groups = a.num_seqs * a.h_v * ScanCfg<E, D, C>::NCB;
  if (!a.final_state || nc < kOverlapMinChunks) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* ss = side_stream(s);
  if (!ss || 5 * groups > 4 * (int64_t)ss->cus) return hipSuccess;
  const double phi = 1.0 - (double)groups / ss->cus;
  const int64_t x = std::min(nc - 1, std::max<int64_t>(1, (int64_t)(nc * kK2OverScan / (kK2OverScan + phi))));
  hipError_t e = launch_k2_fwd<E, D, C, true>(a, 0, x, s);
  if (e == hipSuccess) e = hipEventRecord(ss->first, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->first, 0);
  if (e == hipSuccess) e = launch_scan_fwd<E, D, C, true>(a, 0, x, s);
  if (e == hipSuccess) e = launch_k2_fwd<E, D, C, true>(a, x, nc, ss->stream);
  if (e == hipSuccess) e = hipEventRecord(ss->rest, ss->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(s, ss->rest, 0);
  if (e == hipSuccess) e = launch_scan_fwd<E, D, C, true>(a, x, nc, s);
  *done = true;
  return e;
}

template <typename E, int D, int C>
hipError_t launch_prefill_t(const PrefillArgs& args, hipStream_t s, int first, int last) {
  PrefillArgs a = args;
  a.win_lo = 0;
  a.win_hi = a.max_chunks;
  const unsigned nc = (unsigned)a.max_chunks;
  const unsigned scan_groups = (unsigned)(a.num_seqs * a.h_v * ScanCfg<E, D, C>::NCB);
  const dim3 g_qk(nc * (unsigned)a.h_qk), g_scan(scan_groups);
  if (!a.backward && first == 1 && last == 2) {
    bool done = false;
    const hipError_t e = launch_fwd_overlapped<E, D, C>(a, s, &done);
    if (done || e != hipSuccess) return e;
  }
  for (int stage = first; stage <= last; ++stage) {
    if (a.backward) {
      // the backward pass (which takes no flags): kernel 1 finds the chunks,
      // forms g and b and lays out the K, K^T, Q^T and q.k fragments;
      // kernel 2 adds its own, and the scan saves the chunk-start states
      // and U
      switch (stage) {
        case 1: gdn_k1_chunk_prep<E, D, C><<<g_qk, dim3(kBlock), 0, s>>>(a); break;
        case 2: gdn_k2_inverse_w<E, D, C, false, false, true><<<g_qk, dim3(kBlock), 0, s>>>(a); break;
        case 3: gdn_k3_scan<E, D, C, false, true><<<g_scan, dim3(kScanBlock), 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
      }
      continue;
    }
    // the forward pass: kernel 2 (per chunk and QK head, with kernel 1's
    // work), then the scan
    hipError_t e = hipSuccess;
    switch (stage) {
      case 1: e = launch_k2_fwd<E, D, C, false>(a, 0, a.max_chunks, s); break;
      case 2: e = launch_scan_fwd<E, D, C, false>(a, 0, a.max_chunks, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_prefill_e(const PrefillArgs& a, int d, int c, hipStream_t s, int first, int last) {
  if (d == 128 && c == 64) return launch_prefill_t<E, 128, 64>(a, s, first, last);
  if (d == 128 && c == 16) return launch_prefill_t<E, 128, 16>(a, s, first, last);
  if (d == 16 && c == 64) return launch_prefill_t<E, 16, 64>(a, s, first, last);
  if (d == 16 && c == 16) return launch_prefill_t<E, 16, 16>(a, s, first, last);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int chunk, hipStream_t s,
                          int first_stage, int last_stage) {
  if (dtype == 1) return launch_prefill_e<bf16_t>(a, head_dim, chunk, s, first_stage, last_stage);
  return launch_prefill_e<float>(a, head_dim, chunk, s, first_stage, last_stage);
}

}  // namespace gdn
