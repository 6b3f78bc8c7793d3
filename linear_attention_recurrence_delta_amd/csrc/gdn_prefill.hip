// Prefill (gdn_chunk_fwd): the chunkwise WY-representation evaluation of the
// gated delta rule, page "Qwen3.8-Flash-Next 技术总结", section 2.1 (Gated
// DeltaNet). That section prints the token-serial update and says that the
// GPU algorithm turns the product of Householder-type transitions into block
// matrix products over chunks; the block formulas used here are derived from
// the first form of its update equation. For one V head and a chunk of L <= C
// tokens entering with state S0 (r, i index tokens in the chunk):
//
//   g_r    = sum_{j<=r} log a_j                          kernel 1
//   A[r,i] = b_r (k_r . k_i) exp(g_r - g_i)  (i < r)     kernel 2
//   Tinv   = (I + A)^{-1}                                kernel 2
//   W      = Tinv diag(b exp(g)) K                       kernel 3 (producer waves)
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
// Kernel 3 fuses the W/Ut construction, the inter-chunk state scan and the
// output products: W, Ut, U and the per-chunk states never leave the chip.
//
// Fragment layouts (see gdn_device.h for the lane/element order): a
// "fragment" is 64 lanes x 8 elements; "frag (a, s)" of a matrix X means
// lane l holds row/col a*16 + l%16 and the 8 contraction indices of step s.
//   key_t [c][hq][D/16][C32] : frag (dt, s) of K^T   (row d,     k = token i)
//   tinv  [c][hv][C/16][C32] : frag (rt, s) of Tinv  (row r,     k = token i)
//   qk    [c][hq][C/16][C32] : frag (nt, s) of (q_r . k_j) (col r = query, k = key j)
// with C32 = ceil(C/32); entries past the chunk end are zero.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kBlock = 256;

template <typename E, int D, int C>
struct Cfg {
  static constexpr int DT = D / 16, CT = C / 16;
  static constexpr int DKS = (DT + 1) / 2, CKS = (CT + 1) / 2;
  static constexpr int NS = DT >= 2 ? 2 : 1;   // 16-column state slices per scan workgroup
  static constexpr int BV = 16 * NS;           // state columns per scan workgroup
  static constexpr int NCB = D / BV;           // scan workgroups per (sequence, V head)
  static constexpr int NW = 4;                 // waves per scan workgroup
  static constexpr int NPROD = NW - NS;        // producer waves
  static constexpr int KT_FR = DT * CKS;       // K^T fragments per chunk
  static constexpr int T_FR = CT * CKS;        // Tinv fragments per chunk
  static constexpr int QK_FR = CT * CKS;       // q.k fragments per chunk
  static constexpr int Q_FR = CT * DKS;        // Q fragments per chunk
  static constexpr int W_FR = CT * DKS;        // W fragments per chunk
  static constexpr int VLD = C + 8;            // row stride of the transposed V slice
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

// --------------------------------------------------------------------------
// Kernel 1: chunk table, in-chunk prefix sums of log a and per-chunk b.
// One workgroup per compact chunk slot c in [0, floor(T/C) + N). Each group
// scans the per-sequence chunk counts ceil(L_n / C) to find which sequence
// owns slot c (slots past the last chunk are marked seq = -1); group 0 also
// publishes the per-sequence first-chunk offsets. Then one thread per V head
// writes g[c][h][r] and b[c][h][r] for r < C; past a partial chunk's end g
// repeats the last valid prefix (log a taken as 0) and b is 0.
// --------------------------------------------------------------------------
template <int C>
__global__ __launch_bounds__(kBlock) void gdn_k1_gate_prefix(const PrefillArgs a) {
  __shared__ int s_scan[kBlock];
  __shared__ int s_hit[2];
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x;
  if (tid == 0) { s_hit[0] = -1; s_hit[1] = 0; }
  __syncthreads();
  int carry = 0;
  for (int64_t base = 0; base < a.num_seqs; base += kBlock) {
    const int64_t n = base + tid;
    int cnt = 0;
    if (n < a.num_seqs) {
      const int s0 = a.cu_seqlens ? a.cu_seqlens[n] : 0;
      const int s1 = a.cu_seqlens ? a.cu_seqlens[n + 1] : (int)a.total_tokens;
      cnt = (s1 - s0 + C - 1) / C;
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {
      const int x = (tid >= off) ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += x;
      __syncthreads();
    }
    const int incl = carry + s_scan[tid];
    const int excl = incl - cnt;
    if (n < a.num_seqs) {
      if (c >= excl && c < incl) { s_hit[0] = (int)n; s_hit[1] = (int)(c - excl); }
      if (c == 0) a.seq_chunk_offset[n] = excl;
    }
    carry += s_scan[kBlock - 1];
    __syncthreads();
  }
  if (c == 0 && tid == 0) a.seq_chunk_offset[a.num_seqs] = carry;
  const int n = s_hit[0];
  int4* table = reinterpret_cast<int4*>(a.chunk_table);
  if (n < 0) {
    if (tid == 0) table[c] = make_int4(-1, 0, 0, 0);
    return;
  }
  const int j = s_hit[1];
  const int s0 = a.cu_seqlens ? a.cu_seqlens[n] : 0;
  const int s1 = a.cu_seqlens ? a.cu_seqlens[n + 1] : (int)a.total_tokens;
  const int start = s0 + j * C;
  const int len = min(C, s1 - start);
  if (tid == 0) table[c] = make_int4(n, start, len, j);
  for (int h = tid; h < a.h_v; h += kBlock) {
    float acc = 0.f;
    float* gout = a.gate_prefix + (c * a.h_v + h) * C;
    float* bout = a.beta_chunk + (c * a.h_v + h) * C;
    for (int r = 0; r < C; ++r) {
      float b = 0.f;
      if (r < len) {
        acc += a.log_alpha[(int64_t)(start + r) * a.h_v + h];
        b = a.beta[(int64_t)(start + r) * a.h_v + h];
      }
      gout[r] = acc;
      bout[r] = b;
    }
  }
}

// --------------------------------------------------------------------------
// Kernel 2: per (chunk, V head): A = strict_lower(b_r (k_r . k_i)
// exp(g_r - g_i)), Tinv = (I + A)^{-1}, written as the fragments of
// Tinv diag(b) and Tinv diag(b exp(g)) (the right factors of Ut and W).
// The first V head of each QK group also writes the chunk's K^T and q.k
// fragments, which the QK group's V heads share.
// K K^T (and Q K^T) are formed with MFMA. Tinv is assembled blockwise in
// fp32 over the four waves: the 16 x 16 diagonal blocks by forward
// substitution (one lane per column), then the blocks below them in order
// of distance from the diagonal,
//   Tinv_ij = -Tinv_ii sum_{j<=m<i} A_im Tinv_mj,
// with fp32 16x16x4 MFMAs, one block per wave per distance.
// --------------------------------------------------------------------------

// acc += X Y for 16 x 16 fp32 tiles in LDS (row-major, leading dims lx, ly)
__device__ __forceinline__ f32x4 mma16_f32(const float* X, int lx, const float* Y, int ly, f32x4 acc,
                                           int lane) {
  const int m = lane & 15, k = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[m * lx + 4 * kk + k], Y[(4 * kk + k) * ly + m], acc, 0, 0, 0);
  return acc;
}

template <typename E, int D, int C>
struct InvSmem {
  static constexpr int KLD = D + 8;    // bf16/fp32 row stride of the staged keys and queries
  static constexpr int FLD = C + 4;    // fp32 row stride of C x C tiles (spreads rows over banks)
  static constexpr int XLD = 20;       // row stride of the 16 x 16 scratch tiles
  union {
    struct {
      E ks[C * KLD];                   // keys of the chunk, rows past its end zero
      E qs[C * KLD];                   // queries of the chunk
    } in;
    struct {
      float t[C * FLD];                // Tinv being assembled
      float x[4][16 * XLD];            // one 16 x 16 scratch tile per wave
    } out;
  } u;
  float kk[C * FLD];                   // K K^T (lower tiles), later q.k staging
  float a[C * FLD];                    // A (below the diagonal)
  float gb[2][C];                      // g and b of this V head
};

template <typename E, int D, int C>
__global__ __launch_bounds__(kBlock) void gdn_k2_akk_inverse(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  using SM = InvSmem<E, D, C>;
  constexpr int CT = G::CT, CKS = G::CKS, DKS = G::DKS, KLD = SM::KLD, FLD = SM::FLD, XLD = SM::XLD;
  constexpr int NW = kBlock / 64;
  constexpr int VE = 16 / (int)sizeof(E);                 // elements per 16-byte load
  typedef E VLoad __attribute__((ext_vector_type(VE)));
  __shared__ SM sm;
  // the V heads of one (chunk, QK head), which read the same keys, are
  // consecutive logical ids and so share an XCD
  const int64_t lid = xcd_local_id(blockIdx.x, gridDim.x);
  const int c = (int)(lid / a.h_v), hv = (int)(lid % a.h_v);
  const int4 tab = reinterpret_cast<const int4*>(a.chunk_table)[c];
  if (tab.x < 0) return;
  const int start = tab.y, len = tab.z;
  const int hq = hv / a.group;
  const bool lead = (hv % a.group) == 0;          // writes the QK head's shared fragments
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, l16 = lane & 15;
  const E* kg = static_cast<const E*>(a.k);
  const E* qg = static_cast<const E*>(a.q);

  for (int idx = tid; idx < C * D / VE; idx += kBlock) {
    const int r = idx / (D / VE), d = (idx % (D / VE)) * VE;
    VLoad kv, qv;
#pragma unroll
    for (int e = 0; e < VE; ++e) { kv[e] = to_e<E>(0.f); qv[e] = to_e<E>(0.f); }
    if (r < len) {
      const int64_t gi = ((int64_t)(start + r) * a.h_qk + hq) * D + d;
      kv = *reinterpret_cast<const VLoad*>(kg + gi);
      if (lead) qv = *reinterpret_cast<const VLoad*>(qg + gi);
    }
    *reinterpret_cast<VLoad*>(&sm.u.in.ks[r * KLD + d]) = kv;
    if (lead) *reinterpret_cast<VLoad*>(&sm.u.in.qs[r * KLD + d]) = qv;
  }
  if (tid < 2 * C) {
    const int64_t o = ((int64_t)c * a.h_v + hv) * C + (tid % C);
    sm.gb[tid / C][tid % C] = (tid < C) ? a.gate_prefix[o] : a.beta_chunk[o];
  }
  __syncthreads();

  if (lead) {
    // K^T fragments: frag (dt, s), lane row d, elements token i.
    Frag<E>* ktg = reinterpret_cast<Frag<E>*>(a.key_t) + ((int64_t)c * a.h_qk + hq) * G::KT_FR * 64;
    for (int it = tid; it < G::KT_FR * 64; it += kBlock) {
      const int f = it / 64, ln = it % 64, dt = f / CKS, s = f % CKS, q4 = ln >> 4;
      const int d = 16 * dt + (ln & 15);
      Frag<E> v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = frag_k(s, q4, e);
        v[e] = (i < C) ? sm.u.in.ks[i * KLD + d] : to_e<E>(0.f);
      }
      ktg[it] = v;
    }
  }

  // K K^T lower tiles: CT (CT + 1) / 2 tiles over the waves
  for (int t = wave; t < CT * CT; t += NW) {
    const int mi = t / CT, ni = t % CT;
    if (ni > mi) continue;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks)
      acc = mma(load_frag<E>(&sm.u.in.ks[(16 * mi + l16) * KLD + 32 * ks], quad, D - 32 * ks),
                load_frag<E>(&sm.u.in.ks[(16 * ni + l16) * KLD + 32 * ks], quad, D - 32 * ks), acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.kk[(16 * mi + 4 * quad + i) * FLD + 16 * ni + l16] = acc[i];
  }
  __syncthreads();
  // A below the diagonal (the inverse never reads the rest)
  for (int idx = tid; idx < C * C; idx += kBlock) {
    const int r = idx / C, i = idx % C;
    if (i < r)
      sm.a[r * FLD + i] = sm.gb[1][r] * sm.kk[r * FLD + i] * __expf(fminf(sm.gb[0][r] - sm.gb[0][i], 0.f));
  }
  if (lead) {
    // q.k tiles with key tile <= query tile, staged [query r][key j] in kk
    // (K K^T is consumed by now; a barrier separates the two)
  }
  __syncthreads();
  if (lead) {
    for (int t = wave; t < CT * CT; t += NW) {
      const int kt = t / CT, nt = t % CT;     // key tile, query tile
      if (kt > nt) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks)
        acc = mma(load_frag<E>(&sm.u.in.ks[(16 * kt + l16) * KLD + 32 * ks], quad, D - 32 * ks),
                  load_frag<E>(&sm.u.in.qs[(16 * nt + l16) * KLD + 32 * ks], quad, D - 32 * ks), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.kk[(16 * nt + l16) * FLD + 16 * kt + 4 * quad + i] = acc[i];
    }
  }
  __syncthreads();
  if (lead) {
    // q.k fragments: frag (nt, s), lane col = query r, elements key j.
    Frag<E>* qkg = reinterpret_cast<Frag<E>*>(a.qk) + ((int64_t)c * a.h_qk + hq) * G::QK_FR * 64;
    for (int it = tid; it < G::QK_FR * 64; it += kBlock) {
      const int f = it / 64, ln = it % 64, nt = f / CKS, s = f % CKS, q4 = ln >> 4;
      const int r = 16 * nt + (ln & 15);
      Frag<E> v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = frag_k(s, q4, e);
        v[e] = (j < C && (j >> 4) <= nt) ? to_e<E>(sm.kk[r * FLD + j]) : to_e<E>(0.f);
      }
      qkg[it] = v;
    }
  }
  __syncthreads();     // staged keys and queries are dead from here on; out.t reuses them

  float* Tm = sm.u.out.t;
  // blocks above the diagonal are zero
  for (int idx = tid; idx < C * C; idx += kBlock) {
    const int r = idx / C, i = idx % C;
    if ((i >> 4) > (r >> 4)) Tm[r * FLD + i] = 0.f;
  }
  // diagonal blocks: wave b solves block b, lane j its column j
  for (int b = wave; b < CT; b += NW) {
    if (lane < 16) {
      const int j = lane, o = 16 * b;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) {
          if (i & 1) s1 -= sm.a[(o + r) * FLD + o + i] * x[i];
          else s0 -= sm.a[(o + r) * FLD + o + i] * x[i];
        }
        x[r] = s0 + s1;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tm[(o + r) * FLD + o + j] = x[r];
    }
  }
  __syncthreads();
  // blocks below the diagonal, by distance; one block per wave per distance
#pragma unroll
  for (int dist = 1; dist < CT; ++dist) {
    for (int bi = dist + wave; bi < CT; bi += NW) {
      const int bj = bi - dist;
      float* X = sm.u.out.x[wave];
      f32x4 acc = zero4();
      for (int bm = bj; bm < bi; ++bm)
        acc = mma16_f32(&sm.a[(16 * bi) * FLD + 16 * bm], FLD, &Tm[(16 * bm) * FLD + 16 * bj], FLD, acc, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) X[(4 * quad + i) * XLD + l16] = acc[i];
      acc = mma16_f32(&Tm[(16 * bi) * FLD + 16 * bi], FLD, X, XLD, zero4(), lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) Tm[(16 * bi + 4 * quad + i) * FLD + 16 * bj + l16] = -acc[i];
    }
    __syncthreads();
  }
  // Tinv diag(b) and Tinv diag(b exp(g)) fragments, written one after the other
  Frag<E>* tg = reinterpret_cast<Frag<E>*>(a.tinv) + ((int64_t)c * a.h_v + hv) * 2 * G::T_FR * 64;
  for (int it = tid; it < G::T_FR * 64; it += kBlock) {
    const int f = it / 64, ln = it % 64, rt = f / CKS, s = f % CKS, q4 = ln >> 4;
    const int r = 16 * rt + (ln & 15);
    Frag<E> vb, vg;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = frag_k(s, q4, e);
      const float t = (i < C) ? Tm[r * FLD + i] * sm.gb[1][i] : 0.f;
      vb[e] = to_e<E>(t);
      vg[e] = to_e<E>((i < C) ? t * __expf(sm.gb[0][i]) : 0.f);
    }
    tg[it] = vb;
    tg[G::T_FR * 64 + it] = vg;
  }
}

// --------------------------------------------------------------------------
// Kernel 3: fused W/Ut construction, inter-chunk state scan and outputs.
// One workgroup per (sequence, V head, block of BV state columns), eight
// waves, looping over the sequence's chunks in order with a software
// pipeline:
//   scan waves (one per 16-column slice) process chunk c: with the slice of
//     the state S (D x 16 fp32) held in MFMA accumulators for the whole
//     sequence,
//       O^T  = diag(exp(g)) applied to S^T Q^T      (inter-chunk output)
//       U    = Ut - W S                            (S's accumulator tiles are
//                                                   the B fragments here)
//       O^T += U^T (Q K^T * Dincl)^T                (U's tiles are the A fragments)
//       S    = exp(g_L) S + K^T (exp(g_L - g) * U)
//     and store the chunk's outputs for their columns;
//   producer waves build chunk c+1's W and Ut fragments and the masked,
//     decayed (q.k) fragments in LDS, and double as loaders: they fetch
//     chunk c+3's K^T, Tinv, q.k, g, b and V slice (and chunk c+2's Q) into
//     one of two register sets while the other set, fetched one iteration
//     earlier, is written into LDS for chunk c+2 between the barriers.
// Every LDS region is either double-buffered by chunk parity or written only
// between the two barriers of an iteration after its last reader is done.
// --------------------------------------------------------------------------
constexpr int kScanBlock = 512;

template <typename E, int D, int C>
struct ScanSmem {
  using G = Cfg<E, D, C>;
  Frag<E> kt[2][G::KT_FR * 64];        // K^T fragments, by chunk parity
  Frag<E> qf[G::Q_FR * 64];            // Q fragments of the chunk being scanned
  Frag<E> tf[2][G::T_FR * 64];         // Tinv diag(b), Tinv diag(b exp(g)) of the chunk being produced
  Frag<E> qk[G::QK_FR * 64];           // q.k fragments of the chunk being produced
  Frag<E> wf[2][G::W_FR * 64];         // W fragments, by chunk parity
  Frag<E> pf[2][G::QK_FR * 64];        // masked, decayed q.k fragments, by parity
  f32x4 uf[2][G::NS * G::CT * 64];     // Ut accumulator tiles, by parity
  E vt[G::BV * G::VLD];                // V slice of the chunk being produced, transposed
  float gb[2][2][C];                   // g and b, by chunk parity
};

// One register set of loader data: a chunk's operands plus the next chunk's Q.
template <typename E, int D, int C>
struct ScanFetch {
  using G = Cfg<E, D, C>;
  static constexpr int NL = kScanBlock - 64 * G::NS;                 // loader threads
  static constexpr int FR16 = (int)sizeof(Frag<E>) / 16;             // 16-byte units per lane-fragment
  static constexpr int N_KT = G::KT_FR * 64 * FR16, N_T = 2 * G::T_FR * 64 * FR16, N_QK = G::QK_FR * 64 * FR16;
  static constexpr int N_GB = 2 * C * 4 / 16;
  static constexpr int VU = 16 / (int)sizeof(E);                     // V elements per 16-byte unit
  static constexpr int N_V = C * G::BV / VU;
  static constexpr int N_Q = G::Q_FR * 64;                           // lane-fragments of Q
  static constexpr int P_KT = (N_KT + NL - 1) / NL, P_T = (N_T + NL - 1) / NL;
  static constexpr int P_QK = (N_QK + NL - 1) / NL, P_V = (N_V + NL - 1) / NL;
  static constexpr int P_Q = (N_Q + NL - 1) / NL, P_GB = (N_GB + NL - 1) / NL;
  typedef E VUnit __attribute__((ext_vector_type(VU)));             // one 16-byte unit of V
  u32x4 kt[P_KT], t[P_T], qk[P_QK], gb[P_GB];
  VUnit v[P_V];
  Frag<E> q[P_Q];
};

template <typename E, int D, int C>
__global__ __launch_bounds__(kScanBlock) void gdn_k3_scan(const PrefillArgs a) {
  using G = Cfg<E, D, C>;
  using F = ScanFetch<E, D, C>;
  constexpr int DT = G::DT, CT = G::CT, DKS = G::DKS, CKS = G::CKS, NS = G::NS, BV = G::BV;
  constexpr int NPROD = kScanBlock / 64 - NS;
  __shared__ ScanSmem<E, D, C> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, l16 = lane & 15;
  // the column blocks and V heads of one QK head, which read the same K^T,
  // q.k and Q fragments, are consecutive logical ids and so share an XCD
  const int64_t bid = xcd_local_id(blockIdx.x, gridDim.x);
  const int cb = (int)(bid % G::NCB);
  const int hv = (int)((bid / G::NCB) % a.h_v);
  const int64_t n = bid / ((int64_t)G::NCB * a.h_v);
  const int hq = hv / a.group;
  const int c0 = a.seq_chunk_offset[n], c1 = a.seq_chunk_offset[n + 1];
  // chunk x of this sequence starts at seq_start + (x - c0) * C; computing
  // start and length here keeps table reads off the per-chunk critical path
  const int seq_start = a.cu_seqlens ? a.cu_seqlens[n] : 0;
  const int seq_end = a.cu_seqlens ? a.cu_seqlens[n + 1] : (int)a.total_tokens;
  auto chunk_start = [&](int x) { return seq_start + (x - c0) * C; };
  auto chunk_len = [&](int x) { return min(C, seq_end - chunk_start(x)); };
  const bool is_scan = wave < NS;
  const int slice = wave;                      // scan waves: slice index
  const int pw = wave - NS;                    // producer waves: index
  const int lt = tid - 64 * NS;                // loader thread index (producers only)
  const int col0 = cb * BV;                    // first state column of this workgroup
  const int64_t state_base = (n * a.h_v + hv) * D * D;

  // ---- loaders: global -> registers (chunk x's operands, chunk xq's Q) ----
  // Branch-free: every loader issues the same loads, with indices clamped
  // into range (the last valid unit, row or chunk); what lies outside is
  // masked when the registers are stored. Keeping the loads unconditional
  // lets them stay in flight across the pipeline's barriers.
  auto fetch = [&](F& fr, int x, int xq) __attribute__((always_inline)) {
    const int xc = min(x, c1 - 1);
    const u32x4* ktg = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const Frag<E>*>(a.key_t) + ((int64_t)xc * a.h_qk + hq) * G::KT_FR * 64);
    // both scaled Tinv fragment sets of chunk x are contiguous
    const u32x4* tg = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const Frag<E>*>(a.tinv) + ((int64_t)xc * a.h_v + hv) * 2 * G::T_FR * 64);
    const u32x4* qkg = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const Frag<E>*>(a.qk) + ((int64_t)xc * a.h_qk + hq) * G::QK_FR * 64);
#pragma unroll
    for (int p = 0; p < F::P_KT; ++p) fr.kt[p] = ktg[min(lt + p * F::NL, F::N_KT - 1)];
#pragma unroll
    for (int p = 0; p < F::P_T; ++p) fr.t[p] = tg[min(lt + p * F::NL, F::N_T - 1)];
#pragma unroll
    for (int p = 0; p < F::P_QK; ++p) fr.qk[p] = qkg[min(lt + p * F::NL, F::N_QK - 1)];
#pragma unroll
    for (int p = 0; p < F::P_GB; ++p) {
      const int u = min(lt + p * F::NL, F::N_GB - 1), half = F::N_GB / 2;
      const float* src = (u < half ? a.gate_prefix : a.beta_chunk) + ((int64_t)xc * a.h_v + hv) * C;
      fr.gb[p] = reinterpret_cast<const u32x4*>(src)[u % half];
    }
    const int x_start = chunk_start(xc), x_last = chunk_len(xc) - 1;
    const E* vg = static_cast<const E*>(a.v);
#pragma unroll
    for (int p = 0; p < F::P_V; ++p) {
      const int u = min(lt + p * F::NL, F::N_V - 1);
      const int i = min(u / (BV / F::VU), x_last), part = u % (BV / F::VU);
      fr.v[p] = *reinterpret_cast<const typename F::VUnit*>(
          vg + ((int64_t)(x_start + i) * a.h_v + hv) * D + col0 + part * F::VU);
    }
    const int xqc = min(max(xq, c0), c1 - 1);
    const int q_start = chunk_start(xqc), q_last = chunk_len(xqc) - 1;
    const E* qg = static_cast<const E*>(a.q);
#pragma unroll
    for (int p = 0; p < F::P_Q; ++p) {
      const int u = min(lt + p * F::NL, F::N_Q - 1);
      const int f = u / 64, ln = u % 64, nt = f / DKS, s = f % DKS;
      const int r = min(16 * nt + (ln & 15), q_last);
      fr.q[p] = load_frag<E>(qg + ((int64_t)(q_start + r) * a.h_qk + hq) * D + 32 * s, ln >> 4, D - 32 * s);
    }
  };
  // ---- loaders: registers -> LDS, masking what the fetch clamped ----
  auto store = [&](const F& fr, int x, int xq) __attribute__((always_inline)) {
    if (x < c1) {
      u32x4* kt = reinterpret_cast<u32x4*>(sm.kt[x & 1]);
      u32x4* tf = reinterpret_cast<u32x4*>(sm.tf[0]);
      u32x4* qk = reinterpret_cast<u32x4*>(sm.qk);
#pragma unroll
      for (int p = 0; p < F::P_KT; ++p) { const int u = lt + p * F::NL; if (u < F::N_KT) kt[u] = fr.kt[p]; }
#pragma unroll
      for (int p = 0; p < F::P_T; ++p) { const int u = lt + p * F::NL; if (u < F::N_T) tf[u] = fr.t[p]; }
#pragma unroll
      for (int p = 0; p < F::P_QK; ++p) { const int u = lt + p * F::NL; if (u < F::N_QK) qk[u] = fr.qk[p]; }
#pragma unroll
      for (int p = 0; p < F::P_GB; ++p) {
        const int u = lt + p * F::NL;
        if (u < F::N_GB) reinterpret_cast<u32x4*>(&sm.gb[x & 1][0][0])[u] = fr.gb[p];
      }
      const int x_len = chunk_len(x);
#pragma unroll
      for (int p = 0; p < F::P_V; ++p) {
        const int u = lt + p * F::NL;
        if (u < F::N_V) {
          const int i = u / (BV / F::VU), part = u % (BV / F::VU);
#pragma unroll
          for (int e = 0; e < F::VU; ++e)
            sm.vt[(part * F::VU + e) * G::VLD + i] = (i < x_len) ? fr.v[p][e] : to_e<E>(0.f);
        }
      }
    }
    if (xq >= c0 && xq < c1) {
      const int q_len = chunk_len(xq);
#pragma unroll
      for (int p = 0; p < F::P_Q; ++p) {
        const int u = lt + p * F::NL;
        if (u < F::N_Q) {
          const int nt = (u / 64) / DKS, r = 16 * nt + (u % 64 & 15);
          Frag<E> v = fr.q[p];
          if (r >= q_len) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = to_e<E>(0.f);
          }
          sm.qf[u] = v;
        }
      }
    }
  };

  // scan waves: the slice's D x 16 state columns in accumulator tiles
  f32x4 S[DT];

  auto scan_chunk = [&](int c) __attribute__((always_inline)) {
    const int start = chunk_start(c), len = chunk_len(c), par = c & 1;
    const float* gs = sm.gb[par][0];
    Frag<E> Sf[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) Sf[ks] = acc_to_frag<E>(S[2 * ks], (2 * ks + 1 < DT) ? S[2 * ks + 1] : zero4());
    // Both products that read the state run together, contraction step
    // outermost so that 2 CT independent accumulators interleave, with the
    // next step's LDS fragments loaded before this step's MFMAs:
    //   O^T[col][r] = sum_d S[d][col] q_r[d]   (inter-chunk output)
    //   WS[r][col]  = sum_d W[r][d] S[d][col]
    f32x4 O[CT], WS[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) { O[t] = zero4(); WS[t] = zero4(); }
    Frag<E> qa[CT], wa[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      qa[t] = sm.qf[(t * DKS) * 64 + lane];
      wa[t] = sm.wf[par][(t * DKS) * 64 + lane];
    }
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) {
      Frag<E> qn[CT], wn[CT];
      if (ks + 1 < DKS) {
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          qn[t] = sm.qf[(t * DKS + ks + 1) * 64 + lane];
          wn[t] = sm.wf[par][(t * DKS + ks + 1) * 64 + lane];
        }
      }
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        O[t] = mma(Sf[ks], qa[t], O[t]);
        WS[t] = mma(wa[t], Sf[ks], WS[t]);
      }
      if (ks + 1 < DKS) {
#pragma unroll
        for (int t = 0; t < CT; ++t) { qa[t] = qn[t]; wa[t] = wn[t]; }
      }
    }
    // U = Ut - W S; the inter-chunk output takes exp(g_r) (rows past the
    // chunk end are zeroed by multiplying, not branching)
    f32x4 U[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      U[t] = sm.uf[par][(slice * CT + t) * 64 + lane] - WS[t];
      const int r = 16 * t + l16;
      O[t] *= __expf(gs[r]) * (float)(r < len);
    }
    Frag<E> Uk[CKS];
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) Uk[ks] = acc_to_frag<E>(U[2 * ks], (2 * ks + 1 < CT) ? U[2 * ks + 1] : zero4());
    // decayed rows exp(g_L - g_r) U_r
    const float g_last = gs[len - 1];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * quad + i;
        U[t][i] *= __expf(fminf(g_last - gs[r], 0.f)) * (float)(r < len);
      }
    }
    Frag<E> Ud[CKS];
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) Ud[ks] = acc_to_frag<E>(U[2 * ks], (2 * ks + 1 < CT) ? U[2 * ks + 1] : zero4());
    // S <- exp(g_L) S + K^T Ud (DT independent accumulators per step), and
    // the intra-chunk output O^T += U^T P^T
    const float gam = __expf(g_last);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S[dt] *= gam;
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) {
      Frag<E> ka[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ka[dt] = sm.kt[par][(dt * CKS + ks) * 64 + lane];
      Frag<E> pa[CT];
#pragma unroll
      for (int nt = 0; nt < CT; ++nt)
        if (!causal_zero(nt, ks)) pa[nt] = sm.pf[par][(nt * CKS + ks) * 64 + lane];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) S[dt] = mma(ka[dt], Ud[ks], S[dt]);
#pragma unroll
      for (int nt = 0; nt < CT; ++nt)
        if (!causal_zero(nt, ks)) O[nt] = mma(Uk[ks], pa[nt], O[nt]);
    }
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
  };

  auto produce_chunk = [&](int p) __attribute__((always_inline)) {
    const int par = p & 1;
    const int len = chunk_len(p);
    const float* gp = sm.gb[par][0];
    constexpr int NITEM = DKS + NS + CT;
    for (int item = pw; item < NITEM; item += NPROD) {
      if (item < DKS) {
        // W fragments (rt, ks_d) for every rt: the W^T tiles of d-tiles
        // 2 ks_d and 2 ks_d + 1, from Tinv diag(b exp(g)) and K^T
        const int ksd = item;
        Frag<E> ka[CKS], kb[CKS];
#pragma unroll
        for (int s = 0; s < CKS; ++s) {
          ka[s] = sm.kt[par][((2 * ksd) * CKS + s) * 64 + lane];
          if (2 * ksd + 1 < DT) kb[s] = sm.kt[par][((2 * ksd + 1) * CKS + s) * 64 + lane];
        }
        f32x4 acc0[CT], acc1[CT];
#pragma unroll
        for (int rt = 0; rt < CT; ++rt) { acc0[rt] = zero4(); acc1[rt] = zero4(); }
#pragma unroll
        for (int s = 0; s < CKS; ++s) {
          Frag<E> tb[CT];
#pragma unroll
          for (int rt = 0; rt < CT; ++rt)
            if (!causal_zero(rt, s)) tb[rt] = sm.tf[1][(rt * CKS + s) * 64 + lane];
#pragma unroll
          for (int rt = 0; rt < CT; ++rt) {
            if (causal_zero(rt, s)) continue;            // Tinv is lower triangular
            acc0[rt] = mma(ka[s], tb[rt], acc0[rt]);
            if (2 * ksd + 1 < DT) acc1[rt] = mma(kb[s], tb[rt], acc1[rt]);
          }
        }
#pragma unroll
        for (int rt = 0; rt < CT; ++rt) sm.wf[par][(rt * DKS + ksd) * 64 + lane] = acc_to_frag<E>(acc0[rt], acc1[rt]);
      } else if (item < DKS + NS) {
        // Ut accumulator tiles of slice sl: Tinv diag(b) V
        const int sl = item - DKS;
        const E* vrow = &sm.vt[(16 * sl + l16) * G::VLD];
        Frag<E> vf[CKS];
#pragma unroll
        for (int s = 0; s < CKS; ++s) vf[s] = load_frag<E>(vrow + 32 * s, quad, C - 32 * s);
        f32x4 acc[CT];
#pragma unroll
        for (int rt = 0; rt < CT; ++rt) acc[rt] = zero4();
#pragma unroll
        for (int s = 0; s < CKS; ++s) {
          Frag<E> tb[CT];
#pragma unroll
          for (int rt = 0; rt < CT; ++rt)
            if (!causal_zero(rt, s)) tb[rt] = sm.tf[0][(rt * CKS + s) * 64 + lane];
#pragma unroll
          for (int rt = 0; rt < CT; ++rt)
            if (!causal_zero(rt, s)) acc[rt] = mma(tb[rt], vf[s], acc[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < CT; ++rt) sm.uf[par][(sl * CT + rt) * 64 + lane] = acc[rt];
      } else {
        // masked, decayed q.k fragments of query tile nt
        const int nt = item - DKS - NS;
        const int r = 16 * nt + l16;
        const float gr = gp[r];
#pragma unroll
        for (int s = 0; s < CKS; ++s) {
          if (causal_zero(nt, s)) continue;
          const Frag<E> raw = sm.qk[(nt * CKS + s) * 64 + lane];
          Frag<E> v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = frag_k(s, quad, e);
            // the exponent is clamped at 0 so that masked entries (j > r,
            // where g_r - g_j >= 0) cannot overflow before being zeroed
            const float m = (float)(j <= r && r < len);
            v[e] = to_e<E>(to_f(raw[e]) * (__expf(fminf(gr - gp[j], 0.f)) * m));
          }
          sm.pf[par][(nt * CKS + s) * 64 + lane] = v;
        }
      }
    }
  };

  // The two roles run separate loops with the same barrier sequence (one
  // after the prologue, two per iteration), so each loop keeps only its own
  // registers live: the scan waves the state, the producers the two loader
  // register sets. Iteration c: scan chunk c; produce chunk c + 1; fetch
  // chunk c + 3 (and Q of chunk c + 2) into one set; between the barriers
  // stage the other set (chunk c + 2 and Q of chunk c + 1, fetched one
  // iteration earlier) into LDS.
  if (c1 > c0) {
    if (is_scan) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[dt][i] = a.init_state
                         ? a.init_state[state_base + (int64_t)(16 * dt + 4 * quad + i) * D + col0 + 16 * slice + l16]
                         : 0.f;
      }
      __syncthreads();
      for (int c = c0 - 1; c < c1; ++c) {
        if (c >= c0) scan_chunk(c);
        __syncthreads();
        __syncthreads();
      }
      if (a.final_state) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a.final_state[state_base + (int64_t)(16 * dt + 4 * quad + i) * D + col0 + 16 * slice + l16] = S[dt][i];
        }
      }
    } else {
      F fa, fb;
      fetch(fa, c0, -1);
      store(fa, c0, -1);
      __syncthreads();
      fetch(fa, c0 + 1, c0);
      for (int c = c0 - 1; c < c1; c += 2) {
        fetch(fb, c + 3, c + 2);
        if (c + 1 < c1) produce_chunk(c + 1);
        __syncthreads();
        store(fa, c + 2, c + 1);
        __syncthreads();
        if (c + 1 < c1) {
          fetch(fa, c + 4, c + 3);
          if (c + 2 < c1) produce_chunk(c + 2);
          __syncthreads();
          store(fb, c + 3, c + 2);
          __syncthreads();
        }
      }
    }
  } else if (is_scan && a.final_state) {
    // empty sequence: the final state is the initial state
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

template <typename E, int D, int C>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s, int first, int last) {
  using G = Cfg<E, D, C>;
  const unsigned nc = (unsigned)a.max_chunks;
  const unsigned scan_groups = (unsigned)(a.num_seqs * a.h_v * G::NCB);
  for (int stage = first; stage <= last; ++stage) {
    switch (stage) {
      case 1: gdn_k1_gate_prefix<C><<<dim3(nc), dim3(kBlock), 0, s>>>(a); break;
      case 2: gdn_k2_akk_inverse<E, D, C><<<dim3(nc * (unsigned)a.h_v), dim3(kBlock), 0, s>>>(a); break;
      case 3: gdn_k3_scan<E, D, C><<<dim3(scan_groups), dim3(kScanBlock), 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_prefill_e(const PrefillArgs& a, int d, int c, hipStream_t s, int first, int last) {
  if (d == 128 && c == 64) {
    // fp32 at head dim 128 with 64-token chunks would need ~250 KB of LDS
    // for the fused scan's double-buffered fragments; it is not built.
    if constexpr (std::is_same<E, float>::value) return hipErrorInvalidValue;
    else return launch_prefill_t<E, 128, 64>(a, s, first, last);
  }
  if (d == 128 && c == 16) return launch_prefill_t<E, 128, 16>(a, s, first, last);
  if (d == 16 && c == 64) return launch_prefill_t<E, 16, 64>(a, s, first, last);
  if (d == 16 && c == 16) return launch_prefill_t<E, 16, 16>(a, s, first, last);
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int chunk) {
  if (head_dim != 16 && head_dim != 128) return false;
  if (chunk != 16 && chunk != 64) return false;
  if (dtype == 0 && head_dim == 128 && chunk == 64) return false;
  return dtype == 0 || dtype == 1;
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int chunk, hipStream_t s,
                          int first_stage, int last_stage) {
  if (dtype == 1) return launch_prefill_e<bf16_t>(a, head_dim, chunk, s, first_stage, last_stage);
  return launch_prefill_e<float>(a, head_dim, chunk, s, first_stage, last_stage);
}

}  // namespace gdn
