// Prefill (gdn_chunk_fwd): the chunkwise WY-representation evaluation of the
// gated delta rule, page "Qwen3.8-Flash-Next 技术总结", section 2.1 (Gated
// DeltaNet). That section prints the token-serial update and says that the
// GPU algorithm turns the product of Householder-type transitions into block
// matrix products over chunks; the block formulas used here are derived from
// the first form of its update equation. For one V head and a chunk of L <= C
// tokens entering with state S0 (r, i index tokens in the chunk):
//
//   g_r    = sum_{j<=r} log a_j                               kernel 1
//   A[r,i] = b_r (k_r . k_i) exp(g_r - g_i)  (i < r)          kernel 2
//   Tinv   = (I + A)^{-1}                                     kernel 2
//   W      = Tinv diag(b exp(g)) K,  Ut = Tinv diag(b) V      kernel 3
//   U      = Ut - W S0                                        kernel 4
//   S_end  = exp(g_L) S0 + (exp(g_L - g) * K)^T U             kernel 4
//   O      = diag(exp(g)) Q S0 + (Q K^T * Dincl) U            kernel 5
//            Dincl[r,i] = exp(g_r - g_i) for i <= r, else 0
//
// The rows of U are the delta vectors u_r = b_r (v_r - a_r S_{r-1}^T k_r)
// of the token-serial form, and O is o_r = S_r^T q_r with the post-update
// state. Every column of the state (a dv index) evolves independently, which
// is what lets kernel 4 give each wave a 16-column slice of one head's state.
// exp() is only ever taken of g_r - g_i with i <= r (a non-positive number).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kBlock = 256;

// --------------------------------------------------------------------------
// Kernel 1: chunk table and in-chunk prefix sums of log a.
// One workgroup per compact chunk slot c in [0, floor(T/C) + N). Each group
// scans the per-sequence chunk counts ceil(L_n / C) to find which sequence
// owns slot c (slots past the last chunk are marked seq = -1); group 0 also
// publishes the per-sequence first-chunk offsets. Then one thread per V head
// writes g[c][h][r] for r < C; rows past a partial chunk's end repeat the
// last valid prefix (their log a is taken as 0).
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
    for (int r = 0; r < C; ++r) {
      if (r < len) acc += a.log_alpha[(int64_t)(start + r) * a.h_v + h];
      gout[r] = acc;
    }
  }
}

// --------------------------------------------------------------------------
// Kernel 2: A = strict_lower(b_r (k_r . k_i) exp(g_r - g_i)) and
// Tinv = (I + A)^{-1}. One workgroup per (chunk, QK head): K K^T is formed
// once with MFMA and shared by the QK head's V heads; each wave then inverts
// one V head's unit lower-triangular I + A by forward substitution with one
// lane per column j (x_r = delta_rj - sum_{i<r} A[r,i] x_i, fp32 in
// registers, A read from LDS as a broadcast). Also writes the chunk's keys
// transposed ([d][r], zero past the chunk end) for kernels 3 and 4.
// --------------------------------------------------------------------------
template <typename E, int D, int C>
__global__ __launch_bounds__(kBlock) void gdn_k2_akk_inverse(const PrefillArgs a) {
  constexpr int CT = C / 16, DKS = (D / 16 + 1) / 2, KLD = D + 8, NW = kBlock / 64;
  __shared__ __attribute__((aligned(16))) E Ks[C * KLD];
  __shared__ __attribute__((aligned(16))) float KK[C * C];
  __shared__ __attribute__((aligned(16))) float Ab[NW][C * C];
  __shared__ float sb[NW][C];
  const int c = blockIdx.x, hq = blockIdx.y;
  const int4 tab = reinterpret_cast<const int4*>(a.chunk_table)[c];
  if (tab.x < 0) return;
  const int start = tab.y, len = tab.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, l16 = lane & 15;
  const E* kg = static_cast<const E*>(a.k);

  for (int idx = tid; idx < C * D; idx += kBlock) {
    const int r = idx / D, d = idx % D;
    Ks[r * KLD + d] = (r < len) ? kg[((int64_t)(start + r) * a.h_qk + hq) * D + d] : to_e<E>(0.f);
  }
  __syncthreads();
  E* ktg = static_cast<E*>(a.key_t) + ((int64_t)c * a.h_qk + hq) * D * C;
  for (int idx = tid; idx < C * D; idx += kBlock) {
    const int d = idx / C, r = idx % C;
    ktg[idx] = Ks[r * KLD + d];
  }
  for (int t = wave; t < CT * CT; t += NW) {
    const int mi = t / CT, ni = t % CT;
    if (ni > mi) continue;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) {
      const Frag<E> fa = load_frag<E>(&Ks[(16 * mi + l16) * KLD + 32 * ks], quad, D - 32 * ks);
      const Frag<E> fb = load_frag<E>(&Ks[(16 * ni + l16) * KLD + 32 * ks], quad, D - 32 * ks);
      acc = mma(fa, fb, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) KK[(16 * mi + 4 * quad + i) * C + 16 * ni + l16] = acc[i];
  }
  __syncthreads();

  const float* gch = a.gate_prefix + (int64_t)c * a.h_v * C;
  for (int h0 = 0; h0 < a.group; h0 += NW) {
    const int nh = min(NW, a.group - h0);
    for (int w = 0; w < nh; ++w) {
      const int hv = hq * a.group + h0 + w;
      if (tid < C) sb[w][tid] = (tid < len) ? a.beta[(int64_t)(start + tid) * a.h_v + hv] : 0.f;
    }
    __syncthreads();
    for (int w = 0; w < nh; ++w) {
      const float* gh = gch + (int64_t)(hq * a.group + h0 + w) * C;
      for (int idx = tid; idx < C * C; idx += kBlock) {
        const int r = idx / C, i = idx % C;
        float val = 0.f;
        if (i < r && r < len) val = sb[w][r] * KK[idx] * expf(gh[r] - gh[i]);
        Ab[w][idx] = val;
      }
    }
    __syncthreads();
    if (wave < nh) {
      const int hv = hq * a.group + h0 + wave;
      const float* Aw = Ab[wave];
      float x[C];
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float s = (r == lane) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= Aw[r * C + i] * x[i];
        x[r] = s;
      }
      if (lane < C) {
        E* tg = static_cast<E*>(a.tinv) + ((int64_t)c * a.h_v + hv) * C * C;
#pragma unroll
        for (int r = 0; r < C; ++r) tg[r * C + lane] = to_e<E>(x[r]);
      }
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// Kernel 3: W = Tinv diag(b exp(g)) K and Ut = Tinv diag(b) V. One
// workgroup per (chunk, V head); Tinv and the two right operands (stored
// transposed, contraction index contiguous) are staged in LDS, and the
// 2 x (C/16) x (D/16) output tiles are spread over the four waves. W is
// written row-major; Ut is written in accumulator order
// ([D/16 col tile][C/16 row tile][lane][4]) so kernel 4 reads it back in the
// register layout it needs with one vector load per tile.
// --------------------------------------------------------------------------
template <typename E, int D, int C>
__global__ __launch_bounds__(kBlock) void gdn_k3_wu(const PrefillArgs a) {
  constexpr int CT = C / 16, DT = D / 16, CKS = (CT + 1) / 2, LD = C + 8, NW = kBlock / 64;
  __shared__ __attribute__((aligned(16))) E Ts[C * LD];
  __shared__ __attribute__((aligned(16))) E Kb[D * LD];
  __shared__ __attribute__((aligned(16))) E Vb[D * LD];
  __shared__ float sb[C], sbg[C];
  const int c = blockIdx.x, hv = blockIdx.y;
  const int4 tab = reinterpret_cast<const int4*>(a.chunk_table)[c];
  if (tab.x < 0) return;
  const int start = tab.y, len = tab.z;
  const int hq = hv / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, l16 = lane & 15;
  const int64_t chv = (int64_t)c * a.h_v + hv;

  if (tid < C) {
    const float b = (tid < len) ? a.beta[(int64_t)(start + tid) * a.h_v + hv] : 0.f;
    sb[tid] = b;
    sbg[tid] = b * expf(a.gate_prefix[chv * C + tid]);
  }
  const E* tg = static_cast<const E*>(a.tinv) + chv * C * C;
  for (int idx = tid; idx < C * C; idx += kBlock) Ts[(idx / C) * LD + idx % C] = tg[idx];
  __syncthreads();
  const E* ktg = static_cast<const E*>(a.key_t) + ((int64_t)c * a.h_qk + hq) * D * C;
  for (int idx = tid; idx < C * D; idx += kBlock) {
    const int d = idx / C, i = idx % C;
    Kb[d * LD + i] = to_e<E>(to_f(ktg[idx]) * sbg[i]);
  }
  const E* vg = static_cast<const E*>(a.v);
  for (int idx = tid; idx < C * D; idx += kBlock) {
    const int i = idx / D, d = idx % D;
    Vb[d * LD + i] = (i < len) ? to_e<E>(to_f(vg[((int64_t)(start + i) * a.h_v + hv) * D + d]) * sb[i])
                               : to_e<E>(0.f);
  }
  __syncthreads();

  E* wg = static_cast<E*>(a.w) + chv * C * D;
  E* utg = static_cast<E*>(a.u_tilde) + chv * C * D;
  for (int t = wave; t < 2 * CT * DT; t += NW) {
    const bool is_u = t >= CT * DT;
    const int tt = is_u ? t - CT * DT : t;
    const int mt = tt / DT, nt = tt % DT;
    const E* B = is_u ? Vb : Kb;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) {
      const Frag<E> fa = load_frag<E>(&Ts[(16 * mt + l16) * LD + 32 * ks], quad, C - 32 * ks);
      const Frag<E> fb = load_frag<E>(&B[(16 * nt + l16) * LD + 32 * ks], quad, C - 32 * ks);
      acc = mma(fa, fb, acc);
    }
    if (!is_u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wg[(16 * mt + 4 * quad + i) * D + 16 * nt + l16] = to_e<E>(acc[i]);
    } else {
      Half<E> h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = to_e<E>(acc[i]);
      *reinterpret_cast<Half<E>*>(utg + ((nt * CT + mt) * 64 + lane) * 4) = h;
    }
  }
}

// --------------------------------------------------------------------------
// Kernel 4: inter-chunk state scan. One wave per (sequence, V head, 16-column
// slice of the state); the slice (D x 16 fp32) lives in MFMA accumulators for
// the whole sequence. Per chunk, in order:
//   Sc = S (stored as operand fragments for kernel 5)
//   U  = Ut - W Sc                     (the state's accumulator tiles are
//                                       already the B fragments of this product)
//   S  = exp(g_L) Sc + K^T (exp(g_L - g) * U)
//                                      (U's accumulator tiles are the B fragments)
// U is stored (undecayed) as operand fragments for kernel 5. Loads of W, Ut
// and K^T do not depend on S and are issued ahead by the compiler.
// --------------------------------------------------------------------------
template <typename E, int D, int C>
__global__ __launch_bounds__(64) void gdn_k4_state_scan(const PrefillArgs a) {
  constexpr int CT = C / 16, DT = D / 16, CKS = (CT + 1) / 2, DKS = (DT + 1) / 2;
  const int lane = threadIdx.x, quad = lane >> 4, l16 = lane & 15;
  const int64_t bid = blockIdx.x;
  const int nb = (int)(bid % DT);
  const int hv = (int)((bid / DT) % a.h_v);
  const int64_t n = bid / ((int64_t)DT * a.h_v);
  const int hq = hv / a.group;
  const int col = 16 * nb + l16;
  const int64_t state_base = (n * a.h_v + hv) * D * D;

  f32x4 S[DT];
#pragma unroll
  for (int mt = 0; mt < DT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[mt][i] = a.init_state ? a.init_state[state_base + (int64_t)(16 * mt + 4 * quad + i) * D + col] : 0.f;
  }
  const int4* table = reinterpret_cast<const int4*>(a.chunk_table);
  const int c0 = a.seq_chunk_offset[n], c1 = a.seq_chunk_offset[n + 1];
  for (int c = c0; c < c1; ++c) {
    const int len = table[c].z;
    const int64_t chv = (int64_t)c * a.h_v + hv;
    Frag<E> Sf[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) Sf[ks] = acc_to_frag<E>(S[2 * ks], (2 * ks + 1 < DT) ? S[2 * ks + 1] : zero4());
    Frag<E>* scg = reinterpret_cast<Frag<E>*>(static_cast<E*>(a.s_chunk)) + (chv * DT + nb) * DKS * 64;
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) scg[ks * 64 + lane] = Sf[ks];

    const E* wg = static_cast<const E*>(a.w) + chv * C * D;
    const Half<E>* utg = reinterpret_cast<const Half<E>*>(static_cast<const E*>(a.u_tilde) + chv * C * D) + nb * CT * 64;
    f32x4 U[CT];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks)
        acc = mma(load_frag<E>(wg + (16 * mt + l16) * D + 32 * ks, quad, D - 32 * ks), Sf[ks], acc);
      const Half<E> ut = utg[mt * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) U[mt][i] = to_f(ut[i]) - acc[i];
    }
    Frag<E>* ug = reinterpret_cast<Frag<E>*>(static_cast<E*>(a.u)) + (chv * DT + nb) * CKS * 64;
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks)
      ug[ks * 64 + lane] = acc_to_frag<E>(U[2 * ks], (2 * ks + 1 < CT) ? U[2 * ks + 1] : zero4());

    const float* gch = a.gate_prefix + chv * C;
    const float g_last = gch[len - 1];
#pragma unroll
    for (int mt = 0; mt < CT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * quad + i;
        U[mt][i] *= (r < len) ? expf(g_last - gch[r]) : 0.f;
      }
    }
    Frag<E> Ud[CKS];
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) Ud[ks] = acc_to_frag<E>(U[2 * ks], (2 * ks + 1 < CT) ? U[2 * ks + 1] : zero4());
    const float gam = expf(g_last);
    const E* ktg = static_cast<const E*>(a.key_t) + ((int64_t)c * a.h_qk + hq) * D * C;
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      f32x4 acc = S[mt] * gam;
#pragma unroll
      for (int ks = 0; ks < CKS; ++ks)
        acc = mma(load_frag<E>(ktg + (16 * mt + l16) * C + 32 * ks, quad, C - 32 * ks), Ud[ks], acc);
      S[mt] = acc;
    }
  }
  if (a.final_state) {
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.final_state[state_base + (int64_t)(16 * mt + 4 * quad + i) * D + col] = S[mt][i];
    }
  }
}

// --------------------------------------------------------------------------
// Kernel 5: outputs, computed transposed so that every operand is either a
// plain row-major load or a fragment written by kernel 4:
//   O^T = U^T (K Q^T * Dincl^T) + Sc^T (diag(exp(g)) Q)^T.
// One workgroup per (chunk, V head); wave w handles query tiles w, w+4, ...
// The K Q^T tile is formed in accumulators, masked/decayed in place, and
// used directly as the B fragment of the U^T product.
// --------------------------------------------------------------------------
template <typename E, int D, int C>
__global__ __launch_bounds__(kBlock) void gdn_k5_output(const PrefillArgs a) {
  constexpr int CT = C / 16, DT = D / 16, CKS = (CT + 1) / 2, DKS = (DT + 1) / 2, NW = kBlock / 64;
  __shared__ float gs[C];
  const int c = blockIdx.x, hv = blockIdx.y;
  const int4 tab = reinterpret_cast<const int4*>(a.chunk_table)[c];
  if (tab.x < 0) return;
  const int start = tab.y, len = tab.z;
  const int hq = hv / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, l16 = lane & 15;
  const int64_t chv = (int64_t)c * a.h_v + hv;
  if (tid < C) gs[tid] = a.gate_prefix[chv * C + tid];
  __syncthreads();
  const E* qg = static_cast<const E*>(a.q);
  const E* kg = static_cast<const E*>(a.k);
  const Frag<E>* ufr = reinterpret_cast<const Frag<E>*>(static_cast<const E*>(a.u)) + chv * DT * CKS * 64;
  const Frag<E>* sfr = reinterpret_cast<const Frag<E>*>(static_cast<const E*>(a.s_chunk)) + chv * DT * DKS * 64;
  E* og = static_cast<E*>(a.o);

  for (int nt = wave; nt < CT; nt += NW) {
    const int r = 16 * nt + l16;
    const bool r_ok = r < len;
    const E* qrow = qg + ((int64_t)(start + r) * a.h_qk + hq) * D;
    f32x4 P[CT];
#pragma unroll
    for (int kt = 0; kt < CT; ++kt) {
      const int jrow = 16 * kt + l16;
      const E* krow = kg + ((int64_t)(start + jrow) * a.h_qk + hq) * D;
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks)
        acc = mma(load_frag_masked<E>(krow + 32 * ks, quad, D - 32 * ks, jrow < len),
                  load_frag_masked<E>(qrow + 32 * ks, quad, D - 32 * ks, r_ok), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * kt + 4 * quad + i;
        acc[i] = (j <= r && r_ok) ? acc[i] * expf(gs[r] - gs[j]) : 0.f;
      }
      P[kt] = acc;
    }
    Frag<E> Pf[CKS];
#pragma unroll
    for (int ks = 0; ks < CKS; ++ks) Pf[ks] = acc_to_frag<E>(P[2 * ks], (2 * ks + 1 < CT) ? P[2 * ks + 1] : zero4());
    const float gr = r_ok ? expf(gs[r]) : 0.f;
    Frag<E> Qf[DKS];
#pragma unroll
    for (int ks = 0; ks < DKS; ++ks) {
      const Frag<E> raw = load_frag_masked<E>(qrow + 32 * ks, quad, D - 32 * ks, r_ok);
#pragma unroll
      for (int e = 0; e < 8; ++e) Qf[ks][e] = to_e<E>(to_f(raw[e]) * gr);
    }
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < CKS; ++ks) acc = mma(ufr[(mt * CKS + ks) * 64 + lane], Pf[ks], acc);
#pragma unroll
      for (int ks = 0; ks < DKS; ++ks) acc = mma(sfr[(mt * DKS + ks) * 64 + lane], Qf[ks], acc);
      if (r_ok) {
        Half<E> h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = to_e<E>(acc[i]);
        *reinterpret_cast<Half<E>*>(og + ((int64_t)(start + r) * a.h_v + hv) * D + 16 * mt + 4 * quad) = h;
      }
    }
  }
}

template <typename E, int D, int C>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s, int first, int last) {
  const unsigned nc = (unsigned)a.max_chunks;
  const unsigned scan_waves = (unsigned)(a.num_seqs * a.h_v * (D / 16));
  for (int stage = first; stage <= last; ++stage) {
    switch (stage) {
      case 1: gdn_k1_gate_prefix<C><<<dim3(nc), dim3(kBlock), 0, s>>>(a); break;
      case 2: gdn_k2_akk_inverse<E, D, C><<<dim3(nc, a.h_qk), dim3(kBlock), 0, s>>>(a); break;
      case 3: gdn_k3_wu<E, D, C><<<dim3(nc, a.h_v), dim3(kBlock), 0, s>>>(a); break;
      case 4: gdn_k4_state_scan<E, D, C><<<dim3(scan_waves), dim3(64), 0, s>>>(a); break;
      case 5: gdn_k5_output<E, D, C><<<dim3(nc, a.h_v), dim3(kBlock), 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
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
