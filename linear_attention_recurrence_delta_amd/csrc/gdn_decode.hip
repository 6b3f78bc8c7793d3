// Decode (gdn_decode_step): one token per sequence, the single-token update
// of page "Qwen3.8-Flash-Next 技术总结", section 2.1 (Gated DeltaNet), first
// form of its update equation, applied to the state in place:
//   p = S^T k,  u = b (v - a p),  S <- a S + k u^T,
// with the output o = S_new^T q evaluated in the same pass through the
// identity S_new^T q = a (S^T q) + u (k . q), so the state is read once and
// written once.
//
// The step is a streaming read-modify-write of the fp32 state (64 KiB per
// (sequence, V head) at head dim 128), so it is bound by HBM bandwidth. One
// workgroup owns one (sequence, V head) state: thread (rg, cg) holds rows
// [rg*RPT, rg*RPT+RPT) of columns [4cg, 4cg+4) in registers as 16-byte
// vectors (each wave-wide load covers two full 512-byte rows). The column
// sums S^T k and S^T q are reduced across the row groups through LDS, then
// the update is applied from registers and stored. Loads and stores are
// non-temporal: the state is touched once per step and is larger than the
// last-level cache.
//
// The gate-only variant (S <- a S + b k v^T, the same readout) is the same
// pass with u = b v: S^T k is then not formed.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

template <int D> struct DecodeShape;
template <> struct DecodeShape<128> { static constexpr int RG = 8; };
template <> struct DecodeShape<16> { static constexpr int RG = 4; };

template <typename E, int D, bool P, bool ND>
__global__ __launch_bounds__((D / 4) * DecodeShape<D>::RG) void gdn_kd_decode_step(const DecodeArgs a) {
  constexpr int CG = D / 4, RG = DecodeShape<D>::RG, RPT = D / RG;
  __shared__ f32x4 red_p[RG][CG];
  __shared__ f32x4 red_r[RG][CG];
  __shared__ float red_kq[RG][4];                // k.q, then (raw inputs) |k|^2, |q|^2
  const int64_t nh = blockIdx.x;                 // sequence * h_v + V head
  const int64_t n = nh / a.h_v;
  const int hv = (int)(nh % a.h_v);
  const int hq = hv / a.group;
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;

  const E* kp = static_cast<const E*>(a.k) + (n * a.h_qk + hq) * D + rg * RPT;
  const E* qp = static_cast<const E*>(a.q) + (n * a.h_qk + hq) * D + rg * RPT;
  // k and q stay in the input dtype until used (fewer registers, so that
  // v can be requested with the state without lowering occupancy)
  E kk[RPT], qq[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) { kk[r] = kp[r]; qq[r] = qp[r]; }
  const Half<E> vh = *reinterpret_cast<const Half<E>*>(static_cast<const E*>(a.v) + nh * D + 4 * (tid % (D / 4)));

  f32x4* sp = reinterpret_cast<f32x4*>(a.state + nh * D * D) + (rg * RPT) * CG + cg;
  f32x4 s[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) s[r] = __builtin_nontemporal_load(sp + r * CG);

  f32x4 p = zero4(), rq = zero4();
  float kq = 0.f, k2 = 0.f, q2 = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float kr = to_f(kk[r]), qr = to_f(qq[r]);
    if constexpr (!ND) p += s[r] * kr;
    rq += s[r] * qr;
    kq += kr * qr;
  }
  if constexpr (P) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) { k2 += to_f(kk[r]) * to_f(kk[r]); q2 += to_f(qq[r]) * to_f(qq[r]); }
  }
  if constexpr (!ND) red_p[rg][cg] = p;
  red_r[rg][cg] = rq;
  if (cg == 0) {
    red_kq[rg][0] = kq;
    if constexpr (P) { red_kq[rg][1] = k2; red_kq[rg][2] = q2; }
  }
  __syncthreads();
  p = zero4();
  rq = zero4();
  kq = 0.f;
  k2 = 0.f;
  q2 = 0.f;
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    if constexpr (!ND) p += red_p[g][cg];
    rq += red_r[g][cg];
    kq += red_kq[g][0];
    if constexpr (P) { k2 += red_kq[g][1]; q2 += red_kq[g][2]; }
  }
  float alpha, beta, kscale = 1.f;
  if constexpr (P) {
    // raw inputs: S^T k, S^T q and k.q are linear in k and q, so the unit
    // vectors' values are the raw sums times the inverse norms
    const float ik = inv_norm(k2), iq = inv_norm(q2);
    p *= ik;
    rq *= iq;
    kq *= ik * iq;
    kscale = ik;
    alpha = expf(neg_softplus(a.log_alpha[nh]));
    beta = sigmoid_of(a.beta[nh]);
  } else {
    alpha = expf(a.log_alpha[nh]);
    beta = a.beta[nh];
  }
  f32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = ND ? beta * to_f(vh[e]) : beta * (to_f(vh[e]) - alpha * p[e]);

#pragma unroll
  for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(decay_rank1(s[r], alpha, u, to_f(kk[r]) * kscale), sp + r * CG);

  if (rg == 0) {
    Half<E> h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = to_e<E>(fmaf(alpha, rq[e], u[e] * kq));
    *reinterpret_cast<Half<E>*>(static_cast<E*>(a.o) + nh * D + 4 * cg) = h;
  }
}

// With fused input preparation, q and k arrive raw: their squared norms
// join the column-sum reduction, and the raw sums S^T k, S^T q, k.q are
// rescaled by the inverse norms (they are linear in k and q).
//
// Speculative multi-token verify: K drafted tokens per sequence applied in
// order, K successive steps of the update above in one pass over the state.
// The workgroup's state slice stays in registers across the K tokens; each
// token's column sums are reduced through LDS buffers alternating by token
// parity (one barrier per token). Token j's output is written as it is
// formed. With a snapshot buffer, the state after each token goes to
// snapshot j and `state` is only read (so a caller can keep any accepted
// prefix); without one, the final state replaces `state`. Each token's
// arithmetic is the single-step kernel's, term for term.
template <typename E, int D, bool P, bool ND>
__global__ __launch_bounds__((D / 4) * DecodeShape<D>::RG) void gdn_kd_decode_multi(const DecodeArgs a) {
  constexpr int CG = D / 4, RG = DecodeShape<D>::RG, RPT = D / RG;
  __shared__ f32x4 red_p[2][RG][CG];
  __shared__ f32x4 red_r[2][RG][CG];
  __shared__ float red_kq[2][RG][4];             // k.q, then (raw inputs) |k|^2, |q|^2
  const int64_t nh = blockIdx.x;                 // sequence * h_v + V head
  const int64_t n = nh / a.h_v;
  const int hv = (int)(nh % a.h_v);
  const int hq = hv / a.group;
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int64_t tok_v = a.num_seqs * a.h_v;      // [N, HV] entries per token
  const int64_t tok_q = a.num_seqs * a.h_qk;     // [N, HQ] entries per token

  f32x4* sp = reinterpret_cast<f32x4*>(a.state + nh * D * D) + (rg * RPT) * CG + cg;
  f32x4 s[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) s[r] = __builtin_nontemporal_load(sp + r * CG);

  for (int j = 0; j < a.num_tokens; ++j) {
    const int par = j & 1;
    const E* kp = static_cast<const E*>(a.k) + (j * tok_q + n * a.h_qk + hq) * D + rg * RPT;
    const E* qp = static_cast<const E*>(a.q) + (j * tok_q + n * a.h_qk + hq) * D + rg * RPT;
    float kk[RPT], qq[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) { kk[r] = to_f(kp[r]); qq[r] = to_f(qp[r]); }
    f32x4 p = zero4(), rq = zero4();
    float kq = 0.f, k2 = 0.f, q2 = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      if constexpr (!ND) p += s[r] * kk[r];
      rq += s[r] * qq[r];
      kq += kk[r] * qq[r];
    }
    if constexpr (P) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) { k2 += kk[r] * kk[r]; q2 += qq[r] * qq[r]; }
    }
    if constexpr (!ND) red_p[par][rg][cg] = p;
    red_r[par][rg][cg] = rq;
    if (cg == 0) {
      red_kq[par][rg][0] = kq;
      if constexpr (P) { red_kq[par][rg][1] = k2; red_kq[par][rg][2] = q2; }
    }
    __syncthreads();
    p = zero4();
    rq = zero4();
    kq = 0.f;
    k2 = 0.f;
    q2 = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      if constexpr (!ND) p += red_p[par][g][cg];
      rq += red_r[par][g][cg];
      kq += red_kq[par][g][0];
      if constexpr (P) { k2 += red_kq[par][g][1]; q2 += red_kq[par][g][2]; }
    }
    const int64_t tv = j * tok_v + nh;
    float alpha, beta;
    if constexpr (P) {
      const float ik = inv_norm(k2), iq = inv_norm(q2);
      p *= ik;
      rq *= iq;
      kq *= ik * iq;
#pragma unroll
      for (int r = 0; r < RPT; ++r) kk[r] *= ik;
      alpha = expf(neg_softplus(a.log_alpha[tv]));
      beta = sigmoid_of(a.beta[tv]);
    } else {
      alpha = expf(a.log_alpha[tv]);
      beta = a.beta[tv];
    }
    const E* vp = static_cast<const E*>(a.v) + tv * D + 4 * cg;
    f32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = ND ? beta * to_f(vp[e]) : beta * (to_f(vp[e]) - alpha * p[e]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) s[r] = decay_rank1(s[r], alpha, u, kk[r]);
    if (a.snapshots) {
      f32x4* snp = reinterpret_cast<f32x4*>(a.snapshots + tv * D * D) + (rg * RPT) * CG + cg;
#pragma unroll
      for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(s[r], snp + r * CG);
    }
    if (rg == 0) {
      Half<E> h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = to_e<E>(fmaf(alpha, rq[e], u[e] * kq));
      *reinterpret_cast<Half<E>*>(static_cast<E*>(a.o) + tv * D + 4 * cg) = h;
    }
  }
  if (!a.snapshots) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(s[r], sp + r * CG);
  }
}

template <typename E, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int threads = (D / 4) * DecodeShape<D>::RG;
  const unsigned blocks = (unsigned)(a.num_seqs * a.h_v);
  const dim3 g(blocks), b(threads);
  if (a.prep) {
    if (a.no_delta) gdn_kd_decode_step<E, D, true, true><<<g, b, 0, s>>>(a);
    else gdn_kd_decode_step<E, D, true, false><<<g, b, 0, s>>>(a);
  } else {
    if (a.no_delta) gdn_kd_decode_step<E, D, false, true><<<g, b, 0, s>>>(a);
    else gdn_kd_decode_step<E, D, false, false><<<g, b, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_decode_multi_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int threads = (D / 4) * DecodeShape<D>::RG;
  const unsigned blocks = (unsigned)(a.num_seqs * a.h_v);
  const dim3 g(blocks), b(threads);
  if (a.prep) {
    if (a.no_delta) gdn_kd_decode_multi<E, D, true, true><<<g, b, 0, s>>>(a);
    else gdn_kd_decode_multi<E, D, true, false><<<g, b, 0, s>>>(a);
  } else {
    if (a.no_delta) gdn_kd_decode_multi<E, D, false, true><<<g, b, 0, s>>>(a);
    else gdn_kd_decode_multi<E, D, false, false><<<g, b, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_multi(const DecodeArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == 1) {
    if (head_dim == 128) return launch_decode_multi_t<bf16_t, 128>(a, s);
    if (head_dim == 16) return launch_decode_multi_t<bf16_t, 16>(a, s);
  } else {
    if (head_dim == 128) return launch_decode_multi_t<float, 128>(a, s);
    if (head_dim == 16) return launch_decode_multi_t<float, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == 1) {
    if (head_dim == 128) return launch_decode_t<bf16_t, 128>(a, s);
    if (head_dim == 16) return launch_decode_t<bf16_t, 16>(a, s);
  } else {
    if (head_dim == 128) return launch_decode_t<float, 128>(a, s);
    if (head_dim == 16) return launch_decode_t<float, 16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
