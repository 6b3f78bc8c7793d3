// C ABI of libgdn: argument validation, workspace carving and dispatch to
// the kernel launchers. Host code only; nothing here touches the device
// until every argument has been checked.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status_t fail(gdn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gdn_status_t ok() {
  g_last_error.clear();
  return GDN_SUCCESS;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Validation shared by both entry points. decode selects the decode rules.
gdn_status_t check_dims(const gdn_dims_t* d, bool decode) {
  if (!d) return fail(GDN_ERROR_INVALID_VALUE, "dims is NULL");
  if (d->num_seqs < 1) return fail(GDN_ERROR_INVALID_VALUE, "num_seqs must be >= 1 (got %lld)", (long long)d->num_seqs);
  if (d->total_tokens < 0) return fail(GDN_ERROR_INVALID_VALUE, "total_tokens must be >= 0");
  if (d->total_tokens > INT32_MAX || d->num_seqs > INT32_MAX)
    return fail(GDN_ERROR_INVALID_VALUE, "total_tokens and num_seqs must fit int32 (cu_seqlens is int32)");
  if (d->h_qk < 1 || d->h_v < 1) return fail(GDN_ERROR_INVALID_VALUE, "h_qk and h_v must be >= 1");
  if (d->h_v % d->h_qk) return fail(GDN_ERROR_INVALID_VALUE, "h_v (%d) must be a multiple of h_qk (%d)", d->h_v, d->h_qk);
  if (d->h_v > 65535) return fail(GDN_ERROR_NOT_SUPPORTED, "h_v > 65535 is not supported");
  if (!decode && (d->total_tokens / (d->chunk > 0 ? d->chunk : 1) + d->num_seqs) * d->h_v > INT32_MAX)
    return fail(GDN_ERROR_NOT_SUPPORTED, "too many (chunk, V head) pairs for one launch");
  if (d->dk < 1 || d->dv < 1) return fail(GDN_ERROR_INVALID_VALUE, "dk and dv must be >= 1");
  if (d->dtype != GDN_DTYPE_F32 && d->dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERROR_INVALID_VALUE, "unknown dtype %d", d->dtype);
  if (d->flags & ~(GDN_FLAG_PREPARE_INPUTS | GDN_FLAG_NO_DELTA_RULE)) return fail(GDN_ERROR_INVALID_VALUE, "unknown flags 0x%x", d->flags);
  if (d->dk != d->dv) return fail(GDN_ERROR_NOT_SUPPORTED, "dk != dv is not supported (dk=%d dv=%d)", d->dk, d->dv);
  if (d->dk != 16 && d->dk != 128) return fail(GDN_ERROR_NOT_SUPPORTED, "head dim %d not supported (16 or 128)", d->dk);
  if (decode) {
    if (d->total_tokens != d->num_seqs)
      return fail(GDN_ERROR_INVALID_VALUE, "decode: total_tokens (%lld) must equal num_seqs (%lld)",
                  (long long)d->total_tokens, (long long)d->num_seqs);
  } else {
    if (d->chunk < 1) return fail(GDN_ERROR_INVALID_VALUE, "chunk must be >= 1");
    if (d->chunk != 16 && d->chunk != 64) return fail(GDN_ERROR_NOT_SUPPORTED, "chunk %d not supported (16 or 64)", d->chunk);
    if (!gdn::prefill_supported(d->dtype, d->dk, d->chunk))
      return fail(GDN_ERROR_NOT_SUPPORTED, "no prefill instance for dtype %d, head dim %d, chunk %d", d->dtype,
                  d->dk, d->chunk);
  }
  return GDN_SUCCESS;
}

struct Layout {
  gdn_workspace_layout_t v;
};

// Workspace regions, each 256-byte aligned, in this order.
Layout compute_layout(const gdn_dims_t& d) {
  const size_t esz = d.dtype == GDN_DTYPE_F32 ? 4 : 2;
  const size_t D = d.dk, C = d.chunk, N = d.num_seqs, T = d.total_tokens;
  const size_t HQ = d.h_qk, HV = d.h_v;
  const size_t CT = C / 16, DT = D / 16, CKS = (CT + 1) / 2;
  const size_t NC = T / C + N;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes, 256);
    return o;
  };
  Layout L;
  L.v.max_chunks = (int64_t)NC;
  L.v.chunk_table = take(NC * 16);
  L.v.seq_chunk_offset = take((N + 1) * 4);
  L.v.gate_prefix = take(NC * HV * C * 4);
  L.v.beta_chunk = take(NC * HV * C * 4);
  L.v.tinv = take(NC * HV * CT * CKS * 512 * esz);
  L.v.w = take(NC * HV * CT * ((DT + 1) / 2) * 512 * esz);
  L.v.key_t = take(NC * HQ * DT * CKS * 512 * esz);
  L.v.q_frag = take(NC * HQ * CT * ((DT + 1) / 2) * 512 * esz);
  L.v.pmask = take(NC * HV * CT * CKS * 512 * esz);
  L.v.dtab = take(NC * HV * (2 * C + 4) * 4);
  L.v.total = off;
  return L;
}

// Backward workspace: the forward regions, then the backward operands, each
// 256-byte aligned.
struct BwdLayout {
  Layout fwd;
  size_t k_frag, q_t, kq, pt, wt, tt, sc, ub, dsl, du, total;
};

BwdLayout compute_bwd_layout(const gdn_dims_t& d) {
  const size_t esz = d.dtype == GDN_DTYPE_F32 ? 4 : 2;
  const size_t D = d.dk, C = d.chunk, N = d.num_seqs, T = d.total_tokens;
  const size_t HQ = d.h_qk, HV = d.h_v;
  const size_t CT = C / 16, DT = D / 16, CKS = (CT + 1) / 2, DKS = (DT + 1) / 2;
  const size_t NC = T / C + N;
  BwdLayout L;
  L.fwd = compute_layout(d);
  size_t off = L.fwd.v.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes, 256);
    return o;
  };
  L.k_frag = take(NC * HQ * CT * DKS * 512 * esz);
  L.q_t = take(NC * HQ * DT * CKS * 512 * esz);
  L.kq = take(NC * HQ * CT * CKS * 512 * esz);
  L.pt = take(NC * HV * CT * CKS * 512 * esz);
  L.wt = take(NC * HV * DT * CKS * 512 * esz);
  L.tt = take(NC * HV * C * C * esz);
  L.sc = take(NC * HV * D * D * esz);
  L.ub = take(NC * HV * C * D * esz);
  L.dsl = take(NC * HV * D * D * esz);
  L.du = take(NC * HV * C * D * esz);
  L.total = off;
  return L;
}

// Opt-in debug checks, read from the environment at every call (a value
// other than empty or "0" turns them on):
//   GDN_DEBUG       prefill entry points copy cu_seqlens to the host (on
//                   the call's stream, then wait for it) and reject a table
//                   that is not 0 = c_0 <= c_1 <= ... <= c_N = T with
//                   GDN_ERROR_INVALID_VALUE before enqueueing anything;
//   GDN_DEBUG_SYNC  every entry point waits for its stream after enqueueing
//                   and reports a kernel that failed or faulted as
//                   GDN_ERROR_HIP, naming the entry point.
// Both synchronise with the host, which the calls otherwise never do.
bool env_on(const char* name) {
  const char* v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

gdn_status_t check_cu_seqlens_contents(const int32_t* h, int64_t n, int64_t total) {
  if (h[0] != 0) return fail(GDN_ERROR_INVALID_VALUE, "GDN_DEBUG: cu_seqlens[0] = %d, must be 0", h[0]);
  for (int64_t i = 0; i < n; ++i)
    if (h[i + 1] < h[i])
      return fail(GDN_ERROR_INVALID_VALUE, "GDN_DEBUG: cu_seqlens decreases at %lld (%d > %d)",
                  (long long)(i + 1), h[i], h[i + 1]);
  if (h[n] != total)
    return fail(GDN_ERROR_INVALID_VALUE, "GDN_DEBUG: cu_seqlens[%lld] = %d, must equal total_tokens %lld",
                (long long)n, h[n], (long long)total);
  return GDN_SUCCESS;
}

gdn_status_t debug_check_cu_seqlens(const int32_t* cu, int64_t n, int64_t total, hipStream_t stream) {
  if (!cu || !env_on("GDN_DEBUG")) return GDN_SUCCESS;
  std::vector<int32_t> h((size_t)n + 1);
  hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(GDN_ERROR_HIP, "GDN_DEBUG: reading cu_seqlens: %s", hipGetErrorString(e));
  return check_cu_seqlens_contents(h.data(), n, total);
}

gdn_status_t launch_status(hipError_t e, const char* what, hipStream_t stream) {
  if (e != hipSuccess) return fail(GDN_ERROR_HIP, "%s: %s", what, hipGetErrorString(e));
  if (env_on("GDN_DEBUG_SYNC")) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(GDN_ERROR_HIP, "GDN_DEBUG_SYNC: %s: %s", what, hipGetErrorString(e));
  }
  return ok();
}

// The backward pass's own support check, after check_dims.
gdn_status_t check_backward(const gdn_dims_t& d) {
  if (d.flags) return fail(GDN_ERROR_NOT_SUPPORTED, "the backward pass takes no flags (got 0x%x)", d.flags);
  if (!gdn::backward_supported(d.dtype, d.dk, d.chunk))
    return fail(GDN_ERROR_NOT_SUPPORTED, "the backward pass with fp32 inputs at head dim %d needs chunk 16", d.dk);
  return GDN_SUCCESS;
}

}  // namespace

gdn_status_t gdn::api_fail(gdn_status_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

extern "C" {

const char* gdn_status_string(gdn_status_t s) {
  switch (s) {
    case GDN_SUCCESS: return "GDN_SUCCESS";
    case GDN_ERROR_INVALID_VALUE: return "GDN_ERROR_INVALID_VALUE";
    case GDN_ERROR_NOT_SUPPORTED: return "GDN_ERROR_NOT_SUPPORTED";
    case GDN_ERROR_WORKSPACE: return "GDN_ERROR_WORKSPACE";
    case GDN_ERROR_HIP: return "GDN_ERROR_HIP";
  }
  return "GDN_UNKNOWN_STATUS";
}

const char* gdn_last_error_message(void) { return g_last_error.c_str(); }

size_t gdn_chunk_fwd_workspace_bytes(const gdn_dims_t* dims) {
  if (check_dims(dims, false) != GDN_SUCCESS) return 0;
  ok();
  return compute_layout(*dims).v.total;
}

gdn_status_t gdn_chunk_fwd_workspace_layout(const gdn_dims_t* dims, gdn_workspace_layout_t* layout) {
  const gdn_status_t st = check_dims(dims, false);
  if (st != GDN_SUCCESS) return st;
  if (!layout) return fail(GDN_ERROR_INVALID_VALUE, "layout is NULL");
  *layout = compute_layout(*dims).v;
  return ok();
}

gdn_status_t gdn_chunk_fwd(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return gdn_chunk_fwd_stages(dims, q, k, v, log_alpha, beta, init_state, cu_seqlens, o, final_state,
                              workspace, workspace_bytes, stream, 1, gdn::kPrefillStages);
}

gdn_status_t gdn_chunk_fwd_stages(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                                  const float* log_alpha, const float* beta, const float* init_state,
                                  const int32_t* cu_seqlens, void* o, float* final_state,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream,
                                  int first_stage, int last_stage) {
  if (first_stage < 1 || last_stage > gdn::kPrefillStages || first_stage > last_stage)
    return fail(GDN_ERROR_INVALID_VALUE, "stages %d..%d: need 1 <= first <= last <= %d", first_stage,
                last_stage, gdn::kPrefillStages);
  gdn_status_t st = check_dims(dims, false);
  if (st != GDN_SUCCESS) return st;
  const gdn_dims_t& d = *dims;
  if (!cu_seqlens && d.num_seqs != 1)
    return fail(GDN_ERROR_INVALID_VALUE, "cu_seqlens is NULL but num_seqs = %lld", (long long)d.num_seqs);
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(GDN_ERROR_INVALID_VALUE, "cu_seqlens is not 4-byte aligned");
  if (d.total_tokens > 0) {
    const void* need[] = {q, k, v, o, log_alpha, beta};
    const char* names[] = {"q", "k", "v", "o", "log_alpha", "beta"};
    for (int i = 0; i < 6; ++i) {
      const size_t al = i < 4 ? 16 : 4;
      if (!need[i]) return fail(GDN_ERROR_INVALID_VALUE, "%s is NULL", names[i]);
      if (!aligned(need[i], al)) return fail(GDN_ERROR_INVALID_VALUE, "%s is not %zu-byte aligned", names[i], al);
    }
    if (o == q || o == k || o == v || o == log_alpha || o == beta)
      return fail(GDN_ERROR_INVALID_VALUE, "o must not alias an input");
  }
  if (init_state && !aligned(init_state, 16)) return fail(GDN_ERROR_INVALID_VALUE, "init_state is not 16-byte aligned");
  if (final_state && !aligned(final_state, 16)) return fail(GDN_ERROR_INVALID_VALUE, "final_state is not 16-byte aligned");
  const Layout L = compute_layout(d);
  if (!workspace) return fail(GDN_ERROR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.v.total);
  if (!aligned(workspace, 256)) return fail(GDN_ERROR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.v.total)
    return fail(GDN_ERROR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, L.v.total);

  st = debug_check_cu_seqlens(cu_seqlens, d.num_seqs, d.total_tokens, stream);
  if (st != GDN_SUCCESS) return st;
  char* ws = static_cast<char*>(workspace);
  gdn::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.init_state = init_state;
  a.cu_seqlens = cu_seqlens;
  a.o = o;
  a.final_state = final_state;
  a.chunk_table = reinterpret_cast<int32_t*>(ws + L.v.chunk_table);
  a.seq_chunk_offset = reinterpret_cast<int32_t*>(ws + L.v.seq_chunk_offset);
  a.gate_prefix = reinterpret_cast<float*>(ws + L.v.gate_prefix);
  a.beta_chunk = reinterpret_cast<float*>(ws + L.v.beta_chunk);
  a.tinv = ws + L.v.tinv;
  a.w = ws + L.v.w;
  a.key_t = ws + L.v.key_t;
  a.q_frag = ws + L.v.q_frag;
  a.pmask = ws + L.v.pmask;
  a.dtab = reinterpret_cast<float*>(ws + L.v.dtab);
  a.num_seqs = d.num_seqs;
  a.total_tokens = d.total_tokens;
  a.max_chunks = L.v.max_chunks;
  a.h_qk = d.h_qk;
  a.h_v = d.h_v;
  a.group = d.h_v / d.h_qk;
  a.prep = (d.flags & GDN_FLAG_PREPARE_INPUTS) ? 1 : 0;
  a.no_delta = (d.flags & GDN_FLAG_NO_DELTA_RULE) ? 1 : 0;
  return launch_status(gdn::launch_prefill(a, d.dtype, d.dk, d.chunk, stream, first_stage, last_stage),
                       "gdn_chunk_fwd launch", stream);
}

size_t gdn_chunk_bwd_workspace_bytes(const gdn_dims_t* dims) {
  if (check_dims(dims, false) != GDN_SUCCESS) return 0;
  if (check_backward(*dims) != GDN_SUCCESS) return 0;
  if (dims->flags) {
    fail(GDN_ERROR_NOT_SUPPORTED, "the backward pass takes no flags (got 0x%x)", dims->flags);
    return 0;
  }
  ok();
  return compute_bwd_layout(*dims).total;
}

gdn_status_t gdn_chunk_bwd(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* init_state,
                           const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, void* dq,
                           void* dk, void* dv, float* dlog_alpha, float* dbeta, float* d_init_state,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gdn_chunk_bwd_stages(dims, q, k, v, log_alpha, beta, init_state, cu_seqlens, d_o, d_final_state, dq, dk,
                              dv, dlog_alpha, dbeta, d_init_state, workspace, workspace_bytes, stream, 1,
                              gdn::kBackwardStages);
}

gdn_status_t gdn_chunk_bwd_stages(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                                  const float* log_alpha, const float* beta, const float* init_state,
                                  const int32_t* cu_seqlens, const void* d_o, const float* d_final_state,
                                  void* dq, void* dk, void* dv, float* dlog_alpha, float* dbeta,
                                  float* d_init_state, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, int first_stage, int last_stage) {
  if (first_stage < 1 || last_stage > gdn::kBackwardStages || first_stage > last_stage)
    return fail(GDN_ERROR_INVALID_VALUE, "stages %d..%d: need 1 <= first <= last <= %d", first_stage,
                last_stage, gdn::kBackwardStages);
  gdn_status_t st = check_dims(dims, false);
  if (st != GDN_SUCCESS) return st;
  const gdn_dims_t& d = *dims;
  st = check_backward(d);
  if (st != GDN_SUCCESS) return st;
  if (!cu_seqlens && d.num_seqs != 1)
    return fail(GDN_ERROR_INVALID_VALUE, "cu_seqlens is NULL but num_seqs = %lld", (long long)d.num_seqs);
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return fail(GDN_ERROR_INVALID_VALUE, "cu_seqlens is not 4-byte aligned");
  if (d.total_tokens > 0) {
    const void* need[] = {q, k, v, d_o, dq, dk, dv, log_alpha, beta, dlog_alpha, dbeta};
    const char* names[] = {"q", "k", "v", "d_o", "dq", "dk", "dv", "log_alpha", "beta", "dlog_alpha", "dbeta"};
    for (int i = 0; i < 11; ++i) {
      const size_t al = i < 7 ? 16 : 4;
      if (!need[i]) return fail(GDN_ERROR_INVALID_VALUE, "%s is NULL", names[i]);
      if (!aligned(need[i], al)) return fail(GDN_ERROR_INVALID_VALUE, "%s is not %zu-byte aligned", names[i], al);
    }
    const void* ins[] = {q, k, v, log_alpha, beta, d_o};
    const void* outs[] = {dq, dk, dv, dlog_alpha, dbeta};
    for (const void* o : outs) {
      for (const void* i : ins)
        if (o == i) return fail(GDN_ERROR_INVALID_VALUE, "the gradients must not alias an input");
    }
    for (int i = 0; i < 5; ++i)
      for (int j = i + 1; j < 5; ++j)
        if (outs[i] == outs[j]) return fail(GDN_ERROR_INVALID_VALUE, "two gradient outputs alias");
  }
  if (init_state && !aligned(init_state, 16)) return fail(GDN_ERROR_INVALID_VALUE, "init_state is not 16-byte aligned");
  if (d_final_state && !aligned(d_final_state, 16))
    return fail(GDN_ERROR_INVALID_VALUE, "d_final_state is not 16-byte aligned");
  if (d_init_state && !aligned(d_init_state, 16))
    return fail(GDN_ERROR_INVALID_VALUE, "d_init_state is not 16-byte aligned");
  if (d_init_state && d_init_state == init_state)
    return fail(GDN_ERROR_INVALID_VALUE, "d_init_state must not alias init_state");
  const BwdLayout L = compute_bwd_layout(d);
  if (!workspace) return fail(GDN_ERROR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (!aligned(workspace, 256)) return fail(GDN_ERROR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(GDN_ERROR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, L.total);

  st = debug_check_cu_seqlens(cu_seqlens, d.num_seqs, d.total_tokens, stream);
  if (st != GDN_SUCCESS) return st;
  char* ws = static_cast<char*>(workspace);
  const gdn_workspace_layout_t& F = L.fwd.v;
  gdn::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.init_state = init_state;
  a.cu_seqlens = cu_seqlens;
  a.chunk_table = reinterpret_cast<int32_t*>(ws + F.chunk_table);
  a.seq_chunk_offset = reinterpret_cast<int32_t*>(ws + F.seq_chunk_offset);
  a.gate_prefix = reinterpret_cast<float*>(ws + F.gate_prefix);
  a.beta_chunk = reinterpret_cast<float*>(ws + F.beta_chunk);
  a.tinv = ws + F.tinv;
  a.w = ws + F.w;
  a.key_t = ws + F.key_t;
  a.q_frag = ws + F.q_frag;
  a.pmask = ws + F.pmask;
  a.dtab = reinterpret_cast<float*>(ws + F.dtab);
  a.backward = 1;
  a.k_frag = ws + L.k_frag;
  a.q_t = ws + L.q_t;
  a.kq = ws + L.kq;
  a.pt = ws + L.pt;
  a.wt = ws + L.wt;
  a.tt = ws + L.tt;
  a.sc = ws + L.sc;
  a.ub = ws + L.ub;
  a.dsl = ws + L.dsl;
  a.du = ws + L.du;
  a.d_o = d_o;
  a.d_final = d_final_state;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlog_alpha = dlog_alpha;
  a.dbeta = dbeta;
  a.d_init = d_init_state;
  a.num_seqs = d.num_seqs;
  a.total_tokens = d.total_tokens;
  a.max_chunks = F.max_chunks;
  a.h_qk = d.h_qk;
  a.h_v = d.h_v;
  a.group = d.h_v / d.h_qk;
  return launch_status(gdn::launch_backward(a, d.dtype, d.dk, d.chunk, stream, first_stage, last_stage),
                       "gdn_chunk_bwd launch", stream);
}

gdn_status_t gdn_decode_step(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, float* state, void* o,
                             hipStream_t stream) {
  gdn_status_t st = check_dims(dims, true);
  if (st != GDN_SUCCESS) return st;
  const gdn_dims_t& d = *dims;
  const void* need[] = {q, k, v, state, o, log_alpha, beta};
  const char* names[] = {"q", "k", "v", "state", "o", "log_alpha", "beta"};
  for (int i = 0; i < 7; ++i) {
    const size_t al = i < 5 ? 16 : 4;
    if (!need[i]) return fail(GDN_ERROR_INVALID_VALUE, "%s is NULL", names[i]);
    if (!aligned(need[i], al)) return fail(GDN_ERROR_INVALID_VALUE, "%s is not %zu-byte aligned", names[i], al);
  }
  if (o == q || o == k || o == v || o == log_alpha || o == beta || o == state)
    return fail(GDN_ERROR_INVALID_VALUE, "o must not alias an input");
  gdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.num_seqs = d.num_seqs;
  a.h_qk = d.h_qk;
  a.h_v = d.h_v;
  a.group = d.h_v / d.h_qk;
  a.num_tokens = 1;
  a.snapshots = nullptr;
  a.prep = (d.flags & GDN_FLAG_PREPARE_INPUTS) ? 1 : 0;
  a.no_delta = (d.flags & GDN_FLAG_NO_DELTA_RULE) ? 1 : 0;
  return launch_status(gdn::launch_decode(a, d.dtype, d.dk, stream), "gdn_decode_step launch", stream);
}

gdn_status_t gdn_decode_multi(const gdn_dims_t* dims, int32_t num_tokens, const void* q, const void* k,
                              const void* v, const float* log_alpha, const float* beta, float* state,
                              void* o, float* snapshots, hipStream_t stream) {
  gdn_status_t st = check_dims(dims, true);
  if (st != GDN_SUCCESS) return st;
  const gdn_dims_t& d = *dims;
  if (num_tokens < 1) return fail(GDN_ERROR_INVALID_VALUE, "num_tokens must be >= 1 (got %d)", num_tokens);
  if ((int64_t)num_tokens * d.num_seqs > INT32_MAX)
    return fail(GDN_ERROR_NOT_SUPPORTED, "num_tokens * num_seqs must fit int32");
  const void* need[] = {q, k, v, state, o, log_alpha, beta};
  const char* names[] = {"q", "k", "v", "state", "o", "log_alpha", "beta"};
  for (int i = 0; i < 7; ++i) {
    const size_t al = i < 5 ? 16 : 4;
    if (!need[i]) return fail(GDN_ERROR_INVALID_VALUE, "%s is NULL", names[i]);
    if (!aligned(need[i], al)) return fail(GDN_ERROR_INVALID_VALUE, "%s is not %zu-byte aligned", names[i], al);
  }
  if (o == q || o == k || o == v || o == log_alpha || o == beta || o == state || (snapshots && o == snapshots))
    return fail(GDN_ERROR_INVALID_VALUE, "o must not alias an input");
  if (snapshots && !aligned(snapshots, 16)) return fail(GDN_ERROR_INVALID_VALUE, "snapshots is not 16-byte aligned");
  if (snapshots == state) return fail(GDN_ERROR_INVALID_VALUE, "snapshots must not alias state");
  gdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.num_seqs = d.num_seqs;
  a.h_qk = d.h_qk;
  a.h_v = d.h_v;
  a.group = d.h_v / d.h_qk;
  a.num_tokens = num_tokens;
  a.snapshots = snapshots;
  a.prep = (d.flags & GDN_FLAG_PREPARE_INPUTS) ? 1 : 0;
  a.no_delta = (d.flags & GDN_FLAG_NO_DELTA_RULE) ? 1 : 0;
  return launch_status(gdn::launch_decode_multi(a, d.dtype, d.dk, stream), "gdn_decode_multi launch", stream);
}

}  // extern "C"
