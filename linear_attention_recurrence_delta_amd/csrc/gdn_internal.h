// Internal interface between the C ABI (gdn_api.cpp) and the kernel
// launchers (gdn_prefill.hip, gdn_decode.hip). Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Sets the calling thread's error message (gdn_last_error_message) and
// returns `status`; for entry points defined outside gdn_api.cpp.
gdn_status_t api_fail(gdn_status_t status, const char* fmt, ...);

// Everything one gdn_chunk_fwd call needs on the device. Workspace regions
// are typed pointers carved by the host (see the layout in gdn_api.cpp).
struct PrefillArgs {
  const void* q;            // [T, HQ, D]
  const void* k;            // [T, HQ, D]
  const void* v;            // [T, HV, D]
  const float* log_alpha;   // [T, HV]
  const float* beta;        // [T, HV]
  const float* init_state;  // [N, HV, D, D] or null
  const int32_t* cu_seqlens;  // [N+1] or null (one sequence)
  void* o;                  // [T, HV, D]
  float* final_state;       // [N, HV, D, D] or null
  // workspace (MFMA fragment layouts are described in gdn_prefill.hip)
  int32_t* chunk_table;     // [NC][4]: sequence, first token, length, index in sequence
  int32_t* seq_chunk_offset;  // [N+1]
  float* gate_prefix;       // [NC][HV][C]  in-chunk inclusive prefix of log a
  float* beta_chunk;        // [NC][HV][C]  b per chunk row (0 past the chunk end)
  void* tinv;               // [NC][HV] fragments of (I + A)^{-1} diag(b)
  void* w;                  // [NC][HV] fragments of W = (I + A)^{-1} diag(b exp(g)) K
  void* key_t;              // [NC][HQ] fragments of K^T
  void* q_frag;             // [NC][HQ] fragments of Q
  void* pmask;              // [NC][HV] fragments of the masked, decayed q.k products
  float* dtab;              // [NC][HV][2C+4] scan row factors exp(g), exp(g_L - g), exp(g_L)
  // backward pass only (null in the forward pass); E = the q/k/v dtype
  void* k_frag;             // [NC][HQ] fragments of K (row r, k = d)             kernel 1
  void* q_t;                // [NC][HQ] fragments of Q^T (row d, k = token r)     kernel 1
  void* kq;                 // [NC][HQ] fragments of (q_r . k_j) (col j = key, k = query r)  kernel 1
  void* pt;                 // [NC][HV] fragments of P^T (row j = key, k = query r)  kernel 2
  void* wt;                 // [NC][HV] fragments of W^T (row d, k = token r)     kernel 2
  void* tt;                 // [NC][HV][C][C] E, Tinv^T row-major (tt[i][r] = Tinv[r][i])  kernel 2
  void* sc;                 // [NC][HV][D][D] E, state at each chunk's start      kernel 3
  void* ub;                 // [NC][HV][C][D] E, the chunk's U rows               kernel 3
  void* dsl;                // [NC][HV][D][D] E, dL/d(state at each chunk's end)  reverse scan
  void* du;                 // [NC][HV][C][D] E, dL/dU rows                       reverse scan
  const void* d_o;          // [T, HV, D] dL/do
  const float* d_final;     // [N, HV, D, D] dL/d(final state), or null (zero)
  void* dq;                 // [T, HQ, D]
  void* dk;                 // [T, HQ, D]
  void* dv;                 // [T, HV, D]
  float* dlog_alpha;        // [T, HV]
  float* dbeta;             // [T, HV]
  float* d_init;            // [N, HV, D, D] or null
  int64_t num_seqs;         // N
  int64_t total_tokens;     // T
  int64_t max_chunks;       // NC = floor(T/C) + N
  int64_t win_lo;           // chunk-slot window [win_lo, win_hi) of one launch (set by the
  int64_t win_hi;           //    launcher): kernel 2 forms those slots, the scan runs them
  int32_t h_qk;             // HQ
  int32_t h_v;              // HV
  int32_t group;            // HV / HQ
  int32_t prep;             // 1: raw q, k and gate logits (fused input preparation)
  int32_t no_delta;         // 1: gate-only update S = a S + b k v^T
  int32_t backward;         // 1: kernels 1-3 in their backward-pass modes (the fields
                            //    marked backward pass only are set); chosen by this flag,
                            //    not by which workspace pointers happen to be set
};

struct DecodeArgs {
  const void* q;            // [N, HQ, D]
  const void* k;            // [N, HQ, D]
  const void* v;            // [N, HV, D]
  const float* log_alpha;   // [N, HV]
  const float* beta;        // [N, HV]
  float* state;             // [N, HV, D, D], in place
  void* o;                  // [N, HV, D]
  int64_t num_seqs;
  int32_t h_qk;
  int32_t h_v;
  int32_t group;
  // multi-token verify only: tokens per sequence (inputs and o gain a
  // leading [K] dimension) and the per-token states [K, N, HV, D, D], or
  // null to update `state` in place
  int32_t num_tokens;
  float* snapshots;
  int32_t prep;             // 1: raw q, k and gate logits (fused input preparation)
  int32_t no_delta;         // 1: gate-only update S = a S + b k v^T
};

// Prefill launch stages (1-based): 1 chunk preparation and inverse (kernel
// 2: chunk table, gate prefix sums, K^T and Q fragments, (I + A)^{-1}, W, P,
// row factors), 2 the fused scan. The backward pass runs kernels 1, 2 and 3
// as its stages 1-3 (PrefillArgs::backward).
constexpr int kPrefillStages = 2;

// True when the prefill kernels have an instance for (dtype, head_dim, chunk).
inline bool prefill_supported(int dtype, int head_dim, int chunk) {
  if (head_dim != 16 && head_dim != 128) return false;
  if (chunk != 16 && chunk != 64) return false;
  return dtype == 0 || dtype == 1;
}
// The backward pass has every prefill instance except fp32 at head dim 128
// with 64-token chunks (its reverse scan's fp32 fragments do not fit LDS).
inline bool backward_supported(int dtype, int head_dim, int chunk) {
  return prefill_supported(dtype, head_dim, chunk) && !(dtype == 0 && head_dim == 128 && chunk == 64);
}

// dtype: 0 = fp32, 1 = bf16. Returns the first launch error, if any.
// Runs stages first..last (1-based, inclusive).
hipError_t launch_prefill(const PrefillArgs& args, int dtype, int head_dim, int chunk,
                          hipStream_t stream, int first_stage, int last_stage);
hipError_t launch_decode(const DecodeArgs& args, int dtype, int head_dim, hipStream_t stream);
// Backward pass: kernels 1 and 2 with their backward outputs, the saving
// scan, the reverse state scan and the gradient kernel (gdn_backward.hip).
// Stages (1-based): 1-3 the forward kernels with their backward outputs,
// 4 the reverse state scan, 5 the gradient kernel.
constexpr int kBackwardStages = 5;
hipError_t launch_backward(const PrefillArgs& args, int dtype, int head_dim, int chunk, hipStream_t stream,
                           int first_stage, int last_stage);
hipError_t launch_decode_multi(const DecodeArgs& args, int dtype, int head_dim, hipStream_t stream);

}  // namespace gdn
