/*
 * libgdn -- Gated DeltaNet token mixer for AMD Instinct MI355X (gfx950).
 *
 * The method (page "Qwen3.8-Flash-Next 技术总结：Qwen4 架构的'探路者'",
 * section 2.1 "Gated DeltaNet", state-update equation) keeps one dk x dv
 * state per V head and updates it per token as
 *     S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
 *         = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T
 * with a_t in (0,1] the forget gate and b_t the delta-rule write strength.
 * The layer output of this library is o_t = S_t^T q_t (post-update state,
 * no scaling). Section 2.1 gives the head layout (16 QK heads, 48 V heads,
 * head dim 128): V head h reads QK head h / (h_v / h_qk).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller,
 *    contiguous row-major with the last dimension fastest; q, k, v, o and
 *    states must be 16-byte aligned, log_alpha, beta and cu_seqlens 4-byte.
 *  - The library allocates no device memory and keeps no global state
 *    besides a thread-local error string (gdn_chunk_fwd_noalloc adds its
 *    static device array, described there).
 *  - Calls enqueue work on `stream` (NULL = the default stream) and return
 *    without synchronising; device faults surface at the caller's next sync.
 *  - Invalid arguments return an error status before anything is enqueued;
 *    gdn_last_error_message() then says which argument.
 *  - Supported: dk == dv in {16, 128}; chunk in {16, 64}; h_v % h_qk == 0;
 *    dtype GDN_DTYPE_F32 or GDN_DTYPE_BF16 for q, k, v and o, except the
 *    fp32 backward pass at head dim 128 with chunk 64
 *    (GDN_ERROR_NOT_SUPPORTED; use chunk 16). Gates and states are always
 *    fp32.
 *  - Environment (read at each call, for debugging): GDN_DEBUG=1 makes the
 *    prefill entry points (forward and backward) copy cu_seqlens to the host
 *    and check it before launching, returning GDN_ERROR_INVALID_VALUE for a
 *    table that breaks its contract (this synchronises the stream);
 *    GDN_DEBUG_SYNC=1 makes every entry point wait for its stream after
 *    enqueueing and report a failed kernel as GDN_ERROR_HIP.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_SUCCESS = 0,
  GDN_ERROR_INVALID_VALUE = 1, /* bad pointer, size, alignment or shape */
  GDN_ERROR_NOT_SUPPORTED = 2, /* valid but not built: head dim, chunk, dtype */
  GDN_ERROR_WORKSPACE = 3,     /* workspace missing, misaligned or too small */
  GDN_ERROR_HIP = 4            /* a HIP launch failed; see the message */
} gdn_status_t;

typedef enum {
  GDN_DTYPE_F32 = 0,  /* IEEE float32 q, k, v, o */
  GDN_DTYPE_BF16 = 1  /* bfloat16 q, k, v, o (fp32 accumulation and state) */
} gdn_dtype_t;

/*
 * Flags (gdn_dims_t.flags).
 * GDN_FLAG_PREPARE_INPUTS: fused input preparation. q and k are raw; every
 *   kernel that reads them L2-normalises each (token, head) vector as
 *   x / sqrt(max(sum x^2, 1e-12)) in fp32 (prefill then rounds the unit
 *   vectors to the input dtype for its matrix products). The `log_alpha`
 *   and `beta` arguments carry gate logits a and b, mapped to
 *   log(alpha) = -softplus(a) and beta = sigmoid(b). Section 2.1 makes
 *   the gates data-dependent; these maps are the ones of the configured
 *   input recipe.
 * GDN_FLAG_NO_DELTA_RULE: the gate-only variant that section 2.1 sets
 *   against the gated delta rule (the Mamba2-style forget gate without the
 *   delta rule's correction): S_t = alpha_t S_{t-1} + beta_t k_t v_t^T, with
 *   the same readout o_t = S_t^T q_t, gates, layouts and workspace. beta = 1
 *   gives plain gated linear attention. The delta rule alone (DeltaNet)
 *   needs no flag: it is log_alpha = 0.
 * The flags combine.
 */
enum { GDN_FLAG_PREPARE_INPUTS = 1, GDN_FLAG_NO_DELTA_RULE = 2 };

typedef struct {
  int64_t num_seqs;     /* N >= 1: packed sequences (prefill) or batch (decode) */
  int64_t total_tokens; /* T >= 0: packed tokens; decode: must equal num_seqs */
  int32_t h_qk;         /* QK heads, >= 1 */
  int32_t h_v;          /* V heads, a multiple of h_qk */
  int32_t dk;           /* key/query head dim */
  int32_t dv;           /* value head dim (must equal dk) */
  int32_t chunk;        /* prefill chunk length C (ignored by decode) */
  int32_t dtype;        /* gdn_dtype_t of q, k, v, o */
  int32_t flags;        /* 0 or an OR of GDN_FLAG_PREPARE_INPUTS, GDN_FLAG_NO_DELTA_RULE */
} gdn_dims_t;

/*
 * Prefill of packed variable-length sequences with the chunkwise
 * WY-representation algorithm that section 2.1 names (each chunk of C tokens
 * becomes dense block products; chunks are scanned in order to carry the
 * state), producing the same result as the token-serial update up to
 * rounding.
 *
 *  q, k        [T, h_qk, dk]  dtype
 *  v           [T, h_v, dv]   dtype
 *  log_alpha   [T, h_v]       fp32, log a_t <= 0 (not clamped)
 *  beta        [T, h_v]       fp32, any finite value
 *  init_state  [N, h_v, dk, dv] fp32, or NULL for zeros
 *  cu_seqlens  [N+1] int32 device array: 0 = c_0 <= c_1 <= ... <= c_N = T,
 *              sequence n holds tokens [c_n, c_{n+1}); NULL means one
 *              sequence of T tokens (N must be 1). The contents are a
 *              precondition, checked only under GDN_DEBUG=1; the kernels
 *              clamp every entry into [0, T] (and each end to at least its
 *              start), so a bad table gives wrong results but no access
 *              outside the buffers described here. Empty sequences are
 *              allowed (their final state equals their initial state).
 *  o           [T, h_v, dv]   dtype, written; must not alias any input
 *  final_state [N, h_v, dk, dv] fp32 or NULL; may alias init_state exactly
 *  workspace   device scratch of at least gdn_chunk_fwd_workspace_bytes()
 *              bytes, 256-byte aligned, owned by the caller; its contents on
 *              return are unspecified. Calls that run concurrently need
 *              distinct workspaces.
 *
 * Streams: the work is ordered on `stream` as if all of it were enqueued
 * there. When the scan's workgroups (one per sequence, V head and 32 state
 * columns) would leave at least a fifth of the CUs idle, the input has at
 * least 256 chunk slots, final_state is given and `stream` belongs to the
 * current device, the call also uses one stream per device that the
 * library creates on first use (default priority, on the current device)
 * and keeps for the process: kernel 2 forms the later chunks there
 * while the scan runs the earlier ones, joined to `stream` by events (the
 * fork and join can be captured in a HIP graph). Results are bitwise those
 * of the stage-by-stage calls below, which gdn_chunk_fwd_noalloc makes.
 *
 * Returns GDN_SUCCESS once all kernels are enqueued.
 */
gdn_status_t gdn_chunk_fwd(const gdn_dims_t* dims,
                           const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           const float* init_state, const int32_t* cu_seqlens,
                           void* o, float* final_state,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Diagnostic variant of gdn_chunk_fwd that enqueues only launches
 * first_stage..last_stage, so a profiler or benchmark can put events between
 * them: 1 = chunk table, gate prefix sums, the K^T and Q layouts, Q K^T and
 * K K^T, (I + A)^{-1}, W, the masked and decayed Q K^T and the row factors;
 * 2 = the fused U construction, inter-chunk state scan and output products.
 * Arguments are those of gdn_chunk_fwd. Stage 2 reads what stage 1 left in
 * `workspace`, so a call starting at stage 2 must follow a call that ran
 * stage 1 with identical arguments and workspace on the same stream.
 * gdn_chunk_fwd is gdn_chunk_fwd_stages(..., 1, 2); any other stage range
 * enqueues one launch per stage on `stream`, one after the other. Returns
 * GDN_ERROR_INVALID_VALUE unless 1 <= first_stage <= last_stage <= 2.
 */
gdn_status_t gdn_chunk_fwd_stages(const gdn_dims_t* dims,
                                  const void* q, const void* k, const void* v,
                                  const float* log_alpha, const float* beta,
                                  const float* init_state, const int32_t* cu_seqlens,
                                  void* o, float* final_state,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, int first_stage, int last_stage);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results, with the workspace taken
 * from a device array of GDN_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends. The caller still
 * passes inputs and outputs. Makes no hipMalloc, hipFree or other
 * allocating call, and enqueues everything on `stream`. Dims whose gdn_chunk_fwd_workspace_bytes() exceeds
 * GDN_NOALLOC_SCRATCH_BYTES (at 16 QK / 48 V heads, head dim 128, bf16,
 * chunk 64: about 3,900 tokens) return GDN_ERROR_WORKSPACE before anything
 * is enqueued. The array belongs to the device current at the call, which
 * must be the device of `stream`; its address is looked up once per device
 * on the first call there. All calls on one GPU share that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race, so a
 * caller serialises them. Nothing carries over between calls.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status_t gdn_chunk_fwd_noalloc(const gdn_dims_t* dims,
                                   const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta,
                                   const float* init_state, const int32_t* cu_seqlens,
                                   void* o, float* final_state, hipStream_t stream);

/* Workspace bytes gdn_chunk_fwd needs for these dims; 0 if dims are invalid
 * or unsupported (gdn_last_error_message() says why). The size depends on
 * (num_seqs, total_tokens, h_qk, h_v, dk, chunk, dtype) only. */
size_t gdn_chunk_fwd_workspace_bytes(const gdn_dims_t* dims);

/*
 * Backward pass of gdn_chunk_fwd: gradients of a scalar loss L with respect
 * to every input, given dL/do and dL/d(final state). Section 2.1 presents
 * the chunkwise algorithm as the way to train the layer; the gradients are
 * the derivative of the token-serial update (backpropagation through it),
 * evaluated chunkwise: the forward kernels are run again, the state
 * gradient is carried over the chunks in reverse order, and the per-chunk
 * gradients are formed from it. flags must be 0 (GDN_ERROR_NOT_SUPPORTED
 * otherwise).
 *
 *  q, k, v, log_alpha, beta, init_state, cu_seqlens: as for gdn_chunk_fwd
 *  d_o          [T, h_v, dv] dtype: dL/do
 *  d_final_state [N, h_v, dk, dv] fp32 or NULL (zero): dL/d(final state)
 *  dq, dk       [T, h_qk, dk] dtype, written: a QK head's gradient sums
 *               over the V heads that read it
 *  dv           [T, h_v, dv] dtype, written
 *  dlog_alpha, dbeta [T, h_v] fp32, written: dL/d(log a_t), dL/db_t
 *  d_init_state [N, h_v, dk, dv] fp32 or NULL: dL/d(init_state), written;
 *               may alias d_final_state exactly, not init_state
 *  workspace    device scratch of at least gdn_chunk_bwd_workspace_bytes()
 *               bytes, 256-byte aligned, owned by the caller; contents on
 *               return unspecified
 * The gradients must not alias an input or each other. Returns GDN_SUCCESS
 * once all kernels are enqueued.
 */
gdn_status_t gdn_chunk_bwd(const gdn_dims_t* dims,
                           const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           const float* init_state, const int32_t* cu_seqlens,
                           const void* d_o, const float* d_final_state,
                           void* dq, void* dk, void* dv,
                           float* dlog_alpha, float* dbeta, float* d_init_state,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Diagnostic variant of gdn_chunk_bwd enqueuing launches first..last only
 * (for events between them): 1 = chunk table, gate prefix sums and the K^T,
 * K, Q^T and query-indexed Q K^T layouts; 2 = (I + A)^{-1}, W and the
 * backward operands P^T, W^T and Tinv^T; 3 = the state scan, storing the
 * state at each chunk start and the chunk's U rows instead of outputs;
 * 4 = the reverse state scan; 5 = the gradient kernel. A call starting at stage s > 1 must follow calls that ran
 * stages 1..s-1 with identical arguments and workspace on the same stream.
 * Returns GDN_ERROR_INVALID_VALUE unless 1 <= first_stage <= last_stage <= 5.
 */
gdn_status_t gdn_chunk_bwd_stages(const gdn_dims_t* dims,
                                  const void* q, const void* k, const void* v,
                                  const float* log_alpha, const float* beta,
                                  const float* init_state, const int32_t* cu_seqlens,
                                  const void* d_o, const float* d_final_state,
                                  void* dq, void* dk, void* dv,
                                  float* dlog_alpha, float* dbeta, float* d_init_state,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, int first_stage, int last_stage);

/* Workspace bytes gdn_chunk_bwd needs (gdn_chunk_fwd's and the backward
 * operands); 0 if dims are invalid or unsupported. */
size_t gdn_chunk_bwd_workspace_bytes(const gdn_dims_t* dims);

/*
 * One decode step: one new token for each of N independent sequences, the
 * single-token form of the update in section 2.1 applied in place:
 *     p = S^T k, u = b (v - a p), S <- a S + k u^T, o = S^T q.
 *
 *  q, k       [N, h_qk, dk] dtype
 *  v          [N, h_v, dv]  dtype
 *  log_alpha  [N, h_v] fp32;  beta [N, h_v] fp32
 *  state      [N, h_v, dk, dv] fp32, read and overwritten in place
 *  o          [N, h_v, dv] dtype, written; must not alias any input
 * dims->total_tokens must equal dims->num_seqs; dims->chunk is ignored.
 */
gdn_status_t gdn_decode_step(const gdn_dims_t* dims,
                             const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta,
                             float* state, void* o, hipStream_t stream);

/*
 * Speculative multi-token verify for decode: K drafted tokens per sequence,
 * applied in order as K successive steps of the single-token update of
 * section 2.1 (the same update as gdn_decode_step), in one pass over the
 * state. Result j equals the j-th of K gdn_decode_step calls on the same
 * inputs.
 *
 *  num_tokens K >= 1 (K * N must fit int32)
 *  q, k       [K, N, h_qk, dk] dtype   (token j's gdn_decode_step inputs at j)
 *  v          [K, N, h_v, dv]  dtype
 *  log_alpha  [K, N, h_v] fp32;  beta [K, N, h_v] fp32
 *  state      [N, h_v, dk, dv] fp32
 *  o          [K, N, h_v, dv] dtype, written; must not alias any input
 *  snapshots  [K, N, h_v, dk, dv] fp32 or NULL. Non-NULL: snapshot j gets the
 *             state after token j and `state` is only read, so the caller
 *             can continue from any accepted prefix (from `state` itself if
 *             none is accepted). NULL: `state` is overwritten with the state
 *             after all K tokens. Must not alias `state`.
 * dims->total_tokens must equal dims->num_seqs; dims->chunk is ignored.
 */
gdn_status_t gdn_decode_multi(const gdn_dims_t* dims, int32_t num_tokens,
                              const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta,
                              float* state, void* o, float* snapshots,
                              hipStream_t stream);

/* Static name of a status code. */
const char* gdn_status_string(gdn_status_t status);

/* Thread-local text describing the last error returned on this thread
 * ("" if none). Valid until the next libgdn call on the same thread. */
const char* gdn_last_error_message(void);

/*
 * Diagnostic view of gdn_chunk_fwd's workspace, for tests that compare the
 * per-stage intermediates with a reference. Byte offsets from the workspace
 * base; each region is described where the kernels are defined. Returns
 * GDN_SUCCESS or the validation error of `dims`.
 */
typedef struct {
  size_t chunk_table;  /* int32 [max_chunks][4]: seq, first token, length, index in seq */
  size_t seq_chunk_offset; /* int32 [N+1]: first compact chunk of each sequence */
  size_t gate_prefix;  /* fp32 [max_chunks][h_v][C]: in-chunk inclusive prefix of log a (backward pass) */
  size_t beta_chunk;   /* fp32 [max_chunks][h_v][C]: b of each chunk row, 0 past its end (backward pass) */
  size_t tinv;         /* dtype [max_chunks][h_v]: (I + A)^{-1} diag(b) as MFMA fragments */
  size_t w;            /* dtype [max_chunks][h_v]: W = (I + A)^{-1} diag(b exp(g)) K as MFMA fragments */
  size_t key_t;        /* dtype [max_chunks][h_qk]: K^T as MFMA fragments */
  size_t q_frag;       /* dtype [max_chunks][h_qk]: Q as MFMA fragments */
  size_t pmask;        /* dtype [max_chunks][h_v]: q_r . k_j exp(g_r - g_j), j <= r, as fragments */
  size_t dtab;         /* fp32 [max_chunks][h_v][2C+4]: exp(g_r), exp(g_L - g_r), exp(g_L), pad */
  size_t total;        /* == gdn_chunk_fwd_workspace_bytes(dims) */
  int64_t max_chunks;  /* floor(T / C) + N, the bound on the number of chunks */
} gdn_workspace_layout_t;

gdn_status_t gdn_chunk_fwd_workspace_layout(const gdn_dims_t* dims,
                                            gdn_workspace_layout_t* layout);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
