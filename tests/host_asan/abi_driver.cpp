// Drives the C ABI's host code (gdn_api.cpp) with the HIP stand-ins of
// hip_stub.cpp, built with g++ -fsanitize=address,undefined: validation,
// workspace carving, the arguments handed to the launchers, and the opt-in
// GDN_DEBUG (cu_seqlens contents) and GDN_DEBUG_SYNC paths. Buffers are host
// memory standing in for device memory. Prints "abi driver: N checks ok"
// and exits 0, or names each failed check and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "gdn.h"
#include "stub_state.h"

static int g_checks = 0, g_failed = 0;

#define CHECK(cond)                                                             \
  do {                                                                          \
    ++g_checks;                                                                 \
    if (!(cond)) {                                                              \
      ++g_failed;                                                               \
      fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, \
              #cond, gdn_last_error_message());                                 \
    }                                                                           \
  } while (0)

static bool msg_has(const char* s) { return strstr(gdn_last_error_message(), s) != nullptr; }

// 256-byte aligned host buffer
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes ? bytes : 256) { p = aligned_alloc(256, (n + 255) / 256 * 256); memset(p, 0, n); }
  ~Buf() { free(p); }
  template <typename T> T* as() const { return static_cast<T*>(p); }
  bool holds(const void* q, size_t bytes) const {
    const char* c = static_cast<const char*>(q);
    return c >= static_cast<const char*>(p) && c + bytes <= static_cast<const char*>(p) + n;
  }
};

static gdn_dims_t dims(int64_t n, int64_t t, int32_t hq, int32_t hv, int32_t d, int32_t c, int32_t dt) {
  gdn_dims_t x;
  memset(&x, 0, sizeof(x));
  x.num_seqs = n;
  x.total_tokens = t;
  x.h_qk = hq;
  x.h_v = hv;
  x.dk = x.dv = d;
  x.chunk = c;
  x.dtype = dt;
  return x;
}

struct Prefill {
  gdn_dims_t d;
  size_t esz;
  Buf q, k, v, la, b, init, cu, o, fin, ws;
  Prefill(const gdn_dims_t& dd, const std::vector<int32_t>& table)
      : d(dd), esz(dd.dtype == GDN_DTYPE_BF16 ? 2 : 4),
        q(dd.total_tokens * dd.h_qk * dd.dk * esz), k(dd.total_tokens * dd.h_qk * dd.dk * esz),
        v(dd.total_tokens * dd.h_v * dd.dv * esz), la(dd.total_tokens * dd.h_v * 4), b(dd.total_tokens * dd.h_v * 4),
        init(dd.num_seqs * dd.h_v * dd.dk * dd.dv * 4), cu((dd.num_seqs + 1) * 4),
        o(dd.total_tokens * dd.h_v * dd.dv * esz), fin(dd.num_seqs * dd.h_v * dd.dk * dd.dv * 4),
        ws(gdn_chunk_fwd_workspace_bytes(&dd)) {
    memcpy(cu.p, table.data(), table.size() * 4);
  }
  gdn_status_t run(const int32_t* cu_override = nullptr, bool use_cu = true) {
    return gdn_chunk_fwd(&d, q.p, k.p, v.p, la.as<float>(), b.as<float>(), init.as<float>(),
                         use_cu ? (cu_override ? cu_override : cu.as<int32_t>()) : nullptr, o.p, fin.as<float>(),
                         ws.p, ws.n, nullptr);
  }
};

static void test_validation() {
  gdn_dims_t d = dims(0, 128, 16, 48, 128, 64, GDN_DTYPE_BF16);
  CHECK(gdn_chunk_fwd_workspace_bytes(&d) == 0);
  d = dims(1, 128, 16, 47, 128, 64, GDN_DTYPE_BF16);
  CHECK(gdn_chunk_fwd_workspace_bytes(&d) == 0 && msg_has("multiple"));
  d = dims(1, 128, 16, 48, 64, 64, GDN_DTYPE_BF16);
  gdn_workspace_layout_t lay;
  CHECK(gdn_chunk_fwd_workspace_layout(&d, &lay) == GDN_ERROR_NOT_SUPPORTED);
  d = dims(1, 128, 16, 48, 128, 32, GDN_DTYPE_BF16);
  CHECK(gdn_chunk_fwd_workspace_layout(&d, &lay) == GDN_ERROR_NOT_SUPPORTED);
  d = dims(1, 128, 16, 48, 128, 64, 9);
  CHECK(gdn_chunk_fwd_workspace_layout(&d, &lay) == GDN_ERROR_INVALID_VALUE);
  d = dims(1, 128, 16, 48, 128, 64, GDN_DTYPE_BF16);
  d.flags = 8;
  CHECK(gdn_chunk_fwd_workspace_layout(&d, &lay) == GDN_ERROR_INVALID_VALUE);
  CHECK(gdn_chunk_fwd_workspace_layout(nullptr, &lay) == GDN_ERROR_INVALID_VALUE);
  CHECK(strcmp(gdn_status_string(GDN_ERROR_WORKSPACE), "GDN_ERROR_WORKSPACE") == 0);
  CHECK(strcmp(gdn_status_string((gdn_status_t)99), "GDN_UNKNOWN_STATUS") == 0);
}

static void test_prefill_args() {
  const std::vector<int32_t> table = {0, 100, 100, 250};
  Prefill p(dims(3, 250, 2, 6, 128, 64, GDN_DTYPE_BF16), table);
  gdn_workspace_layout_t lay;
  CHECK(gdn_chunk_fwd_workspace_layout(&p.d, &lay) == GDN_SUCCESS);
  CHECK(lay.total == p.ws.n && lay.max_chunks == 250 / 64 + 3);
  const int before = g_stub.launches;
  CHECK(p.run() == GDN_SUCCESS);
  CHECK(g_stub.launches == before + 1 && g_stub.first == 1 && g_stub.last == 2);
  const gdn::PrefillArgs& a = g_stub.prefill;
  CHECK(a.q == p.q.p && a.k == p.k.p && a.v == p.v.p && a.o == p.o.p && a.cu_seqlens == p.cu.p);
  CHECK(a.num_seqs == 3 && a.total_tokens == 250 && a.group == 3 && a.max_chunks == lay.max_chunks);
  CHECK(a.backward == 0 && a.prep == 0 && a.no_delta == 0);
  // every workspace region starts inside the workspace, 256-byte aligned
  const void* regions[] = {a.chunk_table, a.seq_chunk_offset, a.gate_prefix, a.beta_chunk, a.tinv, a.w,
                           a.key_t, a.q_frag, a.pmask, a.dtab};
  for (const void* r : regions) {
    CHECK(p.ws.holds(r, 1));
    CHECK((reinterpret_cast<uintptr_t>(r) - reinterpret_cast<uintptr_t>(p.ws.p)) % 256 == 0);
  }
  // a workspace one byte short is rejected before any launch
  const int n0 = g_stub.launches;
  CHECK(gdn_chunk_fwd(&p.d, p.q.p, p.k.p, p.v.p, p.la.as<float>(), p.b.as<float>(), nullptr, p.cu.as<int32_t>(),
                      p.o.p, nullptr, p.ws.p, p.ws.n - 1, nullptr) == GDN_ERROR_WORKSPACE);
  CHECK(g_stub.launches == n0);
  // o may not alias an input
  CHECK(gdn_chunk_fwd(&p.d, p.q.p, p.k.p, p.v.p, p.la.as<float>(), p.b.as<float>(), nullptr, p.cu.as<int32_t>(),
                      p.v.p, nullptr, p.ws.p, p.ws.n, nullptr) == GDN_ERROR_INVALID_VALUE);
  // a failed launch maps to GDN_ERROR_HIP
  g_stub.fail_launch = true;
  CHECK(p.run() == GDN_ERROR_HIP && msg_has("launch"));
  g_stub.fail_launch = false;
}

static void test_backward_and_decode_args() {
  gdn_dims_t d = dims(1, 70, 1, 3, 16, 16, GDN_DTYPE_F32);
  const size_t t = 70, e = 4;
  Buf q(t * 16 * e), k(t * 16 * e), v(t * 3 * 16 * e), la(t * 3 * 4), b(t * 3 * 4), dout(t * 3 * 16 * e);
  Buf dq(t * 16 * e), dk(t * 16 * e), dv(t * 3 * 16 * e), dla(t * 3 * 4), db(t * 3 * 4), dinit(3 * 16 * 16 * 4);
  Buf ws(gdn_chunk_bwd_workspace_bytes(&d));
  CHECK(ws.n > 0);
  const int before = g_stub.launches;
  CHECK(gdn_chunk_bwd(&d, q.p, k.p, v.p, la.as<float>(), b.as<float>(), nullptr, nullptr, dout.p, nullptr, dq.p,
                      dk.p, dv.p, dla.as<float>(), db.as<float>(), dinit.as<float>(), ws.p, ws.n, nullptr) ==
        GDN_SUCCESS);
  CHECK(g_stub.launches == before + 1 && g_stub.prefill.backward == 1);
  const gdn::PrefillArgs& a = g_stub.prefill;
  const void* regions[] = {a.chunk_table, a.tinv, a.w, a.key_t, a.k_frag, a.q_t, a.kq, a.pt, a.wt, a.tt,
                           a.sc, a.ub, a.dsl, a.du};
  for (const void* r : regions) CHECK(ws.holds(r, 1));
  // gradients must not alias inputs
  CHECK(gdn_chunk_bwd(&d, q.p, k.p, v.p, la.as<float>(), b.as<float>(), nullptr, nullptr, dout.p, nullptr, q.p,
                      dk.p, dv.p, dla.as<float>(), db.as<float>(), nullptr, ws.p, ws.n, nullptr) ==
        GDN_ERROR_INVALID_VALUE);

  gdn_dims_t dd = dims(4, 4, 2, 6, 128, 64, GDN_DTYPE_BF16);
  Buf sq(4 * 2 * 128 * 2), sk(4 * 2 * 128 * 2), sv(4 * 6 * 128 * 2), sla(4 * 6 * 4), sb(4 * 6 * 4);
  Buf st(4 * 6 * 128 * 128 * 4), so(4 * 6 * 128 * 2);
  const int n0 = g_stub.launches;
  CHECK(gdn_decode_step(&dd, sq.p, sk.p, sv.p, sla.as<float>(), sb.as<float>(), st.as<float>(), so.p, nullptr) ==
        GDN_SUCCESS);
  CHECK(g_stub.launches == n0 + 1 && g_stub.decode.num_seqs == 4 && g_stub.decode.state == st.p);
  dd.total_tokens = 5;
  CHECK(gdn_decode_step(&dd, sq.p, sk.p, sv.p, sla.as<float>(), sb.as<float>(), st.as<float>(), so.p, nullptr) ==
        GDN_ERROR_INVALID_VALUE);
  CHECK(g_stub.launches == n0 + 1);
}

static void test_debug_cu_seqlens() {
  const std::vector<int32_t> good = {0, 64, 64, 200};
  Prefill p(dims(3, 200, 1, 3, 16, 16, GDN_DTYPE_F32), good);
  unsetenv("GDN_DEBUG");
  // off: the table is not read
  int c0 = g_stub.copies;
  CHECK(p.run() == GDN_SUCCESS && g_stub.copies == c0);
  setenv("GDN_DEBUG", "1", 1);
  c0 = g_stub.copies;
  CHECK(p.run() == GDN_SUCCESS && g_stub.copies == c0 + 1);
  const std::vector<std::vector<int32_t>> bad = {{1, 64, 64, 200}, {0, 64, 63, 200}, {0, 64, 64, 199},
                                                 {0, 250, 64, 200}};
  for (const auto& t : bad) {
    Buf cu(t.size() * 4);
    memcpy(cu.p, t.data(), t.size() * 4);
    const int n0 = g_stub.launches;
    CHECK(p.run(cu.as<int32_t>()) == GDN_ERROR_INVALID_VALUE && msg_has("GDN_DEBUG"));
    CHECK(g_stub.launches == n0);          // nothing enqueued
  }
  // no table: nothing to check
  Prefill one(dims(1, 90, 1, 3, 16, 16, GDN_DTYPE_F32), {0, 90});
  c0 = g_stub.copies;
  CHECK(one.run(nullptr, false) == GDN_SUCCESS && g_stub.copies == c0);
  setenv("GDN_DEBUG", "0", 1);
  c0 = g_stub.copies;
  CHECK(p.run() == GDN_SUCCESS && g_stub.copies == c0);
  unsetenv("GDN_DEBUG");
}

static void test_debug_sync() {
  Prefill p(dims(1, 40, 1, 1, 16, 16, GDN_DTYPE_F32), {0, 40});
  unsetenv("GDN_DEBUG_SYNC");
  int s0 = g_stub.syncs;
  CHECK(p.run() == GDN_SUCCESS && g_stub.syncs == s0);
  setenv("GDN_DEBUG_SYNC", "1", 1);
  s0 = g_stub.syncs;
  CHECK(p.run() == GDN_SUCCESS && g_stub.syncs == s0 + 1);
  g_stub.fail_sync = true;
  CHECK(p.run() == GDN_ERROR_HIP && msg_has("GDN_DEBUG_SYNC") && msg_has("gdn_chunk_fwd"));
  g_stub.fail_sync = false;
  unsetenv("GDN_DEBUG_SYNC");
}

int main() {
  test_validation();
  test_prefill_args();
  test_backward_and_decode_args();
  test_debug_cu_seqlens();
  test_debug_sync();
  if (g_failed) {
    fprintf(stderr, "abi driver: %d of %d checks failed\n", g_failed, g_checks);
    return 1;
  }
  printf("abi driver: %d checks ok\n", g_checks);
  return 0;
}
