// Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code (tests/test_sanitize_cpu.py links it with an instrumented capi.cpp and the
// uninstrumented kernels).  Every call here returns before any device work: argument
// validation, workspace sizing, the row-split rule, error strings and the timing hooks.
// Device pointers are fake, aligned or misaligned addresses that the library never
// dereferences on the host.  Prints one line per failed check and exits non-zero on any.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "idx.h"

static int g_fail = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static idx_problem problem(int32_t rows, int32_t heads, int32_t fmt, int64_t num_keys) {
  idx_problem p;
  std::memset(&p, 0, sizeof(p));
  p.rows = rows;
  p.heads = heads;
  p.head_dim = IDX_HEAD_DIM;
  p.fmt = fmt;
  p.q = p.k = fake(0x10000);
  p.w = static_cast<const uint16_t*>(fake(0x20000));
  p.ks = p.ke = static_cast<const int32_t*>(fake(0x30000));
  p.num_keys = num_keys;
  if (fmt == IDX_FMT_MXFP4) p.q_sf = p.k_sf = static_cast<const uint8_t*>(fake(0x40000));
  return p;
}

static void strings_and_rules() {
  for (int c = 1; c >= -8; --c) CHECK(idx_strerror(c) != nullptr && std::strlen(idx_strerror(c)) > 0);
  CHECK(std::strcmp(idx_strerror(IDX_ESCRATCH), idx_strerror(IDX_EWS)) != 0);
  CHECK(idx_version() > 0);
  CHECK(idx_row_split(64, 131072, 256) == 4);
  CHECK(idx_row_split(4096, 65536, 256) == 0);
  CHECK(idx_row_split(8, 65535, 256) == 0);
  CHECK(idx_row_split(8, 65536, 256) == 32);
  CHECK(idx_row_split(0, 1 << 20, 256) == 32);
  CHECK(idx_row_split(1, INT64_MAX, 0) == 0);
}

static void selection() {
  const float* x = static_cast<const float*>(fake(0x10000));
  const int32_t* n = static_cast<const int32_t*>(fake(0x20000));
  int32_t* o = static_cast<int32_t*>(fake(0x30000));
  CHECK(idx_select(x, 1024, nullptr, n, 4, 0, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(x, 1024, nullptr, n, 4, IDX_MAX_TOPK + 1, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(x, 1024, nullptr, n, -1, 16, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(x, -5, nullptr, n, 4, 16, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(x, (int64_t)1 << 40, nullptr, n, 4, 16, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(nullptr, 1024, nullptr, n, 4, 16, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(x, 1024, nullptr, nullptr, 4, 16, o, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(x, 1024, nullptr, n, 4, 16, nullptr, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_select(static_cast<const float*>(fake(0x10002)), 1024, nullptr, n, 4, 16, o, nullptr, 0, nullptr) ==
        IDX_EALIGN);
  CHECK(idx_select(x, 1024, nullptr, n, 0, 16, o, nullptr, 0, nullptr) == IDX_OK);
  CHECK(idx_select_split(x, 1024, nullptr, n, 4, 16, o, nullptr, 0, 1, nullptr) == IDX_EINVAL);
  CHECK(idx_select_split(x, 1024, nullptr, n, 4, 16, o, nullptr, 0, 33, nullptr) == IDX_EINVAL);
  CHECK(idx_select_split(x, 1024, nullptr, n, 4, 16, o, nullptr, 0, -1, nullptr) == IDX_EINVAL);
  CHECK(idx_select_split(x, 1024, static_cast<const int32_t*>(fake(0x20001)), n, 4, 16, o, nullptr, 0, 0,
                         nullptr) == IDX_EALIGN);
  CHECK(idx_select_workspace(0, 1024, 16) == 0);
  CHECK(idx_select_workspace(64, 131072, 2048) > (size_t)64 * 4096 * 4);
  CHECK(idx_select_workspace(1 << 20, 1 << 20, 2048) > ((size_t)1 << 20) * 4096 * 4);
}

static void scoring() {
  float* out = static_cast<float*>(fake(0x50000));
  void* ws = fake(0x100000);
  idx_problem p = problem(64, 32, IDX_FMT_E4M3, 4096);
  CHECK(idx_score_workspace(&p) == 0);
  idx_problem bad = p;
  bad.heads = 48;
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_score_workspace(&bad) == 0);
  bad = p;
  bad.head_dim = 64;
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  bad = p;
  bad.fmt = 3;
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  bad = p;
  bad.q_sf = static_cast<const uint8_t*>(fake(0x40000));
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EFMT);
  bad = p;
  bad.q = fake(0x10008);
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EALIGN);
  bad = p;
  bad.num_keys = 0;
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  bad = p;
  bad.num_keys = (int64_t)1 << 40;
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  bad = p;
  bad.page_table = static_cast<const int32_t*>(fake(0x60000));  // paged without row_req
  CHECK(idx_score(&bad, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_score(&p, out, -1, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_score(&p, nullptr, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  CHECK(idx_score(nullptr, out, 4096, nullptr, 0, nullptr) == IDX_EINVAL);
  idx_problem m = problem(64, 32, IDX_FMT_MXFP4, 4096);
  const size_t need = idx_score_workspace(&m);
  CHECK(need > 0);
  CHECK(idx_score(&m, out, 4096, nullptr, 0, nullptr) == IDX_EWS);
  CHECK(idx_score(&m, out, 4096, ws, need - 1, nullptr) == IDX_EWS);
  CHECK(idx_score(&m, out, 4096, fake(0x100080), need, nullptr) == IDX_EALIGN);
  bad = m;
  bad.k_sf = nullptr;
  CHECK(idx_score(&bad, out, 4096, ws, need, nullptr) == IDX_EFMT);
  idx_problem z = problem(0, 32, IDX_FMT_E4M3, 0);
  CHECK(idx_score(&z, nullptr, 0, nullptr, 0, nullptr) == IDX_OK);
}

static void fused() {
  int32_t* out = static_cast<int32_t*>(fake(0x50000));
  idx_problem p = problem(4096, 64, IDX_FMT_E4M3, 65536);
  const size_t a = idx_fused_workspace(&p, 512), b = idx_fused_workspace(&p, 2048);
  CHECK(a > 0 && a < b);
  CHECK(idx_fused_workspace(&p, 0) == 0);
  CHECK(idx_fused_workspace(&p, IDX_MAX_TOPK + 1) == 0);
  idx_problem huge = problem(INT32_MAX, 64, IDX_FMT_E4M3, INT32_MAX);
  CHECK(idx_fused_workspace(&huge, 2048) > ((size_t)INT32_MAX) * 8192 * 8);
  CHECK(idx_fused_topk(&p, 0, out, fake(0x100000), b, nullptr, nullptr) == IDX_EINVAL);
  CHECK(idx_fused_topk(&p, 2048, nullptr, fake(0x100000), b, nullptr, nullptr) == IDX_EINVAL);
  CHECK(idx_fused_topk(&p, 2048, out, nullptr, 0, nullptr, nullptr) == IDX_EWS);
  CHECK(idx_fused_topk(&p, 2048, out, fake(0x100000), b - 1, nullptr, nullptr) == IDX_EWS);
  CHECK(idx_fused_topk(&p, 2048, out, fake(0x100010), b, nullptr, nullptr) == IDX_EALIGN);
  CHECK(idx_fused_topk(&p, 2048, static_cast<int32_t*>(fake(0x50002)), fake(0x100000), b, nullptr, nullptr) ==
        IDX_EALIGN);
  idx_debug dbg;
  std::memset(&dbg, 0, sizeof(dbg));
  idx_problem d = p;
  d.debug = &dbg;
  dbg.threshold_mode = 3;
  CHECK(idx_fused_topk(&d, 2048, out, fake(0x100000), b, nullptr, nullptr) == IDX_EINVAL);
  dbg.threshold_mode = 0;
  dbg.cap = -1;
  CHECK(idx_fused_topk(&d, 2048, out, fake(0x100000), b, nullptr, nullptr) == IDX_EINVAL);
  dbg.cap = 0;
  dbg.tie_cap = 4097;
  CHECK(idx_fused_topk(&d, 2048, out, fake(0x100000), b, nullptr, nullptr) == IDX_EINVAL);
  dbg.tie_cap = -1;
  CHECK(idx_fused_topk(&d, 2048, out, fake(0x100000), b, nullptr, nullptr) == IDX_EINVAL);
  dbg.tie_cap = 0;
  dbg.cap = 16;
  CHECK(idx_fused_workspace(&d, 2048) < b);
  // zero rows: nothing enqueued, statistics filled
  idx_problem z = problem(0, 32, IDX_FMT_MXFP4, 0);
  idx_stats st;
  std::memset(&st, 0x7F, sizeof(st));
  CHECK(idx_fused_topk(&z, 2048, nullptr, nullptr, 0, &st, nullptr) == IDX_OK);
  CHECK(st.rows == 0 && st.cap == 8192 && st.sample_stride == 71 && st.fallback_rows == 0);
  // no-allocation entry: validation and the scratch limit, before any device work
  CHECK(idx_fused_topk_noalloc(&p, 0, out, nullptr) == IDX_EINVAL);
  CHECK(idx_fused_topk_noalloc(&p, 2048, out, nullptr) == IDX_ESCRATCH);
  CHECK(idx_fused_topk_noalloc(nullptr, 2048, out, nullptr) == IDX_EINVAL);
}

static void other_entries() {
  const int32_t* a = static_cast<const int32_t*>(fake(0x10000));
  int32_t* o = static_cast<int32_t*>(fake(0x20000));
  CHECK(idx_page_slots(a, -1, 4, nullptr, a, a, 2, o, nullptr) == IDX_EINVAL);
  CHECK(idx_page_slots(a, 2, 0, nullptr, a, a, 2, o, nullptr) == IDX_EINVAL);
  CHECK(idx_page_slots(a, 2, 4, nullptr, a, a, 0, o, nullptr) == IDX_EINVAL);
  CHECK(idx_page_slots(nullptr, 2, 4, nullptr, a, a, 2, o, nullptr) == IDX_EINVAL);
  CHECK(idx_page_slots(static_cast<const int32_t*>(fake(0x10002)), 2, 4, nullptr, a, a, 2, o, nullptr) ==
        IDX_EALIGN);
  CHECK(idx_page_slots(nullptr, 0, 4, nullptr, nullptr, nullptr, 2, nullptr, nullptr) == IDX_OK);
  const uint16_t* q = static_cast<const uint16_t*>(fake(0x10000));
  const uint8_t* kc = static_cast<const uint8_t*>(fake(0x20000));
  float* out = static_cast<float*>(fake(0x30000));
  CHECK(idx_sparse_attn(q, kc, kc, 100, a, -1, 24, 2, 8, 0.1f, 1.0f, out, nullptr) == IDX_EINVAL);
  CHECK(idx_sparse_attn(q, kc, kc, 100, a, 2, 25, 2, 8, 0.1f, 1.0f, out, nullptr) == IDX_EINVAL);
  CHECK(idx_sparse_attn(q, kc, kc, 100, a, 2, 66, 2, 8, 0.1f, 1.0f, out, nullptr) == IDX_EINVAL);
  CHECK(idx_sparse_attn(q, kc, kc, 0, a, 2, 24, 2, 8, 0.1f, 1.0f, out, nullptr) == IDX_EINVAL);
  CHECK(idx_sparse_attn(q, kc, kc, 100, nullptr, 2, 24, 2, 8, 0.1f, 1.0f, out, nullptr) == IDX_EINVAL);
  CHECK(idx_sparse_attn(q, kc, kc, 100, a, 2, 24, 2, 8, 1.0f / 0.0f, 1.0f, out, nullptr) == IDX_EINVAL);
  CHECK(idx_sparse_attn(static_cast<const uint16_t*>(fake(0x10008)), kc, kc, 100, a, 2, 24, 2, 8, 0.1f, 1.0f, out,
                        nullptr) == IDX_EALIGN);
  CHECK(idx_sparse_attn(nullptr, nullptr, nullptr, 100, nullptr, 0, 24, 2, 8, 0.1f, 1.0f, nullptr, nullptr) ==
        IDX_OK);
  // timing hooks: range checks; enabling creates events (may fail without a device)
  CHECK(idx_timing_enable(0) == IDX_EINVAL);
  CHECK(idx_timing_enable((1 << 20) + 1) == IDX_EINVAL);
  float ms[5];
  CHECK(idx_timing_read(ms, 1) == IDX_EINVAL);  // not enabled
  const int rc = idx_timing_enable(2);
  CHECK(rc == IDX_OK || rc == IDX_EHIP);
  if (rc == IDX_OK) CHECK(idx_timing_read(nullptr, 1) == IDX_EINVAL);
  CHECK(idx_timing_disable() == IDX_OK);
}

int main() {
  strings_and_rules();
  selection();
  scoring();
  fused();
  other_entries();
  std::printf("%s: %d failed checks\n", g_fail ? "FAIL" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
