// C ABI of libidx.so: argument validation, workspace sizing and carve-up, dispatch of the
// gfx950 kernels.  No device memory is allocated here; the caller owns every buffer.
#include <cmath>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/idx.h"
#include "launch.hpp"

using namespace idx;

namespace {

constexpr int32_t kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr size_t kAlign = 256;

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Device facts cached per device (the ROCm top-k page caches the CU count the same way).
struct DevInfo {
  int checked = 0;  // 0 unknown, 1 ok, -1 not a gfx950
  int cu = 0;
};
DevInfo g_dev[64];
std::mutex g_mu;

int current_device(int* cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return IDX_ENODEV;
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& d = g_dev[dev];
  if (d.checked == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return IDX_ENODEV;
    d.checked = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    d.cu = prop.multiProcessorCount;
  }
  if (d.checked != 1) return IDX_ENODEV;
  if (cu) *cu = d.cu;
  return IDX_OK;
}

int check_problem(const idx_problem* p, DevProblem* out) {
  if (!p) return IDX_EINVAL;
  if (p->rows < 0 || p->head_dim != IDX_HEAD_DIM || (p->heads != 32 && p->heads != 64)) return IDX_EINVAL;
  if (p->fmt != IDX_FMT_E4M3 && p->fmt != IDX_FMT_MXFP4) return IDX_EINVAL;
  if (p->num_keys < 0) return IDX_EINVAL;
  const bool paged = p->page_table != nullptr;
  if (p->fmt == IDX_FMT_E4M3) {
    if (p->q_sf || p->k_sf) return IDX_EFMT;
  } else {
    if (!p->q_sf || !p->k_sf) return IDX_EFMT;
    if (paged) return IDX_EFMT;  // paged K is e4m3 with a per-token scale
  }
  if (p->rows > 0) {
    if (!p->q || !p->k || !p->w || !p->ks || !p->ke) return IDX_EINVAL;
    if (p->num_keys == 0) return IDX_EINVAL;  // the kernels clamp key reads into [0, num_keys)
  }
  if (paged) {
    if (!p->row_req || p->num_req <= 0 || p->max_pages <= 0 || (p->num_keys % IDX_PAGE) != 0) return IDX_EINVAL;
    if ((int64_t)p->max_pages * IDX_PAGE > INT32_MAX) return IDX_EINVAL;
  }
  if (p->num_keys > INT32_MAX) return IDX_EINVAL;
  if (!aligned(p->q, 16) || !aligned(p->k, 16)) return IDX_EALIGN;
  if (!aligned(p->q_sf, 4) || !aligned(p->k_sf, 4) || !aligned(p->k_scale, 4) || !aligned(p->w, 2) ||
      !aligned(p->ks, 4) || !aligned(p->ke, 4) || !aligned(p->page_table, 4) || !aligned(p->row_req, 4))
    return IDX_EALIGN;
  if (out) {
    out->rows = p->rows;
    out->heads = p->heads;
    out->fmt = p->fmt;
    out->q = static_cast<const uint8_t*>(p->q);
    out->q_sf = p->q_sf;
    out->k = static_cast<const uint8_t*>(p->k);
    out->k_sf = p->k_sf;
    out->k_scale = p->k_scale;
    out->w = p->w;
    out->ks = p->ks;
    out->ke = p->ke;
    out->num_keys = p->num_keys;
    out->page_table = p->page_table;
    out->row_req = p->row_req;
    out->num_req = p->num_req;
    out->max_pages = p->max_pages;
    out->key_span = paged ? (int64_t)p->max_pages * IDX_PAGE : p->num_keys;
  }
  return IDX_OK;
}

// Sizes of the fused path for a problem and k.
struct FusedSizes {
  int32_t cap, stride, ns, fb_blocks;
  int64_t key_span, scratch_ld;
  size_t off_thr, off_cnt, off_stats, off_fb, off_slab_s, off_slab_i, off_samp, off_scratch, off_lin, total;
};

FusedSizes fused_sizes(const idx_problem* p, int32_t k) {
  FusedSizes z = {};
  const bool paged = p->page_table != nullptr;
  z.key_span = paged ? (int64_t)p->max_pages * IDX_PAGE : p->num_keys;
  z.cap = 4 * k;
  if (p->debug && p->debug->cap > 0) z.cap = p->debug->cap;
  z.stride = sample_stride_for(k);
  z.ns = (int32_t)((z.key_span + z.stride - 1) / z.stride);
  if (z.ns < 1) z.ns = 1;
  z.fb_blocks = std::max(1, std::min(p->rows, kFbSlots));
  z.scratch_ld = (int64_t)round_up((size_t)std::max<int64_t>(z.key_span, 1), 64);
  const size_t rows = (size_t)std::max(p->rows, 1);
  size_t o = 0;
  z.off_thr = o;
  o = round_up(o + rows * 4, kAlign);
  z.off_cnt = o;
  o = round_up(o + rows * 4, kAlign);
  z.off_stats = o;
  o = round_up(o + kStatSlots * 8, kAlign);
  z.off_fb = o;
  o = round_up(o + kFbCtrlWords * 4 + rows * 4, kAlign);
  z.off_slab_s = o;
  o = round_up(o + rows * (size_t)z.cap * 4, kAlign);
  z.off_slab_i = o;
  o = round_up(o + rows * (size_t)z.cap * 4, kAlign);
  z.off_samp = o;
  o = round_up(o + rows * (size_t)z.ns * 4, kAlign);
  z.off_scratch = o;
  o = round_up(o + (size_t)z.fb_blocks * (size_t)z.scratch_ld * 4, kAlign);
  z.off_lin = o;
  o = round_up(o + lin_ws_bytes((int32_t)rows), kAlign);
  z.total = o;
  return z;
}

int hip_err(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_EHIP; }

// Stage timing record (idx_timing_*): 6 events per timed call.
constexpr int kStageEvents = 6;
struct Timing {
  bool on = false;
  int max_calls = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;
};
Timing g_timing;
std::mutex g_timing_mu;

// Events for the next timed call, or nullptr.
hipEvent_t* next_timing_slot() {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing.on || g_timing.used >= g_timing.max_calls) return nullptr;
  return &g_timing.ev[(size_t)(g_timing.used++) * kStageEvents];
}

int check_select(const float* scores, int64_t ld, const int32_t* len, int32_t rows, int32_t k, int32_t* out) {
  if (rows < 0 || k < 1 || k > IDX_MAX_TOPK || ld < 0 || ld > INT32_MAX) return IDX_EINVAL;
  if (rows > 0 && (!scores || !len || !out)) return IDX_EINVAL;
  if (!aligned(scores, 4) || !aligned(len, 4) || !aligned(out, 4)) return IDX_EALIGN;
  return IDX_OK;
}

}  // namespace

extern "C" {

int32_t idx_version(void) { return kVersion; }

const char* idx_strerror(int code) {
  switch (code) {
    case IDX_OK: return "success";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EFMT: return "operand format does not match the pointers given";
    case IDX_EALIGN: return "misaligned device pointer";
    case IDX_EWS: return "workspace too small";
    case IDX_EHIP: return "HIP runtime or kernel launch error";
    case IDX_ENODEV: return "no gfx950 device is current";
    case IDX_ESCRATCH: return "problem needs more workspace than the library's fixed scratch";
    default: return "unknown error";
  }
}

int32_t idx_row_split(int32_t rows, int64_t row_len, int32_t cu_count) {
  // ROCm top-k page, row_split: rows shorter than 65536 stay in one workgroup; otherwise
  // g = min(CUs / rows, 32) workgroups per row, unless that is fewer than 4.
  constexpr int64_t kMinRowLen = 65536;
  constexpr int32_t kMinSplit = 4, kMaxSplit = 32;
  if (row_len < kMinRowLen) return 0;
  const int32_t g = std::min<int32_t>(cu_count / std::max<int32_t>(rows, 1), kMaxSplit);
  return g < kMinSplit ? 0 : g;
}

size_t idx_select_workspace(int32_t rows, int64_t ld, int32_t k) {
  (void)ld;
  (void)k;
  if (rows <= 0) return 0;
  return select_split_ws_bytes(rows);
}

int idx_select_split(const float* scores, int64_t ld, const int32_t* row_start, const int32_t* len, int32_t rows,
                     int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes, int32_t split, void* stream) {
  int rc = check_select(scores, ld, len, rows, k, out_idx);
  if (rc) return rc;
  if (!aligned(row_start, 4)) return IDX_EALIGN;
  if (split < 0 || split == 1 || split > 32) return IDX_EINVAL;
  if (rows == 0) return IDX_OK;
  if ((rc = current_device(nullptr))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (split == 0) return hip_err(launch_select_single(scores, ld, row_start, len, rows, k, out_idx, s));
  if (!ws || ws_bytes < idx_select_workspace(rows, ld, k)) return IDX_EWS;
  if (!aligned(ws, kAlign)) return IDX_EALIGN;
  return hip_err(launch_select_split(scores, ld, row_start, len, rows, k, split, out_idx, ws, s));
}

int idx_select(const float* scores, int64_t ld, const int32_t* row_start, const int32_t* len, int32_t rows,
               int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_select(scores, ld, len, rows, k, out_idx);
  if (rc) return rc;
  if (rows == 0) return IDX_OK;
  int cu = 0;
  if ((rc = current_device(&cu))) return rc;
  int32_t g = idx_row_split(rows, ld, cu);
  if (g > 0 && (!ws || ws_bytes < idx_select_workspace(rows, ld, k))) g = 0;  // no workspace: one workgroup per row
  return idx_select_split(scores, ld, row_start, len, rows, k, out_idx, ws, ws_bytes, g, stream);
}

int idx_page_slots(const int32_t* idx, int32_t rows, int32_t k, const int32_t* ks, const int32_t* page_table,
                   const int32_t* row_req, int32_t max_pages, int32_t* out, void* stream) {
  if (rows < 0 || k < 1 || max_pages < 1) return IDX_EINVAL;
  if (rows == 0) return IDX_OK;
  if (!idx || !page_table || !row_req || !out) return IDX_EINVAL;
  if (!aligned(idx, 4) || !aligned(out, 4) || !aligned(page_table, 4) || !aligned(row_req, 4) ||
      (ks && !aligned(ks, 4)))
    return IDX_EALIGN;
  int rc = current_device(nullptr);
  if (rc) return rc;
  return hip_err(launch_page_slots(idx, rows, k, ks, page_table, row_req, max_pages, out,
                                   static_cast<hipStream_t>(stream)));
}

int idx_sparse_attn(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, int64_t num_slots,
                    const int32_t* slots, int32_t rows, int32_t hq, int32_t hkv, int32_t width, float softmax_scale,
                    float output_scale, float* out, void* stream) {
  if (rows < 0 || width < 0 || hkv < 1 || hq < 1 || hq % hkv != 0 || hq / hkv > 32 || num_slots < 1)
    return IDX_EINVAL;
  if ((int64_t)rows * hkv > 0x7FFFFFFF) return IDX_EINVAL;
  if (!std::isfinite(softmax_scale) || !std::isfinite(output_scale)) return IDX_EINVAL;
  if (rows == 0) return IDX_OK;
  if (!q || !k_cache || !v_cache || !out || (width > 0 && !slots)) return IDX_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      (slots && !aligned(slots, 4)))
    return IDX_EALIGN;
  int rc = current_device(nullptr);
  if (rc) return rc;
  return hip_err(launch_sparse_attn(q, k_cache, v_cache, num_slots, slots, rows, hq, hkv, width, softmax_scale,
                                    output_scale, out, static_cast<hipStream_t>(stream)));
}

size_t idx_score_workspace(const idx_problem* p) {
  if (check_problem(p, nullptr) != IDX_OK) return 0;
  if (p->rows == 0 || p->fmt != IDX_FMT_MXFP4) return 0;  // only the MXFP4 form keeps per-row pieces
  return lin_ws_bytes(p->rows);
}

int idx_score(const idx_problem* p, float* out, int64_t ld, void* ws, size_t ws_bytes, void* stream) {
  DevProblem P;
  int rc = check_problem(p, &P);
  if (rc) return rc;
  if (p->rows > 0 && !out) return IDX_EINVAL;
  if (ld < 0) return IDX_EINVAL;
  if (!aligned(out, 4)) return IDX_EALIGN;
  if (p->rows == 0) return IDX_OK;
  const size_t need = idx_score_workspace(p);
  if (need > 0 && (!ws || ws_bytes < need)) return IDX_EWS;
  if (need > 0 && !aligned(ws, kAlign)) return IDX_EALIGN;
  if ((rc = current_device(nullptr))) return rc;
  return hip_err(launch_score_store(P, out, ld, ws, static_cast<hipStream_t>(stream)));
}

size_t idx_fused_workspace(const idx_problem* p, int32_t k) {
  if (check_problem(p, nullptr) != IDX_OK || k < 1 || k > IDX_MAX_TOPK) return 0;
  return fused_sizes(p, k).total;
}

int idx_fused_topk(const idx_problem* p, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes, idx_stats* stats,
                   void* stream) {
  DevProblem P;
  int rc = check_problem(p, &P);
  if (rc) return rc;
  if (k < 1 || k > IDX_MAX_TOPK) return IDX_EINVAL;
  if (p->rows > 0 && !out_idx) return IDX_EINVAL;
  if (!aligned(out_idx, 4)) return IDX_EALIGN;
  if (p->debug && (p->debug->threshold_mode < 0 || p->debug->threshold_mode > 2 || p->debug->cap < 0 ||
                   p->debug->tie_cap < 0 || p->debug->tie_cap > kTieCapHost))
    return IDX_EINVAL;
  const FusedSizes z = fused_sizes(p, k);
  if (stats) {
    std::memset(stats, 0, sizeof(*stats));
    stats->rows = p->rows;
    stats->cap = z.cap;
    stats->sample_stride = z.stride;
    stats->sample_keys = z.ns;
  }
  if (p->rows == 0) return IDX_OK;
  if (!ws || ws_bytes < z.total) return IDX_EWS;
  if (!aligned(ws, kAlign)) return IDX_EALIGN;
  int cu = 0;
  if ((rc = current_device(&cu))) return rc;
  char* base = static_cast<char*>(ws);
  FusedPlan F;
  F.k = k;
  F.cu = cu;
  F.cap = z.cap;
  F.stride = z.stride;
  F.ns = z.ns;
  F.fb_blocks = z.fb_blocks;
  F.debug_mode = p->debug ? p->debug->threshold_mode : 0;
  F.debug_row_mod = p->debug ? p->debug->threshold_row_mod : 0;
  F.tie_cap = p->debug && p->debug->tie_cap > 0 ? p->debug->tie_cap : kTieCapHost;
  F.scratch_ld = z.scratch_ld;
  F.thr = reinterpret_cast<float*>(base + z.off_thr);
  F.cnt = reinterpret_cast<int32_t*>(base + z.off_cnt);
  F.stats = reinterpret_cast<long long*>(base + z.off_stats);
  F.want_stats = stats != nullptr;
  F.fb_ctrl = reinterpret_cast<int32_t*>(base + z.off_fb);
  F.fb_list = F.fb_ctrl + kFbCtrlWords;
  F.slab_s = reinterpret_cast<float*>(base + z.off_slab_s);
  F.slab_i = reinterpret_cast<int32_t*>(base + z.off_slab_i);
  F.samp = reinterpret_cast<float*>(base + z.off_samp);
  F.scratch = reinterpret_cast<float*>(base + z.off_scratch);
  F.lin_q8 = F.lin_sf = nullptr;
  lin_carve(base + z.off_lin, p->rows, &F.lin_q8, &F.lin_sf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((rc = hip_err(launch_fused(P, F, out_idx, s, next_timing_slot())))) return rc;
  if (stats) {
    long long h[kStatSlots];
    if (hipMemcpyAsync(h, F.stats, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess) return IDX_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return IDX_EHIP;
    stats->rows_store_all = (int32_t)h[kStatStoreAll];
    stats->rows_sampled = (int32_t)h[kStatSampled];
    stats->fallback_rows = (int32_t)h[kStatFallback];
    stats->max_count = (int32_t)h[kStatMax];
    stats->min_count = h[kStatSampled] > 0 ? (int32_t)h[kStatMin] : 0;
    stats->total_count = h[kStatTotal];
  }
  return IDX_OK;
}

int idx_timing_disable(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing = Timing();
  return IDX_OK;
}

int idx_timing_enable(int32_t max_calls) {
  if (max_calls < 1 || max_calls > (1 << 20)) return IDX_EINVAL;
  idx_timing_disable();
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing.ev.resize((size_t)max_calls * kStageEvents, nullptr);
  for (auto& e : g_timing.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      return IDX_EHIP;
    }
  }
  g_timing.max_calls = max_calls;
  g_timing.used = 0;
  g_timing.on = true;
  return IDX_OK;
}

int idx_timing_read(float* ms, int32_t max_calls) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing.on) return IDX_EINVAL;
  if (!ms || max_calls < 0) return IDX_EINVAL;
  const int n = std::min(g_timing.used, max_calls);
  for (int c = 0; c < n; ++c) {
    hipEvent_t* e = &g_timing.ev[(size_t)c * kStageEvents];
    if (hipEventSynchronize(e[kStageEvents - 1]) != hipSuccess) return IDX_EHIP;
    for (int i = 0; i + 1 < kStageEvents; ++i)
      if (hipEventElapsedTime(&ms[c * (kStageEvents - 1) + i], e[i], e[i + 1]) != hipSuccess) return IDX_EHIP;
  }
  g_timing.used = 0;
  return n;
}

}  // extern "C"
