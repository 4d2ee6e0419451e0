// Host-side launchers of the gfx950 kernels (defined next to the kernels they launch).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idx {

// Raw problem description (device pointers), validated by the C ABI layer.
struct DevProblem {
  int32_t rows, heads, fmt;
  const uint8_t* q;
  const uint8_t* q_sf;
  const uint8_t* k;
  const uint8_t* k_sf;
  const float* k_scale;
  const uint16_t* w;
  const int32_t* ks;
  const int32_t* ke;
  int64_t num_keys;
  const int32_t* page_table;
  const int32_t* row_req;
  int32_t num_req, max_pages;
  int64_t key_span;  // logical key space: num_keys (contiguous) or max_pages * 64 (paged)
};

// Exact fallback: scratch rows (queued rows re-scored at once) and the control words ahead
// of the queued-row list: [0] queued count, [1] head of the rows past the scratch rows,
// [2, 2 + kFbSlots) chunks scored so far of each scratch row's row; then the ticket counter
// of the paged score + filter kernel's persistent workgroups.
constexpr int kFbSlots = 32;
constexpr int kFbCtrlWords = 2 + kFbSlots + 1;
constexpr int kPagedTicketWord = 2 + kFbSlots;

// Per-call plan of the fused path (sizes and workspace carve-up).
struct FusedPlan {
  int32_t k, cap, stride, ns, fb_blocks;
  int32_t cu;  // compute units of the device
  int32_t debug_mode, debug_row_mod;
  int32_t tie_cap;  // tie-buffer capacity of the slab select and the fallback (<= kTieCap)
  int64_t scratch_ld;
  // workspace regions
  float* thr;
  int32_t* cnt;
  long long* stats;  // kStatSlots
  int32_t want_stats;  // update the route counters (only when the caller asks for them)
  int32_t* fb_ctrl;  // kFbCtrlWords control words
  int32_t* fb_list;
  float* slab_s;
  int32_t* slab_i;
  float* samp;
  float* scratch;
  uint8_t* lin_q8;  // pieces of sum_h w_h q_h (contiguous keys)
  uint8_t* lin_sf;
};

// Tie-buffer capacity of the selection (host copy of the device constant kTieCap).
constexpr int kTieCapHost = 4096;

enum StatSlot { kStatStoreAll = 0, kStatSampled, kStatFallback, kStatMax, kStatMin, kStatTotal, kStatSlots = 8 };

// ws: lin_ws_bytes(rows) bytes (contiguous keys; unused when paged).
hipError_t launch_score_store(const DevProblem& P, float* out, int64_t ld, void* ws, hipStream_t s);
size_t lin_ws_bytes(int32_t rows);
void lin_carve(void* ws, int32_t rows, uint8_t** q8, uint8_t** sf);
// ev: optional 6 events recorded at the stage boundaries (before K1a .. after K4).
hipError_t launch_fused(const DevProblem& P, const FusedPlan& F, int32_t* out_idx, hipStream_t s,
                        hipEvent_t* ev = nullptr);

hipError_t launch_page_slots(const int32_t* idx, int32_t rows, int32_t k, const int32_t* ks,
                             const int32_t* page_table, const int32_t* row_req, int32_t max_pages, int32_t* out,
                             hipStream_t s);
hipError_t launch_select_single(const float* x, int64_t ld, const int32_t* row_start, const int32_t* len,
                                int32_t rows, int32_t k, int32_t* out, hipStream_t s);
hipError_t launch_select_split(const float* x, int64_t ld, const int32_t* row_start, const int32_t* len,
                               int32_t rows, int32_t k, int32_t g, int32_t* out, void* ws, hipStream_t s);
size_t select_split_ws_bytes(int32_t rows);
hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* k, const uint8_t* v, int64_t num_slots,
                              const int32_t* slots, int32_t rows, int32_t hq, int32_t hkv, int32_t width,
                              float softmax_scale, float output_scale, float* out, hipStream_t s);

// Score-kernel work decomposition shared with the host sizing code.
int rows_per_block(int heads, int fmt);
int sample_stride_for(int k);  // odd stride S

}  // namespace idx
