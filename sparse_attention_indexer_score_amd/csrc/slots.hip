// Selected logical positions -> physical KV slots of a paged cache (idx_page_slots).
//
// LiteTopK page, section 3 (topk_page_table_transform): with 64-token pages, position pos
// of request q lives in slot page_table[q][pos / 64] * 64 + pos % 64; -1 entries pass
// through.  A flat 1-D grid over rows * k (no grid.y limit on the row count), four entries
// per thread with 16-byte loads and stores when the layout allows it.
#include "common.hpp"
#include "launch.hpp"

namespace idx {

struct SlotArgs {
  const int32_t* idx;
  const int32_t* ks;
  const int32_t* page_table;
  const int32_t* row_req;
  int32_t* out;
  int64_t total;  // rows * k
  int32_t k, max_pages;
};

__device__ __forceinline__ int32_t slot_of(const SlotArgs& A, int64_t e, int32_t v) {
  if (v < 0) return -1;
  const int r = (int)(e / A.k);
  const int64_t pos = (int64_t)(A.ks ? A.ks[r] : 0) + v;
  const int64_t page = pos >> 6;
  if (page >= A.max_pages) return -1;
  const int32_t q = A.row_req[r];
  return A.page_table[(int64_t)q * A.max_pages + page] * kPage + (int32_t)(pos & (kPage - 1));
}

__global__ __launch_bounds__(256) void page_slots_vec_kernel(SlotArgs A) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 entries
  const int64_t e = 4 * g;
  if (e >= A.total) return;
  const int4 v = *reinterpret_cast<const int4*>(A.idx + e);
  int4 o;
  o.x = slot_of(A, e, v.x);
  o.y = slot_of(A, e + 1, v.y);
  o.z = slot_of(A, e + 2, v.z);
  o.w = slot_of(A, e + 3, v.w);
  *reinterpret_cast<int4*>(A.out + e) = o;
}

__global__ __launch_bounds__(256) void page_slots_kernel(SlotArgs A) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= A.total) return;
  A.out[e] = slot_of(A, e, A.idx[e]);
}

hipError_t launch_page_slots(const int32_t* idx, int32_t rows, int32_t k, const int32_t* ks,
                             const int32_t* page_table, const int32_t* row_req, int32_t max_pages, int32_t* out,
                             hipStream_t s) {
  SlotArgs A{idx, ks, page_table, row_req, out, (int64_t)rows * k, k, max_pages};
  if (A.total == 0) return hipSuccess;
  const bool vec = (k % 4 == 0) && ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  const int64_t items = vec ? A.total / 4 : A.total;
  const dim3 grid((unsigned)((items + 255) / 256)), block(256);
  if (vec) page_slots_vec_kernel<<<grid, block, 0, s>>>(A);
  else page_slots_kernel<<<grid, block, 0, s>>>(A);
  return hipGetLastError();
}

}  // namespace idx
