// Exact top-k over materialised fp32 rows (idx_select), gfx950.
//
// ROCm DSA indexer top-k page (sgl-project/sglang#37591): fp32 radix histogram of 12
// bits, exact tie refinement, full-row rescan when the tie buffer overflows, and, for
// long rows at low batch, several workgroups per row ("row split"):
//   split == 0  select_rows_kernel: one 1024-thread workgroup per row (a sampled threshold,
//               one pass into an LDS candidate buffer, radix refinement in LDS; the
//               multi-pass block_select when the sample misjudges the row)
//   split >= 2  seg_collect_kernel g workgroups per row each take the row's sample and
//                                  threshold T (the same in all of them), stream their
//                                  segment of the row and append its candidates (order
//                                  key >= T) to the row's buffer in the workspace
//               seg_merge_kernel   one workgroup per row refines the row's candidates in
//                                  LDS, or selects the whole row with the multi-pass
//                                  block_select when a segment overflowed or the
//                                  candidates are fewer than m
#include "launch.hpp"
#include "select_core.hpp"

namespace idx {

constexpr int kSelThreads = 1024;

// Candidate buffer of the single-workgroup path: 6144 (key, index) pairs, 64 KB of LDS with
// the histogram; with at most 64 VGPRs (8 waves per SIMD) two 1024-thread workgroups fit on
// a CU.
constexpr int kSelCand = 6144;

// Row r's elements: n = len[r] values from offset row_start[r] of the row, clamped into
// [0, ld) whatever the device-side values are, so that reads stay inside the row and the
// padding writes inside out[r][0, k); m = min(k, n).  Returns the element offset of the
// row's first value.
__device__ __forceinline__ int64_t row_span(int64_t ld, const int32_t* row_start, const int32_t* len, int r, int k,
                                            int& n, int& m) {
  int64_t rs = row_start ? row_start[r] : 0;
  rs = rs < 0 ? 0 : (rs > ld ? ld : rs);
  int64_t nn = len[r];
  nn = nn < 0 ? 0 : (nn > ld - rs ? ld - rs : nn);
  n = (int)nn;
  m = min(k, n);
  return (int64_t)r * ld + rs;
}

template <bool LONG>
__global__ __launch_bounds__(kSelThreads, 8) void select_rows_kernel(const float* x, int64_t ld,
                                                                  const int32_t* row_start, const int32_t* len,
                                                                  int32_t k, int32_t* out) {
  __shared__ SelSmemT<kSelCand> sm;
  const int r = blockIdx.x;
  int n, m;
  const int64_t off = row_span(ld, row_start, len, r, k, n, m);
  int32_t* o = out + (int64_t)r * k;
  if (m >= n) {
    for (int j = threadIdx.x; j < n; j += kSelThreads) o[j] = j;
  } else if (m > 0) {
    const float* xr = x + off;
    constexpr int SAMP = LONG ? kSelSamplesLong : kSelSamples, SEG = LONG ? 8 : 64;
    if ((reinterpret_cast<uintptr_t>(xr) & 15) == 0 && n >= 4)  // workgroup-uniform
      block_select_sampled<kSelThreads, true, SelSmemT<kSelCand>, SAMP, SEG>(xr, n, m, o, sm);
    else
      block_select_sampled<kSelThreads, false, SelSmemT<kSelCand>, SAMP, SEG>(xr, n, m, o, sm);
  }
  for (int j = m + threadIdx.x; j < k; j += kSelThreads) o[j] = -1;
}

// Row split workspace, per row r: a buffer of kSelCand candidates (order key, row index),
// the position counter its segments reserve space with (left at 0 by every call), the
// row's threshold T, and one slot per segment (candidates written, largest key, whether
// all of them were written).  Every row with m < n is split, whatever its length: a row no
// longer than the candidate buffer is not sampled (T = 0) and all of its elements are
// candidates.
constexpr int kSplitMax = 32;

struct SegWs {
  uint32_t* ckey;   // [rows][kSelCand]
  int32_t* cidx;    // [rows][kSelCand]
  int32_t* ctr;     // [rows]
  uint32_t* thr;    // [rows]
  int32_t* slot;    // [rows][kSplitMax][3]
};

static SegWs carve(void* ws, int rows) {
  SegWs W;
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* q = p;
    p += (bytes + 255) & ~(size_t)255;
    return q;
  };
  W.ckey = reinterpret_cast<uint32_t*>(take((size_t)rows * kSelCand * 4));
  W.cidx = reinterpret_cast<int32_t*>(take((size_t)rows * kSelCand * 4));
  W.ctr = reinterpret_cast<int32_t*>(take((size_t)rows * 4));
  W.thr = reinterpret_cast<uint32_t*>(take((size_t)rows * 4));
  W.slot = reinterpret_cast<int32_t*>(take((size_t)rows * kSplitMax * 3 * 4));
  return W;
}

size_t select_split_ws_bytes(int32_t rows) {
  auto r256 = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return 2 * r256((size_t)rows * kSelCand * 4) + 2 * r256((size_t)rows * 4) + r256((size_t)rows * kSplitMax * 12);
}

// Segment `part` of g of a row of n elements: a multiple of 4 elements long, so that the
// segments of a 16-byte aligned row start 16-byte aligned.
__device__ __forceinline__ void segment(int n, int g, int part, int& lo, int& hi) {
  const int seg = ((n + g - 1) / g + 3) & ~3;
  lo = (int)min((int64_t)n, (int64_t)part * seg);
  hi = min(n, lo + seg);
}

// Workgroup b runs on XCD b % 8 (workgroups are dealt to the XCDs round-robin): row r's g
// segments are workgroups 8 (g (r / 8) + part) + r % 8, all on XCD r % 8, so that the
// row's sample, which every segment reads, is fetched into one L2 once.  Grid: 8 g
// ceil(rows / 8).
__global__ __launch_bounds__(kSelThreads, 8) void seg_collect_kernel(const float* x, int64_t ld,
                                                                    const int32_t* row_start, const int32_t* len,
                                                                    int32_t rows, int32_t k, int32_t g, SegWs W) {
  using SM = SelSmemT<kSelCand>;
  __shared__ SM sm;
  __shared__ int sh_pos;
  const int local = (int)(blockIdx.x >> 3), part = local % g;
  const int r = (local / g) * 8 + (int)(blockIdx.x & 7);
  if (r >= rows) return;
  int n, m;
  const int64_t off = row_span(ld, row_start, len, r, k, n, m);
  if (m >= n) return;  // the merge kernel writes such rows whole
  int lo, hi;
  segment(n, g, part, lo, hi);
  const float* xr = x + off;
  // The sample of long rows (6144 keys in runs of 8) for every row length: a run-structured
  // top band moves a sample of 32 runs of 64 too far from row to row, and each segment here
  // streams only its own part of the row, so the sample's scattered lines cost the row one
  // read (shared through L2 by its segments) rather than lines its own pass reads anyway.
  constexpr int SAMP = kSelSamplesLong, SEG = 8;
  uint32_t T;
  if ((reinterpret_cast<uintptr_t>(xr + lo) & 15) == 0 && hi - lo >= 4)  // workgroup-uniform
    T = sampled_collect<kSelThreads, true, SM, SAMP, SEG, 4>(xr, n, m, lo, hi - lo, sm);
  else
    T = sampled_collect<kSelThreads, false, SM, SAMP, SEG, 4>(xr, n, m, lo, hi - lo, sm);
  const int c = sm.ntie;
  const int cs = min(c, SM::kCap);
  if (threadIdx.x == 0) sh_pos = cs > 0 ? atomicAdd(&W.ctr[r], cs) : 0;
  __syncthreads();
  const int pos = sh_pos;
  // (the counter may hold anything on a workspace's first use: a place outside the buffer
  // only sends the row to the exact path)
  const bool ok = c <= SM::kCap && pos >= 0 && (int64_t)pos + cs <= SM::kCap;
  if (ok) {
    uint32_t* ck = W.ckey + (int64_t)r * kSelCand + pos;
    int32_t* ci = W.cidx + (int64_t)r * kSelCand + pos;
    for (int t = threadIdx.x; t < cs; t += kSelThreads) {
      ck[t] = sm.tkey[t];
      ci[t] = sm.tidx[t];
    }
  }
  if (threadIdx.x == 0) {
    int32_t* sl = W.slot + ((int64_t)r * kSplitMax + part) * 3;
    sl[0] = cs;
    sl[1] = (int32_t)sm.kmax;
    sl[2] = ok ? 1 : 0;
    if (part == 0) W.thr[r] = T;
  }
}

__global__ __launch_bounds__(kSelThreads) void seg_merge_kernel(const float* x, int64_t ld,
                                                                  const int32_t* row_start, const int32_t* len,
                                                                  int32_t k, int32_t g, int32_t* out, SegWs W) {
  using SM = SelSmemT<kSelCand>;
  __shared__ SM sm;
  __shared__ int sh_total, sh_ok;
  __shared__ uint32_t sh_kmax;
  const int r = blockIdx.x;
  int n, m;
  const int64_t off = row_span(ld, row_start, len, r, k, n, m);
  int32_t* o = out + (int64_t)r * k;
  const float* xr = x + off;
  if (m >= n) {
    for (int j = threadIdx.x; j < n; j += kSelThreads) o[j] = j;
  } else {
    if (threadIdx.x == 0) {
      int total = 0, okall = 1;
      uint32_t kmax = 0u;
      for (int p = 0; p < g; ++p) {
        const int32_t* sl = W.slot + ((int64_t)r * kSplitMax + p) * 3;
        total += sl[0];
        kmax = max(kmax, (uint32_t)sl[1]);
        okall &= sl[2];
      }
      const int X = W.ctr[r] - total;  // start of the row's candidates in its buffer
      sh_ok = okall && X >= 0 && total >= m && (int64_t)X + total <= SM::kCap ? X : -1;
      sh_total = total;
      sh_kmax = kmax;
      sm.ntie = total;
      sm.nout = 0;
    }
    zero_hist<kSelThreads>(sm, kHistBins);
    __syncthreads();
    const int X = sh_ok, total = sh_total;
    if (X >= 0) {
      const uint32_t* ck = W.ckey + (int64_t)r * kSelCand + X;
      const int32_t* ci = W.cidx + (int64_t)r * kSelCand + X;
      for (int t = threadIdx.x; t < total; t += kSelThreads) {
        sm.tkey[t] = ck[t];
        sm.tidx[t] = ci[t];
      }
      __syncthreads();
      const KeyNorm nz = key_norm(W.thr[r], sh_kmax);
      refine_lds<kSelThreads>(1, (uint32_t)m, o, sm, &nz, true);  // keys normalised over [T, max]
    } else {
      block_select<kSelThreads>(RowSrc{xr}, n, m, o, sm);
    }
    if (threadIdx.x == 0) W.ctr[r] = 0;  // the next call's segments reserve from 0
  }
  for (int j = m + threadIdx.x; j < k; j += kSelThreads) o[j] = -1;
}

hipError_t launch_select_single(const float* x, int64_t ld, const int32_t* row_start, const int32_t* len,
                                int32_t rows, int32_t k, int32_t* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  // Rows of a pitch of 2^18 or more take the long-row sample (6144 keys in runs of 8).
  if (ld >= kSelLongRow)
    select_rows_kernel<true><<<dim3(rows), dim3(kSelThreads), 0, s>>>(x, ld, row_start, len, k, out);
  else
    select_rows_kernel<false><<<dim3(rows), dim3(kSelThreads), 0, s>>>(x, ld, row_start, len, k, out);
  return hipGetLastError();
}

hipError_t launch_select_split(const float* x, int64_t ld, const int32_t* row_start, const int32_t* len,
                               int32_t rows, int32_t k, int32_t g, int32_t* out, void* ws, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const SegWs W = carve(ws, rows);
  const int64_t groups = 8 * (int64_t)g * ((rows + 7) / 8);
  seg_collect_kernel<<<dim3((unsigned)groups), dim3(kSelThreads), 0, s>>>(x, ld, row_start, len, rows, k, g, W);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seg_merge_kernel<<<dim3(rows), dim3(kSelThreads), 0, s>>>(x, ld, row_start, len, k, g, out, W);
  return hipGetLastError();
}

}  // namespace idx
