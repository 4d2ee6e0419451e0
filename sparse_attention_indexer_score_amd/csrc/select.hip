// Exact top-k over materialised fp32 rows (idx_select), gfx950.
//
// ROCm DSA indexer top-k page (sgl-project/sglang#37591): fp32 radix histogram of 12
// bits, exact tie refinement, full-row rescan when the tie buffer overflows, and, for
// long rows at low batch, several workgroups per row ("row split"):
//   split == 0  select_rows_kernel: one 1024-thread workgroup per row (a sampled threshold,
//               one pass into an LDS candidate buffer, radix refinement in LDS; the
//               multi-pass block_select when the sample misjudges the row)
//   split >= 2  mb_hist_kernel    g workgroups per row add their segment's level-1
//                                 histogram into a per-row global histogram
//               mb_scatter_kernel every workgroup finds the boundary bin from it, writes
//                                 its elements above the bin to the output and appends
//                                 the bin's elements to a per-row tie buffer
//               mb_refine_kernel  one workgroup per row refines the tie buffer in LDS,
//                                 or reruns the whole row in rescan mode if it overflowed
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

struct SplitWs {
  uint32_t* hist;  // [rows][4096]
  int32_t* pos;    // [rows] output cursor
  int32_t* tcnt;   // [rows] tie count
  uint32_t* tkey;  // [rows][kTieCap]
  int32_t* tidx;   // [rows][kTieCap]
};

static SplitWs carve(void* ws, int rows) {
  SplitWs W;
  char* p = static_cast<char*>(ws);
  W.hist = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * kHistBins * 4;
  W.pos = reinterpret_cast<int32_t*>(p);
  p += (size_t)rows * 4;
  W.tcnt = reinterpret_cast<int32_t*>(p);
  p += (size_t)rows * 4;
  p = reinterpret_cast<char*>(((uintptr_t)p + 255) & ~(uintptr_t)255);
  W.tkey = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * kTieCap * 4;
  W.tidx = reinterpret_cast<int32_t*>(p);
  return W;
}

size_t select_split_ws_bytes(int32_t rows) {
  size_t b = (size_t)rows * kHistBins * 4 + (size_t)rows * 8;
  b = (b + 255) & ~(size_t)255;
  b += (size_t)rows * kTieCap * 8;
  return b + 256;
}

// Clears hist, pos and tcnt (contiguous at the start of the workspace).
__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

__device__ __forceinline__ void segment(int n, int g, int part, int& lo, int& hi) {
  const int seg = (n + g - 1) / g;
  lo = min(n, part * seg);
  hi = min(n, lo + seg);
}

__global__ __launch_bounds__(kSelThreads) void mb_hist_kernel(const float* x, int64_t ld, const int32_t* row_start,
                                                              const int32_t* len, int32_t k, int32_t g, SplitWs W) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x / g, part = blockIdx.x % g;
  int n, m;
  const int64_t row_off = row_span(ld, row_start, len, r, k, n, m);
  if (m >= n) return;  // the refine kernel writes trivial rows
  int lo, hi;
  segment(n, g, part, lo, hi);
  zero_hist<kSelThreads>(sm, kHistBins);
  __syncthreads();
  hist_level1<kSelThreads>(RowSrc{x + row_off + lo}, hi - lo, sm);
  __syncthreads();
  uint32_t* gh = W.hist + (int64_t)r * kHistBins;
  for (int b = threadIdx.x; b < kHistBins; b += kSelThreads)
    if (sm.hist[b]) atomicAdd(&gh[b], sm.hist[b]);
}

__device__ __forceinline__ void load_row_hist(SelSmem& sm, const uint32_t* gh) {
  for (int b = threadIdx.x; b < kHistBins; b += kSelThreads) sm.hist[b] = gh[b];
  __syncthreads();
}

// Elements above the boundary bin, and the bin's elements when they are kept for
// refinement, are gathered in LDS first; one global atomic per workgroup and list then
// reserves their places in the row's output and tie buffer.  At most m <= 2048 elements of
// a row are above the bin (or in it, when it is selected whole) and at most kTieCap are in
// it when ties are kept, so both lists fit.

__global__ __launch_bounds__(kSelThreads) void mb_scatter_kernel(const float* x, int64_t ld,
                                                                 const int32_t* row_start, const int32_t* len,
                                                                 int32_t k, int32_t g, int32_t* out, SplitWs W) {
  __shared__ SelSmem sm;
  __shared__ int32_t eidx[kMaxTopK];
  const int r = blockIdx.x / g, part = blockIdx.x % g;
  int n, m;
  const int64_t off = row_span(ld, row_start, len, r, k, n, m);
  if (m >= n) return;
  load_row_hist(sm, W.hist + (int64_t)r * kHistBins);
  find_boundary<kSelThreads>(sm, kHistBins, (uint32_t)m);
  const uint32_t b1 = (uint32_t)sm.bnd_bin;
  const uint32_t cnt = sm.bnd_count;
  const bool all_bin = cnt == (uint32_t)m - sm.bnd_above;
  const bool keep_ties = !all_bin && cnt <= (uint32_t)kTieCap;
  if (threadIdx.x == 0) {
    sm.nout = 0;
    sm.ntie = 0;
  }
  __syncthreads();
  int lo, hi;
  segment(n, g, part, lo, hi);
  const int l = lane_id();
  // U elements per thread and step, loaded unconditionally at clamped positions (a load under
  // a branch is waited for before the next is issued); lanes past the end are masked.
  constexpr int U = 4;
  for (int base = lo; base < hi; base += U * kSelThreads) {
    uint32_t key_[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * kSelThreads + (int)threadIdx.x;
      key_[u] = order_key(x[off + (j < hi ? j : hi - 1)]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * kSelThreads + (int)threadIdx.x;
      const uint32_t key = key_[u], d = key >> (32 - kHistBits);
      const uint64_t me = wave_ballot(j < hi && (d > b1 || (all_bin && d == b1)));
      const uint64_t mt = wave_ballot(j < hi && keep_ties && d == b1);
      int be = 0, bt = 0;
      if (l == 0) {
        if (me) be = atomicAdd(&sm.nout, __builtin_popcountll(me));
        if (mt) bt = atomicAdd(&sm.ntie, __builtin_popcountll(mt));
      }
      be = readlane(be, 0);
      bt = readlane(bt, 0);
      if ((me >> l) & 1) eidx[be + mask_prefix(me)] = j;
      if ((mt >> l) & 1) {
        const int t = bt + mask_prefix(mt);
        sm.tkey[t] = key;
        sm.tidx[t] = j;
      }
    }
  }
  __syncthreads();
  const int ne = sm.nout, nt = sm.ntie;
  if (threadIdx.x == 0) {
    sm.bnd_bin = ne ? atomicAdd(&W.pos[r], ne) : 0;
    sm.bnd_above = nt ? (uint32_t)atomicAdd(&W.tcnt[r], nt) : 0u;
  }
  __syncthreads();
  const int ob = sm.bnd_bin, tb = (int)sm.bnd_above;
  int32_t* o = out + (int64_t)r * k;
  for (int t = threadIdx.x; t < ne; t += kSelThreads) o[ob + t] = eidx[t];
  for (int t = threadIdx.x; t < nt; t += kSelThreads) {
    W.tkey[(int64_t)r * kTieCap + tb + t] = sm.tkey[t];
    W.tidx[(int64_t)r * kTieCap + tb + t] = sm.tidx[t];
  }
}

__global__ __launch_bounds__(kSelThreads) void mb_refine_kernel(const float* x, int64_t ld,
                                                                const int32_t* row_start, const int32_t* len,
                                                                int32_t k, int32_t* out, SplitWs W) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x;
  int n, m;
  const int64_t off = row_span(ld, row_start, len, r, k, n, m);
  int32_t* o = out + (int64_t)r * k;
  if (m >= n) {
    for (int j = threadIdx.x; j < n; j += kSelThreads) o[j] = j;
  } else {
    load_row_hist(sm, W.hist + (int64_t)r * kHistBins);
    find_boundary<kSelThreads>(sm, kHistBins, (uint32_t)m);
    const uint32_t above = sm.bnd_above;
    const uint32_t cnt = sm.bnd_count;
    const uint32_t need = (uint32_t)m - above;
    __syncthreads();
    if (cnt == need) {
      // every element of the boundary bin was emitted by the scatter kernel
    } else if (cnt <= (uint32_t)kTieCap) {
      for (int t = threadIdx.x; t < (int)cnt; t += kSelThreads) {
        sm.tkey[t] = W.tkey[(int64_t)r * kTieCap + t];
        sm.tidx[t] = W.tidx[(int64_t)r * kTieCap + t];
      }
      if (threadIdx.x == 0) {
        sm.ntie = (int)cnt;
        sm.nout = (int)above;
      }
      __syncthreads();
      refine_lds<kSelThreads>(2, need, o, sm);
    } else {
      // tie buffer overflow: redo the whole row in one workgroup (rescan mode)
      block_select<kSelThreads>(RowSrc{x + off}, n, m, o, sm);
    }
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
  const SplitWs W = carve(ws, rows);
  const int64_t zero_words = (int64_t)rows * (kHistBins + 2);
  const int64_t zb = (zero_words + 255) / 256;
  zero_words_kernel<<<dim3((unsigned)(zb < 1024 ? zb : 1024)), dim3(256), 0, s>>>(W.hist, zero_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)rows * g)), block(kSelThreads);
  mb_hist_kernel<<<grid, block, 0, s>>>(x, ld, row_start, len, k, g, W);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mb_scatter_kernel<<<grid, block, 0, s>>>(x, ld, row_start, len, k, g, out, W);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mb_refine_kernel<<<dim3(rows), block, 0, s>>>(x, ld, row_start, len, k, out, W);
  return hipGetLastError();
}

}  // namespace idx
