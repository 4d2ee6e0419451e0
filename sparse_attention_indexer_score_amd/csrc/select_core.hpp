// Exact top-m selection inside one workgroup (gfx950).
//
// Order: fp32 value descending with -0.0 == +0.0, ties to the lower index (ROCm DSA
// indexer top-k page: fp32 coarse histogram, exact radix tie refinement, full-row rescan
// when the tie buffer overflows).  Every element is given the 64-bit composite key
//     K = order_key(value) << 32 | (0xFFFFFFFF - index)
// which is unique per element and larger for the element that wins.  The top m are
// the m largest K.  K is resolved most-significant digit first in six levels of
// 12/12/8 bits (value) and 12/12/8 bits (inverted index):
//   level 1  an LDS histogram of the top 12 value bits over the whole input;
//   boundary the bin where the count from the top reaches m;
//   then     elements above the boundary bin are selected, elements inside it go to an
//            LDS tie buffer (kTieCap entries) and are refined by the next levels in LDS;
//            if the bin holds more than kTieCap elements the next levels rescan the
//            input instead, keeping only elements whose higher digits match.
// Selection stops at the first level whose boundary bin is entirely selected.
#pragma once
#include "common.hpp"

namespace idx {

struct Level {
  int shift;  // digit = (K >> shift) & ((1 << width) - 1)
  int width;
};
__device__ __forceinline__ Level level_of(int L) {
  // L = 1..6
  switch (L) {
    case 1: return {52, 12};
    case 2: return {40, 12};
    case 3: return {32, 8};
    case 4: return {20, 12};
    case 5: return {8, 12};
    default: return {0, 8};
  }
}

__device__ __forceinline__ uint64_t composite_key(uint32_t okey, int32_t index) {
  return ((uint64_t)okey << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)index);
}

struct SelSmem {
  uint32_t hist[kHistBins];
  uint32_t tkey[kTieCap];
  int32_t tidx[kTieCap];
  uint32_t scan[20];
  int32_t nout;
  int32_t ntie;
  int32_t bnd_bin;
  uint32_t bnd_above;
  uint32_t bnd_count;
};

// Input sources: element j has an order key and an index.
struct RowSrc {  // materialised fp32 row, index = position
  const float* x;
  __device__ __forceinline__ uint32_t key(int j) const { return order_key(x[j]); }
  __device__ __forceinline__ int32_t index(int j) const { return j; }
};
struct PairSrc {  // (score, index) pairs, e.g. a candidate slab row
  const float* s;
  const int32_t* i;
  __device__ __forceinline__ uint32_t key(int j) const { return order_key(s[j]); }
  __device__ __forceinline__ int32_t index(int j) const { return i[j]; }
};

template <int NT>
__device__ __forceinline__ void zero_hist(SelSmem& sm, int nbins) {
  for (int b = threadIdx.x; b < nbins; b += NT) sm.hist[b] = 0;
}

// Largest bin b with (count of bins >= b) >= need; need >= 1 and the total must reach it.
// Results in sm.bnd_*.  Contains barriers.
template <int NT>
__device__ void find_boundary(SelSmem& sm, int nbins, uint32_t need) {
  const int per = (nbins + NT - 1) / NT;
  const int hi = nbins - (int)threadIdx.x * per;  // this thread covers [lo, hi), high bins first
  const int lo = hi - per < 0 ? 0 : hi - per;
  uint32_t local = 0;
  for (int b = lo; b < hi; ++b) local += sm.hist[b];
  uint32_t total;
  uint32_t above = block_exclusive_sum<NT>(local, sm.scan, &total);
  if (hi > lo && above < need && above + local >= need) {
    for (int b = hi - 1; b >= lo; --b) {
      const uint32_t c = sm.hist[b];
      if (above + c >= need) {
        sm.bnd_bin = b;
        sm.bnd_above = above;
        sm.bnd_count = c;
        break;
      }
      above += c;
    }
  }
  __syncthreads();
}

// Wave-aggregated append: lanes with `pred` get consecutive slots from *counter.
// Must be called by all 64 lanes of the wave (converged).
__device__ __forceinline__ int wave_append_slot(bool pred, int32_t* counter) {
  const uint64_t m = wave_ballot(pred);
  if (m == 0) return -1;
  const int leader = __builtin_ctzll(m);
  int base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, __builtin_popcountll(m));
  base = __shfl(base, leader, kWave);
  return pred ? base + mask_prefix(m) : -1;
}

// Emit every element whose composite key has (K >> shift) >= prefix (shift <= 52).
template <int NT, class Src>
__device__ void emit_at_least(const Src& src, int n, int shift, uint64_t prefix, int32_t* out, SelSmem& sm) {
  for (int base = 0; base < n; base += NT) {
    const int j = base + (int)threadIdx.x;
    bool take = false;
    int32_t ix = 0;
    if (j < n) {
      ix = src.index(j);
      take = (composite_key(src.key(j), ix) >> shift) >= prefix;
    }
    const int slot = wave_append_slot(take, &sm.nout);
    if (take) out[slot] = ix;
  }
}

// Refine the LDS tie list (sm.ntie entries, all sharing the digits above level L) until
// `need` more elements are emitted to out[] through sm.nout.  Contains barriers.
template <int NT>
__device__ void refine_lds(int L, uint32_t need, int32_t* out, SelSmem& sm) {
  constexpr int PER = kTieCap / NT;
  for (;; ++L) {
    const Level lv = level_of(L);
    const int nbins = 1 << lv.width;
    const uint32_t dmask = (uint32_t)nbins - 1;
    const int nt = sm.ntie;
    zero_hist<NT>(sm, nbins);
    __syncthreads();
    uint32_t k_[PER];
    int32_t i_[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int t = (int)threadIdx.x + e * NT;
      if (t < nt) {
        k_[e] = sm.tkey[t];
        i_[e] = sm.tidx[t];
        atomicAdd(&sm.hist[(uint32_t)(composite_key(k_[e], i_[e]) >> lv.shift) & dmask], 1u);
      }
    }
    __syncthreads();
    find_boundary<NT>(sm, nbins, need);
    const uint32_t b = (uint32_t)sm.bnd_bin;
    const uint32_t above = sm.bnd_above;
    const uint32_t cnt = sm.bnd_count;
    const bool last = (cnt == need - above);
    if (threadIdx.x == 0) sm.ntie = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int t = (int)threadIdx.x + e * NT;
      uint32_t d = 0;
      if (t < nt) d = (uint32_t)(composite_key(k_[e], i_[e]) >> lv.shift) & dmask;
      const bool emit = (t < nt) && (d > b || (last && d == b));
      const bool keep = (t < nt) && !last && d == b;
      const int so = wave_append_slot(emit, &sm.nout);
      if (emit) out[so] = i_[e];
      const int sk = wave_append_slot(keep, &sm.ntie);
      if (keep) {
        sm.tkey[sk] = k_[e];
        sm.tidx[sk] = i_[e];
      }
    }
    __syncthreads();
    if (last) return;
    need -= above;
  }
}

// Rescan mode: resolve the remaining levels by passes over the whole input.  On entry
// the digits of levels < L are fixed to `prefix` (the value of K >> (shift of level L-1)),
// and `need` elements remain to be chosen among those matching it.  Contains barriers.
template <int NT, class Src>
__device__ void refine_rescan(const Src& src, int n, int L, uint64_t prefix, uint32_t need, int32_t* out,
                              SelSmem& sm) {
  int above_shift = level_of(L - 1).shift;
  for (;; ++L) {
    const Level lv = level_of(L);
    const int nbins = 1 << lv.width;
    const uint32_t dmask = (uint32_t)nbins - 1;
    zero_hist<NT>(sm, nbins);
    __syncthreads();
    for (int base = 0; base < n; base += NT) {
      const int j = base + (int)threadIdx.x;
      if (j < n) {
        const uint64_t K = composite_key(src.key(j), src.index(j));
        if ((K >> above_shift) == prefix) atomicAdd(&sm.hist[(uint32_t)(K >> lv.shift) & dmask], 1u);
      }
    }
    __syncthreads();
    find_boundary<NT>(sm, nbins, need);
    const uint32_t b = (uint32_t)sm.bnd_bin;
    const uint32_t above = sm.bnd_above;
    const uint32_t cnt = sm.bnd_count;
    __syncthreads();
    prefix = (prefix << lv.width) | b;
    above_shift = lv.shift;
    need -= above;
    if (cnt == need) {
      emit_at_least<NT>(src, n, lv.shift, prefix, out, sm);
      return;
    }
  }
}

// Histogram of the level-1 digit over n elements into sm.hist (sm.hist must be zero).
template <int NT, class Src>
__device__ __forceinline__ void hist_level1(const Src& src, int n, SelSmem& sm) {
  constexpr int U = 4;
  int base = 0;
  for (; base + U * NT <= n; base += U * NT) {
    uint32_t k_[U];
#pragma unroll
    for (int u = 0; u < U; ++u) k_[u] = src.key(base + u * NT + (int)threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) atomicAdd(&sm.hist[k_[u] >> (32 - kHistBits)], 1u);
  }
  for (; base < n; base += NT) {
    const int j = base + (int)threadIdx.x;
    if (j < n) atomicAdd(&sm.hist[src.key(j) >> (32 - kHistBits)], 1u);
  }
}

// Top-m of n elements (1 <= m <= n) by composite key; writes exactly m indices to
// out[0..m) in unspecified order.  All NT threads must call it.  Contains barriers.
template <int NT, class Src>
__device__ void block_select(const Src& src, int n, int m, int32_t* out, SelSmem& sm) {
  if (threadIdx.x == 0) {
    sm.nout = 0;
    sm.ntie = 0;
  }
  if (m >= n) {
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += NT) out[j] = src.index(j);
    __syncthreads();
    return;
  }
  zero_hist<NT>(sm, kHistBins);
  __syncthreads();
  hist_level1<NT>(src, n, sm);
  __syncthreads();
  find_boundary<NT>(sm, kHistBins, (uint32_t)m);
  const uint32_t b1 = (uint32_t)sm.bnd_bin;
  const uint32_t above = sm.bnd_above;
  const uint32_t cnt = sm.bnd_count;
  const uint32_t need = (uint32_t)m - above;
  __syncthreads();
  if (cnt == need) {  // the whole boundary bin is selected
    emit_at_least<NT>(src, n, 52, (uint64_t)b1, out, sm);
    __syncthreads();
    return;
  }
  if (cnt <= (uint32_t)kTieCap) {
    for (int base = 0; base < n; base += NT) {
      const int j = base + (int)threadIdx.x;
      uint32_t k = 0;
      int32_t ix = 0;
      uint32_t d = 0;
      if (j < n) {
        k = src.key(j);
        ix = src.index(j);
        d = k >> (32 - kHistBits);
      }
      const bool emit = j < n && d > b1;
      const bool tie = j < n && d == b1;
      const int so = wave_append_slot(emit, &sm.nout);
      if (emit) out[so] = ix;
      const int st = wave_append_slot(tie, &sm.ntie);
      if (tie) {
        sm.tkey[st] = k;
        sm.tidx[st] = ix;
      }
    }
    __syncthreads();
    refine_lds<NT>(2, need, out, sm);
  } else {
    refine_rescan<NT>(src, n, 2, (uint64_t)b1, need, out, sm);
  }
  __syncthreads();
}

// m-th largest order key of n elements (1 <= m <= n): three value levels, each a pass
// over the input.  Returns the key in every thread.  Contains barriers.
template <int NT, class Src>
__device__ uint32_t block_kth_key(const Src& src, int n, int m, SelSmem& sm) {
  uint32_t prefix = 0;
  int above_shift = 32;
  uint32_t need = (uint32_t)m;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int L = 0; L < 3; ++L) {
    const int sh = shifts[L];
    const int nbins = 1 << widths[L];
    zero_hist<NT>(sm, nbins);
    __syncthreads();
    for (int base = 0; base < n; base += NT) {
      const int j = base + (int)threadIdx.x;
      if (j < n) {
        const uint32_t k = src.key(j);
        const bool match = above_shift == 32 ? true : ((k >> above_shift) == prefix);
        if (match) atomicAdd(&sm.hist[(k >> sh) & (uint32_t)(nbins - 1)], 1u);
      }
    }
    __syncthreads();
    find_boundary<NT>(sm, nbins, need);
    const uint32_t b = (uint32_t)sm.bnd_bin;
    need -= sm.bnd_above;
    __syncthreads();
    prefix = (prefix << widths[L]) | b;
    above_shift = sh;
  }
  return prefix;
}

}  // namespace idx
