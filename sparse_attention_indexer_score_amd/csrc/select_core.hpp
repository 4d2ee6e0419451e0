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
//            LDS tie buffer (SM::kCap entries) and are refined by the next levels in LDS;
//            if the bin holds more than SM::kCap elements the next levels rescan the
//            input instead, keeping only elements whose higher digits match.
// Selection stops at the first level whose boundary bin is entirely selected, or once the
// bin holds at most 64 elements, which one wave then ranks directly.
#pragma once
#include <type_traits>

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

// LDS of one selecting workgroup; CAP is the capacity of the tie / candidate buffer.
template <int CAP>
struct SelSmemT {
  static constexpr int kCap = CAP;
  uint32_t hist[kHistBins];
  uint32_t tkey[CAP];
  int32_t tidx[CAP];
  uint32_t scan[20];
  int32_t nout;
  int32_t ntie;
  int32_t bnd_bin;
  uint32_t bnd_above;
  uint32_t bnd_count;
  uint32_t kmin, kmax;
};
using SelSmem = SelSmemT<kTieCap>;

// Input sources: element j has an order key and an index.
struct RowSrc {  // materialised fp32 row, index = position
  const float* x;
  __device__ __forceinline__ uint32_t key(int j) const { return order_key(x[j]); }
  __device__ __forceinline__ int32_t index(int j) const { return j; }
};
struct LdsKeySrc {  // order keys already in LDS, index = position
  const uint32_t* k;
  __device__ __forceinline__ uint32_t key(int j) const { return k[j]; }
  __device__ __forceinline__ int32_t index(int j) const { return j; }
};

// Order-preserving normalisation of keys known to lie in [lo, hi]: (key - lo) << lz with
// lz = the leading zeros of hi - lo, so that the keys' first differing bit becomes the top
// bit and a 12-bit histogram of the result spreads them over its bins (raw order keys of
// scores with one common exponent fall into a handful of bins).  Injective, and inverted
// by denormalize() for keys of the form normalize(k).
struct KeyNorm {
  uint32_t lo;
  int lz;  // 32 when hi == lo: every key maps to 0
  __device__ __forceinline__ uint32_t normalize(uint32_t k) const { return lz >= 32 ? 0u : (k - lo) << lz; }
  __device__ __forceinline__ uint32_t denormalize(uint32_t v) const { return lz >= 32 ? lo : (v >> lz) + lo; }
};
__device__ __forceinline__ KeyNorm key_norm(uint32_t lo, uint32_t hi) {
  return KeyNorm{lo, hi == lo ? 32 : __builtin_clz(hi - lo)};
}
struct NormLdsKeySrc {  // raw order keys in LDS, normalised as they are read; index = position
  const uint32_t* k;
  KeyNorm nz;
  __device__ __forceinline__ uint32_t key(int j) const { return nz.normalize(k[j]); }
  __device__ __forceinline__ int32_t index(int j) const { return j; }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, kWave));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, d, kWave));
  return v;
}
struct PairSrc {  // (score, index) pairs, e.g. a candidate slab row
  const float* s;
  const int32_t* i;
  __device__ __forceinline__ uint32_t key(int j) const { return order_key(s[j]); }
  __device__ __forceinline__ int32_t index(int j) const { return i[j]; }
};

template <int NT, class SM>
__device__ __forceinline__ void zero_hist(SM& sm, int nbins) {
  for (int b = threadIdx.x; b < nbins; b += NT) sm.hist[b] = 0;
}

// Largest bin b with (count of bins >= b) >= need; need >= 1 and the total must reach it.
// Results in sm.bnd_*.  Contains barriers.
template <int NT, class SM>
__device__ void find_boundary(SM& sm, int nbins, uint32_t need) {
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
  lds_sync();
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
template <int NT, class Src, class SM>
__device__ void emit_at_least(const Src& src, int n, int shift, uint64_t prefix, int32_t* out, SM& sm) {
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
// `need` more elements are emitted to out[] through sm.nout.  With nz1, the first level
// normalises the keys it reads (the kept ones are stored normalised for the next levels);
// with zeroed, the caller has already cleared the first level's histogram.  Contains
// barriers.
template <int NT, class SM>
__device__ __forceinline__ void refine_lds(int L, uint32_t need, int32_t* out, SM& sm, const KeyNorm* nz1 = nullptr,
                           bool zeroed = false) {
  constexpr int PER = (SM::kCap + NT - 1) / NT;
  for (bool first = true;; ++L, first = false) {
    const Level lv = level_of(L);
    const int nbins = 1 << lv.width;
    const uint32_t dmask = (uint32_t)nbins - 1;
    const int nt = sm.ntie;
    if (!(first && zeroed)) {
      zero_hist<NT>(sm, nbins);
      __syncthreads();
    }
    uint32_t k_[PER];
    int32_t i_[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int t = (int)threadIdx.x + e * NT;
      if (t < nt) {
        k_[e] = sm.tkey[t];
        if (first && nz1) k_[e] = nz1->normalize(k_[e]);
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
    // Emit and keep with one LDS atomic per wave for each, over all PER elements.
    uint64_t me[PER], mk[PER];
    int te = 0, tk = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int t = (int)threadIdx.x + e * NT;
      uint32_t d = 0;
      if (t < nt) d = (uint32_t)(composite_key(k_[e], i_[e]) >> lv.shift) & dmask;
      me[e] = wave_ballot((t < nt) && (d > b || (last && d == b)));
      mk[e] = wave_ballot((t < nt) && !last && d == b);
      te += __builtin_popcountll(me[e]);
      tk += __builtin_popcountll(mk[e]);
    }
    const int l = lane_id();
    int be = 0, bk = 0;
    if (l == 0) {
      if (te) be = atomicAdd(&sm.nout, te);
      if (tk) bk = atomicAdd(&sm.ntie, tk);
    }
    be = readlane(be, 0);
    bk = readlane(bk, 0);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if ((me[e] >> l) & 1) out[be + mask_prefix(me[e])] = i_[e];
      if ((mk[e] >> l) & 1) {
        const int sk = bk + mask_prefix(mk[e]);
        sm.tkey[sk] = k_[e];
        sm.tidx[sk] = i_[e];
      }
      be += __builtin_popcountll(me[e]);
      bk += __builtin_popcountll(mk[e]);
    }
    __syncthreads();
    if (last) return;
    need -= above;
    if (cnt <= (uint32_t)kWave) {
      // The boundary bin (now the whole tie buffer) fits one wave: wave 0 ranks its
      // elements by composite key directly instead of running further levels.
      if (threadIdx.x < kWave) {
        const bool have = l < (int)cnt;
        const uint32_t kk = have ? sm.tkey[l] : 0u;
        const int32_t ix = have ? sm.tidx[l] : 0;
        const uint64_t K = composite_key(kk, ix);
        int rank = 0;
        for (int u = 0; u < (int)cnt; ++u) {
          const uint64_t Ku = composite_key((uint32_t)readlane((int)kk, u), readlane(ix, u));
          rank += Ku > K ? 1 : 0;
        }
        const bool take = have && rank < (int)need;
        const uint64_t mt = wave_ballot(take);
        const int base = sm.nout;
        if (take) out[base + mask_prefix(mt)] = ix;
      }
      __syncthreads();
      return;
    }
  }
}

// Rescan mode: resolve the remaining levels by passes over the whole input.  On entry
// the digits of levels < L are fixed to `prefix` (the value of K >> (shift of level L-1)),
// and `need` elements remain to be chosen among those matching it.  Contains barriers.
template <int NT, class Src, class SM>
__device__ void refine_rescan(const Src& src, int n, int L, uint64_t prefix, uint32_t need, int32_t* out,
                              SM& sm) {
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
template <int NT, class Src, class SM>
__device__ __forceinline__ void hist_level1(const Src& src, int n, SM& sm) {
  constexpr int U = 4;
  int base = 0;
  for (; base + U * NT <= n; base += U * NT) {
    uint32_t k_[U];
#pragma unroll
    for (int u = 0; u < U; ++u) k_[u] = src.key(base + u * NT + (int)threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) atomicAdd(&sm.hist[k_[u] >> (32 - kHistBits)], 1u);
  }
  if (base < n) {  // the rest: clamped loads (a load under a branch waits before the next)
    uint32_t k_[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + (int)threadIdx.x;
      k_[u] = src.key(j < n ? j : n - 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * NT + (int)threadIdx.x < n) atomicAdd(&sm.hist[k_[u] >> (32 - kHistBits)], 1u);
  }
}

// Top-m of n elements (1 <= m <= n) by composite key; writes exactly m indices to
// out[0..m) in unspecified order.  A boundary bin of more than tie_cap (<= SM::kCap)
// elements is resolved by rescanning the input.  All NT threads must call it.  Contains
// barriers.
template <int NT, class Src, class SM>
__device__ __forceinline__ void block_select(const Src& src, int n, int m, int32_t* out, SM& sm,
                                             int tie_cap = SM::kCap) {
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
  if (cnt <= (uint32_t)tie_cap) {
    // U elements per thread and step, loaded unconditionally (clamped; the extra lanes are
    // masked), so that a step's loads are in flight together.
    constexpr int U = 4;
    for (int base = 0; base < n; base += U * NT) {
      uint32_t k_[U];
      int32_t ix_[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * NT + (int)threadIdx.x;
        const int jj = j < n ? j : n - 1;
        k_[u] = src.key(jj);
        ix_[u] = src.index(jj);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = base + u * NT + (int)threadIdx.x < n;
        const uint32_t d = k_[u] >> (32 - kHistBits);
        const bool emit = in && d > b1;
        const bool tie = in && d == b1;
        const int so = wave_append_slot(emit, &sm.nout);
        if (emit) out[so] = ix_[u];
        const int st = wave_append_slot(tie, &sm.ntie);
        if (tie) {
          sm.tkey[st] = k_[u];
          sm.tidx[st] = ix_[u];
        }
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
// over the input.  Returns the key in every thread; with fewer levels, the smallest key of
// the m-th key's bin at the last level (a lower bound of the m-th key).  Contains barriers.
template <int NT, class Src, class SM, int LEVELS = 3>
__device__ uint32_t block_kth_key(const Src& src, int n, int m, SM& sm, bool zeroed = false) {
  uint32_t prefix = 0;
  int above_shift = 32;
  uint32_t need = (uint32_t)m;
  constexpr int shifts[3] = {20, 8, 0};
  constexpr int widths[3] = {12, 12, 8};
#pragma unroll
  for (int L = 0; L < LEVELS; ++L) {
    const int sh = shifts[L];
    const int nbins = 1 << widths[L];
    if (!(L == 0 && zeroed)) {  // (zeroed: the caller cleared the first level's histogram)
      zero_hist<NT>(sm, nbins);
      lds_sync();
    }
    for (int base = 0; base < n; base += NT) {
      const int j = base + (int)threadIdx.x;
      if (j < n) {
        const uint32_t k = src.key(j);
        const bool match = above_shift == 32 ? true : ((k >> above_shift) == prefix);
        if (match) atomicAdd(&sm.hist[(k >> sh) & (uint32_t)(nbins - 1)], 1u);
      }
    }
    lds_sync();
    find_boundary<NT>(sm, nbins, need);
    const uint32_t b = (uint32_t)sm.bnd_bin;
    need -= sm.bnd_above;
    lds_sync();
    prefix = (prefix << widths[L]) | b;
    above_shift = sh;
  }
  return prefix << shifts[LEVELS - 1];  // LEVELS < 3: the lower edge of the m-th key's bin
}

// Top-m of a materialised row x[0..n) (1 <= m < n) with one full pass over it:
//   1. rows longer than the candidate buffer take a sample of SAMP order keys in
//      SAMP / SEG evenly spaced runs of SEG consecutive elements and a
//      threshold T = the lower edge of the 12-bit bin of the sample's r-th largest key
//      (keys normalised over the sample's range), r = ceil(1.75 m samples / n), so that
//      about 1.75 m elements of the row are expected at or above T, well inside [m, kCap]
//      (shorter rows: T = 0, every element);
//   2. one pass appends every element with key >= T to the LDS buffer (counting past its
//      capacity), with 16-byte loads issued one step ahead when the row is 16-byte
//      aligned, and one LDS atomic per wave and step;
//   3. if the buffer holds between m and SM::kCap elements, its keys are normalised over
//      [T, max] and the radix levels 1.. refine it in LDS; otherwise block_select() reruns
//      the row exactly with full passes.
// The result is exact either way; the sample only decides how much work is done.
// Sample shapes: 2048 keys in 32 runs of 64 (one or two cache lines each) for rows of up to
// a few hundred thousand elements; 6144 keys in 768 runs of 8 for longer rows, where r would
// otherwise fall to single digits and a few runs landing on (or missing) clustered high
// values move T far enough that the count leaves [m, kCap].
constexpr int kSelSamples = 2048;
constexpr int kSelSamplesLong = 6144;
constexpr int kSelLongRow = 1 << 18;  // rows of at least this many elements take the long sample

// Steps 1 and 2 for the elements [lo, lo + len) of the row x[0..n): the sample, and so T,
// is the whole row's whichever segment is streamed, so that every segment of a row keeps
// the same candidates it would in a whole-row pass.  Leaves the segment's candidates
// (order key >= T) in sm.tkey / sm.tidx with their row indices, their count in sm.ntie
// (counting past SM::kCap; only the first kCap are stored), their largest key in sm.kmax,
// sm.nout = 0 and a zeroed histogram; returns T (0 when the row is no longer than kCap).
// VEC: x + lo is 16-byte aligned and len >= 4 (the 16-byte path; otherwise the 4-byte path
// only).  UV: 16-byte loads per thread and step of the streaming pass (a multiple of 4; a
// narrow workgroup takes more, to keep as many bytes in flight).  Contains barriers.
template <int NT, bool VEC, class SM, int SAMP, int SEG, int UV>
__device__ __forceinline__ uint32_t sampled_collect(const float* x, int n, int m, int lo, int len, SM& sm) {
  static_assert(SM::kCap >= SAMP, "the sample lives in the candidate buffer");
  static_assert(SAMP % SEG == 0 && SAMP / SEG >= 2, "whole runs");
  constexpr int NSEG = SAMP / SEG;
  const int l = lane_id();
  // Streaming pass state: 16-byte loads, UV per thread per step, the next step's loads
  // issued before this step's keys are tested.  The first step's loads do not depend on
  // the threshold, so they are issued before the sample is taken and arrive under it.
  static_assert(UV % 4 == 0, "whole groups of 4 vectors");
  const float4* xv = reinterpret_cast<const float4*>(x + lo);
  const int nv = VEC ? len / 4 : 0;  // >= 1 with VEC
  float4 cur[UV], nxt[UV];
  // Unconditional loads (lanes past the end re-read the last vector and are masked when
  // tested): a load under a branch would leave the compiler unable to count the loads in
  // flight, and it would then wait for the step issued ahead before testing this one.
  // Needs nv >= 1.
  auto load = [&](float4* v, int base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < UV; ++u) {
      const int jv = base + u * NT + (int)threadIdx.x;
      v[u] = xv[jv < nv ? jv : nv - 1];
    }
  };
  // The sample's loads go first: loads complete in order, so the sample can be ranked while
  // the first step is still in flight (the barriers up to the streaming pass order LDS only).
  constexpr int SPT = SAMP / NT;
  static_assert(SAMP % NT == 0, "whole sample elements per thread");
  float sv[SPT];
  if (n > SM::kCap) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int t = i * NT + (int)threadIdx.x;
      const int seg = t / SEG, e = t % SEG;
      sv[i] = x[(int64_t)seg * (n - SEG) / (NSEG - 1) + e];
    }
  }
  if constexpr (VEC) load(cur, 0);  // (unconditional, so that the sample's waits can be counted)
  uint32_t T = 0;
  if (threadIdx.x == 0) {
    sm.kmin = 0xFFFFFFFFu;
    sm.kmax = 0u;
  }
  lds_sync();
  if (n > SM::kCap) {
    uint32_t lo_k = 0xFFFFFFFFu, hi_k = 0u;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int t = i * NT + (int)threadIdx.x;
      const uint32_t k = order_key(sv[i]);
      sm.tkey[t] = k;
      lo_k = min(lo_k, k);
      hi_k = max(hi_k, k);
    }
    lo_k = wave_min_u32(lo_k);
    hi_k = wave_max_u32(hi_k);
    if (l == 0) {
      atomicMin(&sm.kmin, lo_k);
      atomicMax(&sm.kmax, hi_k);
    }
    zero_hist<NT>(sm, kHistBins);  // the sample's radix level, cleared under the same barrier
    lds_sync();
    const KeyNorm nz = key_norm(sm.kmin, sm.kmax);
    int64_t rank = ((int64_t)7 * m * SAMP + (int64_t)4 * n - 1) / ((int64_t)4 * n);  // ceil(1.75 m S / n)
    rank = rank < 1 ? 1 : (rank > SAMP ? SAMP : rank);
    T = nz.denormalize(block_kth_key<NT, NormLdsKeySrc, SM, 1>(NormLdsKeySrc{sm.tkey, nz}, SAMP, (int)rank,
                                                                 sm, true));
    lds_sync();
  }
  if (threadIdx.x == 0) {
    sm.ntie = 0;
    sm.nout = 0;
    sm.kmax = 0u;
  }
  zero_hist<NT>(sm, kHistBins);  // for the refinement (the streaming pass does not use it)
  lds_sync();
  uint32_t kmax = 0u;
  // Appends the lanes' keys k_[u] (element ix_[u]) that pass, one LDS atomic per wave.
  auto append = [&](const uint32_t* k_, const bool* ok, const int* ix_, auto Uc) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    uint64_t mk[U];
    int tot = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mk[u] = wave_ballot(ok[u] && k_[u] >= T);
      tot += __builtin_popcountll(mk[u]);
    }
    if (tot) {  // wave-uniform
      int at = 0;
      if (l == 0) at = atomicAdd(&sm.ntie, tot);
      at = readlane(at, 0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if ((mk[u] >> l) & 1) {
          const int slot = at + mask_prefix(mk[u]);
          if (slot < SM::kCap) {
            sm.tkey[slot] = k_[u];
            sm.tidx[slot] = ix_[u];
          }
          kmax = max(kmax, k_[u]);
        }
        at += __builtin_popcountll(mk[u]);
      }
    }
  };
  // Vector part: one append (one LDS atomic per wave) for each 16 keys (4 vectors) of a step.
  for (int base = 0; VEC && base < nv; base += UV * NT) {
    load(nxt, base + UV * NT);  // past the end on the last step: re-reads of the last vector
#pragma unroll
    for (int g = 0; g < UV; g += 4) {
      uint32_t k_[16];
      bool ok[16];
      int ix_[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jv = base + (g + u) * NT + (int)threadIdx.x;
        k_[4 * u + 0] = order_key(cur[g + u].x);
        k_[4 * u + 1] = order_key(cur[g + u].y);
        k_[4 * u + 2] = order_key(cur[g + u].z);
        k_[4 * u + 3] = order_key(cur[g + u].w);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ok[4 * u + c] = jv < nv;
          ix_[4 * u + c] = lo + 4 * jv + c;
        }
      }
      append(k_, ok, ix_, std::integral_constant<int, 16>{});
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) cur[u] = nxt[u];
  }
  // Scalar part: the rest (all of the segment when it is not 16-byte aligned), loads
  // clamped like the vector part's.
  constexpr int U = 8;
  const float* xs = x + lo;
  for (int base = nv * 4; base < len; base += U * NT) {
    uint32_t k_[U];
    bool ok[U];
    int ix_[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + (int)threadIdx.x;
      ok[u] = j < len;
      k_[u] = order_key(xs[ok[u] ? j : len - 1]);
      ix_[u] = lo + j;
    }
    append(k_, ok, ix_, std::integral_constant<int, U>{});
  }
  kmax = wave_max_u32(kmax);
  if (l == 0 && kmax) atomicMax(&sm.kmax, kmax);
  __syncthreads();
  return T;
}

// Top-m of a materialised row x[0..n) (1 <= m < n): sampled_collect() over the whole row,
// then the LDS refinement of its candidates, or the exact multi-pass block_select() when
// the sample misjudged the row.  VEC and UV as for sampled_collect().
template <int NT, bool VEC, class SM, int SAMP = kSelSamples, int SEG = 64, int UV = 4>
__device__ void block_select_sampled(const float* x, int n, int m, int32_t* out, SM& sm) {
  const uint32_t T = sampled_collect<NT, VEC, SM, SAMP, SEG, UV>(x, n, m, 0, n, sm);
  const int c = sm.ntie;
  const KeyNorm nz = key_norm(T, sm.kmax);
  __syncthreads();
  if (c >= m && c <= SM::kCap) {
    refine_lds<NT>(1, (uint32_t)m, out, sm, &nz, true);  // keys normalised over [T, max] as read
  } else {
    block_select<NT>(RowSrc{x}, n, m, out, sm);
  }
}

}  // namespace idx
