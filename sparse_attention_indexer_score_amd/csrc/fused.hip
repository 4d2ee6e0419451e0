// Scoring kernels for gfx950: materialised scores, threshold samples, the fused
// score + filter into the candidate slab, the slab select and the exact fallback.
//
// Route of idx_fused_topk (LiteTopK prefill indexer page, "sampled threshold" and
// sections 1-2; exactness as in the ROCm DSA indexer top-k page):
//   K1a  score_kernel<SAMPLE>     scores of the keys p + j*S (odd stride S, phase p hashed
//                                 from the row block) for every row that sees > cap keys
//   K1b  threshold_kernel         T_r = m-th largest sample score, m chosen so that about
//                                 2.25*k keys of the row reach T_r; T_r = -inf for rows
//                                 that see <= cap keys (they keep every key)
//   K2   score_kernel<FILTER>     score every visible key; (score, key - ks) with
//                                 score >= T_r is appended to the row's slab, count[r]
//                                 keeps counting past cap
//   K3   slab_select_kernel       exact select over the slab; rows with count < min(k, V)
//                                 or count > cap are queued for K4
//   K4   fallback_kernel          re-score a queued row into scratch and select exactly
// If count >= min(k, V) and count <= cap, the slab holds every key whose score reaches the
// k-th largest score, so selecting over it equals selecting over the whole row.
#include "launch.hpp"
#include "score_core.hpp"
#include "select_core.hpp"

namespace idx {

enum : int { MODE_STORE = 0, MODE_FILTER = 1, MODE_SAMPLE = 2 };

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kTile = 32;      // keys per MFMA block

#ifndef IDX_ROWS_PER_WAVE
#define IDX_ROWS_PER_WAVE 2
#endif
constexpr int kRowsPerWave = IDX_ROWS_PER_WAVE;  // rows per wave of the contiguous-K kernel

// Rows per workgroup of the paged kernel (score_kernel) and of score_tiles_kernel.
static int rows_per_block_paged(int heads) { return 4 * (heads == 64 ? 2 : 4); }
int rows_per_block(int heads) { return 4 * kRowsPerWave; }
static int rows_per_block_for(const DevProblem& P) {
  return P.page_table ? rows_per_block_paged(P.heads) : rows_per_block(P.heads);
}

// Odd sample stride: the largest odd S <= 2.25*k/64, so that a row of V keys yields about
// V/S samples of which m ~ 64 lie at or above the threshold (LiteTopK page, section 2:
// single keys at an odd stride, phase hashed against periodic data).
int sample_stride_for(int k) {
  int s = (9 * k) / (4 * 64);
  if (s < 1) s = 1;
  if ((s & 1) == 0) s -= 1;
  return s < 1 ? 1 : s;
}

__device__ __forceinline__ int sample_phase(int row_block, int stride) {
  uint32_t x = (uint32_t)row_block * 0x9E3779B9u + 0x7F4A7C15u;
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return (int)(x % (uint32_t)stride);
}

// Sample slots j with p + j*S in [ks, ke).
__device__ __forceinline__ void sample_range(int ks, int ke, int p, int S, int& jlo, int& jhi) {
  jlo = ks <= p ? 0 : (ks - p + S - 1) / S;
  jhi = ke <= p ? 0 : (ke - p + S - 1) / S;
  if (jhi < jlo) jhi = jlo;
}

struct EpiArgs {
  // STORE
  float* out;
  int64_t ld;
  // FILTER
  const float* thr;
  int32_t* cnt;
  float* slab_s;
  int32_t* slab_i;
  int32_t cap;
  // SAMPLE
  float* samp;
  int32_t ns;
  int32_t stride;
  int32_t skip_le;  // SAMPLE: rows with ke - ks <= skip_le need no samples
};

struct TileWork {
  int32_t nrb;     // row blocks
  int32_t nchunk;  // position chunks per row block
  int32_t chunk;   // positions per chunk (multiple of kTile)
  int32_t pad;
  int64_t total;   // nrb * nchunk
};

// Workgroup -> (row block, chunk).  Workgroups are dealt to the 8 XCDs round-robin, so
// workgroup b runs on XCD b % 8; all row blocks of one chunk go to the same XCD, back to
// back, and the chunk's keys are fetched into that XCD's L2 once.
__device__ __forceinline__ int64_t map_item(const TileWork& W) {
  const int64_t b = blockIdx.x;
  const int64_t x = b & 7, local = b >> 3;
  const int64_t g = local / W.nrb, j = local % W.nrb;
  return (g * 8 + x) * W.nrb + j;
}

__device__ __forceinline__ float finish_score(float head_sum, float kscale) { return head_sum * kscale; }

template <int FMT, int H, int MODE, bool PAGED>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs A, EpiArgs E, TileWork W) {
  constexpr int RW = (H == 64) ? 2 : 4;  // rows per wave
  constexpr int RB = 4 * RW;             // rows per workgroup
  const int64_t item = map_item(W);
  if (item >= W.total) return;
  const int rb = (int)(item % W.nrb);
  const int chunk = (int)(item / W.nrb);
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  const int row0 = rb * RB + wave * RW;
  const int phase = (MODE == MODE_SAMPLE) ? sample_phase(rb, E.stride) : 0;

  // Positions are keys (STORE/FILTER) or sample slots (SAMPLE); plo/phi: valid range.
  int plo[RW], phi[RW], ksr[RW];
  float thr[RW];
  int wlo = 0x7FFFFFFF, whi = 0;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = row0 + i;
    plo[i] = 0;
    phi[i] = 0;
    ksr[i] = 0;
    thr[i] = 0.0f;
    if (r < A.rows) {
      const int ks = A.ks[r], ke = A.ke[r];
      ksr[i] = ks;
      if (MODE == MODE_SAMPLE) {
        if (ke - ks > E.skip_le) sample_range(ks, ke, phase, E.stride, plo[i], phi[i]);
      } else {
        plo[i] = ks;
        phi[i] = ke;
      }
      if (MODE == MODE_FILTER) thr[i] = E.thr[r];
      if (phi[i] > plo[i]) {
        wlo = min(wlo, plo[i]);
        whi = max(whi, phi[i]);
      }
    }
  }
  const int c0 = chunk * W.chunk, c1 = c0 + W.chunk;
  const int t0 = max(c0, wlo) / kTile, t1 = (min(c1, whi) + kTile - 1) / kTile;
  if (t0 >= t1) return;  // wave-uniform: nothing visible in this chunk

  RowOperand<FMT, H> ro[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i)
    if (row0 + i < A.rows) load_row<FMT, H>(ro[i], A, row0 + i);

  for (int t = t0; t < t1; ++t) {
    const int pos = t * kTile + (l & 31);
    const int64_t key = (MODE == MODE_SAMPLE) ? (int64_t)phase + (int64_t)pos * E.stride : (int64_t)pos;
    KeyOperand kshared;
    int64_t phys_shared = 0;
    if constexpr (!PAGED) {
      phys_shared = key < A.num_keys ? key : 0;
      load_key_global<FMT>(kshared, A, phys_shared);
    }
#pragma unroll
    for (int i = 0; i < RW; i += 2) {
      const bool actA = plo[i] < (t + 1) * kTile && phi[i] > t * kTile;
      const bool actB = plo[i + 1] < (t + 1) * kTile && phi[i + 1] > t * kTile;
      if (!actA && !actB) continue;
      float pa = 0.0f, pb = 0.0f;
      int64_t physA = phys_shared, physB = phys_shared;
      if constexpr (PAGED) {
        const bool vA = pos >= plo[i] && pos < phi[i];
        const bool vB = pos >= plo[i + 1] && pos < phi[i + 1];
        physA = vA ? physical_key(A, row0 + i, key) : 0;
        physB = vB ? physical_key(A, row0 + i + 1, key) : 0;
        if (actA) {
          KeyOperand ko;
          load_key_global<FMT>(ko, A, physA);
          pa = row_partial<FMT, H>(ro[i], ko);
        }
        if (actB) {
          KeyOperand ko;
          load_key_global<FMT>(ko, A, physB);
          pb = row_partial<FMT, H>(ro[i + 1], ko);
        }
      } else {
        if (actA) pa = row_partial<FMT, H>(ro[i], kshared);
        if (actB) pb = row_partial<FMT, H>(ro[i + 1], kshared);
      }
      const float hs = combine_halves(pa, pb);
      const bool upper = l >= 32;
      const int ri = upper ? i + 1 : i;
      const int r = row0 + ri;
      const int64_t phys = upper ? physB : physA;
      const bool valid = pos >= (upper ? plo[i + 1] : plo[i]) && pos < (upper ? phi[i + 1] : phi[i]);
      const float score = finish_score(hs, key_scale(A, valid ? phys : 0));
      const int ks = upper ? ksr[i + 1] : ksr[i];
      if constexpr (MODE == MODE_STORE) {
        if (valid) E.out[(int64_t)r * E.ld + (key - ks)] = score;
      } else if constexpr (MODE == MODE_SAMPLE) {
        if (valid) E.samp[(int64_t)r * E.ns + pos] = score;
      } else {
        const float tr = upper ? thr[i + 1] : thr[i];
        const bool pred = valid && score >= tr;
        const uint64_t m = wave_ballot(pred);
        if (m) {
          const uint32_t mA = (uint32_t)m, mB = (uint32_t)(m >> 32);
          int baseA = 0, baseB = 0;
          if (l == 0 && mA) baseA = atomicAdd(&E.cnt[row0 + i], __builtin_popcount(mA));
          if (l == 32 && mB) baseB = atomicAdd(&E.cnt[row0 + i + 1], __builtin_popcount(mB));
          baseA = readlane(baseA, 0);
          baseB = readlane(baseB, 32);
          const int before = mask_prefix(m) - (upper ? __builtin_popcount(mA) : 0);
          const int slot = (upper ? baseB : baseA) + before;
          if (pred && slot < E.cap) {
            const int64_t o = (int64_t)r * E.cap + slot;
            E.slab_s[o] = score;
            E.slab_i[o] = (int32_t)(key - ks);
          }
        }
      }
    }
  }
}

// Contiguous-K scoring kernel (STORE / FILTER / SAMPLE epilogues).
//
// Every row of a workgroup reads the same keys, so a wave holds RW rows' query operands in
// registers and streams 32-key tiles: the tile's key operand is loaded once per wave
// (scalar tile base + per-lane offset, next tile prefetched) and multiplied against all RW
// rows.  Row ranges are wave-uniform and kept in scalar registers; a tile that lies inside
// every row's range takes a branch-free path that issues all MFMAs before the head-reduce
// VALU work, so the reduce of one row overlaps the MFMAs of the next.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int FMT>
__device__ __forceinline__ void load_key_at(KeyOperand& ko, const uint8_t* kbase, const uint8_t* sfbase,
                                            uint32_t off, uint32_t sf_off) {
  constexpr int KB = Fmt<FMT>::kBytes;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if constexpr (FMT == FMT_E4M3) {
      const v4i x0 = *reinterpret_cast<const v4i*>(kbase + off + ks * (KB / 2));
      const v4i x1 = *reinterpret_cast<const v4i*>(kbase + off + ks * (KB / 2) + 16);
      ko.b[ks] = v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      ko.sb[ks] = 127;
    } else {
      const v4i x = *reinterpret_cast<const v4i*>(kbase + off + ks * (KB / 2));
      ko.b[ks] = v8i{x.x, x.y, x.z, x.w, 0, 0, 0, 0};
    }
  }
  if constexpr (FMT == FMT_MXFP4) {
    const int half = lane_id() >> 5;
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(sfbase + sf_off);
    ko.sb[0] = (sw >> (8 * half)) & 0xFF;
    ko.sb[1] = (sw >> (8 * (2 + half))) & 0xFF;
  }
}

template <int FMT, int H>
__device__ __forceinline__ void mfma_row(v16f (&acc)[H / 32], const RowOperand<FMT, H>& ro, const KeyOperand& ko) {
  constexpr int C = Fmt<FMT>::kCode;
#pragma unroll
  for (int mt = 0; mt < H / 32; ++mt) {
    v16f a = {};
    a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ro.a[mt][0], ko.b[0], a, C, C, 0, ro.sa[mt][0], 0, ko.sb[0]);
    a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ro.a[mt][1], ko.b[1], a, C, C, 0, ro.sa[mt][1], 0, ko.sb[1]);
    acc[mt] = a;
  }
}

// Same arithmetic, in the same order, as row_partial().
template <int FMT, int H>
__device__ __forceinline__ float reduce_row(const v16f (&acc)[H / 32], const RowOperand<FMT, H>& ro) {
  float p = 0.0f;
#pragma unroll
  for (int mt = 0; mt < H / 32; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) p = __builtin_fmaf(ro.w[mt][i], relu(acc[mt][i]), p);
  return p;
}

template <int FMT, int H, int MODE, int RW>
__global__ __launch_bounds__(kThreads) void score_tiles_kernel(ScoreArgs A, EpiArgs E, TileWork W) {
  static_assert(RW % 2 == 0, "rows are processed in pairs");
  constexpr int KB = Fmt<FMT>::kBytes;
  constexpr int RB = 4 * RW;
  constexpr int NP = RW / 2;
  const int64_t item = map_item(W);
  if (item >= W.total) return;
  const int rb = (int)(item % W.nrb);
  const int chunk = (int)(item / W.nrb);
  const int wave = uniform(threadIdx.x / kWave);
  const int l = lane_id();
  const int half = l >> 5, col = l & 31;
  const int row0 = rb * RB + wave * RW;
  const int S = (MODE == MODE_SAMPLE) ? E.stride : 1;
  const int phase = (MODE == MODE_SAMPLE) ? sample_phase(rb, S) : 0;

  // Row ranges in position space (keys, or sample slots), wave-uniform.
  int plo[RW], phi[RW], ksr[RW];
  int wlo = 0x7FFFFFFF, whi = 0, full_lo = 0, full_hi = 0x7FFFFFFF;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = row0 + i;
    plo[i] = phi[i] = ksr[i] = 0;
    if (r < A.rows) {
      const int ks = uniform(A.ks[r]), ke = uniform(A.ke[r]);
      ksr[i] = ks;
      if (MODE == MODE_SAMPLE) {
        if (ke - ks > E.skip_le) sample_range(ks, ke, phase, S, plo[i], phi[i]);
      } else {
        plo[i] = ks;
        phi[i] = ke;
      }
    }
    if (phi[i] > plo[i]) {
      wlo = min(wlo, plo[i]);
      whi = max(whi, phi[i]);
    }
    full_lo = max(full_lo, plo[i]);
    full_hi = min(full_hi, phi[i]);
  }
  const int c0 = chunk * W.chunk, c1 = c0 + W.chunk;
  const int t0 = max(c0, wlo) / kTile, t1 = (min(c1, whi) + kTile - 1) / kTile;
  if (t0 >= t1) return;

  RowOperand<FMT, H> ro[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i)
    if (row0 + i < A.rows) load_row<FMT, H>(ro[i], A, row0 + i);

  // Per-lane constants of each row pair: lanes 0-31 carry row 2p, lanes 32-63 row 2p+1.
  float thr_l[NP];
  int ks_l[NP], lo_l[NP], hi_l[NP];
  int64_t row_l[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int i = 2 * p + half;
    row_l[p] = row0 + i;
    ks_l[p] = half ? ksr[2 * p + 1] : ksr[2 * p];
    lo_l[p] = half ? plo[2 * p + 1] : plo[2 * p];
    hi_l[p] = half ? phi[2 * p + 1] : phi[2 * p];
    thr_l[p] = 0.0f;
    if (MODE == MODE_FILTER && row0 + i < A.rows) thr_l[p] = E.thr[row0 + i];
  }

  const int64_t kstep = (int64_t)kTile * S;                 // keys per tile
  const uint32_t off = (uint32_t)(col * S) * KB + half * (KB / 4);
  const uint32_t sf_off = (uint32_t)(col * S) * 4;
  const int64_t last_key = A.num_keys - 1;
  auto tile_key0 = [&](int t) -> int64_t { return (int64_t)phase + (int64_t)t * kstep; };
  auto load_tile = [&](KeyOperand& ko, int t) {
    const int64_t k0 = tile_key0(t);
    if (k0 + (kTile - 1) * (int64_t)S <= last_key) {
      load_key_at<FMT>(ko, A.k + k0 * KB, A.k_sf + k0 * 4, off, sf_off);
    } else {  // ragged tail: clamp every lane to a real key (results are masked)
      int64_t key = k0 + (int64_t)col * S;
      key = key < last_key ? key : last_key;
      load_key_at<FMT>(ko, A.k + key * KB, A.k_sf + key * 4, half * (KB / 4), 0);
    }
  };

  // One tile: MFMAs for all RW rows first, then the head reduce and epilogue per row pair.
  // Rows that do not see (part of) the tile are computed anyway and masked per lane.
  auto compute = [&](const KeyOperand& kc, int t) {
    const int pos = t * kTile + col;
    const int64_t key = tile_key0(t) + (int64_t)col * S;
    const bool full = t * kTile >= full_lo && (t + 1) * kTile <= full_hi;  // wave-uniform
    float kscale = 1.0f;
    if (A.k_scale) kscale = A.k_scale[key < last_key ? key : last_key];
    v16f acc[RW][H / 32];
#pragma unroll
    for (int i = 0; i < RW; ++i) mfma_row<FMT, H>(acc[i], ro[i], kc);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float pa = reduce_row<FMT, H>(acc[2 * p], ro[2 * p]);
      const float pb = reduce_row<FMT, H>(acc[2 * p + 1], ro[2 * p + 1]);
      const float score = finish_score(combine_halves(pa, pb), kscale);
      const bool valid = full || (pos >= lo_l[p] && pos < hi_l[p]);
      if constexpr (MODE == MODE_STORE) {
        if (valid) E.out[row_l[p] * E.ld + (key - ks_l[p])] = score;
      } else if constexpr (MODE == MODE_SAMPLE) {
        if (valid) E.samp[row_l[p] * E.ns + pos] = score;
      } else {
        const bool pred = valid && score >= thr_l[p];
        const uint64_t m = wave_ballot(pred);
        if (m) {
          const uint32_t mA = (uint32_t)m, mB = (uint32_t)(m >> 32);
          int baseA = 0, baseB = 0;
          if (l == 0 && mA) baseA = atomicAdd(&E.cnt[row0 + 2 * p], __builtin_popcount(mA));
          if (l == 32 && mB) baseB = atomicAdd(&E.cnt[row0 + 2 * p + 1], __builtin_popcount(mB));
          baseA = readlane(baseA, 0);
          baseB = readlane(baseB, 32);
          const int slot = (half ? baseB : baseA) + mask_prefix(m) - (half ? __builtin_popcount(mA) : 0);
          if (pred && slot < E.cap) {
            const int64_t o = row_l[p] * E.cap + slot;
            E.slab_s[o] = score;
            E.slab_i[o] = (int32_t)(key - ks_l[p]);
          }
        }
      }
    }
  };

  // Two key buffers, alternating, so the next tile's loads overlap this tile's math.
  KeyOperand ka, kb;
  load_tile(ka, t0);
  int t = t0;
  for (; t + 1 < t1; t += 2) {
    load_tile(kb, t + 1);
    compute(ka, t);
    if (t + 2 < t1) load_tile(ka, t + 2);
    compute(kb, t + 1);
  }
  if (t < t1) compute(ka, t);
}

// ----------------------------------------------------------------------------- K1b

struct ThrArgs {
  const int32_t* ks;
  const int32_t* ke;
  const float* samp;
  float* thr;
  int32_t* cnt;
  long long* stats;
  int32_t* fb_ctrl;
  int32_t rows, k, cap, ns, stride, rb_rows;
  int32_t debug_mode, debug_row_mod;
};

__global__ __launch_bounds__(kThreads) void threshold_kernel(ThrArgs T) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x < kStatSlots) T.stats[threadIdx.x] = (threadIdx.x == kStatMin) ? 0x7FFFFFFF : 0;
  if (r == 0 && threadIdx.x < 2) T.fb_ctrl[threadIdx.x] = 0;
  const int ks = T.ks[r], ke = T.ke[r];
  const int V = ke - ks;
  if (threadIdx.x == 0) T.cnt[r] = 0;
  float tr;
  const bool forced = T.debug_mode != 0 && (T.debug_row_mod <= 0 || r % T.debug_row_mod == 0);
  if (forced) {
    tr = T.debug_mode == 1 ? __builtin_inff() : -__builtin_inff();
  } else if (V <= T.cap) {
    tr = -__builtin_inff();
  } else {
    const int p = sample_phase(r / T.rb_rows, T.stride);
    int jlo, jhi;
    sample_range(ks, ke, p, T.stride, jlo, jhi);
    const int n = jhi - jlo;
    if (n <= 0) {
      tr = -__builtin_inff();
    } else {
      // m-th largest of n samples; m = ceil(2.25 * k * n / V) so that ~2.25k keys pass.
      int64_t m = ((int64_t)9 * T.k * n + 4 * (int64_t)V - 1) / (4 * (int64_t)V);
      if (m < 1) m = 1;
      if (m > n) m = n;
      const uint32_t key = block_kth_key<kThreads>(RowSrc{T.samp + (int64_t)r * T.ns + jlo}, n, (int)m, sm);
      tr = order_key_to_float(key);
    }
  }
  if (threadIdx.x == 0) T.thr[r] = tr;
}

// ----------------------------------------------------------------------------- K3

struct SlabArgs {
  const int32_t* ks;
  const int32_t* ke;
  const int32_t* cnt;
  const float* slab_s;
  const int32_t* slab_i;
  int32_t* out;
  long long* stats;
  int32_t* fb_ctrl;
  int32_t* fb_list;
  int32_t k, cap;
};

__global__ __launch_bounds__(kThreads) void slab_select_kernel(SlabArgs S) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x;
  const int V = S.ke[r] - S.ks[r];
  const int c = S.cnt[r];
  const int need = min(S.k, V);
  int32_t* out = S.out + (int64_t)r * S.k;
  const bool bad = c > S.cap || c < need;
  if (threadIdx.x == 0) {
    atomicAdd((unsigned long long*)&S.stats[V <= S.cap ? kStatStoreAll : kStatSampled], 1ull);
    atomicMax((unsigned long long*)&S.stats[kStatMax], (unsigned long long)c);
    if (V > S.cap) atomicMin((unsigned long long*)&S.stats[kStatMin], (unsigned long long)c);
    atomicAdd((unsigned long long*)&S.stats[kStatTotal], (unsigned long long)c);
    if (bad) {
      atomicAdd((unsigned long long*)&S.stats[kStatFallback], 1ull);
      S.fb_list[atomicAdd(&S.fb_ctrl[0], 1)] = r;
    }
  }
  if (bad) return;  // uniform: the fallback writes this row
  if (need > 0)
    block_select<kThreads>(PairSrc{S.slab_s + (int64_t)r * S.cap, S.slab_i + (int64_t)r * S.cap}, c, need, out, sm);
  for (int j = need + threadIdx.x; j < S.k; j += kThreads) out[j] = -1;
}

// ----------------------------------------------------------------------------- K4

struct FbArgs {
  const int32_t* fb_list;
  int32_t* fb_ctrl;
  float* scratch;
  int64_t scratch_ld;
  int32_t* out;
  int32_t k;
};

template <int FMT, int H>
__global__ __launch_bounds__(kThreads) void fallback_kernel(ScoreArgs A, FbArgs F) {
  __shared__ SelSmem sm;
  __shared__ int sh_item;
  const int wave = threadIdx.x / kWave;
  const int l = lane_id();
  float* mine = F.scratch + (int64_t)blockIdx.x * F.scratch_ld;
  for (;;) {
    if (threadIdx.x == 0) sh_item = atomicAdd(&F.fb_ctrl[1], 1);
    __syncthreads();
    const int item = sh_item;
    __syncthreads();
    if (item >= F.fb_ctrl[0]) break;  // every wave sees the same item and count
    const int r = F.fb_list[item];
    const int ks = A.ks[r], ke = A.ke[r];
    const int V = ke - ks;
    RowOperand<FMT, H> ro;
    load_row<FMT, H>(ro, A, r);
    // Same 32-key tiles (absolute positions) and lane placement as score_kernel.
    for (int t = ks / kTile + wave; t * kTile < ke; t += 4) {
      const int pos = t * kTile + (l & 31);
      const bool valid = pos >= ks && pos < ke;
      const int64_t phys = valid ? physical_key(A, r, pos) : 0;
      KeyOperand ko;
      load_key_global<FMT>(ko, A, phys);
      const float p = row_partial<FMT, H>(ro, ko);
      const float hs = combine_halves(p, p);
      const float score = finish_score(hs, key_scale(A, phys));
      if (l < 32 && valid) mine[pos - ks] = score;
    }
    __syncthreads();
    const int need = min(F.k, V);
    int32_t* out = F.out + (int64_t)r * F.k;
    if (need > 0) block_select<kThreads>(RowSrc{mine}, V, need, out, sm);
    for (int j = need + threadIdx.x; j < F.k; j += kThreads) out[j] = -1;
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------- host

static ScoreArgs score_args(const DevProblem& P) {
  ScoreArgs A;
  A.q = P.q;
  A.q_sf = P.q_sf;
  A.k = P.k;
  A.k_sf = P.k_sf;
  A.k_scale = P.k_scale;
  A.w = P.w;
  A.ks = P.ks;
  A.ke = P.ke;
  A.page_table = P.page_table;
  A.row_req = P.row_req;
  A.max_pages = P.max_pages;
  A.rows = P.rows;
  A.num_keys = P.num_keys;
  return A;
}

static TileWork tile_work(const DevProblem& P, int64_t positions, int chunk) {
  TileWork W;
  const int rb = rows_per_block_for(P);
  W.nrb = (P.rows + rb - 1) / rb;
  W.chunk = chunk;
  W.nchunk = (int)((positions + chunk - 1) / chunk);
  if (W.nchunk < 1) W.nchunk = 1;
  W.pad = 0;
  W.total = (int64_t)W.nrb * W.nchunk;
  return W;
}

static dim3 tile_grid(const TileWork& W) {
  const int64_t groups = (W.nchunk + 7) / 8;
  return dim3((unsigned)(groups * 8 * W.nrb));
}

template <int MODE>
static hipError_t dispatch_score(const DevProblem& P, const EpiArgs& E, const TileWork& W, hipStream_t s) {
  const ScoreArgs A = score_args(P);
  const dim3 grid = tile_grid(W), block(kThreads);
  const bool paged = P.page_table != nullptr;
  constexpr int RW = kRowsPerWave;
  if (P.fmt == FMT_E4M3) {
    if (P.heads == 64) {
      if (paged) score_kernel<FMT_E4M3, 64, MODE, true><<<grid, block, 0, s>>>(A, E, W);
      else score_tiles_kernel<FMT_E4M3, 64, MODE, RW><<<grid, block, 0, s>>>(A, E, W);
    } else {
      if (paged) score_kernel<FMT_E4M3, 32, MODE, true><<<grid, block, 0, s>>>(A, E, W);
      else score_tiles_kernel<FMT_E4M3, 32, MODE, RW><<<grid, block, 0, s>>>(A, E, W);
    }
  } else {
    if (P.heads == 64) score_tiles_kernel<FMT_MXFP4, 64, MODE, RW><<<grid, block, 0, s>>>(A, E, W);
    else score_tiles_kernel<FMT_MXFP4, 32, MODE, RW><<<grid, block, 0, s>>>(A, E, W);
  }
  return hipGetLastError();
}

constexpr int kChunkKeys = 4096;
constexpr int kChunkSamples = 1024;

hipError_t launch_score_store(const DevProblem& P, float* out, int64_t ld, hipStream_t s) {
  if (P.rows == 0) return hipSuccess;
  EpiArgs E = {};
  E.out = out;
  E.ld = ld;
  return dispatch_score<MODE_STORE>(P, E, tile_work(P, P.key_span, kChunkKeys), s);
}

hipError_t launch_fused(const DevProblem& P, const FusedPlan& F, int32_t* out_idx, hipStream_t s, hipEvent_t* ev) {
  if (P.rows == 0) return hipSuccess;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  // K1a: samples
  {
    EpiArgs E = {};
    E.samp = F.samp;
    E.ns = F.ns;
    E.stride = F.stride;
    E.skip_le = F.cap;
    if (F.debug_mode != 0 && F.debug_row_mod <= 0) E.skip_le = 0x7FFFFFFF;  // every row forced
    if ((e = dispatch_score<MODE_SAMPLE>(P, E, tile_work(P, F.ns, kChunkSamples), s)) != hipSuccess)
      return e;
    if ((e = mark(1)) != hipSuccess) return e;
  }
  // K1b: thresholds (also clears counts, stats and the fallback queue)
  {
    ThrArgs T;
    T.ks = P.ks;
    T.ke = P.ke;
    T.samp = F.samp;
    T.thr = F.thr;
    T.cnt = F.cnt;
    T.stats = F.stats;
    T.fb_ctrl = F.fb_ctrl;
    T.rows = P.rows;
    T.k = F.k;
    T.cap = F.cap;
    T.ns = F.ns;
    T.stride = F.stride;
    T.rb_rows = rows_per_block_for(P);
    T.debug_mode = F.debug_mode;
    T.debug_row_mod = F.debug_row_mod;
    threshold_kernel<<<dim3(P.rows), dim3(kThreads), 0, s>>>(T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(2)) != hipSuccess) return e;
  }
  // K2: fused score + filter
  {
    EpiArgs E = {};
    E.thr = F.thr;
    E.cnt = F.cnt;
    E.slab_s = F.slab_s;
    E.slab_i = F.slab_i;
    E.cap = F.cap;
    if ((e = dispatch_score<MODE_FILTER>(P, E, tile_work(P, P.key_span, kChunkKeys), s)) != hipSuccess)
      return e;
    if ((e = mark(3)) != hipSuccess) return e;
  }
  // K3: select over the slab
  {
    SlabArgs S;
    S.ks = P.ks;
    S.ke = P.ke;
    S.cnt = F.cnt;
    S.slab_s = F.slab_s;
    S.slab_i = F.slab_i;
    S.out = out_idx;
    S.stats = F.stats;
    S.fb_ctrl = F.fb_ctrl;
    S.fb_list = F.fb_list;
    S.k = F.k;
    S.cap = F.cap;
    slab_select_kernel<<<dim3(P.rows), dim3(kThreads), 0, s>>>(S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(4)) != hipSuccess) return e;
  }
  // K4: exact fallback for queued rows (exits at once when the queue is empty)
  {
    const ScoreArgs A = score_args(P);
    FbArgs B;
    B.fb_list = F.fb_list;
    B.fb_ctrl = F.fb_ctrl;
    B.scratch = F.scratch;
    B.scratch_ld = F.scratch_ld;
    B.out = out_idx;
    B.k = F.k;
    const dim3 grid(F.fb_blocks), block(kThreads);
    if (P.fmt == FMT_E4M3) {
      if (P.heads == 64) fallback_kernel<FMT_E4M3, 64><<<grid, block, 0, s>>>(A, B);
      else fallback_kernel<FMT_E4M3, 32><<<grid, block, 0, s>>>(A, B);
    } else {
      if (P.heads == 64) fallback_kernel<FMT_MXFP4, 64><<<grid, block, 0, s>>>(A, B);
      else fallback_kernel<FMT_MXFP4, 32><<<grid, block, 0, s>>>(A, B);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(5)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace idx
