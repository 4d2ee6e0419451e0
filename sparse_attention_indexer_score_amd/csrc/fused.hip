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
#include <type_traits>

#include "launch.hpp"
#include "score_core.hpp"
#include "select_core.hpp"

namespace idx {

enum : int { MODE_STORE = 0, MODE_FILTER = 1, MODE_SAMPLE = 2, MODE_ROWSTORE = 3 };

static_assert(kTieCapHost == kTieCap, "host and device tie-buffer capacities differ");

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kTile = 32;      // keys per MFMA block

// Rows per workgroup: 4 waves x RowsPerWave (contiguous kernel: 4 rows per wave for MXFP4
// at 32 heads, else 2); the paged kernel takes a row quad (see score_pages_kernel).
int rows_per_block(int heads, int fmt) { return 4 * (heads == 32 && fmt == FMT_MXFP4 ? 4 : 2); }
static int rows_per_block_paged(int) { return 4; }  // score_pages_kernel: one row quad
static int rows_per_block_for(const DevProblem& P) {
  return P.page_table ? rows_per_block_paged(P.heads) : rows_per_block(P.heads, P.fmt);
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
  // ROWSTORE
  int32_t only_row;
  // paged FILTER: persistent workgroups take their items after the first by this ticket
  int32_t* ticket;
};

struct TileWork {
  int32_t nrb;     // row blocks
  int32_t nchunk;  // position chunks per row block
  int32_t chunk;   // positions per chunk (multiple of kTile)
  int32_t spread;  // 1: every chunk's row blocks are dealt over all XCDs (keys private to a row block)
  int64_t total;   // nrb * nchunk
  int64_t grid;    // workgroups when each takes one item (the mapping's virtual grid)
};

// Workgroup b -> work item (item = chunk * nrb + row block), for b < W.grid.  Workgroups are
// dealt to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8.
//  - At least 8 chunks: chunk c runs on XCD c % 8, its row blocks back to back, so its keys
//    are fetched into that XCD's L2 once and the chunks near the start of the key range,
//    which short rows still reach, are spread over all XCDs.  Grid: ceil(nchunk / 8) * 8
//    * nrb workgroups.
//  - At least 8 chunks and spread (paged keys: a row block's keys are its own, so an XCD
//    gains nothing from holding whole chunks): item (c, j) runs on XCD (c + j) % 8.  Later
//    chunks hold less work (fewer rows reach them), and this keeps the XCDs' shares even.
//    The chunk groups are dealt last first.  Same grid.
//  - Fewer chunks: XCD x takes the x-th eighth of the items, so every XCD has work.  Grid:
//    8 * ceil(total / 8) workgroups.
__device__ __forceinline__ int64_t map_item(const TileWork& W, int64_t b) {
  const int64_t x = b & 7, local = b >> 3;
  if (W.nchunk < 8) return x * ((W.total + 7) / 8) + local;
  int64_t g = local / W.nrb;
  const int64_t j = local % W.nrb;
  if (!W.spread) return (g * 8 + x) * W.nrb + j;
  // Paged keys: chunk groups in reverse, so that the last chunks of the longest requests (few
  // items among many empty ones) start first and the dense first chunks fill the end.
  g = (W.nchunk + 7) / 8 - 1 - g;
  // Chunk c of group g gives XCD x its row blocks r0, r0 + 8, ... with r0 = (x - c) mod 8;
  // over the group's 8 chunks those are nrb items, taken chunk by chunk.
  int64_t rem = j;
  for (int i = 0; i < 8; ++i) {
    const int64_t c = g * 8 + i;
    const int64_t r0 = (x - c) & 7;
    const int64_t n = (W.nrb - r0 + 7) >> 3;
    if (rem < n) return c * W.nrb + r0 + 8 * rem;
    rem -= n;
  }
  return W.total;  // not reached: the group's counts add up to nrb
}

// ============================================================================= scoring core
//
// Two forms of the head reduce, one per operand format.
//
// e4m3 (and paged e4m3) keys: score = kscale * sum_h w_h max(x_h, 0), each ReLU an integer
// max on the bit pattern and each weighted term a VALU fma, in one fixed order per lane.
// The fp8 MFMA does not sum its products exactly in fp32: within each group of 8 products,
// terms far below the group's largest are dropped (measured: one 1.0 product with 2^-18
// products beside it keeps only the 2^-18 terms of the other groups).  A linear term
// computed on the matrix cores would carry that error in full, and cancelling it against
// sum_h w_h |x_h| turns it into an error of the score itself (it is not bounded by the
// score); the direct form has no such cancellation, and a key whose every head dot is
// negative scores exactly 0.
//
// MXFP4 keys: e2m1 products span few binades, so the fp4 and fp6 MFMAs are exact, and the
// ReLU is split to halve the VALU work.  Per (row, key):
//
//   score = kscale * (L + A),   A = sum_h (w_h / 2) |x_h|,   L = sum_h (w_h / 2) x_h,
//
// which equals kscale * sum_h w_h max(x_h, 0) because max(x, 0) = (x + |x|) / 2 (the 1/2
// rides on w, exactly).  A costs one VALU fma (abs source modifier) per head in the head
// reduce.  L is linear in the key: L = u . k with u = sum_h (w_h / 2) q_h, so it runs on
// the matrix cores.  u is split into
// kPieces fp6 (e2m3) vectors with e8m0 block scales: each piece takes the top 4
// significant bits of its block's largest residual, so the residual shrinks at least 16x
// per piece (below 2^-24 of the block maximum after six, the resolution of fp32 itself;
// exact for integer u).  One extra pair of MFMAs per tile multiplies up to two row pairs'
// pieces against the same key
// operand; fp6 runs at the fp4 MFMA rate.  Every kernel that produces a
// score for contiguous keys (materialised scores, samples, fused filter, fallback) runs
// wg_tiles() below, so a (row, key) always gets the same instruction sequence, the same
// MFMA row/column and the same summation order: the scores are bitwise identical.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

constexpr int kPieces = 6;
constexpr int kLinRowBytes = kPieces * 2 * 2 * 32;  // pieces x ksteps x halves x 32 bytes (24 used)
constexpr int kLinRowScales = kPieces * 2 * 2;

// Rows per wave of the contiguous kernel: 4 for MXFP4 at 32 heads (the linear tile then
// serves 4 rows and every key operand read from LDS feeds 8 MFMAs), otherwise 2 (register
// budget: e4m3 operands are twice as wide, 64 heads twice as many).
template <int FMT, int H>
struct RowsPerWave {
  static constexpr int value = (FMT == FMT_MXFP4 && H == 32) ? 4 : 2;
};

struct LinArgs {
  const uint8_t* q8;  // [rows][kPieces][2 ksteps][2 halves][32]: fp6 pieces of u, MFMA lane order
  const uint8_t* sf;  // [rows][kPieces][2][2]: e8m0 scale of hardware block (kstep, half)
};

// ---- preparation: u = sum_h w_h q_h and its pieces, one workgroup of 128 threads per row.
//
// gfx950 operand layouts of v_mfma_scale_f32_32x32x64_f8f6f4 (measured): fp4 and fp6 lanes
// hold K elements [32h, 32h + 32) of lane half h, element p at bits [bits*p, bits*(p+1));
// fp8 byte j of lane half h is K element 16h + j (j < 16) or 32 + 16h + (j - 16); the
// scale of lane half b covers K block [32b, 32b + 32).  MXFP4 keys are in hardware K
// order; e4m3 keys are loaded with byte j of half h = head_dim element 32h + j, i.e. K
// element k holds head_dim element kelem(k).  Piece element p of half h sits at K = 32h + p
// and must hold the head_dim element the key has there.
__device__ __forceinline__ int lin_elem(bool key_fp4, int h, int p) {
  const int k = 32 * h + p;
  if (key_fp4) return k;
  return k < 32 ? 32 * (k / 16) + k % 16 : 32 * ((k - 32) / 16) + 16 + (k - 32) % 16;
}

__device__ __forceinline__ float e2m1_value(int code) {
  const int e = (code >> 1) & 3, m = code & 1;
  const float v = e == 0 ? 0.5f * (float)m : ldexpf((float)(2 + m), e - 2);
  return (code & 8) ? -v : v;
}

__device__ __forceinline__ float e4m3_value(int b) {
  const int e = (b >> 3) & 15, m = b & 7;
  const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
  return (b & 0x80) ? -v : v;
}

// fp6 e2m3 (sign, 2-bit exponent with bias 1, 3-bit mantissa; subnormal step 1/8).
__device__ __forceinline__ float e2m3_value(int c) {
  const int e = (c >> 3) & 3, m = c & 7;
  const float v = e == 0 ? 0.125f * (float)m : ldexpf((float)(8 + m), e - 4);
  return (c & 0x20) ? -v : v;
}

// Round y (|y| < 4) to e2m3, nearest with ties to even; returns the 6-bit code.
__device__ __forceinline__ int e2m3_encode(float y) {
  const int sign = y < 0.0f ? 0x20 : 0;
  const float a = fabsf(y);
  if (a < 1.0f) {
    const int m = (int)__builtin_rintf(a * 8.0f);
    return sign | (m == 8 ? 0x08 : m);
  }
  if (a < 2.0f) {
    const int m = (int)__builtin_rintf((a - 1.0f) * 8.0f);
    return sign | (m == 8 ? 0x10 : 0x08 | m);
  }
  const int m = (int)__builtin_rintf((0.5f * a - 1.0f) * 8.0f);
  return sign | (m == 8 ? 0x18 : 0x10 | m);
}

template <int FMT, int H>
__global__ __launch_bounds__(128) void lin_prep_kernel(const uint8_t* q, const uint8_t* q_sf, const uint16_t* w,
                                                       int rows, bool key_fp4, uint8_t* lin_q8, uint8_t* lin_sf) {
  __shared__ float res[128];
  __shared__ float bmax[4];
  __shared__ uint32_t packed[kPieces][2][2][6];
  const int r = blockIdx.x;
  const int d = threadIdx.x;  // head_dim element
  float u = 0.0f;
  for (int h = 0; h < H; ++h) {
    const int64_t hv = (int64_t)r * H + h;
    float qd;
    if constexpr (FMT == FMT_E4M3) {
      qd = e4m3_value(q[hv * 128 + d]);
    } else {
      const int byte = q[hv * 64 + d / 2];
      qd = ldexpf(e2m1_value((d & 1) ? byte >> 4 : byte & 15), (int)q_sf[hv * 4 + d / 32] - 127);
    }
    u = __builtin_fmaf(bf16_to_f32(w[hv]), qd, u);
  }
  u *= 0.5f;  // the split form's 1/2 (exact)
  // Where element d sits in the pieces: kstep, lane half (= scale block) and position.
  const int ks = d / 64, e = d % 64;
  int hh = 0, pp = 0;
  for (int h = 0; h < 2; ++h)
    for (int p = 0; p < 32; ++p)
      if (lin_elem(key_fp4, h, p) == e) {
        hh = h;
        pp = p;
      }
  for (int i = d; i < kPieces * 2 * 2 * 6; i += 128) (&packed[0][0][0][0])[i] = 0;
  float rd = u;
  for (int c = 0; c < kPieces; ++c) {
    res[ks * 64 + hh * 32 + pp] = fabsf(rd);
    __syncthreads();
    if (d < 4) {
      float m = 0.0f;
      for (int p = 0; p < 32; ++p) m = fmaxf(m, res[d * 32 + p]);
      bmax[d] = m;
    }
    __syncthreads();
    const float m = bmax[ks * 2 + hh];
    int sexp = -127;  // block scale 2^sexp: the block maximum maps into [2, 4)
    if (m > 0.0f) {
      int ex;
      frexpf(m, &ex);
      sexp = max(-127, min(127, ex - 2));
    }
    const int code = e2m3_encode(ldexpf(rd, -sexp));
    rd -= ldexpf(e2m3_value(code), sexp);
    const int bit = 6 * pp;
    atomicOr(&packed[c][ks][hh][bit / 32], (uint32_t)code << (bit % 32));
    if (bit % 32 > 26) atomicOr(&packed[c][ks][hh][bit / 32 + 1], (uint32_t)code >> (32 - bit % 32));
    if (pp == 0) lin_sf[(((int64_t)r * kPieces + c) * 2 + ks) * 2 + hh] = (uint8_t)(sexp + 127);
    __syncthreads();
  }
  for (int i = d; i < kPieces * 2 * 2 * 8; i += 128) {
    const int c = i / 32, k2 = (i / 16) % 2, h2 = (i / 8) % 2, wd = i % 8;
    const uint32_t v = wd < 6 ? packed[c][k2][h2][wd] : 0u;
    reinterpret_cast<uint32_t*>(lin_q8)[((((int64_t)r * kPieces + c) * 2 + k2) * 2 + h2) * 8 + wd] = v;
  }
}

// ---- the wave-level tile routine

template <int FMT, int H>
__device__ __forceinline__ void mfma_row(v16f (&acc)[H / 32], const RowOperand<FMT, H>& ro, const KeyOperand& ko) {
  constexpr int C = Fmt<FMT>::kCode;
#pragma unroll
  for (int mt = 0; mt < H / 32; ++mt) {
    v16f a = {};
    // Scale operands carry both K-steps: the byte select picks K-step ks (byte ks of the
    // query word, byte 2 ks of the key word).
    a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ro.a[mt][0], ko.b[0], a, C, C, 0, ro.sa[mt], 0, ko.sb);
    a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ro.a[mt][1], ko.b[1], a, C, C, 1, ro.sa[mt], 2, ko.sb);
    acc[mt] = a;
  }
}

// Pieces of up to two row pairs of a wave as the A operand of the linear MFMA.  Lane l
// supplies M row (l % 32) = 8g + 4hh + j, which lands in accumulator s = 4g + j of lane
// half hh.  With p = s / kPieces and c = s % kPieces, accumulator s holds
//   c = 0: piece hh of row 2p      (the start value of row 2p's head sum, both halves),
//   c = 1: piece hh of row 2p + 1  (the start value of row 2p + 1's head sum),
//   c >= 2: piece c of row 2p + hh (the row whose score lane half hh receives after the
//           half-wave combine, added then),
// rows counted from row0.  So each row's six pieces reach its score with four adds.
struct LinOperand {
  v8i a[2];
  int sa;  // block scales of the two K-steps, byte ks
};

__device__ __forceinline__ void load_lin(LinOperand& lo, const LinArgs& L, int row0, int rows, int npairs) {
  const int l = lane_id();
  const int m = l & 31, half = l >> 5;
  const int s = 4 * (m >> 3) + (m & 3), hh = (m >> 2) & 1;
  const int p = s / kPieces, c = s % kPieces;
  const int row = row0 + 2 * p + (c == 1 ? 1 : c == 0 ? 0 : hh);
  const int piece = c < 2 ? hh : c;
  const bool ok = p < npairs && row < rows;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ok) {
      const int64_t base = (((int64_t)row * kPieces + piece) * 2 + ks) * 2 + half;
      const v4i x0 = *reinterpret_cast<const v4i*>(L.q8 + base * 32);
      const int2 x1 = *reinterpret_cast<const int2*>(L.q8 + base * 32 + 16);
      lo.a[ks] = v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, 0, 0};
    } else {
      lo.a[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if (ok) {
    const int64_t b0 = (((int64_t)row * kPieces + piece) * 2) * 2 + half;  // K-step 0; K-step 1 is b0 + 2
    lo.sa = (int)L.sf[b0] | ((int)L.sf[b0 + 2] << 8);
  } else {
    lo.sa = 0x7F7F;
  }
}

template <int FMT>
__device__ __forceinline__ v16f mfma_lin(const LinOperand& lo, const KeyOperand& ko) {
  constexpr int C = Fmt<FMT>::kCode;
  v16f a = {};
  a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lo.a[0], ko.b[0], a, 2, C, 0, lo.sa, 0, ko.sb);
  a = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lo.a[1], ko.b[1], a, 2, C, 1, lo.sa, 2, ko.sb);
  return a;
}

// Start value of row r's head sum on this lane half (pieces 0 and 1 of the row, one per
// half, so that the half-wave combine adds them).
__device__ __forceinline__ float lin_start(const v16f& a, int r) { return a[kPieces * (r / 2) + (r & 1)]; }

// Pieces 2.. of pair p's row on this lane half added to the combined head sum x, in order.
__device__ __forceinline__ float add_lin_rest(const v16f& a, int p, float x) {
#pragma unroll
  for (int c = 2; c < kPieces; ++c) x = x + a[kPieces * p + c];
  return x;
}

// The score as it is stored, appended or sampled: clamped at +0.  A sum of ReLU terms is
// never negative, but the split form can round a score whose exact value is 0 (every head
// dot <= 0) to a tiny negative number.  Integer max on the bit pattern: -0.0 and negative
// values become +0.0.  The filter compares unclamped scores against thresholds that are
// either > 0 or -inf, for which both forms give the same answer.
__device__ __forceinline__ float clamp0(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// max(x, 0) of a head dot in the direct form: an integer max on the bit pattern (one VALU
// instruction, no NaN canonicalisation; -0.0 becomes +0.0).
__device__ __forceinline__ float relu_bits(float x) { return clamp0(x); }

// Key tiles are staged through LDS: all four waves of a workgroup use the same keys, so a
// stage of 32-key tiles is fetched once per workgroup with 16-byte loads straight into LDS
// (issued one stage ahead, double-buffered, one barrier per stage) and each wave reads its
// MFMA key operands from LDS.  A stage is kept in regions of 32-byte rows, one region per
// 16-byte part that a lane half reads of a key for one MFMA operand: fp4 has one region per
// K-step, e4m3 two (the two 16-byte loads of a K-step).  Row k of a region holds that part
// for lane halves 0 and 1, swapped when g(k) = 1: a 16-byte read phase takes 8 (or 16)
// lanes, i.e. 8 (16) consecutive keys at one half, which this puts in distinct banks over
// 128 (256) bytes.  A stage is then a dense copy of its keys in another order, so a lane's
// load offset is the same in every stage, and every operand read of a lane sits a constant
// distance from its first.  A stage is 8 fp4 tiles or 4 e4m3 tiles (16 KB either way),
// which keeps two workgroups per CU within LDS.
template <int FMT>
struct StageGeom {
  static constexpr int kTiles = FMT == FMT_MXFP4 ? 8 : 4;  // tiles per stage
  static constexpr int kKB = Fmt<FMT>::kBytes;
  static constexpr int kKeys = kTiles * kTile;             // keys per stage
  static constexpr int kRow = 32;                          // bytes per region row
  static constexpr int kRegion = kKeys * kRow;             // bytes per region
  static constexpr int kBytes = kKeys * kKB;               // codes of one stage
  static constexpr int kStepOff = FMT == FMT_MXFP4 ? kRegion : 2 * kRegion;  // K-step 1 from 0
  static constexpr int kHalfBytes = FMT == FMT_MXFP4 ? 16 : 32;  // a lane half's bytes per K-step
  // Half swap of stage key k (k mod 16 decides: stage and tile starts are multiples of 16
  // keys).  Keys k and k + 4 of an 8-key phase share banks otherwise (32-byte rows over 128
  // bytes of banks), as do keys k and k + 8 of a 16-key phase over 256 bytes.
  static __device__ __forceinline__ int g(int k) { return ((k >> 2) ^ (k >> 3)) & 1; }
  // Byte offset of lane (col, half)'s first operand part within a tile.
  static __device__ __forceinline__ int lane_off(int col, int half) { return col * kRow + ((half ^ g(col)) * 16); }
  // Byte offset within a key's codes of the part that region R holds for lane half h.
  static __device__ __forceinline__ int part_off(int R, int h) {
    if constexpr (FMT == FMT_MXFP4) return R * 32 + h * 16;                       // K-step R
    else return (R >> 1) * 64 + h * 32 + (R & 1) * 16;                          // K-step R / 2
  }
  // Key and byte offset within it that 16-byte LDS slot sidx (>= 0) of a stage holds.
  static_assert((kKeys & (kKeys - 1)) == 0, "power-of-two stage");
  static __device__ __forceinline__ int slot_key(int sidx) { return (int)(((uint32_t)sidx % (2 * kKeys)) >> 1); }
  static __device__ __forceinline__ int slot_off(int sidx) {
    return part_off((int)((uint32_t)sidx / (2 * kKeys)), (sidx & 1) ^ g(slot_key(sidx)));
  }
};

template <int FMT>
struct StageLds {
  uint8_t* codes;  // [2][kBytes]
  uint32_t* sf;    // [2][kKeys] e8m0 words (MXFP4)
  float* ks;       // [2][kKeys] per-key scale (1.0 when absent)
  float* cand_s;   // FILTER: [waves][RW][kCandBuf] candidate scores of this workgroup's rows
  int32_t* cand_i; //         and their key indices relative to ks
  int32_t* pages;  // paged: kPageCache page ids of the call's key range (nullptr: read the table)
};

// Paged keys: page ids a score call touches are read from the page table once, into LDS,
// instead of before every stage's key loads.  2560 ids cover a 16384-key chunk, or 2048
// sample slots at the largest sample stride (71 keys apart).
constexpr int kPageCache = 2560;

// FILTER mode: each wave collects its candidates in an LDS buffer of its own (no LDS
// atomics) and moves them to the global slab in batches, with one global atomic per row
// and batch instead of one per tile (waves that share rows flush separately).
constexpr int kCandBuf = 256;

// Scores of the RW rows [row0, row0 + RW) of this wave on the workgroup's tiles [tA, tB)
// (positions: keys, or sample slots with key = phase + pos * S), with the epilogue of MODE.
// Every wave of the workgroup must call it with the same tA, tB.  Default: every wave has
// rows of its own and scores every tile that meets them.  SHARED: all waves hold the same
// rows and wave w scores tiles w and w + 4 of each stage (paged keys, the fallback); with
// split = 2 two waves share rows and take alternate tiles (slot = which of them).  rmask
// selects the rows that count (the others see no keys); req >= 0 reads keys through
// request req's page table, clamped to klim when given (else to this wave's rows' last
// visible key).  MODE_ROWSTORE writes only row E.only_row, to E.out[key - ks].
template <int FMT, int H, int MODE, int RW, bool SHARED, bool KS = true>
__device__ __forceinline__ void wg_tiles(const ScoreArgs& A, const LinArgs& L, const EpiArgs& E, int row0,
                                         int phase, int S, int c0, int c1, int tA, int tB,
                                         const StageLds<FMT>& sl, int req = -1, uint32_t rmask = ~0u,
                                         int split = 4, int slot = -1, int64_t klim = -1) {
  static_assert(RW % 2 == 0, "rows are processed in pairs");
  using G = StageGeom<FMT>;
  constexpr int KB = G::kKB;
  constexpr int NP = RW / 2;
  const int l = lane_id();
  const int half = l >> 5, col = l & 31;
  const int wave = uniform(threadIdx.x / kWave);

  int plo[RW], phi[RW], ksr[RW];
  int wlo = 0x7FFFFFFF, whi = 0, full_lo = 0, full_hi = 0x7FFFFFFF;
  int lmax = 0;  // paged: largest logical key any active row sees
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = row0 + i;
    plo[i] = phi[i] = ksr[i] = 0;
    if (r < A.rows && ((rmask >> i) & 1)) {
      const int ks = uniform(A.ks[r]), ke = uniform(A.ke[r]);
      lmax = max(lmax, ke - 1);
      ksr[i] = ks;
      if (MODE == MODE_SAMPLE) {
        if (ke - ks > E.skip_le) sample_range(ks, ke, phase, S, plo[i], phi[i]);
      } else {
        plo[i] = ks;
        phi[i] = ke;
        // stored scores stay inside the row pitch (the caller's, or the fallback's scratch
        // row) whatever the device-side range
        if ((MODE == MODE_STORE || MODE == MODE_ROWSTORE) && (int64_t)ke - ks > E.ld) phi[i] = ks + (int)E.ld;
      }
    }
    if (phi[i] > plo[i]) {
      wlo = min(wlo, plo[i]);
      whi = max(whi, phi[i]);
    }
    full_lo = max(full_lo, plo[i]);
    full_hi = min(full_hi, phi[i]);
  }
  const int wt0 = max(c0, wlo) / kTile, wt1 = (min(c1, whi) + kTile - 1) / kTile;  // this wave's tiles

  RowOperand<FMT, H> ro[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i)
    if (row0 + i < A.rows) load_row<FMT, H>(ro[i], A, row0 + i);
  constexpr bool kSplit = SplitRelu<FMT>::value;
  LinOperand lo;
  if constexpr (kSplit) load_lin(lo, L, row0, A.rows, NP);

  float thr_l[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int i = 2 * p + half;
    thr_l[p] = 0.0f;
    if (MODE == MODE_FILTER && row0 + i < A.rows) thr_l[p] = E.thr[row0 + i];
  }
  // Per-lane value of pair p (row 2p on lanes 0-31, row 2p + 1 on lanes 32-63), formed where
  // it is used from the wave-uniform per-row values, so that it holds no VGPR across the
  // tile loop (the empty asm keeps the select from being hoisted out of the loop).
  auto lane_pair = [&](const int (&v)[RW], int p) -> int {
    int a = v[2 * p], b = v[2 * p + 1];
    asm volatile("" : "+v"(a), "+v"(b));
    return half ? b : a;
  };
  auto row_of = [&](int p) -> int64_t { return (int64_t)row0 + 2 * p + half; };
  const int64_t last_key = A.num_keys - 1;
  // Physical key of stage position pos: contiguous keys are clamped to the key array;
  // paged keys (all rows of request `req`) are clamped to the rows' visible range, then
  // mapped through the request's page table (64 keys per page).
  // Page ids outside the key array (invalid input) are clamped so reads stay inside K.
  const int32_t last_page = (int32_t)(A.num_keys / kPage) - 1;
  auto valid_page = [&](int32_t id) -> int32_t { return id < 0 ? 0 : (id > last_page ? last_page : id); };
  // Paged: cache the page ids of every logical key the stage loads can reach (positions
  // [tA * kTile, tA * kTile + nst * kKeys), clamped to lmax like key_of) when they fit.
  int64_t pg_lo = 0;
  bool pg_cached = false;
  if (klim >= 0) lmax = (int)klim;  // the workgroup's key limit (waves with different rows)
  if (req >= 0) {  // logical keys past the page table (ke beyond max_pages pages) stay inside it
    const int64_t table_keys = (int64_t)A.max_pages * kPage - 1;
    lmax = lmax < table_keys ? lmax : (int)table_keys;
  }
  if (req >= 0 && sl.pages) {
    const int64_t nst_keys = (int64_t)((tB - tA + G::kTiles - 1) / G::kTiles) * G::kKeys;
    int64_t k_first = (int64_t)phase + (int64_t)tA * kTile * S;
    int64_t k_last = (int64_t)phase + ((int64_t)tA * kTile + nst_keys - 1) * S;
    k_first = k_first < lmax ? k_first : lmax;
    k_last = k_last < lmax ? k_last : lmax;
    pg_lo = k_first >> 6;
    const int64_t npg = (k_last >> 6) - pg_lo + 1;
    pg_cached = npg <= kPageCache;  // workgroup-uniform
    if (pg_cached) {
      for (int64_t j = threadIdx.x; j < npg; j += kThreads)
        sl.pages[j] = valid_page(A.page_table[(int64_t)req * A.max_pages + pg_lo + j]);
      __syncthreads();
    }
  }
  auto key_of = [&](int64_t pos) -> int64_t {
    const int64_t key = (int64_t)phase + pos * S;
    if (req < 0) return key < last_key ? key : last_key;
    const int64_t lk = key < lmax ? key : lmax;
    const int64_t page = lk >> 6;
    const int32_t id = pg_cached ? sl.pages[page - pg_lo] : valid_page(A.page_table[(int64_t)req * A.max_pages + page]);
    return (int64_t)id * kPage + (lk & (kPage - 1));
  };

  // FILTER: this wave's LDS candidate buffers and their (wave-uniform) fill counts.
  float* cs = MODE == MODE_FILTER ? sl.cand_s + wave * RW * kCandBuf : nullptr;
  int32_t* ci = MODE == MODE_FILTER ? sl.cand_i + wave * RW * kCandBuf : nullptr;
  int ccnt[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) ccnt[i] = 0;
  // Move row i's buffered candidates to the slab: one atomic reserves the slots; slots at
  // or past cap are dropped but still counted (the count then flags the overflow).
  auto flush = [&](int i) {
    const int n = ccnt[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int base = 0;
    if (l == 0) base = atomicAdd(&E.cnt[row0 + i], n);
    base = readlane(base, 0);
    const int64_t row_off = (int64_t)(row0 + i) * E.cap;
    for (int j = l; j < n; j += kWave) {
      const int slot = base + j;
      if (slot < E.cap) {
        E.slab_s[row_off + slot] = cs[i * kCandBuf + j];
        E.slab_i[row_off + slot] = ci[i * kCandBuf + j];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    ccnt[i] = 0;
  };

  // Epilogue of one tile for every row pair, given the pairs' packed scores.
  auto epilogue = [&](int t, const float* score_of, bool known_full) {
    const int pos = t * kTile + col;
    const int64_t key = (int64_t)phase + (int64_t)pos * S;
    const bool full = known_full || (t * kTile >= full_lo && (t + 1) * kTile <= full_hi);  // wave-uniform
    if constexpr (MODE == MODE_FILTER) {
      // One compare and ballot per row pair; the append path runs only for the (rare)
      // tiles that hold a candidate.
      uint64_t m[NP];
      uint64_t any = 0;
      if (full) {
#pragma unroll
        for (int p = 0; p < NP; ++p) m[p] = wave_ballot(score_of[p] >= thr_l[p]);
      } else {
#pragma unroll
        for (int p = 0; p < NP; ++p)
          m[p] = wave_ballot(pos >= lane_pair(plo, p) && pos < lane_pair(phi, p) && score_of[p] >= thr_l[p]);
      }
#pragma unroll
      for (int p = 0; p < NP; ++p) any |= m[p];
      if (any) {  // wave-uniform
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (!m[p]) continue;  // wave-uniform
          const int nA = __builtin_popcountll(m[p] & 0xFFFFFFFFull), nB = __builtin_popcountll(m[p] >> 32);
          if ((m[p] >> l) & 1) {
            const int slot = (half ? ccnt[2 * p + 1] - nA : ccnt[2 * p]) + mask_prefix(m[p]);
            const int o = (2 * p + half) * kCandBuf + slot;
            cs[o] = clamp0(score_of[p]);
            ci[o] = (int32_t)(key - lane_pair(ksr, p));
          }
          ccnt[2 * p] += nA;
          ccnt[2 * p + 1] += nB;
          // A row gains at most kTile candidates per tile: flush before the next could overflow.
          if (ccnt[2 * p] > kCandBuf - kTile) flush(2 * p);
          if (ccnt[2 * p + 1] > kCandBuf - kTile) flush(2 * p + 1);
        }
      }
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float score = clamp0(score_of[p]);
        const bool valid = full || (pos >= lane_pair(plo, p) && pos < lane_pair(phi, p));
        if constexpr (MODE == MODE_STORE) {
          if (valid) E.out[row_of(p) * E.ld + (key - lane_pair(ksr, p))] = score;
        } else if constexpr (MODE == MODE_ROWSTORE) {
          if (valid && row_of(p) == E.only_row) E.out[key - lane_pair(ksr, p)] = score;
        } else {
          if (valid) E.samp[row_of(p) * E.ns + pos] = score;
        }
      }
    }
  };


  // Key operand and half key scale of tile slot i of LDS stage buffer `buf`.
  // This lane's LDS addresses in stage buffer `buf` (codes of key `col` at this lane
  // half's K offset, its block-scale word and key scale), made opaque to the compiler so
  // that each tile's reads use the tile's constant offset from them instead of a register
  // per tile.
  typedef const __attribute__((address_space(3))) uint8_t* lds_ptr;
  struct StageBase {
    lds_ptr codes, sf, ks;
  };
  auto stage_base = [&](int buf) -> StageBase {
    auto opaque = [](const void* p) -> lds_ptr {
      uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
      asm volatile("" : "+v"(a));
      return (lds_ptr)(uintptr_t)a;
    };
    return StageBase{opaque(sl.codes + buf * G::kBytes + G::lane_off(col, half)),
                     opaque(sl.sf + buf * G::kKeys + col), opaque(sl.ks + buf * G::kKeys + col)};
  };
  // Key operand and half key scale of tile slot i of the stage at `sb`.
  auto read_b = [&](const StageBase& sb, int i, KeyOperand& ko, float& kscale) {
    lds_ptr row = sb.codes + i * kTile * G::kRow;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (FMT == FMT_E4M3) {
        const v4i x0 = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(row + ks * G::kStepOff);
        const v4i x1 = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(row + ks * G::kStepOff + G::kRegion);
        ko.b[ks] = v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      } else {
        const v4i x = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(row + ks * G::kStepOff);
        ko.b[ks] = v8i{x.x, x.y, x.z, x.w, 0, 0, 0, 0};
      }
    }
    if constexpr (FMT == FMT_MXFP4) {
      // The key's four block scales, shifted so that bytes 0 and 2 hold this lane half's
      // blocks of K-steps 0 and 1.
      const uint32_t sw = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(sb.sf + i * kTile * 4);
      ko.sb = (int)(sw >> (8 * half));
    } else {
      ko.sb = 0x7F7F7F7F;
    }
    // Without key scales the LDS words hold 1.0 (written once, before the first stage).
    kscale = *reinterpret_cast<const __attribute__((address_space(3))) float*>(sb.ks + i * kTile * 4);
  };
  struct Acc {
    v16f row[RW][H / 32];
    v16f lin;
  };
  auto issue = [&](Acc& a, const KeyOperand& ko) {
    if constexpr (kSplit) a.lin = mfma_lin<FMT>(lo, ko);
#pragma unroll
    for (int r = 0; r < RW; ++r) mfma_row<FMT, H>(a.row[r], ro[r], ko);
  };
  // Head reduce of all RW rows, the rows' chains interleaved for instruction-level
  // parallelism.  Each row's own sum runs over its heads in one fixed order.
  // term(x): |x| (split form) or max(x, 0) (direct form).
  auto term = [](float x) -> float {
    if constexpr (kSplit) return __builtin_fabsf(x);
    else return relu_bits(x);
  };
  auto reduce = [&](const Acc& a, float kscale_f, float* sc) {
    float part[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if constexpr (kSplit) part[r] = lin_start(a.lin, r);
      else part[r] = 0.0f;
    }
#pragma unroll
    for (int mt = 0; mt < H / 32; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int r = 0; r < RW; ++r)
          part[r] = __builtin_fmaf(ro[r].w[mt][i], term(a.row[r][mt][i]), part[r]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float hs = combine_halves(part[2 * p], part[2 * p + 1]);
      // KS = false: no key scales (every factor 1.0, so the product is skipped, not changed)
      if constexpr (kSplit) sc[p] = KS ? add_lin_rest(a.lin, p, hs) * kscale_f : add_lin_rest(a.lin, p, hs);
      else sc[p] = KS ? hs * kscale_f : hs;
    }
  };
  // One tile: key operand from LDS, MFMAs for all RW rows and the linear tile, reduce, epilogue.
  auto compute = [&](const StageBase& sb, int i, int t, bool known_full) {
    KeyOperand ko;
    float ksc;
    read_b(sb, i, ko, ksc);
    Acc a;
    issue(a, ko);
    float sc[NP];
    reduce(a, ksc, sc);
    epilogue(t, sc, known_full);
  };

  // Stage loads straight into LDS (global_load_lds_dwordx4): lane l of wave w writes the 16
  // bytes it fetches to the wave's LDS base + 16 l, so each lane is given the global piece
  // that belongs in its 16-byte slot of the stage layout (G::slot_key, G::slot_off).
  // Block scales and key scales come by 4-byte loads.
  constexpr int kSlots = G::kBytes / 16;
  constexpr int kSlotIters = (kSlots + kThreads - 1) / kThreads;
  const bool has_ks = A.k_scale != nullptr;
  // LDS destination of a stage load, as an address the compiler cannot trace to a variable.
  auto lds_dst = [](const void* p) -> __attribute__((address_space(3))) void* {
    uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
    asm volatile("" : "+s"(a));
    return (__attribute__((address_space(3))) void*)(uintptr_t)a;
  };
  const bool fits32 = (int64_t)phase + ((int64_t)tB + G::kTiles) * kTile * S < 0x7FFFFFFF;
  auto dma = [&](int stage, int buf) {
    const int64_t pos0 = (int64_t)(tA + stage * G::kTiles) * kTile;
    uint8_t* lbase = sl.codes + buf * G::kBytes;
    int ln = l;
    // Paged and sampled stages: the lane-derived slot offsets are recomputed per stage
    // rather than held in registers, which the 64-head paged and the 4-row sample kernels
    // would otherwise spill.
    if constexpr (SHARED || MODE == MODE_SAMPLE) asm volatile("" : "+v"(ln));
    {
      // Paged with the page ids in LDS: key_of in 32-bit arithmetic when every position the
      // stages reach, times the stride, stays below 2^31.
      if (req >= 0 && pg_cached && fits32) {  // wave-uniform
        const int kpos0 = (int)pos0, pbase = (int)pg_lo;
        // Load u fills region u kThreads / (2 kKeys) for the run of 128 stage keys starting at
        // (u kThreads mod 2 kKeys) / 2, and this lane's slot there holds stage key
        // run + kq, half h: the page lookup is made once per run (one for e4m3, two for fp4)
        // and the loads differ only in the part.
        static_assert(kSlots == 4 * kThreads && 2 * G::kKeys % kThreads == 0, "whole regions per load");
        constexpr int kRuns = 2 * G::kKeys / kThreads;
        const int kq = wave * (kWave / 2) + (ln >> 1);
        const int h = (ln & 1) ^ G::g(kq);
        const uint8_t* src[kRuns];
#pragma unroll
        for (int j = 0; j < kRuns; ++j) {
          const int key = min(phase + (kpos0 + j * (kThreads / 2) + kq) * S, lmax);
          const int32_t id = sl.pages[(key >> 6) - pbase];
          src[j] = A.k + (int64_t)id * (kPage * KB) + (key & (kPage - 1)) * KB;
        }
#pragma unroll
        for (int u = 0; u < kSlotIters; ++u) {
          constexpr int kRegionSlots = 2 * G::kKeys;
          const int R = u * kThreads / kRegionSlots, j = (u * kThreads % kRegionSlots) / kThreads;
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[j] + G::part_off(R, h)),
                                           lds_dst(lbase + (u * kThreads + wave * kWave) * 16), 16, 0, 0);
        }
        if (wave * kWave < G::kKeys) {
          const int key = min(phase + (kpos0 + wave * kWave + ln) * S, lmax);
          const int64_t g = (int64_t)sl.pages[(key >> 6) - pbase] * kPage + (key & (kPage - 1));
          if constexpr (FMT == FMT_MXFP4)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A.k_sf + g * 4),
                                             lds_dst(sl.sf + buf * G::kKeys + wave * kWave), 4, 0, 0);
          if (has_ks)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A.k_scale + g),
                                             lds_dst(sl.ks + buf * G::kKeys + wave * kWave), 4, 0, 0);
        }
        return;
      }
    }
    if constexpr (MODE != MODE_SAMPLE && !SHARED) {  // not strided sample positions, not paged keys
      // Contiguous keys with the whole stage inside the key array: the stage holds the codes
      // of kKeys consecutive keys, so a lane's source is the stage's first key plus an offset
      // of its own.  Load u fills region u * kThreads / (2 kKeys) for a run of 128 keys; a
      // wave's 64 slots there are 32 whole keys, 16-key aligned, so the half swap depends on
      // the lane alone.  The lane offset is formed anew in each stage (no register held
      // across the tile loop) and added to a wave-uniform base.
      const int64_t kfirst = (int64_t)phase + pos0;
      if (req < 0 && S == 1 && kfirst + G::kKeys - 1 <= last_key) {  // wave-uniform
        static_assert(kSlots == 4 * kThreads && 2 * G::kKeys % kThreads == 0, "whole regions per load");
        int lv = l;
        asm volatile("" : "+v"(lv));
        const int kq = lv >> 1;
        const uint32_t loff = (uint32_t)(kq * KB + ((lv & 1) ^ G::g(kq)) * G::kHalfBytes);
        const uint8_t* gb = A.k + kfirst * KB + wave * (kWave / 2) * KB;
#pragma unroll
        for (int u = 0; u < kSlotIters; ++u) {
          constexpr int kRegionSlots = 2 * G::kKeys;
          const int R = u * kThreads / kRegionSlots, kb = (u * kThreads % kRegionSlots) / 2;
          const uint32_t ucst = (uint32_t)(kb * KB + G::part_off(R, 0));
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(gb + (loff + ucst)),
                                           lds_dst(lbase + (u * kThreads + wave * kWave) * 16), 16, 0, 0);
        }
        if (G::kKeys >= kThreads || wave * kWave < G::kKeys) {  // wave-uniform (every wave's for fp4)
          const int64_t gk = kfirst + wave * kWave;
          if constexpr (FMT == FMT_MXFP4)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A.k_sf + gk * 4 + (uint32_t)(lv * 4)),
                                             lds_dst(sl.sf + buf * G::kKeys + wave * kWave), 4, 0, 0);
          if (has_ks)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A.k_scale + gk + (uint32_t)lv),
                                             lds_dst(sl.ks + buf * G::kKeys + wave * kWave), 4, 0, 0);
        }
        return;
      }
    }
#pragma unroll
    for (int u = 0; u < kSlotIters; ++u) {
      const int s0 = u * kThreads + wave * kWave;
      if (s0 < kSlots) {  // wave-uniform
        const int sidx = s0 + ln;
        const uint8_t* src = A.k + key_of(pos0 + G::slot_key(sidx)) * KB + G::slot_off(sidx);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         lds_dst(lbase + s0 * 16), 16, 0, 0);
      }
    }
    if (wave * kWave < G::kKeys) {  // wave-uniform
      const int key = wave * kWave + l;
      const int64_t g = key_of(pos0 + key);
      if constexpr (FMT == FMT_MXFP4)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A.k_sf + g * 4),
                                         lds_dst(sl.sf + buf * G::kKeys + wave * kWave),
                                         4, 0, 0);
      if (has_ks)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A.k_scale + g),
                                         lds_dst(sl.ks + buf * G::kKeys + wave * kWave),
                                         4, 0, 0);
    }
  };

  const int nst = (tB - tA + G::kTiles - 1) / G::kTiles;
  if (!has_ks)  // workgroup-uniform: key scale 1.0 in both stage buffers (no load writes them)
    for (int j = threadIdx.x; j < 2 * G::kKeys; j += kThreads) sl.ks[j] = 1.0f;
  dma(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) dma(st + 1, buf ^ 1);
    const int tbase = tA + st * G::kTiles;
    const StageBase sbase = stage_base(buf);
    bool whole = false;  // wave-uniform: every tile of the stage is this wave's and inside all its rows
    // A second copy of the tile loop: 4-row kernels, and the 2-row FILTER kernels (the
    // 2-row STORE and SAMPLE kernels would spill).  Shared rows (paged keys) with two waves
    // per row pair: each wave's tiles i = slot, slot + 2, ... of the stage.
    constexpr bool kWhole = RW >= 4 || MODE == MODE_FILTER;
    constexpr int kStep = SHARED ? 2 : 1;
    if constexpr (kWhole)
      whole = (SHARED ? split == 2 && slot >= 0 : (tbase >= wt0 && tbase + G::kTiles <= min(wt1, tB))) &&
              tbase + G::kTiles <= tB && tbase * kTile >= full_lo && (tbase + G::kTiles) * kTile <= full_hi;
    if (whole) {
      if constexpr (kWhole) {
        // The next tile's key operand is read from LDS once this tile's MFMAs are issued
        // (into the registers they have just read), so the LDS latency runs under this
        // tile's head reduce instead of stalling the next tile's MFMAs.
        const int i0 = SHARED ? slot : 0;
        // Pins the loop's code to an 8-byte boundary: the MXFP4 filter loop ran 1.3 % slower
        // with its code 4 bytes off this placement (every offset measured), the e4m3 loops
        // showed no difference.  Costs at most one s_nop per stage.
        asm volatile(".p2align 3");
        KeyOperand ko;
        float ksc;
        read_b(sbase, i0, ko, ksc);
#pragma unroll
        for (int j = 0; j < G::kTiles / kStep; ++j) {
          const int i = i0 + kStep * j;
          Acc a;
          issue(a, ko);
          const float ksc_i = ksc;
          if (j + 1 < G::kTiles / kStep) read_b(sbase, i + kStep, ko, ksc);
          float sc[NP];
          reduce(a, ksc_i, sc);
          epilogue(tbase + i, sc, true);
        }
      }
    } else if constexpr (kWhole) {
      // With the whole-stage loop above, the stages that reach this loop (a chunk's first and
      // last, and where rows end) are few: rolled, it keeps one copy of the tile code and its
      // candidate flushes instead of kTiles, a third of the kernel's code.
#pragma nounroll
      for (int i = 0; i < G::kTiles; ++i) {
        const int t = tbase + i;
        if (t >= tB) break;  // workgroup-uniform
        const bool mine = SHARED ? ((i % split) == (slot < 0 ? wave : slot)) : (t >= wt0 && t < wt1);
        if (mine) compute(sbase, i, t, false);
      }
    } else {
#pragma unroll
      for (int i = 0; i < G::kTiles; ++i) {
        const int t = tbase + i;
        if (t >= tB) break;  // workgroup-uniform
        const bool mine = SHARED ? ((i % split) == (slot < 0 ? wave : slot)) : (t >= wt0 && t < wt1);
        if (mine) compute(sbase, i, t, false);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next stage
    __syncthreads();
  }
  if constexpr (MODE == MODE_FILTER) {
#pragma unroll
    for (int i = 0; i < RW; ++i)
      if (ccnt[i] > 0) flush(i);
  }
}

template <int FMT>
struct StageShared {
  __attribute__((aligned(16))) uint8_t codes[2 * StageGeom<FMT>::kBytes];
  uint32_t sf[2 * StageGeom<FMT>::kKeys];
  float ks[2 * StageGeom<FMT>::kKeys];
};

// Candidate buffers of the 4 waves (FILTER mode only).
template <int RW, bool ON>
struct CandShared {
  float s[4 * RW * kCandBuf];
  int32_t i[4 * RW * kCandBuf];
};
template <int RW>
struct CandShared<RW, false> {
  float s[1];
  int32_t i[1];
};

template <int FMT, int H, int MODE, bool KS>
__global__ __launch_bounds__(kThreads, 2) void score_tiles_kernel(ScoreArgs A, LinArgs L, EpiArgs E, TileWork W) {
  constexpr int RW = RowsPerWave<FMT, H>::value;
  __shared__ StageShared<FMT> sh;
  __shared__ CandShared<RW, MODE == MODE_FILTER> cand;
  const int64_t item = map_item(W, blockIdx.x);
  if (item >= W.total) return;
  const int rb = (int)(item % W.nrb);
  const int chunk = (int)(item / W.nrb);
  const int wave = uniform(threadIdx.x / kWave);
  const int S = (MODE == MODE_SAMPLE) ? E.stride : 1;
  const int phase = (MODE == MODE_SAMPLE) ? sample_phase(rb, S) : 0;
  const int c0 = chunk * W.chunk, c1 = c0 + W.chunk;
  // Tiles of the workgroup: the union of all its rows' ranges within the chunk.
  int lo = 0x7FFFFFFF, hi = 0;
  for (int r = rb * 4 * RW; r < min(A.rows, (rb + 1) * 4 * RW); ++r) {
    const int ks = uniform(A.ks[r]), ke = uniform(A.ke[r]);
    int plo = ks, phi = ke;
    if (MODE == MODE_SAMPLE) {
      plo = phi = 0;
      if (ke - ks > E.skip_le) sample_range(ks, ke, phase, S, plo, phi);
    }
    if (phi > plo) {
      lo = min(lo, plo);
      hi = max(hi, phi);
    }
  }
  const int tA = max(c0, lo) / kTile, tB = (min(c1, hi) + kTile - 1) / kTile;
  if (tA >= tB) return;  // workgroup-uniform
  const StageLds<FMT> sl{sh.codes, sh.sf, sh.ks, cand.s, cand.i};
  wg_tiles<FMT, H, MODE, RW, false, KS>(A, L, E, rb * 4 * RW + wave * RW, phase, S, c0, c1, tA, tB, sl);
}

// Request of a paged row, clamped to [0, num_req) so an invalid id cannot read outside
// the page table.
__device__ __forceinline__ int request_of(const ScoreArgs& A, int r) {
  const int q = A.row_req[r];
  return q < 0 ? 0 : (q >= A.num_req ? A.num_req - 1 : q);
}

// Paged keys: one work item per (row quad, key chunk).  Rows must read one request's pages
// to share the LDS stage.  When all four rows belong to one request (MTP decode rows), the
// two row pairs share each stage: waves 0/1 hold the pairs and take even tiles, waves 2/3
// the odd ones.  Otherwise each pair is scored on its own with all four waves holding it,
// and a pair that straddles two requests in two one-row passes.
// The FILTER launch with a ticket counter runs persistent workgroups (two per CU): each
// takes item map_item(b) for its own index b first, then b = grid size + the ticket it drew
// while scoring the previous item, until b reaches the virtual grid.  Every b is taken
// once, empty items (chunks past every row's keys, most of a decode batch) cost a loop
// turn instead of a workgroup launch, and the workgroups that finish early take the
// remaining items.
template <int FMT, int H, int MODE>
__global__ __launch_bounds__(kThreads, 2) void score_pages_kernel(ScoreArgs A, LinArgs L, EpiArgs E, TileWork W) {
  __shared__ StageShared<FMT> sh;
  __shared__ CandShared<2, MODE == MODE_FILTER> cand;
  __shared__ int32_t pages[kPageCache];
  __shared__ int sh_next;
  const bool persistent = MODE == MODE_FILTER && E.ticket != nullptr;
  for (int64_t b = blockIdx.x; b < W.grid;) {  // workgroup-uniform
    int next = 0;
    // drawn now and used after the item, so that the atomic's round trip hides under it
    if (persistent && threadIdx.x == 0) next = atomicAdd(E.ticket, 1);
    const int64_t item = map_item(W, b);
    if (item < W.total) {
      const int rb = (int)(item % W.nrb);
      const int chunk = (int)(item / W.nrb);
      const int base = 4 * rb;
      const int S = (MODE == MODE_SAMPLE) ? E.stride : 1;
      const int phase = (MODE == MODE_SAMPLE) ? sample_phase(rb, S) : 0;
      const int c0 = chunk * W.chunk, c1 = c0 + W.chunk;
      const int wave = uniform(threadIdx.x / kWave);
      const StageLds<FMT> sl{sh.codes, sh.sf, sh.ks, cand.s, cand.i, pages};
      // Tile range of the given rows within the chunk (positions: keys or sample slots).
      auto span = [&](int r0, int n, uint32_t rmask, int& tA, int& tB, int& kmax) {
        int lo = 0x7FFFFFFF, hi = 0;
        kmax = 0;
        for (int i = 0; i < n; ++i) {
          const int r = r0 + i;
          if (r >= A.rows || !((rmask >> i) & 1)) continue;
          const int ks = A.ks[r], ke = A.ke[r];
          kmax = max(kmax, ke - 1);
          int plo = ks, phi = ke;
          if (MODE == MODE_SAMPLE) {
            plo = phi = 0;
            if (ke - ks > E.skip_le) sample_range(ks, ke, phase, S, plo, phi);
          }
          if (phi > plo) {
            lo = min(lo, plo);
            hi = max(hi, phi);
          }
        }
        tA = max(c0, lo) / kTile;
        tB = (min(c1, hi) + kTile - 1) / kTile;
      };
      const int nr = min(4, A.rows - base);
      bool one_req = nr == 4;
      for (int i = 1; i < nr && one_req; ++i) one_req = request_of(A, base + i) == request_of(A, base);
      if (one_req) {
        int tA, tB, kmax;
        span(base, 4, 0xFu, tA, tB, kmax);
        if (tA < tB)
          wg_tiles<FMT, H, MODE, 2, true>(A, L, E, base + 2 * (wave & 1), phase, S, c0, c1, tA, tB, sl,
                                          request_of(A, base), ~0u, 2, wave >> 1, kmax);
      } else {
        for (int pr = 0; pr < 2; ++pr) {  // workgroup-uniform
          const int row0 = base + 2 * pr;
          if (row0 >= A.rows) break;
          const bool two = row0 + 1 < A.rows;
          const int q0 = request_of(A, row0), q1 = two ? request_of(A, row0 + 1) : q0;
          for (int pass = 0; pass < (q0 == q1 ? 1 : 2); ++pass) {
            const uint32_t rmask = q0 == q1 ? 3u : (1u << pass);
            int tA, tB, kmax;
            span(row0, 2, rmask, tA, tB, kmax);
            if (tA < tB)
              wg_tiles<FMT, H, MODE, 2, true>(A, L, E, row0, phase, S, c0, c1, tA, tB, sl, pass == 0 ? q0 : q1,
                                              rmask);
            __syncthreads();
          }
        }
      }
    }
    if (!persistent) break;
    if (threadIdx.x == 0) sh_next = next;
    __syncthreads();  // (also: the item's LDS is free for the next)
    b = (int64_t)gridDim.x + sh_next;
    __syncthreads();
  }
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

// Two shapes of the threshold kernel.  Rows with many samples (long contexts): 1024-thread
// workgroups whose threads keep their up to kThrStage / 1024 = 15 sample keys in registers
// (every pass visits a thread's own samples j = thread + 1024 e), so the samples are read
// from memory once instead of once per pass.  Rows with few samples: 256-thread workgroups,
// many per CU.  Rows with more samples than the registers hold read them from global memory
// on every pass.
template <int kThrThreads, int kThrStage>
__global__ __launch_bounds__(kThrThreads) void threshold_kernel(ThrArgs T) {
  __shared__ SelSmemT<64> sm;  // histogram and scan scratch only
  constexpr int PER = kThrStage > 0 ? (kThrStage + kThrThreads - 1) / kThrThreads : 1;
  uint32_t kv[PER];  // this thread's sample keys j = thread + kThrThreads e (staged rows)
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x < kStatSlots) T.stats[threadIdx.x] = (threadIdx.x == kStatMin) ? 0x7FFFFFFF : 0;
  if (r == 0 && threadIdx.x < kFbCtrlWords) T.fb_ctrl[threadIdx.x] = 0;
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
      // Rank m = ceil(2.25 * k * n / V), so that ~2.25k keys pass.  The threshold is the
      // lower edge of the m-th largest sample's bin at 24 bits of the sample keys
      // normalised over [min, max]: a min/max pass, then two 12-bit histogram passes (the
      // second over the first boundary bin only).  A lower bound of that sample that adds
      // the keys of one fine bin; the second level keeps the bin fine when a few far
      // larger samples stretch the range.
      int64_t m = ((int64_t)9 * T.k * n + 4 * (int64_t)V - 1) / (4 * (int64_t)V);
      if (m < 1) m = 1;
      if (m > n) m = n;
      const float* sp = T.samp + (int64_t)r * T.ns + jlo;
      if (threadIdx.x == 0) {
        sm.kmin = 0xFFFFFFFFu;
        sm.kmax = 0u;
      }
      zero_hist<kThrThreads>(sm, kHistBins);
      __syncthreads();
      // The min/max pass reads the samples once; when they fit, their order keys stay in
      // registers for the two histogram passes.
      const bool staged = n <= kThrStage;  // workgroup-uniform (never for kThrStage == 0)
      uint32_t lo = 0xFFFFFFFFu, hi = 0u;
      if constexpr (kThrStage > 0) {
        if (staged) {
          // Every load of the pass issued before any is used: one memory round trip.
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int j = (int)threadIdx.x + e * kThrThreads;
            kv[e] = order_key(sp[j < n ? j : n - 1]);  // unconditional (n >= 1): no branch per load
          }
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            if ((int)threadIdx.x + e * kThrThreads < n) {
              lo = min(lo, kv[e]);
              hi = max(hi, kv[e]);
            }
          }
        }
      }
      if (!staged) {
#pragma unroll 4
        for (int j = threadIdx.x; j < n; j += kThrThreads) {
          const uint32_t k = order_key(sp[j]);
          lo = min(lo, k);
          hi = max(hi, k);
        }
      }
      // f(key) for each of this thread's samples
      auto each_key = [&](auto&& f) __attribute__((always_inline)) {
        if constexpr (kThrStage > 0) {
          if (staged) {
#pragma unroll
            for (int e = 0; e < PER; ++e)
              if ((int)threadIdx.x + e * kThrThreads < n) f(kv[e]);
            return;
          }
        }
        for (int j = threadIdx.x; j < n; j += kThrThreads) f(order_key(sp[j]));
      };
      lo = wave_min_u32(lo);
      hi = wave_max_u32(hi);
      if (lane_id() == 0) {
        atomicMin(&sm.kmin, lo);
        atomicMax(&sm.kmax, hi);
      }
      __syncthreads();
      const KeyNorm nz = key_norm(sm.kmin, sm.kmax);
      each_key([&](uint32_t key) { atomicAdd(&sm.hist[nz.normalize(key) >> (32 - kHistBits)], 1u); });
      __syncthreads();
      find_boundary<kThrThreads>(sm, kHistBins, (uint32_t)m);
      const uint32_t b1 = (uint32_t)sm.bnd_bin;
      const uint32_t m2 = (uint32_t)m - sm.bnd_above;
      __syncthreads();
      zero_hist<kThrThreads>(sm, kHistBins);
      __syncthreads();
      each_key([&](uint32_t key) {
        const uint32_t v = nz.normalize(key);
        if ((v >> (32 - kHistBits)) == b1) atomicAdd(&sm.hist[(v >> (32 - 2 * kHistBits)) & (kHistBins - 1)], 1u);
      });
      __syncthreads();
      find_boundary<kThrThreads>(sm, kHistBins, m2);
      const uint32_t v = (b1 << (32 - kHistBits)) | ((uint32_t)sm.bnd_bin << (32 - 2 * kHistBits));
      tr = order_key_to_float(nz.denormalize(v));
      // Sample scores are clamped at +0, so tr >= 0; tr == 0 keeps every key (and the slab
      // overflows into the fallback) — as -inf, which the filter's unclamped compare needs.
      if (!(tr > 0.0f)) tr = -__builtin_inff();
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
  int32_t k, cap, want_stats, tie_cap;
};

// Candidates of a slab row with keys normalised over the row's [min, max] candidate key:
// their raw keys share their top bits, so without this the first 12-bit radix level would
// put nearly all of them in one bin (and overflow the tie buffer into rescans).
struct NormPairSrc {
  const float* s;
  const int32_t* i;
  KeyNorm nz;
  __device__ __forceinline__ uint32_t key(int j) const { return nz.normalize(order_key(s[j])); }
  __device__ __forceinline__ int32_t index(int j) const { return i[j]; }
};

// One 512-thread workgroup per row (three per CU): a min/max pass over the row's slab
// candidates, then block_select() over their normalised keys; the candidates stay in L2
// across its passes.
constexpr int kSlabThreads = 512;

__global__ __launch_bounds__(kSlabThreads) void slab_select_kernel(SlabArgs S) {
  __shared__ SelSmem sm;
  const int r = blockIdx.x;
  const int V = max(S.ke[r] - S.ks[r], 0);  // (an invalid range ke < ks counts as empty)
  const int c = S.cnt[r];
  const int need = min(S.k, V);
  int32_t* out = S.out + (int64_t)r * S.k;
  const bool bad = c > S.cap || c < need;
  if (threadIdx.x == 0) {
    if (S.want_stats) {  // same-address atomics from every row: only when asked for
      atomicAdd((unsigned long long*)&S.stats[V <= S.cap ? kStatStoreAll : kStatSampled], 1ull);
      atomicMax((unsigned long long*)&S.stats[kStatMax], (unsigned long long)c);
      if (V > S.cap) atomicMin((unsigned long long*)&S.stats[kStatMin], (unsigned long long)c);
      atomicAdd((unsigned long long*)&S.stats[kStatTotal], (unsigned long long)c);
    }
    if (bad) {
      atomicAdd((unsigned long long*)&S.stats[kStatFallback], 1ull);
      S.fb_list[atomicAdd(&S.fb_ctrl[0], 1)] = r;
    }
    sm.kmin = 0xFFFFFFFFu;
    sm.kmax = 0u;
  }
  if (bad) return;  // uniform: the fallback writes this row
  const float* ss = S.slab_s + (int64_t)r * S.cap;
  const int32_t* si = S.slab_i + (int64_t)r * S.cap;
  if (need > 0) {
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    // 8 loads per thread in flight per step, unconditional: a lane past the end re-reads the
    // last candidate (c >= need >= 1), which leaves the minimum and maximum unchanged.
    constexpr int U = 8;
    for (int base = 0; base < c; base += U * kSlabThreads) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * kSlabThreads + (int)threadIdx.x;
        v[u] = ss[j < c ? j : c - 1];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t k = order_key(v[u]);
        lo = min(lo, k);
        hi = max(hi, k);
      }
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane_id() == 0) {
      atomicMin(&sm.kmin, lo);
      atomicMax(&sm.kmax, hi);
    }
    __syncthreads();
    block_select<kSlabThreads>(NormPairSrc{ss, si, key_norm(sm.kmin, sm.kmax)}, c, need, out, sm, S.tie_cap);
  }
  for (int j = need + threadIdx.x; j < S.k; j += kSlabThreads) out[j] = -1;
}

// ----------------------------------------------------------------------------- K4

struct FbArgs {
  const int32_t* fb_list;
  int32_t* fb_ctrl;
  float* scratch;
  int64_t scratch_ld;
  int32_t* out;
  int32_t k, tie_cap;
  int32_t nslots;       // scratch rows (<= kFbSlots)
  int32_t row_tiles;    // tiles a row's keys can span
};

// Top-need of the V scores at x into out (row-relative key indices), exact: the sampled
// select (one pass over the scores in most cases), with the sample idx_select takes for
// long rows (6144 keys in runs of 8; rows of up to 6144 keys take every key) for any row
// length, the better estimate on clustered scores; the full radix passes when the
// tie-capacity override asks for them or for rows under 4 keys.  8 16-byte loads per
// thread in flight in the streaming pass.  (One sample shape and this width keep the
// fallback kernel within its registers: no private-memory spills.)
template <int NT, class SM>
__device__ __forceinline__ void fb_select_row(const float* x, int V, int need, int32_t* out, SM& sm, int tie_cap) {
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0 && V >= 4;  // workgroup-uniform
  if (need >= V || !vec || tie_cap < kTieCap) {
    if (need > 0) block_select<NT>(RowSrc{x}, V, need, out, sm, tie_cap);
  } else {
    block_select_sampled<NT, true, SM, kSelSamplesLong, 8, 8>(x, V, need, out, sm);
  }
}

// K4: exact fallback for the rows K3 queued, in one launch that exits at once when the
// queue is empty.
//  1. The first Q = min(queued, nslots) queued rows are re-scored over the whole grid: work
//     item w is chunk w % nchunk of queue entry w / nchunk, scored into scratch row
//     w / nchunk.  The chunk length (at least 128 tiles) is chosen from Q so that the
//     grid's workgroups (about one per CU) take about one item each; chunks are whole
//     tiles, so no key is written twice.
//  2. After each item the workgroup releases its stores (device scope: each XCD's L2 is
//     written back) and counts the item in the entry's counter; the workgroup that counts
//     the entry's last chunk acquires (its L2 invalidated) and selects the row from its
//     scratch row.
//  3. That workgroup then owns the scratch row and takes further queue entries (a queue
//     longer than nslots) from the shared head, scoring each whole row into it and
//     selecting.
// No workgroup waits on another.  The row is re-scored by wg_tiles() with the same per-key
// arithmetic as the score kernels (contiguous or paged keys; here each wave takes two tiles
// of every stage).  A row's score does not depend on which rows share its wave or which
// workgroup scores which tiles: its MFMA outputs, its head reduce, the half-wave sum (low
// half + high half) and its linear-tile pieces are computed the same way for any pairing,
// so the scores are bitwise the ones the slab was filtered with.  Only the row itself is
// stored; 2 rows per wave keep the register budget of this LDS-heavy kernel.  The stage
// buffers and the select's LDS are never live at once and share one union.
template <int FMT>
union FbShared {
  SelSmemT<kSelSamplesLong> sel;  // tie buffer, or the sampled select's sample and candidates
  StageShared<FMT> stage;
};

template <int FMT, int H>
__global__ __launch_bounds__(kThreads) void fallback_kernel(ScoreArgs A, LinArgs L, FbArgs F) {
  constexpr int RW = 2;
  __shared__ FbShared<FMT> shu;
  __shared__ int sh_word;
  const StageLds<FMT> sl{shu.stage.codes, shu.stage.sf, shu.stage.ks};
  const int queued = F.fb_ctrl[0];
  int32_t* done = F.fb_ctrl + 2;
  // Visible keys of row r, clamped to the scratch row (an invalid range counts as empty or
  // stays inside scratch).
  auto len_of = [&](int r) {
    const int64_t v = (int64_t)A.ke[r] - A.ks[r];
    return (int)(v < 0 ? 0 : (v > F.scratch_ld ? F.scratch_ld : v));
  };
  // Scores of tiles [t0, t1) of row r (clamped to its keys) into scratch row `slot`.
  auto score_tiles = [&](int r, int slot, int t0, int t1) {
    const int ks = A.ks[r], ke = A.ke[r];
    const int lo = ks > t0 * kTile ? ks : t0 * kTile, hi = ke < t1 * kTile ? ke : t1 * kTile;
    EpiArgs E = {};
    E.out = F.scratch + (int64_t)slot * F.scratch_ld;
    E.ld = F.scratch_ld;
    E.only_row = r;
    const int req = A.page_table ? request_of(A, r) : -1;
    wg_tiles<FMT, H, MODE_ROWSTORE, RW, true>(A, L, E, (r / RW) * RW, 0, 1, lo, hi, t0, t1, sl, req,
                                              1u << (r % RW));
  };
  const int Q = queued < F.nslots ? queued : F.nslots;
  constexpr int kMinChunk = 128;  // tiles (4096 keys)
  const int64_t want = ((int64_t)Q * F.row_tiles + gridDim.x - 1) / gridDim.x;
  const int chunk = (int)(want > kMinChunk ? want : kMinChunk);
  const int nchunk = (F.row_tiles + chunk - 1) / chunk;
  const int64_t items = (int64_t)Q * nchunk;
  int64_t w = blockIdx.x;  // next chunk item of this workgroup
  int own = -1;            // scratch row this workgroup owns after selecting its row
  // One loop (one inlined copy of the score and select code): chunk items first, then,
  // for a workgroup that owns a scratch row, whole rows from the shared head.
  for (;;) {  // workgroup-uniform
    int r, slot, t0, t1;
    const bool chunked = w < items;
    if (chunked) {
      slot = (int)(w / nchunk);
      const int c = (int)(w % nchunk);
      r = F.fb_list[slot];
      t0 = A.ks[r] / kTile + c * chunk;
      const int tend = (A.ke[r] + kTile - 1) / kTile;
      t1 = tend < t0 + chunk ? tend : t0 + chunk;
    } else {
      if (own < 0) break;
      if (threadIdx.x == 0) sh_word = F.nslots + atomicAdd(&F.fb_ctrl[1], 1);
      __syncthreads();
      const int item = sh_word;
      __syncthreads();
      if (item >= queued) break;
      r = F.fb_list[item];
      slot = own;
      t0 = A.ks[r] / kTile;
      t1 = (A.ke[r] + kTile - 1) / kTile;
    }
    if (len_of(r) > 0 && t0 < t1) score_tiles(r, slot, t0, t1);
    bool sel = !chunked;
    if (chunked) {
      // Every wave releases its own scores at device scope (L2 written back once its
      // stores have completed: a workgroup barrier does not wait for other waves' global
      // stores), then one increment, itself a release, counts the chunk.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();  // also: the stage buffers are reused next
      if (threadIdx.x == 0)
        sh_word = __hip_atomic_fetch_add(&done[slot], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      sel = sh_word == nchunk - 1;  // the entry's last chunk: its row is complete
      __syncthreads();              // sh_word is rewritten next
      if (sel) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        own = slot;
      }
      w += gridDim.x;
    } else {
      __syncthreads();
    }
    if (sel) {
      const int V = len_of(r), need = min(F.k, V);
      int32_t* out = F.out + (int64_t)r * F.k;
      fb_select_row<kThreads>(F.scratch + (int64_t)slot * F.scratch_ld, V, need, out, shu.sel, F.tie_cap);
      for (int j = need + threadIdx.x; j < F.k; j += kThreads) out[j] = -1;
      __syncthreads();  // the LDS union is reused next
    }
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
  A.num_req = P.num_req;
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
  W.spread = P.page_table != nullptr;
  W.total = (int64_t)W.nrb * W.nchunk;
  W.grid = W.nchunk < 8 ? 8 * ((W.total + 7) / 8) : (int64_t)((W.nchunk + 7) / 8) * 8 * W.nrb;
  return W;
}

static dim3 tile_grid(const TileWork& W) { return dim3((unsigned)W.grid); }

static LinArgs lin_args(const FusedPlan& F) { return LinArgs{F.lin_q8, F.lin_sf}; }

// u = sum_h w_h q_h and its pieces for every row (contiguous keys only).
static hipError_t launch_lin_prep(const DevProblem& P, uint8_t* q8, uint8_t* sf, hipStream_t s) {
  const dim3 grid(P.rows), block(128);
  const bool key_fp4 = P.fmt == FMT_MXFP4;
  if (P.fmt == FMT_E4M3) {
    if (P.heads == 64) lin_prep_kernel<FMT_E4M3, 64><<<grid, block, 0, s>>>(P.q, P.q_sf, P.w, P.rows, key_fp4, q8, sf);
    else lin_prep_kernel<FMT_E4M3, 32><<<grid, block, 0, s>>>(P.q, P.q_sf, P.w, P.rows, key_fp4, q8, sf);
  } else {
    if (P.heads == 64) lin_prep_kernel<FMT_MXFP4, 64><<<grid, block, 0, s>>>(P.q, P.q_sf, P.w, P.rows, key_fp4, q8, sf);
    else lin_prep_kernel<FMT_MXFP4, 32><<<grid, block, 0, s>>>(P.q, P.q_sf, P.w, P.rows, key_fp4, q8, sf);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t dispatch_score(const DevProblem& P, const LinArgs& L, const EpiArgs& E, const TileWork& W,
                                 hipStream_t s, int64_t max_groups = 0) {
  const ScoreArgs A = score_args(P);
  dim3 grid = tile_grid(W);  // (persistent paged FILTER: at most max_groups, the rest by ticket)
  if (max_groups > 0 && grid.x > max_groups) grid.x = (unsigned)max_groups;
  const dim3 block(kThreads);
  if (P.page_table) {  // paged keys are e4m3 (checked at the boundary)
    if (P.heads == 64) score_pages_kernel<FMT_E4M3, 64, MODE><<<grid, block, 0, s>>>(A, L, E, W);
    else score_pages_kernel<FMT_E4M3, 32, MODE><<<grid, block, 0, s>>>(A, L, E, W);
  } else if (P.fmt == FMT_E4M3) {
    if (P.heads == 64) score_tiles_kernel<FMT_E4M3, 64, MODE, true><<<grid, block, 0, s>>>(A, L, E, W);
    else score_tiles_kernel<FMT_E4M3, 32, MODE, true><<<grid, block, 0, s>>>(A, L, E, W);
  } else {
    const bool ks = A.k_scale != nullptr;  // MXFP4 keys usually come without per-key scales
    if (P.heads == 64) {
      if (ks) score_tiles_kernel<FMT_MXFP4, 64, MODE, true><<<grid, block, 0, s>>>(A, L, E, W);
      else score_tiles_kernel<FMT_MXFP4, 64, MODE, false><<<grid, block, 0, s>>>(A, L, E, W);
    } else {
      if (ks) score_tiles_kernel<FMT_MXFP4, 32, MODE, true><<<grid, block, 0, s>>>(A, L, E, W);
      else score_tiles_kernel<FMT_MXFP4, 32, MODE, false><<<grid, block, 0, s>>>(A, L, E, W);
    }
  }
  return hipGetLastError();
}

// Keys per work item of the score kernels: long enough to amortise a workgroup's row
// operand loads (up to 16384), short enough that the grid keeps about 8192 workgroups.
constexpr int64_t kSampleItems = 1024;
static int chunk_keys(const DevProblem& P) {
  const int rb = rows_per_block_for(P);
  const int64_t nrb = (P.rows + rb - 1) / rb;
  int64_t c = (std::max<int64_t>(P.key_span, 1) * nrb + 8191) / 8192;
  c = (c + 4095) / 4096 * 4096;
  return (int)std::min<int64_t>(std::max<int64_t>(c, 4096), 16384);
}
// Sample slots per work item of the sample pass: 2048 (the LDS page cache covers that many at
// the largest stride).  Paged keys, whose row blocks are few and read keys of their own, take
// fewer, so that the pass has about 1024 work items to spread over the CUs; contiguous keys
// gain nothing from that (each item reloads its rows' operands).
static int chunk_samples(const DevProblem& P, int32_t ns) {
  if (P.page_table == nullptr) {
    // Contiguous keys: rows of up to 8192 samples in chunks of 2048; longer rows in equal
    // chunks (a multiple of the tile) of at most 4096, so that each work item's row operand
    // loads and pipeline start are spread over more samples (long: 4 x 3712, 0.225 ->
    // 0.213 ms against 8 x 1856).  Fewer than 8 chunks are dealt to the XCDs in eighths of
    // the item list, so every XCD holds the same work.
    if (ns <= 4 * 2048) return 2048;
    const int64_t nc = ((int64_t)ns + 4095) / 4096;
    const int64_t c = (((int64_t)ns + nc - 1) / nc + kTile - 1) / kTile * kTile;
    return (int)c;
  }
  const int rb = rows_per_block_for(P);
  const int64_t nrb = (P.rows + rb - 1) / rb;
  int64_t c = ((int64_t)std::max(ns, 1) * nrb + kSampleItems - 1) / kSampleItems;
  c = (c + 127) / 128 * 128;
  return (int)std::min<int64_t>(std::max<int64_t>(c, 256), 2048);
}

size_t lin_ws_bytes(int32_t rows) {
  return (size_t)rows * kLinRowBytes + (((size_t)rows * kLinRowScales + 255) & ~(size_t)255) + 256;
}

void lin_carve(void* ws, int32_t rows, uint8_t** q8, uint8_t** sf) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  *q8 = p;
  *sf = p + (size_t)rows * kLinRowBytes;
}

hipError_t launch_score_store(const DevProblem& P, float* out, int64_t ld, void* ws, hipStream_t s) {
  if (P.rows == 0) return hipSuccess;
  LinArgs L{nullptr, nullptr};
  if (P.fmt == FMT_MXFP4) {  // the split form's per-row pieces
    uint8_t *q8, *sf;
    lin_carve(ws, P.rows, &q8, &sf);
    hipError_t e = launch_lin_prep(P, q8, sf, s);
    if (e != hipSuccess) return e;
    L = LinArgs{q8, sf};
  }
  EpiArgs E = {};
  E.out = out;
  E.ld = ld;
  return dispatch_score<MODE_STORE>(P, L, E, tile_work(P, P.key_span, chunk_keys(P)), s);
}

hipError_t launch_fused(const DevProblem& P, const FusedPlan& F, int32_t* out_idx, hipStream_t s, hipEvent_t* ev) {
  if (P.rows == 0) return hipSuccess;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  const LinArgs L = lin_args(F);
  if (P.fmt == FMT_MXFP4 && (e = launch_lin_prep(P, F.lin_q8, F.lin_sf, s)) != hipSuccess) return e;
  // K1a: samples
  {
    EpiArgs E = {};
    E.samp = F.samp;
    E.ns = F.ns;
    E.stride = F.stride;
    E.skip_le = F.cap;
    if (F.debug_mode != 0 && F.debug_row_mod <= 0) E.skip_le = 0x7FFFFFFF;  // every row forced
    if ((e = dispatch_score<MODE_SAMPLE>(P, L, E, tile_work(P, F.ns, chunk_samples(P, F.ns)), s)) != hipSuccess)
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
    if (F.ns >= 2048)
      threshold_kernel<1024, 15360><<<dim3(P.rows), dim3(1024), 0, s>>>(T);
    else
      threshold_kernel<kThreads, 0><<<dim3(P.rows), dim3(kThreads), 0, s>>>(T);
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
    int64_t groups = 0;
    if (P.page_table) {  // persistent: two workgroups per CU (ticket cleared by K1b)
      E.ticket = F.fb_ctrl + kPagedTicketWord;
      groups = 2 * (int64_t)F.cu;
    }
    if ((e = dispatch_score<MODE_FILTER>(P, L, E, tile_work(P, P.key_span, chunk_keys(P)), s, groups)) != hipSuccess)
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
    S.want_stats = F.want_stats;
    S.tie_cap = F.tie_cap;
    slab_select_kernel<<<dim3(P.rows), dim3(kSlabThreads), 0, s>>>(S);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(4)) != hipSuccess) return e;
  }
  // K4: exact fallback for queued rows (exits at once when the queue is empty): the first
  // fb_blocks queued rows re-scored in chunks over the whole chip and selected, any further
  // rows scored and selected one workgroup per row.
  {
    const ScoreArgs A = score_args(P);
    FbArgs B;
    B.fb_list = F.fb_list;
    B.fb_ctrl = F.fb_ctrl;
    B.scratch = F.scratch;
    B.scratch_ld = F.scratch_ld;
    B.out = out_idx;
    B.k = F.k;
    B.tie_cap = F.tie_cap;
    B.nslots = F.fb_blocks;
    B.row_tiles = (int)((F.scratch_ld + kTile - 1) / kTile + 1);  // key span + alignment
    const int64_t items = (int64_t)B.nslots * ((B.row_tiles + 127) / 128);  // at the shortest chunks
    const dim3 grid((unsigned)(items < F.cu ? items : F.cu)), block(kThreads);  // one workgroup per CU
    if (P.fmt == FMT_E4M3) {  // contiguous or paged
      if (P.heads == 64) fallback_kernel<FMT_E4M3, 64><<<grid, block, 0, s>>>(A, L, B);
      else fallback_kernel<FMT_E4M3, 32><<<grid, block, 0, s>>>(A, L, B);
    } else {
      if (P.heads == 64) fallback_kernel<FMT_MXFP4, 64><<<grid, block, 0, s>>>(A, L, B);
      else fallback_kernel<FMT_MXFP4, 32><<<grid, block, 0, s>>>(A, L, B);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(5)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace idx
