// The indexer scoring core for gfx950: operand formats, register-resident query operands,
// key operands and the half-wave combine, shared by every kernel that produces a score
// (materialised scores, threshold samples, the fused filter and the exact fallback all run
// one tile routine), so that all of them produce bitwise-identical scores for the same
// (row, key) — the design rule of the LiteTopK page, section 1 (scoring core identical,
// only the epilogue differs).
//
//   score[r, s] = kscale[s] * sum_h w[r, h] * max(q[r, h] . k[s], 0)
//
// One wave computes a 32 (heads) x 32 (keys) block of dot products with two scaled MFMAs
// v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 each, head_dim = 128).  Operand fragments:
// lane l holds head / key (l % 32) and the 32 consecutive head_dim elements
// [32*(l/32), +32) of the K-step (fp8: 32 bytes, fp4: 16 bytes), with that block's e8m0
// scale (fixed 127 = 1.0 for e4m3).  The accumulator gives lane l key (l % 32) and heads
// 8*(i/4) + 4*(l/32) + (i%4), i = 0..15.  The head reduce runs in VGPRs in a fixed order
// per lane; the two half-waves are then added with v_permlane32_swap, which also packs two
// rows into one register (lanes 0-31 row A, lanes 32-63 row B).
#pragma once
#include "common.hpp"

namespace idx {

enum : int { FMT_E4M3 = 1, FMT_MXFP4 = 2 };

template <int FMT>
struct Fmt;
template <>
struct Fmt<FMT_E4M3> {
  static constexpr int kBytes = 128;  // bytes per head (q) or key (k) vector
  static constexpr int kCode = 0;     // cbsz/blgp operand format: fp8 e4m3
};
template <>
struct Fmt<FMT_MXFP4> {
  static constexpr int kBytes = 64;
  static constexpr int kCode = 4;     // fp4 e2m1
};

// Everything a scoring kernel reads, as raw device pointers.
struct ScoreArgs {
  const uint8_t* q;
  const uint8_t* q_sf;
  const uint8_t* k;
  const uint8_t* k_sf;
  const float* k_scale;
  const uint16_t* w;
  const int32_t* ks;
  const int32_t* ke;
  const int32_t* page_table;
  const int32_t* row_req;
  int32_t max_pages;
  int32_t num_req;
  int32_t rows;
  int64_t num_keys;  // physical keys (contiguous) or slots (paged)
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// MXFP4 scores use the split form of the ReLU (a VALU |x| reduce plus a linear MFMA tile,
// whose sum is twice the score); its factor 1/2 is carried by w here and by the linear
// tile's vector u, both halved exactly (a power of two).
template <int FMT>
struct SplitRelu {
  static constexpr bool value = FMT == FMT_MXFP4;
};

// Query-side operands of one row, held in registers for the life of a wave.
template <int FMT, int H>
struct RowOperand {
  static constexpr int MT = H / 32;
  v8i a[MT][2];
  int sa[MT];  // e8m0 block scales of the two K-steps, byte ks (the MFMA's scale byte select)
  float w[MT][16];  // w of this lane's heads (halved for the split form)
};

template <int FMT, int H>
__device__ __forceinline__ void load_row(RowOperand<FMT, H>& ro, const ScoreArgs& A, int r) {
  constexpr int KB = Fmt<FMT>::kBytes;
  const int l = lane_id();
  const int half = l >> 5;
  const int m = l & 31;
#pragma unroll
  for (int mt = 0; mt < RowOperand<FMT, H>::MT; ++mt) {
    const int64_t hv = (int64_t)r * H + mt * 32 + m;
    const uint8_t* qp = A.q + hv * KB;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (FMT == FMT_E4M3) {
        const v4i* src = reinterpret_cast<const v4i*>(qp + ks * 64 + half * 32);
        const v4i x0 = src[0], x1 = src[1];
        ro.a[mt][ks] = v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      } else {
        const v4i x = *reinterpret_cast<const v4i*>(qp + ks * 32 + half * 16);
        ro.a[mt][ks] = v8i{x.x, x.y, x.z, x.w, 0, 0, 0, 0};
      }
    }
    if constexpr (FMT == FMT_E4M3) {
      ro.sa[mt] = 0x7F7F;  // 1.0 for both K-steps
    } else {
      ro.sa[mt] = (int)A.q_sf[hv * 4 + half] | ((int)A.q_sf[hv * 4 + 2 + half] << 8);
    }
    constexpr float kW = SplitRelu<FMT>::value ? 0.5f : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = mt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      ro.w[mt][i] = kW * bf16_to_f32(A.w[(int64_t)r * H + h]);
    }
  }
}

// Key-side operand of one key per lane (lane l supplies key l % 32 of the block).
struct KeyOperand {
  v8i b[2];
  int sb;  // e8m0 block scales: byte 0 for K-step 0, byte 2 for K-step 1
};

// Add the two half-wave partials of row A (pa) and row B (pb): lanes 0-31 receive the
// head sum of row A for key (l % 32), lanes 32-63 that of row B.  pa == pb gives the
// single-row sum in every lane.
__device__ __forceinline__ float combine_halves(float pa, float pb) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pa), __float_as_uint(pb), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace idx
