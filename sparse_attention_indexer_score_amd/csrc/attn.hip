// Sparse attention of each query row over the KV slots its indexer selected (gfx950): the
// consumer of the top-k (QSA sparse paged attention page, vllm-project/vllm#66512: each
// query row attends to about 2048 tokens chosen by the indexer, logical positions are
// turned into physical slots by a separate pass first, QK runs in bf16 and PV in fp16 with
// the e4m3 cache values converted exactly, fp32 accumulation).
//
//   s_j      = softmax_scale * q[r, h] . k[slot_j, g]          g = h / (hq / hkv)
//   out[r,h] = output_scale * sum_j exp(s_j - m) v[slot_j, g] / sum_j exp(s_j - m)
//
// over the valid slots j of row r (slots outside [0, num_slots) take no part; a row with
// none gives 0).
//
// One workgroup of four waves per (row, KV head); the group's query heads (at most 32) are
// the 32 columns of v_mfma_f32_32x32x16_{bf16,f16}.  The waves take the row's 32-slot tiles
// in turn, each with its own online softmax, and merge at the end in a fixed order.
//   QK:  S^T[32 keys x 32 heads] = K[32 x 128] . Q^T: lane l holds key l % 32 and, for K-step
//        s, the 8 dims 64 (l / 32) + 8 s .. +8 of it; Q is held the same way per head.  The
//        result gives lane l head l % 32 and keys 8 (i / 4) + 4 (l / 32) + (i % 4).
//   PV:  O[32 heads x 128 dims] += P . V with K = keys: the softmax weights are used where
//        the QK result left them (the MFMA's K order is that key order), and the V tile is
//        written transposed into LDS in the same key order, so each lane reads the 8 keys of
//        its dim as two 4-byte words.  Output column c of N-tile n is dim c + 32 n.
#include "common.hpp"
#include "launch.hpp"

namespace idx {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kAttnTile = 32;     // selected slots per tile
constexpr int kVtStride = 36;     // bytes per dim row of a transposed V tile (32 keys + pad)

struct AttnArgs {
  const uint16_t* q;   // bf16 [rows][hq][128]
  const uint8_t* k;    // e4m3 [num_slots][hkv][128]
  const uint8_t* v;
  const int32_t* slots;
  float* out;          // fp32 [rows][hq][128]
  int64_t num_slots;
  int32_t rows, hq, hkv, width;
  float softmax_scale, output_scale;
};

struct AttnShared {
  union {
    uint8_t vt[kAttnWaves][kHeadDim * kVtStride];  // per wave: V tile, [dim][key position]
    struct {
      float o[kAttnWaves][32][kHeadDim];           // per wave: unnormalised outputs
      float m[kAttnWaves][32];                     // running maxima
      float l[kAttnWaves][32];                     // running sums
    } mg;
  };
};

// 8 e4m3 bytes (two words, byte e = element e) as bf16 / fp16 operands, two values per
// conversion instruction (scale 1.0); both conversions are exact (every e4m3 value is a
// bf16 and an fp16 value).
__device__ __forceinline__ v8bf e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, 1.0f, true);
  return v8bf{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
__device__ __forceinline__ v8h e4m3x8_f16(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, true);
  return v8h{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Position of key c (0..31) of a tile in the MFMA K order of the PV product: key
// 16 s + 8 (e / 4) + 4 h + (e % 4) is element 8 h + e of K-step s.
__device__ __forceinline__ int vt_pos(int c) {
  const int r = c & 15;
  return (c & 16) + 8 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

__global__ __launch_bounds__(kAttnThreads, 2) void sparse_attn_kernel(AttnArgs P) {
  __shared__ AttnShared sh;
  const int r = blockIdx.x / P.hkv, g = blockIdx.x % P.hkv;
  const int G = P.hq / P.hkv;
  const int l = lane_id(), c = l & 31, h = l >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // Q^T operands of this lane's head (zero past the group), 8 K-steps.
  v8bf qb[8];
  {
    const bool hv = c < G;
    const uint4* qp = reinterpret_cast<const uint4*>(P.q + ((int64_t)r * P.hq + g * G + (hv ? c : 0)) * kHeadDim + 64 * h);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 x = hv ? qp[s] : make_uint4(0, 0, 0, 0);
      qb[s] = __builtin_bit_cast(v8bf, x);
    }
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16f o[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) o[n] = v16f{};

  const int ntiles = (P.width + kAttnTile - 1) / kAttnTile;
  const int32_t* srow = P.slots + (int64_t)r * P.width;
  struct Tile {
    uint4 kr[4], vr[4];
    bool valid;
  };
  // Every load below is unconditional (a position past the row's end re-reads its last slot
  // id, an invalid slot reads slot 0, and the tile's valid flag masks what was read): a load
  // under a branch would leave the compiler unable to count the loads in flight, and each
  // tile would then wait for the prefetch of the next before its first MFMA.
  auto slot_at = [&](int t) -> int32_t {
    const int j = t * kAttnTile + c;
    return srow[j < P.width ? j : P.width - 1];
  };
  // K / V bytes [64 h, 64 h + 64) of key c of tile t, whose slot id was loaded before.
  auto fetch = [&](int t, int32_t slot, Tile& T) {
    T.valid = t * kAttnTile + c < P.width && slot >= 0 && slot < P.num_slots;
    const int64_t base = ((int64_t)(T.valid ? slot : 0) * P.hkv + g) * kHeadDim + 64 * h;
    const uint4* kp = reinterpret_cast<const uint4*>(P.k + base);
    const uint4* vp = reinterpret_cast<const uint4*>(P.v + base);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      T.kr[u] = kp[u];
      T.vr[u] = vp[u];
    }
  };

  uint8_t* vt = sh.vt[wave];
  Tile cur, nxt;
  int t = wave;
  int32_t sn = 0;  // slot id of this lane's key in the tile after the next
  if (ntiles > 0) {  // (P.width >= 1: the clamped slot reads stay in the row)
    fetch(t, slot_at(t), cur);
    sn = slot_at(t + kAttnWaves);
  }
  for (; t < ntiles; t += kAttnWaves) {
    fetch(t + kAttnWaves, sn, nxt);  // past the last tile: masked re-reads
    sn = slot_at(t + 2 * kAttnWaves);
    // QK over the tile.
    v16f sacc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 w = cur.kr[s >> 1];
      const v8bf a = (s & 1) ? e4m3x8_bf16(w.z, w.w) : e4m3x8_bf16(w.x, w.y);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[s], sacc, 0, 0, 0);
    }
    // V tile, transposed into this wave's LDS region in the PV key order.
    {
      const int pos = vt_pos(c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 v = cur.valid ? cur.vr[u] : make_uint4(0, 0, 0, 0);  // (an invalid key's V may be any bytes)
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int b = 0; b < 16; ++b) vt[(64 * h + 16 * u + b) * kVtStride + pos] = (uint8_t)(wd[b >> 2] >> (8 * (b & 3)));
      }
    }
    // Online softmax of this lane's head over the tile's valid keys.
    const uint64_t vmask = wave_ballot(cur.valid);
    float sv[16];
    float mt = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * h + (i & 3);
      sv[i] = ((vmask >> key) & 1) ? P.softmax_scale * sacc[i] : -__builtin_inff();
      mt = fmaxf(mt, sv[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);
    const bool none = m_new == -__builtin_inff();  // no valid key yet for this head
    const float alpha = none ? 1.0f : __expf(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = none ? 0.0f : __expf(sv[i] - m_new);
      psum += sv[i];
    }
    psum += __shfl_xor(psum, 32, kWave);
    l_run = alpha * l_run + psum;
    m_run = m_new;
    // Rescale the outputs: O row (head) 8 (i / 4) + 4 h + (i % 4) takes that head's factor.
    // Skipped when no head's maximum moved (every factor 1), as in most tiles after the first.
    if (wave_ballot(alpha != 1.0f)) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float ai = __shfl(alpha, 8 * (i >> 2) + 4 * h + (i & 3), kWave);
#pragma unroll
        for (int n = 0; n < 4; ++n) o[n][i] *= ai;
      }
    }
    // PV: two K-steps of 16 keys, four N-tiles of 32 dims.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const v8h pa = v8h{(_Float16)sv[8 * s2 + 0], (_Float16)sv[8 * s2 + 1], (_Float16)sv[8 * s2 + 2],
                         (_Float16)sv[8 * s2 + 3], (_Float16)sv[8 * s2 + 4], (_Float16)sv[8 * s2 + 5],
                         (_Float16)sv[8 * s2 + 6], (_Float16)sv[8 * s2 + 7]};
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint32_t* rowp = reinterpret_cast<const uint32_t*>(vt + (c + 32 * n) * kVtStride + 16 * s2 + 8 * h);
        const v8h vb = e4m3x8_f16(rowp[0], rowp[1]);
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa, vb, o[n], 0, 0, 0);
      }
    }
    // The next tile's V writes must not pass this tile's reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cur = nxt;
  }

  // Merge the four waves' partial results in a fixed order.
  __syncthreads();  // every wave is done with its V tiles (the merge area overlays them)
  if (h == 0) {
    sh.mg.m[wave][c] = m_run;
    sh.mg.l[wave][c] = l_run;
  }
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) sh.mg.o[wave][8 * (i >> 2) + 4 * h + (i & 3)][c + 32 * n] = o[n][i];
  __syncthreads();
  for (int e = threadIdx.x; e < G * kHeadDim; e += kAttnThreads) {
    const int hh = e / kHeadDim, d = e % kHeadDim;
    float ms = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) ms = fmaxf(ms, sh.mg.m[w][hh]);
    float res = 0.0f;
    if (ms != -__builtin_inff()) {
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float mw = sh.mg.m[w][hh];
        const float f = mw == -__builtin_inff() ? 0.0f : __expf(mw - ms);
        num += f * sh.mg.o[w][hh][d];
        den += f * sh.mg.l[w][hh];
      }
      res = P.output_scale * num / den;
    }
    P.out[((int64_t)r * P.hq + g * G + hh) * kHeadDim + d] = res;
  }
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint8_t* k, const uint8_t* v, int64_t num_slots,
                              const int32_t* slots, int32_t rows, int32_t hq, int32_t hkv, int32_t width,
                              float softmax_scale, float output_scale, float* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const AttnArgs A{q, k, v, slots, out, num_slots, rows, hq, hkv, width, softmax_scale, output_scale};
  sparse_attn_kernel<<<dim3((unsigned)((int64_t)rows * hkv)), dim3(kAttnThreads), 0, s>>>(A);
  return hipGetLastError();
}

}  // namespace idx
