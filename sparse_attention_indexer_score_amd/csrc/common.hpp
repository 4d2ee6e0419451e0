// Device-side primitives shared by the gfx950 kernels: types, the fp32 order key and
// wave / workgroup scans built from ballot, mbcnt and LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kHeadDim = 128;
constexpr int kPage = 64;
constexpr int kMaxTopK = 2048;

// Radix histogram of the selection: 12 bits of the fp32 order key per level (the ROCm
// top-k page, constants table: kHistBits = 12); tie buffer of 4096 entries (kTieCap).
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kTieCap = 4096;

// fp32 -> uint32 whose unsigned order is the numeric order of the floats, with -0.0
// mapped onto +0.0 so that the two compare equal (and then tie by key index).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float order_key_to_float(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(b);
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Number of set bits of `mask` below the calling lane.
__device__ __forceinline__ int mask_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t t = __shfl_up(v, d, kWave);
    if (l >= d) v += t;
  }
  return v;
}

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations, not for
// its outstanding global loads (a full __syncthreads() also waits for those), so loads
// issued ahead stay in flight across it.  Callers must not rely on it for global memory.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive prefix sum over the threads of a workgroup of NT threads (thread order),
// and the workgroup total.  `scratch` holds NT/64 + 1 words of LDS.  Contains barriers:
// every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const uint32_t inc = wave_inclusive_sum(v);
  if ((tid & (kWave - 1)) == kWave - 1) scratch[w] = inc;
  lds_sync();
  if (tid == 0) {
    uint32_t run = 0;
    for (int i = 0; i < NW; ++i) {
      uint32_t t = scratch[i];
      scratch[i] = run;
      run += t;
    }
    scratch[NW] = run;
  }
  lds_sync();
  const uint32_t res = scratch[w] + inc - v;
  *total = scratch[NW];
  lds_sync();
  return res;
}

}  // namespace idx
