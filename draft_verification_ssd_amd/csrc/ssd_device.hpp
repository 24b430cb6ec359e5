// Device-side building blocks for the gfx950 verification kernels: element traits for fp32 / bf16
// rows streamed as 16-byte vectors, wave64 and 256-thread block reductions and scans, and the
// per-thread sorted top-F list used for bonus-token guesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace ssd {

constexpr int kThreads = 256;            // every kernel runs 4 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 16;
constexpr int kMaxF = 16;
constexpr int kMaxChunks = 64;           // phase-1 chunks per row
constexpr int kSubElems = 8;             // phase-2 elements per thread (contiguous)
constexpr int kSub = kThreads * kSubElems;  // phase-2 sub-chunk width
constexpr int kMaxSubs = (1 << 22) / kSub;  // sub-chunks of the largest supported row

constexpr uint32_t kFlagBadToken = 0x1u;
constexpr uint32_t kFlagSaguaroNorm = 0x2u;
constexpr uint32_t kFlagBadF = 0x4u;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------------
// Element traits: a row is streamed as uint4 vectors (4 fp32 or 8 bf16 values).
// ---------------------------------------------------------------------------------------------
struct F32T {
  using T = float;
  static constexpr int kVec = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  __device__ static __forceinline__ float one(const T* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
  }
};

struct BF16T {
  using T = uint16_t;
  static constexpr int kVec = 8;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  __device__ static __forceinline__ float one(const T* p, int64_t i) {
    return __uint_as_float(uint32_t(p[i]) << 16);
  }
  __device__ static __forceinline__ void unpack(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xFFFF0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xFFFF0000u);
    o[4] = __uint_as_float(v.z << 16);
    o[5] = __uint_as_float(v.z & 0xFFFF0000u);
    o[6] = __uint_as_float(v.w << 16);
    o[7] = __uint_as_float(v.w & 0xFFFF0000u);
  }
};

// ---------------------------------------------------------------------------------------------
// wave64 reductions (xor butterflies: every lane ends with the bit-identical result)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
// lexicographic max of (hi, lo) key pairs
__device__ __forceinline__ void wave_max_key(uint32_t& hi, uint32_t& lo) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t oh = __shfl_xor(hi, o, 64);
    const uint32_t ol = __shfl_xor(lo, o, 64);
    if (oh > hi || (oh == hi && ol > lo)) {
      hi = oh;
      lo = ol;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 256-thread block reductions over a small shared scratch array (>= kWaves entries).
// The final combine runs in a fixed order, so results are deterministic.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sh[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}
__device__ __forceinline__ int block_min_i(int v, int* sh) {
  v = wave_min_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return min(min(sh[0], sh[1]), min(sh[2], sh[3]));
}
__device__ __forceinline__ int block_max_i(int v, int* sh) {
  v = wave_max_i(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return max(max(sh[0], sh[1]), max(sh[2], sh[3]));
}

// Exclusive scan of one float per thread over the block; returns the exclusive prefix and writes
// the block total as fl(excl[last] + v[last]) so that it equals the last thread's inclusive value.
__device__ __forceinline__ float block_excl_scan(float v, float* sh, float& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  float base = 0.f;
  for (int i = 0; i < w; ++i) base += sh[i];
  const float excl_lane = __shfl_up(inc, 1, 64);
  const float excl = (lane == 0) ? base : base + excl_lane;
  // total: computed by the last thread, broadcast
  __syncthreads();
  if (threadIdx.x == kThreads - 1) sh[kWaves] = excl + v;
  __syncthreads();
  total = sh[kWaves];
  return excl;
}

// order-preserving map of a float to uint32 (larger float -> larger key); used with key 0 = empty
__device__ __forceinline__ uint32_t ordered_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// ---------------------------------------------------------------------------------------------
// Per-thread top-F list, sorted by (value desc, index asc). A thread visits its indices in
// increasing order, so a later equal value never displaces an earlier one: insertion needs a
// strictly larger value than the current F-th entry (thr).
// ---------------------------------------------------------------------------------------------
template <int FM>
struct TopList {
  float v[FM];
  int i[FM];
  float thr;
  int F;

  __device__ __forceinline__ void init(int f) {
    F = f;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      v[j] = -INFINITY;
      i[j] = -1;
    }
    thr = (f > 0) ? -INFINITY : INFINITY;
  }

  // precondition: z > thr
  __device__ __forceinline__ void insert(float z, int idx) {
#pragma unroll
    for (int j = FM - 1; j >= 0; --j) {
      const float pv = (j > 0) ? v[j > 0 ? j - 1 : 0] : INFINITY;
      const int pi = (j > 0) ? i[j > 0 ? j - 1 : 0] : -1;
      if (!(v[j] >= z)) {
        if (pv >= z) {
          v[j] = z;
          i[j] = idx;
        } else {
          v[j] = pv;
          i[j] = pi;
        }
      }
    }
    float t = v[0];
#pragma unroll
    for (int j = 1; j < FM; ++j)
      if (j == F - 1) t = v[j];
    thr = t;
  }

  __device__ __forceinline__ void offer(float z, int idx, int exclude) {
    if (z > thr && idx != exclude) insert(z, idx);
  }

  // entry h as a (hi, lo) key, (0, 0) when absent
  __device__ __forceinline__ void key_at(int h, uint32_t& hi, uint32_t& lo) const {
    float hv = -INFINITY;
    int hidx = -1;
#pragma unroll
    for (int j = 0; j < FM; ++j)
      if (j == h) {
        hv = v[j];
        hidx = i[j];
      }
    if (h < F && hidx >= 0) {
      hi = ordered_key(hv);
      lo = ~uint32_t(hidx);
    } else {
      hi = 0;
      lo = 0;
    }
  }
};

// Merge the per-thread lists of a block into its top F (F <= FM); thread 0 receives the winners
// in out_v / out_i (index -1 for an empty place). sh must hold 2*kWaves uint32.
template <int FM>
__device__ __forceinline__ void block_merge_top(const TopList<FM>& tl, int F, uint32_t* sh,
                                                float* out_v, int* out_i) {
  int head = 0;
  for (int r = 0; r < F; ++r) {
    uint32_t hi, lo;
    tl.key_at(head, hi, lo);
    uint32_t mh = hi, ml = lo;
    wave_max_key(mh, ml);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
      sh[2 * w] = mh;
      sh[2 * w + 1] = ml;
    }
    __syncthreads();
    uint32_t bh = sh[0], bl = sh[1];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) {
      const uint32_t oh = sh[2 * q], ol = sh[2 * q + 1];
      if (oh > bh || (oh == bh && ol > bl)) {
        bh = oh;
        bl = ol;
      }
    }
    if (bh != 0 && hi == bh && lo == bl) ++head;  // indices are unique: one owner
    if (threadIdx.x == 0) {
      out_v[r] = (bh != 0) ? key_to_float(bh) : -INFINITY;
      out_i[r] = (bh != 0) ? int(~bl) : -1;
    }
  }
}

}  // namespace ssd
