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
constexpr int kMaxV = 1 << 20;             // largest supported vocabulary
constexpr int kMaxTiles = kMaxV / kSub;     // tiles of the largest supported row

constexpr uint32_t kFlagBadToken = 0x1u;
constexpr uint32_t kFlagSaguaroNorm = 0x2u;
constexpr uint32_t kFlagBadF = 0x4u;
constexpr uint32_t kFlagTimeout = 0x8u;
constexpr uint32_t kFlagBadC = 0x10u;

// Saguaro factor of a row: the per-row array's entry (a value outside [0, 1] is clamped to it, NaN
// taken as 1, and flagged when `flag` is set), else the call's single factor.
__device__ __forceinline__ float row_saguaro_c(const float* C_per_row, float C, int64_t row, uint32_t* flags,
                                               bool flag) {
  if (!C_per_row) return C;
  const float c = C_per_row[row];
  if (c >= 0.f && c <= 1.f) return c;
  if (flag) atomicOr(flags, kFlagBadC);
  return (c < 0.f) ? 0.f : 1.f;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Cand {
  float v;
  int i;
};

__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(r.x, r.y, r.z, r.w);
}

// Raw buffer reads: a resource over `bytes` bytes from `base` (uniform), read at 32-bit byte
// offsets; a read past `bytes` returns zeros. The fourth descriptor word is the raw-buffer format
// of the gfx9 family. The address of a read is one 32-bit register, not a 64-bit pair.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), short(0), int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, int(byte_off), 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------------------------
// DPP lane exchanges inside 16-lane rows: xor 1, xor 2 (quad permutes), then the half-row and row
// mirrors. Applied in that order, a commutative combine leaves every lane of the row holding the
// bit-identical row result, with no LDS traffic.
// ---------------------------------------------------------------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
// Orders one wave's LDS writes before its later LDS reads when its lanes pass values through LDS
// without a workgroup barrier: every write issued before it is done, and no read after it is
// moved above it (the compiler may otherwise place a branch's reads before another branch's
// writes: lanes are independent threads to it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// maximum and sum over each quad of lanes (every lane of the quad ends with the same bits: the
// pairs are added in either order, then the two pair sums)
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  return fmaxf(v, dpp_f<kDppXor2>(v));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  return v + dpp_f<kDppXor2>(v);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}

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
// wave64 reductions without LDS: DPP inside each 16-lane row (every lane of the row ends with the
// bit-identical row result), then the four row results are read into scalar registers and
// combined in the fixed order (row0 . row1) . (row2 . row3). Every lane returns the same bits.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
// min over the four rows of a value that is already uniform within each row
__device__ __forceinline__ float rows_min(float v) {
  return fminf(fminf(readlane_f(v, 0), readlane_f(v, 16)), fminf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppXor1, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppXor2, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppXor1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppXor2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ bool key_gt(uint32_t ah, uint32_t al, uint32_t bh, uint32_t bl) {
  return ah > bh || (ah == bh && al > bl);
}
// 64-bit DPP move: both halves through the same lane pattern; lanes the row mask leaves out keep v
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = int(uint32_t(v)), hi = int(uint32_t(v >> 32));
  const uint32_t l = uint32_t(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false));
  const uint32_t h = uint32_t(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false));
  return (uint64_t(h) << 32) | l;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
// unsigned 32-bit maximum over the wave: DPP maxima inside 16-lane rows, then row_bcast:15 and
// row_bcast:31 carry rows 0..2 into row 3, whose last lane holds the result (each step one DPP max)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x142, 0xA, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x143, 0xC, 0xF, false)));
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}
// unsigned 64-bit maximum over the wave as two 32-bit maxima: the high words, then the low words of
// the lanes whose high word is that maximum (a 64-bit step would take a compare and two selects)
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = uint32_t(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? uint32_t(v) : 0u);
  return (uint64_t(mh) << 32) | ml;
}
// lexicographic max of (hi, lo) key pairs over the wave
__device__ __forceinline__ void wave_max_key(uint32_t& hi, uint32_t& lo) {
  const uint64_t m = wave_max_u64((uint64_t(hi) << 32) | lo);
  hi = uint32_t(m >> 32);
  lo = uint32_t(m);
}

// Unsigned maxima of quads and minima of 16-lane rows (DPP; every lane of the group ends with
// the group result), and the number of values in a lane's 16-lane row strictly larger than its
// own (each of the 15 row rotations compared once).
__device__ __forceinline__ uint32_t quad_max_u(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  return max(v, dpp_u<kDppXor2>(v));
}
__device__ __forceinline__ uint32_t row16_max_u(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  return max(v, dpp_u<kDppMirror>(v));
}
__device__ __forceinline__ uint32_t row16_min_u(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  return min(v, dpp_u<kDppMirror>(v));
}
template <int D>
__device__ __forceinline__ int larger_at_rotation(uint32_t v) {  // DPP row_ror:D
  return dpp_u<0x120 + D>(v) > v ? 1 : 0;
}
__device__ __forceinline__ int row16_count_larger(uint32_t v) {
  return ((larger_at_rotation<1>(v) + larger_at_rotation<2>(v)) + (larger_at_rotation<3>(v) + larger_at_rotation<4>(v))) +
         ((larger_at_rotation<5>(v) + larger_at_rotation<6>(v)) + (larger_at_rotation<7>(v) + larger_at_rotation<8>(v))) +
         ((larger_at_rotation<9>(v) + larger_at_rotation<10>(v)) + (larger_at_rotation<11>(v) + larger_at_rotation<12>(v))) +
         ((larger_at_rotation<13>(v) + larger_at_rotation<14>(v)) + larger_at_rotation<15>(v));
}

// Inclusive scan over the wave: Hillis-Steele inside each row (DPP row shifts 1, 2, 4, 8), then
// row 0's total is added to row 1 and row 2's to row 3 (row_bcast:15), and row 1's running total
// to rows 2 and 3 (row_bcast:31). Lanes a shift would read from outside the row add 0.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143, kDppWaveShr1 = 0x138;
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowShr1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowShr2, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowShr4, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowShr8, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppBcast15, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppBcast31, 0xC, 0xF, false));
  return v;
}
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppBcast31, 0xC, 0xF, false);
  return v;
}
// value of the previous lane (0 in lane 0)
__device__ __forceinline__ float wave_shift_up1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppWaveShr1, 0xF, 0xF, false));
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
  const float inc = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  float base = 0.f;
  for (int i = 0; i < w; ++i) base += sh[i];
  const float excl_lane = wave_shift_up1(inc);
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

// ---------------------------------------------------------------------------------------------
// Row tiles: thread t of a 256-thread block owns the kSubElems contiguous tokens starting at
// c0 + 8 t of each row. load_raw keeps them packed (one uint4 per 16 bytes); positions at or past
// V read as -inf. Vector loads need the row 16-byte aligned.
// ---------------------------------------------------------------------------------------------
template <class ET>
struct RawTile {
  static constexpr int kWords = kSubElems * sizeof(typename ET::T) / 16;  // uint4 per thread
  uint4 w[kWords];
};

// Vector path: the thread's 8 tokens are whole and 16-byte aligned. Decided once per thread, so a
// run of row loads compiles to back-to-back vector loads with no waits in between.
template <class ET>
__device__ __forceinline__ void load_raw_vec(const typename ET::T* __restrict__ row, int e0,
                                             RawTile<ET>& r) {
#pragma unroll
  for (int h = 0; h < RawTile<ET>::kWords; ++h) r.w[h] = load16(row + e0 + h * ET::kVec);
}

template <class ET>
__device__ __forceinline__ void load_raw_scalar(const typename ET::T* __restrict__ row,
                                                          int e0, int V, RawTile<ET>& r) {
  constexpr int NW = RawTile<ET>::kWords;
  uint32_t words[NW * 4];
  if (sizeof(typename ET::T) == 4) {
#pragma unroll
    for (int e = 0; e < kSubElems; ++e)
      words[e] = (e0 + e < V) ? __float_as_uint(ET::one(row, e0 + e)) : 0xFF800000u;
  } else {
#pragma unroll
    for (int e = 0; e < kSubElems; e += 2) {
      const uint32_t lo = (e0 + e < V) ? (__float_as_uint(ET::one(row, e0 + e)) >> 16) : 0xFF80u;
      const uint32_t hi = (e0 + e + 1 < V) ? (__float_as_uint(ET::one(row, e0 + e + 1)) >> 16) : 0xFF80u;
      words[e / 2] = lo | (hi << 16);
    }
  }
#pragma unroll
  for (int h = 0; h < NW; ++h)
    r.w[h] = make_uint4(words[4 * h], words[4 * h + 1], words[4 * h + 2], words[4 * h + 3]);
}

template <class ET>
__device__ __forceinline__ void load_raw(const typename ET::T* __restrict__ row, int e0, int V,
                                         bool aligned, RawTile<ET>& r) {
  if (aligned && e0 + kSubElems <= V)
    load_raw_vec<ET>(row, e0, r);
  else
    load_raw_scalar<ET>(row, e0, V, r);
}

template <class ET>
__device__ __forceinline__ void unpack_tile(const RawTile<ET>& r, float (&z)[kSubElems]) {
#pragma unroll
  for (int h = 0; h < RawTile<ET>::kWords; ++h) ET::unpack(r.w[h], z + h * ET::kVec);
}

// Residual (qrow != nullptr) or target-row values of this thread's tokens of a tile:
// r = max(p - q w / N, 0) with w = C on the Saguaro set (w_in = C / N, w_out = 1 / N), or r = p.
template <class ET>
__device__ __forceinline__ void sub_values(const typename ET::T* __restrict__ prow,
                                           const typename ET::T* __restrict__ qrow, int c0, int V,
                                           bool aligned, float c, float Lp, float Lq, float w_out,
                                           float w_in, const int* set_entries, int n_set,
                                           float (&r)[kSubElems]) {
  const int e0 = c0 + threadIdx.x * kSubElems;
  RawTile<ET> rp, rq;
  load_raw<ET>(prow, e0, V, aligned, rp);
  if (qrow) load_raw<ET>(qrow, e0, V, aligned, rq);
  float zp[kSubElems], zq[kSubElems];
  unpack_tile<ET>(rp, zp);
  if (qrow) unpack_tile<ET>(rq, zq);
  uint32_t in_set = 0;  // bit e: token e0 + e belongs to the Saguaro set
  for (int f = 0; f < n_set; ++f) {
    const unsigned d = unsigned(set_entries[f] - e0);
    if (d < unsigned(kSubElems)) in_set |= 1u << d;
  }
#pragma unroll
  for (int e = 0; e < kSubElems; ++e) {
    const float pv = ex2(fmaf(zp[e], c, -Lp));
    if (qrow) {
      const float w = ((in_set >> e) & 1u) ? w_in : w_out;
      const float qv = ex2(fmaf(zq[e], c, -Lq)) * w;
      r[e] = fmaxf(pv - qv, 0.f);
    } else {
      r[e] = pv;
    }
    if (e0 + e >= V) r[e] = 0.f;
  }
}

// Scan this thread's values, then the block: per-element inclusive prefixes (relative to the tile
// start) in pre[], tile total returned (equal to the last thread's last inclusive prefix).
__device__ __forceinline__ float sub_scan(const float (&r)[kSubElems], float (&pre)[kSubElems],
                                          float* shf) {
  float run = 0.f;
#pragma unroll
  for (int e = 0; e < kSubElems; ++e) {
    run += r[e];
    pre[e] = run;
  }
  float total;
  const float excl = block_excl_scan(run, shf, total);
#pragma unroll
  for (int e = 0; e < kSubElems; ++e) pre[e] = excl + pre[e];
  return total;
}

}  // namespace ssd
