// gfx950 kernels for the standalone SSD / Saguaro pieces: top-F bonus-token guesses, Saguaro
// down-weighting (alone, with the row's own top-F set, and with the draft token drawn from the
// down-weighted distribution), and the speculation-cache keys and lookup. (Verification itself
// lives in ssd_verify.hip.) Rows are cut into chunks; one 256-thread workgroup streams one chunk
// with 16-byte loads, then, when a row has several chunks, a second launch merges the chunks'
// partial results per row.
#include <hip/hip_runtime.h>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_plan.hpp"

namespace ssd {

// ---------------------------------------------------------------------------------------------
// Phase-1 chunk pass. Thread t streams vectors t, t+256, ... of the chunk [c0, c1), so each
// thread meets its indices in increasing order (the top-F tie rule relies on it).
// STATS: running (mx, s) with s = sum 2^(z c - mx c). FM > 0: per-thread top-F list.
// ---------------------------------------------------------------------------------------------
template <class ET, bool STATS, int FM>
__device__ __forceinline__ void chunk_pass(const typename ET::T* __restrict__ row, int c0, int c1,
                                           bool aligned, float c, int exclude, float& mx, float& s,
                                           TopList<(FM > 0 ? FM : 1)>& tl) {
  constexpr int N = ET::kVec;
  constexpr int U = 32 / N;  // 32 values per thread per batch
  const int t = threadIdx.x;
  const bool topf = (FM > 0) && (tl.F > 0);

  auto consume1 = [&](float z, int idx) {
    if (STATS && z > -INFINITY) {  // a -inf token adds nothing (also before the first finite one)
      if (z > mx) {
        s = (mx > -INFINITY) ? s * ex2((mx - z) * c) : 0.f;
        mx = z;
      }
      s += ex2(fmaf(z, c, -(mx * c)));
    }
    if (FM > 0) {
      if (topf) tl.offer(z, idx, exclude);
    }
  };

  int tail0 = c0;
  if (aligned) {
    const uint4* rv = reinterpret_cast<const uint4*>(row);
    const int v0 = c0 / N;
    const int v1 = v0 + (c1 - c0) / N;
    tail0 = v1 * N;
    for (int vb = v0 + t; vb < v1; vb += kThreads * U) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vi = vb + u * kThreads;
        raw[u] = (vi < v1) ? load16(rv + vi)
                           : make_uint4(ET::kNegInfWord, ET::kNegInfWord, ET::kNegInfWord,
                                        ET::kNegInfWord);
      }
      float z[U * N];
#pragma unroll
      for (int u = 0; u < U; ++u) ET::unpack(raw[u], z + u * N);
      float bm = z[0];
#pragma unroll
      for (int m = 1; m < U * N; ++m) bm = fmaxf(bm, z[m]);
      if (STATS && bm > -INFINITY) {  // a batch of -inf adds nothing (also before the first finite one)
        if (bm > mx) {
          s = (mx > -INFINITY) ? s * ex2((mx - bm) * c) : 0.f;
          mx = bm;
        }
        const float mc = mx * c;
        float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
#pragma unroll
        for (int m = 0; m < U * N; m += 4) {
          acc0 += ex2(fmaf(z[m + 0], c, -mc));
          acc1 += ex2(fmaf(z[m + 1], c, -mc));
          acc2 += ex2(fmaf(z[m + 2], c, -mc));
          acc3 += ex2(fmaf(z[m + 3], c, -mc));
        }
        s += (acc0 + acc1) + (acc2 + acc3);
      }
      if (FM > 0) {
        if (topf && bm > tl.thr) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int base = (vb + u * kThreads) * N;
#pragma unroll
            for (int e = 0; e < N; ++e) tl.offer(z[u * N + e], base + e, exclude);
          }
        }
      }
    }
    // elements after the last whole vector (only when the chunk end is not vector aligned)
    const int e = tail0 + t;
    if (e < c1) consume1(ET::one(row, e), e);
  } else {
    for (int e = c0 + t; e < c1; e += kThreads) consume1(ET::one(row, e), e);
  }
}

// Merge candidate lists: n_lists lists of `stride` entries, of which the first F count. The top F
// (value desc, index asc) go to out[0..F), -1 to out[F..Fmax). Runs on the whole block.
__device__ void merge_lists(const Cand* __restrict__ cands, int n_lists, int stride, int F,
                            int32_t* __restrict__ out, int Fmax, uint32_t* shk,
                            int* sh_set = nullptr) {
  constexpr int kPer = (kMaxChunks * kMaxF + kThreads - 1) / kThreads;
  const int n = n_lists * F;
  if (n <= 4 * 64) {  // up to four keys a lane: wave 0 alone, F rounds of a wave maximum, no barrier
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    uint64_t k[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      k[q] = 0ull;
      if (e < n) {
        const int list = e / F, r = e - list * F;
        const Cand cd = cands[list * stride + r];
        if (cd.i >= 0) k[q] = (uint64_t(ordered_key(cd.v)) << 32) | uint64_t(~uint32_t(cd.i));
      }
    }
    int mine = -1;  // lane f: the f-th best token
    for (int r = 0; r < F; ++r) {
      const uint64_t win = wave_max_u64(max_u64(max_u64(k[0], k[1]), max_u64(k[2], k[3])));
#pragma unroll
      for (int q = 0; q < 4; ++q) k[q] = (k[q] == win) ? 0ull : k[q];  // keys are unique
      if (lane == r) mine = win ? int(~uint32_t(win)) : -1;
    }
    static_assert(kMaxF <= 64, "lane f holds the f-th best");
    if (lane < Fmax) {
      const int v = (lane < F) ? mine : -1;
      out[lane] = v;
      if (sh_set && lane < F) sh_set[lane] = v;
    }
    return;
  }
  uint32_t kh[kPer], kl[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = threadIdx.x + q * kThreads;
    kh[q] = 0;
    kl[q] = 0;
    if (e < n) {
      const int list = e / F, r = e - list * F;
      const Cand cd = cands[list * stride + r];
      if (cd.i >= 0) {
        kh[q] = ordered_key(cd.v);
        kl[q] = ~uint32_t(cd.i);
      }
    }
  }
  for (int r = 0; r < F; ++r) {
    uint32_t bh = 0, bl = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q)
      if (kh[q] > bh || (kh[q] == bh && kl[q] > bl)) {
        bh = kh[q];
        bl = kl[q];
      }
    uint32_t mh = bh, ml = bl;
    wave_max_key(mh, ml);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
      shk[2 * w] = mh;
      shk[2 * w + 1] = ml;
    }
    __syncthreads();
    uint32_t gh = shk[0], gl = shk[1];
#pragma unroll
    for (int q = 1; q < kWaves; ++q)
      if (shk[2 * q] > gh || (shk[2 * q] == gh && shk[2 * q + 1] > gl)) {
        gh = shk[2 * q];
        gl = shk[2 * q + 1];
      }
    if (gh != 0) {
#pragma unroll
      for (int q = 0; q < kPer; ++q)
        if (kh[q] == gh && kl[q] == gl) {
          kh[q] = 0;
          kl[q] = 0;
        }
    }
    if (threadIdx.x == 0) {
      out[r] = (gh != 0) ? int(~gl) : -1;
      if (sh_set) sh_set[r] = (gh != 0) ? int(~gl) : -1;
    }
  }
  for (int r = F + threadIdx.x; r < Fmax; r += kThreads) out[r] = -1;
}

// =============================================================================================
// Standalone top-F guesses
// =============================================================================================
// Each wave keeps a lower bound tau of the F-th best (value desc, index asc) among the tokens it
// has read, and a buffer of candidate keys (ordered value key << 32 | ~index; larger is better)
// in LDS. A batch of 32 tokens per lane whose lane maxima all fall below tau is skipped after one
// ballot; otherwise its tokens at or above tau are appended, and a buffer past max(2F, kTReduce)
// keys is cut to its top F, whose F-th key raises tau (early cuts keep tau near the running F-th
// best, so later batches rarely hold a candidate). The first batch sets tau to the (F+1)-th largest
// lane maximum: F + 1 tokens of distinct lanes reach it, so F of them are not the excluded one.
constexpr int kTBuf = 256;     // candidate keys per wave
constexpr int kTBufSample = 192;  // with the sampling pass's per-lane segment pairs in LDS too
constexpr int kTReduce = 16;   // cut the buffer to its top F beyond max(2F, this) keys
constexpr int kTBatch = 32;    // tokens per lane per batch

__device__ __forceinline__ uint64_t cand_key64(float v, int idx) {
  return (uint64_t(ordered_key(v)) << 32) | uint64_t(~uint32_t(idx));
}

// The top F of the n keys in buf (keys unique, n <= BUF), in order, to buf[0 .. m); returns m <= F.
template <int BUF>
__device__ __forceinline__ int wave_cut_keys(uint64_t* buf, int n, int F) {
  static_assert(BUF % 64 == 0, "whole keys per lane");
  const int lane = threadIdx.x & 63;
  constexpr int kPer = BUF / 64;
  uint64_t k[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) k[i] = (lane + 64 * i < n) ? buf[lane + 64 * i] : 0ull;
  uint64_t mine_out = 0;
  int m = 0;
  for (int f = 0; f < F; ++f) {
    uint64_t mine = k[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) mine = max_u64(mine, k[i]);
    const uint64_t win = wave_max_u64(mine);
    if (win == 0ull) break;
#pragma unroll
    for (int i = 0; i < kPer; ++i) k[i] = (k[i] == win) ? 0ull : k[i];
    if (lane == f) mine_out = win;
    ++m;
  }
  if (lane < m) buf[lane] = mine_out;
  return m;
}

template <class ET, int BUF>
struct TopfWave {
  uint64_t* buf;  // this wave's BUF keys
  int n;          // keys in buf (wave-uniform)
  float tau;      // lower bound of the F-th best so far (wave-uniform); -inf: none yet
  int F, exclude;
  // The workgroup's bound in LDS (order key; 0: none): every wave raises it to its own tau and
  // takes it up before each batch. A wave's tau has F tokens of its own at or above it (F + 1 from
  // the first batch's lane maxima, one of which may be the excluded token), so no token below it is
  // among the row's best F, whichever wave holds the token; the bound only prunes sooner.
  uint32_t* shared_tau;
  __device__ __forceinline__ void take_shared() {
    const uint32_t k = __hip_atomic_load(shared_tau, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (k > ordered_key(tau)) tau = key_to_float(k);
  }
  __device__ __forceinline__ void give_shared() {
    if ((threadIdx.x & 63) == 0 && tau > -INFINITY)
      __hip_atomic_fetch_max(shared_tau, ordered_key(tau), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // one batch: lane tokens z[0..NB) (-inf for a place past the chunk), token index of place e
  // from idx_of(e) (evaluated only for batches that reach tau)
  template <int NB, class Idx>
  __device__ __forceinline__ void batch(const float (&z)[NB], Idx idx_of) {
    float bm = z[0];
#pragma unroll
    for (int e = 1; e < NB; ++e) bm = fmaxf(bm, z[e]);
    batch_bm(z, bm, idx_of);
  }
  // the same with the lane maximum bm of z already formed
  template <int NB, class Idx>
  __device__ __forceinline__ void batch_bm(const float (&z)[NB], float bm, Idx idx_of) {
    // a row with no excluded token skips the per-token index test (uniform)
    if (exclude < 0)
      batch_ex<false>(z, bm, idx_of);
    else
      batch_ex<true>(z, bm, idx_of);
  }
  template <bool EX, int NB, class Idx>
  __device__ __forceinline__ void batch_ex(const float (&z)[NB], float bm, Idx idx_of) {
    auto keep = [&](int e) __attribute__((always_inline)) { return !EX || idx_of(e) != exclude; };
    const int lane = threadIdx.x & 63;
    take_shared();
    if (tau == -INFINITY && n == 0) {  // first batch: tau from the lane maxima
      const int Fp = F + 1;
      float mm = bm, thr = -INFINITY;
      int taken = 0;
      for (int f = 0; f < Fp; ++f) {
        const float cur = wave_max(mm);
        if (!(cur > -INFINITY)) break;
        thr = cur;
        taken += __popcll(__ballot(mm == cur));
        if (taken >= Fp) break;
        mm = (mm == cur) ? -INFINITY : mm;
      }
      if (taken >= Fp) {
        tau = thr;
        give_shared();
      }
    }
    if (__ballot(bm >= tau && bm > -INFINITY) == 0ull) return;  // nothing here reaches tau
    // Groups of GS places: only a group where some lane of the wave reaches tau is examined (a
    // batch that reaches tau mostly does so in one or two places of a few lanes). The candidates
    // are the same, appended in the same order.
    constexpr int GS = (NB % 8 == 0) ? 8 : 1, NG = NB / GS;
    uint32_t gmask = 0;  // wave-uniform: groups with a place at or above tau in some lane
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float gm = z[g * GS];
#pragma unroll
      for (int e = 1; e < GS; ++e) gm = fmaxf(gm, z[g * GS + e]);
      if (__ballot(gm >= tau && gm > -INFINITY) != 0ull) gmask |= 1u << g;
    }
    auto pass = [&](int e) __attribute__((always_inline)) { return z[e] >= tau && z[e] > -INFINITY && keep(e); };
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if ((gmask >> g) & 1u) {
#pragma unroll
        for (int e = g * GS; e < (g + 1) * GS; ++e) cnt += pass(e) ? 1 : 0;
      }
    const int incl = wave_incl_scan_i(cnt);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (n + total <= BUF) {
      int pos = n + incl - cnt;
#pragma unroll
      for (int g = 0; g < NG; ++g)
        if ((gmask >> g) & 1u) {
#pragma unroll
          for (int e = g * GS; e < (g + 1) * GS; ++e)
            if (pass(e)) buf[pos++] = cand_key64(z[e], idx_of(e));
        }
      n += total;
    } else {
      // too many to append at once (ties): one place of every lane at a time, cutting the buffer
      // (and raising tau) whenever the next place would not fit
      for (int e = 0; e < NB; ++e) {
        bool c = z[e] >= tau && z[e] > -INFINITY && keep(e);
        uint64_t m = __ballot(c);
        if (m == 0ull) continue;
        if (n + __popcll(m) > BUF) {
          n = wave_cut_keys<BUF>(buf, n, F);
          if (n == F) {
            tau = key_to_float(uint32_t(buf[F - 1] >> 32));
            give_shared();
          }
          c = c && z[e] >= tau;
          m = __ballot(c);
        }
        if (c) buf[n + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)))] =
            cand_key64(z[e], idx_of(e));
        n += __popcll(m);
      }
    }
    if (n > max(2 * F, kTReduce)) {
      n = wave_cut_keys<BUF>(buf, n, F);
      if (n == F) {
        tau = key_to_float(uint32_t(buf[F - 1] >> 32));
        give_shared();
      }
    }
  }
};

// Running softmax statistics of a lane's tokens: mx = largest logit so far, s = sum of
// 2^(z c - mx c). A place at -inf adds nothing (also before the first finite token).
struct LaneStats {
  float mx = -INFINITY, s = 0.f;
  template <int NB>
  __device__ __forceinline__ void add(const float (&z)[NB], float bm, float c) {
    if (!(bm > -INFINITY)) return;
    if (bm > mx) {
      s = (mx > -INFINITY) ? s * ex2((mx - bm) * c) : 0.f;
      mx = bm;
    }
    const float mc = mx * c;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < NB; ++e) acc[e % 4] += ex2(fmaf(z[e], c, -mc));
    s += (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
};

// =============================================================================================
// Draft-side Saguaro sampling: the inverse CDF of q' in ascending token order
// =============================================================================================
// The streaming pass leaves every segment of seg_len tokens its q mass as a (max c, sum) pair. The
// segment where the cumulative q' mass first exceeds u times the total is found from those pairs
// (one segment per lane, every wave on its own when there are at most 64, else one per thread over
// the block; the set members' share of a segment is scaled by C), then only that segment is read
// again, each thread owning seg_len / 256 consecutive tokens: a block scan of the runs' masses
// names the run, whose thread walks it token by token. When rounding leaves the
// target past the last crossing, the last token of positive mass is taken (segment, then run).
constexpr float kSegEps = 9.5367431640625e-07f;  // 2^-20: a segment's q' mass below this share of
                                                 // its q mass is cancellation left over, not mass
static_assert(kPlanSampleSpan == kThreads * kTBatch, "a sampling segment is whole top-F batches");
// tokens of one thread's run when a segment is one batch (the register-held case below)
constexpr int kRunTok = kPlanSampleSpan / kThreads;

// The segment a row's draw falls in, from the segments' q masses alone (the set's down-weighting
// left out): every wave finds it by itself, lane i taking segment i (ns <= 64); -1 if none. Only a
// guess of the draw's segment, good for requesting its tokens early.
__device__ __forceinline__ int guess_segment(const float2* segm, int ns, float L, float u) {
  const int lane = threadIdx.x & 63;
  float m = 0.f;
  if (lane < ns) {
    const float2 r = segm[lane];
    m = (r.y > 0.f) ? r.y * ex2(r.x - L) : 0.f;
  }
  const float inc = wave_incl_scan(m);
  const float prev = wave_shift_up1(inc);
  const float tau = u * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
  const uint64_t hit = __ballot(m > 0.f && prev + m > tau);
  return hit ? int(__builtin_ctzll(hit)) : -1;
}

// tokens [b0, b1) of row p in ascending order, 16-byte loads when aligned (b0 % kVec == 0)
template <class ET, class Fn>
__device__ __forceinline__ void for_run(const typename ET::T* __restrict__ p, int b0, int b1, bool aligned,
                                        Fn fn) {
  constexpr int N = ET::kVec;
  int e = b0;
  if (aligned) {
    for (; e + N <= b1; e += N) {
      float z[N];
      ET::unpack(load16(p + e), z);
#pragma unroll
      for (int j = 0; j < N; ++j) fn(z[j], e + j);
    }
  }
  for (; e < b1; ++e) fn(ET::one(p, e), e);
}

// Whole block. segm: ns <= 256 segment pairs (LDS); set / zs: the F set members and their logits
// (LDS, -1 for an empty place); L = log2 of the row's normaliser in the units of z c. Writes the
// token (-1 when q' has no mass) and q' of it. shf >= kWaves + 2 floats, shi >= kWaves ints.
// sg0 / pre: a segment guessed earlier and this thread's run of it, already requested (sg0 = -1:
// none); used when the draw does fall in that segment.
template <class ET>
__device__ __forceinline__ void block_sample(const typename ET::T* __restrict__ p, int V, bool aligned,
                                             const float2* segm, int ns, int seg_len, float L, float cc, float Cr,
                                             float Nn, const int* set, const float* zs, int F, float u, float* shf,
                                             int* shi, int32_t* out_token, float* out_prob, uint32_t* flags,
                                             int sg0, const uint4 (&pre)[kRunTok / ET::kVec]) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // q' mass of segment i (i < ns)
  auto seg_mass = [&](int i) {
    const float2 r = segm[i];
    const float mq = (r.y > 0.f) ? r.y * ex2(r.x - L) : 0.f;
    float in_set = 0.f;
    for (int f = 0; f < F; ++f)
      if (set[f] >= i * seg_len && set[f] < (i + 1) * seg_len) in_set += ex2(fmaf(zs[f], cc, -L));
    const float mp = mq - (1.f - Cr) * in_set;
    return (mp > kSegEps * mq) ? mp : 0.f;
  };
  int sg;
  float rem = INFINITY;  // tau less the mass before the segment; +inf: its last token of mass
  if (ns <= 64) {
    // Every wave finds the segment by itself, lane i taking segment i: no barrier. These are the
    // sums the block-wide scan below forms, as every segment sits in its first wave.
    const float m = (lane < ns) ? seg_mass(lane) : 0.f;
    const float inc = wave_incl_scan(m);
    const float prev = wave_shift_up1(inc);  // outside the select: every lane takes part
    const float base = 0.f;
    const float excl = (lane == 0) ? base : base + prev;
    const float tau = u * __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inc), 63));
    const uint64_t hit = __ballot(m > 0.f && excl + m > tau);
    if (hit) {
      sg = __builtin_ctzll(hit);
      rem = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tau - excl), sg));
    } else {
      const uint64_t pos = __ballot(m > 0.f);
      sg = pos ? 63 - __builtin_clzll(pos) : -1;
    }
  } else {
    const float m = (t < ns) ? seg_mass(t) : 0.f;
    float Z;
    const float excl = block_excl_scan(m, shf, Z);
    const float tau = u * Z;
    sg = block_min_i((m > 0.f && excl + m > tau) ? t : INT_MAX, shi);
    if (sg == INT_MAX) {
      sg = block_max_i(m > 0.f ? t : -1, shi);
    } else {
      if (t == sg) shf[kWaves + 1] = tau - excl;
      __syncthreads();
      rem = shf[kWaves + 1];
    }
  }
  if (sg < 0 || !(Nn > 0.f)) {  // no mass: a masked row, or C = 0 with the set holding it all
    if (t == 0) {
      *out_token = -1;
      if (out_prob) *out_prob = 0.f;
      if (L > -INFINITY) atomicOr(flags, kFlagSaguaroNorm);  // N = 0 up to rounding
    }
    return;
  }
  float zmin = INFINITY;  // smallest logit of the set: cheaper membership test
  for (int f = 0; f < F; ++f)
    if (set[f] >= 0) zmin = fminf(zmin, zs[f]);
  auto mass = [&](float z, int e) {
    float wgt = 1.f;
    if (z >= zmin)
      for (int f = 0; f < F; ++f)
        if (set[f] == e) wgt = Cr;
    return wgt * ex2(fmaf(z, cc, -L));
  };
  const int a0 = sg * seg_len, a1 = min(V, a0 + seg_len);
  const int run = seg_len / kThreads;
  const int b0 = min(a1, a0 + t * run), b1 = min(a1, b0 + run);
  // A run of exactly kRunTok tokens of an aligned row (a one-batch segment: the usual case) is read
  // with all its loads in flight at once and its masses kept in registers, so the walk below reads
  // nothing again; any other run streams through for_run. Both take the same steps in the same
  // order, so the result does not depend on which one a thread takes.
  constexpr int N = ET::kVec;
  const bool held = aligned && b1 - b0 == kRunTok;  // b0 is a multiple of kRunTok: 16-byte aligned
  float qr[kRunTok];
  float sum = 0.f, qlp = 0.f;
  int lp = -1;
  if (held) {
    uint4 raw[kRunTok / N];
    if (sg == sg0) {  // requested already
#pragma unroll
      for (int j = 0; j < kRunTok / N; ++j) raw[j] = pre[j];
    } else {
#pragma unroll
      for (int j = 0; j < kRunTok / N; ++j) raw[j] = load16(p + b0 + j * N);
    }
    uint32_t in_set = 0;  // bit j: token b0 + j is a set member (weight Cr, as in mass)
    for (int f = 0; f < F; ++f) {
      const int d = set[f] - b0;
      if (set[f] >= 0 && d >= 0 && d < kRunTok) in_set |= 1u << d;
    }
#pragma unroll
    for (int j = 0; j < kRunTok / N; ++j) ET::unpack(raw[j], qr + j * N);
#pragma unroll
    for (int j = 0; j < kRunTok; ++j) {
      const float q = (((in_set >> j) & 1u) ? Cr : 1.f) * ex2(fmaf(qr[j], cc, -L));
      qr[j] = q;
      sum += q;
      if (q > 0.f) {
        lp = b0 + j;
        qlp = q;
      }
    }
  } else {
    for_run<ET>(p, b0, b1, aligned, [&](float z, int e) {
      const float q = mass(z, e);
      sum += q;
      if (q > 0.f) lp = e;
    });
  }
  // the run holding the target: an exclusive scan of the runs' masses over the block (each wave's
  // total after the earlier waves' totals, in order), then the first run whose end passes it
  const float inc = wave_incl_scan(sum);
  if (lane == 63) shf[w] = inc;
  __syncthreads();
  float base = 0.f;
  for (int i = 0; i < w; ++i) base += shf[i];
  // the cross-lane read outside the select: a lane inside a branch that leaves lane 0 out would
  // read 0 from it
  const float prev = wave_shift_up1(inc);
  const float ex = (lane == 0) ? base : base + prev;
  const uint64_t own = __ballot(sum > 0.f && ex + sum > rem);
  if (lane == 0) shi[w] = own ? w * 64 + __builtin_ctzll(own) : INT_MAX;
  __syncthreads();
  const int owner = min(min(shi[0], shi[1]), min(shi[2], shi[3]));
  int x = -1;
  bool writer = false, have_q = false;
  float qx = 0.f;  // q mass of x, when this thread holds it
  if (owner == INT_MAX) {
    x = block_max_i(lp, shi);
    writer = (t == 0);
  } else if (t == owner) {
    float c = ex;
    if (held) {
#pragma unroll
      for (int j = 0; j < kRunTok; ++j) {  // the running sum stops at the first crossing
        const bool live = x < 0;
        c = live ? c + qr[j] : c;
        const bool hit = live && c > rem;
        x = hit ? b0 + j : x;
        qx = hit ? qr[j] : qx;
      }
      if (x < 0) {
        x = lp;
        qx = qlp;
      }
      have_q = true;
    } else {
      for_run<ET>(p, b0, b1, aligned, [&](float z, int e) {
        if (x < 0) {
          c += mass(z, e);
          if (c > rem) x = e;
        }
      });
      if (x < 0) x = lp;
    }
    writer = true;
  }
  if (writer) {
    *out_token = x;
    if (out_prob) {
      if (x >= 0 && !have_q) qx = mass(ET::one(p, x), x);
      *out_prob = (x >= 0) ? qx / Nn : 0.f;
    }
  }
}

// SAG: ssd_saguaro_topf — the row's statistics in the same pass, and sigma = q mass of the top F
// with N = 1 - (1 - C) sigma once the row is complete (here when a row is one chunk, else in the
// merge kernel). SMP (with SAG): ssd_saguaro_sample — the statistics are kept per segment and a
// token is drawn from q' once the row is complete.
template <class ET, int FM, bool SAG, bool SMP>
__global__ __launch_bounds__(kThreads) void topf_rows_kernel(TopfArgs a) {
  static_assert(SAG || !SMP, "sampling needs the row statistics");
  using T = typename ET::T;
  constexpr int N = ET::kVec;
  constexpr int U = kTBatch / N;  // vectors per lane per batch
  constexpr int NS = SMP ? kPlanMaxSeg : 1;
  constexpr int BUF = SMP ? kTBufSample : kTBuf;
  __shared__ uint64_t sbuf[kWaves][BUF];
  __shared__ uint64_t stop[kWaves][kMaxF];
  __shared__ float shf[2 * kWaves];
  __shared__ float2 lrec[NS][SMP ? kThreads : 1];  // per segment and lane: (max, sum 2^(z c - max c))
  __shared__ float2 segm[NS];                      // per segment, over the block: (max c, sum)
  __shared__ int s_set[SMP ? kMaxF : 1];
  __shared__ float s_zs[SMP ? kMaxF : 1];
  __shared__ float s_lnc[3];
  __shared__ int shi[kWaves];
  LaneStats ls;
  const float cc = a.c2;
  const int item = blockIdx.x;
  const int row = item / a.n1;
  const int chunk = item - row * a.n1;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int F = a.Fmax;
  if (a.F_per_row) {
    F = a.F_per_row[row];
    if (F < 0 || F > a.Fmax) {
      if (chunk == 0 && t == 0) atomicOr(a.flags, kFlagBadF);
      F = F < 0 ? 0 : a.Fmax;
    }
  }
  const int ex = a.exclude ? a.exclude[row] : -1;
  // the row's Saguaro factor and uniform are read now, so they are here when the row is complete
  const bool whole_row = a.n1 == 1;
  const float Cr = (SAG && whole_row) ? row_saguaro_c(a.C_per_row, a.C, row, a.flags, t == 0) : 1.f;
  const float u_row = (SMP && whole_row) ? a.u[row] : 0.f;
  const T* p = reinterpret_cast<const T*>(a.logits) + int64_t(row) * a.row_stride;
  const int c0 = chunk * a.chunk1;
  const int c1 = min(a.V, c0 + a.chunk1);
  __shared__ uint32_t s_tau;
  if (t == 0) s_tau = 0u;
  __syncthreads();
  TopfWave<ET, BUF> tw;
  tw.buf = sbuf[w];
  tw.n = 0;
  tw.tau = -INFINITY;
  tw.F = F;
  tw.exclude = ex;
  tw.shared_tau = &s_tau;
  // SMP: a lane's statistics cover the current segment only; at a segment's end the lane's pair
  // goes to LDS (every lane takes part in every batch, so each segment of the chunk gets all 256)
  // and the lane starts again; the pairs are merged once, after the pass
  int cur_seg = 0, seg_batches = 0;
  const int G = SMP ? a.seg_len / kPlanSampleSpan : 1;
  auto seg_flush = [&]() __attribute__((always_inline)) {
    if constexpr (SMP) lrec[cur_seg][t] = make_float2(ls.mx, ls.s);
    ls.mx = -INFINITY;
    ls.s = 0.f;
  };
  if (F > 0 || SMP) {
    int tail0 = c0;
    if (a.aligned) {
      // thread t reads vectors t, t + 256, ... of the chunk, U per batch
      const uint4* rv = reinterpret_cast<const uint4*>(p);
      const int v0 = c0 / N, v1 = v0 + (c1 - c0) / N;
      tail0 = v1 * N;
      // Batches are numbered by their first vector b0 (the same in every lane: loop control stays
      // scalar). Every lane reads every vector of a batch from a clamped, valid address, so no
      // branch surrounds a read and a wave waits only for the batch it is about to use; vectors
      // past the chunk are replaced by -inf, which only the chunk's last batch needs.
      const __amdgpu_buffer_rsrc_t rsrc = buffer_rsrc(rv, uint32_t(v1) * 16u);
      auto load_batch = [&](int b0, uint4 (&raw)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = buffer_load16(rsrc, uint32_t(min(b0 + t + u * kThreads, v1 - 1)) * 16u);
      };
      auto run_batch = [&](int b0, const uint4 (&raw)[U]) __attribute__((always_inline)) {
        float z[kTBatch];
#pragma unroll
        for (int u = 0; u < U; ++u) ET::unpack(raw[u], z + u * N);
        if (b0 + kThreads * U > v1) {  // uniform: the chunk ends inside this batch
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const bool in = b0 + t + u * kThreads < v1;
#pragma unroll
            for (int e = 0; e < N; ++e) z[u * N + e] = in ? z[u * N + e] : -INFINITY;
          }
        }
        float bm = z[0];
#pragma unroll
        for (int e = 1; e < kTBatch; ++e) bm = fmaxf(bm, z[e]);
        if (SMP) {  // batches come in order, G to a segment
          if (seg_batches == G) {
            seg_flush();
            ++cur_seg;
            seg_batches = 0;
          }
          ++seg_batches;
        }
        if (SAG) ls.add(z, bm, cc);
        if (F > 0) tw.batch_bm(z, bm, [&](int e) { return (b0 + t + (e / N) * kThreads) * N + (e % N); });
      };
      // NBUF batches in flight (a third slowed the bf16 pass): a buffer is read again as soon as it
      // has been examined, so the other is always on its way (reads past the last batch repeat the
      // chunk's last vector). The scheduling barriers keep the reads in this order, so a batch waits
      // only for its own reads: were the batches' reads issued in another order before the loop,
      // the loop's first wait would have to cover them all.
      constexpr int NBUF = 2;
      constexpr int kStep = kThreads * U;
      if (v1 > v0) {
        uint4 rbuf[NBUF][U];
#pragma unroll
        for (int i = 0; i < NBUF; ++i) {
          load_batch(v0 + i * kStep, rbuf[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
        for (int b0 = v0;; b0 += NBUF * kStep) {
#pragma unroll
          for (int i = 0; i < NBUF; ++i) {
            run_batch(b0 + i * kStep, rbuf[i]);
            if (b0 + (i + 1) * kStep >= v1) goto chunk_done;
            __builtin_amdgcn_sched_barrier(0);
            load_batch(b0 + (i + NBUF) * kStep, rbuf[i]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      chunk_done:;
      }
    }
    // elements after the last whole vector, or every element of an unaligned row, one per lane
    for (int e0 = tail0; e0 < c1; e0 += kThreads) {
      const int e = e0 + t;
      float z[1];
      z[0] = (e < c1) ? ET::one(p, e) : -INFINITY;
      if (SMP) {
        const int sg = (e0 - c0) / a.seg_len;
        if (sg != cur_seg) {
          seg_flush();
          cur_seg = sg;
        }
      }
      if (SAG) ls.add(z, z[0], cc);
      if (F > 0) tw.batch_bm(z, z[0], [&](int) { return e; });
    }
    if (SMP) seg_flush();
    tw.n = wave_cut_keys<BUF>(tw.buf, tw.n, F);  // the wave's top F, in order
  }
  if (lane < kMaxF) stop[w][lane] = (lane < tw.n) ? tw.buf[lane] : 0ull;
  float MXc = -INFINITY, S = 0.f;  // the chunk's (max c, sum 2^(z c - max c))
  if (SAG && !SMP && F > 0) {
    const float MX = block_max(ls.mx, shf);
    MXc = MX * cc;
    S = block_sum((ls.s > 0.f) ? ls.s * ex2(ls.mx * cc - MXc) : 0.f, shf + kWaves);
  }
  __syncthreads();
  if constexpr (SMP) {  // segment pairs over the block (16 threads a segment, each 16 lanes), then the chunk's
    static_assert(NS * 16 == kThreads, "16 threads merge each segment's lane pairs");
    const int nseg_c = (c1 - c0 + a.seg_len - 1) / a.seg_len;  // segments this chunk has
    const int sgi = t >> 4, j = t & 15;
    float M = -INFINITY, Ss = 0.f;
    if (sgi < nseg_c) {
      float2 r[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) r[q] = lrec[sgi][q * 16 + j];
#pragma unroll
      for (int q = 0; q < 16; ++q) M = fmaxf(M, r[q].x);
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (r[q].y > 0.f) Ss += r[q].y * ex2(r[q].x * cc - M * cc);
    }
    const float Mr = row16_max(M);
    const float Sr = row16_sum((Ss > 0.f) ? Ss * ex2(M * cc - Mr * cc) : 0.f);
    if (j == 0) {
      segm[sgi] = make_float2(Mr * cc, Sr);
      if (a.n1 > 1 && sgi < nseg_c) a.seg[(int64_t(row) * a.n1 + chunk) * a.nseg + sgi] = make_float2(Mr * cc, Sr);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NS; ++q) MXc = fmaxf(MXc, segm[q].x);
#pragma unroll
    for (int q = 0; q < NS; ++q)
      if (segm[q].y > 0.f) S += segm[q].y * ex2(segm[q].x - MXc);
  }
  // One chunk: this thread's run of the segment the draw most likely falls in (the set, merged
  // next, moves it only near a segment's edge) is requested now, to arrive during that merge.
  int sg0 = -1;
  uint4 pre[kRunTok / N];
#pragma unroll
  for (int j = 0; j < kRunTok / N; ++j) pre[j] = make_uint4(0u, 0u, 0u, 0u);
  if (SMP && a.n1 == 1 && a.aligned && a.seg_len == kPlanSampleSpan) {
    const int ns = (a.V + a.seg_len - 1) / a.seg_len;
    sg0 = guess_segment(segm, ns, MXc + lg2(S), u_row);
    const int a0 = sg0 * a.seg_len, a1 = min(a.V, a0 + a.seg_len);
    const int b0 = min(a1, a0 + t * kRunTok);
    if (sg0 >= 0 && min(a1, b0 + kRunTok) - b0 == kRunTok) {
#pragma unroll
      for (int j = 0; j < kRunTok / N; ++j) pre[j] = load16(p + b0 + j * N);
    }
  }
  if (w == 0) {  // the chunk's top F from the waves' lists
    uint64_t k = 0ull;
    if (F > 0 && lane < kWaves * F) k = stop[lane / F][lane % F];
    uint64_t win_out = 0ull;
    for (int f = 0; f < F; ++f) {
      const uint64_t win = wave_max_u64(k);
      k = (k == win) ? 0ull : k;
      if (lane == f) win_out = win;
    }
    if (a.n1 == 1) {
      int32_t* out = a.out + int64_t(row) * a.Fmax;
      for (int r = lane; r < a.Fmax; r += 64) out[r] = (r < F && win_out) ? int(~uint32_t(win_out)) : -1;
      if (SAG) {  // sigma over the set, from the logits its keys carry
        const float L = MXc + lg2(S);
        const float zk = key_to_float(uint32_t(win_out >> 32));
        const float term = (lane < F && win_out) ? ex2(fmaf(zk, cc, -L)) : 0.f;
        const float sig = (F > 0) ? wave_sum(term) : 0.f;
        const float Nn = 1.f - (1.f - Cr) * sig;
        if (lane == 0) {
          if (a.out_set_mass) a.out_set_mass[row] = sig;
          if (a.out_norm) a.out_norm[row] = Nn;
          if (!(Nn > 0.f)) atomicOr(a.flags, kFlagSaguaroNorm);
        }
        if (SMP) {
          if (lane < F) {
            s_set[lane] = win_out ? int(~uint32_t(win_out)) : -1;
            s_zs[lane] = zk;
          }
          if (lane == 0) {
            s_lnc[0] = L;
            s_lnc[1] = Nn;
            s_lnc[2] = Cr;
          }
        }
      }
    } else {
      if (lane < F) {
        Cand* cd = reinterpret_cast<Cand*>(a.cand) + (int64_t(row) * a.n1 + chunk) * a.Fmax;
        cd[lane] = win_out ? Cand{key_to_float(uint32_t(win_out >> 32)), int(~uint32_t(win_out))}
                           : Cand{-INFINITY, -1};
      }
      if (SAG && lane == 0) a.stats[int64_t(row) * a.n1 + chunk] = make_float2(MXc, S);
    }
  }
  if (SMP && a.n1 == 1) {
    __syncthreads();
    const int ns = (a.V + a.seg_len - 1) / a.seg_len;
    block_sample<ET>(p, a.V, a.aligned != 0, segm, ns, a.seg_len, s_lnc[0], cc, s_lnc[2], s_lnc[1], s_set, s_zs,
                     F, u_row, shf, shi, a.out_token + row, a.out_prob ? a.out_prob + row : nullptr,
                     a.flags, sg0, pre);
  }
}

template <class ET, bool SAG, bool SMP>
__global__ __launch_bounds__(kThreads) void topf_merge_kernel(TopfArgs a) {
  __shared__ uint32_t shk[2 * kWaves];
  __shared__ int s_set[kMaxF];
  __shared__ float s_zs[kMaxF];
  __shared__ float2 s_segm[SMP ? kThreads : 1];
  __shared__ float2 s_chunk[SAG ? kMaxChunks : 1];
  __shared__ float shf[2 * kWaves];
  __shared__ int shi[kWaves];
  __shared__ float s_lnc[3];
  const int row = blockIdx.x;
  int F = a.Fmax;
  if (a.F_per_row) {
    F = a.F_per_row[row];
    F = F < 0 ? 0 : (F > a.Fmax ? a.Fmax : F);
  }
  const typename ET::T* p = reinterpret_cast<const typename ET::T*>(a.logits) + int64_t(row) * a.row_stride;
  const Cand* cd = reinterpret_cast<const Cand*>(a.cand) + int64_t(row) * a.n1 * a.Fmax;
  int32_t* out = a.out + int64_t(row) * a.Fmax;
  const int t = threadIdx.x;
  // the chunk (and, sampling, segment) pairs are loaded first so that they arrive during the merge
  float2 chunk_pair = make_float2(-INFINITY, 0.f), seg_pair = make_float2(-INFINITY, 0.f);
  const int ns = SMP ? (a.V + a.seg_len - 1) / a.seg_len : 0;
  if (SAG && t < a.n1) chunk_pair = a.stats[int64_t(row) * a.n1 + t];
  if (SMP && t < ns) seg_pair = a.seg[int64_t(row) * a.n1 * a.nseg + t];
  const float u_row = SMP ? a.u[row] : 0.f;
  const float Cr = SAG ? row_saguaro_c(a.C_per_row, a.C, row, a.flags, t == 0) : 1.f;
  merge_lists(cd, F > 0 ? a.n1 : 0, a.Fmax, F, out, a.Fmax, shk, s_set);
  if (SAG) {
    if (t < a.n1) s_chunk[t] = chunk_pair;
    if (SMP && t < ns) s_segm[t] = seg_pair;
    __syncthreads();  // the set (thread 0 wrote it) and the pairs
    if (t < F) s_zs[t] = (s_set[t] >= 0) ? ET::one(p, s_set[t]) : 0.f;
    __syncthreads();
  }
  if (SAG && t == 0) {  // the row's normaliser, then sigma from the set's logits
    float sig = 0.f;
    float L = -INFINITY;
    {
      float M = -INFINITY;
      for (int q = 0; q < a.n1; ++q) M = fmaxf(M, s_chunk[q].x);
      float S = 0.f;
      for (int q = 0; q < a.n1; ++q)
        if (s_chunk[q].y > 0.f) S += s_chunk[q].y * ex2(s_chunk[q].x - M);
      L = M + lg2(S);
      for (int f = 0; f < F; ++f)
        if (s_set[f] >= 0) sig += ex2(fmaf(s_zs[f], a.c2, -L));
    }
    const float Nn = 1.f - (1.f - Cr) * sig;
    if (a.out_set_mass) a.out_set_mass[row] = sig;
    if (a.out_norm) a.out_norm[row] = Nn;
    if (!(Nn > 0.f)) atomicOr(a.flags, kFlagSaguaroNorm);
    s_lnc[0] = L;
    s_lnc[1] = Nn;
    s_lnc[2] = Cr;
  }
  if (SMP) {
    __syncthreads();
    uint4 none[kRunTok / ET::kVec];
#pragma unroll
    for (int j = 0; j < kRunTok / ET::kVec; ++j) none[j] = make_uint4(0u, 0u, 0u, 0u);
    block_sample<ET>(p, a.V, a.aligned != 0, s_segm, ns, a.seg_len, s_lnc[0], a.c2, s_lnc[2], s_lnc[1], s_set,
                     s_zs, F, u_row, shf, shi, a.out_token + row, a.out_prob ? a.out_prob + row : nullptr,
                     a.flags, -1, none);
  }
}

// =============================================================================================
// Saguaro adjust
// =============================================================================================
template <class ET>
__global__ __launch_bounds__(kThreads) void sag_rows_kernel(SagArgs a) {
  using T = typename ET::T;
  __shared__ float shf[8];
  const int item = blockIdx.x;
  const int row = item / a.n1;
  const int chunk = item - row * a.n1;
  const T* p = reinterpret_cast<const T*>(a.logits) + int64_t(row) * a.row_stride;
  const int c0 = chunk * a.chunk1;
  const int c1 = min(a.V, c0 + a.chunk1);
  float mx = -INFINITY, s = 0.f;
  TopList<1> tl;
  tl.init(0);
  chunk_pass<ET, true, 0>(p, c0, c1, a.aligned != 0, a.c2, -1, mx, s, tl);
  const float MX = block_max(mx, shf);
  const float part = (s > 0.f) ? s * ex2(mx * a.c2 - MX * a.c2) : 0.f;
  const float S = block_sum(part, shf);
  if (threadIdx.x == 0) a.stats[int64_t(row) * a.n1 + chunk] = make_float2(MX * a.c2, S);
}

template <class ET>
__global__ __launch_bounds__(kThreads) void sag_finalize_kernel(SagArgs a) {
  using T = typename ET::T;
  __shared__ float2 s_part[kMaxChunks];
  __shared__ int s_set[kMaxF];
  __shared__ float s_zs[kMaxF];
  __shared__ float s_L, s_N, s_C;
  const int chunk = blockIdx.x, row = blockIdx.y, t = threadIdx.x;
  const int F = a.F, V = a.V;
  const T* p = reinterpret_cast<const T*>(a.logits) + int64_t(row) * a.row_stride;
  if (t < a.n1) s_part[t] = a.stats[int64_t(row) * a.n1 + t];
  int my = -1;
  if (t < F) {
    const int sv = a.set[int64_t(row) * F + t];
    my = (unsigned(sv) < unsigned(V)) ? sv : -1;
    s_set[t] = my;
    s_zs[t] = (my >= 0) ? ET::one(p, my) : 0.f;
  }
  __syncthreads();
  if (t < F && my >= 0)
    for (int g = 0; g < t; ++g)
      if (s_set[g] == my) my = -1;
  __syncthreads();
  if (t < F) s_set[t] = my;
  __syncthreads();
  if (t == 0) {
    float M = -INFINITY;
    for (int q = 0; q < a.n1; ++q) M = fmaxf(M, s_part[q].x);
    float S = 0.f;
    for (int q = 0; q < a.n1; ++q)
      if (s_part[q].y > 0.f) S += s_part[q].y * ex2(s_part[q].x - M);
    const float L = M + lg2(S);
    float sig = 0.f;
    for (int f = 0; f < F; ++f)
      if (s_set[f] >= 0) sig += ex2(fmaf(s_zs[f], a.c2, -L));
    const float Cr = row_saguaro_c(a.C_per_row, a.C, row, a.flags, chunk == 0);
    const float N = 1.f - (1.f - Cr) * sig;
    s_L = L;
    s_N = N;
    s_C = Cr;
    if (chunk == 0) {
      if (a.out_set_mass) a.out_set_mass[row] = sig;
      if (a.out_norm) a.out_norm[row] = N;
      if (!(N > 0.f)) atomicOr(a.flags, kFlagSaguaroNorm);
    }
  }
  __syncthreads();
  if (!a.out_probs) return;
  const float L = s_L, w_out = 1.f / s_N, w_in = s_C / s_N;
  const int c0 = chunk * a.chunk_out;
  const int c1 = min(V, c0 + a.chunk_out);
  int nin = 0;
  for (int f = 0; f < F; ++f)
    if (s_set[f] >= c0 && s_set[f] < c1) ++nin;
  float* out = a.out_probs + int64_t(row) * V;
  auto qval = [&](float z, int idx) {
    float w = w_out;
    if (nin > 0)
      for (int f = 0; f < F; ++f)
        if (s_set[f] == idx) w = w_in;
    return ex2(fmaf(z, a.c2, -L)) * w;
  };
  // fp32 output rows start 16-byte aligned only when V % 4 == 0 (and the buffer is aligned)
  if (a.aligned && a.out_aligned) {
    constexpr int N = ET::kVec;
    const int v0 = c0 / N, v1 = v0 + (c1 - c0) / N;
    const uint4* rv = reinterpret_cast<const uint4*>(p);
    for (int vi = v0 + t; vi < v1; vi += kThreads) {
      float z[N];
      ET::unpack(load16(rv + vi), z);
#pragma unroll
      for (int h = 0; h < N / 4; ++h) {
        const int base = vi * N + h * 4;
        float4 o = make_float4(qval(z[h * 4 + 0], base + 0), qval(z[h * 4 + 1], base + 1),
                               qval(z[h * 4 + 2], base + 2), qval(z[h * 4 + 3], base + 3));
        *reinterpret_cast<float4*>(out + base) = o;
      }
    }
    for (int e = v1 * N + t; e < c1; e += kThreads) out[e] = qval(ET::one(p, e), e);
  } else {
    for (int e = c0 + t; e < c1; e += kThreads) out[e] = qval(ET::one(p, e), e);
  }
}

// =============================================================================================
// Speculation cache
// =============================================================================================
__global__ __launch_bounds__(kThreads) void cache_keys_kernel(CacheKeysArgs a) {
  const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (g >= int64_t(a.B) * a.budget) return;
  const int b = int(g / a.budget), slot = int(g - int64_t(b) * a.budget);
  int k = 0;
  while (k < a.K && slot >= a.off[k + 1]) ++k;
  const int rank = slot - a.off[k];
  const int tok = (a.last && k == a.K) ? a.last[int64_t(b) * a.Glast + rank]
                                       : a.guesses[(int64_t(b) * (a.last ? a.K : a.K + 1) + k) * a.Gmax + rank];
  a.cache_k[g] = (tok >= 0) ? k : -1;
  a.cache_tok[g] = (tok >= 0) ? tok : -1;
}

// One workgroup. Wave w takes sequences w, w + 4, ..., four at a time: lane j reads slot j of each
// (64 slots a round), so the reads of four sequences are in flight together, and a ballot names
// the first matching slot. The miss count is summed in a fixed order.
__global__ __launch_bounds__(kThreads) void cache_lookup_kernel(CacheLookupArgs a) {
  __shared__ int shi[8];
  constexpr int kSeq = 4;  // sequences per wave per round
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int miss = 0;  // lane 0 of each wave
  for (int b0 = w * kSeq; b0 < a.B; b0 += kWaves * kSeq) {
    int kq[kSeq], tq[kSeq], slot[kSeq];
#pragma unroll
    for (int i = 0; i < kSeq; ++i) {
      const int b = min(b0 + i, a.B - 1);  // clamped: every read in bounds
      kq[i] = a.k[b];
      tq[i] = a.tok[b];
      slot[i] = -1;
    }
    for (int j0 = 0; j0 < a.budget; j0 += 64) {
      const int j = j0 + lane;
      const int jc = min(j, a.budget - 1);
      int ckv[kSeq], ctv[kSeq];
#pragma unroll
      for (int i = 0; i < kSeq; ++i) {
        const int64_t base = int64_t(min(b0 + i, a.B - 1)) * a.budget + jc;
        ckv[i] = a.cache_k[base];
        ctv[i] = a.cache_tok[base];
      }
#pragma unroll
      for (int i = 0; i < kSeq; ++i) {
        const uint64_t hit = __ballot(j < a.budget && ckv[i] == kq[i] && ctv[i] == tq[i]);
        if (slot[i] < 0 && hit) slot[i] = j0 + __builtin_ctzll(hit);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kSeq; ++i)
        if (b0 + i < a.B) {
          a.out_slot[b0 + i] = slot[i];
          miss += (slot[i] < 0);
        }
    }
  }
  // block sum of integers
  for (int o = 32; o >= 1; o >>= 1) miss += __shfl_xor(miss, o, 64);
  if ((threadIdx.x & 63) == 0) shi[threadIdx.x >> 6] = miss;
  __syncthreads();
  if (threadIdx.x == 0) a.out_miss[0] = shi[0] + shi[1] + shi[2] + shi[3];
}

// Keys and lookup in one launch (one workgroup): wave w takes sequences 4w .. 4w + 3, then 16 further
// on; lane j forms the key of slot j of each of the four (64 slots a round) as cache_keys_kernel
// does, with every read of the four issued together, writes it, and a ballot names the first slot
// equal to the sequence's outcome. The miss count is summed in a fixed order.
__global__ __launch_bounds__(kThreads) void cache_keys_lookup_kernel(CacheKeysArgs ka, CacheLookupArgs la) {
  __shared__ int shi[kWaves];
  constexpr int kSeq = 4;  // sequences per wave per round
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rows = ka.last ? ka.K : ka.K + 1;  // position rows in `guesses`
  int miss = 0;  // lane 0 of each wave
  for (int b0 = w * kSeq; b0 < ka.B; b0 += kWaves * kSeq) {
    int kq[kSeq], tq[kSeq], slot[kSeq];
#pragma unroll
    for (int i = 0; i < kSeq; ++i) {
      const int b = min(b0 + i, ka.B - 1);  // clamped: every read in bounds
      kq[i] = la.k[b];
      tq[i] = la.tok[b];
      slot[i] = -1;
    }
    for (int j0 = 0; j0 < ka.budget; j0 += 64) {
      const int j = min(j0 + lane, ka.budget - 1);  // clamped; lanes past the budget write nothing
      int k = 0;
      while (k < ka.K && j >= ka.off[k + 1]) ++k;
      const int rank = j - ka.off[k];
      int tok[kSeq];
#pragma unroll
      for (int i = 0; i < kSeq; ++i) {
        const int64_t b = min(b0 + i, ka.B - 1);
        tok[i] = (ka.last && k == ka.K) ? ka.last[b * ka.Glast + rank] : ka.guesses[(b * rows + k) * ka.Gmax + rank];
      }
#pragma unroll
      for (int i = 0; i < kSeq; ++i) {
        const bool mine = j0 + lane < ka.budget && b0 + i < ka.B;
        if (mine) {
          const int64_t g = int64_t(b0 + i) * ka.budget + j;
          ka.cache_k[g] = (tok[i] >= 0) ? k : -1;
          ka.cache_tok[g] = (tok[i] >= 0) ? tok[i] : -1;
        }
        const uint64_t m = __ballot(mine && tok[i] >= 0 && k == kq[i] && tok[i] == tq[i]);
        if (slot[i] < 0 && m) slot[i] = j0 + __builtin_ctzll(m);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kSeq; ++i)
        if (b0 + i < ka.B) {
          la.out_slot[b0 + i] = slot[i];
          miss += (slot[i] < 0);
        }
    }
  }
  if (lane == 0) shi[w] = miss;
  __syncthreads();
  if (threadIdx.x == 0) la.out_miss[0] = (shi[0] + shi[1]) + (shi[2] + shi[3]);
}

__global__ void clear_flags_kernel(uint32_t* flags) { *flags = 0u; }

// Read-only streaming of n16 16-byte words, each read once, four loads in flight per thread: the
// read bandwidth a kernel reaches on this device for a footprint (a measurement helper). The sink
// is written only when the words' xor takes one particular value, which keeps the loads live.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                               uint32_t* sink) {
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = load16(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = load16(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}


// =============================================================================================
// launchers
// =============================================================================================
static hipError_t last_error() { return hipGetLastError(); }

template <class ET, int FM, bool SAG, bool SMP>
static hipError_t launch_topf_s(const TopfArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((topf_rows_kernel<ET, FM, SAG, SMP>), dim3(unsigned(int64_t(a.R) * a.n1)),
                     dim3(kThreads), 0, st, a);
  hipError_t e = last_error();
  if (e != hipSuccess || a.n1 == 1) return e;
  hipLaunchKernelGGL((topf_merge_kernel<ET, SAG, SMP>), dim3(a.R), dim3(kThreads), 0, st, a);
  return last_error();
}
template <class ET, int FM>
static hipError_t launch_topf_t(const TopfArgs& a, hipStream_t st) {
  if (a.u) return launch_topf_s<ET, FM, true, true>(a, st);
  return a.sag ? launch_topf_s<ET, FM, true, false>(a, st) : launch_topf_s<ET, FM, false, false>(a, st);
}

template <class ET>
static hipError_t launch_topf_e(const TopfArgs& a, hipStream_t st) {
  if (a.Fmax <= 4) return launch_topf_t<ET, 4>(a, st);
  if (a.Fmax <= 8) return launch_topf_t<ET, 8>(a, st);
  return launch_topf_t<ET, 16>(a, st);
}

hipError_t launch_topf(const TopfArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_topf_e<BF16T>(a, st) : launch_topf_e<F32T>(a, st);
}

template <class ET>
static hipError_t launch_sag_e(const SagArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((sag_rows_kernel<ET>), dim3(unsigned(int64_t(a.R) * a.n1)), dim3(kThreads), 0,
                     st, a);
  hipError_t e = last_error();
  if (e != hipSuccess) return e;
  const int nx = a.out_probs ? a.n_out : 1;
  hipLaunchKernelGGL((sag_finalize_kernel<ET>), dim3(nx, a.R), dim3(kThreads), 0, st, a);
  return last_error();
}

hipError_t launch_saguaro(const SagArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_sag_e<BF16T>(a, st) : launch_sag_e<F32T>(a, st);
}

hipError_t launch_cache_keys(const CacheKeysArgs& a, hipStream_t st) {
  const int64_t n = int64_t(a.B) * a.budget;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_keys_kernel, dim3(unsigned((n + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, st, a);
  return last_error();
}

hipError_t launch_cache_keys_lookup(const CacheKeysArgs& ka, const CacheLookupArgs& la, hipStream_t st) {
  hipLaunchKernelGGL(cache_keys_lookup_kernel, dim3(1), dim3(kThreads), 0, st, ka, la);
  return last_error();
}

hipError_t launch_cache_lookup(const CacheLookupArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(cache_lookup_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return last_error();
}

hipError_t launch_stream_read(const void* p, int64_t n16, uint32_t* sink, hipStream_t st) {
  const int64_t g = (n16 + kThreads - 1) / kThreads;
  const unsigned grid = unsigned(g < 1 ? 1 : (g > kStreamReadGrid ? kStreamReadGrid : g));
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint4*>(p), n16, sink);
  return last_error();
}

hipError_t launch_clear_flags(uint32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, st, flags);
  return last_error();
}

}  // namespace ssd
