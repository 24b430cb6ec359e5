// Batched lossless draft verification on gfx950: one launch per round of sequences.
//
// Work unit: one 256-thread workgroup per (sequence b, tile of 2048 tokens). A tile covers the
// same token range of all 2K+1 rows of its sequence (K draft rows, K+1 target rows), so the T
// tiles of a sequence together stream every logit of it exactly once.
//
//  phase 1   Each thread loads 8 contiguous tokens of every row (16-byte vector loads, all rows of
//            a load group in flight together), forms max and sum 2^(z c - max) per row with
//            c = log2(e)/T, and merges them over 16-lane groups with DPP. The threads that hold a
//            draft token or a Saguaro-set token publish its logit straight from registers. On
//            draft rows the tile's top-F candidates are filtered against a wave threshold and
//            compacted into LDS. Partials go out with write-through (agent-coherent) stores; once
//            they have completed, one atomic per tile counts the tile in.
//  decide    The tile that arrives last merges the row statistics in one fixed order, takes the
//            accept decisions and k, writes k and the accept probabilities, and publishes a small
//            decision record behind a flag that the other tiles wait for.
//  residual  Every tile sums r = max(p_k - q'_k, 0) (or p_K when all drafts pass) over its token
//            range, re-reading the two rows from cache, keeps r in registers and publishes the sum.
//  bonus     Every tile scans the T sums in the same order (the same bits everywhere); the tile
//            whose range holds u_K R finds the token in its registers. Tiles 0..K-1 merge the
//            top-F guesses of draft row = tile while the sums come in.
//
// The waits are bounded spins (a timeout is flagged, never hung). They need every tile of a
// sequence resident at once, so one launch covers only as many sequences as the device keeps
// resident; the host issues one launch per round of sequences.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kTile = kSub;  // 2048 tokens
constexpr int kMaxR2 = 2 * kMaxK + 1;
constexpr int kGroupsPerBlock = kThreads / 16;
constexpr int kCandW = 40;  // filtered top-F candidates kept per draft row per wave
constexpr int kCandSel = (kWaves * kCandW + 63) / 64;  // candidates per lane at selection
static_assert(kCandW >= kMaxF + 1, "a wave region must hold an exact top-(F+1)");

// per-sequence control words (64 x uint32): the phase-1 arrival counter
constexpr int kCtlArrive = 0;
// Per-sequence decision record: 64-bit words (call tag << 32 | value), each written once per
// call, so a reader knows a word is current when its tag matches the call's.
constexpr int kDecK = 0, kDecLp = 1, kDecLq = 2, kDecWout = 3, kDecWin = 4, kDecNset = 5,
              kDecSet = 6, kDecWords = kDecSet + kMaxF;
static_assert(kDecWords <= 32 && kDecWords <= 64, "decision record exceeds its 256 bytes");
static_assert(kGzPerSeq >= 2 * kMaxK + kMaxK * kMaxF, "token-logit slots too small");

__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return uint64_t(__float_as_uint(a)) | (uint64_t(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float(uint32_t(v)); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float(uint32_t(v >> 32)); }
__device__ __forceinline__ uint64_t cand_key(float v, int idx) {  // larger = better; 0 = none
  return (uint64_t(ordered_key(v)) << 32) | uint64_t(~uint32_t(idx));
}
template <class P>
__device__ __forceinline__ void st_agent(P* p, P v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) { return (uint64_t(tag) << 32) | v; }
template <class P>
__device__ __forceinline__ P ld_agent(const P* p) {
  return __hip_atomic_load(const_cast<P*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait for this thread's outstanding vector-memory operations (stores included) to complete
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// store the logit of token `tok` to *dst if this thread holds it (one conditional store per
// element: selecting the element by index would send the thread's tokens through scratch memory)
__device__ __forceinline__ void store_if_held(float* dst, const float (&z)[kSubElems], int e0, int tok) {
#pragma unroll
  for (int e = 0; e < kSubElems; ++e)
    if (e0 + e == tok) st_agent(dst, z[e]);
}

#ifdef SSD_TRACE
// phase timestamps per workgroup (100 MHz clock), for performance analysis builds only
#define TRACE(i)                                                                      \
  do {                                                                                \
    if (threadIdx.x == 0 && a.trace) a.trace[blockIdx.x * 16 + (i)] = wall_clock64(); \
  } while (0)
#else
#define TRACE(i) \
  do {           \
  } while (0)
#endif

struct Shared {
  // per sequence, as given
  int F[kMaxK];           // top-F guesses per draft position
  int xe[kMaxK];          // draft tokens
  float u[kMaxK + 1];     // uniforms
  int sv[kMaxK * kMaxF];  // Saguaro-set entries
  // phase 1
  float2 g16[kMaxR2][kGroupsPerBlock];  // (max c, sum) per 16-lane group
  int ncw[kMaxK][kWaves];
  uint64_t cand[kMaxK][kWaves][kCandW];
  uint64_t best[kMaxK][kMaxF];
  int leader;
  // decision (last tile to arrive)
  float2 part[kThreads];
  float L[kMaxR2];
  float zg[2 * kMaxK];      // logits at the draft tokens: draft rows 0..K-1, then target rows
  float zs[kMaxK * kMaxF];  // draft logits at the set entries
  int set[kMaxK * kMaxF];   // de-duplicated in-range set entries, -1 elsewhere
  // the decision record, as every tile uses it
  int k, nset;
  float Lp, Lq, w_out, w_in;
  int myset[kMaxF];
  // bonus
  float res[kMaxTiles];
  int cstar, clamp, fallback, first, lastp;
  float base, target, R;
  uint64_t wtop[kWaves][kMaxF];
  float shf[8];
  int shi[8];
  uint32_t shk[2 * kWaves];
};

template <class ET, int FM>
__global__ __launch_bounds__(kThreads, 4) void verify_fused_kernel(VerifyArgs a) {
  using T = typename ET::T;
  constexpr int G = (sizeof(T) == 2) ? 9 : 5;  // rows per load group (36-40 VGPRs of payload)
  __shared__ Shared sh;

  const int t = threadIdx.x, lane = t & 63, grp = t >> 4;
  const int K = a.K, V = a.V, R2 = 2 * K + 1, nT = a.T, sF = a.sF;
  const float cc = a.c2;
  const bool aligned = a.aligned != 0;
  const int tile = blockIdx.x % nT;
  const int b = a.b0 + int(blockIdx.x) / nT;
  const int c0 = tile * kTile;
  const int e0 = c0 + t * kSubElems;
  const T* draft = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride;
  const T* target = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride;
  auto row_ptr = [&](int r) -> const T* {
    return (r < K) ? draft + int64_t(r) * V : target + int64_t(r - K) * V;
  };
  uint32_t* ctl = a.ctl + int64_t(b) * 64;
  uint64_t* dec = a.dec + int64_t(b) * 32;
  const uint32_t tag = a.epoch;
  float* gz = a.gz + int64_t(b) * kGzPerSeq;  // [0, 2K) token logits, [2K, 2K + K sF) set logits

  // Per-sequence inputs, one copy per wave in registers (lane i holds position i, entry q of the
  // Saguaro sets sits in lane q % 64 of sv_v[q / 64]). They are loaded before the rows and read
  // with readlane, so no row waits on LDS or on a scalar load.
  const int x_v = a.x[b * K + min(lane, K - 1)];
  const float u_v = a.u[b * (K + 1) + min(lane, K)];
  int sv0 = -1, sv1 = -1, sv2 = -1, sv3 = -1;  // K * sF <= 256 entries: four per lane at most
  if (sF > 0) {
    const int nS = K * sF;
    const int* ss = a.sset + int64_t(b) * nS;
    sv0 = ss[min(lane, nS - 1)];
    if (nS > 64) sv1 = ss[min(lane + 64, nS - 1)];
    if (nS > 128) sv2 = ss[min(lane + 128, nS - 1)];
    if (nS > 192) sv3 = ss[min(lane + 192, nS - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the row loads
  auto set_entry = [&](int q) -> int {  // q wave-uniform
    if (q < 64) return __builtin_amdgcn_readlane(sv0, q);
    if (q < 128) return __builtin_amdgcn_readlane(sv1, q - 64);
    if (q < 192) return __builtin_amdgcn_readlane(sv2, q - 128);
    return __builtin_amdgcn_readlane(sv3, q - 192);
  };

  // ---- phase 1: statistics, token logits and top-F candidates of this tile
  TRACE(0);
  const int w = t >> 6;
  const int Fp = a.topfFmax + 1;  // candidates kept per wave: one more than the guesses
  const bool vec = aligned && e0 + kSubElems <= V;  // this thread's tokens load as vectors
  auto row_group = [&](int g0) __attribute__((always_inline)) {
    RawTile<ET> raw[G];
    // every slot of the group is loaded (past the last row: the last row again, a cache hit) and
    // consumed below, so no load is left pending at the loop's back edge
    if (vec) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        load_raw_vec<ET>(row_ptr(min(g0 + j, R2 - 1)), e0, raw[j]);
        __builtin_amdgcn_sched_barrier(0);  // issue in row order: row j is consumed j-th
      }
    } else {
#pragma unroll
      for (int j = 0; j < G; ++j) load_raw_scalar<ET>(row_ptr(min(g0 + j, R2 - 1)), e0, V, raw[j]);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int r = g0 + j;
      float z[kSubElems];
      unpack_tile<ET>(raw[j], z);
      float m = z[0];
#pragma unroll
      for (int e = 1; e < kSubElems; ++e) m = fmaxf(m, z[e]);
      float s = 0.f;
      const float mc = m * cc;
      if (m > -INFINITY) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int e = 0; e < kSubElems; e += 2) {
          s0 += ex2(fmaf(z[e], cc, -mc));
          s1 += ex2(fmaf(z[e + 1], cc, -mc));
        }
        s = s0 + s1;
      }
      // row16_max, keeping the 4- and 8-lane group maxima for the top-F threshold
      const float m2 = fmaxf(m, dpp_f<kDppXor1>(m));
      const float m4 = fmaxf(m2, dpp_f<kDppXor2>(m2));
      const float m8 = fmaxf(m4, dpp_f<kDppHalfMirror>(m4));
      const float M = fmaxf(m8, dpp_f<kDppMirror>(m8));
      const float Mc = M * cc;
      const float sc = (s > 0.f) ? s * ex2(mc - Mc) : 0.f;
      const float S = row16_sum(sc);
      if ((t & 15) == 0 && r < R2) sh.g16[r][grp] = make_float2(Mc, S);
      if (j == 0 && g0 == 0) TRACE(8);
      if (FM == 0 || r >= K) continue;
      // Top-F candidates of a draft row into this wave's region. The sampled token is dropped
      // only at selection, so the filter keeps the wave's top Fp = F_max + 1 tokens. Threshold:
      // the smallest maximum over the non-empty groups of the coarsest grouping (16, 8, 4 or 1
      // lanes) that has at least Fp non-empty groups; Fp groups then each hold a token at least
      // that large, so every top-Fp token of the wave passes. Positions past V read as -inf and
      // never pass. With fewer than Fp non-empty lanes everything finite passes.
      constexpr float kInf = __builtin_inff();
      int lvl = (Fp <= 4) ? 0 : (Fp <= 8) ? 1 : (Fp <= 16) ? 2 : 3;
      if (lvl == 0 && __popcll(__ballot(M > -kInf) & 0x0001000100010001ull) < Fp) lvl = 1;
      if (lvl == 1 && __popcll(__ballot(m8 > -kInf) & 0x0101010101010101ull) < Fp) lvl = 2;
      if (lvl == 2 && __popcll(__ballot(m4 > -kInf) & 0x1111111111111111ull) < Fp) lvl = 3;
      float g;
      if (lvl == 0) {
        g = (M > -kInf) ? M : kInf;
      } else if (lvl == 1) {
        const float h = (m8 > -kInf) ? m8 : kInf;
        g = fminf(h, dpp_f<kDppMirror>(h));
      } else if (lvl == 2) {
        const float q = (m4 > -kInf) ? m4 : kInf;
        g = fminf(q, dpp_f<kDppHalfMirror>(q));
        g = fminf(g, dpp_f<kDppMirror>(g));
      } else {
        g = (m > -kInf) ? m : kInf;
        g = fminf(g, dpp_f<kDppXor1>(g));
        g = fminf(g, dpp_f<kDppXor2>(g));
        g = fminf(g, dpp_f<kDppHalfMirror>(g));
        g = fminf(g, dpp_f<kDppMirror>(g));
      }
      const bool few = lvl == 3 && __popcll(__ballot(m > -kInf)) < Fp;
      const float thr = few ? -__FLT_MAX__ : rows_min(g);
      int total = 0;
#pragma unroll
      for (int e = 0; e < kSubElems; ++e) total += __popcll(__ballot(z[e] >= thr));
      uint64_t* region = sh.cand[r][w];
      if (total <= kCandW) {  // compaction: slot = running count + lanes below in the mask
        int base = 0;
#pragma unroll
        for (int e = 0; e < kSubElems; ++e) {
          const bool pass = z[e] >= thr;
          const uint64_t mk = __ballot(pass);
          if (mk) {
            if (pass) {
              const int slot = base + int(__builtin_amdgcn_mbcnt_hi(
                                          uint32_t(mk >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mk), 0u)));
              region[slot] = cand_key(z[e], e0 + e);
            }
            base += __popcll(mk);
          }
        }
      } else {  // too many pass (ties, a short last tile): the wave's exact top Fp from registers
        uint32_t ph = 0xFFFFFFFFu, pl = 0xFFFFFFFFu;
        for (int f = 0; f < Fp; ++f) {
          uint32_t bh = 0, bl = 0;
#pragma unroll
          for (int e = 0; e < kSubElems; ++e) {
            const bool ok = z[e] > -INFINITY;
            const uint32_t kh = ok ? ordered_key(z[e]) : 0u;
            const uint32_t kl = ok ? ~uint32_t(e0 + e) : 0u;
            if (key_gt(ph, pl, kh, kl) && key_gt(kh, kl, bh, bl)) {
              bh = kh;
              bl = kl;
            }
          }
          wave_max_key(bh, bl);
          if (lane == 0) region[f] = (uint64_t(bh) << 32) | bl;
          ph = bh;
          pl = bl;
        }
        total = Fp;
      }
      if (lane == 0) sh.ncw[r][w] = total;
    }
    // Token logits once the group's rows have landed (the per-sequence registers are read only
    // now, so no row waits on them). A tile stores only tokens in its own range.
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int r = g0 + j;
      if (r >= 2 * K) continue;
      const int xr = __builtin_amdgcn_readlane(x_v, r < K ? r : r - K);
      const bool own_x = (xr >> 11) == tile && xr < V;
      bool own_set = false;
      if (r < K)
        for (int f = 0; f < sF; ++f) {
          const int sv = set_entry(r * sF + f);
          own_set |= (sv >> 11) == tile && sv < V;
        }
      if (!own_x && !own_set) continue;
      // unpack again rather than keep the statistics pass's floats alive (an empty asm hides the
      // packed words' provenance; it emits no instruction)
#pragma unroll
      for (int h = 0; h < RawTile<ET>::kWords; ++h)
        asm volatile("" : "+v"(raw[j].w[h].x), "+v"(raw[j].w[h].y), "+v"(raw[j].w[h].z), "+v"(raw[j].w[h].w));
      float z[kSubElems];
      unpack_tile<ET>(raw[j], z);
      if (own_x && unsigned(xr - e0) < unsigned(kSubElems)) store_if_held(gz + r, z, e0, xr);
      if (own_set)
        for (int f = 0; f < sF; ++f) {
          const int sv = set_entry(r * sF + f);
          if (unsigned(sv - e0) < unsigned(kSubElems) && sv < V)
            store_if_held(gz + 2 * K + r * sF + f, z, e0, sv);
        }
    }
  };
  // A single group runs outside any loop, so the per-sequence loads above stay visibly older
  // than the row loads and reading them waits only for them.
  if (R2 <= G) {
    row_group(0);
  } else {
    for (int g0 = 0; g0 < R2; g0 += G) row_group(g0);
  }
  TRACE(9);
  if (t < K) {
    sh.xe[t] = x_v;
    sh.F[t] = a.topfF[t];
  }
  if (t <= K) sh.u[t] = u_v;
  if (t < 64) {
    if (t < K * sF) sh.sv[t] = sv0;
    if (t + 64 < K * sF) sh.sv[t + 64] = sv1;
    if (t + 128 < K * sF) sh.sv[t + 128] = sv2;
    if (t + 192 < K * sF) sh.sv[t + 192] = sv3;
  }
  __syncthreads();
  if (FM > 0) {  // wave w selects the F best candidates (value desc, index asc) of rows w, w+4, ...
    for (int r = w; r < K; r += kWaves) {
      const int F = sh.F[r];
      const int xs = sh.xe[r];
      uint64_t key[kCandSel];  // candidate q = lane + 64 i is entry q % kCandW of wave q / kCandW
#pragma unroll
      for (int i = 0; i < kCandSel; ++i) {
        const int q = lane + 64 * i, ww = q / kCandW, sl = q - ww * kCandW;
        key[i] = (ww < kWaves && sl < sh.ncw[r][ww]) ? sh.cand[r][ww][sl] : 0ull;
        if (uint32_t(key[i]) == ~uint32_t(xs)) key[i] = 0;  // the sampled token is never a guess
      }
      for (int f = 0; f < F; ++f) {
        uint64_t mine = key[0];
#pragma unroll
        for (int i = 1; i < kCandSel; ++i) mine = (key[i] > mine) ? key[i] : mine;
        uint32_t hi = uint32_t(mine >> 32), lo = uint32_t(mine);
        wave_max_key(hi, lo);
        const uint64_t win = (uint64_t(hi) << 32) | lo;
        if (lane == 0) sh.best[r][f] = win;
#pragma unroll
        for (int i = 0; i < kCandSel; ++i)
          if (key[i] == win) key[i] = 0;  // keys are unique: only the winner is cleared
      }
    }
    __syncthreads();
  }
  TRACE(10);

  // ---- publish the tile's partials; once they have completed, count the tile in
  if (t < R2) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kGroupsPerBlock; ++q) M = fmaxf(M, sh.g16[t][q].x);
    float S = 0.f;
#pragma unroll
    for (int q = 0; q < kGroupsPerBlock; ++q) {
      const float2 v = sh.g16[t][q];
      if (v.y > 0.f) S += v.y * ex2(v.x - M);
    }
    st_agent(a.stats + (int64_t(b) * R2 + t) * nT + tile, pack2(M, S));
  }
  if (FM > 0 && t < K * a.topfFmax) {
    const int r = t / a.topfFmax, f = t - r * a.topfFmax;
    if (f < sh.F[r])
      st_agent(a.cand + ((int64_t(b) * K + r) * nT + tile) * a.topfFmax + f, sh.best[r][f]);
  }
  wait_vmem();
  __syncthreads();
  if (t == 0) sh.leader = (atomicAdd(ctl + kCtlArrive, 1u) == unsigned(nT - 1));
  __syncthreads();
  TRACE(1);

  // ---- decide: the last tile to arrive merges the statistics and publishes the decision
  if (sh.leader) {
    if (t == 0) st_agent(ctl + kCtlArrive, 0u);  // every tile has arrived: ready for the next call
    // token logits first, so their loads overlap the statistics loads
    float zg_v = 0.f, zs_v = 0.f;
    int set_v = -1;
    if (t < 2 * K) {
      const int xr = sh.xe[t < K ? t : t - K];
      if (unsigned(xr) < unsigned(V)) zg_v = ld_agent(gz + t);
    }
    if (t < K * sF) {
      set_v = (unsigned(sh.sv[t]) < unsigned(V)) ? sh.sv[t] : -1;
      if (set_v >= 0) zs_v = ld_agent(gz + 2 * K + t);
    }
    // 16-lane group g merges rows g, g + 16, g + 32: lane l takes tiles l, l + 16, ..., then the
    // group combines its lanes with DPP (a fixed order, the same bits on every run)
    for (int r = grp; r < R2; r += kGroupsPerBlock) {
      const uint64_t* st = a.stats + (int64_t(b) * R2 + r) * nT;
      float M = -INFINITY, S = 0.f;
      constexpr int kAhead = 8;  // loads in flight per lane
      for (int q0 = (t & 15); q0 < nT; q0 += kAhead * 16) {
        uint64_t vals[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
          const int q = q0 + i * 16;
          vals[i] = (q < nT) ? ld_agent(st + q) : 0ull;
        }
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
          const float m = lo_f(vals[i]), s = hi_f(vals[i]);
          if (s > 0.f) {
            if (m > M) {
              S = S * ex2(M - m) + s;
              M = m;
            } else {
              S += s * ex2(m - M);
            }
          }
        }
      }
      const float Mr = row16_max(M);
      const float Sr = row16_sum((S > 0.f) ? S * ex2(M - Mr) : 0.f);
      if ((t & 15) == 0) sh.L[r] = Mr + lg2(Sr);
    }
    TRACE(11);
    if (t < 2 * K) sh.zg[t] = zg_v;
    if (t < K * sF) {
      const int i = t / sF, f = t - i * sF;
      for (int g = 0; g < f && set_v >= 0; ++g)  // the first occurrence of a token counts
        if (sh.sv[i * sF + g] == set_v) set_v = -1;
      sh.set[t] = set_v;
      sh.zs[t] = zs_v;
    }
    __syncthreads();
    TRACE(12);
    if (t < 64) {  // wave 0: lane i takes the accept test of position i
      const float C = a.C;
      const int i = min(lane, K - 1);
      const float Lq = sh.L[i], Lp = sh.L[K + i];
      const int xi = sh.xe[i];
      const bool xok = unsigned(xi) < unsigned(V);
      if (lane < K && !xok) atomicOr(a.flags, kFlagBadToken);
      float Nn = 1.f;
      bool xin = false;
      if (sF > 0) {  // Saguaro: N = 1 - (1 - C) sigma, sigma = q mass of the set
        float sig = 0.f;
        for (int f = 0; f < sF; ++f) {
          const int sv = sh.set[i * sF + f];
          if (sv < 0) continue;
          sig += ex2(fmaf(sh.zs[i * sF + f], cc, -Lq));
          if (sv == xi) xin = true;
        }
        Nn = 1.f - (1.f - C) * sig;
        if (lane < K && !(Nn > 0.f)) atomicOr(a.flags, kFlagSaguaroNorm);
      }
      bool accept;
      float ai;
      if (!xok) {
        accept = false;
        ai = 0.f;
      } else {
        const float w = xin ? C : 1.f;
        const float dp = fmaf(sh.zg[K + i], cc, -Lp);  // log2 p(x)
        const float dq = fmaf(sh.zg[i], cc, -Lq);      // log2 q(x)
        if (w == 0.f || dq == -INFINITY) {             // q'(x) = 0: accept iff p(x) > 0
          accept = dp > -INFINITY;
          ai = accept ? 1.f : 0.f;
        } else {
          const float ratio = ex2(dp - dq) * (Nn / w);  // p(x) / q'(x)
          accept = sh.u[i] < ratio;
          ai = fminf(1.f, ratio);
        }
      }
      if (a.aprob_out && lane < K) a.aprob_out[b * K + lane] = ai;
      const uint64_t rej = __ballot(lane < K && !accept);
      const int k = rej ? __builtin_ctzll(rej) : K;  // first rejection
      const float Nk = (k < K) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Nn), k)) : 1.f;
      if (lane == 0) {
        a.k_out[b] = k;
        int n = 0;
        if (k < K)
          for (int f = 0; f < sF; ++f) {
            const int sv = sh.set[k * sF + f];
            if (sv >= 0) sh.myset[n++] = sv;
          }
        for (int f = n; f < kMaxF; ++f) sh.myset[f] = -1;
        sh.k = k;
        sh.nset = n;
        sh.Lp = sh.L[K + k];
        sh.Lq = (k < K) ? sh.L[k] : 0.f;
        sh.w_out = 1.f / Nk;
        sh.w_in = C / Nk;
      }
    }
    __syncthreads();
    if (t < kDecWords) {  // publish the record, one tagged word per thread
      uint32_t v;
      if (t == kDecK) v = uint32_t(sh.k);
      else if (t == kDecLp) v = __float_as_uint(sh.Lp);
      else if (t == kDecLq) v = __float_as_uint(sh.Lq);
      else if (t == kDecWout) v = __float_as_uint(sh.w_out);
      else if (t == kDecWin) v = __float_as_uint(sh.w_in);
      else if (t == kDecNset) v = uint32_t(sh.nset);
      else v = uint32_t(sh.myset[t - kDecSet]);
      st_agent(dec + t, tagged(tag, v));
    }
    TRACE(13);
  } else if (t < 64) {
    // wave 0 polls the record until every word carries this call's tag
    uint64_t v = 0;
    for (int spins = 0;; ++spins) {
      v = (lane < kDecWords) ? ld_agent(dec + lane) : tagged(tag, 0u);
      if (__all(uint32_t(v >> 32) == tag)) break;
      if (spins > a.spin_limit) {
        if (lane == 0) atomicOr(a.flags, kFlagTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const uint32_t x = uint32_t(v);
    if (lane == kDecK) sh.k = int(x);
    if (lane == kDecLp) sh.Lp = __uint_as_float(x);
    if (lane == kDecLq) sh.Lq = __uint_as_float(x);
    if (lane == kDecWout) sh.w_out = __uint_as_float(x);
    if (lane == kDecWin) sh.w_in = __uint_as_float(x);
    if (lane == kDecNset) sh.nset = int(x);
    if (lane >= kDecSet && lane < kDecWords) sh.myset[lane - kDecSet] = int(x);
  }
  TRACE(2);
  __syncthreads();
  TRACE(3);
  const int k = min(max(sh.k, 0), K);  // in range even if a timed-out wait read a stale record
  const bool resid = k < K;
  const T* prow = target + int64_t(k) * V;
  const T* qrow = resid ? draft + int64_t(k) * V : nullptr;
  const float Lp = sh.Lp, Lq = sh.Lq, w_out = sh.w_out, w_in = sh.w_in;
  const int nset = resid ? min(max(sh.nset, 0), kMaxF) : 0;

  // ---- residual mass of this tile (the values stay in registers), published
  float rv[kSubElems], pre[kSubElems];
  sub_values<ET>(prow, qrow, c0, V, aligned, cc, Lp, Lq, w_out, w_in, sh.myset, nset, rv);
  const float total = sub_scan(rv, pre, sh.shf);
  if (t == 0) st_agent(a.res + int64_t(b) * nT + tile, tagged(tag, __float_as_uint(total)));
  TRACE(4);

  // ---- top-F guesses of draft rows tile, tile + T, ... while the other tiles finish: each
  // wave takes its own top F of the tiles' candidates, then wave 0 merges the four lists. Keys
  // are unique (a token lives in one tile), so round f picks the largest key below round f-1's.
  for (int r = tile; FM > 0 && r < K; r += nT) {
    const int F = sh.F[r];
    int32_t* out = a.topf_out + (int64_t(b) * K + r) * a.topfFmax;
    const uint64_t* cd = a.cand + (int64_t(b) * K + r) * nT * a.topfFmax;
    const int n = nT * F;
    constexpr int kKeep = 4;
    uint64_t keys[kKeep];
#pragma unroll
    for (int i = 0; i < kKeep; ++i) {
      const int q = t + i * kThreads;
      keys[i] = 0;
      if (q < n) {
        const int tl = q / F, ff = q - tl * F;
        keys[i] = ld_agent(cd + int64_t(tl) * a.topfFmax + ff);
      }
    }
    uint32_t ph = 0xFFFFFFFFu, pl = 0xFFFFFFFFu;
    for (int f = 0; f < F; ++f) {
      uint64_t bk = 0;
      const uint64_t prev = (uint64_t(ph) << 32) | pl;
#pragma unroll
      for (int i = 0; i < kKeep; ++i)
        if (keys[i] < prev && keys[i] > bk) bk = keys[i];
      for (int q = t + kKeep * kThreads; q < n; q += kThreads) {  // beyond what registers hold
        const int tl = q / F, ff = q - tl * F;
        const uint64_t v = ld_agent(cd + int64_t(tl) * a.topfFmax + ff);
        if (v < prev && v > bk) bk = v;
      }
      ph = uint32_t(bk >> 32);
      pl = uint32_t(bk);
      wave_max_key(ph, pl);
      if (lane == 0) sh.wtop[w][f] = (uint64_t(ph) << 32) | pl;
    }
    __syncthreads();
    if (t < 64) {
      const uint64_t key = (lane < kWaves * F) ? sh.wtop[lane / F][lane % F] : 0ull;
      ph = 0xFFFFFFFFu;
      pl = 0xFFFFFFFFu;
      for (int f = 0; f < F; ++f) {
        const uint64_t prev = (uint64_t(ph) << 32) | pl;
        const uint64_t bk = (key < prev) ? key : 0ull;
        ph = uint32_t(bk >> 32);
        pl = uint32_t(bk);
        wave_max_key(ph, pl);
        if (lane == 0) out[f] = (ph | pl) ? int(~pl) : -1;
      }
      for (int f = F + lane; f < a.topfFmax; f += 64) out[f] = -1;
    }
    __syncthreads();
    TRACE(14);
  }

  // ---- bonus: every tile scans the T masses the same way; the owner of u_K R draws the token
  {
    const int per = (nT + kThreads - 1) / kThreads;  // consecutive tiles per thread
    const int q0 = min(t * per, nT), q1 = min(nT, q0 + per);
    const uint64_t* rs = a.res + int64_t(b) * nT;
    for (int spins = 0;; ++spins) {  // poll until this call's masses of all tiles are in
      bool ok = true;
      for (int q = q0; q < q1; ++q) {
        const uint64_t v = ld_agent(rs + q);
        ok = ok && uint32_t(v >> 32) == tag;
        sh.res[q] = __uint_as_float(uint32_t(v));
      }
      if (__all(ok)) break;
      if (spins > a.spin_limit) {
        if (lane == 0) atomicOr(a.flags, kFlagTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __syncthreads();
    TRACE(5);
  }
  if (t < 64) {  // wave 0 scans the masses: lane l takes consecutive tiles [l per, (l + 1) per)
    const int per = (nT + 63) / 64;
    const int q0 = min(lane * per, nT), q1 = min(nT, q0 + per);
    float run = 0.f;
    for (int q = q0; q < q1; ++q) run += sh.res[q];
    const float inc = wave_incl_scan(run);
    const float Rtot = readlane_f(inc, 63);
    const float target_v = sh.u[K] * Rtot;
    int first = INT_MAX, lastpos = -1;
    float p = wave_shift_up1(inc), base = 0.f;
    for (int q = q0; q < q1; ++q) {
      const float nxt = p + sh.res[q];
      if (sh.res[q] > 0.f) lastpos = q;
      if (first == INT_MAX && nxt > target_v) {
        first = q;
        base = p;
      }
      p = nxt;
    }
    const int cf = wave_min_i(first);
    const int cl = wave_max_i(lastpos);
    if (first != INT_MAX && first == cf) sh.base = base;
    if (lane == 0) {
      sh.cstar = (cf != INT_MAX) ? cf : cl;  // u R past the total by rounding: last tile with mass
      sh.clamp = (cf == INT_MAX);
      sh.fallback = (cf == INT_MAX && cl < 0);  // all-zero residual (rounding only)
      sh.target = target_v;
      sh.R = Rtot;
      sh.first = INT_MAX;
      sh.lastp = -1;
    }
  }
  __syncthreads();
  if (!sh.fallback && sh.cstar == tile) {
    int first = INT_MAX, lastp = -1;
#pragma unroll
    for (int e = 0; e < kSubElems; ++e)
      if (rv[e] > 0.f) {
        lastp = e0 + e;
        if (first == INT_MAX && !sh.clamp && sh.base + pre[e] > sh.target) first = e0 + e;
      }
    first = wave_min_i(first);
    lastp = wave_max_i(lastp);
    if (lane == 0) {
      if (first != INT_MAX) atomicMin(&sh.first, first);
      if (lastp >= 0) atomicMax(&sh.lastp, lastp);
    }
    __syncthreads();
    if (t == 0) {
      a.bonus_out[b] = (sh.first != INT_MAX) ? sh.first : sh.lastp;
      if (a.rmass_out) a.rmass_out[b] = resid ? sh.R : 1.f;
    }
  } else if (sh.fallback && tile == 0) {
    // residual identically zero (rounding only): draw from the target row p_k itself, R = 1
    const float target_v = sh.u[K];
    float run = 0.f;
    int found = -1, lastp = -1;
    for (int q = 0; q < nT && found < 0; ++q) {
      sub_values<ET>(prow, nullptr, q * kTile, V, aligned, cc, Lp, 0.f, 1.f, 1.f, sh.myset, 0, rv);
      const float tot = sub_scan(rv, pre, sh.shf);
      const int f0 = q * kTile + t * kSubElems;
      int first = INT_MAX, lp = -1;
#pragma unroll
      for (int e = 0; e < kSubElems; ++e)
        if (rv[e] > 0.f) {
          lp = f0 + e;
          if (first == INT_MAX && run + pre[e] > target_v) first = f0 + e;
        }
      first = block_min_i(first, sh.shi);
      lp = block_max_i(lp, sh.shi);
      if (lp >= 0) lastp = lp;
      if (first != INT_MAX) found = first;
      run += tot;
    }
    if (t == 0) {
      a.bonus_out[b] = (found >= 0) ? found : lastp;
      if (a.rmass_out) a.rmass_out[b] = 0.f;
    }
  }
  TRACE(6);

  TRACE(7);
}

// ---------------------------------------------------------------------------------------------
// launch: grids of whole sequences whose tiles all fit the device at once
// ---------------------------------------------------------------------------------------------
template <class ET, int FM>
static int capacity_blocks() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(verify_fused_kernel<ET, FM>), kThreads, 0) != hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <class ET, int FM>
static hipError_t launch_fused(VerifyArgs a, hipStream_t st) {
  const int cap = capacity_blocks<ET, FM>();
  if (cap < a.T) return hipErrorInvalidConfiguration;
  const int per_round = cap / a.T;  // whole sequences whose tiles are all resident at once
  const int B = a.B;
  for (int b0 = 0; b0 < B; b0 += per_round) {
    const int nb = (B - b0 < per_round) ? (B - b0) : per_round;
    a.b0 = b0;
    hipLaunchKernelGGL((verify_fused_kernel<ET, FM>), dim3(unsigned(nb * a.T)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class ET>
static hipError_t launch_verify_e(const VerifyArgs& a, hipStream_t st) {
  if (a.topfFmax == 0) return launch_fused<ET, 0>(a, st);
  if (a.topfFmax <= 4) return launch_fused<ET, 4>(a, st);
  if (a.topfFmax <= 8) return launch_fused<ET, 8>(a, st);
  return launch_fused<ET, 16>(a, st);
}

hipError_t launch_verify(const VerifyArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_verify_e<BF16T>(a, st) : launch_verify_e<F32T>(a, st);
}

}  // namespace ssd
