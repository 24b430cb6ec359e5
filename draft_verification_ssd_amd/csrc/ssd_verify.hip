// Batched lossless draft verification on gfx950: one launch per round of sequences.
//
// Work unit: one 256-thread workgroup per (sequence b, tile of 2048 tokens). A tile covers the
// same token range of all 2K+1 rows of its sequence (K draft rows, K+1 target rows), so the T
// tiles of a sequence together stream every logit of it exactly once.
//
//  phase 1  Each thread loads 8 contiguous tokens of every row (16-byte vector loads, all rows in
//           flight together), forms max and sum 2^(z c - max) with c = log2(e)/T per row, reduces
//           them across 16-lane groups with DPP, and, on draft rows, keeps the tile's top-F
//           candidates. Partials go out with write-through (agent-coherent) stores; after they
//           complete, one atomic per tile bumps the sequence's arrival counter.
//  wait     The tiles of a sequence wait for each other (bounded spin on the counter; a timeout is
//           flagged, never hung). A launch holds only as many workgroups as the device keeps
//           resident at once, so every tile it waits for is running.
//  phase 2  Every tile merges the sequence's row statistics in one fixed order (so all tiles get
//           the same bits), takes the accept decisions and k, and sums the residual
//           max(p_k - q'_k, 0) (or p_K when all drafts pass) over its token range, re-reading the
//           two rows from cache. The last tile to publish its sum finds the tile holding u_K R and
//           scans it for the bonus token. Tiles 0..K-1 merge the top-F guesses of draft row = tile.
//
// One launch covers the sequences [b0, b0 + gridDim.x / T): workgroup w serves tile w % T of
// sequence b0 + w / T. When a batch needs more workgroups than the device holds at once, the host
// issues one launch per round of sequences.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kTile = kSub;  // 2048 tokens
constexpr int kMaxR2 = 2 * kMaxK + 1;
constexpr int kGroupsPerBlock = kThreads / 16;
constexpr int kMaxCand = 160;  // filtered top-F candidates kept per draft row per tile

__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return uint64_t(__float_as_uint(a)) | (uint64_t(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float(uint32_t(v)); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float(uint32_t(v >> 32)); }
__device__ __forceinline__ uint64_t cand_key(float v, int idx) {  // larger = better; 0 = none
  return (uint64_t(ordered_key(v)) << 32) | uint64_t(~uint32_t(idx));
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class P>
__device__ __forceinline__ P ld_agent(const P* p) {
  return __hip_atomic_load(const_cast<P*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// raw storage bits of one logit (the conversion is deferred so the load is not waited for early)
template <class ET>
__device__ __forceinline__ uint32_t raw_bits(const typename ET::T* p, int i) {
  return uint32_t(p[i]);
}
template <>
__device__ __forceinline__ uint32_t raw_bits<F32T>(const float* p, int i) {
  return __float_as_uint(p[i]);
}
template <class ET>
__device__ __forceinline__ float bits_to_f(uint32_t v) {
  return (sizeof(typename ET::T) == 2) ? __uint_as_float(v << 16) : __uint_as_float(v);
}
// wait for this thread's outstanding vector-memory operations (stores included) to complete
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

#ifdef SSD_TRACE
// phase timestamps per workgroup (100 MHz clock), for performance analysis builds only
#define TRACE(i)                                                                  \
  do {                                                                            \
    if (threadIdx.x == 0 && a.trace) a.trace[blockIdx.x * 16 + (i)] = wall_clock64(); \
  } while (0)
#else
#define TRACE(i) \
  do {           \
  } while (0)
#endif

struct Shared {
  // per sequence
  int F[kMaxK];  // top-F guesses per draft position
  int xe[kMaxK];  // draft tokens as given (top-F exclusion), staged once
  int x[kMaxK];
  float u[kMaxK + 1];
  float zq[kMaxK], zp[kMaxK];
  int set[kMaxK * kMaxF];
  float zs[kMaxK * kMaxF];
  // phase 1
  float2 g16[kMaxR2][kGroupsPerBlock];  // (max c, sum) per 16-lane group
  int ncand[kMaxK];
  uint64_t cand[kMaxK][kMaxCand];
  uint64_t best[kMaxK][kMaxF];
  int overflow[kMaxK];
  // phase 2
  float2 part[kThreads];
  float L[kMaxR2];
  float N[kMaxK];
  int myset[kMaxF];
  int nmyset, k, last, cstar, clamp, fallback;
  float target, base, R;
  float ai[kMaxK];
  float res[kMaxTiles];
  float shf[8];
  int shi[8];
  uint32_t shk[2 * kWaves];
  float wv[kMaxF];
  int wi[kMaxF];
};

template <class ET, int FM>
__global__ __launch_bounds__(kThreads, 4) void verify_fused_kernel(VerifyArgs a) {
  using T = typename ET::T;
  constexpr int G = (sizeof(T) == 2) ? 9 : 5;  // rows per load group (36-40 VGPRs of payload)
  __shared__ Shared sh;

  const int t = threadIdx.x, lane = t & 63, grp = t >> 4;
  const int K = a.K, V = a.V, R2 = 2 * K + 1, nT = a.T;
  const float cc = a.c2;
  const bool aligned = a.aligned != 0;
  const int tile = blockIdx.x % nT;
  const int c0 = tile * kTile;
  const int e0 = c0 + t * kSubElems;

  {
    const int b = a.b0 + int(blockIdx.x) / nT;
    const T* draft = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride;
    const T* target = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride;
    auto row_ptr = [&](int r) -> const T* {
      return (r < K) ? draft + int64_t(r) * V : target + int64_t(r - K) * V;
    };
    uint32_t* cnt1 = a.cnt + int64_t(b) * 64;
    uint32_t* cnt2 = cnt1 + 32;

    // ---- per-sequence scalars for phase 2. Their first-level loads are issued now; the gathers
    // that depend on them go out after the first row group's loads, and the values stay raw in
    // registers until after phase 1, so none of this delays the tile stream.
    const int x_ld = (t < K) ? a.x[b * K + t] : -1;
    const float u_r = (t <= K) ? a.u[b * (K + 1) + t] : 0.f;
    const int sv_ld = (t < K * a.sF) ? a.sset[int64_t(b) * K * a.sF + t] : -1;
    int x_r = -1, my_set = -1;
    uint32_t zq_bits = 0, zp_bits = 0, zs_bits = 0;

    // ---- phase 1: statistics and top-F candidates of this tile, rows in load groups of G
    TRACE(0);
    if (t < kMaxK) {
      sh.ncand[t] = 0;
      sh.F[t] = (t < K) ? a.topfF[t] : 0;  // uniform-index reads of the kernel arguments
    }
    __syncthreads();
    const bool vec = aligned && e0 + kSubElems <= V;  // this thread's tokens load as vectors
    for (int g0 = 0; g0 < R2; g0 += G) {
      RawTile<ET> raw[G];
      // every slot of the group is loaded (past the last row: the last row again, a cache hit)
      // and consumed below, so no load is left pending at the loop's back edge
      if (vec) {
#pragma unroll
        for (int j = 0; j < G; ++j) load_raw_vec<ET>(row_ptr(min(g0 + j, R2 - 1)), e0, raw[j]);
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j) load_raw_scalar<ET>(row_ptr(min(g0 + j, R2 - 1)), e0, V, raw[j]);
      }
      if (g0 == 0) {
        // the draft tokens reach LDS after the row loads are in flight (waiting for them drains
        // only the loads issued before the rows)
        if (t < K) sh.xe[t] = x_ld;
        __syncthreads();
        if (t < K) {
          if (unsigned(x_ld) < unsigned(V)) {
            x_r = x_ld;
            zq_bits = raw_bits<ET>(draft + int64_t(t) * V, x_ld);
            zp_bits = raw_bits<ET>(target + int64_t(t) * V, x_ld);
          } else if (tile == 0) {
            atomicOr(a.flags, kFlagBadToken);
          }
        }
        if (t < K * a.sF) {
          my_set = (unsigned(sv_ld) < unsigned(V)) ? sv_ld : -1;
          if (my_set >= 0) zs_bits = raw_bits<ET>(draft + int64_t(t / a.sF) * V, sv_ld);
        }
      }
      // statistics: thread max, sum 2^(z c - max c), merged over 16-lane groups by DPP
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
        const float M = row16_max(m);
        const float Mc = M * cc;
        const float sc = (s > 0.f) ? s * ex2(mc - Mc) : 0.f;
        const float S = row16_sum(sc);
        if ((t & 15) == 0 && r < R2) sh.g16[r][grp] = make_float2(Mc, S);
        if (j == 0 && g0 == 0) TRACE(8);
        // top-F candidates of a draft row (sampled token left out), filtered against a wave
        // threshold, then appended to the row's candidate list in LDS
        if (FM > 0 && r < K && a.topfF[r] > 0) {
          const int F = a.topfF[r];
          const int xr = sh.xe[r];
          float lm = -INFINITY;
#pragma unroll
          for (int e = 0; e < kSubElems; ++e)
            if (e0 + e != xr && e0 + e < V) lm = fmaxf(lm, z[e]);
          // Threshold: the smallest of G group maxima, G in {4, 8, 16} the first >= F (groups of
          // 16, 8 or 4 lanes). F of those groups each hold a token at least that large, so every
          // top-F token of the wave, hence of the tile, passes the filter.
          lm = fmaxf(lm, dpp_f<kDppXor1>(lm));
          lm = fmaxf(lm, dpp_f<kDppXor2>(lm));  // quad maxima
          float gmin;
          if (F <= 4) {
            lm = fmaxf(lm, dpp_f<kDppHalfMirror>(lm));
            lm = fmaxf(lm, dpp_f<kDppMirror>(lm));  // 16-lane group maxima
            gmin = lm;
          } else if (F <= 8) {
            lm = fmaxf(lm, dpp_f<kDppHalfMirror>(lm));  // 8-lane group maxima
            gmin = fminf(lm, dpp_f<kDppMirror>(lm));
          } else {
            gmin = fminf(lm, dpp_f<kDppHalfMirror>(lm));
            gmin = fminf(gmin, dpp_f<kDppMirror>(gmin));
          }
          gmin = fminf(gmin, __shfl_xor(gmin, 16, 64));
          const float thr = fminf(gmin, __shfl_xor(gmin, 32, 64));
          uint32_t pass = 0;
#pragma unroll
          for (int e = 0; e < kSubElems; ++e) {
            const int idx = e0 + e;
            if (z[e] >= thr && z[e] > -INFINITY && idx != xr && idx < V) pass |= 1u << e;
          }
          if (pass) {
            int slot = atomicAdd(&sh.ncand[r], __popc(pass));
#pragma unroll
            for (int e = 0; e < kSubElems; ++e)
              if ((pass >> e) & 1u) {
                if (slot < kMaxCand) sh.cand[r][slot] = cand_key(z[e], e0 + e);
                ++slot;
              }
          }
        }
      }
    }
    TRACE(9);
    if (t < K) {
      sh.x[t] = x_r;
      sh.zq[t] = bits_to_f<ET>(zq_bits);
      sh.zp[t] = bits_to_f<ET>(zp_bits);
    }
    if (t <= K) sh.u[t] = u_r;
    if (t < K * a.sF) {
      sh.set[t] = my_set;
      sh.zs[t] = bits_to_f<ET>(zs_bits);
    }
    __syncthreads();
    if (FM > 0) {  // wave w selects the F best candidates (value desc, index asc) of rows w, w+4, ...
      const int w = t >> 6;
      for (int r = w; r < K; r += kWaves) {
        const int F = sh.F[r];
        const int n = sh.ncand[r];
        if (n > kMaxCand) {
          if (lane == 0) sh.overflow[r] = 1;
          continue;
        }
        if (lane == 0) sh.overflow[r] = 0;
        uint64_t key[3];  // kMaxCand <= 3 * 64
#pragma unroll
        for (int i = 0; i < 3; ++i) key[i] = (lane + 64 * i < n) ? sh.cand[r][lane + 64 * i] : 0ull;
        for (int f = 0; f < F; ++f) {
          uint64_t mine = key[0];
#pragma unroll
          for (int i = 1; i < 3; ++i) mine = (key[i] > mine) ? key[i] : mine;
          uint32_t hi = uint32_t(mine >> 32), lo = uint32_t(mine);
          wave_max_key(hi, lo);
          const uint64_t win = (uint64_t(hi) << 32) | lo;
          if (lane == 0) sh.best[r][f] = win;
#pragma unroll
          for (int i = 0; i < 3; ++i)
            if (key[i] == win) key[i] = 0;  // keys are unique: only the winner is cleared
        }
      }
    }
    __syncthreads();
    TRACE(10);
    if (FM > 0) {
      // exact fallback when ties flood the candidate list: reload the row (from cache), keep
      // per-thread sorted lists and merge them block-wide
      for (int r = 0; r < K; ++r) {
        if (!sh.overflow[r]) continue;
        const int F = a.topfF[r];
        RawTile<ET> rw;
        load_raw<ET>(row_ptr(r), e0, V, aligned, rw);
        float z[kSubElems];
        unpack_tile<ET>(rw, z);
        TopList<(FM > 0 ? FM : 1)> tl;
        tl.init(F);
#pragma unroll
        for (int e = 0; e < kSubElems; ++e)
          if (e0 + e < V) tl.offer(z[e], e0 + e, sh.xe[r]);
        block_merge_top<(FM > 0 ? FM : 1)>(tl, F, sh.shk, sh.wv, sh.wi);
        if (t == 0)
          for (int f = 0; f < F; ++f) sh.best[r][f] = (sh.wi[f] >= 0) ? cand_key(sh.wv[f], sh.wi[f]) : 0;
        __syncthreads();
      }
    }

    // ---- publish the tile's partials, then arrive
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
    TRACE(1);
    wait_vmem();
    __syncthreads();
    if (t == 0) atomicAdd(cnt1, 1u);

    // ---- wait for the other tiles of the sequence
    if (t == 0) {
      int spins = 0;
      while (ld_agent(cnt1) < unsigned(nT)) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > a.spin_limit) {
          atomicOr(a.flags, kFlagTimeout);
          break;
        }
      }
    }
    // de-duplicate the Saguaro sets meanwhile (first occurrence of each token counts)
    if (t < K * a.sF && my_set >= 0) {
      const int i = t / a.sF, f = t - i * a.sF;
      for (int g = 0; g < f; ++g)
        if (sh.set[i * a.sF + g] == my_set) my_set = -1;
    }
    __syncthreads();
    TRACE(2);
    if (t < K * a.sF) sh.set[t] = my_set;

    // ---- phase 2: merge statistics (thread (r, j) takes tiles j, j + TPR, ... of row r)
    const int TPR = kThreads / R2;
    {
      const int r = t / TPR, j = t - r * TPR;
      float M = -INFINITY, S = 0.f;
      if (r < R2) {
        const uint64_t* st = a.stats + (int64_t(b) * R2 + r) * nT;
        constexpr int kAhead = 8;  // loads in flight per thread
        uint64_t vals[kAhead];
        for (int q0 = j; q0 < nT; q0 += kAhead * TPR) {
#pragma unroll
          for (int i = 0; i < kAhead; ++i) {
            const int q = q0 + i * TPR;
            vals[i] = (q < nT) ? ld_agent(st + q) : 0ull;
          }
#pragma unroll
          for (int i = 0; i < kAhead; ++i) {
          const uint64_t v = vals[i];
          const float m = lo_f(v), s = hi_f(v);
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
      }
      sh.part[t] = make_float2(M, S);
    }
    __syncthreads();
    if (t < R2) {
      float M = -INFINITY;
      for (int j = 0; j < TPR; ++j) M = fmaxf(M, sh.part[t * TPR + j].x);
      float S = 0.f;
      for (int j = 0; j < TPR; ++j) {
        const float2 v = sh.part[t * TPR + j];
        if (v.y > 0.f) S += v.y * ex2(v.x - M);
      }
      sh.L[t] = M + lg2(S);
    }
    __syncthreads();

    TRACE(3);
    // ---- accept decisions (bit-identical in every tile of the sequence)
    if (t == 0) {
      int k = K;
      const float C = a.C;
      for (int i = 0; i < K; ++i) {
        const float Lq = sh.L[i], Lp = sh.L[K + i];
        float Nn = 1.f;
        bool xin = false;
        if (a.sF > 0) {
          float sig = 0.f;
          for (int f = 0; f < a.sF; ++f) {
            const int sv = sh.set[i * a.sF + f];
            if (sv < 0) continue;
            sig += ex2(fmaf(sh.zs[i * a.sF + f], cc, -Lq));
            if (sv == sh.x[i]) xin = true;
          }
          Nn = 1.f - (1.f - C) * sig;
          if (!(Nn > 0.f) && tile == 0) atomicOr(a.flags, kFlagSaguaroNorm);
        }
        sh.N[i] = Nn;
        bool accept;
        float ai;
        if (sh.x[i] < 0) {
          accept = false;
          ai = 0.f;
        } else {
          const float w = xin ? C : 1.f;
          const float dp = fmaf(sh.zp[i], cc, -Lp);  // log2 p(x)
          const float dq = fmaf(sh.zq[i], cc, -Lq);  // log2 q(x)
          if (w == 0.f || dq == -INFINITY) {         // q'(x) = 0: accept iff p(x) > 0
            accept = dp > -INFINITY;
            ai = accept ? 1.f : 0.f;
          } else {
            const float ratio = ex2(dp - dq) * (Nn / w);  // p(x) / q'(x)
            accept = sh.u[i] < ratio;
            ai = fminf(1.f, ratio);
          }
        }
        sh.ai[i] = ai;
        if (k == K && !accept) k = i;
      }
      sh.k = k;
      int n = 0;
      if (k < K)
        for (int f = 0; f < a.sF; ++f) {
          const int sv = sh.set[k * a.sF + f];
          if (sv >= 0) sh.myset[n++] = sv;
        }
      sh.nmyset = n;
    }
    __syncthreads();
    const int k = sh.k;
    const bool resid = k < K;
    const T* prow = target + int64_t(k) * V;
    const T* qrow = resid ? draft + int64_t(k) * V : nullptr;
    const float Lp = sh.L[K + k];
    const float Lq = resid ? sh.L[k] : 0.f;
    const float Nk = resid ? sh.N[k] : 1.f;
    const float w_out = 1.f / Nk, w_in = a.C / Nk;
    const int nset = sh.nmyset;

    // ---- residual mass of this tile, published; the last tile to arrive draws the bonus
    float rv[kSubElems], pre[kSubElems];
    sub_values<ET>(prow, qrow, c0, V, aligned, cc, Lp, Lq, w_out, w_in, sh.myset, nset, rv);
    const float total = sub_scan(rv, pre, sh.shf);
    TRACE(4);
    if (t == 0) {
      st_agent(a.res + int64_t(b) * nT + tile, total);
      wait_vmem();
      const unsigned old = atomicAdd(cnt2, 1u);
      sh.last = (old == unsigned(nT - 1));
    }
    __syncthreads();
    TRACE(5);

    if (sh.last) {
      for (int q = t; q < nT; q += kThreads) sh.res[q] = ld_agent(a.res + int64_t(b) * nT + q);
      __syncthreads();
      if (t == 0) {
        st_agent(cnt1, 0u);  // every tile has passed both counters: reset them for the next call
        st_agent(cnt2, 0u);
        float P = 0.f;
        for (int q = 0; q < nT; ++q) P += sh.res[q];
        const float target_v = sh.u[K] * P;
        int cstar = -1, last_pos = -1;
        float run = 0.f, base = 0.f;
        for (int q = 0; q < nT; ++q) {
          const float nxt = run + sh.res[q];
          if (sh.res[q] > 0.f) last_pos = q;
          if (cstar < 0 && nxt > target_v) {
            cstar = q;
            base = run;
          }
          run = nxt;
        }
        int clamp = 0;
        if (cstar < 0 && last_pos >= 0) {  // rounding pushed u R past the total
          cstar = last_pos;
          clamp = 1;
        }
        sh.fallback = (cstar < 0);  // all-zero residual
        sh.cstar = cstar;
        sh.clamp = clamp;
        sh.base = base;
        sh.target = target_v;
        sh.R = P;
      }
      __syncthreads();
      int bonus = -1;
      if (!sh.fallback) {
        const int cs = sh.cstar;
        sub_values<ET>(prow, qrow, cs * kTile, V, aligned, cc, Lp, Lq, w_out, w_in, sh.myset, nset, rv);
        sub_scan(rv, pre, sh.shf);
        const int f0 = cs * kTile + t * kSubElems;
        int first = INT_MAX, lastp = -1;
#pragma unroll
        for (int e = 0; e < kSubElems; ++e)
          if (rv[e] > 0.f) {
            lastp = f0 + e;
            if (first == INT_MAX && !sh.clamp && sh.base + pre[e] > sh.target) first = f0 + e;
          }
        first = block_min_i(first, sh.shi);
        lastp = block_max_i(lastp, sh.shi);
        bonus = (first != INT_MAX) ? first : lastp;
      } else {
        // residual identically zero (rounding only): draw from the target row p_k, R = 1
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
        bonus = (found >= 0) ? found : lastp;
      }
      if (t == 0) {
        a.k_out[b] = k;
        a.bonus_out[b] = bonus;
        if (a.rmass_out) a.rmass_out[b] = resid ? sh.R : 1.f;
      }
      if (a.aprob_out && t < K) a.aprob_out[b * K + t] = sh.ai[t];
      TRACE(6);
    }

    // ---- top-F guesses of draft rows tile, tile + T, ... (off the bonus's critical path). Keys
    // are unique (a token lives in one tile), so round f picks the largest key below round f-1's
    // winner.
    for (int r = tile; FM > 0 && r < K; r += nT) {
      const int F = a.topfF[r];
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
      uint64_t prev = ~uint64_t(0);
      for (int f = 0; f < F; ++f) {
        uint64_t bk = 0;
#pragma unroll
        for (int i = 0; i < kKeep; ++i)
          if (keys[i] < prev && keys[i] > bk) bk = keys[i];
        for (int q = t + kKeep * kThreads; q < n; q += kThreads) {  // beyond what registers hold
          const int tl = q / F, ff = q - tl * F;
          const uint64_t v = ld_agent(cd + int64_t(tl) * a.topfFmax + ff);
          if (v < prev && v > bk) bk = v;
        }
        uint32_t hi = uint32_t(bk >> 32), lo = uint32_t(bk);
        wave_max_key(hi, lo);
        __syncthreads();
        if (lane == 0) {
          sh.shk[2 * (t >> 6)] = hi;
          sh.shk[2 * (t >> 6) + 1] = lo;
        }
        __syncthreads();
        uint32_t gh = sh.shk[0], gl = sh.shk[1];
#pragma unroll
        for (int q = 1; q < kWaves; ++q)
          if (sh.shk[2 * q] > gh || (sh.shk[2 * q] == gh && sh.shk[2 * q + 1] > gl)) {
            gh = sh.shk[2 * q];
            gl = sh.shk[2 * q + 1];
          }
        const uint64_t win = (uint64_t(gh) << 32) | gl;
        if (t == 0) out[f] = (win != 0) ? int(~gl) : -1;
        prev = win;
      }
      for (int f = F + t; f < a.topfFmax; f += kThreads) out[f] = -1;
    }
    TRACE(7);
  }
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
