// Batched lossless draft verification on gfx950: one launch per call, or two for batches whose tiles
// do not all fit on the device at once (the streaming form, at the end of this file).
//
// Work unit: one 256-thread workgroup per (sequence b, tile of TILE tokens). A tile covers the same
// token range of every row of its sequence (K draft rows, K+1 target rows) and keeps all of them
// in registers from the first load to the last use, so every logit is read from memory once.
// Inside a tile, wave w owns tokens [w WTOK, (w + 1) WTOK); lane l holds E of them as NV 16-byte
// chunks, chunk j of lane l at token j CTOK + l VEC of the wave's range (VEC tokens per 16 bytes),
// so every load instruction of a wave reads 1 KB of contiguous memory.
//
//  statistics  A tile issues the loads of all its rows at once, then per row forms the lane maximum
//              and the sum of 2^(z c - max c) (c = log2(e) / T), merges them over the tile and
//              publishes the tile's (max c, sum) as two words tagged with the call. Draft rows also
//              mark the lanes that can hold one of the tile's best F+1 tokens and copy those lanes'
//              values to LDS (the top-F candidates); so does the extra draft row K, read for its
//              guesses only, when they are asked for.
//  arrival     The tile claims its residual chunk and adds one to its sequence's arrival counter.
//              The tile that brings the count to T, the closer, knows every tile has published.
//  decide      Wave 0 of the closer, alone, merges the T statistics of every row in one fixed
//              order, takes the accept decisions (k and the terms of the residual) and publishes
//              them as a small record of tagged words; wave 0 of every other tile polls the record.
//  guesses     Meanwhile waves 1 .. 3 of every tile select its best F per draft row from the copies
//              and publish them (waves 2 and 3 from the arrival on, wave 1 once it has learned the
//              tile's role and handed it to wave 0 through LDS).
//  residual    Each tile, once it has the decision (the record read within a bounded number of
//              polls), forms r = max(p_k - q'_k, 0) (p_K when every draft passes) from the rows in
//              registers and publishes its mass, tagged.
//  bonus       Every tile reads the T masses and finds the tile whose range holds u_K R; that tile
//              finds the token inside it from its registers (the closer, reading its two rows
//              again, if it gave its chunk up). The closer returns the sequence's counters to zero;
//              the last sequence advances the call tag.
//  merge       Guess row r of the sequence is merged by tile r mod T (waves 2 and 3), from every
//              tile's published keys, once its bonus work is done.
//
// The closer waits only on tiles that have arrived, never on one that may not have started, and a
// tile that has polled for the record its bound gives its chunk up and exits; the closer computes
// every chunk given up. So no workgroup needs another to be resident, and the result is the same
// on a busy device; an idle one gets it sooner.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ssd.h"
#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_plan.hpp"

namespace ssd {

constexpr int kMaxR2 = 2 * kMaxK + 1;
constexpr int kMaxT = kMaxV / kPlanMinTile;  // tiles of the longest row at the smallest tile
constexpr int kGroupsPerBlock = kThreads / 16;
// Per draft row and wave, the top-F candidates live in an LDS region of kRegW 64-bit words: either
// the raw chunks of the wave's hot lanes (at most Lay::HOT of them, kHot for any type), or a list of
// (float bits << 32 | ~token) entries from the compaction filter.
constexpr int kRegW = 64;
constexpr int kHot = 16;
static_assert(kRegW >= kMaxF + 1, "a wave region must hold an exact top-(F+1)");
static_assert(kRegW <= 64, "a key-list region gives at most one entry per lane");
// decision record: 64-bit words (call tag << 32 | value)
constexpr int kDecK = 0, kDecLp = 1, kDecLq = 2, kDecWout = 3, kDecWin = 4, kDecNset = 5, kDecSet = 6,
              kDecWords = kDecSet + kMaxF;
static_assert(kDecWords <= kPlanDecWords, "decision record exceeds its workspace slot");
// claim word states of a tile's residual chunk
constexpr uint32_t kClaimOwner = 1, kClaimAbandoned = 2, kClaimCloser = 3;
constexpr int kGroup = 4;  // chunks given up that the closer computes at once
// The thread that counts its tile in and publishes the tile's mass: lane 0 of wave 1. A wave's stores
// retire in order with its reads, so a wave waiting for a read (an atomic's count, a poll) also
// waits for every store it issued before; wave 0 publishes the statistics and polls, wave 1 does not.
constexpr int kSignalThread = 64;

#ifndef SSD_VERIFY_PRIO
#define SSD_VERIFY_PRIO 1  // phase-1 issue priority by progress
#endif
#ifndef SSD_VERIFY_AHEAD
#define SSD_VERIFY_AHEAD 4  // row slots of a tile in flight before the first is consumed
#endif

#ifdef SSD_TRACE
// analysis builds only: 100 MHz timestamps per workgroup at each step (slot i of 16), and values
constexpr int kTraceSlots = 16;
// the counter is read through the scalar memory path; waiting right after the read keeps the sample
// from being taken only at some later wait
__device__ __forceinline__ uint64_t trace_clock() {
  uint64_t v;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v));
  return v;
}
#define TRACE(i)                                                                                        \
  do {                                                                                                  \
    if (threadIdx.x == 0 && a.trace) a.trace[int64_t(blockIdx.x) * kTraceSlots + (i)] = trace_clock(); \
  } while (0)
#define TRACEV(i, v)                                                                         \
  do {                                                                                       \
    if (threadIdx.x == 0 && a.trace) a.trace[int64_t(blockIdx.x) * kTraceSlots + (i)] = (v); \
  } while (0)
#define TRACE_AT(i, thr)                                                                               \
  do {                                                                                                 \
    if (threadIdx.x == (thr) && a.trace) a.trace[int64_t(blockIdx.x) * kTraceSlots + (i)] = trace_clock(); \
  } while (0)
#else
#define TRACE_AT(i, thr) \
  do {                   \
  } while (0)
#define TRACE(i) \
  do {           \
  } while (0)
#define TRACEV(i, v) \
  do {               \
  } while (0)
#endif

template <class ET, int NV>
struct Lay {
  using T = typename ET::T;
  static constexpr int VEC = 16 / int(sizeof(T));  // tokens per 16-byte chunk
  static constexpr int E = NV * VEC;               // tokens per lane and row
  static constexpr int WTOK = 64 * E;              // tokens per wave
  static constexpr int CTOK = 64 * VEC;            // tokens per chunk across a wave
  static constexpr int TILE = kThreads * E;        // tokens per tile
  // hot-lane copies: lanes of one selection round per slot, slots per round, rounds per wave region
  static constexpr int SPR = 64 / E;
  // hot lanes a wave copies: 16 for fp32 (16 guesses take the copy), 8 for bf16, whose rounds read
  // every slot
  static constexpr int HOT = (sizeof(T) == 4) ? 16 : 8;
  static_assert(HOT <= kHot, "the lane-id table holds kHot lanes per wave");
  static constexpr int PARTS = (HOT + SPR - 1) / SPR;
  static constexpr int SEL = kWaves * PARTS;
  static_assert(HOT * NV * 2 <= kRegW, "a wave region must hold HOT lanes' chunks");
  // token of element q of a lane whose first token is bl
  __device__ static __forceinline__ int tok(int bl, int q) { return bl + (q / VEC) * CTOK + (q % VEC); }
};

template <int NV>
struct Raw {
  uint4 w[NV];
};

// One row's chunks of a lane. Aligned rows (AL) take 16-byte loads from a clamped, valid address
// (a chunk lies wholly inside or wholly past the row; the ones past V are masked after unpacking).
// Rows not 16-byte aligned take element loads, positions past V reading as -inf.
template <class ET>
__device__ __forceinline__ uint4 chunk_scalar(const typename ET::T* row, int tok0, int V) {
  uint32_t wd[4];
  if (sizeof(typename ET::T) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v = __float_as_uint(ET::one(row, min(tok0 + i, V - 1)));
      wd[i] = (tok0 + i < V) ? v : 0xFF800000u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __float_as_uint(ET::one(row, min(tok0 + 2 * i, V - 1))) >> 16;
      const uint32_t hi = __float_as_uint(ET::one(row, min(tok0 + 2 * i + 1, V - 1))) >> 16;
      wd[i] = ((tok0 + 2 * i < V) ? lo : 0xFF80u) | (((tok0 + 2 * i + 1 < V) ? hi : 0xFF80u) << 16);
    }
  }
  return make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

template <class ET, int NV, bool AL>
__device__ __forceinline__ void load_row(const typename ET::T* row, int bl, int V, Raw<NV>& r) {
  using LY = Lay<ET, NV>;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if (AL)
      r.w[j] = load16(row + min(bl + j * LY::CTOK, V - LY::VEC));
    else
      r.w[j] = chunk_scalar<ET>(row, bl + j * LY::CTOK, V);
  }
}

// tail: the tile has chunks past V (aligned rows only; element loads read -inf there already)
template <class ET, int NV>
__device__ __forceinline__ void unpack_row(const Raw<NV>& r, int bl, int V, bool tail, float (&z)[Lay<ET, NV>::E]) {
  using LY = Lay<ET, NV>;
#pragma unroll
  for (int j = 0; j < NV; ++j) ET::unpack(r.w[j], z + j * LY::VEC);
  if (tail) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const bool in = bl + j * LY::CTOK < V;
#pragma unroll
      for (int e = 0; e < LY::VEC; ++e) z[j * LY::VEC + e] = in ? z[j * LY::VEC + e] : -INFINITY;
    }
  }
}

__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) { return (uint64_t(tag) << 32) | v; }
// An empty instruction that takes v and gives it back: arithmetic on v cannot move above it. Used on
// a value a returning atomic brings back inside a one-lane branch, so the wave waits for the atomic
// where the value is read, not where it is issued.
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return uint32_t(w >> 32); }
__device__ __forceinline__ float val_f(uint64_t w) { return __uint_as_float(uint32_t(w)); }
template <class P>
__device__ __forceinline__ void st_agent(P* p, P v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class P>
__device__ __forceinline__ P ld_agent(const P* p) {
  return __hip_atomic_load(const_cast<P*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS of a workgroup. RK: the draft rows whose top-F candidates it keeps (K + 1 at most, the extra
// row included; sized by the kernel's row budget, so a kernel for short drafts leaves room for more
// workgroups on a CU).
template <int RK>
struct SharedT {
  // per sequence, as given
  int F[kMaxK + 1];       // guesses per draft row (row K: the extra draft row)
  float C[kMaxK];         // Saguaro factor per draft position
  int xe[kMaxK + 1];      // draft tokens (-1 for the extra row: nothing excluded)
  float u[kMaxK + 1];     // uniforms
  int sv[kMaxK * kMaxF];  // Saguaro-set entries
  float zg[2 * kMaxK];    // logits at the draft tokens: draft rows 0..K-1, then target rows 0..K-1
  float zs[kMaxK * kMaxF];  // draft logits at the set entries
  int set[kMaxK * kMaxF];   // de-duplicated in-range set entries, -1 elsewhere
  // statistics
  float2 g16[2 * RK - 1][kGroupsPerBlock];  // (max c, sum) per 16-lane group and row
  float L[kMaxR2];                      // log2 normaliser of every row (merged over the tiles)
  // top-F candidates per draft row and wave: nseg < 0 means -nseg hot lanes copied their raw
  // chunks (lane ids in hl), nseg >= 0 that many key entries
  uint64_t reg[RK][kWaves][kRegW];
  int nseg[RK][kWaves];
  int hl[RK][kWaves][kHot];
  uint32_t thr[RK][kWaves];  // the copy's threshold key: smaller tokens are no candidates
  uint32_t fb[kWaves];          // draft rows the wave filters again (bit r)
  uint64_t spare[kWaves][64];   // where the compaction's failing tokens are written
  // the decision record, as this tile uses it
  int k, nset;
  float Lp, Lq, w_out, w_in;
  int myset[kMaxF];
  // roles and waits
  int role;   // bit 0 closer
  int ready;  // waves 1 .. 3 that have staged their inputs (wave 1: and published the role)
  int go;    // the record (owners) or the masses (bonus) were read in time
  int todo, alldone, drawn;
  int todo_list[kMaxT];       // chunks given up, listed for the closer
  uint32_t took[(kMaxT + 31) / 32];  // bit q: the closer computed chunk q
  float wtg[kGroup][kWaves];  // per-wave masses of a group of such chunks
  // residual and bonus
  float wt[kWaves];
  float res[kMaxT];
  int cstar, clamp, fallback;
  int wfirst[kWaves], wlastp[kWaves];  // the tile search's per-wave crossing and last token of mass
  float base, target, R;
};

// Residual values of a lane's E tokens: r = max(p - q w / N, 0) with w = C on the Saguaro set
// (w_in = C / N, w_out = 1 / N), or r = p when `resid` is false; 0 past V.
template <class ET, int NV>
__device__ __forceinline__ void residual_values(const float (&zp)[Lay<ET, NV>::E], const float (&zq)[Lay<ET, NV>::E],
                                                bool resid, int bl, int V, float c, float Lp, float Lq, float w_out,
                                                float w_in, const int* set, int n_set, float (&rv)[Lay<ET, NV>::E]) {
  using LY = Lay<ET, NV>;
  uint32_t in_set = 0;  // bit q: element q is a Saguaro-set token
  for (int f = 0; f < n_set; ++f) {
    const int d = set[f] - bl;
    if (d >= 0) {
      const int j = d / LY::CTOK, rem = d - j * LY::CTOK;
      if (j < NV && rem < LY::VEC) in_set |= 1u << (j * LY::VEC + rem);
    }
  }
#pragma unroll
  for (int q = 0; q < LY::E; ++q) {
    const float pv = ex2(fmaf(zp[q], c, -Lp));
    if (resid) {
      const float w = ((in_set >> q) & 1u) ? w_in : w_out;
      rv[q] = fmaxf(pv - ex2(fmaf(zq[q], c, -Lq)) * w, 0.f);
    } else {
      rv[q] = pv;
    }
    if (LY::tok(bl, q) >= V) rv[q] = 0.f;
  }
}

// The tile's mass in one fixed order (lane, then DPP over the wave, then the waves in order); every
// thread returns the same bits. FENCED: barriers before and after keep wt_sh's other uses apart;
// without, the caller has a barrier right before and one right after (its next user's).
template <int E, bool FENCED = true>
__device__ __forceinline__ float tile_mass(const float (&rv)[E], float* wt_sh) {
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < E; ++q) s += rv[q];
  s = wave_sum(s);
  if (FENCED) __syncthreads();
  if ((threadIdx.x & 63) == 0) wt_sh[threadIdx.x >> 6] = s;
  __syncthreads();
  const float tot = (wt_sh[0] + wt_sh[1]) + (wt_sh[2] + wt_sh[3]);
  if (FENCED) __syncthreads();
  return tot;
}

// Prefix sums of the residual values in token order, relative to the tile start. Token order inside
// a tile is (wave, chunk, lane, element): element sums per chunk, a DPP scan over lanes per chunk,
// chunk bases per wave, wave bases per tile.
template <class ET, int NV>
__device__ __forceinline__ void tile_prefix(const float (&rv)[Lay<ET, NV>::E], float* wt_sh, float (&pre)[Lay<ET, NV>::E]) {
  using LY = Lay<ET, NV>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float pin[NV], cb[NV + 1];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < LY::VEC; ++e) sum += rv[j * LY::VEC + e];
    pin[j] = wave_incl_scan(sum);
  }
  cb[0] = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) cb[j + 1] = cb[j] + readlane_f(pin[j], 63);
  __syncthreads();
  if (lane == 0) wt_sh[w] = cb[NV];
  __syncthreads();
  float wb = 0.f, total = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i == w) wb = total;
    total += wt_sh[i];
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float p = wb + cb[j] + wave_shift_up1(pin[j]);
#pragma unroll
    for (int e = 0; e < LY::VEC; ++e) {
      p += rv[j * LY::VEC + e];
      pre[j * LY::VEC + e] = p;
    }
  }
  __syncthreads();
}

// The workgroup's search of its tile for the bonus token: the first token (ascending id) whose
// base + prefix exceeds target, or the last token of positive mass with clamp or when rounding
// leaves the tile's prefixes short of target (the crossing is then the tile's end, within
// rounding). Every thread returns the token (-1 when the tile holds no positive mass); *crossed, when
// asked, tells whether it is a crossing rather than the last token of mass.
template <class ET, int NV, class SH>
__device__ __forceinline__ int tile_search(const float (&rv)[Lay<ET, NV>::E], const float (&pre)[Lay<ET, NV>::E],
                                           int bl, float base, float target, bool clamp, SH& sh,
                                           bool* crossed = nullptr) {
  using LY = Lay<ET, NV>;
  int first = INT_MAX, lastp = -1;
#pragma unroll
  for (int q = 0; q < LY::E; ++q)
    if (rv[q] > 0.f) {
      const int tk = LY::tok(bl, q);
      lastp = max(lastp, tk);
      if (!clamp && base + pre[q] > target) first = min(first, tk);
    }
  first = wave_min_i(first);
  lastp = wave_max_i(lastp);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.wfirst[w] = first;
    sh.wlastp[w] = lastp;
  }
  __syncthreads();
  int f = sh.wfirst[0], l = sh.wlastp[0];
#pragma unroll
  for (int ww = 1; ww < kWaves; ++ww) {
    f = min(f, sh.wfirst[ww]);
    l = max(l, sh.wlastp[ww]);
  }
  __syncthreads();  // the slots are written again by the next search
  if (crossed) *crossed = f != INT_MAX;
  return (f != INT_MAX) ? f : l;
}

// The bonus scan over the T tile masses in sh.res (wave 0; every workgroup that runs it gets the same
// bits): the tile where the cumulative mass first exceeds u_K R and the base before it, or the last
// tile with mass when rounding leaves u_K R past the total, or the all-zero fallback.
template <class SH>
__device__ __forceinline__ void scan_masses(SH& sh, int nT, float uK) {
  const int lane = threadIdx.x & 63;
  const int per = (nT + 63) / 64;  // lane l takes consecutive tiles [l per, (l + 1) per)
  const int q0 = min(lane * per, nT), q1 = min(nT, q0 + per);
  float run = 0.f;
  for (int q = q0; q < q1; ++q) run += sh.res[q];
  const float inc = wave_incl_scan(run);
  const float Rtot = readlane_f(inc, 63);
  const float target_v = uK * Rtot;
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
  // lanes hold ascending runs of tiles: the first crossing is the lowest such lane's, the last tile
  // of mass the highest such lane's
  const uint64_t fm = __ballot(first != INT_MAX), lm = __ballot(lastpos >= 0);
  const int fl = fm ? int(__builtin_ctzll(fm)) : -1, ll = lm ? 63 - int(__builtin_clzll(lm)) : -1;
  const int cf = (fl >= 0) ? __builtin_amdgcn_readlane(first, fl) : INT_MAX;
  const int cl = (ll >= 0) ? __builtin_amdgcn_readlane(lastpos, ll) : -1;
  if (lane == fl) sh.base = base;
  if (lane == 0) {
    sh.cstar = (cf != INT_MAX) ? cf : cl;  // u R past the total by rounding: last tile with mass
    sh.clamp = (cf == INT_MAX);
    sh.fallback = (cf == INT_MAX && cl < 0);  // all-zero residual (rounding only)
    sh.target = target_v;
    sh.R = Rtot;
  }
}

// Residual identically zero (rounding only): the bonus is drawn from the target row p_k itself
// (prow, whose log2 normaliser is Lp), tile by tile in token order. Every thread returns the token.
template <class ET, int NV, bool AL, class SH>
__device__ __forceinline__ int fallback_draw(const typename ET::T* prow, int V, int nT, float cc, float Lp, float uK,
                                             SH& sh) {
  using LY = Lay<ET, NV>;
  constexpr int E = LY::E;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float run = 0.f;
  int found = -1, lastp = -1;
  for (int q = 0; q < nT && found < 0; ++q) {
    const int blq = q * LY::TILE + w * LY::WTOK + lane * LY::VEC;
    const bool tq = AL && ((q + 1) * LY::TILE > V);
    Raw<NV> rp;
    load_row<ET, NV, AL>(prow, blq, V, rp);
    float zp[E], v2[E], p2[E];
    unpack_row<ET, NV>(rp, blq, V, tq, zp);
    residual_values<ET, NV>(zp, zp, false, blq, V, cc, Lp, 0.f, 1.f, 1.f, sh.myset, 0, v2);
    tile_prefix<ET, NV>(v2, sh.wt, p2);
    const float tot = tile_mass<E>(v2, sh.wt);
    bool crossed;
    const int tk = tile_search<ET, NV>(v2, p2, blq, run, uK, false, sh, &crossed);
    // a crossing in this tile (the search's first token), or its last positive token
    if (crossed) found = tk;
    if (tk >= 0) lastp = tk;
    run += tot;
  }
  return (found >= 0) ? found : lastp;
}

// Two layouts of a guess row's keys across one wave: by tile (T <= 64 tiles and F <= 4 guesses:
// lane q holds tile q's F keys, which its selection published in descending order) or spread (lane
// l holds keys l, l + 64, ...: key q is guess q mod F of tile q / F).
__device__ __forceinline__ bool guess_row_by_tile(int nT, int F) { return nT <= 64 && F <= 4; }

// The two words of every key of guess row r, requested by one wave in the row's layout: every lane
// reads a clamped, valid address; the keys past the row's are replaced by the merge.
template <int kM>
__device__ __forceinline__ void request_guess_row(const VerifyArgs& a, int b, int r, uint64_t (&hi)[kM], uint64_t (&lo)[kM]) {
  static_assert(kM >= 4, "the by-tile layout holds 4 keys a lane");
  const int lane = threadIdx.x & 63;
  const int K = a.K, nT = a.T;
  const int F = a.topfF[r], F1 = max(F, 1);
  const uint64_t* cd = a.cand + (int64_t(b) * (K + 1) + r) * a.Tcap * a.Fcap * 2;
  if (guess_row_by_tile(nT, F)) {
    const uint64_t* ct = cd + int64_t(min(lane, nT - 1)) * a.Fcap * 2;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (f >= F) break;
      hi[f] = ld_agent(ct + 2 * f);
      lo[f] = ld_agent(ct + 2 * f + 1);
    }
  }
  // (the spread layout requests its keys in the merge itself)
}

// The merge of sequence b's guesses of draft row r by one wave, once every tile of the sequence
// has published its own best F of the row (each key two words tagged with the call; the polls only
// wait for the words to be seen). Keys are unique (a token lives in one tile), so round f picks the
// largest key below round f-1's. kM: keys per lane held in registers (more keys per row: every round
// reads them again). hi/lo: the row's words if `requested` already (request_guess_row).
template <int kM, class SH>
__device__ __forceinline__ void merge_guess_row(const VerifyArgs& a, const SH& sh, int b, uint32_t tag,
                                                int long_bound, int r, uint64_t (&hi)[kM], uint64_t (&lo)[kM],
                                                bool requested) {
  const int lane = threadIdx.x & 63;
  const int K = a.K, nT = a.T, Tc = a.Tcap;
  const int F = __builtin_amdgcn_readfirstlane(sh.F[r]), F1 = max(F, 1);
  const int width = (r < K) ? a.topfFmax : a.lastF;
  int32_t* out = (r < K) ? a.topf_out + (int64_t(b) * K + r) * a.topfFmax : a.topf_last_out + int64_t(b) * a.lastF;
  const uint64_t* cd = a.cand + (int64_t(b) * (K + 1) + r) * Tc * a.Fcap * 2;
  const int n = nT * F;
  if (guess_row_by_tile(nT, F)) {
    // lane q: tile q's keys in descending order; round f takes the wave maximum of the lanes' heads
    // and the lane that held it moves its head on
    if (!requested) request_guess_row<kM>(a, b, r, hi, lo);
    for (int spins = 0;; ++spins) {
      __builtin_amdgcn_sched_barrier(0);
      bool ok = true;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const bool in = f < F && lane < nT;
        hi[f] = in ? hi[f] : tagged(tag, 0u);
        lo[f] = in ? lo[f] : tagged(tag, 0u);
        ok = ok && tag_of(hi[f]) == tag && tag_of(lo[f]) == tag;
      }
      if (__all(ok)) break;
      if (spins > long_bound) {
        if (!ok) atomicOr(a.flags, kFlagTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      request_guess_row<kM>(a, b, r, hi, lo);
    }
    uint64_t key[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) key[f] = (uint64_t(uint32_t(hi[f])) << 32) | uint32_t(lo[f]);
    int h = 0;
    uint64_t head = key[0];
    for (int f = 0; f < F; ++f) {
      const uint64_t win = wave_max_u64(head);
      if (lane == 0) out[f] = win ? int(~uint32_t(win)) : -1;
      if (head == win) {  // keys are unique: only the winner's lane moves on (0 stays 0)
        ++h;
        head = (h == 1) ? key[1] : (h == 2) ? key[2] : (h == 3) ? key[3] : 0ull;
      }
    }
  } else if (n <= 64 * kM) {
    // every key's two words requested at once, then the tags checked (read again if not yet in)
    uint64_t hk[kM], lk[kM];
    for (int spins = 0;; ++spins) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < kM; ++i) {
        const int q = lane + 64 * i;
        const int tl = q / F1, ff = q - tl * F1;
        const uint64_t* cw = cd + (int64_t(min(tl, nT - 1)) * a.Fcap + ff) * 2;
        hk[i] = (q < n) ? ld_agent(cw) : tagged(tag, 0u);
        lk[i] = (q < n) ? ld_agent(cw + 1) : tagged(tag, 0u);
      }
#pragma unroll
      for (int i = 0; i < kM; ++i) ok = ok && tag_of(hk[i]) == tag && tag_of(lk[i]) == tag;
      if (__all(ok)) break;
      if (spins > long_bound) {
        if (!ok) atomicOr(a.flags, kFlagTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    uint64_t key[kM];
#pragma unroll
    for (int i = 0; i < kM; ++i) key[i] = (uint64_t(uint32_t(hk[i])) << 32) | uint32_t(lk[i]);
    for (int f = 0; f < F; ++f) {
      uint64_t mine = key[0];
#pragma unroll
      for (int i = 1; i < kM; ++i) mine = max_u64(mine, key[i]);
      const uint64_t win = wave_max_u64(mine);
      if (lane == 0) out[f] = win ? int(~uint32_t(win)) : -1;
#pragma unroll
      for (int i = 0; i < kM; ++i) key[i] = (key[i] == win) ? 0ull : key[i];
    }
  } else {  // many tiles: every round reads the keys again, taking the largest below the last
    uint64_t prev = ~0ull;
    for (int f = 0; f < F; ++f) {
      uint64_t best = 0;
      for (int q = lane; q < n; q += 64) {
        const int tl = q / F1, ff = q - tl * F1;
        const uint64_t* cw = cd + (int64_t(tl) * a.Fcap + ff) * 2;
        uint64_t h = 0, l = 0;
        for (int spins = 0;; ++spins) {
          h = ld_agent(cw);
          l = ld_agent(cw + 1);
          if (tag_of(h) == tag && tag_of(l) == tag) break;
          if (spins > long_bound) {
            atomicOr(a.flags, kFlagTimeout);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        const uint64_t kq = (uint64_t(uint32_t(h)) << 32) | uint32_t(l);
        best = (kq < prev && kq > best) ? kq : best;
      }
      const uint64_t win = wave_max_u64(best);
      if (lane == 0) out[f] = win ? int(~uint32_t(win)) : -1;
      prev = win;
    }
  }
  for (int f = F + lane; f < width; f += 64) out[f] = -1;
}

// The merge of sequence b's guess rows first, first + step, ... by one workgroup (wave w takes the
// w-th of them, then every kWaves-th).
template <int kM, class SH>
__device__ __forceinline__ void merge_guesses_seq(const VerifyArgs& a, const SH& sh, int b, uint32_t tag,
                                                  int long_bound, int first = 0, int step = 1) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.K;
  const bool guess_rows = a.topfFmax > 0;
  const int KG = K + (a.lastF > 0 ? 1 : 0);
  for (int r = first + w * step; r < KG; r += kWaves * step) {
    if (r < K && !guess_rows) continue;
    uint64_t hi[kM], lo[kM];
    merge_guess_row<kM>(a, sh, b, tag, long_bound, r, hi, lo, false);
  }
}

// One round of the decision's merge reads: row r, tiles q0, q0 + 4, ... (kMergeAhead of them, both
// words of each; a tile past the row's tiles reads the last tile's words, in bounds, and counts as an
// empty statistic).
constexpr int kMergeAhead = 8;
struct StatsRound {
  uint64_t m[kMergeAhead], s[kMergeAhead];
};
__device__ __forceinline__ void load_stats_round(const uint64_t* st, int nT, uint32_t tag, int q0, StatsRound& v) {
  // every lane reads (a clamped tile); every read is issued before any value is selected, so the
  // wave waits once for all of them
#pragma unroll
  for (int i = 0; i < kMergeAhead; ++i) {
    const int qc = min(q0 + 4 * i, nT - 1);
    v.m[i] = ld_agent(st + 2 * qc);
    v.s[i] = ld_agent(st + 2 * qc + 1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kMergeAhead; ++i) {
    const bool in = q0 + 4 * i < nT;
    v.m[i] = in ? v.m[i] : tagged(tag, 0xFF800000u);
    v.s[i] = in ? v.s[i] : tagged(tag, 0u);
  }
}

// The decision of sequence b, taken by wave 0 alone (no barrier: the caller makes sh visible to the
// other waves). Inputs in LDS, visible to wave 0: sh.xe, sh.C, sh.u, sh.sv, sh.zg (logits at the
// draft tokens: draft rows, then target rows) and sh.zs (draft logits at the set entries); the
// last two may instead be written by `stage`, which runs once the statistics' requests are out
// (so the requests of both are in flight together).
// Every tile's statistics are merged in one fixed order: quad g of the wave merges rows g, g + 16,
// ...; lane l of the quad takes tiles l, l + 4, l + 8, ... in ascending order, then the quad combines
// its lanes. Each statistic is read once its two words carry the call's tag, polling at most `bound`
// times; false if some word was not seen by then (nothing decided; with flag_timeout the device
// flag is set). Then the accept tests (lane i = position i), the decision left in sh (k, the
// residual's normalisers, weights and set); record: published as the sequence's record; outputs: k
// and the accept probabilities written.
struct NoStage {
  __device__ void operator()() const {}
};
// One wave's part of the merge of every tile's statistics: rows 16 wi + 64 i + g (quad g), i >= 0,
// of a merge that nw waves share (wi = 0, nw = 1: every row). Each row's arithmetic is the same
// whichever wave takes it. Returns whether some word was not seen within the bound.
template <class SH>
__device__ __forceinline__ bool merge_stats_part(const VerifyArgs& a, SH& sh, int b, uint32_t tag, int bound,
                                                 int wi, int nw) {
  const int lane = threadIdx.x & 63, grp = lane >> 2, sub = lane & 3;
  const int R2 = 2 * a.K + 1, nT = a.T;
  const uint64_t* stb = a.stats + int64_t(b) * R2 * a.Tcap * 2;
  bool miss = false;
  for (int r0 = 16 * wi; r0 < R2; r0 += 16 * nw) {
    const int r = min(r0 + grp, R2 - 1);  // quads past the rows merge the last row again, unused
    const uint64_t* st = stb + int64_t(r) * a.Tcap * 2;
    float M = -INFINITY, S = 0.f;
    for (int qb = 0; qb < nT; qb += 4 * kMergeAhead) {
      StatsRound v;
      for (int spins = 0;; ++spins) {  // until both words of each tile carry this call's tag
        load_stats_round(st, nT, tag, qb + sub, v);
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kMergeAhead; ++i) ok = ok && tag_of(v.m[i]) == tag && tag_of(v.s[i]) == tag;
        if (__all(ok)) break;
        if (spins >= bound) {
          miss = miss || !ok;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      // the round's maximum first, then every sum scaled to it (independent terms; a tile without
      // mass adds nothing)
      float Mn = M;
#pragma unroll
      for (int i = 0; i < kMergeAhead; ++i)
        if (val_f(v.s[i]) > 0.f) Mn = fmaxf(Mn, val_f(v.m[i]));
      float Sn = (S > 0.f) ? S * ex2(M - Mn) : 0.f;
#pragma unroll
      for (int i = 0; i < kMergeAhead; ++i) {
        const float m = val_f(v.m[i]), s = val_f(v.s[i]);
        Sn += (s > 0.f) ? s * ex2(m - Mn) : 0.f;
      }
      M = Mn;
      S = Sn;
    }
    const float Mr = quad_max(M);
    const float Sr = quad_sum((S > 0.f) ? S * ex2(M - Mr) : 0.f);
    if (sub == 0 && r0 + grp < R2) sh.L[r0 + grp] = Mr + lg2(Sr);
  }
  return __any(miss);
}

template <class SH, class Stage = NoStage>
__device__ __forceinline__ bool decide_wave0(const VerifyArgs& a, SH& sh, int b, uint32_t tag, int bound,
                                             bool flag_timeout, bool record, bool outputs, Stage&& stage = Stage{},
                                             bool merged = false, bool merge_miss = false) {
  const int lane = threadIdx.x & 63;
  const int K = a.K, V = a.V, sF = a.sF;
  const float cc = a.c2;
  uint64_t* dec = a.dec + int64_t(b) * kPlanDecWords;
  // the statistics merged here, or already by several waves (merged: sh.L is visible)
  const bool miss = merged ? merge_miss : merge_stats_part(a, sh, b, tag, bound, 0, 1);
  stage();          // the caller's inputs of the accept tests, put in LDS now (stage: the caller's)
  wave_lds_sync();  // sh.L and those inputs before the lanes read them
  if (miss) {
    if (flag_timeout && lane == 0) atomicOr(a.flags, kFlagTimeout);
    return false;
  }
  // the Saguaro set entries that count (in range, first occurrence in their position's set)
  for (int j = lane; j < K * sF; j += 64) {
    const int i = j / sF, f = j - i * sF;
    const int sv = sh.sv[j];
    int set_v = (unsigned(sv) < unsigned(V)) ? sv : -1;
    for (int g = 0; g < f && set_v >= 0; ++g)
      if (sh.sv[i * sF + g] == set_v) set_v = -1;
    sh.set[j] = set_v;
  }
  wave_lds_sync();
  // lane i takes the accept test of position i
  const int i = min(lane, K - 1);
  const float C = sh.C[i];  // Saguaro factor of position i
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
    const float wx = xin ? C : 1.f;
    const float dp = fmaf(sh.zg[K + i], cc, -Lp);  // log2 p(x)
    const float dq = fmaf(sh.zg[i], cc, -Lq);      // log2 q(x)
    if (wx == 0.f || dq == -INFINITY) {            // q'(x) = 0: accept iff p(x) > 0
      accept = dp > -INFINITY;
      ai = accept ? 1.f : 0.f;
    } else {
      const float ratio = ex2(dp - dq) * (Nn / wx);  // p(x) / q'(x)
      accept = sh.u[i] < ratio;
      ai = fminf(1.f, ratio);
    }
  }
  if (outputs && a.aprob_out && lane < K) a.aprob_out[b * K + lane] = ai;
  const uint64_t rej = __ballot(lane < K && !accept);
  const int kk = rej ? __builtin_ctzll(rej) : K;  // first rejection
  const float Nk = (kk < K) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Nn), kk)) : 1.f;
  const float Ck = (kk < K) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(C), kk)) : 1.f;
  // the residual's terms, published as the record straight from registers: lane j writes word j
  // (the set of row k keeps its -1 holes: duplicates and out-of-range entries, which the residual
  // skips)
  const int nset = (kk < K) ? sF : 0;
  const float Lpk = sh.L[K + kk], Lqk = (kk < K) ? sh.L[kk] : 0.f;
  const int f = lane - kDecSet;
  const int sv = (f >= 0 && f < nset) ? sh.set[kk * sF + f] : -1;
  uint32_t v = uint32_t(sv);
  if (lane == kDecK) v = uint32_t(kk);
  if (lane == kDecLp) v = __float_as_uint(Lpk);
  if (lane == kDecLq) v = __float_as_uint(Lqk);
  if (lane == kDecWout) v = __float_as_uint(1.f / Nk);
  if (lane == kDecWin) v = __float_as_uint(Ck / Nk);
  if (lane == kDecNset) v = uint32_t(nset);
  if (record && lane < kDecSet + sF) st_agent(dec + lane, tagged(tag, v));
  if (lane == 0) {
    if (outputs) a.k_out[b] = kk;
    sh.k = kk;
    sh.nset = nset;
    sh.Lp = Lpk;
    sh.Lq = Lqk;
    sh.w_out = 1.f / Nk;
    sh.w_in = Ck / Nk;
  }
  if (lane < kMaxF) sh.myset[lane] = (lane < nset) ? sh.set[kk * sF + lane] : -1;
  return true;
}

// KM: register rows per tile are 2 KM + 1 (draft slots 0..KM-1, target slots KM..2KM), K <= KM.
// NV: 16-byte chunks per lane and row. AL: every row 16-byte aligned. SPLIT: the streaming form's
// first grid (statistics and guesses of every tile, nothing else; see the end of this file).
template <class ET, int KM, int NV, bool AL, bool SPLIT>
__global__ __launch_bounds__(kThreads, SPLIT ? kStreamWgPerCu : kVerifyWgPerCu) void verify_kernel(VerifyArgs a) {
  using T = typename ET::T;
  using LY = Lay<ET, NV>;
  constexpr int E = LY::E;
  constexpr int RM = 2 * KM + 1;
  __shared__ SharedT<KM + 1> sh;

  const int t = threadIdx.x, lane = t & 63, grp = t >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, in a scalar register
  const int K = a.K, V = a.V, R2 = 2 * K + 1, nT = a.T, sF = a.sF, Tc = a.Tcap;
  const float cc = a.c2;
  const int tile = blockIdx.x % nT;
  const int b = int(blockIdx.x) / nT;
  const int c0 = tile * LY::TILE;
  const int bl = c0 + w * LY::WTOK + lane * LY::VEC;  // first token of this lane
  const T* draft = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride;
  const T* target = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride;
  auto row_ptr = [&](int r) -> const T* {  // logical row r: draft rows 0..K-1, target rows K..2K
    return (r < K) ? draft + int64_t(r) * V : target + int64_t(r - K) * V;
  };
  uint32_t* ctr = a.seqctl + int64_t(b) * kPlanSeqCtlWords;  // [0] arrivals
  uint64_t* chunk = a.chunk + int64_t(b) * Tc * 2;
  uint64_t* dec = a.dec + int64_t(b) * kPlanDecWords;
  // The call's tag is one past the last call's. The last sequence to finish stores it, after every
  // tile of the call has started, so every tile reads the same value here.
  const uint32_t tag_ld = ld_agent(a.gtag);
  TRACE(0);
  // guesses of draft rows 0..K-1 (the sampled token excluded) and of the extra draft row K (nothing
  // excluded): KG rows go through the guess steps
  const bool guess_rows = a.topfFmax > 0, guess_last = a.lastF > 0;
  const bool guesses = guess_rows || guess_last;
  const int KG = K + (guess_last ? 1 : 0);
  const bool tail = AL && (c0 + LY::TILE > V);  // aligned rows: chunks past V in this tile

  // per-sequence inputs, loaded before the rows and staged to LDS after them
  const int x_v = (t < K) ? a.x[b * K + t] : -1;
  const float u_v = (t <= K) ? a.u[b * (K + 1) + t] : 0.f;
  int sv_v = -1;
  if (t < K * sF) sv_v = a.sset[int64_t(b) * K * sF + t];
  const int xg = (t < 2 * K) ? a.x[b * K + (t < K ? t : t - K)] : -1;

  const float c_v = (t < K) ? a.Cpos[t] : 1.f;
  const int f_v = (t <= K) ? a.topfF[t] : 0;
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the row loads

  // ---- the rows of the tile, in slot order (draft slots, then target): kAhead slots in flight at
  // first, then one more issued per slot consumed, so the requests of all workgroups interleave and
  // every workgroup's first rows land early. A slot past the sequence's rows loads the last row
  // again (a cache hit) and is never used. All rows stay in registers to the end.
  Raw<NV> raw[RM];
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int r = (s < KM) ? min(s, K - 1) : K + min(s - KM, K);
    load_row<ET, NV, AL>(row_ptr(r), bl, V, raw[s]);
  };
  // (the streaming form issues every row at once: its rows' registers are held anyway, and no
  // workgroup of it waits for another)
  constexpr int kAhead = SPLIT ? RM : ((SSD_VERIFY_AHEAD < RM) ? SSD_VERIFY_AHEAD : RM);
#pragma unroll
  for (int s = 0; s < kAhead; ++s) issue(s);
  __builtin_amdgcn_sched_barrier(0);

  const int Fp = max(a.topfFmax, a.lastF) + 1;  // candidates kept per wave: one more than the guesses
  if (lane == 0)  // rows not 16-byte aligned: every guess row is filtered from memory
    sh.fb[w] = AL ? 0u : ((guess_rows ? (1u << K) - 1u : 0u) | (guess_last ? 1u << K : 0u));

  // ---- statistics of every row, and the hot-lane copies of the draft rows
  // max and sum 2^(z c - max c) of one row over the lane's tokens, merged over 16-lane groups;
  // returns the order key of the lane's maximum (0: no finite token)
  auto row_stats = [&](const float (&z)[E], int r) __attribute__((always_inline)) -> uint32_t {
    float m = z[0];
#pragma unroll
    for (int q = 1; q < E; ++q) m = fmaxf(m, z[q]);
    const float mc = m * cc;
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < E; ++q) s[q & 3] += ex2(fmaf(z[q], cc, -mc));
    const bool fin = m > -INFINITY;  // a lane with no finite token adds nothing (its terms are NaN)
    const uint32_t mk = fin ? ordered_key(m) : 0u;
    const uint32_t Mk = row16_max_u(mk);  // the group's maximum through its order key
    const float Mc = (Mk ? key_to_float(Mk) : -INFINITY) * cc;
    const float S = row16_sum(fin ? ((s[0] + s[1]) + (s[2] + s[3])) * ex2(mc - Mc) : 0.f);
    if ((t & 15) == 0) sh.g16[r][grp] = make_float2(Mc, S);
    return mk;
  };
  // Draft rows r0 .. r0+nb-1 (nb <= 4) at once: the threshold of a row is the Fp-th largest of its
  // 16 quad maxima (quad = 4 lanes). Lanes 16 i + q gather quad q's maximum of row i, count the
  // quads of their row with a larger one (15 DPP row rotations); the smallest maximum with fewer
  // than Fp larger ones is it. At least Fp quads, so at least Fp lanes, reach it, so the lanes that
  // reach it ("hot") hold every top-Fp token of the wave: a token of any other lane has Fp larger
  // ones, the maxima of those lanes. With fewer than Fp non-empty quads the threshold is 0 and
  // every non-empty lane is hot. Hot lanes copy their raw chunks into the row's region (chunks past
  // V are dropped at selection); a row with more hot lanes than slots is filtered again later.
  auto draft_batch = [&](const Raw<NV>* rw, const uint32_t* mk, int r0, int nb) __attribute__((always_inline)) {
    if (Fp > LY::HOT) {  // more guesses than slots: every row of the batch is filtered later
      if (lane == 0)
        for (int i = 0; i < nb; ++i) sh.fb[w] |= 1u << (r0 + i);
      return;
    }
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nb) {
        const uint32_t g = uint32_t(__builtin_amdgcn_ds_bpermute((lane & 15) << 4, int(quad_max_u(mk[i]))));
        v = ((lane >> 4) == i) ? g : v;
      }
    }
    const uint32_t th = row16_min_u(row16_count_larger(v) < Fp ? v : 0xFFFFFFFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nb) {
        const int r = r0 + i;
        const uint32_t thr = uint32_t(__builtin_amdgcn_readlane(int(th), 16 * i));
        const bool hot = mk[i] >= thr && mk[i] != 0u;
        const uint64_t hm = __ballot(hot);
        const int n = __popcll(hm);
        if (n <= LY::HOT) {
          if (hot) {
            const int sl = __builtin_amdgcn_mbcnt_hi(uint32_t(hm >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(hm), 0u));
            uint4* dst = reinterpret_cast<uint4*>(&sh.reg[r][w][0]) + sl * NV;
#pragma unroll
            for (int j = 0; j < NV; ++j) dst[j] = rw[i].w[j];
            sh.hl[r][w][sl] = lane;
          }
          if (lane == 0) {
            sh.nseg[r][w] = -n;
            sh.thr[r][w] = max(thr, 0x00800000u);  // above the key of -inf
          }
        } else if (lane == 0) {
          sh.fb[w] |= 1u << r;
        }
      }
    }
  };
  // The extra draft row K (its guesses only) is read where the row slots run out; without it the
  // read repeats target row K (just loaded, a cache hit), so no branch surrounds the load.
  Raw<NV> rk;
  {
    uint32_t mk[KM];
#pragma unroll
    for (int s = 0; s < RM; ++s) {
      if (s + kAhead < RM) issue(s + kAhead);
      if (s + kAhead == RM) load_row<ET, NV, AL>(guess_last ? draft + int64_t(K) * V : target + int64_t(K) * V, bl, V, rk);
#if SSD_VERIFY_PRIO
      // A wave's issue priority falls as it gets through its rows, so the waves of the workgroups
      // that share a CU finish their statistics close together rather than the oldest first.
      if constexpr (!SPLIT) {
        const int q = (4 * s) / RM;  // a constant once the loop is unrolled
        if (q == 0) __builtin_amdgcn_s_setprio(3);
        else if (q == 1) __builtin_amdgcn_s_setprio(2);
        else if (q == 2) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
#endif
      __builtin_amdgcn_sched_barrier(0);
      if (s < KM) {
        mk[s] = 0u;
        if (s < K) {
          float z[E];
          unpack_row<ET, NV>(raw[s], bl, V, tail, z);
          mk[s] = row_stats(z, s);
        }
        if (AL && s % 4 == 3 && s - 3 < K && guess_rows)
          draft_batch(raw + (s - 3), mk + (s - 3), s - 3, min(4, K - (s - 3)));
      } else if (s - KM <= K) {
        float z[E];
        unpack_row<ET, NV>(raw[s], bl, V, tail, z);
        row_stats(z, K + (s - KM));
      }
    }
  }
  if (AL && guess_last) {
    float z[E];
    unpack_row<ET, NV>(rk, bl, V, tail, z);
    float m = z[0];
#pragma unroll
    for (int q = 1; q < E; ++q) m = fmaxf(m, z[q]);
    const uint32_t mkK = (m > -INFINITY) ? ordered_key(m) : 0u;
    draft_batch(&rk, &mkK, K, 1);
  }
  if (t < K) {
    sh.xe[t] = x_v;
    sh.C[t] = c_v;
  }
  if (t <= K) sh.F[t] = f_v;
  if (t == K) sh.xe[K] = -1;
  if (t <= K) sh.u[t] = u_v;
  if (t < K * sF) sh.sv[t] = sv_v;
  if (t == 0) sh.ready = 0;
  const uint32_t tag = (tag_ld + 1u == 0u) ? 1u : tag_ld + 1u;
#if SSD_VERIFY_PRIO
  if constexpr (!SPLIT) __builtin_amdgcn_s_setprio(0);
#endif
  __syncthreads();
  TRACE(1);

  // the tile's (max c, sum) of every row, tagged with the call (thread t < R2: row t)
  auto publish_stats = [&]() __attribute__((always_inline)) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kGroupsPerBlock; ++q) M = fmaxf(M, sh.g16[t][q].x);
    float S = 0.f;
#pragma unroll
    for (int q = 0; q < kGroupsPerBlock; ++q) {
      const float2 v = sh.g16[t][q];
      if (v.y > 0.f) S += v.y * ex2(v.x - M);
    }
    uint64_t* st = a.stats + ((int64_t(b) * R2 + t) * Tc + tile) * 2;
    st_agent(st, tagged(tag, __float_as_uint(M)));
    st_agent(st + 1, tagged(tag, __float_as_uint(S)));
  };
  // ---- the tile's guesses: its best F per draft row, published as tagged halves of 64-bit keys
  // (order key of the value << 32 | ~token)
  // Draft row r of a wave the hot-lane copy could not take: compaction of the tokens at or above
  // the threshold into the wave's region (exact top Fp from registers if too many pass).
  auto lane_thr = [&](float m, int& n) __attribute__((always_inline)) -> float {
    float mm = m, thr = -INFINITY;
    int taken = 0;
#pragma unroll 1
    for (int f = 0; f < Fp; ++f) {
      const float cur = wave_max(mm);
      if (!(cur > -INFINITY)) break;
      thr = cur;
      taken += __popcll(__ballot(mm == cur));
      if (taken >= Fp) break;
      mm = (mm == cur) ? -INFINITY : mm;
    }
    n = taken;
    return thr;
  };
  auto row_filter = [&](const float (&z)[E], int r) __attribute__((always_inline)) {
    float m = z[0];
#pragma unroll
    for (int q = 1; q < E; ++q) m = fmaxf(m, z[q]);
    int n;
    const float thr0 = lane_thr(m, n);
    const float thr = (n < Fp) ? -__FLT_MAX__ : thr0;  // fewer than Fp finite lanes: all finite pass
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < E; ++q) cnt += (z[q] >= thr) ? 1 : 0;
    const int incl = wave_incl_scan_i(cnt);
    int total = __builtin_amdgcn_readlane(incl, 63);
    uint64_t* region = sh.reg[r][w];
    if (total <= kRegW) {
      int slot = incl - cnt;
      uint64_t* spare = &sh.spare[w][lane];
#pragma unroll
      for (int q = 0; q < E; ++q) {
        const bool pass = z[q] >= thr;
        uint64_t* dst = pass ? region + slot : spare;
        *dst = (uint64_t(__float_as_uint(z[q])) << 32) | uint64_t(~uint32_t(LY::tok(bl, q)));
        slot += pass ? 1 : 0;
      }
    } else {  // too many pass (ties): the wave's exact top Fp from registers
      uint64_t prev = ~0ull;
#pragma unroll 1
      for (int f = 0; f < Fp; ++f) {
        uint64_t best = 0;
#pragma unroll
        for (int q = 0; q < E; ++q) {
          const uint64_t kq = (z[q] > -INFINITY)
                                  ? (uint64_t(ordered_key(z[q])) << 32) | uint64_t(~uint32_t(LY::tok(bl, q)))
                                  : 0ull;
          best = (kq < prev && kq > best) ? kq : best;
        }
        best = wave_max_u64(best);
        const uint32_t bh = uint32_t(best >> 32);
        if (lane == 0)  // raw float bits, as the compaction writes them (0 = none)
          region[f] = bh ? (uint64_t(__float_as_uint(key_to_float(bh))) << 32) | uint32_t(best) : 0ull;
        prev = best;
      }
      total = Fp;
    }
    if (lane == 0) sh.nseg[r][w] = total;
  };
  auto publish_guess = [&](int r, int f, uint64_t kv) __attribute__((always_inline)) {
    uint64_t* cw = a.cand + (((int64_t(b) * (K + 1) + r) * Tc + tile) * a.Fcap + f) * 2;
    st_agent(cw, tagged(tag, uint32_t(kv >> 32)));
    st_agent(cw + 1, tagged(tag, uint32_t(kv)));
  };
  // rows the hot-lane copy could not take (ties, more guesses than copy slots, rows not 16-byte
  // aligned): read again from cache and filtered (every thread calls it)
  auto refilter = [&]() __attribute__((always_inline)) {
    if ((sh.fb[0] | sh.fb[1] | sh.fb[2] | sh.fb[3]) != 0u) {
      uint32_t fbm = __builtin_amdgcn_readfirstlane(sh.fb[w]);
      while (fbm) {
        const int r = __builtin_ctz(fbm);
        fbm &= fbm - 1u;
        Raw<NV> rr;
        load_row<ET, NV, AL>(draft + int64_t(r) * V, bl, V, rr);  // guess rows are draft rows
        float z[E];
        unpack_row<ET, NV>(rr, bl, V, tail, z);
        row_filter(z, r);
      }
      __syncthreads();
    }
  };
  // The wave selects the F best candidates (value desc, index asc) of draft row r and hands each
  // to emit(r, f, key) on lane 0, in descending order (no barrier). Candidate round i reads the
  // region of wave i / PARTS: a copy gives lane l element l % E of slot l / E + SPR (i % PARTS); a
  // key list gives lane l its entry l + 64 (i % PARTS).
  auto select_row = [&](int r, auto&& emit) __attribute__((always_inline)) {
    {
      const int F = sh.F[r];
      const int e = lane % E;
      int n[kWaves];
      uint32_t th[kWaves];
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        n[ww] = __builtin_amdgcn_readfirstlane(sh.nseg[r][ww]);
        th[ww] = uint32_t(__builtin_amdgcn_readfirstlane(sh.thr[r][ww]));
      }
      if constexpr (sizeof(T) == 2) {
        // bf16: 32-bit keys, the value's 16-bit order key above 0xFFFF - (token - c0), so a larger
        // key is a larger value, then a smaller token; 0 = none (every real key is above 2^23).
        // Every read is issued first (clamped, in bounds), then the keys are formed. NP parts of
        // every wave's slots are read: the second only when some wave copied more than SPR lanes
        // (a key list never needs it), so the usual row forms half the keys.
        const uint32_t xs_l = uint32_t(sh.xe[r] - c0);  // the sampled token, relative to the tile
        auto select = [&](auto np) __attribute__((always_inline)) {
          constexpr int NP = decltype(np)::value, NSEL = kWaves * NP;
          uint32_t rawv[NSEL];
          int hlv[NSEL];
#pragma unroll
          for (int i = 0; i < NSEL; ++i) {
            const int ww = i / NP, slc = min(lane / E + LY::SPR * (i % NP), LY::HOT - 1);
            rawv[i] = reinterpret_cast<const uint16_t*>(&sh.reg[r][ww][0])[slc * E + e];
            hlv[i] = sh.hl[r][ww][slc];
          }
          uint32_t key[NSEL];
#pragma unroll
          for (int i = 0; i < NSEL; ++i) {
            const int ww = i / NP, part = i % NP;
            const int sl = lane / E + LY::SPR * part;
            const uint32_t raw16 = rawv[i];
            const uint32_t ok16 = (raw16 & 0x8000u) ? (~raw16 & 0xFFFFu) : (raw16 | 0x8000u);
            const uint32_t tl = uint32_t(ww * LY::WTOK + hlv[i] * LY::VEC + LY::tok(0, e));
            // th is above the key of -inf; the sampled token is never a guess
            const bool ok = (n[ww] < 0) & (sl < -n[ww]) & (ok16 >= (th[ww] >> 16)) & (int(tl) < V - c0) & (tl != xs_l);
            key[i] = ok ? (ok16 << 16) | (0xFFFFu - tl) : 0u;
            if (n[ww] > 64 * part) {  // uniform: a key list (its tokens lie in this tile)
              const uint64_t ent = sh.reg[r][ww][min(lane + 64 * part, kRegW - 1)];
              const uint32_t tk = uint32_t(int(~uint32_t(ent)) - c0);
              const uint32_t o16 = ordered_key(__uint_as_float(uint32_t(ent >> 32))) >> 16;
              key[i] = (lane + 64 * part < n[ww] && uint32_t(ent) != 0u && tk != xs_l)  // lo 0 = none
                           ? (o16 << 16) | (0xFFFFu - tk)
                           : 0u;
            }
          }
          for (int f = 0; f < F; ++f) {
            uint32_t mine = key[0];
#pragma unroll
            for (int i = 1; i < NSEL; ++i) mine = max(mine, key[i]);
            const uint32_t win = wave_max_u32(mine);
#pragma unroll
            for (int i = 0; i < NSEL; ++i) key[i] = (key[i] == win) ? 0u : key[i];  // keys are unique
            if (lane == 0) {  // back to the 64-bit (order key of the float, ~token) form
              const uint32_t h = win >> 16;
              const uint32_t okf = (h << 16) | ((h & 0x8000u) ? 0u : 0xFFFFu);
              emit(r, f, win ? (uint64_t(okf) << 32) | uint64_t(~uint32_t(c0 + int(0xFFFFu - (win & 0xFFFFu))))
                             : 0ull);
            }
          }
        };
        bool wide = false;  // uniform: some wave copied more lanes than one part holds
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) wide = wide || n[ww] < -LY::SPR;
        if (LY::PARTS > 1 && wide)
          select(std::integral_constant<int, LY::PARTS>{});
        else
          select(std::integral_constant<int, 1>{});
      } else {
        const int xs = sh.xe[r];
        uint64_t key[LY::SEL];
#pragma unroll
        for (int i = 0; i < LY::SEL; ++i) {
          const int ww = i / LY::PARTS, part = i % LY::PARTS;
          key[i] = 0;
          const int sl = lane / E + LY::SPR * part;
          if (n[ww] < 0 && LY::SPR * part < -n[ww]) {  // uniform: some slot of this part holds a copy
            const int slc = min(sl, LY::HOT - 1);
            const float v = ET::one(reinterpret_cast<const T*>(&sh.reg[r][ww][0]) + slc * E, e);
            const int tok = c0 + ww * LY::WTOK + sh.hl[r][ww][slc] * LY::VEC + LY::tok(0, e);
            const uint32_t kv = ordered_key(v);
            const bool ok = (sl < -n[ww]) & (kv >= th[ww]) & (tok < V) & (tok != xs);
            key[i] = ok ? (uint64_t(kv) << 32) | uint64_t(~uint32_t(tok)) : 0ull;
          } else if (n[ww] > 64 * part) {  // key list
            const uint64_t ent = sh.reg[r][ww][min(lane + 64 * part, kRegW - 1)];
            const float v = __uint_as_float(uint32_t(ent >> 32));
            const int tok = int(~uint32_t(ent));
            if (lane + 64 * part < n[ww] && uint32_t(ent) != 0u && tok != xs)  // entry lo 0 = none
              key[i] = (uint64_t(ordered_key(v)) << 32) | uint32_t(ent);
          }
        }
        // the nonzero keys (a few per wave region) into one list, one per lane: the F rounds then
        // take a single key per lane (more than 64: rounds over all of them)
        uint64_t* lst = sh.spare[w];
        int N = 0;
#pragma unroll
        for (int i = 0; i < LY::SEL; ++i) {
          const uint64_t m = __ballot(key[i] != 0ull);
          if (m) {
            const int at = N + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
            if (key[i] != 0ull && at < 64) lst[at] = key[i];
            N += __popcll(m);
          }
        }
        wave_lds_sync();  // the list's entries come from other lanes
        if (N <= 64) {
          uint64_t mine = (lane < N) ? lst[lane] : 0ull;
          for (int f = 0; f < F; ++f) {
            const uint64_t win = wave_max_u64(mine);
            if (lane == 0) emit(r, f, win);
            mine = (mine == win) ? 0ull : mine;  // keys are unique: only the winner is cleared
          }
        } else {
          for (int f = 0; f < F; ++f) {
            uint64_t mine = key[0];
#pragma unroll
            for (int i = 1; i < LY::SEL; ++i) mine = max_u64(mine, key[i]);
            const uint64_t win = wave_max_u64(mine);
            if (lane == 0) emit(r, f, win);
#pragma unroll
            for (int i = 0; i < LY::SEL; ++i) key[i] = (key[i] == win) ? 0ull : key[i];
          }
        }
      }
    }
  };
  // the streaming form: every row's best F published, wave w taking rows w, w + 4, ...
  auto tile_guesses = [&]() __attribute__((always_inline)) {
    refilter();
    for (int r = w; r < KG; r += kWaves) select_row(r, publish_guess);
  };
  const int long_bound = a.wait_polls * 8 + 4096;  // waits on tiles known to have arrived


  if constexpr (SPLIT) {  // the streaming form: statistics and guesses, resid_kernel takes the rest
    if (t < R2) publish_stats();
    if (guesses) tile_guesses();
    TRACE(9);
    return;
  }

  // rows the hot-lane copy could not take are filtered again before the tile arrives: the waves
  // that select below run beside the decision and meet no barrier until the residual
  if (guesses) refilter();

  // ---- publish the tile's statistics, claim the residual chunk, arrive (the signalling thread; the
  // closer also counts the sequence in: every tile of the sequence has read the call's tag once the
  // closer arrives; the count comes back while it works, and the last sequence advances the tag at
  // its end)
  if (t < R2) publish_stats();
  uint32_t seqs_before = 0;
  int role = 0;
  if (t == kSignalThread) {
    st_agent(chunk + 2 * tile, tagged(tag, kClaimOwner));
    if (add_agent(ctr, 1u) + 1u == uint32_t(nT)) {
      st_agent(ctr, 0u);  // every tile has counted itself in: back to zero
      seqs_before = add_agent(a.gdone, 1u);
      role = 1;
    }
  }
  // Waves 1 .. 3 check in (wave 1 once it knows the role and has put it in LDS), and wave 0, alone,
  // then takes the decision (the closer: its lanes put the point reads' logits in LDS first) or
  // reads the record (every other tile). Meanwhile waves 1 .. 3 select the tile's guesses: row r by
  // wave 2, 3, 1 for r = 0, 1, 2 (mod 3), waves 2 and 3 from the arrival on, wave 1 once the role
  // is known.
  if (w == 1) {
    const int rl = __builtin_amdgcn_readlane(role, 0);
    if (lane == 0) sh.role = rl;
    TRACE_AT(14, 64);
  }
  if (w == 2) TRACE_AT(15, 128);
  // (LDS ordering only: a release of every address space would make the wave wait for its own
  // requests in flight, the closer's count of finished sequences among them)
  if (w != 0 && lane == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __hip_atomic_fetch_add(&sh.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (w == 0) {
    while (__hip_atomic_load(&sh.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kWaves - 1)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    TRACE(2);
    if ((sh.role & 1) != 0) {
      // the logits at the draft tokens and at the Saguaro-set entries, requested ahead of the
      // statistics (every lane reads: a lane without an entry the row's first token): lane i the
      // draft token of row i (i < 2K), and the set entries lane, lane + 64, ... (K sF <= 4 * 64)
      constexpr int kSetSlots = (kMaxK * kMaxF + 63) / 64;
      const int nss = (K * sF + 63) >> 6;  // set slots a lane takes
      const bool g_ok = lane < 2 * K && unsigned(xg) < unsigned(V);
      const float zg_r = ET::one(row_ptr(lane < 2 * K ? lane : 0), g_ok ? xg : 0);
      float zs_r[kSetSlots];
      bool s_ok[kSetSlots];
#pragma unroll
      for (int m = 0; m < kSetSlots; ++m) {
        zs_r[m] = 0.f;
        s_ok[m] = false;
        if (m < nss) {
          const int j = lane + 64 * m;
          const int sv = (j < K * sF) ? sh.sv[j] : -1;
          s_ok[m] = unsigned(sv) < unsigned(V);
          zs_r[m] = ET::one(row_ptr(j < K * sF ? j / sF : 0), s_ok[m] ? sv : 0);
        }
      }
      decide_wave0(a, sh, b, tag, long_bound, true, true, true, [&]() __attribute__((always_inline)) {
        if (lane < 2 * K) sh.zg[lane] = g_ok ? zg_r : 0.f;
#pragma unroll
        for (int m = 0; m < kSetSlots; ++m)
          if (m < nss && lane + 64 * m < K * sF) sh.zs[lane + 64 * m] = s_ok[m] ? zs_r[m] : 0.f;
      });
      TRACE(3);
      if (lane == 0) sh.go = 1;
    } else {
      // poll the record until every word it needs carries this call's tag
      const int nw = kDecSet + sF;
      bool ok = false;
      uint64_t v = 0;
      for (int n = 0;; ++n) {
        v = (lane < nw) ? ld_agent(dec + lane) : tagged(tag, 0u);
        if (__all(tag_of(v) == tag)) {
          ok = true;
          break;
        }
        if (n >= a.wait_polls) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (ok) {
        const uint32_t x = uint32_t(v);
        if (lane == kDecK) sh.k = int(x);
        if (lane == kDecLp) sh.Lp = __uint_as_float(x);
        if (lane == kDecLq) sh.Lq = __uint_as_float(x);
        if (lane == kDecWout) sh.w_out = __uint_as_float(x);
        if (lane == kDecWin) sh.w_in = __uint_as_float(x);
        if (lane == kDecNset) sh.nset = int(x);
        if (lane >= kDecSet && lane < kDecSet + kMaxF) sh.myset[lane - kDecSet] = (lane < nw) ? int(x) : -1;
      }
      if (lane == 0) {
        sh.go = ok ? 1 : 0;
        if (!ok) st_agent(chunk + 2 * tile, tagged(tag, kClaimAbandoned));  // the closer computes it
      }
    }
  } else if (guesses) {
    for (int r = (w == 2) ? 0 : (w == 3) ? 1 : 2; r < KG; r += 3) select_row(r, publish_guess);
    TRACE_AT(11, 64 * w);
  }
  __syncthreads();
  const bool closer = (sh.role & 1) != 0;
  TRACE(4);
  TRACEV(12, uint64_t(sh.role) | (uint64_t(sh.go) << 8));

  // ---- residual of this tile from the rows in registers (target slot KM + k, draft slot k): its
  // values and prefix sums stay in registers, its mass is published
  float rv[E], pre[E];
#pragma unroll
  for (int q = 0; q < E; ++q) rv[q] = pre[q] = 0.f;
  int k = K;
  int nset = 0;
  if (sh.go) {
    k = min(max(__builtin_amdgcn_readfirstlane(sh.k), 0), K);
    nset = (k < K) ? min(max(sh.nset, 0), kMaxF) : 0;
    Raw<NV> rp = raw[KM], rq = raw[0];
#pragma unroll
    for (int s = 0; s <= KM; ++s)
      if (s == k) {
        rp = raw[KM + s];
        rq = raw[s < KM ? s : KM - 1];
      }
    float zp[E], zq[E];
    unpack_row<ET, NV>(rp, bl, V, tail, zp);
    unpack_row<ET, NV>(rq, bl, V, tail, zq);
    residual_values<ET, NV>(zp, zq, k < K, bl, V, cc, sh.Lp, sh.Lq, sh.w_out, sh.w_in, sh.myset, nset, rv);
    // (the barrier before the residual, and tile_prefix's first one, keep sh.wt's uses apart)
    const float total = tile_mass<E, false>(rv, sh.wt);
    if (t == kSignalThread) st_agent(chunk + 2 * tile + 1, tagged(tag, __float_as_uint(total)));
    TRACE(5);
    tile_prefix<ET, NV>(rv, sh.wt, pre);
  }
  // the merger waves (guess row r is merged by tile r mod T, waves 2 and 3 taking its rows in turn)
  // request their first row's keys now: every tile published its own before it read the record,
  // and the merge itself waits until the tile's bonus work is done
  uint64_t mhi[4], mlo[4];
  int mrow = -1;
  if (guesses && w >= 2) {
    const int r = tile + (w - 2) * nT;
    if (r < KG && !(r < K && !guess_rows)) {
      request_guess_row<4>(a, b, r, mhi, mlo);
      mrow = r;
    }
  }
  const bool go = sh.go != 0;

  // the residual values of tile q, its two rows read again
  auto refetch_values = [&](int q, float (&vals)[E]) __attribute__((always_inline)) -> int {
    const int blq = q * LY::TILE + w * LY::WTOK + lane * LY::VEC;
    const bool tq = AL && ((q + 1) * LY::TILE > V);
    Raw<NV> rp, rq;
    load_row<ET, NV, AL>(target + int64_t(k) * V, blq, V, rp);
    load_row<ET, NV, AL>(draft + int64_t(min(k, K - 1)) * V, blq, V, rq);
    float zp[E], zq[E];
    unpack_row<ET, NV>(rp, blq, V, tq, zp);
    unpack_row<ET, NV>(rq, blq, V, tq, zq);
    residual_values<ET, NV>(zp, zq, k < K, blq, V, cc, sh.Lp, sh.Lq, sh.w_out, sh.w_in, sh.myset, nset, vals);
    return blq;
  };

  // ---- the masses of all T tiles into sh.res: the closer waits for the owners and computes the
  // chunks they gave up; an owner polls them (a bounded number of times)
  if (closer) {
    for (int i = t; i < (nT + 31) / 32; i += kThreads) sh.took[i] = 0u;  // ordered by the loop's barrier
    for (int spins = 0;;) {
      // wave 0: masses that are in go to sh.res; the chunks given up are listed in ascending order
      if (t < 64) {
        bool all_in = true;
        int n_ab = 0;
        for (int c0 = 0; c0 < nT; c0 += 64) {
          const int c = c0 + lane;
          bool ab = false;
          if (c < nT) {
            const uint64_t mw = ld_agent(chunk + 2 * c + 1);
            if (tag_of(mw) == tag) {
              sh.res[c] = val_f(mw);
            } else {
              all_in = false;
              ab = ld_agent(chunk + 2 * c) == tagged(tag, kClaimAbandoned);
            }
          }
          const uint64_t m = __ballot(ab);
          if (ab)
            sh.todo_list[n_ab + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)))] = c;
          n_ab += __popcll(m);
        }
        const bool all = __all(all_in);
        if (lane == 0) {
          sh.todo = n_ab;
          sh.alldone = all ? 1 : 0;
        }
      }
      __syncthreads();
      if (sh.alldone) break;
      const int n_ab = sh.todo;
      if (n_ab > 0) {
        // the chunks given up, kGroup at a time: both rows of every chunk of a group are read at
        // once, then each chunk's mass is formed in tile_mass's order (the owner's bits)
        for (int g0 = 0; g0 < n_ab; g0 += kGroup) {
          const int gn = min(kGroup, n_ab - g0);
          int cs[kGroup];
          Raw<NV> rp[kGroup], rq[kGroup];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            cs[i] = sh.todo_list[g0 + min(i, gn - 1)];
            const int blq = cs[i] * LY::TILE + w * LY::WTOK + lane * LY::VEC;
            load_row<ET, NV, AL>(target + int64_t(k) * V, blq, V, rp[i]);
            load_row<ET, NV, AL>(draft + int64_t(min(k, K - 1)) * V, blq, V, rq[i]);
          }
          if (t < gn) {
            st_agent(chunk + 2 * cs[t], tagged(tag, kClaimCloser));
            atomicOr(&sh.took[cs[t] >> 5], 1u << (cs[t] & 31));
          }
          float part[kGroup];
#pragma unroll
          for (int i = 0; i < kGroup; ++i) {
            const int blq = cs[i] * LY::TILE + w * LY::WTOK + lane * LY::VEC;
            const bool tq = AL && ((cs[i] + 1) * LY::TILE > V);
            float zp[E], zq[E], v2[E];
            unpack_row<ET, NV>(rp[i], blq, V, tq, zp);
            unpack_row<ET, NV>(rq[i], blq, V, tq, zq);
            residual_values<ET, NV>(zp, zq, k < K, blq, V, cc, sh.Lp, sh.Lq, sh.w_out, sh.w_in, sh.myset, nset, v2);
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < E; ++q) sum += v2[q];
            part[i] = wave_sum(sum);
          }
          if (lane == 0) {
#pragma unroll
            for (int i = 0; i < kGroup; ++i) sh.wtg[i][w] = part[i];
          }
          __syncthreads();
          if (t < gn) {
            const float tot = (sh.wtg[t][0] + sh.wtg[t][1]) + (sh.wtg[t][2] + sh.wtg[t][3]);
            st_agent(chunk + 2 * cs[t] + 1, tagged(tag, __float_as_uint(tot)));
          }
          __syncthreads();
        }
        continue;
      }
      if (++spins > long_bound) {
        if (t == 0) atomicOr(a.flags, kFlagTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      __syncthreads();
    }
    if (t == 0) sh.go = 1;
  } else if (go) {
    if (t < 64) {
      bool ok = false;
      for (int n = 0;; ++n) {
        bool in = true;
        for (int c = lane; c < nT; c += 64) {
          const uint64_t mw = ld_agent(chunk + 2 * c + 1);
          in = in && tag_of(mw) == tag;
          sh.res[c] = val_f(mw);
        }
        if (__all(in)) {
          ok = true;
          break;
        }
        // the record was read, so the closer runs: every mass arrives (an owner that gives up
        // has its chunk computed by the closer)
        if (n >= long_bound) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (lane == 0) {
        sh.go = ok ? 1 : 0;
        if (!ok) atomicOr(a.flags, kFlagTimeout);
      }
    }
  }
  __syncthreads();
  TRACE(closer ? 7 : 6);

  // ---- the bonus (one copy for every role): the scan of the T masses, then the tile whose range
  // holds u_K R draws the token from its registers.
  if (sh.go) {
    if (t < 64) scan_masses(sh, nT, sh.u[K]);
    __syncthreads();
    TRACE(13);
    if (!sh.fallback && sh.cstar == tile) {
      const int tok = tile_search<ET, NV>(rv, pre, bl, sh.base, sh.target, sh.clamp != 0, sh);
      if (t == 0) {
        a.bonus_out[b] = tok;
        if (a.rmass_out) a.rmass_out[b] = (k < K) ? sh.R : 1.f;
      }
      TRACE(8);
    }
  }

  if (closer) {
    if (sh.fallback) {  // residual identically zero (rounding only): drawn from p_k itself, R = 0
      const int tok = fallback_draw<ET, NV, AL>(target + int64_t(k) * V, V, nT, cc, sh.Lp, sh.u[K], sh);
      if (t == 0) {
        a.bonus_out[b] = tok;
        if (a.rmass_out) a.rmass_out[b] = 0.f;
      }
    } else if (sh.cstar != tile && ((sh.took[sh.cstar >> 5] >> (sh.cstar & 31)) & 1u) != 0u) {
      // the owning tile gave its chunk up (computed here): the closer reads its two rows again and
      // draws; any other owner draws from its registers, having read the record
      const int cs = sh.cstar;
      float v2[E], p2[E];
      const int blq = refetch_values(cs, v2);
      tile_prefix<ET, NV>(v2, sh.wt, p2);
      const int tok = tile_search<ET, NV>(v2, p2, blq, sh.base, sh.target, sh.clamp != 0, sh);
      if (t == 0) {
        a.bonus_out[b] = tok;
        if (a.rmass_out) a.rmass_out[b] = (k < K) ? sh.R : 1.f;
      }
      TRACE(8);
    }
  }
  // ---- the sequence is done; the last sequence of the call advances the call tag
  if (closer && t == kSignalThread) {
    opaque(seqs_before);
    if (seqs_before + 1u == uint32_t(a.B)) {
      st_agent(a.gdone, 0u);
      st_agent(a.gtag, tag);
    }
  }
  // ---- the guess rows of the merger waves, now that the tile's bonus work is done
  if (guesses && w >= 2) {
    int turn = 0;
    for (int r = tile; r < KG; r += nT, ++turn) {
      if ((turn & 1) != w - 2 || (r < K && !guess_rows)) continue;
      merge_guess_row<4>(a, sh, b, tag, long_bound, r, mhi, mlo, r == mrow);
      TRACE_AT(10, 64 * w);
    }
  }
  TRACE(9);
}

// ---------------------------------------------------------------------------------------------
// The streaming form. When a batch has more tiles than the device runs at once, the workgroups go
// through it in waves, and a tile that waits for its sequence's decision holds a slot that a tile
// not yet started could stream in: the waits add up over the waves. So the work is cut where a
// tile would wait, into two grids whose workgroups never wait for ones that have not arrived:
//   verify_kernel<SPLIT>  every tile: every row read once, statistics and guesses published; no
//                         counter, no decision (its rows are issued all at once)
//   resid_kernel          G workgroups per sequence, each over a run of consecutive tiles: the
//                         statistics merged and the accept decisions taken (every workgroup of the
//                         sequence takes the same ones, from the same words in the same order), the
//                         run's residual masses published (the tile's two residual rows read
//                         again, 2 of the 2K+1 rows, the next tile's in flight), a share of the
//                         guesses merged; the last workgroup of the sequence to arrive scans the
//                         masses and draws the bonus
// Tiles, merge orders, mass sums and the search are those of the one-launch form, so both forms give
// the same bits.
// ---------------------------------------------------------------------------------------------
template <class ET, int NV, bool AL>
__global__ __launch_bounds__(kThreads, kResidWgPerCu) void resid_kernel(VerifyArgs a) {
  using T = typename ET::T;
  using LY = Lay<ET, NV>;
  constexpr int E = LY::E;
  __shared__ SharedT<1> sh;  // (no candidate regions: the first grid selected the guesses)

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int K = a.K, V = a.V, nT = a.T, sF = a.sF, Tc = a.Tcap, G = a.groups;
  const float cc = a.c2;
  const int b = int(blockIdx.x) / G, g = int(blockIdx.x) - b * G;
  const int run = (nT + G - 1) / G;  // tiles per workgroup
  const int q0 = min(g * run, nT), q1 = min(nT, q0 + run);
  const T* draft = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride;
  const T* target = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride;
  auto row_ptr = [&](int r) -> const T* { return (r < K) ? draft + int64_t(r) * V : target + int64_t(r - K) * V; };
  uint32_t* ctr = a.seqctl + int64_t(b) * kPlanSeqCtlWords;
  uint64_t* chunk = a.chunk + int64_t(b) * Tc * 2;
  // the call's tag: the first grid left the last call's tag in place; the last sequence to finish
  // here advances it, once every workgroup of this grid has read it
  const uint32_t tag_ld = ld_agent(a.gtag);
  const uint32_t tag = (tag_ld + 1u == 0u) ? 1u : tag_ld + 1u;
  const int long_bound = a.wait_polls * 8 + 4096;

  // ---- the decision (the sequence's inputs, the logits the accept tests read, every statistic)
  const int x_v = (t < K) ? a.x[b * K + t] : -1;
  const float u_v = (t <= K) ? a.u[b * (K + 1) + t] : 0.f;
  const int sv_v = (t < K * sF) ? a.sset[int64_t(b) * K * sF + t] : -1;
  const int xg = (t < 2 * K) ? a.x[b * K + (t < K ? t : t - K)] : -1;
  const bool g_ok = t < 2 * K && unsigned(xg) < unsigned(V);
  const float zg = ET::one(row_ptr(t < 2 * K ? t : 0), g_ok ? xg : 0);
  const bool s_ok = t < K * sF && unsigned(sv_v) < unsigned(V);
  const float zs = ET::one(row_ptr(t < K * sF ? t / sF : 0), s_ok ? sv_v : 0);
  if (t < K) {
    sh.xe[t] = x_v;
    sh.C[t] = a.Cpos[t];
  }
  if (t <= K) {
    sh.F[t] = a.topfF[t];
    sh.u[t] = u_v;
  }
  if (t == K) sh.xe[K] = -1;
  if (t < K * sF) {
    sh.sv[t] = sv_v;
    sh.zs[t] = s_ok ? zs : 0.f;
  }
  if (t < 2 * K) sh.zg[t] = g_ok ? zg : 0.f;
  __syncthreads();
  // every wave merges its share of the rows (the same arithmetic per row as the one-launch form's
  // wave 0), then wave 0 decides
  const bool miss = __syncthreads_or(merge_stats_part(a, sh, b, tag, long_bound, w, kWaves) ? 1 : 0) != 0;
  if (w == 0) decide_wave0(a, sh, b, tag, long_bound, true, false, g == 0, NoStage{}, true, miss);
  __syncthreads();
  const int k = min(max(__builtin_amdgcn_readfirstlane(sh.k), 0), K);
  const int nset = (k < K) ? min(max(sh.nset, 0), kMaxF) : 0;
  const float uK = sh.u[K];

  // ---- the run's residual masses: target row k, draft row k (none when every draft passed: the
  // target row's address again, a cache hit); the next tile's rows load while one is summed
  const T* prow = target + int64_t(k) * V;
  const T* qrow = (k < K) ? draft + int64_t(k) * V : prow;
  auto lane_base = [&](int q) { return q * LY::TILE + w * LY::WTOK + lane * LY::VEC; };
  auto load2 = [&](int q, Raw<NV>& rp, Raw<NV>& rq) __attribute__((always_inline)) {
    load_row<ET, NV, AL>(prow, lane_base(q), V, rp);
    load_row<ET, NV, AL>(qrow, lane_base(q), V, rq);
  };
  auto values = [&](int q, const Raw<NV>& rp, const Raw<NV>& rq, float (&rv)[E]) __attribute__((always_inline)) {
    const int blq = lane_base(q);
    const bool tq = AL && ((q + 1) * LY::TILE > V);
    float zp[E], zq[E];
    unpack_row<ET, NV>(rp, blq, V, tq, zp);
    unpack_row<ET, NV>(rq, blq, V, tq, zq);
    residual_values<ET, NV>(zp, zq, k < K, blq, V, cc, sh.Lp, sh.Lq, sh.w_out, sh.w_in, sh.myset, nset, rv);
  };
  auto mass = [&](int q, const Raw<NV>& rp, const Raw<NV>& rq) __attribute__((always_inline)) {
    float rv[E];
    values(q, rp, rq, rv);
    const float total = tile_mass<E>(rv, sh.wt);
    if (t == 0) st_agent(chunk + 2 * q + 1, tagged(tag, __float_as_uint(total)));
  };
  // kRunGroup tiles at a time: every read of the group is issued, then the tiles are summed in
  // order (a tile index past the run reads the run's last tile again: in bounds, unused, so no
  // branch surrounds a read); nothing is carried from one group to the next, so no buffer has to be
  // copied while its reads are in flight
  constexpr int kRunGroup = 4;
  for (int qg = q0; qg < q1; qg += kRunGroup) {
    Raw<NV> rp[kRunGroup], rq[kRunGroup];
#pragma unroll
    for (int i = 0; i < kRunGroup; ++i) load2(min(qg + i, q1 - 1), rp[i], rq[i]);
#pragma unroll
    for (int i = 0; i < kRunGroup; ++i)
      if (qg + i < q1) mass(qg + i, rp[i], rq[i]);
  }
  // a share of the guess merge: guess rows g, g + G, ...
  if (a.topfFmax > 0 || a.lastF > 0) merge_guesses_seq<8>(a, sh, b, tag, long_bound, g, G);
  __syncthreads();
  uint32_t seqs_before = 0;  // (as in verify_kernel: the sequence counted in once all have arrived)
  if (t == 0) {
    const bool last = add_agent(ctr, 1u) + 1u == uint32_t(G);
    if (last) {
      st_agent(ctr, 0u);  // every workgroup has counted itself in: back to zero
      seqs_before = add_agent(a.gdone, 1u);
    }
    sh.role = last ? 1 : 0;
  }
  __syncthreads();
  if (!sh.role) return;

  // ---- the last workgroup of the sequence: every mass has been published (the polls only wait for
  // the words to be seen), the scan, the draw
  if (t < 64) {
    bool ok = false;
    for (int n = 0;; ++n) {
      bool in = true;
      for (int c = lane; c < nT; c += 64) {
        const uint64_t mw = ld_agent(chunk + 2 * c + 1);
        in = in && tag_of(mw) == tag;
        sh.res[c] = val_f(mw);
      }
      if (__all(in)) {
        ok = true;
        break;
      }
      if (n >= long_bound) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok && lane == 0) atomicOr(a.flags, kFlagTimeout);
  }
  __syncthreads();
  if (t < 64) scan_masses(sh, nT, uK);
  __syncthreads();
  int tok;
  float rm;
  if (sh.fallback) {
    tok = fallback_draw<ET, NV, AL>(prow, V, nT, cc, sh.Lp, uK, sh);
    rm = 0.f;
  } else {  // the tile whose range holds u_K R: its two rows read again
    const int cs = sh.cstar;
    Raw<NV> rp, rq;
    load2(cs, rp, rq);
    float rv[E], pre[E];
    values(cs, rp, rq, rv);
    tile_prefix<ET, NV>(rv, sh.wt, pre);
    tok = tile_search<ET, NV>(rv, pre, lane_base(cs), sh.base, sh.target, sh.clamp != 0, sh);
    rm = (k < K) ? sh.R : 1.f;
  }
  if (t == 0) {
    a.bonus_out[b] = tok;
    if (a.rmass_out) a.rmass_out[b] = rm;
    opaque(seqs_before);
    if (seqs_before + 1u == uint32_t(a.B)) {  // the last sequence of the call
      st_agent(a.gdone, 0u);
      st_agent(a.gtag, tag);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// launch: one grid of every (sequence, tile); no workgroup needs another to be resident
// ---------------------------------------------------------------------------------------------
static_assert(kThreads == kVerifyThreads, "the host plan sizes tiles for this workgroup");

template <class ET, int KM, int NV, bool AL>
static hipError_t launch_v(const VerifyArgs& a, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(a.B) * a.T));
  if (!a.split) {
    hipLaunchKernelGGL((verify_kernel<ET, KM, NV, AL, false>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((verify_kernel<ET, KM, NV, AL, true>), grid, dim3(kThreads), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((resid_kernel<ET, NV, AL>), dim3(unsigned(int64_t(a.B) * a.groups)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <class ET>
static hipError_t launch_verify_e(const VerifyArgs& a, const VerifyPlan& p, hipStream_t st) {
  if (!p.AL) {
    if (p.KM == 4) return launch_v<ET, 4, 1, false>(a, st);
    if (p.KM == 8) return launch_v<ET, 8, 1, false>(a, st);
    return launch_v<ET, 16, 1, false>(a, st);
  }
  if (p.KM == 4) return p.NV == 2 ? launch_v<ET, 4, 2, true>(a, st) : launch_v<ET, 4, 1, true>(a, st);
  if (p.KM == 8) return p.NV == 2 ? launch_v<ET, 8, 2, true>(a, st) : launch_v<ET, 8, 1, true>(a, st);
  return launch_v<ET, 16, 1, true>(a, st);
}

hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& p, bool bf16, hipStream_t st) {
  return bf16 ? launch_verify_e<BF16T>(a, p, st) : launch_verify_e<F32T>(a, p, st);
}

// ---------------------------------------------------------------------------------------------
// The allocation-free variant's workspace: one array per device, part of the code object (zero when
// it loads). Host code never uses the name as an address: the device address comes from
// hipGetSymbolAddress, once per device, and is what the kernels are given.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kScratchDevices];  // per device: the array's device address, once looked up

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}
}  // namespace

hipError_t noalloc_scratch(void** out, size_t ctrl_bytes, hipStream_t st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) % 256) != 0) return hipErrorInvalidValue;
    // the control words (call tag, sequence count, arrival counters) must start at zero: cleared
    // ahead of the first launch on this device (a fill kernel, not a memset, so that a capturing
    // caller records no memset node)
    const int64_t n = int64_t(std::min(ctrl_bytes, size_t(SSD_NOALLOC_SCRATCH_BYTES)) / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, st, static_cast<uint32_t*>(ptr), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ssd
