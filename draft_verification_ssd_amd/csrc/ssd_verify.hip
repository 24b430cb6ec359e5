// Batched lossless draft verification on gfx950: one launch per round of sequences.
//
// Work unit: one 256-thread workgroup per (sequence b, tile of kTileTok tokens). A tile covers the
// same token range of all 2K+1 rows of its sequence (K draft rows, K+1 target rows), so the T
// tiles of a sequence together stream every logit of it exactly once. Inside a tile, wave w owns
// tokens [w * 64 kE, (w + 1) * 64 kE); lane l holds kE of them in 16-byte chunks j: chunk j of lane
// l starts at token j * 64 VEC + l VEC of the wave's range (VEC tokens per 16 bytes), so every
// load instruction of a wave reads 1 KB of contiguous memory.
//
//  phase 1   Each lane loads its chunks of every row of a load group at once, forms max and
//            sum 2^(z c - max) per row with c = log2(e)/T, and merges them over 16-lane groups with
//            DPP. Partials go out with write-through (agent-coherent) stores; once they have
//            completed, one atomic per tile counts the tile in.
//  top-F     While it waits for the decision, a tile re-reads its draft rows from cache and keeps
//            the candidates of each wave that pass a threshold every top-F token of the wave
//            passes (from the same DPP maxima), selects the tile's best F per row and publishes them.
//  decide    The tile that arrives last merges the row statistics in one fixed order, gathers the
//            logits at the draft tokens, takes the accept decisions and k, writes k and the accept
//            probabilities, and publishes a small decision record of words tagged with the call,
//            which the other tiles poll.
//  residual  Every tile sums r = max(p_k - q'_k, 0) (or p_K when all drafts pass) over its token
//            range, re-reading the two rows from cache, keeps r and its prefix sums in registers
//            and publishes the tagged sum.
//  bonus     Every tile scans the T sums in the same order (the same bits everywhere); the tile
//            whose range holds u_K R finds the token in its registers. Tiles 0..K-1 merge the
//            top-F guesses of draft row = tile while the sums come in.
//
// Code size matters here: the hot loops stay compact (only the all-vector load mode is unrolled
// over rows; tail tiles and unaligned rows take rolled loops) so they fit the instruction cache.
//
// The waits are bounded spins (a timeout is flagged, never hung). They need every tile of a
// sequence resident at once, so one launch covers only as many sequences as the device keeps
// resident; the host issues one launch per round of sequences.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_plan.hpp"

namespace ssd {

constexpr int kE = 16;                   // tokens per lane per row
constexpr int kTileTok = kThreads * kE;  // tokens per tile
static_assert(kTileTok == kPlanTile, "host plan and kernel disagree on the tile size");
constexpr int kMaxVT = (kMaxV + kTileTok - 1) / kTileTok;  // tiles of the longest row
constexpr int kMaxR2 = 2 * kMaxK + 1;
constexpr int kGroupsPerBlock = kThreads / 16;
constexpr int kCandW = 40;  // filtered top-F candidates kept per draft row per wave
constexpr int kCandSel = (kWaves * kCandW + 63) / 64;  // candidates per lane at selection
static_assert(kCandW >= kMaxF + 1, "a wave region must hold an exact top-(F+1)");

// Per-sequence control words (64 x uint32): the phase-1 arrival counter, and the tag of the
// sequence's last call. A call's tag is the last tag + 1 (never 0, the value of a zero-filled
// workspace), so it advances on every launch, graph replays included, with no host state.
constexpr int kCtlArrive = 0, kCtlTag = 16;
// Per-sequence decision record: 64-bit words (call tag << 32 | value), each written once per
// call, so a reader knows a word is current when its tag matches the call's.
constexpr int kDecK = 0, kDecLp = 1, kDecLq = 2, kDecWout = 3, kDecWin = 4, kDecNset = 5,
              kDecSet = 6, kDecWords = kDecSet + kMaxF;
static_assert(kDecWords <= 32, "decision record exceeds its 256 bytes");

// token layout of one lane's kE tokens of a row
template <class ET>
struct Lay {
  static constexpr int VEC = 16 / int(sizeof(typename ET::T));  // tokens per 16-byte chunk
  static constexpr int NV = kE / VEC;                           // chunks per lane
  static constexpr int WTOK = 64 * kE;                          // tokens per wave
  static constexpr int CTOK = 64 * VEC;                         // tokens per chunk across a wave
  // element q of a lane whose first token is bl
  __device__ static __forceinline__ int tok(int bl, int q) { return bl + (q / VEC) * CTOK + (q % VEC); }
  // element of token x in the lane whose first token is bl, or -1
  __device__ static __forceinline__ int elem(int bl, int x) {
    const int d = x - bl;
    if (d < 0) return -1;
    const int j = d / CTOK, rem = d - j * CTOK;
    return (j < NV && rem < VEC) ? j * VEC + rem : -1;
  }
};

template <class ET>
struct RowRaw {
  uint4 w[Lay<ET>::NV];
};

template <class ET>
__device__ __forceinline__ void row_load_vec(const typename ET::T* row, int bl, RowRaw<ET>& r) {
#pragma unroll
  for (int j = 0; j < Lay<ET>::NV; ++j) r.w[j] = load16(row + bl + j * Lay<ET>::CTOK);
}

// one 16-byte chunk element by element; positions at or past V read as -inf. Every element is
// loaded (from a clamped index) and masked afterwards, so no load waits behind a branch.
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

template <class ET>
__device__ __forceinline__ void row_load_scalar(const typename ET::T* row, int bl, int V, RowRaw<ET>& r) {
#pragma unroll
  for (int j = 0; j < Lay<ET>::NV; ++j) r.w[j] = chunk_scalar<ET>(row, bl + j * Lay<ET>::CTOK, V);
}

template <class ET>
__device__ __forceinline__ void row_unpack(const RowRaw<ET>& r, float (&z)[kE]) {
#pragma unroll
  for (int j = 0; j < Lay<ET>::NV; ++j) ET::unpack(r.w[j], z + j * Lay<ET>::VEC);
}

// Rows whose length is a whole number of chunks (16-byte aligned rows): a chunk lies wholly
// inside or wholly past the row. The load reads a clamped, valid chunk; mask_tail then turns the
// chunks past V into -inf once they are unpacked (so no second copy of the words stays live).
template <class ET>
__device__ __forceinline__ void row_load_clamped(const typename ET::T* row, int bl, int V, RowRaw<ET>& r) {
#pragma unroll
  for (int j = 0; j < Lay<ET>::NV; ++j)
    r.w[j] = load16(row + min(bl + j * Lay<ET>::CTOK, V - Lay<ET>::VEC));
}
template <class ET>
__device__ __forceinline__ void mask_tail(float (&z)[kE], int bl, int V) {
#pragma unroll
  for (int j = 0; j < Lay<ET>::NV; ++j) {
    const bool in = bl + j * Lay<ET>::CTOK < V;
#pragma unroll
    for (int e = 0; e < Lay<ET>::VEC; ++e) z[j * Lay<ET>::VEC + e] = in ? z[j * Lay<ET>::VEC + e] : -INFINITY;
  }
}

// Load modes, chosen per tile: 0 every chunk whole (vector loads), 1 aligned rows with chunks past
// V (clamped vector loads; mask_tail after unpacking), 2 rows not 16-byte aligned (element
// loads, masked as they load).
template <class ET, int MODE>
__device__ __forceinline__ void row_load_m(const typename ET::T* row, int bl, int V, RowRaw<ET>& r) {
  if (MODE == 0)
    row_load_vec<ET>(row, bl, r);
  else if (MODE == 1)
    row_load_clamped<ET>(row, bl, V, r);
  else
    row_load_scalar<ET>(row, bl, V, r);
}
// row load and unpack with a runtime mode (the residual pass)
template <class ET>
__device__ __forceinline__ void row_fetch(const typename ET::T* row, int bl, int V, int mode, float (&z)[kE]) {
  RowRaw<ET> r;
  if (mode == 2)
    row_load_scalar<ET>(row, bl, V, r);
  else if (mode == 1)
    row_load_clamped<ET>(row, bl, V, r);
  else
    row_load_vec<ET>(row, bl, r);
  row_unpack<ET>(r, z);
  if (mode == 1) mask_tail<ET>(z, bl, V);
}


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

#ifdef SSD_TRACE
// phase timestamps per workgroup (100 MHz clock), for performance analysis builds only
#define TRACE(i)                                                                      \
  do {                                                                                \
    if (threadIdx.x == 0 && a.trace) a.trace[blockIdx.x * 32 + (i)] = wall_clock64(); \
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
  uint64_t spare[kWaves][64];  // where the compaction's failing tokens are written
  int leader;
  // decision (last tile to arrive)
  float L[kMaxR2];
  float zg[2 * kMaxK];      // logits at the draft tokens: draft rows 0..K-1, then target rows
  float zs[kMaxK * kMaxF];  // draft logits at the set entries
  int set[kMaxK * kMaxF];   // de-duplicated in-range set entries, -1 elsewhere
  // the decision record, as every tile uses it
  int k, nset;
  float Lp, Lq, w_out, w_in;
  int myset[kMaxF];
  // residual and bonus
  float wt[kWaves];
  float res[kMaxVT];
  int cstar, clamp, fallback, first, lastp;
  float base, target, R;
  uint64_t wtop[kWaves][kMaxF];
};

// Residual values of a lane's kE tokens of one tile and their prefix sums in token order, relative
// to the tile start: r = max(p - q w / N, 0) with w = C on the Saguaro set (w_in = C / N,
// w_out = 1 / N), or r = p when qrow is null. Returns the tile total (every lane, same bits).
// Token order inside a tile is (wave, chunk, lane, element); the sums follow it: element sums per
// chunk, a DPP scan over lanes per chunk, chunk bases per wave, wave bases per tile.
template <class ET>
__device__ __forceinline__ float tile_residual(const typename ET::T* prow, const typename ET::T* qrow,
                                               int bl, int V, int mode, float c, float Lp, float Lq,
                                               float w_out, float w_in, const int* set, int n_set,
                                               float* wt_sh, float (&rv)[kE], float (&pre)[kE]) {
  using LY = Lay<ET>;
  float zp[kE], zq[kE];
  row_fetch<ET>(prow, bl, V, mode, zp);
  if (qrow) row_fetch<ET>(qrow, bl, V, mode, zq);
  uint32_t in_set = 0;  // bit q: element q is a Saguaro-set token
  for (int f = 0; f < n_set; ++f) {
    const int q = LY::elem(bl, set[f]);
    if (q >= 0) in_set |= 1u << q;
  }
#pragma unroll
  for (int q = 0; q < kE; ++q) {
    const float pv = ex2(fmaf(zp[q], c, -Lp));
    if (qrow) {
      const float w = ((in_set >> q) & 1u) ? w_in : w_out;
      rv[q] = fmaxf(pv - ex2(fmaf(zq[q], c, -Lq)) * w, 0.f);
    } else {
      rv[q] = pv;
    }
    if (LY::tok(bl, q) >= V) rv[q] = 0.f;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float pin[LY::NV], cb[LY::NV + 1];
#pragma unroll
  for (int j = 0; j < LY::NV; ++j) {
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < LY::VEC; ++e) sum += rv[j * LY::VEC + e];
    pin[j] = wave_incl_scan(sum);
  }
  cb[0] = 0.f;
#pragma unroll
  for (int j = 0; j < LY::NV; ++j) cb[j + 1] = cb[j] + readlane_f(pin[j], 63);
  __syncthreads();
  if (lane == 0) wt_sh[w] = cb[LY::NV];
  __syncthreads();
  float wb = 0.f, total = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i == w) wb = total;
    total += wt_sh[i];
  }
#pragma unroll
  for (int j = 0; j < LY::NV; ++j) {
    float p = wb + cb[j] + wave_shift_up1(pin[j]);
#pragma unroll
    for (int e = 0; e < LY::VEC; ++e) {
      p += rv[j * LY::VEC + e];
      pre[j * LY::VEC + e] = p;
    }
  }
  return total;
}

template <class ET, int FM, int G>
__global__ __launch_bounds__(kThreads, 2) void verify_fused_kernel(VerifyArgs a) {
  using T = typename ET::T;
  using LY = Lay<ET>;
  __shared__ Shared sh;

  const int t = threadIdx.x, lane = t & 63, grp = t >> 4, w = t >> 6;
  const int K = a.K, V = a.V, R2 = 2 * K + 1, nT = a.T, sF = a.sF;
  const float cc = a.c2;
  const bool aligned = a.aligned != 0;
  const int tile = blockIdx.x % nT;
  const int b = a.b0 + int(blockIdx.x) / nT;
  const int c0 = tile * kTileTok;
  const int wb0 = c0 + w * LY::WTOK;     // first token of this wave
  const int bl = wb0 + lane * LY::VEC;   // first token of this lane
  const T* draft = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride;
  const T* target = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride;
  auto row_ptr = [&](int r) -> const T* {
    return (r < K) ? draft + int64_t(r) * V : target + int64_t(r - K) * V;
  };
  uint32_t* ctl = a.ctl + int64_t(b) * 64;
  uint64_t* dec = a.dec + int64_t(b) * 32;
  const uint32_t tag_ld = ld_agent(ctl + kCtlTag);  // read before this tile arrives (see below)

  // per-sequence inputs, loaded before the rows and staged to LDS after phase 1
  const int x_v = (t < K) ? a.x[b * K + t] : -1;
  const float u_v = (t <= K) ? a.u[b * (K + 1) + t] : 0.f;
  int sv_v = -1;
  if (t < K * sF) sv_v = a.sset[int64_t(b) * K * sF + t];
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the row loads

  // load mode of this tile (uniform): whole vector chunks everywhere but in a row's last tile
  const int mode = !aligned ? 2 : (c0 + kTileTok <= V ? 0 : 1);

  // ---- phase 1: row statistics of this tile
  TRACE(0);
  // max and sum 2^(z c - max) of one row over the lane's tokens, merged over 16-lane groups
  auto row_stats = [&](const float (&z)[kE], int r) __attribute__((always_inline)) {
    float m = z[0];
#pragma unroll
    for (int q = 1; q < kE; ++q) m = fmaxf(m, z[q]);
    float s = 0.f;
    const float mc = m * cc;
    if (m > -INFINITY) {
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int q = 0; q < kE; q += 4) {
        s0 += ex2(fmaf(z[q], cc, -mc));
        s1 += ex2(fmaf(z[q + 1], cc, -mc));
        s2 += ex2(fmaf(z[q + 2], cc, -mc));
        s3 += ex2(fmaf(z[q + 3], cc, -mc));
      }
      s = (s0 + s1) + (s2 + s3);
    }
    const float M = row16_max(m);
    const float Mc = M * cc;
    const float S = row16_sum((s > 0.f) ? s * ex2(mc - Mc) : 0.f);
    if ((t & 15) == 0) sh.g16[r][grp] = make_float2(Mc, S);
  };
  if (mode != 2) {
    // aligned rows: every row of a group in flight at once, consumed in load order; chunks past V
    // (a row's last tile) are loaded from a clamped address and masked
    for (int g0 = 0; g0 < R2; g0 += G) {
      RowRaw<ET> raw[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        row_load_clamped<ET>(row_ptr(min(g0 + j, R2 - 1)), bl, V, raw[j]);
        __builtin_amdgcn_sched_barrier(0);  // issue in row order
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float z[kE];
        row_unpack<ET>(raw[j], z);
        if (mode == 1) mask_tail<ET>(z, bl, V);
        if (g0 + j < R2) row_stats(z, g0 + j);
        if (j == 0 && g0 == 0) TRACE(8);
      }
    }
  } else {
    // rows not 16-byte aligned: one row at a time
#pragma unroll 1
    for (int r = 0; r < R2; ++r) {
      float z[kE];
      row_fetch<ET>(row_ptr(r), bl, V, mode, z);
      row_stats(z, r);
    }
  }
  TRACE(9);
  if (t < K) {
    sh.xe[t] = x_v;
    sh.F[t] = a.topfF[t];
  }
  if (t <= K) sh.u[t] = u_v;
  if (t < K * sF) sh.sv[t] = sv_v;
  __syncthreads();

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
  wait_vmem();
  __syncthreads();
  if (t == 0) sh.leader = (atomicAdd(ctl + kCtlArrive, 1u) == unsigned(nT - 1));
  // Every tile read the last tag before its arrival (its loads completed before the atomic), so
  // the leader may advance it now.
  const uint32_t tag = (tag_ld + 1u == 0u) ? 1u : tag_ld + 1u;
  __syncthreads();
  TRACE(1);

  // ---- top-F guesses, per tile: each draft row's candidates are filtered into per-wave LDS regions,
  // the tile's best F per row go to the workspace, then a word tagged with the call says they are
  // in. Run while the tile would otherwise wait (non-leaders before the decision record, the
  // leader after publishing its residual mass), re-reading the draft rows from cache.
  const int Fp = a.topfFmax + 1;  // candidates kept per wave: one more than the guesses
  // Top-F candidates of draft row r of this tile into this wave's LDS region.
  auto row_filter = [&](const float (&z)[kE], int r) __attribute__((always_inline)) {
    float m = z[0];
#pragma unroll
    for (int q = 1; q < kE; ++q) m = fmaxf(m, z[q]);
    const float m2 = fmaxf(m, dpp_f<kDppXor1>(m));
    const float m4 = fmaxf(m2, dpp_f<kDppXor2>(m2));
    const float m8 = fmaxf(m4, dpp_f<kDppHalfMirror>(m4));
    const float M = fmaxf(m8, dpp_f<kDppMirror>(m8));
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
        const float q4 = (m4 > -kInf) ? m4 : kInf;
        g = fminf(q4, dpp_f<kDppHalfMirror>(q4));
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
      // Compaction without a scalar round trip per token: per-lane counts, a DPP scan for each
      // lane's first slot, then one LDS write per token, the tokens that fail going to a
      // per-lane spare slot. An entry holds the raw float bits and ~token.
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < kE; ++q) cnt += (z[q] >= thr) ? 1 : 0;
      const int incl = wave_incl_scan_i(cnt);
      int total = __builtin_amdgcn_readlane(incl, 63);
      uint64_t* region = sh.cand[r][w];
      if (total <= kCandW) {
        int slot = incl - cnt;
        uint64_t* spare = &sh.spare[w][lane];
#pragma unroll
        for (int q = 0; q < kE; ++q) {
          const bool pass = z[q] >= thr;
          uint64_t* dst = pass ? region + slot : spare;
          *dst = (uint64_t(__float_as_uint(z[q])) << 32) | uint64_t(~uint32_t(LY::tok(bl, q)));
          slot += pass ? 1 : 0;
        }
      } else {  // too many pass (ties, a short last tile): the wave's exact top Fp from registers
        uint32_t ph = 0xFFFFFFFFu, pl = 0xFFFFFFFFu;
#pragma unroll 1
        for (int f = 0; f < Fp; ++f) {
          uint32_t bh = 0, blo = 0;
#pragma unroll
          for (int q = 0; q < kE; ++q) {
            const bool ok = z[q] > -INFINITY;
            const uint32_t kh = ok ? ordered_key(z[q]) : 0u;
            const uint32_t kl = ok ? ~uint32_t(LY::tok(bl, q)) : 0u;
            if (key_gt(ph, pl, kh, kl) && key_gt(kh, kl, bh, blo)) {
              bh = kh;
              blo = kl;
            }
          }
          wave_max_key(bh, blo);
          if (lane == 0)  // raw float bits, as the compaction writes them (0 = none)
            region[f] = bh ? (uint64_t(__float_as_uint(key_to_float(bh))) << 32) | blo : 0ull;
          ph = bh;
          pl = blo;
        }
        total = Fp;
      }
      if (lane == 0) sh.ncw[r][w] = total;
  };
  auto topf_tile = [&]() __attribute__((always_inline)) {
    if (mode != 2) {
      // four draft rows in flight at once, then filtered one after another
      constexpr int kQ = 4;
#pragma unroll 1
      for (int r0 = 0; r0 < K; r0 += kQ) {
        RowRaw<ET> raw[kQ];
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
          row_load_clamped<ET>(row_ptr(min(r0 + j, K - 1)), bl, V, raw[j]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
          if (r0 + j >= K) continue;
          float z[kE];
          row_unpack<ET>(raw[j], z);
          if (mode == 1) mask_tail<ET>(z, bl, V);
          if (r0 + j == 0) TRACE(16);
          row_filter(z, r0 + j);
          if (r0 + j == 0) TRACE(17);
        }
      }
    } else {
#pragma unroll 1
      for (int r = 0; r < K; ++r) {
        float z[kE];
        row_fetch<ET>(row_ptr(r), bl, V, mode, z);
        row_filter(z, r);
      }
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
          const uint64_t e = (ww < kWaves && sl < sh.ncw[r][ww]) ? sh.cand[r][ww][sl] : 0ull;
          key[i] = uint32_t(e) ? (uint64_t(ordered_key(__uint_as_float(uint32_t(e >> 32)))) << 32) |
                                     uint32_t(e)
                               : 0ull;
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
    TRACE(19);
    if (t < K * a.topfFmax) {
      const int r = t / a.topfFmax, f = t - r * a.topfFmax;
      if (f < sh.F[r])
        st_agent(a.cand + ((int64_t(b) * K + r) * nT + tile) * a.topfFmax + f, sh.best[r][f]);
    }
    wait_vmem();
    __syncthreads();
    if (t == 0) st_agent(a.cready + int64_t(b) * nT + tile, tagged(tag, 1u));
  };
  if (FM > 0 && !sh.leader) topf_tile();
  TRACE(10);

  // ---- decide: the last tile to arrive merges the statistics and publishes the decision
  if (sh.leader) {
    if (t == 0) {  // every tile has arrived: ready for the next call
      st_agent(ctl + kCtlArrive, 0u);
      st_agent(ctl + kCtlTag, tag);
    }
    // logits at the draft tokens (draft and target rows 0..K-1) and at the Saguaro-set tokens,
    // gathered from the rows; issued first, so they overlap the statistics loads
    float zg_v = 0.f, zs_v = 0.f;
    int set_v = -1;
    if (t < 2 * K) {
      const int xr = sh.xe[t < K ? t : t - K];
      if (unsigned(xr) < unsigned(V)) zg_v = ET::one(row_ptr(t), xr);
    }
    if (t < K * sF) {
      set_v = (unsigned(sh.sv[t]) < unsigned(V)) ? sh.sv[t] : -1;
      if (set_v >= 0) zs_v = ET::one(row_ptr(t / sF), set_v);
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

  // ---- residual mass of this tile (values and prefix sums stay in registers), published
  float rv[kE], pre[kE];
  const float total = tile_residual<ET>(prow, qrow, bl, V, mode, cc, Lp, Lq, w_out, w_in, sh.myset,
                                        nset, sh.wt, rv, pre);
  if (t == 0) st_agent(a.res + int64_t(b) * nT + tile, tagged(tag, __float_as_uint(total)));
  TRACE(4);
  if (FM > 0 && sh.leader) topf_tile();

  // ---- top-F guesses of draft rows tile, tile + T, ... while the other tiles finish: each
  // wave takes its own top F of the tiles' candidates, then wave 0 merges the four lists. Keys
  // are unique (a token lives in one tile), so round f picks the largest key below round f-1's.
  if (FM > 0 && tile < K) {  // every tile's candidates must be in
    const int per = (nT + kThreads - 1) / kThreads;
    const int q0 = min(t * per, nT), q1 = min(nT, q0 + per);
    const uint64_t* cr = a.cready + int64_t(b) * nT;
    for (int spins = 0;; ++spins) {
      bool ok = true;
      for (int q = q0; q < q1; ++q) ok = ok && uint32_t(ld_agent(cr + q) >> 32) == tag;
      if (__all(ok)) break;
      if (spins > a.spin_limit) {
        if (lane == 0) atomicOr(a.flags, kFlagTimeout);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __syncthreads();
  }
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
    for (int q = 0; q < kE; ++q)
      if (rv[q] > 0.f) {
        const int tk = LY::tok(bl, q);
        lastp = max(lastp, tk);
        if (!sh.clamp && sh.base + pre[q] > sh.target) first = min(first, tk);
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
      const int blq = q * kTileTok + w * LY::WTOK + lane * LY::VEC;
      const int mq = !aligned ? 2 : ((q + 1) * kTileTok <= V ? 0 : 1);
      const float tot = tile_residual<ET>(prow, nullptr, blq, V, mq, cc, Lp, 0.f, 1.f, 1.f, sh.myset, 0,
                                          sh.wt, rv, pre);
      int first = INT_MAX, lp = -1;
#pragma unroll
      for (int e = 0; e < kE; ++e)
        if (rv[e] > 0.f) {
          const int tk = LY::tok(blq, e);
          lp = max(lp, tk);
          if (run + pre[e] > target_v) first = min(first, tk);
        }
      first = wave_min_i(first);
      lp = wave_max_i(lp);
      __syncthreads();
      if (t == 0) {
        sh.first = INT_MAX;
        sh.lastp = -1;
      }
      __syncthreads();
      if (lane == 0) {
        if (first != INT_MAX) atomicMin(&sh.first, first);
        if (lp >= 0) atomicMax(&sh.lastp, lp);
      }
      __syncthreads();
      if (sh.lastp >= 0) lastp = sh.lastp;
      if (sh.first != INT_MAX) found = sh.first;
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
template <class ET, int FM, int G>
static int capacity_blocks() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(verify_fused_kernel<ET, FM, G>), kThreads, 0) != hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

template <class ET, int FM, int G>
static hipError_t launch_fused(VerifyArgs a, hipStream_t st) {
  const int cap = capacity_blocks<ET, FM, G>();
  if (cap < a.T) return hipErrorInvalidConfiguration;
  const int per_round = cap / a.T;  // whole sequences whose tiles are all resident at once
  const int B = a.B;
  for (int b0 = 0; b0 < B; b0 += per_round) {
    const int nb = (B - b0 < per_round) ? (B - b0) : per_round;
    a.b0 = b0;
    hipLaunchKernelGGL((verify_fused_kernel<ET, FM, G>), dim3(unsigned(nb * a.T)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Rows per load group: bf16 9 (K <= 4 in one group, 8 VGPRs of payload per row and lane), fp32 5
// (16 VGPRs per row). Larger K runs several groups; a smaller K loads the last row again for the
// unused slots (cache hits) and skips their arithmetic.
template <class ET, int FM>
static hipError_t launch_g(const VerifyArgs& a, hipStream_t st) {
  return launch_fused<ET, FM, (sizeof(typename ET::T) == 2 ? 9 : 5)>(a, st);
}

template <class ET>
static hipError_t launch_verify_e(const VerifyArgs& a, hipStream_t st) {
  if (a.topfFmax == 0) return launch_g<ET, 0>(a, st);
  if (a.topfFmax <= 4) return launch_g<ET, 4>(a, st);
  if (a.topfFmax <= 8) return launch_g<ET, 8>(a, st);
  return launch_g<ET, 16>(a, st);
}

hipError_t launch_verify(const VerifyArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_verify_e<BF16T>(a, st) : launch_verify_e<F32T>(a, st);
}

}  // namespace ssd
