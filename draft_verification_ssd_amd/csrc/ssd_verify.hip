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
//            DPP; the draft rows' lanes that can hold a top-F token copy their chunks to LDS. The
//            tile's (max, sum) per row goes out as words tagged with the call, written through
//            to memory (agent-coherent stores).
//  top-F     While it waits for the decision, a tile selects its best F per draft row from those
//            copies (rows with too many candidate lanes are re-read from cache and filtered) and
//            publishes them as tagged words.
//  decide    The first tile past phase 1 claims the decision; it polls every tile's statistics,
//            merges them in one fixed order, gathers the logits at the draft tokens, takes the
//            accept decisions and k, writes k and the accept probabilities, and publishes a small
//            decision record of tagged words, which the other tiles poll.
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
constexpr int kAhead = 4;  // phase-1 rows in flight per lane
// Per draft row and wave, the top-F candidates live in an LDS region of kRegW 64-bit words:
// either the raw chunks of the wave's hot lanes (at most kHot of them, see hot_dump), or a list of
// (float bits << 32 | ~token) entries from the compaction filter.
constexpr int kRegW = 48;
constexpr int kSel = 8;  // candidates per lane at selection: two rounds of 64 per wave region
static_assert(kRegW >= kMaxF + 1, "a wave region must hold an exact top-(F+1)");
static_assert(kRegW <= 64, "a key-list region gives at most one entry per lane");
template <class ET>
constexpr int hot_slots() {
  return (kRegW * 8 / (kE * int(sizeof(typename ET::T)))) < 8 ? (kRegW * 8 / (kE * int(sizeof(typename ET::T))))
                                                               : 8;
}
static_assert(kSel % kWaves == 0 && 8 * kE <= 64 * (kSel / kWaves), "selection rounds must cover a region's dump");

// Per-sequence control words (64 x uint32): word kCtlTag holds the tag of the sequence's last
// call. A call's tag is the last tag + 1 (never 0, the value of a zero-filled workspace), so it
// advances on every launch, graph replays included, with no host state. Word kCtlLead holds the
// tag of the call whose deciding tile has claimed it.
constexpr int kCtlTag = 16, kCtlLead = 32;

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
#define TRACEV(i, v)                                                                  \
  do {                                                                                \
    if (threadIdx.x == 0 && a.trace) a.trace[blockIdx.x * 32 + (i)] = (v);            \
  } while (0)
#else
#define TRACEV(i, v) \
  do {               \
  } while (0)
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
  // top-F candidates per draft row and wave: nseg < 0 means -nseg hot lanes dumped their raw
  // chunks (lane ids in hl), nseg >= 0 that many key entries
  uint64_t reg[kMaxK][kWaves][kRegW];
  int nseg[kMaxK][kWaves];
  int hl[kMaxK][kWaves][8];
  uint32_t thr[kMaxK][kWaves];  // the dump's threshold key: smaller tokens are no candidates
  uint32_t fb[kWaves];  // draft rows the wave filters again after phase 1 (bit r)
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

// MB: workgroups per CU the register allocation is sized for. 2 fits the whole kernel in registers;
// 4 holds twice the sequences per launch at the cost of a few spilled registers, and is taken
// only when it needs fewer launches (rounds of resident sequences) than 2.
template <class ET, int FM, int G, int MB>
__global__ __launch_bounds__(kThreads, MB) void verify_fused_kernel(VerifyArgs a) {
  using T = typename ET::T;
  using LY = Lay<ET>;
  __shared__ Shared sh;

  const int t = threadIdx.x, lane = t & 63, grp = t >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, in a scalar register
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
  // This call's tag is one past the sequence's last. Every word a tile publishes carries it, so
  // the load below has returned before the tile publishes anything; the deciding tile stores the
  // new tag once it has seen every tile's statistics.
  const uint32_t tag_ld = ld_agent(ctl + kCtlTag);

  // per-sequence inputs, loaded before the rows and staged to LDS after phase 1
  const int x_v = (t < K) ? a.x[b * K + t] : -1;
  const float u_v = (t <= K) ? a.u[b * (K + 1) + t] : 0.f;
  int sv_v = -1;
  if (t < K * sF) sv_v = a.sset[int64_t(b) * K * sF + t];
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the row loads

  // load mode of this tile (uniform): whole vector chunks everywhere but in a row's last tile
  const int mode = !aligned ? 2 : (c0 + kTileTok <= V ? 0 : 1);
  const int Fp = a.topfFmax + 1;  // candidates kept per wave: one more than the guesses
  constexpr int kHot = hot_slots<ET>();
  if (FM > 0 && lane == 0) sh.fb[w] = (mode == 2) ? (1u << K) - 1u : 0u;

  // ---- phase 1: row statistics of this tile, and the top-F candidates of its draft rows
  TRACE(0);
  // max and sum 2^(z c - max) of one row over the lane's tokens, merged over 16-lane groups;
  // returns the lane's maximum
  // Returns the order key of the lane's maximum (0: no finite token).
  auto row_stats = [&](const float (&z)[kE], int r) __attribute__((always_inline)) -> uint32_t {
    float m = z[0];
#pragma unroll
    for (int q = 1; q < kE; ++q) m = fmaxf(m, z[q]);
    const float mc = m * cc;
    float s0 = ex2(fmaf(z[0], cc, -mc)), s1 = ex2(fmaf(z[1], cc, -mc));
    float s2 = ex2(fmaf(z[2], cc, -mc)), s3 = ex2(fmaf(z[3], cc, -mc));
#pragma unroll
    for (int q = 4; q < kE; q += 4) {
      s0 += ex2(fmaf(z[q], cc, -mc));
      s1 += ex2(fmaf(z[q + 1], cc, -mc));
      s2 += ex2(fmaf(z[q + 2], cc, -mc));
      s3 += ex2(fmaf(z[q + 3], cc, -mc));
    }
    const bool fin = m > -INFINITY;  // a lane with no finite token adds nothing (its terms are NaN)
    const uint32_t mk = fin ? ordered_key(m) : 0u;
    const uint32_t Mk = row16_max_u(mk);  // the row's maximum through its order key
    const float Mc = (Mk ? key_to_float(Mk) : -INFINITY) * cc;
    const float S = row16_sum(fin ? ((s0 + s1) + (s2 + s3)) * ex2(mc - Mc) : 0.f);
    if ((t & 15) == 0) sh.g16[r][grp] = make_float2(Mc, S);
    return mk;
  };
  // The Fp-th largest lane maximum of the wave, tied lanes counted: take the largest remaining
  // maximum and every lane that holds it until Fp lanes are taken. n = lanes taken; n < Fp when
  // fewer lanes hold a finite token. Wave-uniform.
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
  // Draft rows during phase 1, up to four at once (rows g0 + jb + i, i < 4, of the load group).
  // The threshold of a row is the Fp-th largest of its 16 quad maxima (quad = 4 lanes): lanes
  // 16 i + q gather quad q's maximum of row i, count the quads of their row with a larger one
  // (15 DPP row rotations), and the smallest maximum with fewer than Fp larger ones is it. At
  // least Fp quads, so at least Fp lanes, reach it, so the lanes that reach it ("hot") hold every
  // top-Fp token of the wave: a token of any other lane has Fp larger ones, the maxima of those
  // lanes. With fewer than Fp non-empty quads the threshold is 0 and every non-empty lane is hot.
  // Hot lanes copy their raw chunks into the row's region (chunks past V are dropped at
  // selection); a row with more hot lanes than slots is filtered again after phase 1.
  auto draft_batch = [&](const RowRaw<ET>* raw, const uint32_t* mk, int r0, int nb) __attribute__((always_inline)) {
    if (Fp > kHot) {  // more guesses than slots: every row of the batch is filtered later
      if (lane == 0)
        for (int i = 0; i < nb; ++i)
          if (r0 + i < K) sh.fb[w] |= 1u << (r0 + i);
      return;
    }
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nb) {
        const uint32_t g = uint32_t(__builtin_amdgcn_ds_bpermute((lane & 15) << 4, int(quad_max_u(mk[i]))));
        v = ((lane >> 4) == i && r0 + i < K) ? g : v;
      }
    }
    const uint32_t th = row16_min_u(row16_count_larger(v) < Fp ? v : 0xFFFFFFFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nb && r0 + i < K) {
        const int r = r0 + i;
        const uint32_t thr = uint32_t(__builtin_amdgcn_readlane(int(th), 16 * i));
        const bool hot = mk[i] >= thr && mk[i] != 0u;
        const uint64_t hm = __ballot(hot);
        const int n = __popcll(hm);
        if (n <= kHot) {
          if (hot) {
            const int sl = __builtin_amdgcn_mbcnt_hi(uint32_t(hm >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(hm), 0u));
            uint4* dst = reinterpret_cast<uint4*>(&sh.reg[r][w][0]) + sl * LY::NV;
#pragma unroll
            for (int j = 0; j < LY::NV; ++j) dst[j] = raw[i].w[j];
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
  if (mode != 2) {
    // aligned rows: every row of a group in flight at once, consumed in load order; chunks past V
    // (a row's last tile) are loaded from a clamped address and masked
    for (int g0 = 0; g0 < R2; g0 += G) {
      RowRaw<ET> raw[G];
      uint32_t mk[G];  // order keys of the lane maxima (0: no finite token)
      // kAhead rows in flight: the rest of the group is issued one row per row consumed, so the
      // requests of all workgroups interleave and every workgroup's first rows land early
#pragma unroll
      for (int j = 0; j < G && j < kAhead; ++j) {
        row_load_clamped<ET>(row_ptr(min(g0 + j, R2 - 1)), bl, V, raw[j]);
        __builtin_amdgcn_sched_barrier(0);  // issue in row order
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (j + kAhead < G) row_load_clamped<ET>(row_ptr(min(g0 + j + kAhead, R2 - 1)), bl, V, raw[j + kAhead]);
        __builtin_amdgcn_sched_barrier(0);
        float z[kE];
        row_unpack<ET>(raw[j], z);
        if (mode == 1) mask_tail<ET>(z, bl, V);
        mk[j] = 0u;
        if (g0 + j < R2) mk[j] = row_stats(z, g0 + j);
        // after every fourth row (and the group's last), the draft rows among the last four
        constexpr int kB = 4;
        if (FM > 0 && ((j % kB) == kB - 1 || j == G - 1)) {
          const int jb = j - (j % kB);
          if (g0 + jb < K) draft_batch(raw + jb, mk + jb, g0 + jb, j - jb + 1);
        }
      }
    }
  } else {
    // rows not 16-byte aligned: one row at a time (their top-F filter runs after phase 1)
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
  const uint32_t tag = (tag_ld + 1u == 0u) ? 1u : tag_ld + 1u;
  __syncthreads();

  // ---- publish the tile's partials: max and sum of each row, one tagged word each
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
    uint64_t* st = a.stats + ((int64_t(b) * R2 + t) * nT + tile) * 2;
    st_agent(st, tagged(tag, __float_as_uint(M)));
    st_agent(st + 1, tagged(tag, __float_as_uint(S)));
  }
  TRACE(1);

  // ---- top-F guesses, per tile: the tile's best F per draft row go to the workspace, then a word
  // tagged with the call says they are in. Runs while the tile waits for the decision.
  // Draft row r of a row that phase 1 could not filter: compaction of the tokens at or above the
  // threshold into the wave's region (exact top Fp from registers if too many pass).
  auto row_filter = [&](const float (&z)[kE], int r) __attribute__((always_inline)) {
    float m = z[0];
#pragma unroll
    for (int q = 1; q < kE; ++q) m = fmaxf(m, z[q]);
    int n;
    const float thr0 = lane_thr(m, n);
    const float thr = (n < Fp) ? -__FLT_MAX__ : thr0;  // fewer than Fp finite lanes: all finite pass
    // Compaction without a scalar round trip per token: per-lane counts, a DPP scan for each
    // lane's first slot, then one LDS write per token, the tokens that fail going to a per-lane
    // spare slot. An entry holds the raw float bits and ~token.
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kE; ++q) cnt += (z[q] >= thr) ? 1 : 0;
    const int incl = wave_incl_scan_i(cnt);
    int total = __builtin_amdgcn_readlane(incl, 63);
    uint64_t* region = sh.reg[r][w];
    if (total <= kRegW) {
      int slot = incl - cnt;
      uint64_t* spare = &sh.spare[w][lane];
#pragma unroll
      for (int q = 0; q < kE; ++q) {
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
        for (int q = 0; q < kE; ++q) {
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
  // the tile's guess f of draft row r as two words tagged with the call (high, low half of the key)
  auto publish_guess = [&](int r, int f, uint64_t kv) __attribute__((always_inline)) {
    uint64_t* cw = a.cand + (((int64_t(b) * K + r) * nT + tile) * a.topfFmax + f) * 2;
    st_agent(cw, tagged(tag, uint32_t(kv >> 32)));
    st_agent(cw + 1, tagged(tag, uint32_t(kv)));
  };
  auto topf_tile = [&]() __attribute__((always_inline)) {
    // rows the hot-lane copy could not take: re-read from cache and filtered into the regions
    if ((sh.fb[0] | sh.fb[1] | sh.fb[2] | sh.fb[3]) != 0u) {
      uint32_t fbm = __builtin_amdgcn_readfirstlane(sh.fb[w]);
      while (fbm) {
        const int r = __builtin_ctz(fbm);
        fbm &= fbm - 1u;
        float z[kE];
        row_fetch<ET>(row_ptr(r), bl, V, mode, z);
        row_filter(z, r);
      }
      __syncthreads();
    }
    // Wave w selects the F best candidates (value desc, index asc) of rows w, w + 4, ... and
    // publishes them itself. Candidate round i reads the region of wave i / 2: a dump gives lane
    // l element l % 16 of slot l / 16 + 4 (i % 2); a key list (rows filtered after phase 1) gives
    // lane l its entry l + 64 (i % 2).
    for (int r = w; r < K; r += kWaves) {
      const int F = sh.F[r];
      if constexpr (sizeof(T) == 2) {
        // bf16: 32-bit keys, the value's 16-bit order key above 0xFFFF - (token - c0), so a larger
        // key is a larger value, then a smaller token; 0 = none (every real key is above 2^23).
        // Every read is issued first (clamped, in bounds), then the keys are formed.
        const uint32_t xs_l = uint32_t(sh.xe[r] - c0);  // the sampled token, relative to the tile
        const int e = lane & 15;
        int n[kWaves];
        uint32_t th[kWaves];
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          n[ww] = __builtin_amdgcn_readfirstlane(sh.nseg[r][ww]);
          th[ww] = uint32_t(__builtin_amdgcn_readfirstlane(sh.thr[r][ww])) >> 16;
        }
        constexpr int kParts = kSel / kWaves;
        uint32_t rawv[kSel];
        int hlv[kSel];
#pragma unroll
        for (int i = 0; i < kSel; ++i) {
          const int ww = i / kParts, slc = min((lane >> 4) + 4 * (i % kParts), kHot - 1);
          rawv[i] = reinterpret_cast<const uint16_t*>(&sh.reg[r][ww][0])[slc * kE + e];
          hlv[i] = sh.hl[r][ww][slc];
        }
        uint32_t key[kSel];
#pragma unroll
        for (int i = 0; i < kSel; ++i) {
          const int ww = i / kParts, part = i % kParts;
          const int sl = (lane >> 4) + 4 * part;
          const uint32_t raw = rawv[i];
          const uint32_t ok16 = (raw & 0x8000u) ? (~raw & 0xFFFFu) : (raw | 0x8000u);
          const uint32_t tl = uint32_t(ww * LY::WTOK + hlv[i] * LY::VEC + LY::tok(0, e));
          // th is above the key of -inf; the sampled token is never a guess
          const bool ok = (sl < -n[ww]) & (ok16 >= th[ww]) & (int(tl) < V - c0) & (tl != xs_l);
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
          for (int i = 1; i < kSel; ++i) mine = max(mine, key[i]);
          const uint32_t win = wave_max_u32(mine);
#pragma unroll
          for (int i = 0; i < kSel; ++i) key[i] = (key[i] == win) ? 0u : key[i];  // keys are unique
          if (lane == 0) {  // back to the 64-bit (order key of the float, ~token) form
            const uint32_t h = win >> 16;
            const uint32_t okf = (h << 16) | ((h & 0x8000u) ? 0u : 0xFFFFu);
            publish_guess(r, f, win ? (uint64_t(okf) << 32) |
                                         uint64_t(~uint32_t(c0 + int(0xFFFFu - (win & 0xFFFFu))))
                                    : 0ull);
          }
        }
      } else {
        const int xs = sh.xe[r];
        const int e = lane & 15;
        uint64_t key[kSel];
#pragma unroll
        for (int i = 0; i < kSel; ++i) {
          constexpr int kParts = kSel / kWaves;
          const int ww = i / kParts, part = i % kParts;
          const int n = __builtin_amdgcn_readfirstlane(sh.nseg[r][ww]);
          key[i] = 0;
          if (n < 0 && 4 * part < -n) {  // uniform: some slot of this quarter holds a dump
            const uint32_t th = __builtin_amdgcn_readfirstlane(sh.thr[r][ww]);
            const int sl = (lane >> 4) + 4 * part;
            const int slc = min(sl, kHot - 1);
            const float v = ET::one(reinterpret_cast<const T*>(&sh.reg[r][ww][0]) + slc * kE, e);
            const int tok = c0 + ww * LY::WTOK + sh.hl[r][ww][slc] * LY::VEC + LY::tok(0, e);
            const uint32_t kv = ordered_key(v);
            // th is above the key of -inf; the sampled token is never a guess
            const bool ok = (sl < -n) & (kv >= th) & (tok < V) & (tok != xs);
            key[i] = ok ? (uint64_t(kv) << 32) | uint64_t(~uint32_t(tok)) : 0ull;
          } else if (n > 64 * part) {  // key list
            const uint64_t ent = sh.reg[r][ww][min(lane + 64 * part, kRegW - 1)];
            const float v = __uint_as_float(uint32_t(ent >> 32));
            const int tok = int(~uint32_t(ent));
            if (lane + 64 * part < n && uint32_t(ent) != 0u && tok != xs)  // entry lo 0 = none
              key[i] = (uint64_t(ordered_key(v)) << 32) | uint32_t(ent);
          }
        }
        // the nonzero keys (a few per wave region) into one list, one per lane: the F rounds then
        // take a single key per lane (more than 64: rounds over all of them)
        uint64_t* lst = sh.spare[w];
        int N = 0;
#pragma unroll
        for (int i = 0; i < kSel; ++i) {
          const uint64_t m = __ballot(key[i] != 0ull);
          if (m) {
            const int at = N + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
            if (key[i] != 0ull && at < 64) lst[at] = key[i];
            N += __popcll(m);
          }
        }
        if (N <= 64) {
          uint64_t mine = (lane < N) ? lst[lane] : 0ull;
          for (int f = 0; f < F; ++f) {
            const uint64_t win = wave_max_u64(mine);
            if (lane == 0) publish_guess(r, f, win);
            mine = (mine == win) ? 0ull : mine;  // keys are unique: only the winner is cleared
          }
        } else {
          for (int f = 0; f < F; ++f) {
            uint64_t mine = key[0];
#pragma unroll
            for (int i = 1; i < kSel; ++i) mine = max_u64(mine, key[i]);
            const uint64_t win = wave_max_u64(mine);
            if (lane == 0) publish_guess(r, f, win);
#pragma unroll
            for (int i = 0; i < kSel; ++i) key[i] = (key[i] == win) ? 0ull : key[i];
          }
        }
      }
    }
  };

  // ---- claim the decision: the first tile past phase 1 swaps the lead word from the last call's
  // tag to this call's. It has the most time to spare before the last statistics arrive, so its
  // own top-F pass costs the decision nothing. The answer is read after the pass.
  uint32_t seen = tag_ld;
  bool won = false;
  if (t == 0)
    won = __hip_atomic_compare_exchange_strong(ctl + kCtlLead, &seen, tag, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
  if (FM > 0) topf_tile();
  TRACE(10);
  if (t == 0) {
    // a word that holds neither the last tag nor this one is left from a call that timed out:
    // claim from whatever it holds
    for (int i = 0; i < 8 && !won && seen != tag; ++i)
      won = __hip_atomic_compare_exchange_strong(ctl + kCtlLead, &seen, tag, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh.leader = won ? 1 : 0;
  }
  __syncthreads();
  const bool leader = sh.leader != 0;
  // ---- decide: the claiming tile waits for every tile's statistics, merges them, takes the
  // decisions and publishes them in a record of tagged words, which the other tiles poll
  float rv[kE], pre[kE];
  {
    if (leader) {
      // logits at the draft tokens (draft and target rows 0..K-1) and at the Saguaro-set tokens,
      // gathered from the rows; issued first, so they overlap the top-F pass and the statistics loads
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
        const uint64_t* st = a.stats + (int64_t(b) * R2 + r) * nT * 2;
        float M = -INFINITY, S = 0.f;
        constexpr int kAhead = 4;  // tiles per lane per polling round
        for (int q0 = (t & 15); q0 < nT; q0 += kAhead * 16) {
          uint64_t mv[kAhead], sv[kAhead];
          for (int spins = 0;; ++spins) {  // until both words of each tile carry this call's tag
            bool ok = true;
#pragma unroll
            for (int i = 0; i < kAhead; ++i) {
              const int q = q0 + i * 16;
              mv[i] = (q < nT) ? ld_agent(st + 2 * q) : tagged(tag, 0xFF800000u);
              sv[i] = (q < nT) ? ld_agent(st + 2 * q + 1) : tagged(tag, 0u);
              ok = ok && uint32_t(mv[i] >> 32) == tag && uint32_t(sv[i] >> 32) == tag;
            }
            if (__all(ok)) break;
            if (spins > a.spin_limit) {
              if (!ok) atomicOr(a.flags, kFlagTimeout);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
#pragma unroll
          for (int i = 0; i < kAhead; ++i) {
            const float m = lo_f(mv[i]), s = lo_f(sv[i]);
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
      // thread 0 has seen row 0 of every tile with this call's tag, so every tile has read the
      // previous tag: the next call may start from this one
      if (t == 0) st_agent(ctl + kCtlTag, tag);
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
      if (t < 64) {  // wave 0: lane i takes the accept test of position i
        const int i = min(lane, K - 1);
        const float C = a.Cpos[i];  // Saguaro factor of position i
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
        const float Ck = (k < K) ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(C), k)) : 1.f;
        // the record, straight from registers: lane j publishes word j (the set of row k keeps
        // its -1 holes: duplicates and out-of-range entries, which the residual skips)
        const int nset = (k < K) ? sF : 0;
        const float Lpk = sh.L[K + k], Lqk = (k < K) ? sh.L[k] : 0.f;
        const int f = lane - kDecSet;
        const int sv = (f >= 0 && f < nset) ? sh.set[k * sF + f] : -1;
        uint32_t v = uint32_t(sv);
        if (lane == kDecK) v = uint32_t(k);
        if (lane == kDecLp) v = __float_as_uint(Lpk);
        if (lane == kDecLq) v = __float_as_uint(Lqk);
        if (lane == kDecWout) v = __float_as_uint(1.f / Nk);
        if (lane == kDecWin) v = __float_as_uint(Ck / Nk);
        if (lane == kDecNset) v = uint32_t(nset);
        if (lane < kDecWords) st_agent(dec + lane, tagged(tag, v));
        // this tile's own copy, for its residual
        if (lane == 0) {
          a.k_out[b] = k;
          sh.k = k;
          sh.nset = nset;
          sh.Lp = Lpk;
          sh.Lq = Lqk;
          sh.w_out = 1.f / Nk;
          sh.w_in = Ck / Nk;
        }
        if (f >= 0 && f < kMaxF) sh.myset[f] = sv;
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
    const int k = min(max(sh.k, 0), K);
    const bool resid = k < K;
    const T* prow = target + int64_t(k) * V;
    const T* qrow = resid ? draft + int64_t(k) * V : nullptr;
    const float Lp = sh.Lp, Lq = sh.Lq, w_out = sh.w_out, w_in = sh.w_in;
    const int nset = resid ? min(max(sh.nset, 0), kMaxF) : 0;

    // ---- residual mass of this tile (values and prefix sums stay in registers), published
    const float total = tile_residual<ET>(prow, qrow, bl, V, mode, cc, Lp, Lq, w_out, w_in, sh.myset,
                                          nset, sh.wt, rv, pre);
    if (t == 0) st_agent(a.res + int64_t(b) * nT + tile, tagged(tag, __float_as_uint(total)));
    TRACE(4);
  }
  const int k = min(max(sh.k, 0), K);
  const bool resid = k < K;
  const T* prow = target + int64_t(k) * V;
  const float Lp = sh.Lp;

  // ---- top-F guesses of draft rows tile, tile + T, ...: wave 0 merges the tiles' candidates. Keys
  // are unique (a token lives in one tile), so round f picks the largest key below round f-1's.
  // Each key is two words tagged with the call; a lane polls its own.
  for (int r = tile; FM > 0 && w == 0 && r < K; r += nT) {
    const int F = sh.F[r];
    int32_t* out = a.topf_out + (int64_t(b) * K + r) * a.topfFmax;
    const uint64_t* cd = a.cand + (int64_t(b) * K + r) * nT * a.topfFmax * 2;
    const int n = nT * F;
    auto cand_at = [&](int q) -> uint64_t {  // key q = (tile q / F, guess q % F), once tagged
      const int tl = q / F, ff = q - tl * F;
      const uint64_t* cw = cd + (int64_t(tl) * a.topfFmax + ff) * 2;
      uint64_t hi = 0, lo = 0;
      for (int spins = 0;; ++spins) {
        hi = ld_agent(cw);
        lo = ld_agent(cw + 1);
        if (uint32_t(hi >> 32) == tag && uint32_t(lo >> 32) == tag) break;
        if (spins > a.spin_limit) {
          atomicOr(a.flags, kFlagTimeout);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
    };
    constexpr int kM = 4;  // keys per lane held in registers
    if (n <= 64 * kM) {
      uint64_t key[kM];
#pragma unroll
      for (int i = 0; i < kM; ++i) key[i] = (lane + 64 * i < n) ? cand_at(lane + 64 * i) : 0ull;
      for (int f = 0; f < F; ++f) {
        uint64_t mine = key[0];
#pragma unroll
        for (int i = 1; i < kM; ++i) mine = max_u64(mine, key[i]);
        const uint64_t win = wave_max_u64(mine);
        if (lane == 0) out[f] = win ? int(~uint32_t(win)) : -1;
#pragma unroll
        for (int i = 0; i < kM; ++i) key[i] = (key[i] == win) ? 0ull : key[i];
      }
    } else {  // many tiles: every round re-reads the keys, taking the largest below the last
      uint64_t prev = ~0ull;
      for (int f = 0; f < F; ++f) {
        uint64_t best = 0;
        for (int q = lane; q < n; q += 64) {
          const uint64_t kq = cand_at(q);
          best = (kq < prev && kq > best) ? kq : best;
        }
        const uint64_t win = wave_max_u64(best);
        if (lane == 0) out[f] = win ? int(~uint32_t(win)) : -1;
        prev = win;
      }
    }
    for (int f = F + lane; f < a.topfFmax; f += 64) out[f] = -1;
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
template <class ET, int FM, int G, int MB>
static int capacity_blocks() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(verify_fused_kernel<ET, FM, G, MB>), kThreads, 0) != hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = per_cu * cus;
  }
  return cache[dev];
}

// launches of the MB variant for a.B sequences (0: the device cannot hold one sequence's tiles)
template <class ET, int FM, int G, int MB>
static int rounds_needed(const VerifyArgs& a) {
  const int cap = capacity_blocks<ET, FM, G, MB>();
  if (cap < a.T) return 0;
  const int per_round = cap / a.T;
  return (a.B + per_round - 1) / per_round;
}

template <class ET, int FM, int G, int MB>
static hipError_t launch_fused(VerifyArgs a, hipStream_t st, int* n_launches) {
  const int cap = capacity_blocks<ET, FM, G, MB>();
  if (cap < a.T) return hipErrorInvalidConfiguration;
  const int per_round = cap / a.T;  // whole sequences whose tiles are all resident at once
  const int B = a.B;
  if (n_launches) {  // count only
    *n_launches = (B + per_round - 1) / per_round;
    return hipSuccess;
  }
  for (int b0 = 0; b0 < B; b0 += per_round) {
    const int nb = (B - b0 < per_round) ? (B - b0) : per_round;
    a.b0 = b0;
    hipLaunchKernelGGL((verify_fused_kernel<ET, FM, G, MB>), dim3(unsigned(nb * a.T)), dim3(kThreads), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Rows per load group: bf16 9 (K <= 4 in one group, 8 VGPRs of payload per row and lane), fp32 5
// (16 VGPRs per row). Larger K runs several groups; a smaller K loads the last row again for the
// unused slots (cache hits) and skips their arithmetic.
template <class ET, int FM>
static hipError_t launch_g(const VerifyArgs& a, hipStream_t st, int* n) {
  constexpr int G = (sizeof(typename ET::T) == 2 ? 9 : 5);
  // four workgroups per CU only when that saves launches (measured: 7 -> 5 launches for 128
  // sequences of 152064 fp32 logits, 373 -> 352 us a step; one launch of 16 sequences is ~4 %
  // slower with the spills, so it keeps two)
  const int r2 = rounds_needed<ET, FM, G, 2>(a), r4 = rounds_needed<ET, FM, G, 4>(a);
  if (r4 > 0 && (r2 == 0 || r4 < r2)) return launch_fused<ET, FM, G, 4>(a, st, n);
  return launch_fused<ET, FM, G, 2>(a, st, n);
}

template <class ET>
static hipError_t launch_verify_e(const VerifyArgs& a, hipStream_t st, int* n) {
  if (a.topfFmax == 0) return launch_g<ET, 0>(a, st, n);
  if (a.topfFmax <= 4) return launch_g<ET, 4>(a, st, n);
  if (a.topfFmax <= 8) return launch_g<ET, 8>(a, st, n);
  return launch_g<ET, 16>(a, st, n);
}

hipError_t launch_verify(const VerifyArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_verify_e<BF16T>(a, st, nullptr) : launch_verify_e<F32T>(a, st, nullptr);
}

int count_verify_launches(const VerifyArgs& a, bool bf16) {
  int n = -1;
  const hipError_t e = bf16 ? launch_verify_e<BF16T>(a, nullptr, &n) : launch_verify_e<F32T>(a, nullptr, &n);
  return e == hipSuccess ? n : -1;
}

}  // namespace ssd
