// gfx950 kernels for batched lossless draft verification and the SSD / Saguaro pieces.
//
// Verification (one call = one round for B sequences) runs in two launches:
//   phase 1  verify_rows:   every draft and target row is cut into chunks; one 256-thread
//            workgroup streams one chunk with 16-byte loads and leaves (max, sum 2^(z c - max))
//            of z c = z log2(e) / T, plus, on draft rows, its chunk's top-F candidates.
//   phase 2  verify_decide: one workgroup per (sequence, 2048-token sub-chunk). Each merges the
//            row statistics of its sequence (fixed order, so all agree bit for bit), takes the
//            accept decisions and k, then sums the residual max(p_k - q'_k, 0) (or p_K when every
//            draft is accepted) over its sub-chunk. The last workgroup of the sequence to finish
//            (an atomic counter) locates the sub-chunk holding u_K * R and scans it for the bonus.
// Top-F guesses and Saguaro down-weighting reuse the phase-1 chunk pass.
#include <hip/hip_runtime.h>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"
#include "ssd_plan.hpp"

namespace ssd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Cand {
  float v;
  int i;
};

__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(r.x, r.y, r.z, r.w);
}

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
    if (STATS) {
      if (z > mx) {
        s = s * ex2((mx - z) * c);
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
      if (STATS) {
        if (bm > mx) {
          s = s * ex2((mx - bm) * c);
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
                            int32_t* __restrict__ out, int Fmax, uint32_t* shk) {
  constexpr int kPer = (kMaxChunks * kMaxF + kThreads - 1) / kThreads;
  const int n = n_lists * F;
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
    if (threadIdx.x == 0) out[r] = (gh != 0) ? int(~gl) : -1;
  }
  for (int r = F + threadIdx.x; r < Fmax; r += kThreads) out[r] = -1;
}

// =============================================================================================
// Verification
// =============================================================================================
template <class ET, int FM>
__global__ __launch_bounds__(kThreads) void verify_rows_kernel(VerifyArgs a) {
  using T = typename ET::T;
  __shared__ float shf[8];
  __shared__ uint32_t shk[2 * kWaves];
  __shared__ float wv[kMaxF];
  __shared__ int wi[kMaxF];

  const int item = blockIdx.x;
  const int row = item / a.n1;
  const int chunk = item - row * a.n1;
  const int R2 = 2 * a.K + 1;
  const int b = row / R2, j = row - b * R2;

  if (item == 0)  // phase 2 starts after this launch completes: reset its arrival counters
    for (int i = threadIdx.x; i < a.B; i += kThreads) a.cnt[i * 16] = 0u;

  const T* p;
  int F = 0, ex = -1;
  if (j < a.K) {
    p = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride + int64_t(j) * a.V;
    if (FM > 0) {
      F = a.topfF[j];
      ex = a.x[b * a.K + j];
    }
  } else {
    p = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride + int64_t(j - a.K) * a.V;
  }
  const int c0 = chunk * a.chunk1;
  const int c1 = min(a.V, c0 + a.chunk1);

  float mx = -INFINITY, s = 0.f;
  TopList<(FM > 0 ? FM : 1)> tl;
  tl.init(F);
  chunk_pass<ET, true, FM>(p, c0, c1, a.aligned != 0, a.c2, ex, mx, s, tl);

  const float MX = block_max(mx, shf);
  const float part = (s > 0.f) ? s * ex2(mx * a.c2 - MX * a.c2) : 0.f;
  const float S = block_sum(part, shf);
  if (threadIdx.x == 0) a.stats[int64_t(row) * a.n1 + chunk] = make_float2(MX * a.c2, S);

  if (FM > 0 && F > 0) {
    block_merge_top<(FM > 0 ? FM : 1)>(tl, F, shk, wv, wi);
    if (threadIdx.x == 0) {
      Cand* cd = reinterpret_cast<Cand*>(a.cand) +
                 (int64_t(b * a.K + j) * a.n1 + chunk) * a.topfFmax;
      for (int r = 0; r < F; ++r) cd[r] = Cand{wv[r], wi[r]};
    }
  }
}

// residual (or target-row) values of the 8 contiguous elements of this thread in a sub-chunk
template <class ET>
__device__ __forceinline__ void sub_values(const typename ET::T* __restrict__ prow,
                                           const typename ET::T* __restrict__ qrow, int c0, int V,
                                           bool aligned, float c, float Lp, float Lq, float w_out,
                                           float w_in, const int* set_entries, int n_set,
                                           float (&r)[kSubElems]) {
  const int e0 = c0 + threadIdx.x * kSubElems;
  float zp[kSubElems], zq[kSubElems];
  const bool full = aligned && (e0 + kSubElems <= V);
  if (full) {
#pragma unroll
    for (int h = 0; h < kSubElems / ET::kVec; ++h) {
      const uint4 v = load16(prow + e0 + h * ET::kVec);
      ET::unpack(v, zp + h * ET::kVec);
    }
    if (qrow) {
#pragma unroll
      for (int h = 0; h < kSubElems / ET::kVec; ++h) {
        const uint4 v = load16(qrow + e0 + h * ET::kVec);
        ET::unpack(v, zq + h * ET::kVec);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSubElems; ++e) {
      const int idx = e0 + e;
      zp[e] = (idx < V) ? ET::one(prow, idx) : -INFINITY;
      zq[e] = (qrow && idx < V) ? ET::one(qrow, idx) : -INFINITY;
    }
  }
#pragma unroll
  for (int e = 0; e < kSubElems; ++e) {
    const float pv = ex2(fmaf(zp[e], c, -Lp));
    if (qrow) {
      float w = w_out;
      for (int f = 0; f < n_set; ++f)
        if (set_entries[f] == e0 + e) w = w_in;
      const float qv = ex2(fmaf(zq[e], c, -Lq)) * w;
      r[e] = fmaxf(pv - qv, 0.f);
    } else {
      r[e] = pv;
    }
    if (e0 + e >= V) r[e] = 0.f;
  }
}

// Scan this thread's 8 values, then the block: returns per-element inclusive prefixes relative to
// the sub-chunk start in pre[], and the sub-chunk total.
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

template <class ET, int FM>
__global__ __launch_bounds__(kThreads) void verify_decide_kernel(VerifyArgs a) {
  using T = typename ET::T;
  __shared__ float2 s_part[(2 * kMaxK + 1) * kMaxChunks];
  __shared__ float s_L[2 * kMaxK + 1];
  __shared__ float s_zq[kMaxK], s_zp[kMaxK], s_u[kMaxK + 1], s_N[kMaxK];
  __shared__ int s_x[kMaxK];
  __shared__ int s_set[kMaxK * kMaxF];
  __shared__ float s_zs[kMaxK * kMaxF];
  __shared__ int s_k, s_last, s_cstar, s_clamp, s_fallback;
  __shared__ float s_target, s_base, s_R;
  __shared__ float s_res[kMaxSubs];
  __shared__ float shf[8];
  __shared__ int shi[8];
  __shared__ uint32_t shk[2 * kWaves];
  __shared__ int s_myset[kMaxF];
  __shared__ int s_nmyset;

  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int K = a.K, V = a.V, R2 = 2 * K + 1, n1 = a.n1, sF = a.sF, n2 = gridDim.x;
  const float cc = a.c2;
  const T* draft = reinterpret_cast<const T*>(a.draft) + int64_t(b) * a.dstride;
  const T* target = reinterpret_cast<const T*>(a.target) + int64_t(b) * a.tstride;

  // ---- 1. gather this sequence's row statistics, tokens, uniforms and set logits
  for (int e = t; e < R2 * n1; e += kThreads) s_part[e] = a.stats[int64_t(b) * R2 * n1 + e];
  if (t < K) {
    const int x = a.x[b * K + t];
    const bool ok = unsigned(x) < unsigned(V);
    s_x[t] = ok ? x : -1;
    s_zq[t] = ok ? ET::one(draft + int64_t(t) * V, x) : 0.f;
    s_zp[t] = ok ? ET::one(target + int64_t(t) * V, x) : 0.f;
    if (!ok && c == 0) atomicOr(a.flags, kFlagBadToken);
  }
  if (t <= K) s_u[t] = a.u[b * (K + 1) + t];
  int my_set = -1;
  if (t < K * sF) {
    const int i = t / sF;
    const int sv = a.sset[int64_t(b) * K * sF + t];
    const bool ok = unsigned(sv) < unsigned(V);
    my_set = ok ? sv : -1;
    s_set[t] = my_set;
    s_zs[t] = ok ? ET::one(draft + int64_t(i) * V, sv) : 0.f;
  }
  __syncthreads();
  if (t < K * sF && my_set >= 0) {  // keep the first occurrence of each token only
    const int i = t / sF, f = t - i * sF;
    for (int g = 0; g < f; ++g)
      if (s_set[i * sF + g] == my_set) my_set = -1;
  }
  __syncthreads();
  if (t < K * sF) s_set[t] = my_set;

  // ---- 2. merge chunk statistics: L = log2 of the row's partition function in units of z c
  if (t < R2) {
    float M = -INFINITY;
    for (int q = 0; q < n1; ++q) M = fmaxf(M, s_part[t * n1 + q].x);
    float S = 0.f;
    for (int q = 0; q < n1; ++q) {
      const float2 v = s_part[t * n1 + q];
      if (v.y > 0.f) S += v.y * ex2(v.x - M);
    }
    s_L[t] = M + lg2(S);
  }
  __syncthreads();

  // ---- 3. accept decisions (identical in every workgroup of the sequence)
  if (t == 0) {
    int k = K;
    const float C = a.C;
    for (int i = 0; i < K; ++i) {
      const float Lq = s_L[i], Lp = s_L[K + i];
      float N = 1.f;
      bool xin = false;
      if (sF > 0) {
        float sig = 0.f;
        for (int f = 0; f < sF; ++f) {
          const int sv = s_set[i * sF + f];
          if (sv < 0) continue;
          sig += ex2(fmaf(s_zs[i * sF + f], cc, -Lq));
          if (sv == s_x[i]) xin = true;
        }
        N = 1.f - (1.f - C) * sig;
        if (!(N > 0.f) && c == 0) atomicOr(a.flags, kFlagSaguaroNorm);
      }
      s_N[i] = N;
      bool accept;
      float ai;
      if (s_x[i] < 0) {
        accept = false;
        ai = 0.f;
      } else {
        const float w = xin ? C : 1.f;
        const float dp = fmaf(s_zp[i], cc, -Lp);  // log2 p(x)
        const float dq = fmaf(s_zq[i], cc, -Lq);  // log2 q(x)
        if (w == 0.f || dq == -INFINITY) {        // q'(x) = 0: accept iff p(x) > 0
          accept = dp > -INFINITY;
          ai = accept ? 1.f : 0.f;
        } else {
          const float ratio = ex2(dp - dq) * (N / w);  // p(x) / q'(x)
          accept = s_u[i] < ratio;
          ai = fminf(1.f, ratio);
        }
      }
      if (a.aprob_out && c == 0) a.aprob_out[b * K + i] = ai;
      if (k == K && !accept) k = i;
    }
    s_k = k;
  }
  __syncthreads();
  const int k = s_k;

  // ---- top-F guesses of the draft rows (independent of k)
  if (FM > 0) {
    for (int jr = c; jr < K; jr += n2) {
      const int F = a.topfF[jr];
      int32_t* out = a.topf_out + (int64_t(b) * K + jr) * a.topfFmax;
      const Cand* cd = reinterpret_cast<const Cand*>(a.cand) + int64_t(b * K + jr) * n1 * a.topfFmax;
      merge_lists(cd, F > 0 ? n1 : 0, a.topfFmax, F, out, a.topfFmax, shk);
    }
  }

  // ---- 4. residual (k < K) or target row K (k == K) over sub-chunk c
  const bool resid = k < K;
  const T* prow = target + int64_t(k) * V;
  const T* qrow = resid ? draft + int64_t(k) * V : nullptr;
  const float Lp = s_L[K + k];
  const float Lq = resid ? s_L[k] : 0.f;
  const float N = resid ? s_N[k] : 1.f;
  const float w_out = 1.f / N, w_in = a.C / N;
  if (t == 0) {
    int n = 0;
    if (resid)
      for (int f = 0; f < sF; ++f) {
        const int sv = s_set[k * sF + f];
        if (sv >= 0) s_myset[n++] = sv;
      }
    s_nmyset = n;
  }
  __syncthreads();
  const int nset = s_nmyset;
  const bool aligned = a.aligned != 0;

  float r[kSubElems], pre[kSubElems];
  sub_values<ET>(prow, qrow, c * kSub, V, aligned, cc, Lp, Lq, w_out, w_in, s_myset, nset, r);
  const float total = sub_scan(r, pre, shf);
  if (t == 0) {
    a.res[int64_t(b) * n2 + c] = total;
    __threadfence();
    const unsigned old = atomicAdd(&a.cnt[b * 16], 1u);
    s_last = (old == unsigned(n2 - 1));
  }
  __syncthreads();
  if (!s_last) return;

  // ---- 5. last workgroup of the sequence: inverse-CDF search for the bonus token
  __threadfence();
  for (int e = t; e < n2; e += kThreads) s_res[e] = __hip_atomic_load(
      a.res + int64_t(b) * n2 + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (t == 0) {
    a.cnt[b * 16] = 0u;
    float P = 0.f;
    for (int q = 0; q < n2; ++q) P += s_res[q];
    const float R = P;
    const float target_v = s_u[K] * R;
    int cstar = -1, last_pos = -1;
    float run = 0.f, base = 0.f;
    for (int q = 0; q < n2; ++q) {
      const float nxt = run + s_res[q];
      if (s_res[q] > 0.f) last_pos = q;
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
      base = 0.f;
    }
    s_fallback = (cstar < 0);  // all-zero residual
    s_cstar = cstar;
    s_clamp = clamp;
    s_base = base;
    s_target = target_v;
    s_R = R;
  }
  __syncthreads();

  int bonus = -1;
  if (!s_fallback) {
    const int cs = s_cstar;
    sub_values<ET>(prow, qrow, cs * kSub, V, aligned, cc, Lp, Lq, w_out, w_in, s_myset, nset, r);
    sub_scan(r, pre, shf);
    const int e0 = cs * kSub + t * kSubElems;
    int first = INT_MAX, lastp = -1;
#pragma unroll
    for (int e = 0; e < kSubElems; ++e) {
      if (r[e] > 0.f) {
        lastp = e0 + e;
        if (first == INT_MAX && !s_clamp && s_base + pre[e] > s_target) first = e0 + e;
      }
    }
    first = block_min_i(first, shi);
    lastp = block_max_i(lastp, shi);
    bonus = (first != INT_MAX) ? first : lastp;
  } else {
    // residual identically zero: draw from the target row p_k itself (R = 1)
    const float target_v = s_u[K];
    float run = 0.f;
    int found = -1, lastp = -1;
    for (int q = 0; q < n2 && found < 0; ++q) {
      sub_values<ET>(prow, nullptr, q * kSub, V, aligned, cc, Lp, 0.f, 1.f, 1.f, s_myset, 0, r);
      const float tot = sub_scan(r, pre, shf);
      const int e0 = q * kSub + t * kSubElems;
      int first = INT_MAX, lp = -1;
#pragma unroll
      for (int e = 0; e < kSubElems; ++e)
        if (r[e] > 0.f) {
          lp = e0 + e;
          if (first == INT_MAX && run + pre[e] > target_v) first = e0 + e;
        }
      first = block_min_i(first, shi);
      lp = block_max_i(lp, shi);
      if (lp >= 0) lastp = lp;
      if (first != INT_MAX) found = first;
      run += tot;
    }
    bonus = (found >= 0) ? found : lastp;
  }
  if (t == 0) {
    a.k_out[b] = k;
    a.bonus_out[b] = bonus;
    if (a.rmass_out) a.rmass_out[b] = resid ? s_R : 1.f;
  }
}

// =============================================================================================
// Standalone top-F guesses
// =============================================================================================
template <class ET, int FM>
__global__ __launch_bounds__(kThreads) void topf_rows_kernel(TopfArgs a) {
  using T = typename ET::T;
  __shared__ uint32_t shk[2 * kWaves];
  __shared__ float wv[kMaxF];
  __shared__ int wi[kMaxF];
  const int item = blockIdx.x;
  const int row = item / a.n1;
  const int chunk = item - row * a.n1;
  int F = a.Fmax;
  if (a.F_per_row) {
    F = a.F_per_row[row];
    if (F < 0 || F > a.Fmax) {
      if (chunk == 0 && threadIdx.x == 0) atomicOr(a.flags, kFlagBadF);
      F = F < 0 ? 0 : a.Fmax;
    }
  }
  const int ex = a.exclude ? a.exclude[row] : -1;
  const T* p = reinterpret_cast<const T*>(a.logits) + int64_t(row) * a.row_stride;
  const int c0 = chunk * a.chunk1;
  const int c1 = min(a.V, c0 + a.chunk1);
  float mx = -INFINITY, s = 0.f;
  TopList<FM> tl;
  tl.init(F);
  chunk_pass<ET, false, FM>(p, c0, c1, a.aligned != 0, 1.f, ex, mx, s, tl);
  block_merge_top<FM>(tl, F, shk, wv, wi);
  if (threadIdx.x == 0) {
    if (a.n1 == 1) {
      int32_t* out = a.out + int64_t(row) * a.Fmax;
      for (int r = 0; r < a.Fmax; ++r) out[r] = (r < F) ? wi[r] : -1;
    } else {
      Cand* cd = reinterpret_cast<Cand*>(a.cand) + (int64_t(row) * a.n1 + chunk) * a.Fmax;
      for (int r = 0; r < F; ++r) cd[r] = Cand{wv[r], wi[r]};
    }
  }
}

__global__ __launch_bounds__(kThreads) void topf_merge_kernel(TopfArgs a) {
  __shared__ uint32_t shk[2 * kWaves];
  const int row = blockIdx.x;
  int F = a.Fmax;
  if (a.F_per_row) {
    F = a.F_per_row[row];
    F = F < 0 ? 0 : (F > a.Fmax ? a.Fmax : F);
  }
  const Cand* cd = reinterpret_cast<const Cand*>(a.cand) + int64_t(row) * a.n1 * a.Fmax;
  merge_lists(cd, F > 0 ? a.n1 : 0, a.Fmax, F, a.out + int64_t(row) * a.Fmax, a.Fmax, shk);
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
  __shared__ float s_L, s_N;
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
    const float N = 1.f - (1.f - a.C) * sig;
    s_L = L;
    s_N = N;
    if (chunk == 0) {
      if (a.out_set_mass) a.out_set_mass[row] = sig;
      if (a.out_norm) a.out_norm[row] = N;
      if (!(N > 0.f)) atomicOr(a.flags, kFlagSaguaroNorm);
    }
  }
  __syncthreads();
  if (!a.out_probs) return;
  const float L = s_L, w_out = 1.f / s_N, w_in = a.C / s_N;
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
  const int tok = a.guesses[(int64_t(b) * (a.K + 1) + k) * a.Gmax + rank];
  a.cache_k[g] = (tok >= 0) ? k : -1;
  a.cache_tok[g] = (tok >= 0) ? tok : -1;
}

__global__ __launch_bounds__(kThreads) void cache_lookup_kernel(CacheLookupArgs a) {
  __shared__ int shi[8];
  int miss = 0;
  for (int b = threadIdx.x; b < a.B; b += kThreads) {
    const int k = a.k[b], tok = a.tok[b];
    int slot = -1;
    const int32_t* ck = a.cache_k + int64_t(b) * a.budget;
    const int32_t* ct = a.cache_tok + int64_t(b) * a.budget;
    for (int j = 0; j < a.budget; ++j)
      if (ck[j] == k && ct[j] == tok) {
        slot = j;
        break;
      }
    a.out_slot[b] = slot;
    miss += (slot < 0);
  }
  // block sum of integers
  for (int o = 32; o >= 1; o >>= 1) miss += __shfl_xor(miss, o, 64);
  if ((threadIdx.x & 63) == 0) shi[threadIdx.x >> 6] = miss;
  __syncthreads();
  if (threadIdx.x == 0) a.out_miss[0] = shi[0] + shi[1] + shi[2] + shi[3];
}

__global__ void clear_flags_kernel(uint32_t* flags) { *flags = 0u; }

// =============================================================================================
// launchers
// =============================================================================================
static hipError_t last_error() { return hipGetLastError(); }

template <class ET, int FM>
static hipError_t launch_verify_t(const VerifyArgs& a, int n2, hipStream_t st) {
  const int64_t items = int64_t(a.B) * (2 * a.K + 1) * a.n1;
  hipLaunchKernelGGL((verify_rows_kernel<ET, FM>), dim3(unsigned(items)), dim3(kThreads), 0, st, a);
  hipError_t e = last_error();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_decide_kernel<ET, FM>), dim3(n2, a.B), dim3(kThreads), 0, st, a);
  return last_error();
}

template <class ET>
static hipError_t launch_verify_e(const VerifyArgs& a, int n2, hipStream_t st) {
  if (a.topfFmax == 0) return launch_verify_t<ET, 0>(a, n2, st);
  if (a.topfFmax <= 4) return launch_verify_t<ET, 4>(a, n2, st);
  if (a.topfFmax <= 8) return launch_verify_t<ET, 8>(a, n2, st);
  return launch_verify_t<ET, 16>(a, n2, st);
}

hipError_t launch_verify(const VerifyArgs& a, int n2, bool bf16, hipStream_t st) {
  return bf16 ? launch_verify_e<BF16T>(a, n2, st) : launch_verify_e<F32T>(a, n2, st);
}

template <class ET, int FM>
static hipError_t launch_topf_t(const TopfArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((topf_rows_kernel<ET, FM>), dim3(unsigned(int64_t(a.R) * a.n1)), dim3(kThreads),
                     0, st, a);
  hipError_t e = last_error();
  if (e != hipSuccess || a.n1 == 1) return e;
  hipLaunchKernelGGL(topf_merge_kernel, dim3(a.R), dim3(kThreads), 0, st, a);
  return last_error();
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

hipError_t launch_cache_lookup(const CacheLookupArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(cache_lookup_kernel, dim3(1), dim3(kThreads), 0, st, a);
  return last_error();
}

hipError_t launch_clear_flags(uint32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, st, flags);
  return last_error();
}

}  // namespace ssd
