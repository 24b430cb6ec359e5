// extern "C" entry points: argument validation (before any HIP call), workspace carving, launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <vector>

#include "ssd.h"
#include "ssd_launch.hpp"
#include "ssd_plan.hpp"

using namespace ssd;

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810018921;

int elem_size(ssd_dtype d) { return d == SSD_BF16 ? 2 : 4; }
bool dtype_ok(int d) { return d == SSD_F32 || d == SSD_BF16; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0 && have >= need;
}
bool temp_ok(float T) { return std::isfinite(T) && T > 0.f; }
bool c_ok(float C) { return C >= 0.f && C <= 1.f; }  // false for NaN
template <class P>
P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}
ssd_status hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

// Verification workgroups the current device runs at once (its CU count, looked up once per
// device, times the workgroups per CU); 256 CUs when no device answers.
int verify_slots() {
  constexpr int kDevs = 64;
  static std::atomic<int> cus[kDevs];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 256 * kVerifyWgPerCu;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n * kVerifyWgPerCu;
}
// The streaming form (two launches): when the batch has more tiles than the device runs at once
bool verify_split(int B, int T) { return int64_t(B) * T > verify_slots(); }


}  // namespace

#ifdef SSD_TRACE
static void* ssd_trace_buffer = nullptr;
#endif

extern "C" {

const char* ssd_status_string(ssd_status s) {
  switch (s) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported dtype";
    case SSD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case SSD_ERR_HIP: return "HIP launch error";
    case SSD_ERR_SCRATCH_LIMIT: return "shape needs more than the allocation-free variant's static array holds";
  }
  return "unknown status";
}

// ------------------------------------------------------------------------------------------------
size_t ssd_verify_workspace_bytes(int B, int K, int V, int topf_F_max) {
  if (B < 0 || B > SSD_MAX_B || K < 1 || K > SSD_MAX_K || V < 1 || V > SSD_MAX_V || topf_F_max < 0 ||
      topf_F_max > SSD_MAX_F)
    return 0;
  return verify_layout(B, K, V, topf_F_max).total;
}

}  // extern "C"

// Both verify entry points: every argument is validated before any HIP call. `noalloc_flags`
// non-null selects the allocation-free variant: the workspace is the library's static array of the
// current device and the device-error flags go to the caller's word.
static ssd_status verify_impl(const void* draft_logits, int64_t draft_seq_stride, const void* target_logits,
                              int64_t target_seq_stride, ssd_dtype dtype, int B, int K, int V,
                              float temperature, const int32_t* draft_tokens, const float* uniforms,
                              const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                              const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                              int32_t* accepted_len, int32_t* bonus_token, float* accept_prob,
                              float* residual_mass, const ssd_verify_opts* opts, void* workspace,
                              size_t workspace_bytes, uint32_t* noalloc_flags, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_UNSUPPORTED;
  if (B < 0 || B > SSD_MAX_B || K < 1 || K > SSD_MAX_K || V < 1 || V > SSD_MAX_V)
    return SSD_ERR_INVALID_ARG;
  if (!temp_ok(temperature)) return SSD_ERR_INVALID_ARG;
  if (sag_F < 0 || sag_F > SSD_MAX_F || (sag_F > 0 && (!sag_set || !c_ok(sag_C))))
    return SSD_ERR_INVALID_ARG;
  if (sag_F > 0 && sag_C_pos)
    for (int i = 0; i < K; ++i)
      if (!c_ok(sag_C_pos[i])) return SSD_ERR_INVALID_ARG;
  if (topf_F_max < 0 || topf_F_max > SSD_MAX_F || (topf_F_max > 0 && !topf_out))
    return SSD_ERR_INVALID_ARG;
  if (topf_F)
    for (int i = 0; i < K; ++i)
      if (topf_F[i] < 0 || topf_F[i] > topf_F_max) return SSD_ERR_INVALID_ARG;
  int wait_polls = (opts && opts->wait_polls >= 0) ? opts->wait_polls : -1;
  if (wait_polls > (1 << 20)) return SSD_ERR_INVALID_ARG;
  const int lastF = opts ? opts->topf_last_F : 0;
  const int launch_mode = opts ? opts->launch_mode : 0;
  if (launch_mode < 0 || launch_mode > 2) return SSD_ERR_INVALID_ARG;
  if (lastF < 0 || lastF > SSD_MAX_F || (lastF > 0 && !opts->topf_last_out)) return SSD_ERR_INVALID_ARG;
  if (draft_seq_stride < int64_t(lastF > 0 ? K + 1 : K) * V || target_seq_stride < int64_t(K + 1) * V)
    return SSD_ERR_INVALID_ARG;
  if (B == 0) return SSD_OK;
  if (!draft_logits || !target_logits || !draft_tokens || !uniforms || !accepted_len ||
      !bonus_token)
    return SSD_ERR_INVALID_ARG;
  const VerifyLayout L = verify_layout(B, K, V, std::max(topf_F_max, lastF));
  if (noalloc_flags) {
    if (L.total > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_SCRATCH_LIMIT;
    if (noalloc_scratch(&workspace, L.off_stats, stream) != hipSuccess) return SSD_ERR_HIP;
    workspace_bytes = SSD_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws_ok(workspace, workspace_bytes, L.total)) return SSD_ERR_WORKSPACE;

  const bool bf16 = dtype == SSD_BF16;
  const int es = elem_size(dtype);
  const bool aligned = aligned16(draft_logits) && aligned16(target_logits) && (int64_t(V) * es) % 16 == 0 &&
                       (draft_seq_stride * es) % 16 == 0 && (target_seq_stride * es) % 16 == 0;
  const VerifyPlan P = plan_verify(B, K, V, bf16, aligned);
  if (wait_polls < 0) wait_polls = SSD_DEFAULT_WAIT_POLLS;
  VerifyArgs a;
  std::memset(&a, 0, sizeof(a));
  a.draft = draft_logits;
  a.dstride = draft_seq_stride;
  a.target = target_logits;
  a.tstride = target_seq_stride;
  a.B = B;
  a.K = K;
  a.V = V;
  a.T = P.T;
  a.c2 = float(kLog2e / double(temperature));
  a.x = draft_tokens;
  a.u = uniforms;
  a.sset = sag_F > 0 ? sag_set : nullptr;
  a.sF = sag_F;
  for (int i = 0; i < K; ++i) a.Cpos[i] = sag_F > 0 ? (sag_C_pos ? sag_C_pos[i] : sag_C) : 1.f;
  for (int i = 0; i < K; ++i) a.topfF[i] = topf_F ? topf_F[i] : topf_F_max;
  a.topfF[K] = lastF;
  a.topfFmax = topf_F_max;
  a.lastF = lastF;
  a.Fcap = L.Fcap;
  a.topf_out = topf_out;
  a.topf_last_out = lastF > 0 ? opts->topf_last_out : nullptr;
  a.k_out = accepted_len;
  a.bonus_out = bonus_token;
  a.aprob_out = accept_prob;
  a.rmass_out = residual_mass;
  a.flags = noalloc_flags ? noalloc_flags : at<uint32_t>(workspace, 0);
  a.gtag = at<uint32_t>(workspace, 4);
  a.gdone = at<uint32_t>(workspace, 8);
  a.seqctl = at<uint32_t>(workspace, L.off_seqctl);
  a.stats = at<uint64_t>(workspace, L.off_stats);
  a.chunk = at<uint64_t>(workspace, L.off_chunk);
  a.dec = at<uint64_t>(workspace, L.off_dec);
  a.cand = at<uint64_t>(workspace, L.off_cand);
  a.Tcap = L.Tcap;
  a.wait_polls = wait_polls;
  a.aligned = aligned ? 1 : 0;
  a.split = (launch_mode == 2 || (launch_mode == 0 && verify_split(B, P.T))) ? 1 : 0;
  // the streaming form's second grid: about one workgroup per slot, each over a run of tiles
  a.groups = int(std::min<int64_t>(P.T, std::max<int64_t>(1, (verify_slots() + B - 1) / B)));
#ifdef SSD_TRACE
  a.trace = static_cast<uint64_t*>(ssd_trace_buffer);
#endif
  return hip_status(launch_verify(a, P, bf16, stream));
}

extern "C" {

ssd_status ssd_verify_ex(const void* draft_logits, int64_t draft_seq_stride, const void* target_logits,
                         int64_t target_seq_stride, ssd_dtype dtype, int B, int K, int V,
                         float temperature, const int32_t* draft_tokens, const float* uniforms,
                         const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                         const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                         int32_t* accepted_len, int32_t* bonus_token, float* accept_prob,
                         float* residual_mass, const ssd_verify_opts* opts, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return verify_impl(draft_logits, draft_seq_stride, target_logits, target_seq_stride, dtype, B, K, V,
                     temperature, draft_tokens, uniforms, sag_set, sag_F, sag_C, sag_C_pos, topf_F, topf_F_max,
                     topf_out, accepted_len, bonus_token, accept_prob, residual_mass, opts, workspace,
                     workspace_bytes, nullptr, stream);
}

ssd_status ssd_verify_noalloc(const void* draft_logits, int64_t draft_seq_stride, const void* target_logits,
                              int64_t target_seq_stride, ssd_dtype dtype, int B, int K, int V,
                              float temperature, const int32_t* draft_tokens, const float* uniforms,
                              const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                              const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                              int32_t* accepted_len, int32_t* bonus_token, float* accept_prob,
                              float* residual_mass, uint32_t* device_flags, hipStream_t stream) {
  if (!device_flags) return SSD_ERR_INVALID_ARG;
  return verify_impl(draft_logits, draft_seq_stride, target_logits, target_seq_stride, dtype, B, K, V,
                     temperature, draft_tokens, uniforms, sag_set, sag_F, sag_C, sag_C_pos, topf_F, topf_F_max,
                     topf_out, accepted_len, bonus_token, accept_prob, residual_mass, nullptr, nullptr, 0,
                     device_flags, stream);
}

#ifdef SSD_TRACE
// analysis builds only: device buffer of 16 timestamps per verification workgroup
void ssd_set_trace_buffer(void* device_buffer) { ssd_trace_buffer = device_buffer; }
#endif

ssd_status ssd_verify(const void* draft_logits, int64_t draft_seq_stride, const void* target_logits,
                      int64_t target_seq_stride, ssd_dtype dtype, int B, int K, int V,
                      float temperature, const int32_t* draft_tokens, const float* uniforms,
                      const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                      const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                      int32_t* accepted_len, int32_t* bonus_token, float* accept_prob,
                      float* residual_mass, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return ssd_verify_ex(draft_logits, draft_seq_stride, target_logits, target_seq_stride, dtype, B, K, V,
                       temperature, draft_tokens, uniforms, sag_set, sag_F, sag_C, sag_C_pos, topf_F,
                       topf_F_max, topf_out, accepted_len, bonus_token, accept_prob, residual_mass, nullptr,
                       workspace, workspace_bytes, stream);
}

int ssd_verify_launches(int B, int K, int V, ssd_dtype dtype, int topf_F_max) {
  if (!dtype_ok(dtype)) return -1;
  if (B < 0 || B > SSD_MAX_B || K < 1 || K > SSD_MAX_K || V < 1 || V > SSD_MAX_V) return -1;
  if (topf_F_max < 0 || topf_F_max > SSD_MAX_F) return -1;
  if (B == 0) return 0;
  return verify_split(B, plan_verify(B, K, V, dtype == SSD_BF16, true).T) ? 2 : 1;
}

int ssd_verify_tiles(int B, int K, int V, ssd_dtype dtype) {
  if (!dtype_ok(dtype)) return -1;
  if (B < 0 || B > SSD_MAX_B || K < 1 || K > SSD_MAX_K || V < 1 || V > SSD_MAX_V) return -1;
  return plan_verify(B, K, V, dtype == SSD_BF16, true).T;
}

// ------------------------------------------------------------------------------------------------
ssd_status ssd_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!data || !sink || bytes % 16 != 0 || !aligned16(data)) return SSD_ERR_INVALID_ARG;
  if (bytes == 0) return SSD_OK;
  return hip_status(launch_stream_read(data, int64_t(bytes / 16), sink, stream));
}


// ------------------------------------------------------------------------------------------------
size_t ssd_topf_workspace_bytes(int R, int V, int F_max) {
  if (R < 0 || V < 1 || V > SSD_MAX_V || F_max < 1 || F_max > SSD_MAX_F) return 0;
  return topf_layout(R, V, F_max).total;
}

ssd_status ssd_topf_guess(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                          const int32_t* exclude, const int32_t* F_per_row, int F_max,
                          int32_t* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_UNSUPPORTED;
  if (R < 0 || R > (1 << 24) || V < 1 || V > SSD_MAX_V || F_max < 1 || F_max > SSD_MAX_F ||
      row_stride < V)
    return SSD_ERR_INVALID_ARG;
  if (R == 0) return SSD_OK;
  if (!logits || !out) return SSD_ERR_INVALID_ARG;
  const TopfLayout L = topf_layout(R, V, F_max);
  if (!ws_ok(workspace, workspace_bytes, L.total)) return SSD_ERR_WORKSPACE;
  const int es = elem_size(dtype);
  TopfArgs a;
  std::memset(&a, 0, sizeof(a));
  a.logits = logits;
  a.row_stride = row_stride;
  a.R = R;
  a.V = V;
  a.exclude = exclude;
  a.F_per_row = F_per_row;
  a.Fmax = F_max;
  a.out = out;
  a.flags = at<uint32_t>(workspace, 0);
  a.cand = at<void>(workspace, L.off_cand);
  a.n1 = L.rp.n1;
  a.chunk1 = L.rp.chunk1;
  a.aligned = aligned16(logits) && (row_stride * es) % 16 == 0;
  return hip_status(launch_topf(a, dtype == SSD_BF16, stream));
}

// ------------------------------------------------------------------------------------------------
size_t ssd_saguaro_topf_workspace_bytes(int R, int V, int F_max) {
  if (R < 0 || V < 1 || V > SSD_MAX_V || F_max < 1 || F_max > SSD_MAX_F) return 0;
  return topf_layout(R, V, F_max).total;
}

ssd_status ssd_saguaro_topf(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                            float temperature, const int32_t* F_per_row, int F_max, float C,
                            const float* C_per_row, int32_t* out_set, float* out_set_mass,
                            float* out_norm, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_UNSUPPORTED;
  if (R < 0 || R > (1 << 24) || V < 1 || V > SSD_MAX_V || F_max < 1 || F_max > SSD_MAX_F ||
      row_stride < V || !temp_ok(temperature) || !c_ok(C))
    return SSD_ERR_INVALID_ARG;
  if (R == 0) return SSD_OK;
  if (!logits || !out_set) return SSD_ERR_INVALID_ARG;
  const TopfLayout L = topf_layout(R, V, F_max);
  if (!ws_ok(workspace, workspace_bytes, L.total)) return SSD_ERR_WORKSPACE;
  const int es = elem_size(dtype);
  TopfArgs a;
  std::memset(&a, 0, sizeof(a));
  a.logits = logits;
  a.row_stride = row_stride;
  a.R = R;
  a.V = V;
  a.exclude = nullptr;
  a.F_per_row = F_per_row;
  a.Fmax = F_max;
  a.out = out_set;
  a.flags = at<uint32_t>(workspace, 0);
  a.cand = at<void>(workspace, L.off_cand);
  a.n1 = L.rp.n1;
  a.chunk1 = L.rp.chunk1;
  a.aligned = aligned16(logits) && (row_stride * es) % 16 == 0;
  a.sag = 1;
  a.c2 = float(kLog2e / double(temperature));
  a.C = C;
  a.C_per_row = C_per_row;
  a.stats = at<float2>(workspace, L.off_stats);
  a.out_set_mass = out_set_mass;
  a.out_norm = out_norm;
  return hip_status(launch_topf(a, dtype == SSD_BF16, stream));
}

// ------------------------------------------------------------------------------------------------
size_t ssd_saguaro_sample_workspace_bytes(int R, int V, int F_max) {
  if (R < 0 || V < 1 || V > SSD_MAX_V || F_max < 0 || F_max > SSD_MAX_F) return 0;
  return sample_layout(R, V, F_max).total;
}

ssd_status ssd_saguaro_sample(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                              float temperature, const int32_t* F_per_row, int F_max, float C,
                              const float* C_per_row, const float* u, int32_t* out_token,
                              float* out_prob, int32_t* out_set, float* out_set_mass, float* out_norm,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_UNSUPPORTED;
  if (R < 0 || R > (1 << 24) || V < 1 || V > SSD_MAX_V || F_max < 0 || F_max > SSD_MAX_F ||
      row_stride < V || !temp_ok(temperature) || !c_ok(C))
    return SSD_ERR_INVALID_ARG;
  if (R == 0) return SSD_OK;
  if (!logits || !u || !out_token || (F_max > 0 && !out_set)) return SSD_ERR_INVALID_ARG;
  const SampleLayout L = sample_layout(R, V, F_max);
  if ((V + int64_t(L.seg_len) - 1) / L.seg_len > 256) return SSD_ERR_INVALID_ARG;  // not reached for V <= SSD_MAX_V
  if (!ws_ok(workspace, workspace_bytes, L.total)) return SSD_ERR_WORKSPACE;
  const int es = elem_size(dtype);
  TopfArgs a;
  std::memset(&a, 0, sizeof(a));
  a.logits = logits;
  a.row_stride = row_stride;
  a.R = R;
  a.V = V;
  a.exclude = nullptr;
  a.F_per_row = F_max > 0 ? F_per_row : nullptr;
  a.Fmax = F_max;
  a.out = out_set;
  a.flags = at<uint32_t>(workspace, 0);
  a.cand = at<void>(workspace, L.t.off_cand);
  a.n1 = L.t.rp.n1;
  a.chunk1 = L.t.rp.chunk1;
  a.aligned = aligned16(logits) && (row_stride * es) % 16 == 0;
  a.sag = 1;
  a.c2 = float(kLog2e / double(temperature));
  a.C = C;
  a.C_per_row = C_per_row;
  a.stats = at<float2>(workspace, L.t.off_stats);
  a.out_set_mass = out_set_mass;
  a.out_norm = out_norm;
  a.u = u;
  a.out_token = out_token;
  a.out_prob = out_prob;
  a.seg_len = L.seg_len;
  a.nseg = L.nseg;
  a.seg = at<float2>(workspace, L.off_seg);
  return hip_status(launch_topf(a, dtype == SSD_BF16, stream));
}

// ------------------------------------------------------------------------------------------------
size_t ssd_saguaro_workspace_bytes(int R, int V) {
  if (R < 0 || V < 1 || V > SSD_MAX_V) return 0;
  return saguaro_layout(R, V).total;
}

ssd_status ssd_saguaro_adjust(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                              float temperature, const int32_t* set, int F, float C,
                              const float* C_per_row, float* out_probs, float* out_set_mass,
                              float* out_norm, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_UNSUPPORTED;
  if (R < 0 || R > 65535 || V < 1 || V > SSD_MAX_V || row_stride < V || !temp_ok(temperature) ||
      F < 0 || F > SSD_MAX_F || (F > 0 && !set) || !c_ok(C))
    return SSD_ERR_INVALID_ARG;
  if (R == 0) return SSD_OK;
  if (!logits) return SSD_ERR_INVALID_ARG;
  const SaguaroLayout L = saguaro_layout(R, V);
  if (!ws_ok(workspace, workspace_bytes, L.total)) return SSD_ERR_WORKSPACE;
  const int es = elem_size(dtype);
  SagArgs a;
  std::memset(&a, 0, sizeof(a));
  a.logits = logits;
  a.row_stride = row_stride;
  a.R = R;
  a.V = V;
  a.c2 = float(kLog2e / double(temperature));
  a.set = set;
  a.F = F;
  a.C = C;
  a.C_per_row = C_per_row;
  a.out_probs = out_probs;
  a.out_set_mass = out_set_mass;
  a.out_norm = out_norm;
  a.flags = at<uint32_t>(workspace, 0);
  a.stats = at<float2>(workspace, L.off_stats);
  a.n1 = L.rp.n1;
  a.chunk1 = L.rp.chunk1;
  a.n_out = L.n_out;
  a.chunk_out = L.chunk_out;
  a.aligned = aligned16(logits) && (row_stride * es) % 16 == 0;
  a.out_aligned = out_probs && aligned16(out_probs) && V % 4 == 0;
  return hip_status(launch_saguaro(a, dtype == SSD_BF16, stream));
}

// ------------------------------------------------------------------------------------------------
ssd_status ssd_fanout_alloc(int K, double a, double r, int budget, int32_t* out_F,
                            double* out_F_cont) {
  if (K < 0 || K > 4096 || !(a > 0.0 && a < 1.0) || !(r > 0.0) || !std::isfinite(r) ||
      budget < 0 || !out_F)
    return SSD_ERR_INVALID_ARG;
  // P(k): geometric acceptance law; F_k / F_0 = (P(k) / P(0))^(1/(1+r)) from the stationarity of
  // the Lagrangian of sum_k P(k) F_k^-r + lambda (sum_k F_k - budget).
  std::vector<double> w(K + 1);
  double total = 0.0;
  for (int k = 0; k <= K; ++k) {
    const double Pk = (k < K) ? (1.0 - a) * std::pow(a, k) : std::pow(a, K);
    const double P0 = (K > 0) ? (1.0 - a) : 1.0;
    w[k] = std::pow(Pk / P0, 1.0 / (1.0 + r));
    total += w[k];
  }
  std::vector<double> frac(K + 1);
  int64_t used = 0;
  for (int k = 0; k <= K; ++k) {
    const double f = double(budget) * w[k] / total;
    if (out_F_cont) out_F_cont[k] = f;
    const double fl = std::floor(f);
    out_F[k] = int32_t(fl);
    frac[k] = f - fl;
    used += out_F[k];
  }
  // largest remainders first, ties to the smaller k
  for (int64_t left = budget - used; left > 0; --left) {
    int best = -1;
    for (int k = 0; k <= K; ++k)
      if (frac[k] >= 0.0 && (best < 0 || frac[k] > frac[best])) best = k;
    if (best < 0) break;
    out_F[best] += 1;
    frac[best] = -1.0;
  }
  return SSD_OK;
}

// ------------------------------------------------------------------------------------------------
namespace {
bool speed_args_ok(double h, double E_hit, double E_miss, double T_p, double T_b) {
  return h >= 0.0 && h <= 1.0 && E_hit >= 0.0 && E_miss >= 0.0 && T_p >= 0.0 && T_b >= 0.0 &&
         std::isfinite(E_hit) && std::isfinite(E_miss) && std::isfinite(T_p) && std::isfinite(T_b);
}
// tokens per round (A) and the round's time (D + miss wait) of one backup choice
double round_tokens(double h, double E_hit, double E_miss) { return h * E_hit + (1.0 - h) * E_miss; }
}  // namespace

ssd_status ssd_batch_speedup(double h, double E_hit, double E_miss, double T_p, double T_b, int b,
                             double* out_speedup) {
  if (!speed_args_ok(h, E_hit, E_miss, T_p, T_b) || b < 1 || !out_speedup) return SSD_ERR_INVALID_ARG;
  const double wait = (1.0 - std::pow(h, double(b))) * T_b;  // the batch waits unless all b hit
  *out_speedup = round_tokens(h, E_hit, E_miss) / (std::max(1.0, T_p) + wait);
  return SSD_OK;
}

ssd_status ssd_backup_crossover(double h, double E_hit, double E_miss_neural, double T_neural,
                                double E_miss_fast, double T_fast, double T_p, double* out_b_star,
                                int32_t* out_fast_wins_large) {
  if (!speed_args_ok(h, E_hit, E_miss_neural, T_p, T_neural) ||
      !speed_args_ok(h, E_hit, E_miss_fast, T_p, T_fast) || !out_b_star)
    return SSD_ERR_INVALID_ARG;
  const double D = std::max(1.0, T_p);
  const double An = round_tokens(h, E_hit, E_miss_neural), Af = round_tokens(h, E_hit, E_miss_fast);
  // the speedups are An / (D + x T_neural) and Af / (D + x T_fast) with x = 1 - h^b in (0, 1): one
  // linear equation in x
  if (out_fast_wins_large) *out_fast_wins_large = (Af * (D + T_neural) >= An * (D + T_fast)) ? 1 : 0;
  const double slope = Af * T_neural - An * T_fast;
  *out_b_star = std::nan("");
  if (slope == 0.0 || !(h > 0.0 && h < 1.0)) return SSD_OK;
  const double x = D * (An - Af) / slope;
  if (x > 0.0 && x < 1.0) *out_b_star = std::log1p(-x) / std::log(h);
  return SSD_OK;
}

// ------------------------------------------------------------------------------------------------
}  // extern "C"

// The keys' arguments, checked and packed (SSD_OK also for an empty batch or budget, with a.B or
// a.budget 0: nothing to launch).
static ssd_status keys_args(int B, int K, int G_max, const int32_t* guesses, const int32_t* guesses_last,
                            int G_last, const int32_t* fanout, int budget, int32_t* cache_k, int32_t* cache_tok,
                            CacheKeysArgs& a) {
  std::memset(&a, 0, sizeof(a));
  if (B < 0 || B > SSD_MAX_B || K < 1 || K > SSD_MAX_K || G_max < 1 || G_max > SSD_MAX_F ||
      budget < 0 || !fanout || (guesses_last && (G_last < 1 || G_last > SSD_MAX_F)))
    return SSD_ERR_INVALID_ARG;
  int64_t off = 0;
  for (int k = 0; k <= K; ++k) {
    const int width = (guesses_last && k == K) ? G_last : G_max;
    if (fanout[k] < 0 || fanout[k] > width) return SSD_ERR_INVALID_ARG;
    a.off[k] = int(off);
    off += fanout[k];
  }
  if (off != budget) return SSD_ERR_INVALID_ARG;
  a.off[K + 1] = budget;
  if (B == 0 || budget == 0) return SSD_OK;
  if (!guesses || !cache_k || !cache_tok) return SSD_ERR_INVALID_ARG;
  a.B = B;
  a.K = K;
  a.Gmax = G_max;
  a.budget = budget;
  a.guesses = guesses;
  a.last = guesses_last;
  a.Glast = G_last;
  a.cache_k = cache_k;
  a.cache_tok = cache_tok;
  return SSD_OK;
}

extern "C" {

ssd_status ssd_cache_keys(int B, int K, int G_max, const int32_t* guesses, const int32_t* guesses_last,
                          int G_last, const int32_t* fanout, int budget, int32_t* cache_k,
                          int32_t* cache_tok, hipStream_t stream) {
  CacheKeysArgs a;
  const ssd_status st = keys_args(B, K, G_max, guesses, guesses_last, G_last, fanout, budget, cache_k, cache_tok, a);
  if (st != SSD_OK || a.B == 0 || a.budget == 0) return st;
  return hip_status(launch_cache_keys(a, stream));
}

ssd_status ssd_cache_keys_lookup(int B, int K, int G_max, const int32_t* guesses, const int32_t* guesses_last,
                                 int G_last, const int32_t* fanout, int budget, const int32_t* accepted_len,
                                 const int32_t* bonus_token, int32_t* cache_k, int32_t* cache_tok,
                                 int32_t* out_slot, int32_t* out_miss_count, hipStream_t stream) {
  CacheKeysArgs ka;
  const ssd_status st = keys_args(B, K, G_max, guesses, guesses_last, G_last, fanout, budget, cache_k, cache_tok, ka);
  if (st != SSD_OK) return st;
  if (!out_miss_count || (B > 0 && (!accepted_len || !bonus_token || !out_slot))) return SSD_ERR_INVALID_ARG;
  CacheLookupArgs la;
  std::memset(&la, 0, sizeof(la));
  la.B = B;
  la.budget = budget;
  la.cache_k = cache_k;
  la.cache_tok = cache_tok;
  la.k = accepted_len;
  la.tok = bonus_token;
  la.out_slot = out_slot;
  la.out_miss = out_miss_count;
  ka.B = B;  // an empty budget still writes every slot -1 and the miss count
  ka.budget = budget;
  return hip_status(launch_cache_keys_lookup(ka, la, stream));
}

ssd_status ssd_cache_lookup(int B, int budget, const int32_t* cache_k, const int32_t* cache_tok,
                            const int32_t* accepted_len, const int32_t* bonus_token,
                            int32_t* out_slot, int32_t* out_miss_count, hipStream_t stream) {
  if (B < 0 || B > SSD_MAX_B || budget < 0 || !out_miss_count) return SSD_ERR_INVALID_ARG;
  if (B > 0 && (!accepted_len || !bonus_token || !out_slot)) return SSD_ERR_INVALID_ARG;
  if (B > 0 && budget > 0 && (!cache_k || !cache_tok)) return SSD_ERR_INVALID_ARG;
  CacheLookupArgs a;
  a.B = B;
  a.budget = budget;
  a.cache_k = cache_k;
  a.cache_tok = cache_tok;
  a.k = accepted_len;
  a.tok = bonus_token;
  a.out_slot = out_slot;
  a.out_miss = out_miss_count;
  return hip_status(launch_cache_lookup(a, stream));
}

// ------------------------------------------------------------------------------------------------
ssd_status ssd_read_flags(void* workspace, uint32_t* out_flags, int clear, hipStream_t stream) {
  if (!workspace || !out_flags) return SSD_ERR_INVALID_ARG;
  uint32_t host = 0;
  if (hipMemcpyAsync(&host, workspace, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return SSD_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SSD_ERR_HIP;
  *out_flags = host;
  if (clear) return hip_status(launch_clear_flags(static_cast<uint32_t*>(workspace), stream));
  return SSD_OK;
}

}  // extern "C"
