// Kernel argument blocks and launchers (internal to the library). Arguments are passed by value
// as one kernarg struct per launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {


struct VerifyArgs {
  const void* draft;
  int64_t dstride;  // elements between consecutive sequences
  const void* target;
  int64_t tstride;
  int B, K, V;
  int b0;    // first sequence of this launch
  int T;     // 4096-token tiles per row
  float c2;  // log2(e) / T
  const int32_t* x;
  const float* u;
  const int32_t* sset;
  int sF;
  float Cpos[16];  // Saguaro factor per draft position
  int topfF[16];
  int topfFmax;
  int32_t* topf_out;
  int32_t* k_out;
  int32_t* bonus_out;
  float* aprob_out;
  float* rmass_out;
  // workspace views
  uint32_t* flags;
  uint32_t* ctl;     // per sequence, 64 words: the last call's tag
  uint64_t* dec;     // per sequence, 32 tagged words: the decision record (k, log-normalisers, set)
  uint64_t* stats;   // [B][2K+1][T][2] tagged max c and sum per tile
  uint64_t* cand;    // [B][K][T][topfFmax][2] candidate keys per tile, two tagged halves each
  uint64_t* res;     // [B][T] residual mass per tile, tagged with the call
  int spin_limit;
  int aligned;  // every logit row starts 16-byte aligned
  uint64_t* trace;  // per-workgroup phase timestamps (analysis builds only), or null
};

struct TopfArgs {
  const void* logits;
  int64_t row_stride;
  int R, V;
  const int32_t* exclude;
  const int32_t* F_per_row;
  int Fmax;
  int32_t* out;
  uint32_t* flags;
  void* cand;
  int n1, chunk1;
  int aligned;
  // Saguaro over the row's own top-F set (ssd_saguaro_topf): row statistics in the same pass
  int sag;           // 0: top-F only
  float c2, C;       // log2(e) / T, Saguaro scale
  const float* C_per_row;  // device [R] Saguaro scale per row, or null (C)
  float2* stats;     // [R][n1] (max c, sum 2^(z c - max c)) per chunk (when n1 > 1)
  float* out_set_mass;
  float* out_norm;
  // draft-side sampling from q' (ssd_saguaro_sample): one uniform per row
  const float* u;      // device [R], or null: no sampling
  int32_t* out_token;  // [R]
  float* out_prob;     // [R] q' of the sampled token, or null
  int seg_len, nseg;   // tokens per segment (a whole number of 8192-token batches), segments per chunk
  float2* seg;         // [R][n1 * nseg] (max c, sum) per segment (when n1 > 1)
};

struct SagArgs {
  const void* logits;
  int64_t row_stride;
  int R, V;
  float c2;
  const int32_t* set;
  int F;
  float C;
  const float* C_per_row;  // device [R] Saguaro scale per row, or null (C)
  float* out_probs;
  float* out_set_mass;
  float* out_norm;
  uint32_t* flags;
  float2* stats;
  int n1, chunk1;
  int n_out, chunk_out;
  int aligned;
  int out_aligned;
};

struct CacheKeysArgs {
  int B, K, Gmax, budget;
  const int32_t* guesses;  // [B, K+1, Gmax], or [B, K, Gmax] with last
  const int32_t* last;     // [B, Glast] position K's guesses, or null
  int Glast;
  int off[18];  // slot offset of each position k (prefix sums of the fan-out), off[K+1] = budget
  int32_t* cache_k;
  int32_t* cache_tok;
};

struct CacheLookupArgs {
  int B, budget;
  const int32_t* cache_k;
  const int32_t* cache_tok;
  const int32_t* k;
  const int32_t* tok;
  int32_t* out_slot;
  int32_t* out_miss;
};

hipError_t launch_verify(const VerifyArgs& a, bool bf16, hipStream_t st);
// kernel launches launch_verify issues for these arguments on the current device (-1 on error)
int count_verify_launches(const VerifyArgs& a, bool bf16);
hipError_t launch_topf(const TopfArgs& a, bool bf16, hipStream_t st);  // also ssd_saguaro_topf (a.sag)
hipError_t launch_saguaro(const SagArgs& a, bool bf16, hipStream_t st);
hipError_t launch_cache_keys(const CacheKeysArgs& a, hipStream_t st);
hipError_t launch_cache_lookup(const CacheLookupArgs& a, hipStream_t st);
hipError_t launch_clear_flags(uint32_t* flags, hipStream_t st);

}  // namespace ssd
