// Kernel argument blocks and launchers (internal to the library). Arguments are passed by value
// as one kernarg struct per launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr int kStreamReadGrid = 8192;  // workgroups of ssd_stream_read (its sink holds one word each)


struct VerifyArgs {
  const void* draft;
  int64_t dstride;  // elements between consecutive sequences
  const void* target;
  int64_t tstride;
  int B, K, V;
  int T;     // tiles per row (of 256 * NV * 16 / sizeof(element) tokens)
  float c2;  // log2(e) / T
  const int32_t* x;
  const float* u;
  const int32_t* sset;
  int sF;
  float Cpos[16];  // Saguaro factor per draft position
  int topfF[17];   // guesses per draft row; [K]: the extra draft row K (no exclusion)
  int topfFmax;    // width of topf_out rows (0: no guesses of rows 0..K-1)
  int lastF;       // guesses of draft row K (0: none)
  int Fcap;        // guesses per row and tile the candidate region holds
  int32_t* topf_out;
  int32_t* topf_last_out;
  int32_t* k_out;
  int32_t* bonus_out;
  float* aprob_out;
  float* rmass_out;
  // workspace views
  uint32_t* flags;   // sticky device-error flags
  uint32_t* gtag;    // the last call's tag
  uint32_t* gdone;   // sequences finished by the running call
  uint32_t* seqctl;  // [kSeqCtlMax][kPlanSeqCtlWords] arrivals (word 0)
  uint64_t* stats;   // [B][2K+1][Tcap][2]
  uint64_t* chunk;   // [B][Tcap][2] claim word, mass word
  uint64_t* dec;     // [B][kPlanDecWords] decision record
  uint64_t* cand;    // [B][K+1][Tcap][Fcap][2]
  int Tcap;
  int wait_polls;    // polls a workgroup spends waiting on the others of its sequence
  int aligned;       // every logit row starts 16-byte aligned
  int split;         // the streaming form: statistics and guesses, then decision, residual and bonus
  int groups;        // the streaming form: workgroups per sequence of its second grid
  uint64_t* trace;   // per-workgroup phase timestamps (analysis builds only), or null
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

// tiles per row and the kernel variant a call takes (the same plan for sizing and launching)
struct VerifyPlan {
  int KM;   // register rows per tile: 2 KM + 1 (KM = 4, 8 or 16)
  int NV;   // 16-byte chunks per lane and row (1 or 2)
  int T;    // tiles per row
  bool AL;  // every row 16-byte aligned (vector loads)
};
constexpr int kVerifyThreads = 256;  // threads of a verification workgroup
constexpr int kVerifyWgPerCu = 2;    // verification workgroups a CU runs at once (register budget)
constexpr int kStreamWgPerCu = 3;    // the same for the streaming form's first grid
constexpr int kResidWgPerCu = 2;     // and for its second grid (residual masses, draw, guess merge)
inline VerifyPlan plan_verify(int B, int K, int V, bool bf16, bool aligned) {
  VerifyPlan p;
  p.AL = aligned;
  p.KM = (K <= 4) ? 4 : (K <= 8 ? 8 : 16);
  // two chunks per lane and row keep 2 KM + 1 rows in at most 136 registers (one chunk for 33
  // rows, for 17 rows of bf16, whose two chunks would spill, and for rows not 16-byte aligned,
  // whose element loads hold a register per token in flight); a batch that would not give every CU
  // a workgroup takes one chunk (twice the tiles)
  p.NV = (!aligned || p.KM == 16 || (p.KM == 8 && bf16)) ? 1 : 2;
  const int es = bf16 ? 2 : 4;
  auto tiles = [&](int nv) { return int((int64_t(V) + kVerifyThreads * nv * (16 / es) - 1) / (kVerifyThreads * nv * (16 / es))); };
  if (p.NV == 2 && int64_t(B) * tiles(2) < 256) p.NV = 1;
  p.T = tiles(p.NV);
  return p;
}
hipError_t launch_verify(const VerifyArgs& a, const VerifyPlan& p, bool bf16, hipStream_t st);
// Device address of the allocation-free verification's static array on the current device; the
// first call on a device looks it up and clears its first ctrl_bytes with a fill kernel on st.
hipError_t noalloc_scratch(void** out, size_t ctrl_bytes, hipStream_t st);
hipError_t launch_stream_read(const void* p, int64_t n16, uint32_t* out, hipStream_t st);
hipError_t launch_topf(const TopfArgs& a, bool bf16, hipStream_t st);  // also ssd_saguaro_topf (a.sag)
hipError_t launch_saguaro(const SagArgs& a, bool bf16, hipStream_t st);
hipError_t launch_cache_keys(const CacheKeysArgs& a, hipStream_t st);
hipError_t launch_cache_lookup(const CacheLookupArgs& a, hipStream_t st);
hipError_t launch_cache_keys_lookup(const CacheKeysArgs& ka, const CacheLookupArgs& la, hipStream_t st);
hipError_t launch_clear_flags(uint32_t* flags, hipStream_t st);

}  // namespace ssd
