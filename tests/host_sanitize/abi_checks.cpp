// Host-side checks of the C ABI built with AddressSanitizer and UndefinedBehaviorSanitizer: every
// device entry point is called with arguments its validation rejects (so no launch is reached: the
// launchers below abort if one is), and the host-only entry points and workspace helpers run over
// sweeps up to the largest supported shapes. Exit status 0 and "abi checks ok" on success.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ssd.h"
#include "ssd_launch.hpp"

// The device side is not linked: reaching any of these means a validation let a bad call through.
namespace ssd {
[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "launch reached: %s\n", what);
  std::abort();
}
hipError_t launch_verify(const VerifyArgs&, const VerifyPlan&, bool, hipStream_t) { reached("verify"); }
hipError_t noalloc_scratch(void**, size_t, hipStream_t) { reached("noalloc scratch"); }
hipError_t launch_stream_read(const void*, int64_t, uint32_t*, hipStream_t) { reached("stream read"); }
hipError_t launch_topf(const TopfArgs&, bool, hipStream_t) { reached("topf"); }
hipError_t launch_saguaro(const SagArgs&, bool, hipStream_t) { reached("saguaro"); }
hipError_t launch_cache_keys(const CacheKeysArgs&, hipStream_t) { reached("cache keys"); }
hipError_t launch_cache_lookup(const CacheLookupArgs&, hipStream_t) { reached("cache lookup"); }
hipError_t launch_cache_keys_lookup(const CacheKeysArgs&, const CacheLookupArgs&, hipStream_t) { reached("keys lookup"); }
hipError_t launch_clear_flags(uint32_t*, hipStream_t) { reached("clear flags"); }
}  // namespace ssd

static int failures = 0;
#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

// a pointer that validation may test for null but must never dereference
static void* const FAKE = reinterpret_cast<void*>(0x1000);
template <class T>
static T* fk() { return static_cast<T*>(FAKE); }

static ssd_status verify(int B, int K, int V, ssd_dtype dt, float T, int64_t ds, int64_t ts, int sF, float C,
                         const int32_t* topfF, int Fmax, bool out_null = false, const ssd_verify_opts* o = nullptr) {
  return ssd_verify_ex(FAKE, ds, FAKE, ts, dt, B, K, V, T, fk<int32_t>(), fk<float>(), sF ? fk<int32_t>() : nullptr, sF, C,
                       nullptr, topfF, Fmax, Fmax ? fk<int32_t>() : nullptr, out_null ? nullptr : fk<int32_t>(),
                       fk<int32_t>(), nullptr, nullptr, o, nullptr, 0, nullptr);
}

int main() {
  // status strings
  for (int s = 0; s <= 5; ++s) EXPECT(std::strlen(ssd_status_string(ssd_status(s))) > 0);
  EXPECT(std::strcmp(ssd_status_string(ssd_status(99)), "unknown status") == 0);

  // verification: every bad argument, each on an otherwise valid call whose workspace is missing
  const int K = 4, V = 1000;
  const int64_t ds = int64_t(K) * V, ts = int64_t(K + 1) * V;
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0) == SSD_ERR_WORKSPACE);
  EXPECT(verify(2, K, V, ssd_dtype(7), 1.f, ds, ts, 0, 1.f, nullptr, 0) == SSD_ERR_UNSUPPORTED);
  for (int B : {-1, SSD_MAX_B + 1}) EXPECT(verify(B, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  for (int k : {0, SSD_MAX_K + 1}) EXPECT(verify(2, k, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  for (int v : {0, SSD_MAX_V + 1}) EXPECT(verify(2, K, v, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  for (float T : {0.f, -1.f, NAN, INFINITY}) EXPECT(verify(2, K, V, SSD_F32, T, ds, ts, 0, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  for (float C : {-0.1f, 1.5f, NAN}) EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 3, C, nullptr, 0) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, SSD_MAX_F + 1, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, SSD_MAX_F + 1) == SSD_ERR_INVALID_ARG);
  const int32_t badF[4] = {1, 2, 9, 0};
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, badF, 3) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds - 1, ts, 0, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts - 1, 0, 1.f, nullptr, 0) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0, true) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(0, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0) == SSD_OK);  // empty batch
  ssd_verify_opts o{1 << 21, 0, nullptr};
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0, false, &o) == SSD_ERR_INVALID_ARG);
  o = ssd_verify_opts{-1, 3, nullptr};  // extra-row guesses without an output
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0, false, &o) == SSD_ERR_INVALID_ARG);
  o = ssd_verify_opts{-1, 3, fk<int32_t>()};  // ... or without draft row K in the stride
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds, ts, 0, 1.f, nullptr, 0, false, &o) == SSD_ERR_INVALID_ARG);
  EXPECT(verify(2, K, V, SSD_F32, 1.f, ds + V, ts, 0, 1.f, nullptr, 0, false, &o) == SSD_ERR_WORKSPACE);

  // the allocation-free form: past its array before any HIP call, and a null flags word
  EXPECT(ssd_verify_noalloc(FAKE, int64_t(16) << 20, FAKE, int64_t(17) << 20, SSD_F32, 4096, 16, 1 << 20, 1.f,
                            fk<int32_t>(), fk<float>(), nullptr, 0, 1.f, nullptr, nullptr, 0, nullptr, fk<int32_t>(),
                            fk<int32_t>(), nullptr, nullptr, fk<uint32_t>(), nullptr) == SSD_ERR_SCRATCH_LIMIT);
  EXPECT(ssd_verify_noalloc(FAKE, ds, FAKE, ts, SSD_F32, 2, K, V, 1.f, fk<int32_t>(), fk<float>(), nullptr, 0, 1.f,
                            nullptr, nullptr, 0, nullptr, fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr,
                            nullptr) == SSD_ERR_INVALID_ARG);

  // workspace sizes over a sweep up to the largest shapes: defined, growing with B, and 0 when rejected
  for (int k : {1, 4, 8, 16})
    for (int v : {1, 7, 1023, 1024, 128256, 152064, 1 << 20})
      for (int f : {0, 3, 16}) {
        size_t last = 0;
        for (int b : {0, 1, 16, 128, 4096, SSD_MAX_B}) {
          const size_t w = ssd_verify_workspace_bytes(b, k, v, f);
          EXPECT(w > 0 && w >= last);
          last = w;
        }
        EXPECT(ssd_verify_tiles(16, k, v, SSD_BF16) >= 1 && ssd_verify_tiles(1, k, v, SSD_F32) >= 1);
        // two launches once the tiles exceed what 256 CUs run at once (2 each; no device answers here)
        const int want = 16 * ssd_verify_tiles(16, k, v, SSD_BF16) > 512 ? 2 : 1;
        EXPECT(ssd_verify_launches(16, k, v, SSD_BF16, f) == want && ssd_verify_launches(0, k, v, SSD_F32, f) == 0);
      }
  EXPECT(ssd_verify_workspace_bytes(-1, 4, 10, 0) == 0 && ssd_verify_workspace_bytes(1, 4, 10, 17) == 0);
  for (int r : {1, 16, 768, 8192, 100000})
    for (int v : {1, 5003, 128256, 1 << 20})
      for (int f : {0, 1, 16}) {
        EXPECT(ssd_topf_workspace_bytes(r, v, f) > 0 || f == 0);
        EXPECT((ssd_saguaro_topf_workspace_bytes(r, v, f) > 0) == (f > 0));  // a set needs F >= 1
        EXPECT(ssd_saguaro_sample_workspace_bytes(r, v, f) > 0);
        EXPECT(ssd_saguaro_workspace_bytes(r, v) > 0);
      }

  // standalone kernels: rejected before a launch
  EXPECT(ssd_topf_guess(FAKE, 100, SSD_F32, 2, 100, nullptr, nullptr, SSD_MAX_F + 1, fk<int32_t>(), nullptr, 0, nullptr) ==
         SSD_ERR_INVALID_ARG);
  EXPECT(ssd_topf_guess(FAKE, 99, SSD_F32, 2, 100, nullptr, nullptr, 3, fk<int32_t>(), nullptr, 0, nullptr) ==
         SSD_ERR_INVALID_ARG);
  EXPECT(ssd_topf_guess(FAKE, 100, SSD_F32, 2, 100, nullptr, nullptr, 3, fk<int32_t>(), nullptr, 0, nullptr) ==
         SSD_ERR_WORKSPACE);
  EXPECT(ssd_saguaro_adjust(FAKE, 100, SSD_F32, 2, 100, 0.f, nullptr, 0, 1.f, nullptr, nullptr, fk<float>(), fk<float>(),
                            nullptr, 0, nullptr) == SSD_ERR_INVALID_ARG);
  EXPECT(ssd_saguaro_topf(FAKE, 100, SSD_F32, 2, 100, 1.f, nullptr, 3, 2.f, nullptr, fk<int32_t>(), fk<float>(),
                          fk<float>(), nullptr, 0, nullptr) == SSD_ERR_INVALID_ARG);
  EXPECT(ssd_saguaro_sample(FAKE, 100, SSD_F32, 2, 100, 1.f, nullptr, 3, 0.5f, nullptr, nullptr, fk<int32_t>(),
                            fk<float>(), fk<int32_t>(), fk<float>(), fk<float>(), nullptr, 0, nullptr) == SSD_ERR_INVALID_ARG);
  EXPECT(ssd_stream_read(nullptr, 1024, fk<uint32_t>(), nullptr) == SSD_ERR_INVALID_ARG);
  EXPECT(ssd_read_flags(nullptr, fk<uint32_t>(), 1, nullptr) == SSD_ERR_INVALID_ARG);

  // cache keys and lookup
  const int32_t fan[5] = {3, 2, 2, 2, 3};
  EXPECT(ssd_cache_keys(2, 4, 3, fk<int32_t>(), nullptr, 0, fan, 11, fk<int32_t>(), fk<int32_t>(),
                        nullptr) == SSD_ERR_INVALID_ARG);  // budget != sum
  EXPECT(ssd_cache_keys(2, 4, 2, fk<int32_t>(), nullptr, 0, fan, 12, fk<int32_t>(), fk<int32_t>(), nullptr) ==
         SSD_ERR_INVALID_ARG);  // F_0 = 3 > G_max
  EXPECT(ssd_cache_lookup(-1, 12, nullptr, nullptr, nullptr, nullptr, nullptr, fk<int32_t>(), nullptr) ==
         SSD_ERR_INVALID_ARG);
  EXPECT(ssd_cache_keys_lookup(2, 4, 3, fk<int32_t>(), nullptr, 0, fan, 12, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(),
                               fk<int32_t>(), fk<int32_t>(), nullptr, nullptr) == SSD_ERR_INVALID_ARG);

  // host-only entry points over grids of arguments
  for (int k = 1; k <= SSD_MAX_K; ++k)
    for (double a : {0.0, 0.3, 0.7, 0.95, 1.0})
      for (double r : {0.0, 0.5, 1.0, 3.0})
        for (int budget : {0, 1, 12, 32, 1000}) {
          std::vector<int32_t> F(k + 1);
          std::vector<double> Fc(k + 1);
          const ssd_status s = ssd_fanout_alloc(k, a, r, budget, F.data(), Fc.data());
          if (s == SSD_OK) {
            int sum = 0;
            for (int i = 0; i <= k; ++i) sum += F[i];
            EXPECT(sum == budget);
          }
        }
  EXPECT(ssd_fanout_alloc(0, 0.5, 1.0, 12, nullptr, nullptr) == SSD_ERR_INVALID_ARG);
  for (double h : {0.0, 0.5, 0.92, 1.0})
    for (int b : {1, 24, 1000000}) {
      double S = 0;
      EXPECT(ssd_batch_speedup(h, 4.0, 2.0, 0.5, 1.0, b, &S) == SSD_OK && std::isfinite(S) && S > 0);
    }
  double S = 0;
  EXPECT(ssd_batch_speedup(1.5, 4.0, 2.0, 0.5, 1.0, 4, &S) == SSD_ERR_INVALID_ARG);
  double bs = 0;
  int32_t fast = -1;
  EXPECT(ssd_backup_crossover(0.9, 4.0, 3.0, 1.0, 1.2, 0.05, 0.5, &bs, &fast) == SSD_OK);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi checks ok\n");
  return 0;
}
