/*
 * ssd.h — C ABI of the MI355X (gfx950) library for batched lossless draft verification and the
 * speculative-speculative-decoding (SSD / Saguaro) pieces around it.
 *
 * Sources (page titles):
 *   [SSD]   "论文阅读：Speculative Speculative Decoding — 消除推测解码的最后一个顺序瓶颈"
 *           (xiaohongrsx.github.io/posts/ssd-paper-reading)
 *   [SD7.3] "7.3 Speculative Decoding：投机采样加速" (aiknowledge.cn)
 *   [HW]    "推测解码：用一个“小模型”骗出 3 倍推理速度" (bbs.huaweicloud.com/blogs/510880)
 *
 * Conventions shared by every entry point
 *   - Every device pointer is caller-owned device memory (e.g. a torch tensor's storage). The
 *     library allocates nothing and keeps no state between calls: calls on different streams with
 *     different workspaces are independent.
 *   - Device calls enqueue work on `stream` and return once it is launched; nothing synchronises.
 *   - Arguments are validated on the host before any launch. Any error code means nothing was
 *     launched, except SSD_ERR_HIP (a launch was rejected by the runtime).
 *   - Device data is not validated up front (that would need a synchronisation). Out-of-range
 *     token ids are never dereferenced: the kernel records a flag in the workspace instead (see
 *     ssd_read_flags) and treats the position as rejected.
 *   - Logit rows hold V values of `dtype`, contiguous. Every row must have at least one finite
 *     logit; NaN and +inf logits give undefined results.
 *   - Sizes: 1 <= K <= SSD_MAX_K, 1 <= V <= SSD_MAX_V, 0 <= B <= SSD_MAX_B. A batch of zero rows
 *     or sequences is a successful no-op.
 *   - Workspaces: device memory of at least the size the matching *_workspace_bytes helper
 *     returns, 256-byte aligned, zero-filled before its first use. Its first 4 bytes hold the
 *     sticky device-error flags. ssd_verify keeps counters in it that every call leaves at zero,
 *     and tags every other word it writes with a per-call number, so one workspace serves calls of
 *     any shape (B, K, V, F) in turn, each sized for its own shape, with no re-zeroing. One
 *     workspace serves one call at a time: calls that share a workspace must be ordered on one
 *     stream.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_MAX_K 16
#define SSD_MAX_F 16
#define SSD_MAX_V (1 << 20)
#define SSD_MAX_B 65535

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1,
  SSD_ERR_UNSUPPORTED = 2,
  SSD_ERR_WORKSPACE = 3,
  SSD_ERR_HIP = 4,
  SSD_ERR_SCRATCH_LIMIT = 5 /* the shape needs more than SSD_NOALLOC_SCRATCH_BYTES (ssd_verify_noalloc) */
} ssd_status;

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Device-error flag bits (sticky, OR-ed into the workspace's first word). */
#define SSD_FLAG_BAD_TOKEN 0x1u     /* a draft token id outside [0, V) */
#define SSD_FLAG_SAGUARO_NORM 0x2u  /* Saguaro normaliser N <= 0 (C = 0 with S holding all mass) */
#define SSD_FLAG_BAD_F 0x4u         /* a per-row F outside [0, F_max] (clamped) */
#define SSD_FLAG_TIMEOUT 0x8u       /* a wait on workgroups that had already arrived gave up (never
                                       expected: it means a device fault; the outputs are not valid) */
#define SSD_FLAG_BAD_C 0x10u        /* a per-row Saguaro C outside [0, 1] (clamped; NaN as 1) */

/* ---------------------------------------------------------------------------------------------
 * ssd_verify — one round of verification for B sequences.
 *
 * Defines: [SD7.3] 7.3.2 (steps 3-4) and 7.3.3; [HW] "二、猜 + 验" and "三、接受概率为什么是对的";
 * [SSD] "接受-拒绝机制" and "SSD 的核心思想" (the outcome (k, t)).
 *   q_i = softmax(draft row i / T), p_i = softmax(target row i / T).
 *   With a Saguaro set S_i ([SSD] "Saguaro 优化二"): q'_i = q_i * (C on S_i, 1 elsewhere) / N_i,
 *   N_i = 1 - (1 - C) * sum_{s in S_i} q_i(s); without one, q'_i = q_i.
 *   Position i accepts x_i iff u_i * q'_i(x_i) < p_i(x_i); k = number of leading accepts.
 *   If k < K the bonus token is drawn from r = max(p_k - q'_k, 0) / R, R = sum r, by inverse CDF
 *   with u_K: the first token t (ascending id) whose cumulative r exceeds u_K * R. If k = K it is
 *   drawn the same way from p_K (R = 1). An all-zero residual (rounding only) falls back to p_k.
 *   Optionally, the top-F guesses of every verified draft row ([SSD] "怎么猜奖励 token"): the F
 *   largest raw logits excluding x_i, ties to the smaller id, -1 padded, -inf never returned.
 *
 * Arguments (row (b, i) of a logits array starts at element b * seq_stride + i * V):
 *   draft_logits      device [B, >=K rows, V] of dtype; rows i < K are read. draft_seq_stride >= K*V.
 *   target_logits     device [B, >=K+1 rows, V]; rows i <= K. target_seq_stride >= (K+1)*V.
 *   dtype             SSD_F32 or SSD_BF16 (both arrays).
 *   temperature       T, finite and > 0.
 *   draft_tokens      device int32 [B, K].
 *   uniforms          device fp32 [B, K+1], each in [0, 1); column K samples the bonus.
 *   sag_set, sag_F    device int32 [B, K, sag_F] Saguaro sets (entries < 0, >= V or repeated are
 *                     ignored), or NULL with sag_F = 0. 0 <= sag_F <= SSD_MAX_F.
 *   sag_C             C in [0, 1]; ignored when sag_F = 0.
 *   sag_C_pos         host fp32 [K]: position i down-weights its set by sag_C_pos[i] in [0, 1]
 *                     instead of sag_C (a per-position C, the direction [SSD] "关于逐位置 的思考"
 *                     names; the pages' own C is one value), or NULL (sag_C everywhere). Copied
 *                     at the call. A uniform array gives the bits of the single-value call.
 *   topf_F            host int32 [K]: guesses wanted per draft position (0..topf_F_max), or NULL
 *                     (= topf_F_max everywhere).
 *   topf_F_max        0..SSD_MAX_F; 0 disables the guesses.
 *   topf_out          device int32 [B, K, topf_F_max] or NULL when topf_F_max = 0.
 *   accepted_len      device int32 [B] out: k in 0..K.
 *   bonus_token       device int32 [B] out.
 *   accept_prob       device fp32 [B, K] out or NULL: min(1, p_i(x_i) / q'_i(x_i)) at every i.
 *   residual_mass     device fp32 [B] out or NULL: R (1 when k = K; 0 when the residual was all zero
 *                     and the bonus came from p_k).
 *   workspace         device scratch of ssd_verify_workspace_bytes(B, K, V, topf_F_max) bytes.
 * Launch: one kernel of B * T workgroups (T tiles per row, ssd_verify_tiles), or, when the batch
 * has more tiles than the device runs at once, that grid followed by one of a few workgroups per
 * sequence (ssd_verify_launches, ssd_verify_opts.launch_mode). The tiles of a sequence exchange partial results through the
 * workspace, but no workgroup ever needs another to be resident at the same time: a tile that has
 * polled for the rest of its sequence a bounded number of times (see ssd_verify_opts.wait_polls for
 * the default) hands its remaining work to the sequence's last tile and exits. The outputs are
 * therefore the same on a device busy with other work; an idle device only gets them sooner.
 * Errors: SSD_ERR_INVALID_ARG (null required pointer, bad size/stride/T/C/F), SSD_ERR_UNSUPPORTED
 * (dtype), SSD_ERR_WORKSPACE (too small or misaligned), SSD_ERR_HIP.
 * ------------------------------------------------------------------------------------------- */
#define SSD_DEFAULT_WAIT_POLLS 2048
/* Workspace bytes for calls of this shape; topf_F_max is the largest number of guesses per row
 * the calls make (including ssd_verify_opts.topf_last_F). */
size_t ssd_verify_workspace_bytes(int B, int K, int V, int topf_F_max);
/* Kernel launches ssd_verify issues for 16-byte aligned rows on the current device: 1, or 2 (the
 * streaming form) when the batch has more tiles (B x ssd_verify_tiles) than the device runs at once
 * (2 per CU); 0 for B = 0, -1 for arguments it rejects. */
int ssd_verify_launches(int B, int K, int V, ssd_dtype dtype, int topf_F_max);
/* Tiles per logit row (workgroups per sequence) of ssd_verify for this shape with 16-byte aligned
 * rows (rows that are not take 1024-token fp32 / 2048-token bf16 tiles), -1 if rejected. */
int ssd_verify_tiles(int B, int K, int V, ssd_dtype dtype);

ssd_status ssd_verify(const void* draft_logits, int64_t draft_seq_stride,
                      const void* target_logits, int64_t target_seq_stride,
                      ssd_dtype dtype, int B, int K, int V, float temperature,
                      const int32_t* draft_tokens, const float* uniforms,
                      const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                      const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                      int32_t* accepted_len, int32_t* bonus_token,
                      float* accept_prob, float* residual_mass,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Options of ssd_verify_ex (ssd_verify takes the defaults).
 *   wait_polls     How many times a tile polls for the rest of its sequence (its statistics, then
 *                  its residual masses) before it leaves its work to the sequence's last tile; 0
 *                  makes every tile but the last hand its work over at once. < 0:
 *                  SSD_DEFAULT_WAIT_POLLS. Any value gives the same outputs; it only moves work
 *                  between workgroups. At most 1 << 20.
 *   topf_last_F    0..SSD_MAX_F: also the top guesses of draft row K (the row after the last drafted
 *                  token, [SSD] "怎么猜奖励 token": the outcome k = K), with no token excluded, read
 *                  in the same pass. Needs draft_seq_stride >= (K+1) V. 0: none.
 *   topf_last_out  device int32 [B, topf_last_F] (-1 padded) when topf_last_F > 0.
 *   launch_mode    0: by shape (below); 1: one launch; 2: the streaming form, two launches. One
 *                  launch keeps every row of a tile in registers from its statistics to its
 *                  residual, the tile waiting for its sequence's decision. The streaming form ends
 *                  each tile once its statistics and guesses are out; a second grid takes the
 *                  decision and reads the two residual rows again, so no tile waits. By shape, a batch with more tiles than the device runs at
 *                  once (where waiting tiles would hold slots that others could stream in) takes
 *                  the streaming form. Both give the same outputs, bit for bit. Other values:
 *                  SSD_ERR_INVALID_ARG. */
typedef struct ssd_verify_opts {
  int32_t wait_polls;
  int32_t topf_last_F;
  int32_t* topf_last_out;
  int32_t launch_mode;
} ssd_verify_opts;

ssd_status ssd_verify_ex(const void* draft_logits, int64_t draft_seq_stride,
                         const void* target_logits, int64_t target_seq_stride,
                         ssd_dtype dtype, int B, int K, int V, float temperature,
                         const int32_t* draft_tokens, const float* uniforms,
                         const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                         const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                         int32_t* accepted_len, int32_t* bonus_token,
                         float* accept_prob, float* residual_mass, const ssd_verify_opts* opts,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_verify_noalloc — ssd_verify for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * the same kernel, with its workspace taken from a static device array of the library instead of
 * the caller.
 *   Arguments as ssd_verify, without workspace / workspace_bytes, plus
 *   device_flags  device uint32 [1], caller-owned: the call ORs its SSD_FLAG_* bits into it (sticky;
 *                 the caller zeroes it, e.g. with ssd_read_flags(device_flags, &f, 1, stream)).
 * Limit: shapes with ssd_verify_workspace_bytes(B, K, V, topf_F_max) <= SSD_NOALLOC_SCRATCH_BYTES;
 * larger ones return SSD_ERR_SCRATCH_LIMIT before any HIP call. The array (one per device, 32 MiB,
 * held until the process ends) is set up by the first call on each device (its address looked up,
 * its control words cleared by a fill kernel on `stream`); no call allocates or frees anything.
 * Every call on a device shares that device's array and leaves it ready for the next (counters back
 * at zero, other words tagged with the call): calls that overlap on one device, on different
 * streams, race and must not be issued.
 * Errors: as ssd_verify, SSD_ERR_INVALID_ARG also for a null device_flags, SSD_ERR_SCRATCH_LIMIT.
 * ------------------------------------------------------------------------------------------- */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ssd_status ssd_verify_noalloc(const void* draft_logits, int64_t draft_seq_stride,
                              const void* target_logits, int64_t target_seq_stride,
                              ssd_dtype dtype, int B, int K, int V, float temperature,
                              const int32_t* draft_tokens, const float* uniforms,
                              const int32_t* sag_set, int sag_F, float sag_C, const float* sag_C_pos,
                              const int32_t* topf_F, int topf_F_max, int32_t* topf_out,
                              int32_t* accepted_len, int32_t* bonus_token,
                              float* accept_prob, float* residual_mass, uint32_t* device_flags,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_topf_guess — top-F bonus-token guesses of R rows ([SSD] "怎么猜奖励 token"): per row the
 * F largest raw logits, excluding one token, ties to the smaller id; -inf never returned; -1 pads.
 *   logits      device [R rows, V] of dtype; row r starts at element r * row_stride (>= V).
 *   exclude     device int32 [R] (-1 = none) or NULL.
 *   F_per_row   device int32 [R] in [0, F_max] or NULL (= F_max). Out-of-range values are clamped
 *               and flagged (SSD_FLAG_BAD_F).
 *   F_max       1..SSD_MAX_F.
 *   out         device int32 [R, F_max].
 *   workspace   ssd_topf_workspace_bytes(R, V, F_max) bytes.
 * ------------------------------------------------------------------------------------------- */
size_t ssd_topf_workspace_bytes(int R, int V, int F_max);

ssd_status ssd_topf_guess(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                          const int32_t* exclude, const int32_t* F_per_row, int F_max,
                          int32_t* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_saguaro_adjust — Saguaro down-weighting of R draft rows ([SSD] "Saguaro 优化二",
 * "解法：操纵草稿分布"): q = softmax(row / T); sigma = sum_{s in S} q(s) over the distinct in-range
 * entries of S; N = 1 - (1 - C) sigma; q' = q * (C on S, 1 elsewhere) / N.
 *   logits        device [R rows, V]; row r at element r * row_stride (>= V).
 *   set, F        device int32 [R, F] (-1 pads; out-of-range and repeated entries ignored), F in
 *                 0..SSD_MAX_F (set may be NULL iff F = 0).
 *   C             in [0, 1].
 *   C_per_row     device fp32 [R] (row r uses C_per_row[r]; a value outside [0, 1] is clamped,
 *                 NaN taken as 1, and flagged SSD_FLAG_BAD_C) or NULL (C for every row).
 *   out_probs     device fp32 [R, V] q' or NULL (then nothing of size V is written).
 *   out_set_mass  device fp32 [R] sigma, or NULL.
 *   out_norm      device fp32 [R] N, or NULL. N <= 0 is flagged (SSD_FLAG_SAGUARO_NORM).
 *   workspace     ssd_saguaro_workspace_bytes(R, V) bytes.
 * ------------------------------------------------------------------------------------------- */
size_t ssd_saguaro_workspace_bytes(int R, int V);

ssd_status ssd_saguaro_adjust(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                              float temperature, const int32_t* set, int F, float C,
                              const float* C_per_row, float* out_probs, float* out_set_mass,
                              float* out_norm, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_saguaro_topf — the speculation cache's branch rows in one pass each ([SSD] "Saguaro 优化二",
 * "怎么猜奖励 token"): the set S of a row is its F_r largest logits (the tokens the cache holds;
 * ties to the smaller index, never a -inf logit, -1 pads), q = softmax(row / T),
 * sigma = sum_{s in S} q(s) and N = 1 - (1 - C) sigma, the normaliser of the down-weighted q'.
 * Gives what ssd_topf_guess (no exclusion) followed by ssd_saguaro_adjust with that set gives,
 * reading each row once.
 *   logits        device [R rows, V]; row r at element r * row_stride (>= V).
 *   F_per_row     device int32 [R] (0..F_max; out of range flagged SSD_FLAG_BAD_F) or NULL (F_max).
 *   F_max         1..SSD_MAX_F.  C in [0, 1].  temperature > 0 and finite.
 *   C_per_row     device fp32 [R] per-row C (as for ssd_saguaro_adjust) or NULL (C everywhere).
 *   out_set       device int32 [R, F_max] out.
 *   out_set_mass  device fp32 [R] sigma, or NULL.
 *   out_norm      device fp32 [R] N, or NULL. N <= 0 is flagged (SSD_FLAG_SAGUARO_NORM).
 *   workspace     ssd_saguaro_topf_workspace_bytes(R, V, F_max) bytes.
 * ------------------------------------------------------------------------------------------- */
size_t ssd_saguaro_topf_workspace_bytes(int R, int V, int F_max);

ssd_status ssd_saguaro_topf(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                            float temperature, const int32_t* F_per_row, int F_max, float C,
                            const float* C_per_row, int32_t* out_set, float* out_set_mass,
                            float* out_norm, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_saguaro_sample — the draft's sampling step with Saguaro, one pass over each row ([SSD]
 * "Saguaro 优化二：Saguaro 采样", "解法：操纵草稿分布"): what ssd_saguaro_topf computes (the set S =
 * the row's F_r largest logits, sigma, N), and a draft token drawn from q' = q (C on S, 1 elsewhere)
 * / N with the row's uniform u by the inverse CDF in ascending token order: the first token whose
 * cumulative q' exceeds u, or the last token of positive mass when rounding leaves u past the total
 * (the reading used for the bonus token). q' itself is never written.
 *   logits, row_stride, dtype, R, V, temperature, F_per_row, C, C_per_row, out_set, out_set_mass,
 *                 out_norm: as for ssd_saguaro_topf, except F_max may be 0 (plain sampling from q;
 *                 out_set may then be NULL).
 *   u             device fp32 [R] uniforms in [0, 1) (not checked: u >= 1 gives the last token of
 *                 positive mass, u < 0 the first).
 *   out_token     device int32 [R] the sampled token; -1 when q' has no mass: every logit -inf, or
 *                 the set holding all of q's mass with C = 0 (N = 0 up to rounding), which is also
 *                 flagged SSD_FLAG_SAGUARO_NORM.
 *   out_prob      device fp32 [R] q' of the sampled token (0 with -1), or NULL.
 *   workspace     ssd_saguaro_sample_workspace_bytes(R, V, F_max) bytes.
 * Logits must be finite or -inf. Rows are cut into segments of a whole number of 8192-token spans;
 * after the pass only the segment holding the drawn token is read again.
 * ------------------------------------------------------------------------------------------- */
size_t ssd_saguaro_sample_workspace_bytes(int R, int V, int F_max);

ssd_status ssd_saguaro_sample(const void* logits, int64_t row_stride, ssd_dtype dtype, int R, int V,
                              float temperature, const int32_t* F_per_row, int F_max, float C,
                              const float* C_per_row, const float* u, int32_t* out_token,
                              float* out_prob, int32_t* out_set, float* out_set_mass, float* out_norm,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_fanout_alloc — geometric fan-out of a cache budget ([SSD] "最优扇出度分配"). Host only,
 * synchronous. P(k) = (1-a) a^k for k < K and a^K for k = K; minimising sum_k P(k) F_k^-r under
 * sum_k F_k = budget gives F_k proportional to P(k)^(1/(1+r)). Integers: floor, then the leftover
 * units go to the largest fractional parts, ties to the smaller k.
 *   K >= 0, 0 < a < 1, r > 0, budget >= 0.
 *   out_F       host int32 [K+1].
 *   out_F_cont  host double [K+1] continuous optimum, or NULL.
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_fanout_alloc(int K, double a, double r, int budget, int32_t* out_F,
                            double* out_F_cont);

/* ---------------------------------------------------------------------------------------------
 * ssd_batch_speedup — expected speedup over autoregressive decoding of a batch of b sequences
 * ([SSD] "SSD 的核心思想" speedup formula; "解法：根据 batch 大小切换备用推测器"). The page's formulas
 * are lost; this reading keeps every quantity its text names, with times in units of one target
 * verification: a round costs max(1, T_p) (the verification, or the primary speculator when it is
 * slower), and the whole batch waits T_b for the backup speculator whenever any of its b sequences
 * misses (probability 1 - h^b):  S(b) = (h E_hit + (1 - h) E_miss) / (max(1, T_p) + (1 - h^b) T_b).
 * Host only, synchronous.
 *   h in [0, 1] the hit rate of one sequence; E_hit, E_miss >= 0 expected tokens a round yields on a
 *   hit / a miss; T_p, T_b >= 0 finite; b >= 1.  out_speedup  host double.
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_batch_speedup(double h, double E_hit, double E_miss, double T_p, double T_b, int b,
                             double* out_speedup);

/* ---------------------------------------------------------------------------------------------
 * ssd_backup_crossover — the batch size at which a fast backup speculator (E_miss_fast, T_fast)
 * and a neural one (E_miss_neural, T_neural) give the same ssd_batch_speedup ([SSD] "解法：根据
 * batch 大小切换备用推测器": small batches take the better drafts, large ones the shorter wait).
 * With x = 1 - h^b and A = h E_hit + (1 - h) E_miss, equality is one linear equation in x; its root
 * x* in (0, 1) gives b* = ln(1 - x*) / ln h. Host only, synchronous.
 *   Arguments as for ssd_batch_speedup.
 *   out_b_star           host double: b* (real), NaN when the two never cross at any b > 0.
 *   out_fast_wins_large  host int32 (or NULL): 1 if the fast backup is at least as good as b grows
 *                        without bound. The caller picks the fast backup for batches past b* when
 *                        this is 1 (or compares ssd_batch_speedup of the two at its batch size).
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_backup_crossover(double h, double E_hit, double E_miss_neural, double T_neural,
                                double E_miss_fast, double T_fast, double T_p, double* out_b_star,
                                int32_t* out_fast_wins_large);

/* ---------------------------------------------------------------------------------------------
 * ssd_cache_keys — keys of each sequence's speculation cache ([SSD] "SSD 的核心思想": an outcome
 * (k, t) is k accepted drafts and bonus t; "怎么猜奖励 token"). For k = 0..K the F_k guesses of
 * draft position k occupy consecutive slots (position K is the draft row after the last drafted
 * token); a guess of -1 leaves an empty slot (-1, -1).
 *   guesses       device int32 [B, K+1, G_max] (-1 padded), F_k <= G_max; or, with guesses_last,
 *                 [B, K, G_max] for positions 0..K-1 (the layout of ssd_verify's topf_out).
 *   guesses_last  device int32 [B, G_last] position K's guesses (the layout of ssd_topf_guess's
 *                 out), F_K <= G_last; or NULL (position K in guesses). Lets the cache be keyed
 *                 straight from the two calls' outputs, with no copy into one buffer.
 *   fanout        host int32 [K+1], sum = budget.
 *   cache_k, cache_tok  device int32 [B, budget] out.
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_cache_keys(int B, int K, int G_max, const int32_t* guesses, const int32_t* guesses_last,
                          int G_last, const int32_t* fanout, int budget, int32_t* cache_k,
                          int32_t* cache_tok, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_cache_lookup — look the verification outcome up in each sequence's cache ([SSD]
 * "SSD 的核心思想": a hit means the next draft is ready with zero wait; "Saguaro 优化三": the batch
 * waits for every miss). out_slot[b] = first slot j with (cache_k, cache_tok)[b, j] =
 * (accepted_len[b], bonus_token[b]), else -1; out_miss_count[0] = number of -1 (deterministic).
 *   cache_k, cache_tok  device int32 [B, budget] (k = -1 marks an empty slot); budget >= 0.
 *   accepted_len, bonus_token  device int32 [B].
 *   out_slot    device int32 [B];  out_miss_count  device int32 [1].
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_cache_lookup(int B, int budget, const int32_t* cache_k, const int32_t* cache_tok,
                            const int32_t* accepted_len, const int32_t* bonus_token,
                            int32_t* out_slot, int32_t* out_miss_count, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_cache_keys_lookup — ssd_cache_keys and ssd_cache_lookup in one launch ([SSD] "SSD 的核心思想",
 * "实现细节：缓存怎么建"): the same cache_k / cache_tok, out_slot and out_miss_count as the two
 * calls in turn, with the keys formed and matched in registers. Arguments as the two calls'.
 * Errors: SSD_ERR_INVALID_ARG as either call, SSD_ERR_HIP.
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_cache_keys_lookup(int B, int K, int G_max, const int32_t* guesses, const int32_t* guesses_last,
                                 int G_last, const int32_t* fanout, int budget, const int32_t* accepted_len,
                                 const int32_t* bonus_token, int32_t* cache_k, int32_t* cache_tok,
                                 int32_t* out_slot, int32_t* out_miss_count, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_read_flags — copy a workspace's device-error flags to *out_flags (host) and, if clear != 0,
 * reset them. Synchronises `stream`.
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_read_flags(void* workspace, uint32_t* out_flags, int clear, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * ssd_stream_read — measurement helper (not part of the verification path): reads `bytes` bytes of
 * device memory once, 16 bytes per load, the way a bandwidth-bound kernel streams its input, and
 * nothing else. Timing it over a footprint gives the read bandwidth the device reaches for it (the
 * ceiling the verification kernel is compared with).
 *   data   device, 16-byte aligned; bytes a multiple of 16.
 *   sink   device uint32 [8192], written only in a case that never arises in practice.
 * ------------------------------------------------------------------------------------------- */
ssd_status ssd_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* ssd_status_string(ssd_status s);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
