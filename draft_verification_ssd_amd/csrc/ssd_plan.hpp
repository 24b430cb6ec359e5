// Host-side launch planning: how rows are cut into workgroup chunks, and the workspace layout
// that those chunks need. The *_workspace_bytes entry points and the launchers both use these
// functions, so a workspace sized by the helper always fits the launch.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ssd {

constexpr int kPlanThreads = 256;
constexpr int kPlanMaxChunks = 64;
constexpr int kPlanTargetGroups = 2048;  // enough workgroups to cover 256 CUs several times over
constexpr int kPlanMinChunk = 2048;      // elements per workgroup, at least one vector per thread
constexpr int kPlanSub = 2048;           // phase-2 sub-chunk (256 threads x 8 elements)
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct RowPlan {
  int n1;      // chunks per row
  int chunk1;  // elements per chunk (multiple of 8)
};

// Cut `rows` rows of V elements into chunks: aim for kPlanTargetGroups workgroups in total while
// keeping each chunk at least kPlanMinChunk elements and at most kPlanMaxChunks per row.
inline RowPlan plan_rows(int64_t rows, int V) {
  int64_t n1 = ceil_div(kPlanTargetGroups, rows > 0 ? rows : 1);
  int64_t cap = ceil_div(V, kPlanMinChunk);
  if (cap > kPlanMaxChunks) cap = kPlanMaxChunks;
  if (n1 > cap) n1 = cap;
  if (n1 < 1) n1 = 1;
  int64_t chunk = ceil_div(ceil_div(V, n1), 8) * 8;
  RowPlan p;
  p.chunk1 = int(chunk);
  p.n1 = int(ceil_div(V, chunk));
  return p;
}

// Verification tiles: 256 threads x (NV 16-byte chunks of every row); the host picks NV per call.
// The smallest tile is 1024 tokens (fp32, one chunk), so a row of V tokens has at most
// ceil(V / 1024) tiles: the workspace is sized for that many whatever tile the call takes.
constexpr int kPlanMinTile = 1024;
constexpr int kSeqCtlMax = 65536;     // per-sequence counter slots: one for every sequence index
constexpr int kPlanSeqCtlWords = 8;   // 32 bytes per sequence: arrivals (word 0), then spare
constexpr int kPlanDecWords = 32;     // decision record: 256 bytes per sequence

struct VerifyLayout {
  int Tcap;     // tiles per row the regions are sized for
  int Fcap;     // guesses per row the candidate region is sized for
  size_t off_seqctl, off_stats, off_chunk, off_dec, off_cand, total;
};

// Workspace of ssd_verify:
//   [0, 256)      word 0 sticky flags, word 1 the last call's tag, word 2 sequences finished by the
//                 running call
//   seqctl        counters per sequence index (the arrivals of its tiles in word 0),
//                 at a fixed place for every sequence index 0 .. kSeqCtlMax-1, so no call of any
//                 shape writes data where another call keeps a counter
//   stats         [B][2K+1][Tcap][2] tagged (max c, sum) per row and tile
//   chunk         [B][Tcap][2] tagged claim word and residual mass word per tile
//   dec           [B][kPlanDecWords] tagged decision record per sequence
//   cand          [B][K+1][Tcap][Fcap][2] tagged halves of each tile's guesses
// Every data word carries the tag of the call that wrote it (tags grow by one per call), so a word
// left by an earlier call, of any shape, never passes for the running call's. Counters are back
// at zero whenever no call runs; a zero-filled workspace is a valid start.
inline VerifyLayout verify_layout(int B, int K, int V, int topf_F_max) {
  VerifyLayout L;
  L.Tcap = int(ceil_div(V, kPlanMinTile));
  L.Fcap = topf_F_max > 0 ? topf_F_max : 1;
  size_t off = kAlign;
  L.off_seqctl = off;
  off = align_up(off + size_t(kSeqCtlMax) * kPlanSeqCtlWords * 4);
  L.off_stats = off;
  off = align_up(off + size_t(B) * (2 * K + 1) * L.Tcap * 16);
  L.off_chunk = off;
  off = align_up(off + size_t(B) * L.Tcap * 16);
  L.off_dec = off;
  off = align_up(off + size_t(B) * kPlanDecWords * 8);
  L.off_cand = off;
  off = align_up(off + size_t(B) * (K + 1) * L.Tcap * L.Fcap * 16);
  L.total = off;
  return L;
}

struct TopfLayout {
  RowPlan rp;
  size_t off_cand, off_stats, total;
};

// Top-F chunks are longer than the statistics chunks: each wave's candidate search has a fixed
// cost (its first threshold, the final cut, the merge of the chunks), so whole rows are kept
// whenever the rows alone give the device a few workgroups per CU.
constexpr int kTopfTargetGroups = 768;
constexpr int kTopfMinChunk = 8192;  // one 8192-token batch of a workgroup; 16384 kept 16 rows of
                                     // 128256 bf16 in 128 workgroups, 2.3 us slower

inline int64_t topf_chunks(int R, int V) {
  int64_t n1 = ceil_div(kTopfTargetGroups, R > 0 ? R : 1);
  int64_t cap = ceil_div(V, kTopfMinChunk);
  if (cap > kPlanMaxChunks) cap = kPlanMaxChunks;
  if (n1 > cap) n1 = cap;
  if (n1 < 1) n1 = 1;
  return n1;
}

inline TopfLayout topf_layout(int R, int V, int F_max) {
  TopfLayout L;
  const int64_t n1 = topf_chunks(R, V);
  const int64_t chunk = ceil_div(ceil_div(V, n1), 8) * 8;
  L.rp.chunk1 = int(chunk);
  L.rp.n1 = int(ceil_div(V, chunk));
  L.off_cand = kAlign;
  L.off_stats = align_up(L.off_cand + size_t(R) * L.rp.n1 * F_max * 8);
  // chunk statistics (ssd_saguaro_topf) only when a row has several chunks
  L.total = align_up(L.off_stats + (L.rp.n1 > 1 ? size_t(R) * L.rp.n1 * 8 : 0));
  return L;
}

// Draft-side sampling (ssd_saguaro_sample) runs the top-F pass with the row cut into segments of
// seg_len tokens, a whole number of the pass's 8192-token batches, at most kPlanMaxSeg per chunk;
// chunks are a whole number of segments, so segment g of a row covers tokens
// [g seg_len, (g + 1) seg_len) whatever the chunking. Each segment's (max c, sum) pair locates the
// sampled token's segment; only that segment is read again.
constexpr int kPlanSampleSpan = 8192;  // tokens of one top-F batch of a workgroup (256 lanes x 32)
constexpr int kPlanMaxSeg = 16;

struct SampleLayout {
  TopfLayout t;
  int seg_len, nseg;  // tokens per segment, segments per chunk
  size_t off_seg;     // [R][n1 * nseg] float2 segment pairs (when n1 > 1)
  size_t total;
};

inline SampleLayout sample_layout(int R, int V, int F_max) {
  SampleLayout L;
  const int64_t n1 = topf_chunks(R, V);
  const int64_t len0 = ceil_div(V, n1);
  const int64_t G = ceil_div(ceil_div(len0, kPlanSampleSpan), kPlanMaxSeg);
  const int64_t seg = G * kPlanSampleSpan;
  const int64_t chunk = ceil_div(len0, seg) * seg;
  L.seg_len = int(seg);
  L.nseg = int(chunk / seg);
  L.t.rp.chunk1 = int(chunk);
  L.t.rp.n1 = int(ceil_div(V, chunk));
  const size_t n1s = size_t(L.t.rp.n1);
  L.t.off_cand = kAlign;
  L.t.off_stats = align_up(L.t.off_cand + size_t(R) * n1s * size_t(F_max) * 8);
  L.off_seg = align_up(L.t.off_stats + (n1s > 1 ? size_t(R) * n1s * 8 : 0));
  L.total = align_up(L.off_seg + (n1s > 1 ? size_t(R) * n1s * L.nseg * 8 : 0));
  L.t.total = L.total;
  return L;
}

struct SaguaroLayout {
  RowPlan rp;
  int n_out;  // materialisation chunks per row
  int chunk_out;
  size_t off_stats, total;
};

inline SaguaroLayout saguaro_layout(int R, int V) {
  SaguaroLayout L;
  L.rp = plan_rows(R, V);
  RowPlan o = plan_rows(R, V);
  L.n_out = o.n1;
  L.chunk_out = o.chunk1;
  L.off_stats = kAlign;
  L.total = align_up(L.off_stats + size_t(R) * L.rp.n1 * 8);
  return L;
}

}  // namespace ssd
