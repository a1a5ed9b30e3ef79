// Host-side declarations shared by the libfastgen translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fastgen.h"

namespace fg {

// Kernel timing hooks (no-ops unless fg_kernel_timing_enable(1)).
void timed_begin(int kernel_id, hipStream_t st);
void timed_end(hipStream_t st);

struct ProfileArgs {
  int dtype, D, B, Hq, Hkv, n;
  int k_f, w_l;
  double T;
  const void* Q;
  const void* K;
  const uint8_t* cls;
  float* lse2;       // [B*Hq*n] log2-domain row log-sum-exp (workspace)
  float* lse_out;    // optional natural-log copy
  float* cum;        // [B*Hkv*n]
  float* band;       // [B*Hkv*n]
  uint32_t* fmask;   // [B*Hkv*ceil(n/32)]
  float* recovery;   // [B*Hkv*5]
  uint8_t* policy;   // [B*Hkv]
  // small grids split the sweeps: key chunks of sweep 1 (partial max/sum per row,
  // merged by the column sweep as it loads each row) and row chunks of sweep 2 (partial column sums,
  // added by the select pass); nullptr / chunk >= n means no split
  int kchunk, rchunk;
  float2* rs_part;   // [ceil(n/kchunk), B*Hq, n]
  float2* cs_part;   // [ceil(n/rchunk), B*Hkv, n]
  bool lse_ready;    // lse2 already written (by the attention kernel): skip sweep 1
  int cus;           // compute units of the device (steers the launch shape only)
};

// Sweep tiling shared by the launcher and the workspace query.
constexpr int kSweepRowsPerWG = 256;   // query rows per sweep-1 workgroup
constexpr int kSweepKeysPerWG = 256;   // keys per sweep-2 workgroup
constexpr int kSplitMinChunk = 256;    // smallest chunk of a split sweep (sizes the partial buffers)
constexpr long long kSplitBelowGroups = 1024;  // split when the unsplit grid has fewer workgroups
constexpr int kSplitOverheadItems = 192;       // a workgroup's fixed cost (launch, operand and first-tile loads), in keys (rows) of work

// A block of R keys (sweep 1: the causal keys of a row block) or rows (sweep 2:
// the rows at or below a key block) is split into split_count(R, S) chunks of
// nearly equal size at 32-item granularity; chunk ch is
// [split_begin(R, c, ch), min(R, split_begin(R, c, ch + 1))).  The count is
// the one a plain split into S-item chunks would give, so every chunk has at
// most S items and the partial buffers keep their layout.
__host__ __device__ inline int split_count(int R, int S) { return R <= S ? 1 : (R + S - 1) / S; }
__host__ __device__ inline int split_begin(int R, int c, int ch) {
  const int U = (R + 31) / 32;
  return 32 * (int)(((long long)ch * U) / c);
}

// Items of block i: sweep 1 row block rb has min(n, 256 (rb + 1)) causal keys,
// sweep 2 key block kb has n - 256 kb rows at or below it.
inline int sweep_block_items(bool rows_of_key_block, int n, int i) {
  return rows_of_key_block ? n - kSweepKeysPerWG * i : (n < kSweepRowsPerWG * (i + 1) ? n : kSweepRowsPerWG * (i + 1));
}

// Chunk size of a split sweep: the candidate S >= kSplitMinChunk that minimises
// the estimated span, rounds of `slots` concurrent workgroups times the
// largest chunk (plus a workgroup's fixed cost) -- a small grid is bound by its
// last round, not by its total work.
inline int choose_split_chunk(int n, int nblocks, long long mult, bool rows_of_key_block, int slots) {
  static const int kCand[] = {256, 288, 320, 352, 384, 448, 512, 576, 640, 768, 896, 1024, 1280, 1536, 1792,
                              2048, 2560, 3072, 4096, 6144, 8192, 12288, 16384, 24576, 32768};
  int best = n;
  long long best_cost = -1;
  for (int S : kCand) {
    if (S >= n) break;
    long long count = 0;
    int maxc = 0;
    for (int i = 0; i < nblocks; ++i) {
      const int R = sweep_block_items(rows_of_key_block, n, i);
      const int c = split_count(R, S);
      count += c;
      const int per = 32 * (((R + 31) / 32 + c - 1) / c);   // the largest of the c balanced chunks
      const int size = per < R ? per : R;
      maxc = size > maxc ? size : maxc;
    }
    count *= mult;
    const long long rounds = (count + slots - 1) / slots;
    const long long cost = rounds * (maxc + kSplitOverheadItems);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

struct SweepSplit {
  int kchunk, rchunk;
  bool rs_split, cs_split;
  size_t rs_bytes, cs_bytes;
};
// cus: compute units; with bf16 operands sweep 1 runs three workgroups per CU, sweep 2 three when
// sweep 1 is not split and two when it is (it then merges sweep 1's partial statistics); fp32 runs
// two of each.  The slots only steer the chunk sizes, never the buffer sizes.
inline SweepSplit sweep_split(int B, int Hq, int Hkv, int n, int cus, bool bf16) {
  SweepSplit p{};
  const int n_rb = (n + kSweepRowsPerWG - 1) / kSweepRowsPerWG;
  const int n_kb = (n + kSweepKeysPerWG - 1) / kSweepKeysPerWG;
  p.rs_split = (long long)B * Hq * n_rb < kSplitBelowGroups && n > kSplitMinChunk;
  p.cs_split = (long long)B * Hkv * n_kb < kSplitBelowGroups && n > kSplitMinChunk;
  const int rs_slots = cus * (bf16 ? 3 : 2), cs_slots = cus * (bf16 && !p.rs_split ? 3 : 2);
  p.kchunk = p.rs_split ? choose_split_chunk(n, n_rb, (long long)B * Hq, false, rs_slots) : n_rb * kSweepRowsPerWG;
  p.rchunk = p.cs_split ? choose_split_chunk(n, n_kb, (long long)B * Hkv, true, cs_slots) : n;
  p.rs_bytes = p.rs_split ? (size_t)split_count(n, kSplitMinChunk) * B * Hq * n * sizeof(float) * 2 : 0;
  p.cs_bytes = p.cs_split ? (size_t)split_count(n, kSplitMinChunk) * B * Hkv * n * sizeof(float) * 2 : 0;
  return p;
}

hipError_t launch_profile_sweeps(const ProfileArgs& a, hipStream_t st);

// Causal attention output of the prompt (bf16), with the row log-sum-exp.
struct AttentionArgs {
  int D, B, Hq, Hkv, n;
  const void* Q;
  const void* K;
  const void* V;
  void* O;           // [B*Hq*n, D] bf16
  float* lse2;       // [B*Hq*n] log2-domain row log-sum-exp, or nullptr
  float* lse_out;    // [B*Hq*n] natural-log copy, or nullptr
  int cus;           // compute units of the device (steers the launch shape only)
};
hipError_t launch_attention(const AttentionArgs& a, hipStream_t st);

// Per-row level bins of the prompt's attention (one sweep over the causal scores).
struct RowBinsArgs {
  int dtype, D, B, Hq, Hkv, n, w_l;
  const void* Q;
  const void* K;
  const uint8_t* cls;      // [B, n] token classes
  const uint32_t* fmask;   // [B*Hkv, ceil(n/32)] frequent-set bits
  const float* lse;        // [B*Hq*n] row log-sum-exp of the scaled scores, natural log (times lse_scale:
  float lse_scale;         //   log2(e) for natural-log input, 1 for the sweeps' own log2-domain values)
  float* bins;             // [B*Hq*n, 5] special, punct, frequent, local, rest
};
hipError_t launch_rowbins(const RowBinsArgs& a, hipStream_t st);
// R_k from the row bins of each (b, KV head), policy, and the least kept share over the rows.
hipError_t launch_rowbins_reduce(const float* bins, int H, int G, int n, double T, float* recovery, uint8_t* policy,
                                 float* row_min, hipStream_t st);
hipError_t launch_select(const ProfileArgs& a, hipStream_t st);
hipError_t launch_head_map_accumulate(const float* recovery, const uint8_t* policy, double* rec_sum, int32_t* count,
                                      int P, int H, hipStream_t st);
hipError_t launch_head_map_finish(const double* rec_sum, double n_prompts, double T, float* mean, uint8_t* policy,
                                  int H, hipStream_t st);

struct PlanArgs {
  int B, Hkv, n, w_l;
  int max_new, max_new_kept;
  const uint8_t* cls;
  const uint8_t* policy;
  const uint32_t* fmask;
  int32_t* kept_count;
  int32_t* ring;
  int32_t* capacity;
  int64_t* row_offset;
  int64_t* work_offset;
  int64_t* totals;
  int chunk_rows;
};
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);

struct GatherArgs {
  int dtype, D, B, Hkv, n, w_l;
  const void* K;
  const void* V;
  const uint8_t* cls;
  const uint8_t* policy;
  const uint32_t* fmask;
  const int64_t* row_offset;
  const int32_t* ring;
  const int64_t* work_offset;
  void* Kc;
  void* Vc;
  int32_t* pos;
  int32_t* len;
  int32_t* work;
  uint32_t* error_word;
  int chunk_rows;
  int64_t total_rows, n_work;   // the cache's capacities
  int items_per_head;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);

struct DecodeArgs {
  int dtype, D, B, Hq, Hkv, w_l, p;
  int64_t n_work;
  const void* q;
  const void* k_new;
  const void* v_new;
  const uint8_t* new_class;
  float* out;
  float* part;       // [n_work * G * (D + 2)]
  void* Kc;
  void* Vc;
  int32_t* pos;
  const int64_t* row_offset;
  int32_t* len;
  const int32_t* capacity;
  const int32_t* ring;
  const uint8_t* policy;
  const int64_t* work_offset;
  int32_t* work;     // [n_work * 4] (head, first row, first absolute row, rows in use)
  uint32_t* error_word;
  int chunk_rows;
  int items_per_head;   // partial-state slots per head
  int64_t total_rows;   // cache rows allocated
  bool partials_only;   // skip the merge launch (the cache is left unchanged)
  // frequent set re-ranked during generation (nullptr: the static policy)
  float* score;         // [total_rows] cumulative score per cache row
  const uint8_t* cls_all;   // [B, n_total] class of every position
  int n_total;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

constexpr int kDecodeSubRows = 128;   // rows of a decode work item whose loads are issued together
// Rows per decode work item: kDecodeSubRows doubled up to 2048 until a head of
// n rows has at most 64 items (long heads: fewer partial states to merge).
inline int decode_chunk_rows(int n) {
  int c = kDecodeSubRows;
  while (c < 2048 && (n + c - 1) / c > 64) c *= 2;
  return c;
}
constexpr int kMaxGroup = 8;       // query heads per KV head supported by decode

// Decode-time tracking (level shares of a step's attention, cumulative key scores).
struct TrackArgs {
  int dtype, D, B, Hq, Hkv, w_l, p, n_prompt, n_total;
  int64_t n_work;
  const void* q;
  const void* Kc;
  const int32_t* pos;
  const int32_t* work;
  const int64_t* work_offset;
  const uint8_t* cls;        // [B, n_total] class of every position
  const uint32_t* fmask;     // [B*Hkv, ceil(n_prompt/32)]
  float* score;              // [total_rows] in/out
  float* level_bins;         // [B*Hkv, 5]
  void* workspace;
  int chunk_rows, items_per_head;
};
// workspace: per (head, item slot, query head) a (max, sum) pair, then per (head, item slot) 5 bins
inline size_t track_stats_bytes(int64_t heads, int64_t slots, int G) {
  return (((size_t)heads * slots * G * 8) + 255) & ~(size_t)255;
}
inline size_t track_workspace_bytes(int64_t heads, int64_t slots, int G) {
  return track_stats_bytes(heads, slots, G) + (size_t)heads * slots * 5 * 4;
}
hipError_t launch_track(const TrackArgs& a, hipStream_t st);
hipError_t launch_track_init(const int64_t* row_offset, const int32_t* pos, const float* cum, float* score, int H,
                             int n_prompt, hipStream_t st);

// Micro-benchmarks of the chip's ceilings (measurement only).
hipError_t launch_peak_mfma(const void* operands, float* out, int iters, int blocks, hipStream_t st);
hipError_t launch_peak_exp(float* out, int iters, int blocks, hipStream_t st);
hipError_t launch_peak_mfma_softmax(const void* operands, float* out, int iters, int blocks, hipStream_t st);
hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, bool nontemporal, int blocks, hipStream_t st);
hipError_t launch_peak_read(const void* src, size_t bytes, bool nontemporal, int blocks, unsigned* out,
                            hipStream_t st);

}  // namespace fg
