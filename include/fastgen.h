/*
 * libfastgen -- FastGen's head-wise attention profiling, KV compaction and
 * compressed-cache decode on AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the hyper.ai summary pages of "Model Tells You What to
 * Discard: Adaptive KV Cache Compression for LLMs" (Ge et al., ICLR 2024),
 * section Method.  The calls mirror its two-phase inference: profile every
 * attention head while the prompt is encoded, build head-specific caches
 * K_C, V_C = f(K, V, C), then generate with those caches, reusing the policy
 * picked on the prompt for every new token.
 *
 * Conventions (every call):
 *  - Pointers are DEVICE memory unless marked [host].  The caller owns all
 *    memory; the library never allocates or frees device memory.  Size queries
 *    tell the caller what to allocate.
 *  - Every call only enqueues work on the given stream and returns; nothing is
 *    synchronised except fg_cache_error (documented below).
 *  - All argument checks run on the host before any launch.  On failure the
 *    call returns a status, writes nothing and launches nothing; the reason is
 *    available from fg_last_error() (thread-local string).
 *  - A failed kernel launch returns FG_ERR_HIP.  No C++ exception crosses this
 *    interface.
 *  - Supported: head_dim in {64, 128}; dtype bf16 or fp32 (inputs and caches);
 *    n_q_heads % n_kv_heads == 0 with group G = n_q_heads / n_kv_heads <= 8;
 *    seq_len >= 1; 0 < T <= 1; 0 <= r_l, r_f <= 1.  Tensors are contiguous,
 *    row-major, 16-byte aligned.
 *
 * Notation: B batch, Hq / Hkv query / KV heads, n prompt length, d head_dim,
 * k_f = floor(r_f * n) frequent keys, w_l = floor(r_l * n) local window
 * (both in fp64).  Levels / policies: 0 special, 1 special+punct,
 * 2 special+punct+frequent, 3 special+punct+frequent+local, 4 full.
 */
#ifndef FASTGEN_H
#define FASTGEN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FG_OK = 0,
  FG_ERR_INVALID_ARG = 1,   /* bad pointer, shape or parameter */
  FG_ERR_UNSUPPORTED = 2,   /* valid but not supported (head_dim, dtype, G > 8) */
  FG_ERR_WORKSPACE = 3,     /* workspace missing or too small */
  FG_ERR_CAPACITY = 4,      /* a cache ran out of rows (see fg_cache_error) */
  FG_ERR_HIP = 5            /* a HIP runtime call or launch failed */
} fg_status;

typedef enum { FG_DTYPE_BF16 = 0, FG_DTYPE_F32 = 1 } fg_dtype;

enum { FG_TOKEN_NORMAL = 0, FG_TOKEN_SPECIAL = 1, FG_TOKEN_PUNCT = 2 };

enum {
  FG_POLICY_SPECIAL = 0,
  FG_POLICY_SPECIAL_PUNCT = 1,
  FG_POLICY_SPF = 2,
  FG_POLICY_SPFL = 3,
  FG_POLICY_FULL = 4
};

/* [host] shape of one attention layer's prompt */
typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, seq_len, head_dim;
  int32_t dtype; /* fg_dtype */
} fg_shape;

/* [host] budgets and recover ratio (Method, policy paragraph and constraint equation) */
typedef struct {
  double r_l, r_f, T;
} fg_params;

/* ------------------------------------------------------------------ profiling */

/* Bytes of workspace fg_profile needs: per-row log-sum-exp [B*Hq*n] fp32 and
 * the banded column sums [B*Hkv*n] fp32. */
size_t fg_profile_workspace_size(const fg_shape* shape);

/*
 * fg_profile -- head-wise profiling of one layer's prompt (Method, second
 * paragraph: the attention map A = softmax(Q K^T) and the policy argmin under
 * |A - softmax(Q K_C^T)| <= 1 - T; policy paragraph; shortlist equation).
 *
 * Per (batch entry b, KV head h) with query heads g of its group:
 *   A^g_ij   = softmax_j(q^g_i . k_j / sqrt(d)) over j <= i (causal);
 *   cum[j]   = sum_g sum_{i >= j} A^g_ij   (cumulative attention score);
 *   F        = the k_f keys with the largest cum, ties to the lower index;
 *   level(i, j) = 0 special(j), 1 punct(j), 2 j in F, 3 i - j < w_l, else 4;
 *   R_k      = (1 / (G n)) sum_g sum_i sum_{j : level(i,j) <= k} A^g_ij
 *              (retained share of attention; per row this is one minus half
 *              the L1 distance of the constraint), R_4 = 1;
 *   policy   = min { k : R_k >= T }.
 *
 * Q [B,Hq,n,d], K [B,Hkv,n,d] (dtype of shape), post-rotary.
 * token_class [B,n] u8 (FG_TOKEN_*).
 * Outputs: policy [B*Hkv] u8; cum_score [B*Hkv*n] fp32; recovery [B*Hkv*5] fp32;
 *          freq_mask [B*Hkv*ceil(n/32)] u32, bit (j % 32) of word j / 32 set
 *          iff j in F.
 * Optional outputs (NULL to skip): lse_out [B*Hq*n] fp32, natural-log
 *          log-sum-exp of each row's scaled scores; band_out [B*Hkv*n] fp32,
 *          sum_g sum_{j <= i < j + w_l} A^g_ij.
 * workspace: at least fg_profile_workspace_size(shape) bytes.
 */
fg_status fg_profile(const fg_shape* shape, const fg_params* params,
                     const void* Q, const void* K, const uint8_t* token_class,
                     uint8_t* policy, float* cum_score, float* recovery, uint32_t* freq_mask,
                     float* lse_out, float* band_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fg_attention -- the prompt's causal attention output, the pass the profiling
 * rides on (Method, first paragraph: heads are profiled while the prompt is
 * encoded).  Per batch entry b and query head hq with KV head h = hq / G:
 *   O[b,hq,i,:] = sum_{j <= i} A_ij V[b,h,j,:],  A_ij = softmax_j(q_i . k_j / sqrt(d)).
 * bf16 only (FG_ERR_UNSUPPORTED for fp32): Q [B,Hq,n,d], K, V [B,Hkv,n,d],
 * O [B,Hq,n,d] bf16 (caller-allocated, may not alias the inputs), all 16-byte
 * aligned.  lse_out [B*Hq*n] fp32 (optional, NULL to skip): natural-log
 * log-sum-exp of each row's scaled scores.  No workspace.
 */
fg_status fg_attention(const fg_shape* shape, const void* Q, const void* K, const void* V, void* O,
                       float* lse_out, hipStream_t stream);

/*
 * fg_profile_attention -- fg_profile fused with fg_attention: the attention
 * output O is computed together with the row statistics the profiling needs,
 * so the profiling adds only its column sweep and the policy selection.
 * Arguments and outputs as fg_profile plus V (input) and O (output) as
 * fg_attention; bf16 only.  workspace: fg_profile_workspace_size(shape) bytes.
 */
fg_status fg_profile_attention(const fg_shape* shape, const fg_params* params,
                               const void* Q, const void* K, const void* V, const uint8_t* token_class,
                               void* O, uint8_t* policy, float* cum_score, float* recovery,
                               uint32_t* freq_mask, float* lse_out, float* band_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fg_profile_row_bins -- per query row, the attention mass on each shortlist
 * level (hyper.ai summary of "Model Tells You What to Discard", Method: the
 * constraint equation taken row by row, with the levels of the shortlist
 * equation).  For batch entry b, query head hq (KV head h = hq / G) and row i:
 *   bins[b,hq,i,l] = sum_{j <= i, level(i,j) = l} A_ij,  A_ij = softmax_j(q_i . k_j / sqrt(d)),
 * level 0 special, 1 punct, 2 frequent (j in F of (b,h)), 3 local (i - j < w_l,
 * w_l = floor(r_l n)), 4 the rest; a key takes the first level that holds it.
 * Summed over the rows and the G query heads of (b,h) and divided by G n, the
 * running sums of bins[..., 0..k] are fg_profile's recovery R_k; per row they
 * give the kept share of each row (the worst-served rows of a head).
 * Q, K, token_class as fg_profile (16-byte aligned Q, K); freq_mask and lse
 * as fg_profile's outputs for the same inputs and params (lse: its lse_out,
 * [B*Hq*n] fp32 natural log).  bins [B*Hq*n*5] fp32, caller-allocated.  Only
 * params->r_l is read (T and r_f are checked but unused).  No workspace.
 * FG_ERR_INVALID_ARG for NULL pointers or misaligned Q, K; FG_ERR_UNSUPPORTED
 * for shapes fg_profile rejects, more than 65535 batch entries, or more than
 * 2^32 threads in one launch (256 per query head and 256-row block).
 */
fg_status fg_profile_row_bins(const fg_shape* shape, const fg_params* params, const void* Q, const void* K,
                              const uint8_t* token_class, const uint32_t* freq_mask, const float* lse, float* bins,
                              hipStream_t stream);

/*
 * fg_profile_rows -- fg_profile with the per-row level bins as the recovery
 * route (the constraint equation of Method read row by row: each row's kept
 * share under each shortlist entry, then averaged).  The sweeps and the top-k
 * run as in fg_profile (cum_score, freq_mask as there); then the row-bins sweep
 * (fg_profile_row_bins) bins every row of every query head on the matrix cores,
 * and a reduction per (b, KV head) gives
 *   R_k = (1 / (G n)) sum_g sum_i sum_{l <= k} bins[g][i][l]   (fp64 sums), R_4 = 1,
 *   policy = min { k : R_k >= T },
 *   row_min[k] = min over the G n rows of sum_{l <= k} bins[g][i][l]  (the least
 *                kept share of any row; row_min[4] = the least row total),
 * written to recovery [B*Hkv*5], policy [B*Hkv] and row_min [B*Hkv*5] (optional,
 * NULL to skip).  R_k equals fg_profile's column-sum route up to rounding.
 * bins_out [B*Hq*n*5] fp32 (optional) receives the bins; else they live in the
 * workspace of fg_profile_rows_workspace_size(shape) bytes.  Errors as
 * fg_profile and fg_profile_row_bins.
 */
size_t fg_profile_rows_workspace_size(const fg_shape* shape);
fg_status fg_profile_rows(const fg_shape* shape, const fg_params* params, const void* Q, const void* K,
                          const uint8_t* token_class, uint8_t* policy, float* cum_score, float* recovery,
                          uint32_t* freq_mask, float* row_min, float* bins_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Multi-prompt head map (jisaku.com glossary entry "FastGen", section
 * Profiling phase: heads are typed once from sample prompts, the map is saved
 * and applied at inference).  Profile P prompts (one fg_profile call with
 * batch = prompts, or several calls), add each call's outputs with
 * fg_head_map_accumulate, then fg_head_map_finish gives each KV head the first
 * shortlist entry whose recovery averaged over the prompts reaches T.  Apply
 * the map by passing its policy (repeated over the batch) to fg_compact_plan /
 * fg_compact together with the prompt's own freq_mask.
 *
 * fg_head_map_accumulate: recovery [n_prompts * n_kv_heads * 5] fp32 and
 *   policy [n_prompts * n_kv_heads] u8 as fg_profile wrote them; rec_sum
 *   [n_kv_heads * 5] fp64 and policy_count [n_kv_heads * 5] int32 are running
 *   sums (in/out), zeroed by the caller before the first call; the sums run
 *   prompt by prompt in a fixed order.
 * fg_head_map_finish: n_prompts = the total added; mean_recovery
 *   [n_kv_heads * 5] fp32 = rec_sum / n_prompts; policy [n_kv_heads] u8 = the
 *   first k < 4 with rec_sum[k] / n_prompts >= T (fp64 compare), else 4.
 */
fg_status fg_head_map_accumulate(int32_t n_prompts, int32_t n_kv_heads, const float* recovery, const uint8_t* policy,
                                 double* rec_sum, int32_t* policy_count, hipStream_t stream);
fg_status fg_head_map_finish(int32_t n_kv_heads, int64_t n_prompts, const fg_params* params, const double* rec_sum,
                             float* mean_recovery, uint8_t* policy, hipStream_t stream);

/* ------------------------------------------------------------------ compaction */

/*
 * Ragged per-(b, KV head) cache: a POD view of caller-owned buffers.  Head
 * hd = b * Hkv + h owns rows [row_offset[hd], row_offset[hd+1]).  The first
 * ring[hd] rows are the local window's ring (policy 3 only: w_l - 1 slots,
 * slot = position mod (w_l - 1)); after them come the permanent rows in the
 * order they were kept.  Rows [0, len[hd]) are in use; a row whose pos is -1
 * is empty.  The kept-index list of a head is the sorted set of pos >= 0 over
 * its rows in use.
 */
typedef struct {
  void* k;                 /* [total_rows, d] cache dtype */
  void* v;                 /* [total_rows, d] */
  int32_t* pos;            /* [total_rows] absolute token position, -1 = empty */
  const int64_t* row_offset;  /* [B*Hkv + 1] */
  int32_t* len;            /* [B*Hkv] rows in use (ring + permanent) */
  const int32_t* capacity; /* [B*Hkv] */
  const int32_t* ring;     /* [B*Hkv] ring slots */
  const uint8_t* policy;   /* [B*Hkv] */
  const int64_t* work_offset; /* [B*Hkv + 1] decode work items per head (prefix) */
  int32_t* work;           /* [n_work * 4] decode work items: (head, first row of the head,
                              first absolute row, rows in use); fg_compact fills it and every
                              fg_decode_step append keeps the rows-in-use count current */
  uint32_t* error_word;    /* [1] sticky device error bits: 1 = an append found its head full,
                              2 = the compaction plan did not fit total_rows / n_work /
                              items_per_head (the heads that do not fit are left empty) */
  int64_t total_rows;      /* [host] rows allocated */
  int64_t n_work;          /* [host] work items */
  int64_t items_per_head;  /* [host] largest work-item count of a head (partial-state slots
                              per head in the decode workspace) */
  int32_t n_prompt;        /* [host] n */
  int32_t w_l;             /* [host] local window */
  int32_t next_pos;        /* [host] position of the next generated token (starts at n) */
  int32_t chunk_rows;      /* [host] cache rows per decode work item (set by fg_compact) */
  fg_shape shape;          /* [host] */
} fg_cache;

/* Rows of decode work per item (the split-K chunk of fg_decode_step) for a
 * prompt shape: 128 rows, doubled up to 2048 until a head of seq_len rows has
 * at most 64 items.  0 for an invalid shape. */
int32_t fg_decode_chunk_rows(const fg_shape* shape);

/*
 * fg_compact_plan -- size the head-specific caches (Method, second paragraph:
 * K_C, V_C = f(K, V, C)).  Per head: the prompt keys that the first generated
 * token keeps, {j < n : level(n, j) <= policy}, split into permanent rows
 * (special, punct, frequent, or everything for policy 4) and ring rows
 * (policy 3: normal keys inside the local window).
 * Inputs from fg_profile: policy, freq_mask.  max_new_tokens: generated tokens
 * the caches must hold room for; max_new_kept (<= max_new_tokens): upper bound
 * on generated special/punct tokens (room for heads with policy < 4).
 * Outputs: kept_count [B*Hkv] prompt keys kept; ring [B*Hkv]; capacity [B*Hkv]
 * = ring + permanent prompt rows + (policy 4 ? max_new_tokens : max_new_kept);
 * row_offset [B*Hkv+1] and work_offset [B*Hkv+1] (exclusive prefix sums; a
 * head has max(1, ceil(capacity / fg_decode_chunk_rows(shape))) work items);
 * totals [3] = {total rows, total work items, largest item count of a head}.
 * The caller reads totals to the host (the one synchronisation of the path) to
 * allocate the cache and set total_rows, n_work and items_per_head.
 */
fg_status fg_compact_plan(const fg_shape* shape, const fg_params* params,
                          const uint8_t* token_class, const uint8_t* policy,
                          const uint32_t* freq_mask, int32_t max_new_tokens, int32_t max_new_kept,
                          int32_t* kept_count, int32_t* ring, int32_t* capacity,
                          int64_t* row_offset, int64_t* work_offset, int64_t* totals,
                          hipStream_t stream);

/*
 * fg_compact -- gather the kept K/V rows of every head into the cache,
 * permanent rows in ascending position; fill pos, len, the decode work list,
 * and clear error_word.  cache must hold the buffers sized from
 * fg_compact_plan (k, v, pos with total_rows rows; work with n_work items)
 * and its row_offset, capacity, ring, policy, work_offset arrays; n_prompt,
 * w_l, next_pos and chunk_rows are set by this call.  Rows are byte copies.
 * total_rows, n_work and items_per_head are capacities: a cache allocated for
 * an earlier plan can be refilled without reading the new totals (no host
 * synchronisation), and a plan that exceeds them sets bit 2 of error_word
 * (read with fg_cache_error) and leaves the heads that do not fit empty,
 * with every write kept inside the buffers.
 */
fg_status fg_compact(const fg_shape* shape, const fg_params* params,
                     const void* K, const void* V, const uint8_t* token_class,
                     const uint8_t* policy, const uint32_t* freq_mask,
                     fg_cache* cache, hipStream_t stream);

/* ------------------------------------------------------------------ decode */

/* Workspace bytes for fg_decode_step: B*Hkv * items_per_head * G * (d + 2)
 * fp32 partial states (one slot per work item, at a fixed stride per head). */
size_t fg_decode_workspace_size(const fg_cache* cache);

/*
 * fg_decode_step -- one generated token at position p = cache->next_pos for
 * every (b, KV head) (Method, first paragraph: generation with head-specific
 * caches; stability paragraph: the prompt's policy is reused).
 *   attend set  = cache rows in use with pos >= 0, plus the new token itself
 *                 when level(p, p) <= policy;
 *   out^g       = softmax(q^g . k_j / sqrt(d)) weighted sum of v_j over it
 *                 (zeros if empty);
 *   afterwards the cache holds {j <= p : level(p + 1, j) <= policy}: the new
 *   row is appended (special; punct if policy >= 1; normal if policy 4) or
 *   written to ring slot p mod (w_l - 1) (normal, policy 3), and the ring slot
 *   of position p + 1 - w_l is freed.
 * q [B,Hq,d], k_new / v_new [B,Hkv,d] (cache dtype); new_class [B] u8 or NULL
 * (all normal); out [B,Hq,d] fp32.  An append beyond capacity is skipped and
 * sets bit 1 of error_word.  Increments cache->next_pos.  Two kernel launches:
 * every work item writes a partial softmax state to its slot, then one
 * workgroup per head merges the head's slots and updates that head's cache.
 * Steps on one cache must be issued in order on one stream.
 */
fg_status fg_decode_step(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                         const uint8_t* new_class, float* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fg_decode_step_noalloc -- fg_decode_step for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, arguments, outputs and errors, but the partial
 * softmax states live in a static device array of the library instead of a
 * caller workspace.  Nothing is allocated: no hipMalloc, no hipFree.
 * Limit: fg_decode_workspace_size(cache) must not exceed
 * fg_decode_noalloc_max_bytes() (16 MiB); a larger cache returns
 * FG_ERR_WORKSPACE with a message (use fg_decode_step with a workspace).
 * The array is per GPU (it holds its memory until the process ends) and keeps
 * the last call's contents; every slot the merge reads is written by the same
 * call first, so nothing needs clearing.  All calls on one GPU share it:
 * calls that overlap on one GPU (different streams, or several host threads)
 * race and give wrong outputs -- issue them in order on one stream.
 */
size_t fg_decode_noalloc_max_bytes(void);
fg_status fg_decode_step_noalloc(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 const uint8_t* new_class, float* out, hipStream_t stream);

/* fg_decode_partials -- only the first (split-K) launch of fg_decode_step for
 * the next position: reads the cache and q [B,Hq,d] and writes the partial
 * states into workspace; the cache, its next_pos and any output are left
 * unchanged, so calls may repeat (e.g. to time that launch alone).  Errors as
 * fg_decode_step. */
fg_status fg_decode_partials(const fg_cache* cache, const void* q, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Synchronises the stream and reads error_word: FG_OK, or FG_ERR_CAPACITY
 * when an append was dropped.  *bits_out [host] receives the raw bits if not NULL. */
fg_status fg_cache_error(const fg_cache* cache, uint32_t* bits_out, hipStream_t stream);

/* ------------------------------------------------------------------ decode-time tracking */

/*
 * Accumulated attention during generation (Method, last paragraph: the policy
 * is reused because a head's accumulated attention keeps its shape from the
 * prompt step into later decode steps).  Call fg_decode_track after an
 * fg_decode_step with that step's queries q; with p = cache->next_pos - 1 (the
 * position the step generated), per (b, KV head) hd over the rows the cache
 * holds after the step:
 *   a_gj = softmax_j(q_g . k_j / sqrt(d)) over the cached positions j;
 *   level_bins[hd][k] = (1/G) sum_g sum_{j : level(p, j) = k} a_gj, k = 0..4
 *     (level as fg_profile: 0 special, 1 punct, 2 frequent, 3 p - j < w_l, 4 other);
 *   row_score[row] += sum_g a_gj  (a row holding position p starts from 0).
 * Over a full cache (every head with policy 4) the bins are the level shares
 * of the generated token's whole attention row, the figure to set beside the
 * prompt's recovery.
 *
 * fg_decode_track_init: row_score [total_rows] fp32 := cum_score [B*Hkv*n_prompt]
 *   (fg_profile's output) at rows holding prompt positions, 0 elsewhere.
 * fg_decode_track: token_class [B, n_total] u8 classes of positions
 *   0 .. n_total - 1 (prompt and generated; n_total >= next_pos); freq_mask as
 *   fg_profile wrote it; row_score in/out; level_bins [B*Hkv*5] fp32 out;
 *   workspace fg_decode_track_workspace_size(cache) bytes.  Errors: no step
 *   decoded yet (next_pos == n_prompt) or n_total < next_pos -> FG_ERR_INVALID_ARG.
 */
/*
 * fg_decode_step_dynamic -- fg_decode_step with the frequent set re-ranked
 * during generation (heads of policy 3, local + frequent; every other head as
 * fg_decode_step).  The policy paragraph of Method ranks the frequent set by
 * cumulative attention; here the ranking continues while generating with a
 * fixed budget: after the step's output, the key the local window drops
 * (position p + 1 - w_l, held in the ring slot the new token takes or frees)
 * replaces the cached frequent key of the lowest row_score (ties: the larger
 * position) when its own row_score is larger; otherwise it is dropped as in
 * fg_decode_step.  Frequent keys are the cached rows of class normal outside
 * the ring.  row_score [total_rows] fp32 as kept by fg_decode_track_init and
 * fg_decode_track (call fg_decode_track after every step so the scores are
 * current); token_class [B, n_total] u8 with n_total >= next_pos (classes of
 * every earlier position).  Other arguments, outputs and errors as fg_decode_step.
 */
fg_status fg_decode_step_dynamic(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 const uint8_t* new_class, const uint8_t* token_class, int32_t n_total,
                                 float* row_score, float* out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

fg_status fg_decode_track_init(const fg_cache* cache, const float* cum_score, float* row_score, hipStream_t stream);
size_t fg_decode_track_workspace_size(const fg_cache* cache);
fg_status fg_decode_track(const fg_cache* cache, const void* q, const uint8_t* token_class, int32_t n_total,
                          const uint32_t* freq_mask, float* row_score, float* level_bins, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ measurement */

/*
 * Micro-benchmarks of the chip's own ceilings.  They take no part in the method;
 * they measure the rates the profiling and decode kernels are set against:
 *
 * fg_peak_mfma_bf16: `blocks` workgroups of 256 threads (4 wave64) each run
 *   `iters` iterations of 4 independent v_mfma_f32_32x32x16_bf16 accumulator
 *   chains on register operands: 4 * 32768 * iters flops per wave, i.e.
 *   blocks * 4 * 4 * 32768 * iters flops per call.  operands: 1024 x 16 bytes of
 *   bf16 values read once (16-byte aligned); out [blocks * 256] fp32 (sums kept
 *   so the work is not removed).
 * fg_peak_exp: `blocks` x 256 threads each run `iters` iterations of 8
 *   independent chains x <- 2^(-x) (one v_exp_f32 each): blocks * 256 * 8 * iters
 *   exponentials per call.  out [blocks * 256] fp32.
 * fg_peak_mfma_softmax: `blocks` workgroups of 512 threads (8 wave64; waves w
 *   and w + 4 share a SIMD).  Waves 0-3 run fg_peak_mfma_bf16's loop; waves 4-7
 *   run, per lane and iteration, 8 independent score updates of the profiling
 *   sweeps' softmax (x <- 2^(x c - m), sum += x: one FMA, one v_exp_f32, one
 *   add), i.e. the sweeps' ratio of one score update per lane to each 256 MFMA
 *   flops.  blocks * 4 * 4 * 32768 * iters MFMA flops per call; operands and out
 *   as for fg_peak_mfma_bf16 with out [blocks * 512].  Its MFMA rate is the
 *   ceiling of a sweep whose two kinds of work overlap as well as different
 *   waves of one SIMD can overlap them.
 * fg_peak_copy: copy `bytes` (a multiple of 16, both pointers 16-byte aligned,
 *   not overlapping) from src to dst with 16-byte loads and stores over a
 *   grid-stride loop of `blocks` x 256 threads; nontemporal != 0 stores
 *   non-temporally (as the compaction's gather does).
 * fg_peak_read: read `bytes` (a positive multiple of 16, src 16-byte aligned)
 *   with 16-byte loads, 8 in flight per thread, over a grid-stride loop of
 *   `blocks` x 256 threads; nontemporal != 0 loads non-temporally (as the
 *   decode's split-K launch does).  out [blocks * 256] u32 receives each
 *   thread's XOR of the words it read (kept so the loads are not removed).
 * Errors: FG_ERR_INVALID_ARG for NULL or misaligned pointers, iters < 1,
 * blocks < 1, a byte count that is not a positive multiple of 16, or
 * overlapping copy buffers; FG_ERR_HIP for a failed launch.
 */
fg_status fg_peak_mfma_bf16(const void* operands, float* out, int32_t iters, int32_t blocks, hipStream_t stream);
fg_status fg_peak_exp(float* out, int32_t iters, int32_t blocks, hipStream_t stream);
fg_status fg_peak_mfma_softmax(const void* operands, float* out, int32_t iters, int32_t blocks,
                               hipStream_t stream);
fg_status fg_peak_copy(const void* src, void* dst, size_t bytes, int32_t nontemporal, int32_t blocks,
                       hipStream_t stream);
fg_status fg_peak_read(const void* src, size_t bytes, int32_t nontemporal, int32_t blocks, uint32_t* out,
                       hipStream_t stream);

/* ------------------------------------------------------------------ diagnostics */

const char* fg_status_string(fg_status status);
const char* fg_last_error(void);

/* Kernel timing: when enabled, every launch is bracketed by HIP events on its
 * stream (not for launches recorded into a HIP graph).  fg_kernel_timing_read
 * synchronises those events and returns up to max records (kernel id,
 * milliseconds) accumulated since the last read. */
enum {
  FG_K_ROWSTATS = 0, FG_K_COLSUMS = 1, FG_K_SELECT = 2, FG_K_PLAN = 3, FG_K_SCAN = 4,
  FG_K_GATHER = 5,     /* also writes the decode work list */
  FG_K_WORKLIST = 6,   /* reserved: no separate launch */
  FG_K_DECODE = 7, FG_K_DECODE_MERGE = 8, FG_K_ATTENTION = 9, FG_K_TRACK = 10,
  FG_K_ROWBINS = 11, FG_K_ROWBINS_REDUCE = 12, FG_K_COUNT = 13
};
void fg_kernel_timing_enable(int enable);
int32_t fg_kernel_timing_read(int32_t* kernel_ids, float* ms, int32_t max);
const char* fg_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* FASTGEN_H */
