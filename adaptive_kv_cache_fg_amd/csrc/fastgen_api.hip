// C ABI of libfastgen: argument validation, workspace carving, launches,
// status codes and kernel timing.  Every check runs on the host before any
// launch; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fg_internal.h"

namespace {

thread_local std::string g_last_error;

fg_status fail(fg_status s, const char* msg) {
  g_last_error = msg;
  return s;
}

fg_status hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return FG_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr float kLog2eHost = 1.4426950408889634f;

size_t elem_size(int dtype) { return dtype == FG_DTYPE_BF16 ? 2 : 4; }

fg_status check_shape(const fg_shape* s) {
  if (!s) return fail(FG_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->seq_len < 1)
    return fail(FG_ERR_INVALID_ARG, "batch, heads and seq_len must be >= 1");
  if (s->n_q_heads % s->n_kv_heads != 0) return fail(FG_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (s->head_dim != 64 && s->head_dim != 128) return fail(FG_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (s->dtype != FG_DTYPE_BF16 && s->dtype != FG_DTYPE_F32) return fail(FG_ERR_UNSUPPORTED, "dtype must be bf16 or fp32");
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(FG_ERR_UNSUPPORTED, "group size must be 1, 2, 4 or 8");
  if (s->seq_len > (1 << 24)) return fail(FG_ERR_UNSUPPORTED, "seq_len above 2^24");
  const double rows = (double)s->batch * s->n_q_heads * s->seq_len;
  if (rows * s->head_dim > 4.0e12) return fail(FG_ERR_UNSUPPORTED, "tensor too large");
  if ((double)s->batch * s->n_kv_heads > 2.0e9) return fail(FG_ERR_UNSUPPORTED, "too many heads");
  return FG_OK;
}

fg_status check_params(const fg_params* p) {
  if (!p) return fail(FG_ERR_INVALID_ARG, "params is NULL");
  if (!(p->T > 0.0 && p->T <= 1.0)) return fail(FG_ERR_INVALID_ARG, "T must lie in (0, 1]");
  if (!(p->r_l >= 0.0 && p->r_l <= 1.0) || !(p->r_f >= 0.0 && p->r_f <= 1.0))
    return fail(FG_ERR_INVALID_ARG, "r_l and r_f must lie in [0, 1]");
  return FG_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

void budgets(const fg_shape* s, const fg_params* p, int* k_f, int* w_l) {
  *k_f = (int)std::floor(p->r_f * (double)s->seq_len);
  *w_l = (int)std::floor(p->r_l * (double)s->seq_len);
}

// ---------------------------------------------------------------- kernel timing
struct TimingRec {
  int id;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
thread_local TimingRec g_open = {-1, nullptr, nullptr};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing only: no system-scope fence (cache write-back) when the event is recorded
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace fg {

void timed_begin(int kernel_id, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_open.id = -1;
  if (!g_timing) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  g_open = {kernel_id, a, b};
  (void)hipEventRecord(a, st);
}

void timed_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_open.id < 0) return;
  (void)hipEventRecord(g_open.stop, st);
  g_recs.push_back(g_open);
  g_open.id = -1;
}

}  // namespace fg

extern "C" {

const char* fg_status_string(fg_status s) {
  switch (s) {
    case FG_OK: return "ok";
    case FG_ERR_INVALID_ARG: return "invalid argument";
    case FG_ERR_UNSUPPORTED: return "unsupported";
    case FG_ERR_WORKSPACE: return "workspace too small";
    case FG_ERR_CAPACITY: return "cache capacity exceeded";
    case FG_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* fg_last_error(void) { return g_last_error.c_str(); }

const char* fg_kernel_name(int32_t id) {
  static const char* names[FG_K_COUNT] = {"profile_rowstats", "profile_colsums", "profile_select",
                                          "compact_plan",     "compact_scan",    "compact_gather",
                                          "compact_worklist", "decode_partials", "decode_merge",
                                          "attention",        "decode_track",    "profile_rowbins",
                                          "profile_rowbins_reduce"};
  return (id >= 0 && id < FG_K_COUNT) ? names[id] : "unknown";
}

void fg_kernel_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
}

int32_t fg_kernel_timing_read(int32_t* ids, float* ms, int32_t max) {
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs.swap(g_recs);
  }
  int32_t k = 0;
  auto emit = [&](const TimingRec& r) {
    float t = -1.f;
    if (hipEventSynchronize(r.stop) == hipSuccess) (void)hipEventElapsedTime(&t, r.start, r.stop);
    if (k < max && ids && ms) {
      ids[k] = r.id;
      ms[k] = t;
      ++k;
    }
  };
  for (const TimingRec& r : recs) emit(r);
  std::lock_guard<std::mutex> lk(g_tmu);
  for (const TimingRec& r : recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  return k;
}

namespace {

// Sweep workgroups that run at once on the current device (two per compute
// unit); it only steers the chunk size of a split sweep.
int sweep_slots() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    v = 2 * cus;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace

size_t fg_profile_workspace_size(const fg_shape* s) {
  if (check_shape(s) != FG_OK) return 0;
  const size_t rows_q = (size_t)s->batch * s->n_q_heads * s->seq_len;
  const size_t rows_k = (size_t)s->batch * s->n_kv_heads * s->seq_len;
  // buffer sizes do not depend on the slot count (it only steers the chunk size)
  const fg::SweepSplit sp = fg::sweep_split(s->batch, s->n_q_heads, s->n_kv_heads, s->seq_len, 256, true);
  return align256(rows_q * sizeof(float)) + align256(rows_k * sizeof(float)) + align256(sp.rs_bytes) +
         align256(sp.cs_bytes);
}

namespace {

fg_status check_attention(const fg_shape* shape, const void* Q, const void* K, const void* V, const void* O) {
  if (shape->dtype != FG_DTYPE_BF16) return fail(FG_ERR_UNSUPPORTED, "attention output needs bf16 inputs");
  if (!V || !O) return fail(FG_ERR_INVALID_ARG, "V and O must not be NULL");
  if (!aligned16(V) || !aligned16(O)) return fail(FG_ERR_INVALID_ARG, "V and O must be 16-byte aligned");
  const size_t o_bytes = (size_t)shape->batch * shape->n_q_heads * shape->seq_len * shape->head_dim * 2;
  const size_t kv_bytes = (size_t)shape->batch * shape->n_kv_heads * shape->seq_len * shape->head_dim * 2;
  auto overlaps = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlaps(O, o_bytes, Q, o_bytes) || overlaps(O, o_bytes, K, kv_bytes) || overlaps(O, o_bytes, V, kv_bytes))
    return fail(FG_ERR_INVALID_ARG, "O must not overlap Q, K or V");
  return FG_OK;
}

fg::AttentionArgs attention_args(const fg_shape* shape, const void* Q, const void* K, const void* V, void* O) {
  fg::AttentionArgs a{};
  a.D = shape->head_dim;
  a.B = shape->batch;
  a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads;
  a.n = shape->seq_len;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.cus = sweep_slots() / 2;
  return a;
}

// fg_profile and fg_profile_attention: V and O are NULL for the former
fg_status profile_impl(const fg_shape* shape, const fg_params* params, const void* Q, const void* K, const void* V,
                       const uint8_t* token_class, void* O, uint8_t* policy, float* cum_score, float* recovery,
                       uint32_t* freq_mask, float* lse_out, float* band_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  fg_status s = check_shape(shape);
  if (s != FG_OK) return s;
  if ((s = check_params(params)) != FG_OK) return s;
  if (!Q || !K || !token_class || !policy || !cum_score || !recovery || !freq_mask)
    return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(FG_ERR_INVALID_ARG, "Q and K must be 16-byte aligned");
  const bool with_output = V || O;
  if (with_output && (s = check_attention(shape, Q, K, V, O)) != FG_OK) return s;
  const size_t need = fg_profile_workspace_size(shape);
  if (!workspace || workspace_bytes < need) return fail(FG_ERR_WORKSPACE, "profile workspace too small");
  fg::ProfileArgs a{};
  a.dtype = shape->dtype;
  a.D = shape->head_dim;
  a.B = shape->batch;
  a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads;
  a.n = shape->seq_len;
  budgets(shape, params, &a.k_f, &a.w_l);
  a.T = params->T;
  a.Q = Q;
  a.K = K;
  a.cls = token_class;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  a.lse2 = reinterpret_cast<float*>(ws);
  const size_t rows_q = (size_t)a.B * a.Hq * a.n;
  const size_t rows_k = (size_t)a.B * a.Hkv * a.n;
  a.band = band_out ? band_out : reinterpret_cast<float*>(ws + align256(rows_q * sizeof(float)));
  const fg::SweepSplit sp = fg::sweep_split(a.B, a.Hq, a.Hkv, a.n, sweep_slots() / 2, a.dtype == FG_DTYPE_BF16);
  unsigned char* parts = ws + align256(rows_q * sizeof(float)) + align256(rows_k * sizeof(float));
  a.kchunk = sp.kchunk;
  a.rchunk = sp.rchunk;
  a.cus = sweep_slots() / 2;
  a.rs_part = sp.rs_split ? reinterpret_cast<float2*>(parts) : nullptr;
  a.cs_part = sp.cs_split ? reinterpret_cast<float2*>(parts + align256(sp.rs_bytes)) : nullptr;
  a.lse_out = lse_out;
  a.cum = cum_score;
  a.fmask = freq_mask;
  a.recovery = recovery;
  a.policy = policy;
  if (with_output) {                               // the attention kernel writes the row statistics
    fg::AttentionArgs at = attention_args(shape, Q, K, V, O);
    at.lse2 = a.lse2;
    at.lse_out = lse_out;
    const hipError_t e = fg::launch_attention(at, stream);
    if (e != hipSuccess) return hip_fail(e, "attention");
    a.lse_ready = true;
    a.rs_part = nullptr;
  }
  hipError_t e = fg::launch_profile_sweeps(a, stream);
  if (e != hipSuccess) return hip_fail(e, "profile sweeps");
  e = fg::launch_select(a, stream);
  if (e != hipSuccess) return hip_fail(e, "profile select");
  return FG_OK;
}

}  // namespace

fg_status fg_profile(const fg_shape* shape, const fg_params* params, const void* Q, const void* K,
                     const uint8_t* token_class, uint8_t* policy, float* cum_score, float* recovery,
                     uint32_t* freq_mask, float* lse_out, float* band_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return profile_impl(shape, params, Q, K, nullptr, token_class, nullptr, policy, cum_score, recovery, freq_mask,
                      lse_out, band_out, workspace, workspace_bytes, stream);
}

fg_status fg_profile_attention(const fg_shape* shape, const fg_params* params, const void* Q, const void* K,
                               const void* V, const uint8_t* token_class, void* O, uint8_t* policy, float* cum_score,
                               float* recovery, uint32_t* freq_mask, float* lse_out, float* band_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!V || !O) return fail(FG_ERR_INVALID_ARG, "V and O must not be NULL");
  return profile_impl(shape, params, Q, K, V, token_class, O, policy, cum_score, recovery, freq_mask, lse_out,
                      band_out, workspace, workspace_bytes, stream);
}

fg_status fg_attention(const fg_shape* shape, const void* Q, const void* K, const void* V, void* O, float* lse_out,
                       hipStream_t stream) {
  fg_status s = check_shape(shape);
  if (s != FG_OK) return s;
  if (!Q || !K) return fail(FG_ERR_INVALID_ARG, "Q and K must not be NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(FG_ERR_INVALID_ARG, "Q and K must be 16-byte aligned");
  if ((s = check_attention(shape, Q, K, V, O)) != FG_OK) return s;
  fg::AttentionArgs a = attention_args(shape, Q, K, V, O);
  a.lse_out = lse_out;
  const hipError_t e = fg::launch_attention(a, stream);
  if (e != hipSuccess) return hip_fail(e, "attention");
  return FG_OK;
}

fg_status fg_profile_row_bins(const fg_shape* shape, const fg_params* params, const void* Q, const void* K,
                              const uint8_t* token_class, const uint32_t* freq_mask, const float* lse, float* bins,
                              hipStream_t stream) {
  fg_status s = check_shape(shape);
  if (s != FG_OK) return s;
  if ((s = check_params(params)) != FG_OK) return s;
  if (!Q || !K || !token_class || !freq_mask || !lse || !bins)
    return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(Q) || !aligned16(K)) return fail(FG_ERR_INVALID_ARG, "Q and K must be 16-byte aligned");
  if (shape->batch > 65535) return fail(FG_ERR_UNSUPPORTED, "more than 65535 batch entries");
  if ((double)shape->n_q_heads * ((shape->seq_len + 255) / 256) * 256 > 4294967295.0)
    return fail(FG_ERR_UNSUPPORTED, "too many query heads x row blocks for one launch");
  fg::RowBinsArgs a{};
  a.dtype = shape->dtype;
  a.D = shape->head_dim;
  a.B = shape->batch;
  a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads;
  a.n = shape->seq_len;
  int k_f = 0;
  budgets(shape, params, &k_f, &a.w_l);
  a.Q = Q;
  a.K = K;
  a.cls = token_class;
  a.fmask = freq_mask;
  a.lse = lse;
  a.lse_scale = kLog2eHost;
  a.bins = bins;
  const hipError_t e = fg::launch_rowbins(a, stream);
  if (e != hipSuccess) return hip_fail(e, "row bins");
  return FG_OK;
}

size_t fg_profile_rows_workspace_size(const fg_shape* s) {
  if (check_shape(s) != FG_OK) return 0;
  return fg_profile_workspace_size(s) + align256((size_t)s->batch * s->n_q_heads * s->seq_len * 5 * sizeof(float));
}

fg_status fg_profile_rows(const fg_shape* shape, const fg_params* params, const void* Q, const void* K,
                          const uint8_t* token_class, uint8_t* policy, float* cum_score, float* recovery,
                          uint32_t* freq_mask, float* row_min, float* bins_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  fg_status s = check_shape(shape);
  if (s != FG_OK) return s;
  if ((s = check_params(params)) != FG_OK) return s;
  if (shape->batch > 65535) return fail(FG_ERR_UNSUPPORTED, "more than 65535 batch entries");
  if ((double)shape->n_q_heads * ((shape->seq_len + 255) / 256) * 256 > 4294967295.0)
    return fail(FG_ERR_UNSUPPORTED, "too many query heads x row blocks for one launch");
  const size_t need = fg_profile_rows_workspace_size(shape);
  if (!workspace || workspace_bytes < need) return fail(FG_ERR_WORKSPACE, "profile workspace too small");
  // the sweeps and the top-k: lse2 (log2 domain) at the start of the workspace, cum, F
  s = profile_impl(shape, params, Q, K, nullptr, token_class, nullptr, policy, cum_score, recovery, freq_mask,
                   nullptr, nullptr, workspace, workspace_bytes, stream);
  if (s != FG_OK) return s;
  const size_t bins_off = fg_profile_workspace_size(shape);
  float* bins = bins_out ? bins_out : reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + bins_off);
  fg::RowBinsArgs a{};
  a.dtype = shape->dtype;
  a.D = shape->head_dim;
  a.B = shape->batch;
  a.Hq = shape->n_q_heads;
  a.Hkv = shape->n_kv_heads;
  a.n = shape->seq_len;
  int k_f = 0;
  budgets(shape, params, &k_f, &a.w_l);
  a.Q = Q;
  a.K = K;
  a.cls = token_class;
  a.fmask = freq_mask;
  a.lse = static_cast<const float*>(workspace);            // the sweeps' lse2
  a.lse_scale = 1.0f;
  a.bins = bins;
  hipError_t e = fg::launch_rowbins(a, stream);
  if (e != hipSuccess) return hip_fail(e, "row bins");
  e = fg::launch_rowbins_reduce(bins, shape->batch * shape->n_kv_heads, shape->n_q_heads / shape->n_kv_heads,
                                shape->seq_len, params->T, recovery, policy, row_min, stream);
  if (e != hipSuccess) return hip_fail(e, "row bins reduce");
  return FG_OK;
}

fg_status fg_head_map_accumulate(int32_t n_prompts, int32_t n_kv_heads, const float* recovery, const uint8_t* policy,
                                 double* rec_sum, int32_t* policy_count, hipStream_t stream) {
  if (n_prompts < 1 || n_kv_heads < 1) return fail(FG_ERR_INVALID_ARG, "n_prompts and n_kv_heads must be >= 1");
  if ((double)n_prompts * n_kv_heads * 5 > 2.0e9) return fail(FG_ERR_UNSUPPORTED, "too many prompts x heads");
  if (!recovery || !policy || !rec_sum || !policy_count) return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  const hipError_t e = fg::launch_head_map_accumulate(recovery, policy, rec_sum, policy_count, n_prompts, n_kv_heads,
                                                      stream);
  if (e != hipSuccess) return hip_fail(e, "head map accumulate");
  return FG_OK;
}

fg_status fg_head_map_finish(int32_t n_kv_heads, int64_t n_prompts, const fg_params* params, const double* rec_sum,
                             float* mean_recovery, uint8_t* policy, hipStream_t stream) {
  fg_status s = check_params(params);
  if (s != FG_OK) return s;
  if (n_kv_heads < 1 || n_prompts < 1) return fail(FG_ERR_INVALID_ARG, "n_prompts and n_kv_heads must be >= 1");
  if (!rec_sum || !mean_recovery || !policy) return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  const hipError_t e = fg::launch_head_map_finish(rec_sum, (double)n_prompts, params->T, mean_recovery, policy,
                                                  n_kv_heads, stream);
  if (e != hipSuccess) return hip_fail(e, "head map finish");
  return FG_OK;
}

int32_t fg_decode_chunk_rows(const fg_shape* shape) {
  if (check_shape(shape) != FG_OK) return 0;
  return fg::decode_chunk_rows(shape->seq_len);
}

fg_status fg_compact_plan(const fg_shape* shape, const fg_params* params, const uint8_t* token_class,
                          const uint8_t* policy, const uint32_t* freq_mask, int32_t max_new_tokens,
                          int32_t max_new_kept, int32_t* kept_count, int32_t* ring, int32_t* capacity,
                          int64_t* row_offset, int64_t* work_offset, int64_t* totals, hipStream_t stream) {
  fg_status s = check_shape(shape);
  if (s != FG_OK) return s;
  if ((s = check_params(params)) != FG_OK) return s;
  if (!token_class || !policy || !freq_mask || !kept_count || !ring || !capacity || !row_offset || !work_offset ||
      !totals)
    return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (max_new_tokens < 0 || max_new_kept < 0 || max_new_kept > max_new_tokens)
    return fail(FG_ERR_INVALID_ARG, "need 0 <= max_new_kept <= max_new_tokens");
  if ((double)shape->seq_len + max_new_tokens > 2.0e9) return fail(FG_ERR_UNSUPPORTED, "capacity above 2^31");
  fg::PlanArgs a{};
  a.B = shape->batch;
  a.Hkv = shape->n_kv_heads;
  a.n = shape->seq_len;
  int k_f = 0;
  budgets(shape, params, &k_f, &a.w_l);
  a.max_new = max_new_tokens;
  a.max_new_kept = max_new_kept;
  a.cls = token_class;
  a.policy = policy;
  a.fmask = freq_mask;
  a.kept_count = kept_count;
  a.ring = ring;
  a.capacity = capacity;
  a.row_offset = row_offset;
  a.work_offset = work_offset;
  a.totals = totals;
  a.chunk_rows = fg::decode_chunk_rows(shape->seq_len);
  hipError_t e = fg::launch_plan(a, stream);
  if (e != hipSuccess) return hip_fail(e, "compact plan");
  return FG_OK;
}

static fg_status check_cache_views(const fg_cache* c, const fg_shape* shape) {
  if (!c) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  if (!c->k || !c->v || !c->pos || !c->row_offset || !c->len || !c->capacity || !c->ring || !c->policy ||
      !c->work_offset || !c->error_word || (c->n_work > 0 && !c->work))
    return fail(FG_ERR_INVALID_ARG, "a cache buffer is NULL");
  if (!aligned16(c->k) || !aligned16(c->v)) return fail(FG_ERR_INVALID_ARG, "cache k and v must be 16-byte aligned");
  if (c->total_rows < 0 || c->total_rows > 0x7fffffff || c->n_work < 0 || c->n_work > 0x7fffffff / 4)
    return fail(FG_ERR_INVALID_ARG, "bad total_rows or n_work (both must fit 32-bit row and item indices)");
  if (c->items_per_head < 1 || c->items_per_head > 0x7fffffff ||
      (int64_t)shape->batch * shape->n_kv_heads * c->items_per_head < c->n_work)
    return fail(FG_ERR_INVALID_ARG, "items_per_head must be the largest work-item count of a head");
  return FG_OK;
}

fg_status fg_compact(const fg_shape* shape, const fg_params* params, const void* K, const void* V,
                     const uint8_t* token_class, const uint8_t* policy, const uint32_t* freq_mask, fg_cache* cache,
                     hipStream_t stream) {
  fg_status s = check_shape(shape);
  if (s != FG_OK) return s;
  if ((s = check_params(params)) != FG_OK) return s;
  if ((s = check_cache_views(cache, shape)) != FG_OK) return s;
  if (!K || !V || !token_class || !policy || !freq_mask) return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(K) || !aligned16(V)) return fail(FG_ERR_INVALID_ARG, "K and V must be 16-byte aligned");
  fg::GatherArgs a{};
  a.dtype = shape->dtype;
  a.D = shape->head_dim;
  a.B = shape->batch;
  a.Hkv = shape->n_kv_heads;
  a.n = shape->seq_len;
  int k_f = 0;
  budgets(shape, params, &k_f, &a.w_l);
  a.K = K;
  a.V = V;
  a.cls = token_class;
  a.policy = policy;
  a.fmask = freq_mask;
  a.row_offset = cache->row_offset;
  a.ring = cache->ring;
  a.work_offset = cache->work_offset;
  a.Kc = cache->k;
  a.Vc = cache->v;
  a.pos = cache->pos;
  a.len = cache->len;
  a.work = cache->work;
  a.error_word = cache->error_word;
  a.chunk_rows = fg::decode_chunk_rows(shape->seq_len);
  a.total_rows = cache->total_rows;
  a.n_work = cache->n_work;
  a.items_per_head = (int)cache->items_per_head;
  hipError_t e = fg::launch_gather(a, stream);
  if (e != hipSuccess) return hip_fail(e, "compact gather");
  cache->shape = *shape;
  cache->n_prompt = shape->seq_len;
  cache->w_l = a.w_l;
  cache->next_pos = shape->seq_len;
  cache->chunk_rows = a.chunk_rows;
  return FG_OK;
}

size_t fg_decode_workspace_size(const fg_cache* c) {
  if (!c || check_shape(&c->shape) != FG_OK) return 0;
  const int G = c->shape.n_q_heads / c->shape.n_kv_heads;
  const int64_t slots = (int64_t)c->shape.batch * c->shape.n_kv_heads * (c->items_per_head > 0 ? c->items_per_head : 1);
  return align256((size_t)slots * G * (c->shape.head_dim + 2) * sizeof(float));
}

// Shared by fg_decode_step and fg_decode_partials (partials_only: no merge
// launch, the cache and next_pos are left unchanged, k_new / v_new / out unused).
static fg_status decode_launch(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                               const uint8_t* new_class, float* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, bool partials_only, float* row_score = nullptr,
                               const uint8_t* token_class = nullptr, int32_t n_total = 0) {
  if (!cache) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  fg_status s = check_shape(&cache->shape);
  if (s != FG_OK) return s;
  if ((s = check_cache_views(cache, &cache->shape)) != FG_OK) return s;
  if (!q || (!partials_only && (!k_new || !v_new || !out))) return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(q)) return fail(FG_ERR_INVALID_ARG, "q must be 16-byte aligned");
  if (cache->next_pos < cache->n_prompt || cache->next_pos >= 0x7fffffff)
    return fail(FG_ERR_INVALID_ARG, "cache position out of range (was fg_compact called?)");
  if (cache->chunk_rows != fg::decode_chunk_rows(cache->shape.seq_len))
    return fail(FG_ERR_INVALID_ARG, "cache chunk_rows does not match its shape (was fg_compact called?)");
  if (!workspace || workspace_bytes < fg_decode_workspace_size(cache))
    return fail(FG_ERR_WORKSPACE, "decode workspace too small");
  fg::DecodeArgs a{};
  a.dtype = cache->shape.dtype;
  a.D = cache->shape.head_dim;
  a.B = cache->shape.batch;
  a.Hq = cache->shape.n_q_heads;
  a.Hkv = cache->shape.n_kv_heads;
  a.w_l = cache->w_l;
  a.p = cache->next_pos;
  a.n_work = cache->n_work;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_class = new_class;
  a.out = out;
  a.part = static_cast<float*>(workspace);
  a.Kc = cache->k;
  a.Vc = cache->v;
  a.pos = cache->pos;
  a.row_offset = cache->row_offset;
  a.len = cache->len;
  a.capacity = cache->capacity;
  a.ring = cache->ring;
  a.policy = cache->policy;
  a.work_offset = cache->work_offset;
  a.work = cache->work;
  a.error_word = cache->error_word;
  a.chunk_rows = cache->chunk_rows;
  a.items_per_head = (int)cache->items_per_head;
  a.total_rows = cache->total_rows;
  a.partials_only = partials_only;
  a.score = row_score;
  a.cls_all = token_class;
  a.n_total = n_total;
  hipError_t e = fg::launch_decode(a, stream);
  if (e != hipSuccess) return hip_fail(e, "decode step");
  if (!partials_only) cache->next_pos += 1;
  return FG_OK;
}

fg_status fg_decode_step(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                         const uint8_t* new_class, float* out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return decode_launch(cache, q, k_new, v_new, new_class, out, workspace, workspace_bytes, stream, false);
}

fg_status fg_decode_step_dynamic(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 const uint8_t* new_class, const uint8_t* token_class, int32_t n_total,
                                 float* row_score, float* out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (!cache) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  if (!token_class || !row_score) return fail(FG_ERR_INVALID_ARG, "token_class and row_score must not be NULL");
  if (n_total < cache->next_pos) return fail(FG_ERR_INVALID_ARG, "token_class must cover every position so far");
  return decode_launch(cache, q, k_new, v_new, new_class, out, workspace, workspace_bytes, stream, false, row_score,
                       token_class, n_total);
}

}  // extern "C"

// ---------------------------------------------------------------- decode without a caller workspace
// The partial softmax states of fg_decode_step_noalloc live in this file-scope
// device array (one copy per GPU, held until the process ends).  Host code
// never uses the array's name as an address: the device address is taken once
// per device with hipGetSymbolAddress and kept per device.
namespace {

constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of the scratch array (looked up on the first call per device).
fg_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FG_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FG_OK;
}

}  // namespace

extern "C" {

size_t fg_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

fg_status fg_decode_step_noalloc(fg_cache* cache, const void* q, const void* k_new, const void* v_new,
                                 const uint8_t* new_class, float* out, hipStream_t stream) {
  if (!cache) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  fg_status s = check_shape(&cache->shape);
  if (s != FG_OK) return s;
  if ((s = check_cache_views(cache, &cache->shape)) != FG_OK) return s;
  const size_t need = fg_decode_workspace_size(cache);
  if (need > kDecodeScratchBytes) {
    g_last_error = "decode state of " + std::to_string(need) + " bytes exceeds the static scratch of " +
                   std::to_string(kDecodeScratchBytes) + " bytes; use fg_decode_step with a workspace";
    return FG_ERR_WORKSPACE;
  }
  void* ptr = nullptr;
  if ((s = scratch_for_current_device(&ptr)) != FG_OK) return s;
  return decode_launch(cache, q, k_new, v_new, new_class, out, ptr, kDecodeScratchBytes, stream, false);
}

fg_status fg_decode_partials(const fg_cache* cache, const void* q, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (!cache) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  fg_cache c = *cache;                                  // next_pos is not advanced
  return decode_launch(&c, q, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, true);
}

fg_status fg_decode_track_init(const fg_cache* cache, const float* cum_score, float* row_score, hipStream_t stream) {
  if (!cache) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  fg_status s = check_shape(&cache->shape);
  if (s != FG_OK) return s;
  if ((s = check_cache_views(cache, &cache->shape)) != FG_OK) return s;
  if (!cum_score || !row_score) return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (cache->n_prompt != cache->shape.seq_len) return fail(FG_ERR_INVALID_ARG, "cache not compacted");
  const hipError_t e = fg::launch_track_init(cache->row_offset, cache->pos, cum_score, row_score,
                                             cache->shape.batch * cache->shape.n_kv_heads, cache->n_prompt, stream);
  if (e != hipSuccess) return hip_fail(e, "track init");
  return FG_OK;
}

size_t fg_decode_track_workspace_size(const fg_cache* c) {
  if (!c || check_shape(&c->shape) != FG_OK || c->items_per_head < 1) return 0;
  return fg::track_workspace_bytes((int64_t)c->shape.batch * c->shape.n_kv_heads, c->items_per_head,
                                   c->shape.n_q_heads / c->shape.n_kv_heads);
}

fg_status fg_decode_track(const fg_cache* cache, const void* q, const uint8_t* token_class, int32_t n_total,
                          const uint32_t* freq_mask, float* row_score, float* level_bins, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (!cache) return fail(FG_ERR_INVALID_ARG, "cache is NULL");
  fg_status s = check_shape(&cache->shape);
  if (s != FG_OK) return s;
  if ((s = check_cache_views(cache, &cache->shape)) != FG_OK) return s;
  if (!q || !token_class || !freq_mask || !row_score || !level_bins)
    return fail(FG_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(q)) return fail(FG_ERR_INVALID_ARG, "q must be 16-byte aligned");
  if (cache->n_prompt != cache->shape.seq_len || cache->next_pos <= cache->n_prompt || cache->next_pos >= 0x7fffffff)
    return fail(FG_ERR_INVALID_ARG, "no decode step to track (call after fg_decode_step)");
  if (n_total < cache->next_pos) return fail(FG_ERR_INVALID_ARG, "token_class must cover every position so far");
  if (cache->chunk_rows != fg::decode_chunk_rows(cache->shape.seq_len))
    return fail(FG_ERR_INVALID_ARG, "cache chunk_rows does not match its shape (was fg_compact called?)");
  const size_t need = fg_decode_track_workspace_size(cache);
  if (!workspace || workspace_bytes < need) return fail(FG_ERR_WORKSPACE, "track workspace too small");
  fg::TrackArgs a{};
  a.dtype = cache->shape.dtype;
  a.D = cache->shape.head_dim;
  a.B = cache->shape.batch;
  a.Hq = cache->shape.n_q_heads;
  a.Hkv = cache->shape.n_kv_heads;
  a.w_l = cache->w_l;
  a.p = cache->next_pos - 1;
  a.n_prompt = cache->n_prompt;
  a.n_total = n_total;
  a.n_work = cache->n_work;
  a.q = q;
  a.Kc = cache->k;
  a.pos = cache->pos;
  a.work = cache->work;
  a.work_offset = cache->work_offset;
  a.cls = token_class;
  a.fmask = freq_mask;
  a.score = row_score;
  a.level_bins = level_bins;
  a.workspace = workspace;
  a.chunk_rows = cache->chunk_rows;
  a.items_per_head = (int)cache->items_per_head;
  if (a.n_work == 0) return FG_OK;
  const hipError_t e = fg::launch_track(a, stream);
  if (e != hipSuccess) return hip_fail(e, "decode track");
  return FG_OK;
}

fg_status fg_peak_mfma_bf16(const void* operands, float* out, int32_t iters, int32_t blocks, hipStream_t stream) {
  if (!operands || !out) return fail(FG_ERR_INVALID_ARG, "operands and out must not be NULL");
  if (!aligned16(operands)) return fail(FG_ERR_INVALID_ARG, "operands must be 16-byte aligned");
  if (iters < 1 || blocks < 1) return fail(FG_ERR_INVALID_ARG, "iters and blocks must be >= 1");
  const hipError_t e = fg::launch_peak_mfma(operands, out, iters, blocks, stream);
  if (e != hipSuccess) return hip_fail(e, "peak mfma");
  return FG_OK;
}

fg_status fg_peak_mfma_softmax(const void* operands, float* out, int32_t iters, int32_t blocks,
                               hipStream_t stream) {
  if (!operands || !out) return fail(FG_ERR_INVALID_ARG, "operands and out must not be NULL");
  if (!aligned16(operands)) return fail(FG_ERR_INVALID_ARG, "operands must be 16-byte aligned");
  if (iters < 1 || blocks < 1) return fail(FG_ERR_INVALID_ARG, "iters and blocks must be >= 1");
  const hipError_t e = fg::launch_peak_mfma_softmax(operands, out, iters, blocks, stream);
  if (e != hipSuccess) return hip_fail(e, "peak mfma softmax");
  return FG_OK;
}

fg_status fg_peak_exp(float* out, int32_t iters, int32_t blocks, hipStream_t stream) {
  if (!out) return fail(FG_ERR_INVALID_ARG, "out must not be NULL");
  if (iters < 1 || blocks < 1) return fail(FG_ERR_INVALID_ARG, "iters and blocks must be >= 1");
  const hipError_t e = fg::launch_peak_exp(out, iters, blocks, stream);
  if (e != hipSuccess) return hip_fail(e, "peak exp");
  return FG_OK;
}

fg_status fg_peak_copy(const void* src, void* dst, size_t bytes, int32_t nontemporal, int32_t blocks,
                       hipStream_t stream) {
  if (!src || !dst) return fail(FG_ERR_INVALID_ARG, "src and dst must not be NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(FG_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0) return fail(FG_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (blocks < 1) return fail(FG_ERR_INVALID_ARG, "blocks must be >= 1");
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return fail(FG_ERR_INVALID_ARG, "src and dst overlap");
  const hipError_t e = fg::launch_peak_copy(src, dst, bytes, nontemporal != 0, blocks, stream);
  if (e != hipSuccess) return hip_fail(e, "peak copy");
  return FG_OK;
}

fg_status fg_peak_read(const void* src, size_t bytes, int32_t nontemporal, int32_t blocks, uint32_t* out,
                       hipStream_t stream) {
  if (!src || !out) return fail(FG_ERR_INVALID_ARG, "src and out must not be NULL");
  if (!aligned16(src)) return fail(FG_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0) return fail(FG_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (blocks < 1) return fail(FG_ERR_INVALID_ARG, "blocks must be >= 1");
  const hipError_t e = fg::launch_peak_read(src, bytes, nontemporal != 0, blocks, out, stream);
  if (e != hipSuccess) return hip_fail(e, "peak read");
  return FG_OK;
}

fg_status fg_cache_error(const fg_cache* cache, uint32_t* bits_out, hipStream_t stream) {
  if (!cache || !cache->error_word) return fail(FG_ERR_INVALID_ARG, "cache or error_word is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  uint32_t bits = 0;
  e = hipMemcpy(&bits, cache->error_word, sizeof(bits), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "read error word");
  if (bits_out) *bits_out = bits;
  return bits ? fail(FG_ERR_CAPACITY, "a cache append exceeded its capacity") : FG_OK;
}

}  // extern "C"
