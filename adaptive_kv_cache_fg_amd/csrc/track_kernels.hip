// Decode-time tracking of accumulated attention: after a decode step, the
// attention of the step's queries over each head's cache, split by shortlist
// level, and every cached key's cumulative attention score carried on from the
// prompt.
//
// FastGen reuses the prompt's policy during generation because a head's
// accumulated attention keeps its shape from prompt encoding into decoding
// (hyper.ai summary of "Model Tells You What to Discard", Method, last
// paragraph, which compares accumulated scores at the prompt step and at later
// decode steps).  These kernels measure that on the device: the level shares of
// each generated token's attention (over a full cache: how its attention splits
// between special, punct, frequent, local and other keys) and the cumulative
// score of every cached key, the quantity that ranks the frequent set, updated
// step by step.
//
// Three launches over the decode work list (one workgroup per work item, rows
// spread over lanes as in the decode kernels):
//   stats:  per item and query head, max and sum of 2^x over its rows
//           (x = q . k * log2(e) / sqrt(d));
//   apply:  every workgroup merges its head's item stats into the row
//           log-sum-exp, recomputes x, and for each row adds
//           w = sum_g 2^(x_g - lse2_g) to its score (a row holding the step's
//           own token starts from 0) and w to its level's bin; per-item bins
//           go to the workspace;
//   bins:   per head, the items' bins summed in item order, divided by G.
// Every sum runs in a fixed order, so results do not depend on scheduling.
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

namespace {

template <typename T> struct Row16;
template <> struct Row16<__bf16> {
  static constexpr int N = 8;
  using raw_t = bf16x8;
  static __device__ __forceinline__ void cvt(const raw_t& v, float* out) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  }
};
template <> struct Row16<float> {
  static constexpr int N = 4;
  using raw_t = f32x4;
  static __device__ __forceinline__ void cvt(const raw_t& v, float* out) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = v[e];
  }
};

constexpr int kTrackThreads = 256;

// x_g = q_g . k_row * c for the G query heads; every lane of the row's group gets the sums
template <typename T, int D, int G>
__device__ __forceinline__ void row_scores(const float (&qv)[G][Row16<T>::N], const T* krow, int sl, float c,
                                           float (&x)[G]) {
  using V = Row16<T>;
  constexpr int LPR = D / V::N;
  float kv[V::N];
  V::cvt(*reinterpret_cast<const typename V::raw_t*>(krow + sl * V::N), kv);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < V::N; ++e) s = fmaf(qv[g][e], kv[e], s);
    x[g] = group_sum<LPR>(s) * c;
  }
}

template <typename T, int D, int G>
__device__ __forceinline__ void load_q(const T* q, int hd, int sl, float (&qv)[G][Row16<T>::N]) {
  using V = Row16<T>;
#pragma unroll
  for (int g = 0; g < G; ++g)
    V::cvt(*reinterpret_cast<const typename V::raw_t*>(q + ((size_t)hd * G + g) * D + sl * V::N), qv[g]);
}

}  // namespace

template <typename T, int D, int G>
__global__ __launch_bounds__(kTrackThreads) void track_stats_kernel(const T* __restrict__ q,
                                                                    const int32_t* __restrict__ work,
                                                                    const T* __restrict__ Kc,
                                                                    const int32_t* __restrict__ pos,
                                                                    float2* __restrict__ stats, int S, int CH,
                                                                    float c) {
  using V = Row16<T>;
  constexpr int LPR = D / V::N, RPP = kWave / LPR, kWaves = kTrackThreads / kWave;
  __shared__ float sm[kWaves][G], sl[kWaves][G];
  const int4 wk = reinterpret_cast<const int4*>(work)[blockIdx.x];   // (head, first row, first absolute row, rows)
  if (wk.x < 0) return;                                              // an empty item (uniform)
  const int hd = wk.x, k_item = wk.y / CH, abs0 = wk.z, n_use = wk.w;
  const int wave = wave_id(), lane = threadIdx.x & 63, sub = lane / LPR, sl_ = lane % LPR;
  float qv[G][V::N];
  load_q<T, D, G>(q, hd, sl_, qv);
  float m[G], l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
  }
  for (int r = wave * RPP + sub; r - sub < n_use; r += kWaves * RPP) {   // the row group's loop is uniform
    const bool in = r < n_use;
    const int64_t gr = (int64_t)abs0 + (in ? r : 0);
    float x[G];
    row_scores<T, D, G>(qv, Kc + gr * D, sl_, c, x);
    const bool valid = in && pos[gr] >= 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!valid) continue;
      const float mn = fmaxf(m[g], x[g]);
      l[g] = l[g] * fast_exp2(m[g] - mn) + fast_exp2(x[g] - mn);
      m[g] = mn;
    }
  }
  // lanes of one row group hold the same values; merge the RPP groups of the wave, then the waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    for (int o = LPR; o < kWave; o <<= 1) {
      const float mo = __shfl_xor(m[g], o), lo = __shfl_xor(l[g], o);
      const float mn = fmaxf(m[g], mo);
      l[g] = l[g] * fast_exp2(m[g] - mn) + lo * fast_exp2(mo - mn);
      m[g] = mn;
    }
    if (lane == 0) {
      sm[wave][g] = m[g];
      sl[wave][g] = l[g];
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = kNegBig, L = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float mn = fmaxf(M, sm[w][g]);
      L = L * fast_exp2(M - mn) + sl[w][g] * fast_exp2(sm[w][g] - mn);
      M = mn;
    }
    stats[((size_t)hd * S + k_item) * G + g] = make_float2(M, L);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kTrackThreads) void track_apply_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ work, const int64_t* __restrict__ work_offset,
    const T* __restrict__ Kc, const int32_t* __restrict__ pos, const float2* __restrict__ stats,
    const uint8_t* __restrict__ cls, const uint32_t* __restrict__ fmask, float* __restrict__ score,
    float* __restrict__ bins_part, int Hkv, int S, int CH, int n_prompt, int n_total, int w_l, int p, float c) {
  using V = Row16<T>;
  constexpr int LPR = D / V::N, RPP = kWave / LPR, kWaves = kTrackThreads / kWave;
  __shared__ float sbin[kWaves][5];
  const int4 wk = reinterpret_cast<const int4*>(work)[blockIdx.x];
  if (wk.x < 0) return;
  const int hd = wk.x, k_item = wk.y / CH, abs0 = wk.z, n_use = wk.w;
  const int b = hd / Hkv;
  const int wave = wave_id(), lane = threadIdx.x & 63, sub = lane / LPR, sl_ = lane % LPR;
  // the head's row log-sum-exp per query head, merged from its items in item order (every wave alike)
  const int64_t n_it = work_offset[hd + 1] - work_offset[hd];
  const int n_items = (int)(n_it < S ? n_it : S);
  float lse2[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float M = kNegBig, L = 0.f;
    for (int i0 = 0; i0 < n_items; i0 += kWave) {
      const int i = i0 + lane;
      const float2 st = i < n_items ? stats[((size_t)hd * S + i) * G + g] : make_float2(kNegBig, 0.f);
      float mm = st.y > 0.f ? st.x : kNegBig;
      for (int o = 1; o < kWave; o <<= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
      float ll = st.y > 0.f ? st.y * fast_exp2(st.x - mm) : 0.f;
      for (int o = 1; o < kWave; o <<= 1) ll += __shfl_xor(ll, o);
      const float mn = fmaxf(M, mm);
      L = L * fast_exp2(M - mn) + ll * fast_exp2(mm - mn);
      M = mn;
    }
    lse2[g] = L > 0.f ? M + fast_log2(L) : INFINITY;          // no row in use: every weight is 0
  }
  float qv[G][V::N];
  load_q<T, D, G>(q, hd, sl_, qv);
  const int nw = (n_prompt + 31) >> 5;
  const size_t cls_base = (size_t)b * n_total;
  float bin[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = wave * RPP + sub; r - sub < n_use; r += kWaves * RPP) {
    const bool in = r < n_use;
    const int64_t gr = (int64_t)abs0 + (in ? r : 0);
    float x[G];
    row_scores<T, D, G>(qv, Kc + gr * D, sl_, c, x);
    const int j = pos[gr];
    if (!in || j < 0 || sl_ != 0) continue;                   // one lane per row from here on
    float w = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) w += fast_exp2(x[g] - lse2[g]);
    score[gr] = (j == p ? 0.f : score[gr]) + w;
    const uint8_t cj = j < n_total ? cls[cls_base + j] : kNormal;
    const bool fj = j < n_prompt && ((fmask[(size_t)hd * nw + (j >> 5)] >> (j & 31)) & 1u);
    const int lev = cj == kSpecial ? 0 : cj == kPunct ? 1 : fj ? 2 : (p - j < w_l) ? 3 : 4;
#pragma unroll
    for (int k = 0; k < 5; ++k) bin[k] += (k == lev) ? w : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    float v = bin[k];
    for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o);
    if (lane == 0) sbin[wave][k] = v;
  }
  __syncthreads();
  if (threadIdx.x < 5) {
    float v = 0.f;
    for (int w = 0; w < kWaves; ++w) v += sbin[w][threadIdx.x];
    bins_part[((size_t)hd * S + k_item) * 5 + threadIdx.x] = v;
  }
}

__global__ __launch_bounds__(256) void track_bins_kernel(const int64_t* __restrict__ work_offset,
                                                         const float* __restrict__ bins_part,
                                                         float* __restrict__ level_bins, int H, int S, int G) {
  const int hd = blockIdx.x * blockDim.x + threadIdx.x;
  if (hd >= H) return;
  const int64_t n_it = work_offset[hd + 1] - work_offset[hd];
  const int n_items = (int)(n_it < S ? n_it : S);
  float v[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n_items; ++i)
#pragma unroll
    for (int k = 0; k < 5; ++k) v[k] += bins_part[((size_t)hd * S + i) * 5 + k];
#pragma unroll
  for (int k = 0; k < 5; ++k) level_bins[(size_t)hd * 5 + k] = v[k] / (float)G;
}

// Scores of a freshly compacted cache: a row holding prompt position j starts at
// cum[head][j]; every other row at 0.
__global__ __launch_bounds__(256) void track_init_kernel(const int64_t* __restrict__ row_offset,
                                                         const int32_t* __restrict__ pos,
                                                         const float* __restrict__ cum, float* __restrict__ score,
                                                         int n_prompt) {
  const int hd = blockIdx.x;
  const int64_t r0 = row_offset[hd], r1 = row_offset[hd + 1];
  for (int64_t r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
    const int j = pos[r];
    score[r] = (j >= 0 && j < n_prompt) ? cum[(size_t)hd * n_prompt + j] : 0.f;
  }
}

template <typename T, int D, int G>
static hipError_t launch_track_t(const TrackArgs& a, hipStream_t st) {
  const float c = kLog2e / sqrtf((float)D);
  const int S = a.items_per_head;
  float2* stats = reinterpret_cast<float2*>(a.workspace);
  float* bins_part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(a.workspace) +
                                              track_stats_bytes(a.B * a.Hkv, S, G));
  track_stats_kernel<T, D, G><<<dim3((unsigned)a.n_work), dim3(kTrackThreads), 0, st>>>(
      (const T*)a.q, a.work, (const T*)a.Kc, a.pos, stats, S, a.chunk_rows, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  track_apply_kernel<T, D, G><<<dim3((unsigned)a.n_work), dim3(kTrackThreads), 0, st>>>(
      (const T*)a.q, a.work, a.work_offset, (const T*)a.Kc, a.pos, stats, a.cls, a.fmask, a.score, bins_part, a.Hkv,
      S, a.chunk_rows, a.n_prompt, a.n_total, a.w_l, a.p, c);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int H = a.B * a.Hkv;
  track_bins_kernel<<<dim3((unsigned)((H + 255) / 256)), dim3(256), 0, st>>>(a.work_offset, bins_part,
                                                                            a.level_bins, H, S, G);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_track_g(const TrackArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_track_t<T, D, 1>(a, st);
    case 2: return launch_track_t<T, D, 2>(a, st);
    case 4: return launch_track_t<T, D, 4>(a, st);
    default: return launch_track_t<T, D, 8>(a, st);
  }
}

hipError_t launch_track(const TrackArgs& a, hipStream_t st) {
  timed_begin(FG_K_TRACK, st);
  hipError_t e;
  if (a.dtype == FG_DTYPE_BF16)
    e = a.D == 128 ? launch_track_g<__bf16, 128>(a, st) : launch_track_g<__bf16, 64>(a, st);
  else
    e = a.D == 128 ? launch_track_g<float, 128>(a, st) : launch_track_g<float, 64>(a, st);
  timed_end(st);
  return e;
}

hipError_t launch_track_init(const int64_t* row_offset, const int32_t* pos, const float* cum, float* score, int H,
                             int n_prompt, hipStream_t st) {
  track_init_kernel<<<dim3((unsigned)H), dim3(256), 0, st>>>(row_offset, pos, cum, score, n_prompt);
  return hipGetLastError();
}

}  // namespace fg
