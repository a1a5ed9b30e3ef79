// Frequent-set selection, per-policy recovery and policy choice, one
// workgroup per (batch entry, KV head).
//
// hyper.ai summary of "Model Tells You What to Discard", Method: the frequent
// policy keeps the tokens with the largest cumulative attention, budgeted by a
// ratio r_f (policy paragraph); the shortlist is the nested unions special,
// +punct, +frequent, +local, full (shortlist equation); the chosen entry is
// the cheapest whose reconstruction stays within 1 - T of the attention map
// (constraint equation).
//
// * Top-k: radix select on the fp32 bit patterns of cum (non-negative, so the
//   patterns order like the values), four 8-bit digits from the top, giving
//   the exact k-th largest pattern; keys above it are taken, and among keys
//   equal to it the lowest indices (a ballot / popcount prefix in index order).
// * Recovery: every pair (i, j) falls at the first shortlist level that keeps
//   it, so the mass a level adds is a column-sum identity over keys:
//   special keys add cum_j at level 0, punct keys at level 1, frequent keys at
//   level 2, and every other key adds only its local band sum at level 3.
//   The O(n) reduction runs in fp64.
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

// Block sums of four fp64 values at once (one shuffle ladder and one barrier
// for all four); the totals are valid in thread 0.
template <int NT>
__device__ __forceinline__ void block_sum4(double (&v)[4], double (*red)[NT / 64]) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] += __shfl_xor(v[k], o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < 4; ++k) red[k][wave] = v[k];
  __syncthreads();
  if (threadIdx.x == 0)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      double t = 0.0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[k][w];
      v[k] = t;
    }
}

// NT threads per workgroup.  VPT > 0: each thread holds the scores (and band sums) of
// keys tid + k * NT, k < VPT, in registers for every pass (n <= VPT * NT); VPT = 0:
// every pass reads them from memory (long prompts).
template <int VPT, int NT>
__global__ __launch_bounds__(NT) void select_kernel(float* __restrict__ cum, float* __restrict__ band,
                                                             const float2* __restrict__ cs_part, int rchunk,
                                                             const uint8_t* __restrict__ cls, int Hkv, int n, int G,
                                                             int k_f, double T, uint32_t* __restrict__ fmask,
                                                             float* __restrict__ recovery, uint8_t* __restrict__ policy) {
  constexpr int NV = VPT > 0 ? VPT : 1;
  __shared__ unsigned hist[256];
  __shared__ unsigned s_sel, s_rem, s_cnt;
  __shared__ int wave_cnt[NT / 64];
  __shared__ double red[4][NT / 64];

  const int bh = blockIdx.x, b = bh / Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_waves = blockDim.x >> 6;
  const int n_it = (n + NT - 1) / NT;                     // key batches of NT
  float cv[NV], bv[NV];
  if (cs_part) {
    // the column sweep ran in row chunks: add each key's partial sums in chunk order
    const int nbh = gridDim.x;
    for (int it = 0; it < (VPT > 0 ? VPT : n_it); ++it) {
      const int j = it * NT + tid;
      float cs = 0.f, bs = 0.f;
      if (j < n) {
        const int nc = split_count(n - (j / kSweepKeysPerWG) * kSweepKeysPerWG, rchunk);
        for (int ch = 0; ch < nc; ++ch) {
          const float2 v = cs_part[((size_t)ch * nbh + bh) * n + j];
          cs += v.x;
          bs += v.y;
        }
        cum[(size_t)bh * n + j] = cs;
        band[(size_t)bh * n + j] = bs;
      }
      if (VPT > 0) {
        cv[it < NV ? it : 0] = cs;
        bv[it < NV ? it : 0] = bs;
      }
    }
    if (VPT == 0) __syncthreads();
  } else if (VPT > 0) {
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int j = it * NT + tid;
      cv[it] = j < n ? cum[(size_t)bh * n + j] : 0.f;
      bv[it] = j < n ? band[(size_t)bh * n + j] : 0.f;
    }
  }
  const float* cu = cum + (size_t)bh * n;
  const float* bd = band + (size_t)bh * n;
  const uint8_t* cl = cls + (size_t)b * n;
  uint8_t cv_cls[NV];                             // token classes of this thread's keys, loaded up front
#pragma unroll
  for (int it = 0; it < NV; ++it) {
    const int j = it * NT + tid;
    cv_cls[it] = (VPT > 0 && j < n) ? cl[j] : (uint8_t)0;
  }
  const int nw = (n + 31) / 32;
  auto score_of = [&](int it, int j) -> float { return VPT > 0 ? cv[it < NV ? it : 0] : cu[j]; };
  auto band_of = [&](int it, int j) -> float { return VPT > 0 ? bv[it < NV ? it : 0] : bd[j]; };

  // mode 0: nothing selected, 1: everything, 2: threshold + ties
  const int mode = k_f <= 0 ? 0 : (k_f >= n ? 1 : 2);
  uint32_t thr = 0;
  int take_eq = 0;
  bool all_eq = false;                            // every key equal to the threshold is taken
  if (mode == 2) {
    uint32_t prefix = 0, pmask = 0;
    int remaining = k_f;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int it = 0; it < (VPT > 0 ? VPT : 1); ++it) {
        if (VPT > 0) {
          const int j = it * NT + tid;
          const uint32_t u = __float_as_uint(score_of(it, j));
          if (j < n && (u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        } else {
          for (int j = tid; j < n; j += blockDim.x) {
            const uint32_t u = __float_as_uint(cu[j]);
            if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 255-4l .. 252-4l (descending); a prefix over lanes finds the
        // bin where the count of larger-or-equal digits reaches `remaining`
        int h[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { h[e] = (int)hist[255 - 4 * lane - e]; tot += h[e]; }
        int incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        const int excl = incl - tot;
        if (excl < remaining && remaining <= incl) {
          int acc = excl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (acc + h[e] >= remaining) {
              s_sel = (unsigned)(255 - 4 * lane - e);
              s_rem = (unsigned)(remaining - acc);
              s_cnt = (unsigned)h[e];
              break;
            }
            acc += h[e];
          }
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_sel << shift;
      pmask |= 0xFFu << shift;
      remaining = (int)s_rem;
      __syncthreads();
    }
    thr = prefix;
    take_eq = remaining;
    all_eq = (int)s_cnt == remaining;             // the last pass's bin holds exactly the keys equal to thr
  }

  double m_s = 0.0, m_p = 0.0, m_f = 0.0, m_b = 0.0;
  int run = 0;                                   // equal-to-threshold keys seen at lower indices
#pragma unroll
  for (int it = 0; it < (VPT > 0 ? VPT : 1); ++it) {
    for (int base = it * NT; base < (VPT > 0 ? min(n, (it + 1) * NT) : n); base += blockDim.x) {
      const int j = base + tid;
      const bool valid = j < n;
      const float v = valid ? score_of(it, j) : 0.f;
      const uint32_t u = __float_as_uint(v);
      bool sel = (mode == 1 || (mode == 2 && all_eq)) && valid && (mode == 1 || u >= thr);
      if (mode == 2 && !all_eq) {                 // some keys equal to thr are left out: rank them by index
        const bool eq = valid && u == thr;
        const unsigned long long bal = __ballot(eq);
        if (lane == 0) wave_cnt[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < n_waves; ++w) {
          const int cw = wave_cnt[w];
          before += (w < wave) ? cw : 0;
          total += cw;
        }
        const int rank = run + before + __popcll(bal & ((1ull << lane) - 1ull));
        sel = (valid && u > thr) || (eq && rank < take_eq);
        run += total;
        __syncthreads();
      }
      const unsigned long long sb = __ballot(sel);
      if (lane == 0) {
        const int w0 = (base + wave * 64) / 32;
        if (w0 < nw) fmask[(size_t)bh * nw + w0] = (uint32_t)(sb & 0xFFFFFFFFull);
        if (w0 + 1 < nw) fmask[(size_t)bh * nw + w0 + 1] = (uint32_t)(sb >> 32);
      }
      if (valid) {
        const uint8_t c = VPT > 0 ? cv_cls[it < NV ? it : 0] : cl[j];
        if (c == kSpecial) m_s += v;
        else if (c == kPunct) m_p += v;
        else if (sel) m_f += v;
        else m_b += band_of(it, j);
      }
    }
  }
  double ms[4] = {m_s, m_p, m_f, m_b};
  block_sum4<NT>(ms, red);
  m_s = ms[0];
  m_p = ms[1];
  m_f = ms[2];
  m_b = ms[3];
  if (tid == 0) {
    const double denom = (double)G * (double)n;
    double R[5];
    R[0] = m_s / denom;
    R[1] = (m_s + m_p) / denom;
    R[2] = (m_s + m_p + m_f) / denom;
    R[3] = (m_s + m_p + m_f + m_b) / denom;
    R[4] = 1.0;
    int pol = 4;
    for (int k = 0; k < 5; ++k)
      if (R[k] >= T) { pol = k; break; }
    for (int k = 0; k < 5; ++k) recovery[(size_t)bh * 5 + k] = (float)R[k];
    policy[bh] = (uint8_t)pol;
  }
}

template <int NT>
static void launch_select_nt(const ProfileArgs& a, hipStream_t st) {
  const int per = (a.n + NT - 1) / NT;
  auto kern = per <= 1 ? select_kernel<1, NT> : per <= 2 ? select_kernel<2, NT> : per <= 4 ? select_kernel<4, NT> :
              per <= 8 ? select_kernel<8, NT> : per <= 16 ? select_kernel<16, NT> :
              per <= 32 ? select_kernel<32, NT> : select_kernel<0, NT>;
  kern<<<dim3(a.B * a.Hkv), dim3(NT), 0, st>>>(a.cum, a.band, a.cs_part, a.rchunk, a.cls, a.Hkv, a.n, a.Hq / a.Hkv,
                                               a.k_f, a.T, a.fmask, a.recovery, a.policy);
}

hipError_t launch_select(const ProfileArgs& a, hipStream_t st) {
  timed_begin(FG_K_SELECT, st);
  // One workgroup per head.  A head's selection is a chain of barriers, so while every head's
  // workgroup is resident at once (two 1024-thread workgroups per CU) the widest workgroup is the
  // fastest; with more heads than that, narrower workgroups keep every head resident instead of
  // running the heads in rounds.
  const int heads = a.B * a.Hkv;
  if (heads <= 2 * a.cus) launch_select_nt<1024>(a, st);
  else if (heads <= 4 * a.cus) launch_select_nt<512>(a, st);
  else launch_select_nt<256>(a, st);
  timed_end(st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- multi-prompt head map
// jisaku.com glossary entry "FastGen", section Profiling phase: heads are typed
// once from a set of sample prompts and the resulting map is applied at
// inference.  Each KV head's recovery is summed over the prompts in fp64 (a
// fixed order: prompt by prompt) with a count of the per-prompt policies; the
// map's policy is the first shortlist entry whose mean recovery reaches T.
__global__ __launch_bounds__(256) void head_map_accumulate_kernel(const float* __restrict__ recovery,
                                                                  const uint8_t* __restrict__ policy,
                                                                  double* __restrict__ rec_sum,
                                                                  int32_t* __restrict__ count, int P, int H) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  double s[5];
  int c[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    s[k] = rec_sum[h * 5 + k];
    c[k] = count[h * 5 + k];
  }
  for (int p = 0; p < P; ++p) {
    const size_t hd = (size_t)p * H + h;
#pragma unroll
    for (int k = 0; k < 5; ++k) s[k] += (double)recovery[hd * 5 + k];
    const int pol = min((int)policy[hd], 4);
#pragma unroll
    for (int k = 0; k < 5; ++k) c[k] += (k == pol);
  }
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    rec_sum[h * 5 + k] = s[k];
    count[h * 5 + k] = c[k];
  }
}

__global__ __launch_bounds__(256) void head_map_finish_kernel(const double* __restrict__ rec_sum, double n_prompts,
                                                              double T, float* __restrict__ mean,
                                                              uint8_t* __restrict__ policy, int H) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  int pol = 4;
  for (int k = 4; k >= 0; --k) {
    const double m = rec_sum[h * 5 + k] / n_prompts;
    mean[h * 5 + k] = (float)m;
    if (k < 4 && m >= T) pol = k;
  }
  policy[h] = (uint8_t)pol;
}

hipError_t launch_head_map_accumulate(const float* recovery, const uint8_t* policy, double* rec_sum, int32_t* count,
                                      int P, int H, hipStream_t st) {
  head_map_accumulate_kernel<<<dim3((unsigned)((H + 255) / 256)), dim3(256), 0, st>>>(recovery, policy, rec_sum,
                                                                                      count, P, H);
  return hipGetLastError();
}

hipError_t launch_head_map_finish(const double* rec_sum, double n_prompts, double T, float* mean, uint8_t* policy,
                                  int H, hipStream_t st) {
  head_map_finish_kernel<<<dim3((unsigned)((H + 255) / 256)), dim3(256), 0, st>>>(rec_sum, n_prompts, T, mean,
                                                                                  policy, H);
  return hipGetLastError();
}

}  // namespace fg
