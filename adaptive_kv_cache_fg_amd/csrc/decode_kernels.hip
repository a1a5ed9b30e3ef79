// Decode-step attention over ragged head-specific caches, with the policy's
// eviction of the new token (hyper.ai summary of "Model Tells You What to
// Discard", Method, first paragraph: generation keeps head-specific caches;
// stability paragraph: the policy chosen on the prompt is reused).
//
// One launch per step, split-K over the cache: every work item is a 128-row
// chunk of one head.  A workgroup issues each 64-row half's 16-byte K/V loads
// up front (one row is spread over D*size/16 lanes; a wave covers several rows
// per pass), reduces the G query heads' dot products with cross-lane shuffles
// and keeps an online softmax (running max, sum, weighted V) per query head.
// It stores one partial (max, sum, acc[D]) per query head and signals a
// per-head arrival counter; the last workgroup of the head to arrive merges
// the partials, adds the new token when the policy lets it attend to itself,
// writes the fp32 output and updates the cache: append (special; punct when
// policy >= 1; every token under policy 4) or ring slot p mod (w_l - 1)
// (normal tokens under policy 3), freeing the slot of the key that leaves the
// window.  Items past a head's rows in use only signal, so the static work
// list covers the cache's whole capacity.
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
  static constexpr int N = 8;
  using raw_t = bf16x8;
  static __device__ __forceinline__ void cvt(const raw_t& v, float* out) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  using raw_t = f32x4;
  static __device__ __forceinline__ void cvt(const raw_t& v, float* out) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = v[e];
  }
};

// Merge of one head's partial states, the new token, the output and the cache
// update (run by the last-arriving workgroup, or by the combine kernel).
template <typename T, int D, int G, int NT>
__device__ __forceinline__ void decode_tail(
    int hd, int L, const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const uint8_t* __restrict__ new_class, float* __restrict__ out, const float* __restrict__ part,
    const int64_t* __restrict__ work_offset, T* __restrict__ Kc, T* __restrict__ Vc, int32_t* __restrict__ pos,
    const int64_t* __restrict__ row_offset, int32_t* __restrict__ len, const int32_t* __restrict__ capacity,
    const int32_t* __restrict__ ring, const uint8_t* __restrict__ policy, int32_t* __restrict__ arrive,
    uint32_t* __restrict__ error_word, int Hkv, int w_l, int p, float c) {
  constexpr int kWaves = 4;
  constexpr int GD = G * D;
  constexpr int NGRP = GD >= NT ? 1 : NT / GD;     // item groups in the merge
  __shared__ float cm[NGRP][GD], cs[NGRP][GD], ca[NGRP][GD];
  __shared__ float s_self[G];
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int b = hd / Hkv;
  const int pol = policy[hd];
  const uint8_t cls = new_class ? new_class[b] : kNormal;
  const int lvl_self = cls == kSpecial ? 0 : (cls == kPunct ? 1 : (w_l >= 1 ? 3 : 4));
  const bool att_self = lvl_self <= pol;
  const T* kn = k_new + (size_t)hd * D;
  const T* vn = v_new + (size_t)hd * D;
  for (int g = wave; g < G; g += NT / kWave) {          // the new token's scores
    const T* qg = q + ((size_t)hd * G + g) * D;
    float s = 0.f;
    for (int t = lane; t < D; t += kWave) s = fmaf(to_f32(qg[t]), to_f32(kn[t]), s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) s_self[g] = s * c;
  }
  const int64_t w0 = work_offset[hd];
  const int n_items = (int)(work_offset[hd + 1] - w0);
  __syncthreads();                                      // s_self visible
  // one round of independent loads: thread (output o, item group grp) merges its
  // items' partial states online; the groups are merged in LDS below
  {
    const int grp = tid / GD;
    if (grp < NGRP) {
      for (int o = tid % GD; o < GD; o += NT) {
        const int g = o / D, dd = o % D;
        float M = kNegBig, Ls = 0.f, As = 0.f;
#pragma unroll 4
        for (int w = grp; w < n_items; w += NGRP) {
          const float* pp = part + ((size_t)(w0 + w) * G + g) * (D + 2);
          const float mw = pp[0], lw = pp[1], aw = pp[2 + dd];
          const bool live = lw > 0.f;                  // an empty item stored only (max, sum)
          const float mn = live ? fmaxf(M, mw) : M;
          const float s1 = fast_exp2(M - mn);
          const float s2 = live ? fast_exp2(mw - mn) : 0.f;
          Ls = fmaf(Ls, s1, live ? lw * s2 : 0.f);
          As = fmaf(As, s1, live ? aw * s2 : 0.f);
          M = mn;
        }
        cm[grp][o] = M;
        cs[grp][o] = Ls;
        ca[grp][o] = As;
      }
    }
  }
  __syncthreads();
  for (int o = tid; o < GD; o += blockDim.x) {
    const int g = o / D, dd = o % D;
    float M = att_self ? s_self[g] : kNegBig;
#pragma unroll
    for (int r = 0; r < NGRP; ++r) M = fmaxf(M, cm[r][o]);
    float Ls = 0.f, As = 0.f;
#pragma unroll
    for (int r = 0; r < NGRP; ++r) {
      const float a = fast_exp2(cm[r][o] - M);
      Ls = fmaf(cs[r][o], a, Ls);
      As = fmaf(ca[r][o], a, As);
    }
    if (att_self) {
      const float a = fast_exp2(s_self[g] - M);
      Ls += a;
      As = fmaf(a, to_f32(vn[dd]), As);
    }
    out[((size_t)hd * G + g) * D + dd] = Ls > 0.f ? As / Ls : 0.f;
  }

  // cache update: afterwards the cache holds {j <= p : level(p + 1, j) <= policy}
  const int R = ring[hd];
  const int64_t base_h = row_offset[hd];
  const bool to_ring = (cls == kNormal) && pol == 3 && w_l >= 2 && R > 0;
  const bool to_perm = cls == kSpecial || (cls == kPunct && pol >= 1) || (cls == kNormal && pol == 4);
  const int slot = R > 0 ? p % R : 0;
  int64_t dst = -1;
  if (to_ring) dst = base_h + slot;
  else if (to_perm && L < capacity[hd]) dst = base_h + L;
  if (dst >= 0) {
    for (int t = tid; t < D; t += blockDim.x) {
      Kc[dst * D + t] = kn[t];
      Vc[dst * D + t] = vn[t];
    }
  }
  if (tid == 0) {
    if (pol == 3 && R > 0 && !to_ring) pos[base_h + slot] = -1;   // key p + 1 - w_l leaves the window
    if (dst >= 0) pos[dst] = p;
    if (to_perm) {
      if (dst >= 0) len[hd] = L + 1;
      else atomicOr(error_word, 1u);
    }
    arrive[hd] = 0;
  }
}

template <typename T, int D, int G, bool FUSED>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const uint8_t* __restrict__ new_class, float* __restrict__ out, float* __restrict__ part,
    const int32_t* __restrict__ work, const int64_t* __restrict__ work_offset, T* __restrict__ Kc,
    T* __restrict__ Vc, int32_t* __restrict__ pos, const int64_t* __restrict__ row_offset, int32_t* __restrict__ len,
    const int32_t* __restrict__ capacity, const int32_t* __restrict__ ring, const uint8_t* __restrict__ policy,
    int32_t* __restrict__ arrive, uint32_t* __restrict__ error_word, int Hkv, int w_l, int p, float c) {
  using V16 = Vec16<T>;
  using raw_t = typename V16::raw_t;
  constexpr int E = V16::N;                 // elements per lane per row
  constexpr int LPR = D / E;                // lanes per row
  constexpr int RPP = kWave / LPR;          // rows per wave pass
  constexpr int kWaves = 4;
  constexpr int kSubRows = kDecodeChunk;    // rows whose loads are issued together
  constexpr int RPW = kSubRows / kWaves;    // rows per wave per pass
  constexpr int NP = RPW / RPP;             // passes per wave
  constexpr int GD = G * D;
  __shared__ float sm[kWaves][G], sl[kWaves][G];
  __shared__ float sacc[kWaves][G][D];
  __shared__ int s_last;

  const int item = blockIdx.x;
  const int hd = work[2 * item], start = work[2 * item + 1];
  const int L = len[hd];
  const int end = min(start + kDecodeChunk, L);
  const int64_t base = row_offset[hd];
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int sub = lane / LPR, sl_ = lane % LPR;
  float* mypart = part + (size_t)item * G * (D + 2);

  if (start < L) {
    // ---- partial softmax state of this chunk
    float qv[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) V16::cvt(*reinterpret_cast<const raw_t*>(q + ((size_t)hd * G + g) * D + sl_ * E), qv[g]);
    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = kNegBig;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
    }
    for (int r0 = start; r0 < end; r0 += kSubRows) {    // wave-uniform
    raw_t kr[NP], vr[NP];
    bool valid[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {                     // every load of the sub-batch in flight at once
      const int row = r0 + wave * RPW + i * RPP + sub;
      const bool in = row < end;
      const int64_t gr = base + (in ? row : start);
      kr[i] = *reinterpret_cast<const raw_t*>(Kc + gr * D + sl_ * E);
      vr[i] = *reinterpret_cast<const raw_t*>(Vc + gr * D + sl_ * E);
      valid[i] = in && pos[gr] >= 0;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float kv[E], vv[E];
      V16::cvt(kr[i], kv);
      V16::cvt(vr[i], vv);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(qv[g][e], kv[e], s);
        s = group_sum<LPR>(s);
        if (valid[i]) {
          const float x = s * c;
          const float mn = fmaxf(m[g], x);
          const float al = fast_exp2(m[g] - mn), pw = fast_exp2(x - mn);
          l[g] = fmaf(l[g], al, pw);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = fmaf(acc[g][e], al, pw * vv[e]);
          m[g] = mn;
        }
      }
    }
    }
    // merge the RPP row groups of the wave (lanes with equal sl_)
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mo = __shfl_xor(m[g], o), lo = __shfl_xor(l[g], o);
        const float mn = fmaxf(m[g], mo);
        const float a1 = fast_exp2(m[g] - mn), a2 = fast_exp2(mo - mn);
        l[g] = l[g] * a1 + lo * a2;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float ao = __shfl_xor(acc[g][e], o);
          acc[g][e] = acc[g][e] * a1 + ao * a2;
        }
        m[g] = mn;
      }
    }
    if (sub == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (sl_ == 0) { sm[wave][g] = m[g]; sl[wave][g] = l[g]; }
#pragma unroll
        for (int e = 0; e < E; ++e) sacc[wave][g][sl_ * E + e] = acc[g][e];
      }
    }
    __syncthreads();
    for (int t = tid; t < GD; t += blockDim.x) {        // merge the 4 waves
      const int g = t / D, dd = t % D;
      float mx = sm[0][g];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm[w][g]);
      float ls = 0.f, as = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float a = fast_exp2(sm[w][g] - mx);
        ls += sl[w][g] * a;
        as += sacc[w][g][dd] * a;
      }
      mypart[(size_t)g * (D + 2) + 2 + dd] = as;
      if (dd == 0) { mypart[(size_t)g * (D + 2)] = mx; mypart[(size_t)g * (D + 2) + 1] = ls; }
    }
  } else if (tid < G) {                                  // nothing in use here: an empty state
    mypart[(size_t)tid * (D + 2)] = kNegBig;
    mypart[(size_t)tid * (D + 2) + 1] = 0.f;
  }

  if (!FUSED) return;                                    // the combine kernel merges the partials
  // ---- arrival: the last workgroup of the head merges and updates the cache.
  // Every wave waits for its partial stores to complete, the barrier orders
  // them before thread 0's device-scope release (L2 write-back), and the last
  // arriver acquires (L1/L2 invalidate) before anyone reads the partials.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int n_items = (int)(work_offset[hd + 1] - work_offset[hd]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int prev = __hip_atomic_fetch_add(&arrive[hd], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == n_items - 1;
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_last) return;

  decode_tail<T, D, G, 256>(hd, L, q, k_new, v_new, new_class, out, part, work_offset, Kc, Vc, pos, row_offset, len,
                       capacity, ring, policy, arrive, error_word, Hkv, w_l, p, c);
}

// Combine launch of the two-kernel decode step: one workgroup per head, wide
// enough that each thread merges only a few partial states.
constexpr int kCombineThreads = 1024;

template <typename T, int D, int G>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const uint8_t* __restrict__ new_class, float* __restrict__ out, const float* __restrict__ part,
    const int64_t* __restrict__ work_offset, T* __restrict__ Kc, T* __restrict__ Vc, int32_t* __restrict__ pos,
    const int64_t* __restrict__ row_offset, int32_t* __restrict__ len, const int32_t* __restrict__ capacity,
    const int32_t* __restrict__ ring, const uint8_t* __restrict__ policy, int32_t* __restrict__ arrive,
    uint32_t* __restrict__ error_word, int Hkv, int w_l, int p, float c) {
  const int hd = blockIdx.x;
  decode_tail<T, D, G, kCombineThreads>(hd, len[hd], q, k_new, v_new, new_class, out, part, work_offset, Kc, Vc, pos, row_offset,
                       len, capacity, ring, policy, arrive, error_word, Hkv, w_l, p, c);
}

#ifndef FG_DECODE_FUSED
#define FG_DECODE_FUSED 0
#endif

template <typename T, int D, int G>
static hipError_t launch_decode_tg(const DecodeArgs& a, hipStream_t st) {
  const float c = kLog2e / sqrtf((float)D);
  const int H = a.B * a.Hkv;
  timed_begin(FG_K_DECODE, st);
  decode_step_kernel<T, D, G, FG_DECODE_FUSED != 0><<<dim3((unsigned)a.n_work), dim3(256), 0, st>>>(
      (const T*)a.q, (const T*)a.k_new, (const T*)a.v_new, a.new_class, a.out, a.part, a.work, a.work_offset,
      (T*)a.Kc, (T*)a.Vc, a.pos, a.row_offset, a.len, a.capacity, a.ring, a.policy, a.arrive, a.error_word, a.Hkv,
      a.w_l, a.p, c);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && !FG_DECODE_FUSED) {
    decode_combine_kernel<T, D, G><<<dim3(H), dim3(kCombineThreads), 0, st>>>(
        (const T*)a.q, (const T*)a.k_new, (const T*)a.v_new, a.new_class, a.out, a.part, a.work_offset,
        (T*)a.Kc, (T*)a.Vc, a.pos, a.row_offset, a.len, a.capacity, a.ring, a.policy, a.arrive, a.error_word,
        a.Hkv, a.w_l, a.p, c);
    e = hipGetLastError();
  }
  timed_end(st);
  return e;
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_decode_tg<T, D, 1>(a, st);
    case 2: return launch_decode_tg<T, D, 2>(a, st);
    case 4: return launch_decode_tg<T, D, 4>(a, st);
    case 8: return launch_decode_tg<T, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == FG_DTYPE_BF16)
    return a.D == 128 ? launch_decode_t<__bf16, 128>(a, st) : launch_decode_t<__bf16, 64>(a, st);
  return a.D == 128 ? launch_decode_t<float, 128>(a, st) : launch_decode_t<float, 64>(a, st);
}

}  // namespace fg
