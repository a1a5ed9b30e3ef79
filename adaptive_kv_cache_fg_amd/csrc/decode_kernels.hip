// Decode-step attention over ragged head-specific caches, with the policy's
// eviction of the new token (hyper.ai summary of "Model Tells You What to
// Discard", Method, first paragraph: generation keeps head-specific caches;
// stability paragraph: the policy chosen on the prompt is reused).
//
// Split-K over the cache: every work item is a 64-row chunk of one head's
// rows.  A workgroup streams its chunk with 16-byte loads (one row is spread
// over D*size/16 lanes; a wave covers several rows per pass), reduces the
// G query heads' dot products with cross-lane shuffles, and keeps an online
// softmax (running max, sum, weighted V) per query head; it writes one partial
// (max, sum, acc[D]) per query head.  Items that start past a head's rows in
// use exit at once, so the static work list covers the cache's whole capacity.
//
// The combine workgroup of each head merges its partials, adds the new token
// when the policy lets it attend to itself, writes the fp32 output, and then
// updates the cache: append (special; punct when policy >= 1; every token
// under policy 4), or ring slot p mod (w_l - 1) (normal tokens under policy
// 3), freeing the slot of the key that leaves the window.
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const __bf16* p, float* out) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* out) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = v[e];
  }
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(const T* __restrict__ q, const T* __restrict__ Kc,
                                                             const T* __restrict__ Vc, const int32_t* __restrict__ pos,
                                                             const int64_t* __restrict__ row_offset,
                                                             const int32_t* __restrict__ len,
                                                             const int32_t* __restrict__ work, int Hkv, float c,
                                                             float* __restrict__ part) {
  constexpr int E = Vec16<T>::N;            // elements per lane per row
  constexpr int LPR = D / E;                // lanes per row
  constexpr int RPP = kWave / LPR;          // rows per wave pass
  constexpr int kWaves = 4;
  __shared__ float sm[kWaves][G], sl[kWaves][G];
  __shared__ float sacc[kWaves][G][D];

  const int item = blockIdx.x;
  const int hd = work[2 * item], start = work[2 * item + 1];
  const int L = len[hd];
  if (start >= L) return;                    // whole workgroup: nothing in use here
  const int end = min(start + kDecodeChunk, L);
  const int64_t base = row_offset[hd];
  const int b = hd / Hkv, h = hd % Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane / LPR, sl_ = lane % LPR;

  float qv[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g)
    Vec16<T>::load(q + ((size_t)(b * Hkv + h) * G + g) * D + sl_ * E, qv[g]);

  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  for (int r0 = start + wave * RPP; r0 < end; r0 += kWaves * RPP) {   // wave-uniform trip count
    const int row = r0 + sub;
    const bool in = row < end;
    const int64_t gr = base + (in ? row : start);
    const bool valid = in && pos[gr] >= 0;
    float kv[E], vv[E];
    Vec16<T>::load(Kc + gr * D + sl_ * E, kv);
    Vec16<T>::load(Vc + gr * D + sl_ * E, vv);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) s = fmaf(qv[g][e], kv[e], s);
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
      if (valid) {
        const float x = s * c;
        const float mn = fmaxf(m[g], x);
        const float al = fast_exp2(m[g] - mn), p = fast_exp2(x - mn);
        l[g] = fmaf(l[g], al, p);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = fmaf(acc[g][e], al, p * vv[e]);
        m[g] = mn;
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
  // merge the 4 waves: thread t handles (g, dim) pairs
  float* out = part + (size_t)item * G * (D + 2);
  for (int t = tid; t < G * D; t += blockDim.x) {
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
    out[(size_t)g * (D + 2) + 2 + dd] = as;
    if (dd == 0) { out[(size_t)g * (D + 2)] = mx; out[(size_t)g * (D + 2) + 1] = ls; }
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const uint8_t* __restrict__ new_class, float* __restrict__ out, const float* __restrict__ part,
    const int32_t* __restrict__ work, const int64_t* __restrict__ work_offset, T* __restrict__ Kc, T* __restrict__ Vc,
    int32_t* __restrict__ pos, const int64_t* __restrict__ row_offset, int32_t* __restrict__ len,
    const int32_t* __restrict__ capacity, const int32_t* __restrict__ ring, const uint8_t* __restrict__ policy,
    uint32_t* __restrict__ error_word, int Hkv, int w_l, int p, float c) {
  __shared__ float s_self[G];
  __shared__ float s_kn[D], s_vn[D];
  const int hd = blockIdx.x, b = hd / Hkv, h = hd % Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = len[hd];
  const int pol = policy[hd];
  const uint8_t cls = new_class ? new_class[b] : kNormal;
  const int lvl_self = cls == kSpecial ? 0 : (cls == kPunct ? 1 : (w_l >= 1 ? 3 : 4));
  const bool att_self = lvl_self <= pol;

  const T* kn = k_new + (size_t)hd * D;
  const T* vn = v_new + (size_t)hd * D;
  for (int t = tid; t < D; t += blockDim.x) { s_kn[t] = to_f32(kn[t]); s_vn[t] = to_f32(vn[t]); }
  __syncthreads();
  // the new token's scores: wave w handles query heads w, w + 4, ...
  for (int g = wave; g < G; g += 4) {
    const T* qg = q + ((size_t)hd * G + g) * D;
    float s = 0.f;
    for (int t = lane; t < D; t += kWave) s = fmaf(to_f32(qg[t]), s_kn[t], s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) s_self[g] = s * c;
  }
  __syncthreads();

  const int64_t w0 = work_offset[hd], w1 = work_offset[hd + 1];
  for (int t = tid; t < G * D; t += blockDim.x) {
    const int g = t / D, dd = t % D;
    float mx = att_self ? s_self[g] : kNegBig;
    for (int64_t w = w0; w < w1; ++w) {
      if (work[2 * w + 1] >= L) break;                     // items past the rows in use wrote nothing
      mx = fmaxf(mx, part[((size_t)w * G + g) * (D + 2)]);
    }
    float ls = 0.f, as = 0.f;
    for (int64_t w = w0; w < w1; ++w) {
      if (work[2 * w + 1] >= L) break;
      const float* pp = part + ((size_t)w * G + g) * (D + 2);
      const float a = fast_exp2(pp[0] - mx);
      ls = fmaf(pp[1], a, ls);
      as = fmaf(pp[2 + dd], a, as);
    }
    if (att_self) {
      const float a = fast_exp2(s_self[g] - mx);
      ls += a;
      as = fmaf(a, s_vn[dd], as);
    }
    out[((size_t)hd * G + g) * D + dd] = ls > 0.f ? as / ls : 0.f;
  }

  // cache update: after this step the cache holds {j <= p : level(p + 1, j) <= policy}
  const int R = ring[hd];
  const int64_t base = row_offset[hd];
  const bool to_ring = (cls == kNormal) && pol == 3 && w_l >= 2 && R > 0;
  const bool to_perm = cls == kSpecial || (cls == kPunct && pol >= 1) || (cls == kNormal && pol == 4);
  const int slot = R > 0 ? p % R : 0;
  int64_t dst = -1;
  if (to_ring) {
    dst = base + slot;
  } else if (to_perm) {
    if (L < capacity[hd]) dst = base + L;
  }
  __syncthreads();   // every thread has read len / partials before it changes
  if (dst >= 0) {
    for (int t = tid; t < D; t += blockDim.x) {
      Kc[dst * D + t] = kn[t];
      Vc[dst * D + t] = vn[t];
    }
  }
  if (tid == 0) {
    if (pol == 3 && R > 0 && !to_ring) pos[base + slot] = -1;   // key p + 1 - w_l leaves the window
    if (dst >= 0) pos[dst] = p;
    if (to_perm) {
      if (dst >= 0) len[hd] = L + 1;
      else atomicOr(error_word, 1u);
    }
  }
}

template <typename T, int D, int G>
static hipError_t launch_decode_tg(const DecodeArgs& a, hipStream_t st) {
  const float c = kLog2e / sqrtf((float)D);
  const int H = a.B * a.Hkv;
  timed_begin(FG_K_DECODE_PARTIAL, st);
  if (a.n_work > 0)
    decode_partial_kernel<T, D, G><<<dim3((unsigned)a.n_work), dim3(256), 0, st>>>(
        (const T*)a.q, (const T*)a.Kc, (const T*)a.Vc, a.pos, a.row_offset, a.len, a.work, a.Hkv, c, a.part);
  timed_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timed_begin(FG_K_DECODE_COMBINE, st);
  decode_combine_kernel<T, D, G><<<dim3(H), dim3(256), 0, st>>>(
      (const T*)a.q, (const T*)a.k_new, (const T*)a.v_new, a.new_class, a.out, a.part, a.work, a.work_offset,
      (T*)a.Kc, (T*)a.Vc, a.pos, a.row_offset, a.len, a.capacity, a.ring, a.policy, a.error_word, a.Hkv, a.w_l, a.p,
      c);
  timed_end(st);
  return hipGetLastError();
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
