// Decode-step attention over ragged head-specific caches, with the policy's
// eviction of the new token (hyper.ai summary of "Model Tells You What to
// Discard", Method, first paragraph: generation keeps head-specific caches;
// stability paragraph: the policy chosen on the prompt is reused).
//
// Two launches per step, split-K over the cache.  Every work item is a
// 128-row chunk of one head and carries (head, first row, first absolute row,
// rows in use), so a workgroup's only dependent load before its K/V loads is
// that 16-byte item.  It issues all of its chunk's 16-byte K/V loads at once
// (one row is spread over D*size/16 lanes; a wave covers several rows per
// pass), reduces the G query heads' dot products with DPP lane sums, keeps an
// online softmax (running max, sum, weighted V) per query head, and stores one
// partial state (max, sum, acc[D]) per query head into its slot; slots sit at
// a fixed stride per head, so the merge's loads of them need no index lookup.
// The merge launch (one workgroup per head) issues the per-head scalars, the
// new token's q . k_new and all slot loads of a batch together, combines the
// partials, adds the new token when the policy lets it attend to itself,
// writes the fp32 output and updates the cache: append (special; punct when
// policy >= 1; every token under policy 4) or ring slot p mod (w_l - 1)
// (normal tokens under policy 3), freeing the slot of the key that leaves the
// window; an append also bumps the rows-in-use count of the work item that
// holds the new row.
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

// Merge launch: one workgroup per query head merges its KV head's partial
// states for that query head, adds the new token, writes the output; the
// workgroup of the group's first query head also updates the KV head's cache,
// before its merge (the update reads none of the merge's inputs, so its stores
// are under way while the merge computes).
// Every load is issued before its first use: the per-head scalars, the new
// token's q . k_new and K/V row, and the partial slots in batches of kBatch
// items per thread (masked by the head's item count afterwards, so they do not
// wait for it).  NT threads: 256 when at most two batches cover a head's items
// (a smaller workgroup starts and drains sooner: 256 measured about 1 us per step
// faster than 512 at the Llama-1-65B shape), else 1024.
constexpr int kMergeBatch = 8;                     // items per thread whose loads are in flight together

// HAS_CLASS = false: new_class is NULL and every generated token is normal.
template <typename T, int D, int G, bool HAS_CLASS, int NT>
__global__ __launch_bounds__(NT) void decode_merge_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    const uint8_t* __restrict__ new_class, float* __restrict__ out, const float* __restrict__ part,
    const int64_t* __restrict__ work_offset, int32_t* __restrict__ work, T* __restrict__ Kc, T* __restrict__ Vc,
    int32_t* __restrict__ pos, const int64_t* __restrict__ row_offset, int32_t* __restrict__ len,
    const int32_t* __restrict__ capacity, const int32_t* __restrict__ ring, const uint8_t* __restrict__ policy,
    uint32_t* __restrict__ error_word, float* __restrict__ score, const uint8_t* __restrict__ cls_all, int n_total,
    int Hkv, int w_l, int p, int S, int CH, int64_t total_rows, int64_t n_work, float c) {
  static_assert(NT % D == 0, "one output per thread");
  constexpr int NGRP = NT / D;                     // thread groups splitting the item list
  constexpr int kBatch = kMergeBatch;
  constexpr int kWavesPerHead = D / kWave;         // waves reducing the query head's q . k_new
  __shared__ float cm[NGRP][D], cs[NGRP][D], ca[NGRP][D];
  __shared__ float s_wave[NT / kWave];
  __shared__ unsigned long long s_key[NT / kWave];
  __shared__ int s_row[NT / kWave];
  const int qh = blockIdx.x, hd = qh / G, g = qh % G;   // query head, its KV head, its index in the group
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int dd = tid % D, grp = tid / D;           // this thread's output dimension and item group
  const float* hpart = part + (size_t)hd * S * G * (D + 2) + (size_t)g * (D + 2);   // slot k at k * G * (D + 2)

  // ---- every load up front, unconditional (straight-line code, so none waits on another)
  const int64_t w0 = work_offset[hd], w1 = work_offset[hd + 1];
  const int pol = policy[hd];
  const uint8_t cls = HAS_CLASS ? new_class[hd / Hkv] : kNormal;
  const int R = ring[hd];
  const int64_t base_h = row_offset[hd];
  // the head's rows, its work items and its partial slots all lie inside the cache's buffers (the
  // compaction's own test): else the plan did not fit (error bit 2), the head's items are empty,
  // none of its slots is merged and its cache gets no update
  const bool fits = row_offset[hd + 1] <= total_rows && w1 <= n_work && w1 - w0 <= S;
  const int n_items = fits ? (int)(w1 - w0) : 0;
  const int cap = capacity[hd];
  const int L = len[hd];                           // rows in use before this step (see the deferred store)
  const float qv = to_f32(q[(size_t)qh * D + dd]);
  const float kv_self = to_f32(k_new[(size_t)hd * D + dd]);   // thread dd holds k_new[dd], v_new[dd]
  const float vv_self = to_f32(v_new[(size_t)hd * D + dd]);
  float mv[kBatch], lv[kBatch], av[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const float* pp = hpart + (size_t)min(grp + k * NGRP, S - 1) * G * (D + 2);
    mv[k] = pp[0];
    lv[k] = pp[1];
    av[k] = pp[2 + dd];
  }

  // The new row count and the work item's rows-in-use count are stored only after the merge's barrier
  // below: every thread reads len[hd] above and uses it (dst) before that barrier, so no thread can
  // see the incremented count (a store in the update itself could reach a late wave's load).
  bool bump = false, overflow = false;
  if (g == 0 && fits) {                           // one cache update per KV head, before the merge
    // ---- cache update: afterwards the cache holds {j <= p : level(p + 1, j) <= policy}
    const bool to_ring = (cls == kNormal) && pol == 3 && w_l >= 2 && R > 0;
    const bool to_perm = cls == kSpecial || (cls == kPunct && pol >= 1) || (cls == kNormal && pol == 4);
    const int slot = R > 0 ? p % R : 0;

    // ---- frequent set re-ranked during generation (score != nullptr): the key the window drops
    // (the ring slot's occupant, position p + 1 - w_l) replaces the cached frequent key of the
    // lowest score (ties: the larger position) when its own score is larger.  Frequent keys are the
    // permanent rows of class normal.  The branch is uniform across the workgroup.
    if (score != nullptr && pol == 3 && R > 0) {
      const int64_t srow = base_h + slot;
      const int j_out = pos[srow];
      if (j_out >= 0) {
        const size_t cb = (size_t)(hd / Hkv) * n_total;
        unsigned long long best = ~0ull;                 // (score bits, 0x7fffffff - position): smallest wins
        int best_row = -1;
        for (int r = R + tid; r < L; r += NT) {
          const int jp = pos[base_h + r];
          if (jp < 0 || jp >= n_total || cls_all[cb + jp] != kNormal) continue;
          const unsigned long long key = ((unsigned long long)__float_as_uint(score[base_h + r]) << 32) |
                                         (unsigned)(0x7fffffff - jp);   // scores are >= 0: bits order like values
          if (key < best) {
            best = key;
            best_row = r;
          }
        }
        for (int o = 1; o < kWave; o <<= 1) {
          const unsigned long long ok = __shfl_xor(best, o);
          const int orow = __shfl_xor(best_row, o);
          if (ok < best) {
            best = ok;
            best_row = orow;
          }
        }
        if (lane == 0) {
          s_key[wave] = best;
          s_row[wave] = best_row;
        }
        __syncthreads();
        best = s_key[0];
        best_row = s_row[0];
        for (int w = 1; w < NT / kWave; ++w)
          if (s_key[w] < best) {
            best = s_key[w];
            best_row = s_row[w];
          }
        const float s_out = score[srow];
        if (best != ~0ull && s_out > __uint_as_float((unsigned)(best >> 32))) {
          const int64_t drow = base_h + best_row;
          if (tid < D) {                                 // the same threads write the new token's row below
            Kc[drow * D + tid] = Kc[srow * D + tid];
            Vc[drow * D + tid] = Vc[srow * D + tid];
          }
          if (tid == 0) {
            pos[drow] = j_out;
            score[drow] = s_out;
          }
        }
      }
    }
    int64_t dst = -1;
    if (to_ring) dst = base_h + slot;
    else if (to_perm && L < cap) dst = base_h + L;
    if (dst >= 0 && tid < D) {                       // threads 0..D-1 hold element tid of the new row
      Kc[dst * D + tid] = T(kv_self);
      Vc[dst * D + tid] = T(vv_self);
    }
    if (tid == 0) {
      if (pol == 3 && R > 0 && !to_ring) pos[base_h + slot] = -1;   // key p + 1 - w_l leaves the window
      if (dst >= 0) pos[dst] = p;
      bump = to_perm && dst >= 0;
      overflow = to_perm && dst < 0;
    }
  }
  // ---- the new token's score: lane sums, then the D / 64 waves of one item group in LDS
  // (every wave reduces; only group 0's entries are read)
  const float sw = group_sum<kWave>(qv * kv_self);
  if (lane == 0) s_wave[wave] = sw;
  // ---- thread (dd, grp) merges items grp, grp + NGRP, ... online
  float M = kNegBig, Ls = 0.f, As = 0.f;
  for (int wb = grp;;) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      // slots past the head's items hold stale data; an empty item stored only (max, sum)
      const bool live = wb + k * NGRP < n_items && lv[k] > 0.f;
      const float mn = live ? fmaxf(M, mv[k]) : M;
      const float s1 = fast_exp2(M - mn);
      const float s2 = live ? fast_exp2(mv[k] - mn) : 0.f;
      Ls = fmaf(Ls, s1, live ? lv[k] * s2 : 0.f);
      As = fmaf(As, s1, live ? av[k] * s2 : 0.f);
      M = mn;
    }
    wb += NGRP * kBatch;
    if (wb >= n_items) break;                       // long lists: the next batch
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float* pp = hpart + (size_t)min(wb + k * NGRP, S - 1) * G * (D + 2);
      mv[k] = pp[0];
      lv[k] = pp[1];
      av[k] = pp[2 + dd];
    }
  }
  cm[grp][dd] = M;
  cs[grp][dd] = Ls;
  ca[grp][dd] = As;
  const int lvl_self = cls == kSpecial ? 0 : (cls == kPunct ? 1 : (w_l >= 1 ? 3 : 4));
  const bool att_self = lvl_self <= pol;
  __syncthreads();
  if (bump) {                                      // thread 0 of the updating workgroup (see above)
    len[hd] = L + 1;
    const int64_t wi = w0 + L / CH;                // the item that holds row L
    work[4 * wi + 3] = L % CH + 1;
  }
  if (overflow) atomicOr(error_word, 1u);
  if (grp == 0) {
    float s_self = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerHead; ++w) s_self += s_wave[w];
    s_self *= c;
    float Mx = att_self ? s_self : kNegBig;
#pragma unroll
    for (int r = 0; r < NGRP; ++r) Mx = fmaxf(Mx, cm[r][dd]);
    float Lt = 0.f, At = 0.f;
#pragma unroll
    for (int r = 0; r < NGRP; ++r) {
      const float a = fast_exp2(cm[r][dd] - Mx);
      Lt = fmaf(cs[r][dd], a, Lt);
      At = fmaf(ca[r][dd], a, At);
    }
    if (att_self) {
      const float a = fast_exp2(s_self - Mx);
      Lt += a;
      At = fmaf(a, vv_self, At);
    }
    out[(size_t)qh * D + dd] = Lt > 0.f ? At / Lt : 0.f;
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_partials_kernel(
    const T* __restrict__ q, float* __restrict__ part, const int32_t* __restrict__ work,
    const T* __restrict__ Kc, const T* __restrict__ Vc, const int32_t* __restrict__ pos, int S, int CH,
    float c) {
  using V16 = Vec16<T>;
  using raw_t = typename V16::raw_t;
  constexpr int E = V16::N;                 // elements per lane per row
  constexpr int LPR = D / E;                // lanes per row
  constexpr int RPP = kWave / LPR;          // rows per wave pass
  constexpr int kWaves = 4;
  constexpr int RPW = kDecodeSubRows / kWaves;   // rows per wave per sub-batch
  constexpr int NP = RPW / RPP;             // passes per wave per sub-batch
  constexpr int GD = G * D;
  static_assert(RPW % RPP == 0, "sub-batch must split evenly over the waves");
  __shared__ float sm[kWaves][G], sl[kWaves][G];
  __shared__ float sacc[kWaves][G][D];

  const int item = blockIdx.x;
  const int4 wk = reinterpret_cast<const int4*>(work)[item];   // (head, first row, first absolute row, rows in use)
  const int hd = max(wk.x, 0), k_item = wk.y / CH, abs0 = wk.z, n_use = wk.w;   // head -1: an empty item
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int sub = lane / LPR, sl_ = lane % LPR;
  float* mypart = part + ((size_t)hd * S + min(k_item, S - 1)) * G * (D + 2);

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
  // Sub-batches of kDecodeSubRows rows, all loads of one in flight at once.  The
  // first has no branch between the item and its loads (a branch on loaded data
  // would wait for it): lanes past the item's rows in use read q's first row
  // and the item itself instead of a cache row (both always exist) and are
  // masked, so an item with no rows in use stores the empty state (max -big,
  // sum 0).
  for (int r0 = 0;;) {
    raw_t kr[NP], vr[NP];
    int pr[NP];
    bool in[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int row = r0 + wave * RPW + i * RPP + sub;
      in[i] = row < n_use;
      const int64_t gr = (int64_t)abs0 + row;
      // non-temporal: each cache row is read once per step (a read-only stream measured about 8 %
      // faster with non-temporal loads, and the whole step about 9 % at the Llama-1-65B shape)
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const raw_t*>((in[i] ? Kc + gr * D : q) + sl_ * E));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const raw_t*>((in[i] ? Vc + gr * D : q) + sl_ * E));
      pr[i] = in[i] ? pos[gr] : work[0];
    }
    // scores of the sub-batch's rows first, then one rescale of the running
    // state per query head and a plain weighted sum over the rows
    float x[NP][G];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float kv[E];
      V16::cvt(kr[i], kv);
      const bool valid = in[i] && pr[i] >= 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(qv[g][e], kv[e], s);
        s = group_sum<LPR>(s);
        x[i][g] = valid ? s * c : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int i = 0; i < NP; ++i) mx = fmaxf(mx, x[i][g]);
      const float al = fast_exp2(m[g] - mx);
      l[g] *= al;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] *= al;
      m[g] = mx;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float vv[E];
      V16::cvt(vr[i], vv);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = fast_exp2(x[i][g] - m[g]);   // 0 for masked rows
        l[g] += pw;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pw, vv[e], acc[g][e]);
      }
    }
    r0 += kDecodeSubRows;
    if (r0 >= n_use) break;
  }
  {
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
    if (wk.x < 0) return;                              // an empty item (past the plan's total): no slot
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
      if (dd == 0) {
        mypart[(size_t)g * (D + 2)] = mx;
        mypart[(size_t)g * (D + 2) + 1] = ls;
      }
    }
  }

}

template <typename T, int D, int G>
static hipError_t launch_decode_tg(const DecodeArgs& a, hipStream_t st) {
  const float c = kLog2e / sqrtf((float)D);
  const int H = a.B * a.Hkv;
  timed_begin(FG_K_DECODE, st);
  decode_partials_kernel<T, D, G><<<dim3((unsigned)a.n_work), dim3(256), 0, st>>>(
      (const T*)a.q, a.part, a.work, (const T*)a.Kc, (const T*)a.Vc, a.pos, a.items_per_head, a.chunk_rows, c);
  timed_end(st);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && !a.partials_only) {
    timed_begin(FG_K_DECODE_MERGE, st);
    const bool small = a.items_per_head <= 2 * (256 / D) * kMergeBatch;
    auto kern = a.new_class ? (small ? decode_merge_kernel<T, D, G, true, 256> : decode_merge_kernel<T, D, G, true, 1024>)
                            : (small ? decode_merge_kernel<T, D, G, false, 256> : decode_merge_kernel<T, D, G, false, 1024>);
    kern<<<dim3(H * G), dim3(small ? 256 : 1024), 0, st>>>(
        (const T*)a.q, (const T*)a.k_new, (const T*)a.v_new, a.new_class, a.out, a.part, a.work_offset, a.work,
        (T*)a.Kc, (T*)a.Vc, a.pos, a.row_offset, a.len, a.capacity, a.ring, a.policy, a.error_word, a.score,
        a.cls_all, a.n_total, a.Hkv, a.w_l, a.p, a.items_per_head, a.chunk_rows, a.total_rows, a.n_work, c);
    timed_end(st);
    e = hipGetLastError();
  }
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
