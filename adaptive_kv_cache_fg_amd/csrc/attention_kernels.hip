// Causal attention output of the prompt on gfx950: O = softmax(Q K^T / sqrt(d)) V
// per query head, with each row's log-sum-exp as a side output.
//
// FastGen profiles every head while the prompt is encoded (hyper.ai summary of
// "Model Tells You What to Discard", Method, first paragraph): the model runs
// this attention anyway, and its row statistics are exactly what the profiling
// sweep over columns needs.  Computing O here and handing lse to the column
// sweep makes the row-statistics sweep of the profiling disappear; what
// profiling then adds is the column sweep and the policy selection.
//
// One workgroup = 4 waves; a wave owns 32 * QB query rows (QB blocks of 32)
// and walks the keys of its causal prefix in tiles of KT keys.  K and V tiles
// are staged into double-buffered LDS with direct global-to-LDS loads.  Per
// 32-key unit and query block:
//   S^T  = K Q^T          (K rows from LDS as the A operand, the wave's Q rows
//                          as the register-resident B operand; a lane owns one
//                          query column, so the softmax row reductions stay in
//                          the lane pair l, l ^ 32)
//   P^T  = 2^(S^T c - m)  (online max m per query, rescaled lazily: only when
//                          the running max grows by more than kRescaleLog2)
//   O^T += V^T P^T        (P^T straight from the S^T accumulators converted to
//                          bf16 -- the MFMA k index is permuted so that a lane's
//                          own accumulator registers form its B operand -- and
//                          V^T read from the row-major V tile with the
//                          transposing LDS read ds_read_b64_tr_b16).
// O^T keeps a lane's query in its column too, so the rescale of O by
// exp2(m_old - m_new) is a per-lane scalar multiply.
#include <algorithm>

#include "fg_common.h"
#include "fg_internal.h"
#include "fg_tiles.h"

namespace fg {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kAttnVPadSlots = 4;       // V rows padded by 64 bytes: the 4 rows of a transposed read hit disjoint banks
constexpr float kRescaleLog2 = 8.0f;    // running max kept until a row's max grows by more than 2^8

// A operand of O^T += V^T P^T for the 16 keys k0 .. k0 + 15 of a unit and output
// dims d0 .. d0 + 31.  MFMA k index 8 h + e (h = lane / 32) stands for key
// k0 + 8 (e / 4) + 4 h + e % 4, the key the S^T accumulator register 8 t + e of
// the same lane holds (t = k-step).  ds_read_b64_tr_b16 gives lane i of a
// 16-lane group element e = M[4 e + i / 4][i % 4], M[L] being the four 16-bit
// values at the address lane L passed; lane L therefore passes row
// k0 + 4 h + L / 4, columns d + 4 (L % 4) .. + 3, which returns
// V[k0 + 4 h + e][d0 + lane % 32] in element e (and k0 + 8 + ... for the second read).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const unsigned char* vt, int k0, int d0, int lane) {
  constexpr int kRB = D * 2 + 16 * kAttnVPadSlots;
  const int g = lane >> 4, L = lane & 15;
  const int key = k0 + 4 * (g >> 1) + (L >> 2);
  const int d = d0 + 16 * (g & 1) + 4 * (L & 3);
  const unsigned char* p = vt + key * kRB + d * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 8 * kRB));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// KS key groups of 4 waves per workgroup: with KS = 2 the two groups take the
// first and the second half of the row block's key tiles (same query rows,
// their own LDS tiles) and are merged through LDS at the end, which halves the
// longest workgroup of a small grid.
template <int D, int QB, int KT, int KS>
__global__ __launch_bounds__(256 * KS) void attention_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                        const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                        float* __restrict__ lse2, float* __restrict__ lse_out, int Hq,
                                                        int Hkv, int n, int n_rb, float c) {
  using M = Mfma<__bf16>;
  constexpr int NK = D / M::KS;           // MFMA k-steps of q . k
  constexpr int NS = D / 32;              // 32-wide output slices
  constexpr int RW = 32 * QB;             // query rows per wave
  constexpr int RG = 4 * RW;              // query rows per workgroup
  constexpr int NU = KT / 32;             // 32-key units per tile
  constexpr int kKRB = D * 2 + kPadBytes;
  constexpr int kVRB = D * 2 + 16 * kAttnVPadSlots;
  static_assert(NU >= 1 && KT % 32 == 0, "key tile must be whole units");
  static_assert(KS == 1 || KS == 2, "one or two key groups");
  __shared__ __attribute__((aligned(16))) unsigned char ktile[KS][2][KT * kKRB];
  __shared__ __attribute__((aligned(16))) unsigned char vtile[KS][2][KT * kVRB];

  // heaviest row blocks first; the blocks of one head are Hq apart in launch
  // order, so with Hq a multiple of 8 they share an XCD (and its L2) for K, V
  const int hq = (int)(blockIdx.x % Hq), rb = n_rb - 1 - (int)(blockIdx.x / Hq);
  const int b = blockIdx.y, G = Hq / Hkv;
  const size_t bh = (size_t)b * Hq + hq;
  const size_t kvh = ((size_t)b * Hkv + hq / G) * (size_t)n * D;
  const __bf16* Qh = Q + bh * n * D;
  const __bf16* Kh = K + kvh;
  const __bf16* Vh = V + kvh;

  const int grp = wave_id() / 4, wave = wave_id() % 4, lane = threadIdx.x & 63;
  const int q0 = rb * RG + wave * RW;                    // this wave's first query row
  const int qlast = q0 + RW - 1;
  const int kend = min(n, (rb + 1) * RG);               // keys any row of the workgroup sees
  const int ntiles = (kend + KT - 1) / KT;
  const int tpg = (ntiles + KS - 1) / KS;                // key tiles per group (the last group may have fewer)
  const int t_beg = grp * tpg, t_end = min(ntiles, t_beg + tpg);

  bf16x8 qop[QB][NK];
#pragma unroll
  for (int cb = 0; cb < QB; ++cb) {
    const int qr = min(q0 + 32 * cb + (lane & 31), n - 1);   // rows past n are computed and dropped
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qop[cb][kk] = global_operand<__bf16, D>(Qh + (size_t)qr * D, kk, lane);
  }

  f32x16 oacc[QB][NS];
#pragma unroll
  for (int cb = 0; cb < QB; ++cb)
#pragma unroll
    for (int s = 0; s < NS; ++s) oacc[cb][s] = f32x16{};
  float m[QB], l[QB];                                    // running max (log2 units), partial sum of this lane's keys
#pragma unroll
  for (int cb = 0; cb < QB; ++cb) {
    m[cb] = kNegBig;
    l[cb] = 0.f;
  }

  auto unit_active = [&](int key0) { return key0 <= qlast && key0 < kend; };   // wave-uniform
  auto scores = [&](const unsigned char* kt, int kh, f32x16 (&acc)[QB]) {
    bf16x8 a[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) a[kk] = lds_operand<__bf16, D>(kt, 32 * kh + (lane & 31), kk, lane);
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) acc[cb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) acc[cb] = M::mac(a[kk], qop[cb][kk], acc[cb]);
  };
  // softmax numerators of one unit (keys key0 ..) and their product with V
  auto finish = [&](const unsigned char* vt, int kh, int key0, f32x16 (&acc)[QB]) {
    if (key0 + 31 > q0 || key0 + 32 > kend) {            // wave-uniform: diagonal or ragged unit
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
        const int qrow = q0 + 32 * cb + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + acc_row(r, lane);
          if (key > qrow || key >= kend) acc[cb][r] = -INFINITY;
        }
      }
    }
    float mc[QB];
    bool grow = false;
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
      const float mx = tree_max16(acc[cb]);
      mc[cb] = fmaxf(mx, __shfl_xor(mx, 32)) * c;       // the unit's max of this query (both lane halves)
      grow |= mc[cb] > m[cb] + kRescaleLog2;
    }
    if (__any(grow)) {                                   // rare after the first units of a row
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
        const float mn = mc[cb] > m[cb] + kRescaleLog2 ? mc[cb] : m[cb];
        const float alpha = fast_exp2(m[cb] - mn);
        l[cb] *= alpha;
#pragma unroll
        for (int s = 0; s < NS; ++s) oacc[cb][s] *= alpha;
        m[cb] = mn;
      }
    }
    bf16x8 pb[QB][2];
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(acc[cb][r], c, -m[cb]));
      l[cb] += tree_sum16(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[cb][0][e] = (__bf16)p[e];
        pb[cb][1][e] = (__bf16)p[8 + e];
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 va = v_operand<D>(vt, 32 * kh + 16 * t, 32 * s, lane);
#pragma unroll
        for (int cb = 0; cb < QB; ++cb) oacc[cb][s] = M::mac(va, pb[cb][t], oacc[cb][s]);
      }
  };

  LdsLoader<__bf16, D, KT> kload;
  LdsLoader<__bf16, D, KT, kAttnVPadSlots> vload;
  kload.init(wave, lane);
  vload.init(wave, lane);
  if (t_beg < t_end) {                                   // group-uniform
    kload.issue(Kh, t_beg * KT, n, ktile[grp][0], wave);
    vload.issue(Vh, t_beg * KT, n, vtile[grp][0], wave);
  }
  wait_lds_loads();
  __syncthreads();
  f32x16 acc[2][QB];                                     // [buffer][query block]: one unit of 32 keys
  for (int i = 0; i < tpg; ++i) {                        // every group runs tpg steps (one barrier each)
    const int t = t_beg + i;
    const int k0 = t * KT;
    if (t + 1 < t_end) {                                 // in flight during this tile's MFMAs
      kload.issue(Kh, k0 + KT, n, ktile[grp][(i + 1) & 1], wave);
      vload.issue(Vh, k0 + KT, n, vtile[grp][(i + 1) & 1], wave);
    }
    if (t < t_end) {                                     // group-uniform: the last group may run out first
      const unsigned char* kt = ktile[grp][i & 1];
      const unsigned char* vt = vtile[grp][i & 1];
      // units pipelined within the tile: the scores of unit kh are issued before
      // the softmax and P V of unit kh - 1
      int pend = -1;
#pragma unroll
      for (int kh = 0; kh < NU; ++kh) {
        const bool act = unit_active(k0 + 32 * kh);
        if (act) scores(kt, kh, acc[kh & 1]);
        if (pend >= 0) finish(vt, pend, k0 + 32 * pend, acc[pend & 1]);
        pend = act ? kh : -1;
      }
      if (pend >= 0) finish(vt, pend, k0 + 32 * pend, acc[pend & 1]);
    }
    wait_lds_loads();
    __syncthreads();
  }
  if constexpr (KS == 2) {
    // group 1 hands its (max, sum, O) to the lane of group 0 that holds the same query
    // rows and output dims (the tiles are no longer read: the last barrier above)
    constexpr int kFields = QB * NS * 16 + 2 * QB;
    static_assert(4 * 64 * kFields * 4 <= (int)sizeof(ktile), "merge area must fit the key tiles");
    float* xs = reinterpret_cast<float*>(&ktile[0][0][0]) + (size_t)wave * kFields * 64;
    if (grp == 1) {
#pragma unroll
      for (int cb = 0; cb < QB; ++cb) {
        xs[(2 * cb) * 64 + lane] = m[cb];
        xs[(2 * cb + 1) * 64 + lane] = l[cb];
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
          for (int r = 0; r < 16; ++r) xs[(2 * QB + (cb * NS + s2) * 16 + r) * 64 + lane] = oacc[cb][s2][r];
      }
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int cb = 0; cb < QB; ++cb) {
      const float m1 = xs[(2 * cb) * 64 + lane], l1 = xs[(2 * cb + 1) * 64 + lane];
      const float mn = fmaxf(m[cb], m1);
      const float a0 = fast_exp2(m[cb] - mn), a1 = fast_exp2(m1 - mn);
      l[cb] = l[cb] * a0 + l1 * a1;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[cb][s2][r] = oacc[cb][s2][r] * a0 + xs[(2 * QB + (cb * NS + s2) * 16 + r) * 64 + lane] * a1;
      m[cb] = mn;
    }
  }

  // lanes l and l ^ 32 summed disjoint keys of the same query under the same max
#pragma unroll
  for (int cb = 0; cb < QB; ++cb) {
    const float L = l[cb] + __shfl_xor(l[cb], 32);
    const int qrow = q0 + 32 * cb + (lane & 31);
    if (qrow < n) {
      const float inv = 1.0f / L;
      __bf16* orow = O + (bh * n + qrow) * D;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // accumulators 4 j .. 4 j + 3 hold output dims 32 s + 8 j + 4 (lane / 32) + 0..3
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (__bf16)(oacc[cb][s][4 * j + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * s + 8 * j + 4 * (lane >> 5)) = o;
        }
      if (lane < 32) {
        const float v = m[cb] + fast_log2(L);
        if (lse2) lse2[bh * n + qrow] = v;
        if (lse_out) lse_out[bh * n + qrow] = v * kLn2;
      }
    }
  }
}

// Two key groups per workgroup when the grid is bound by its longest workgroup
// rather than by its total work: the longest workgroup (the last row block)
// walks 2 n_rb key tiles, the whole grid B Hq n_rb (n_rb + 1) over two
// workgroups per CU; splitting its keys halves the former and leaves the latter.
template <int D, int QB, int KT>
static hipError_t launch_attention_t(const AttentionArgs& a, hipStream_t st) {
  constexpr int RG = 128 * QB;
  const int n_rb = (a.n + RG - 1) / RG;
  const float c = kLog2e / sqrtf((float)D);
  const bool split = (long long)a.B * a.Hq * (n_rb + 1) < 4LL * a.cus;
  timed_begin(FG_K_ATTENTION, st);
  if (split) {
    attention_kernel<D, QB, KT, 2><<<dim3((unsigned)(a.Hq * n_rb), a.B), dim3(512), 0, st>>>(
        (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (__bf16*)a.O, a.lse2, a.lse_out, a.Hq, a.Hkv, a.n,
        n_rb, c);
  } else {
    attention_kernel<D, QB, KT, 1><<<dim3((unsigned)(a.Hq * n_rb), a.B), dim3(256), 0, st>>>(
        (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (__bf16*)a.O, a.lse2, a.lse_out, a.Hq, a.Hkv, a.n,
        n_rb, c);
  }
  timed_end(st);
  return hipGetLastError();
}

hipError_t launch_attention(const AttentionArgs& a, hipStream_t st) {
  if (a.D == 128) return launch_attention_t<128, 1, 64>(a, st);
  return launch_attention_t<64, 1, 64>(a, st);
}

}  // namespace fg
