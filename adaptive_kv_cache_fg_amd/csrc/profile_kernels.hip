// Head-wise profiling of the prompt on gfx950: two MFMA sweeps over the causal
// score matrix S = Q K^T / sqrt(d).
//
// FastGen's profiling (hyper.ai summary of "Model Tells You What to Discard",
// Method, second paragraph and policy paragraph) needs, per head, the
// attention map A = softmax(S) only through two per-key reductions: the
// cumulative attention of each key (column sums of A, which rank the frequent
// set) and the attention that rows inside the local window give each key (the
// local band).  With those two vectors and the token classes every policy's
// retained mass follows in O(n), so A is never stored:
//
//   sweep 1 (row statistics): one workgroup per 256 query rows, streaming key
//     tiles through double-buffered LDS (next tile's loads in flight during
//     the current tile's MFMAs), keeps an online max / sum of exp2 per query row and
//     writes lse2_i = log2 sum_j 2^{x_ij} with x_ij = S_ij * log2(e).
//   sweep 2 (column sums): one workgroup per 256 keys (all query heads of the
//     KV group), streaming query tiles through LDS, recomputes S, forms
//     P_ij = 2^{x_ij - lse2_i} in fp32 and accumulates each key's column and
//     band sums in registers -- no atomics, no partial buffers, a fixed
//     summation order.
//
// MFMA orientation: sweep 1 computes K Q^T tiles so that a lane owns one query
// row (row reductions stay in-lane); sweep 2 computes Q K^T tiles so that a
// lane owns one key (column reductions stay in-lane).  The operand held in
// registers is the one the workgroup owns (Q rows in sweep 1, K rows in
// sweep 2); the streamed operand is staged in LDS once per workgroup.
#include <algorithm>

#include "fg_common.h"
#include "fg_internal.h"
#include "fg_tiles.h"

namespace fg {

constexpr int kRowsPerWave = 64;  // sweep 1: query rows per wave (two MFMA column blocks)
constexpr int kRowsPerWG = kSweepRowsPerWG;   // sweep 1: 4 waves x 64 query rows
constexpr int kKeyTile = 64;      // sweep 1: keys staged per LDS tile (2 units of 32 keys; 35 KB of LDS for
                                  // both buffers at bf16, d = 128, so three workgroups fit a CU)
constexpr int kKeysPerWave = 64;  // sweep 2: keys per wave (two MFMA column blocks)
constexpr int kKeysPerWG = kSweepKeysPerWG;   // sweep 2: 4 waves x 64 keys
// sweep 2: query rows staged per LDS tile -- 64 (2 slices of 32 rows; 35 KB of LDS for both buffers at
// bf16, d = 128, so three workgroups fit a CU), 128 for the kernel that merges a split sweep 1 (two
// workgroups per CU, so the larger tile halves its barriers)
template <bool RS_SPLIT> constexpr int kRowTile = RS_SPLIT ? 128 : 64;

// Waves per SIMD the sweeps are compiled for: three for bf16 (at most 168 VGPRs), where a third wave
// overlaps the matrix cores and the softmax VALU of the others better than two; no bound otherwise
// (fp32 operands take twice the registers, and three waves would spill).
template <typename T> constexpr int kSweepMinWaves = 1;
template <> constexpr int kSweepMinWaves<__bf16> = 3;

// ---------------------------------------------------------------- sweep 1: row statistics
// A wave owns 64 query rows as two 32-column MFMA blocks (cb = 0, 1) whose B
// operands stay in registers; every A operand (32 keys x KS dims) read from the
// staged K tile feeds both blocks, halving LDS traffic per MFMA.
// Three waves per SIMD at bf16 (the few values that do not fit 168 VGPRs are the tile loader's row
// indices, reloaded only on a ragged last tile): 6 % faster than two at the Llama-1-65B shape.
template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kSweepMinWaves<T>))) void rowstats_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                       float* __restrict__ lse2, float* __restrict__ lse_out,
                                                       float2* __restrict__ rs_part, int Hq, int Hkv, int n,
                                                       int n_rb, int kchunk, float c) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int NK = D / M::KS;
  constexpr int kRB = D * (int)sizeof(T) + kPadBytes;
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][kKeyTile * kRB];

  const int nbh = Hq * (gridDim.y);                      // B * Hq (grid.y = batch)
  const int bh = blockIdx.y * Hq + (int)(blockIdx.x % Hq);
  // (row block, key chunk) of this workgroup, heaviest row blocks first; without
  // splitting (rs_part == nullptr) every row block is one chunk
  int rem = (int)(blockIdx.x / Hq), rb = n_rb - 1, ch = 0;
  for (; rb > 0; --rb) {
    const int nc = split_count(min(n, (rb + 1) * kRowsPerWG), kchunk);
    if (rem < nc) break;
    rem -= nc;
  }
  ch = rem;
  const int n_keys = min(n, (rb + 1) * kRowsPerWG);       // causal keys of the row block, split in balanced chunks
  const int n_ch = split_count(n_keys, kchunk);
  const int b = bh / Hq, hq = bh % Hq, G = Hq / Hkv;
  const T* Qh = Q + (size_t)bh * n * D;
  const T* Kh = K + ((size_t)b * Hkv + hq / G) * n * D;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int q0 = rb * kRowsPerWG + wave * kRowsPerWave;  // this wave's first query row

  op_t qop[2][NK];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int qr = min(q0 + 32 * cb + (lane & 31), n - 1);   // rows past n are discarded below
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qop[cb][kk] = global_operand<T, D>(Qh + (size_t)qr * D, kk, lane);
  }

  float m[2] = {kNegBig, kNegBig}, l[2] = {0.f, 0.f};
  const int kbeg = split_begin(n_keys, n_ch, ch);         // this chunk's keys [kbeg, kend)
  const int kend = min(n_keys, split_begin(n_keys, n_ch, ch + 1));
  const int ntiles = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  const int qlast = q0 + kRowsPerWave - 1;

  // One unit = 32 keys (half a staged tile) x this wave's 64 rows: 16 MFMAs into
  // acc[cb], then an online-softmax update per query block.  Units are software
  // pipelined: the MFMAs of unit u+1 are issued before the softmax of unit u, in
  // one basic block, so the matrix cores and the VALU work at the same time.
  auto unit_active = [&](int key0) { return key0 <= qlast && key0 < kend; };   // wave-uniform
  auto mfma_unit = [&](const unsigned char* kt, int kh, f32x16 (&acc)[2]) {
    op_t a[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) a[kk] = lds_operand<T, D>(kt, 32 * kh + (lane & 31), kk, lane);
    acc[0] = f32x16{};
    acc[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      acc[0] = M::mac(a[kk], qop[0][kk], acc[0]);
      acc[1] = M::mac(a[kk], qop[1][kk], acc[1]);
    }
  };
  auto needs_mask = [&](int key0) { return key0 + 31 > q0 || key0 + 32 > kend; };   // wave-uniform
  // Deferred row maximum: a unit's exponents are taken against the row's reference m[cb], which is
  // raised (and the running sum rescaled) only when some value of the unit lies more than 2^64 above
  // it -- at the row's first unit (m = -big) and rarely after -- so most units need no max tree and
  // no rescale.  (m, l) then stands for l * 2^m with l < 2^75 (at most 2048 terms of at most 2^64
  // each between raises), which every consumer of (max, sum) pairs handles unchanged.
  auto softmax_update = [&](f32x16 (&acc)[2]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(acc[cb][r], c, -m[cb]));
      float ts = tree_sum16(e);
      if (__any(!(ts <= 0x1p64f))) {                         // wave-uniform: raise the reference
        const float m_new = fmaxf(m[cb], tree_max16(acc[cb]) * c);
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(acc[cb][r], c, -m_new));
        ts = tree_sum16(e);
        l[cb] *= fast_exp2(m[cb] - m_new);
        m[cb] = m_new;
      }
      l[cb] += ts;
    }
  };
  auto softmax_unit = [&](int key0, f32x16 (&acc)[2]) {
    if (needs_mask(key0)) {                                  // diagonal or ragged unit: mask
      // accumulator r holds key key0 + acc_row0(r) + 4 * (lane >> 5); it is masked when past the query
      // row or past the chunk: one per-lane threshold against compile-time key offsets
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int qrow = q0 + 32 * cb + (lane & 31);
        const int th = min(qrow, kend - 1) - key0 - 4 * (lane >> 5);   // key offset > th: masked
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row0(r) > th) acc[cb][r] = -INFINITY;
      }
    }
    softmax_update(acc);
  };
  LdsLoader<T, D, kKeyTile> ldr;
  ldr.init(wave, lane);
  ldr.issue(Kh, kbeg, n, ktile[0], wave);
  wait_lds_loads();
  __syncthreads();
  f32x16 acc[2][2];                                          // [buffer][query block], one unit of 32 keys
  int pend_key = -1;                                         // unit whose softmax is pending in acc[1]
  constexpr int NU = kKeyTile / 32;                          // 32-key units per staged tile (even)
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = kbeg + t * kKeyTile;
    if (t + 1 < ntiles) ldr.issue(Kh, k0 + kKeyTile, n, ktile[(t + 1) & 1], wave);   // in flight during the MFMAs below
    const unsigned char* kt = ktile[t & 1];
#pragma unroll
    for (int kh = 0; kh < NU; ++kh) {
      const int key0 = k0 + 32 * kh;
      const bool act = unit_active(key0);
      if (act) mfma_unit(kt, kh, acc[kh & 1]);
      if (pend_key >= 0) softmax_unit(pend_key, acc[(kh & 1) ^ 1]);   // independent of the MFMAs above
      pend_key = act ? key0 : -1;
    }
    wait_lds_loads();
    __syncthreads();
  }
  if (pend_key >= 0) softmax_unit(pend_key, acc[(NU - 1) & 1]);
  // lanes l and l ^ 32 saw disjoint key subsets of the same query row
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float m_o = __shfl_xor(m[cb], 32), l_o = __shfl_xor(l[cb], 32);
    const float M2 = fmaxf(m[cb], m_o);
    const float L = l[cb] * fast_exp2(m[cb] - M2) + l_o * fast_exp2(m_o - M2);
    const int qrow = q0 + 32 * cb + (lane & 31);
    if (lane < 32 && qrow < n) {
      if (rs_part) {                                       // one key chunk: keep (max, sum) for the merge
        rs_part[((size_t)ch * nbh + bh) * n + qrow] = make_float2(M2, L);
      } else {
        const float v = log2_of_scaled(M2, L);
        lse2[(size_t)bh * n + qrow] = v;
        if (lse_out) lse_out[(size_t)bh * n + qrow] = v * kLn2;
      }
    }
  }
}

// ---------------------------------------------------------------- sweep 2: column and band sums
// A wave owns 64 keys as two 32-column MFMA blocks (kc = 0, 1) held in
// registers; every A operand (32 query rows x KS dims) read from the staged Q
// tile feeds both blocks.
// RS_SPLIT: sweep 1 was split over key chunks (rs_part holds their (max, sum) pairs); the unsplit
// kernel carries none of the merge's state, which is what lets it run three waves per SIMD at bf16.
template <typename T, int D, bool RS_SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RS_SPLIT ? 1 : kSweepMinWaves<T>)))
void colsums_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                      float* __restrict__ lse2, float* __restrict__ cum,
                                                      float* __restrict__ band, float2* __restrict__ cs_part,
                                                      const float2* __restrict__ rs_part, int kchunk,
                                                      float* __restrict__ lse_out, int Hq, int Hkv, int n,
                                                      int n_kb, int rchunk, int w_l, float c) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int NK = D / M::KS;
  constexpr int kRB = D * (int)sizeof(T) + kPadBytes;
  __shared__ __attribute__((aligned(16))) unsigned char qtile[2][kRowTile<RS_SPLIT> * kRB];
  __shared__ __attribute__((aligned(16))) float lse_t[2][kRowTile<RS_SPLIT>];

  const int nbh = Hkv * (gridDim.y);                     // B * Hkv (grid.y = batch)
  const int bh = blockIdx.y * Hkv + (int)(blockIdx.x % Hkv);
  // (key block, row chunk) of this workgroup, key block 0 (most rows) first;
  // without splitting (cs_part == nullptr) every key block is one chunk
  int rem = (int)(blockIdx.x / Hkv), kb = 0;
  for (; kb < n_kb - 1; ++kb) {
    const int nc = split_count(n - kb * kKeysPerWG, rchunk);
    if (rem < nc) break;
    rem -= nc;
  }
  const int ch = rem;
  const int n_rows = n - kb * kKeysPerWG;                 // rows at or below the key block, split in balanced chunks
  const int n_ch = split_count(n_rows, rchunk);
  const int b = bh / Hkv, h = bh % Hkv, G = Hq / Hkv;
  const T* Kh = K + (size_t)bh * n * D;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int j0 = kb * kKeysPerWG + wave * kKeysPerWave;   // this wave's first key

  op_t kop[2][NK];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int kr = min(j0 + 32 * kc + (lane & 31), n - 1);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kop[kc][kk] = global_operand<T, D>(Kh + (size_t)kr * D, kk, lane);
  }

  float cum_acc[2] = {0.f, 0.f}, band_acc[2] = {0.f, 0.f};   // per key; summed per query head first
  float cum_g[2] = {0.f, 0.f}, band_g[2] = {0.f, 0.f};
  const int i_begin = kb * kKeysPerWG + split_begin(n_rows, n_ch, ch);   // this chunk's query rows [i_begin, i_end)
  const int i_end = kb * kKeysPerWG + min(n_rows, split_begin(n_rows, n_ch, ch + 1));
  const int ntiles = (i_end - i_begin + kRowTile<RS_SPLIT> - 1) / kRowTile<RS_SPLIT>;   // query tiles per query head
  const int total = G * ntiles;
  LdsLoader<T, D, kRowTile<RS_SPLIT>> ldr;
  ldr.init(wave, lane);
  float lpre = 0.f;
  // With sweep 1 split over key chunks (rs_part), a row's log-sum-exp is merged here from the
  // chunks' (max, sum) pairs: the first kPre pairs are loaded with the tile, the merge waits for
  // the tile's commit; the key block 0 workgroups (which see every row once) write the merged
  // lse2 (so it is complete after either sweep layout) and lse_out.
  constexpr int kPre = 8;
  float2 pre[kPre];
  int pre_nc = 0, pre_row = 0;
  size_t pre_qh = 0;
  const int nbq = Hq * (int)gridDim.y;                   // B * Hq
  // tiles run over (query head g, row tile) with the row tile fastest, from the
  // last rows down: every key block's rows end at n, so workgroups of one head
  // running side by side stream the same Q tiles (shared through L2).  The next
  // tile to issue is tracked incrementally (no integer division per tile).
  int ig = 0, it = 0;
  auto issue = [&](int u) {                                      // tile u = (ig, it) of the sequence
    const int i0 = i_begin + (ntiles - 1 - it) * kRowTile<RS_SPLIT>;   // last rows first (see below)
    const size_t qh = (size_t)b * Hq + (size_t)h * G + ig;
    ldr.issue(Q + qh * n * D, i0, n, qtile[u & 1], wave);
    if (threadIdx.x < kRowTile<RS_SPLIT>) {
      const int row = i0 + (int)threadIdx.x;
      if constexpr (!RS_SPLIT) {
        lpre = row < i_end ? lse2[qh * n + row] : INFINITY;
      } else {
        const int rr = min(row, n - 1);
        pre_nc = split_count(min(n, (rr / kRowsPerWG + 1) * kRowsPerWG), kchunk);
        pre_row = row;
        pre_qh = qh;
#pragma unroll
        for (int k = 0; k < kPre; ++k) pre[k] = rs_part[((size_t)min(k, pre_nc - 1) * nbq + qh) * n + rr];
      }
    }
    if (++it == ntiles) { it = 0; ++ig; }
  };
  auto commit = [&](int u) {                                     // tile u's lse2 into its LDS slot
    wait_lds_loads();
    if (threadIdx.x < kRowTile<RS_SPLIT>) {
      if constexpr (RS_SPLIT) {
        float Mx = kNegBig, Ls = 0.f;
        auto merge = [&](float2 v) {
          if (v.y > 0.f) {
            const float mn = fmaxf(Mx, v.x);
            Ls = Ls * fast_exp2(Mx - mn) + v.y * fast_exp2(v.x - mn);
            Mx = mn;
          }
        };
#pragma unroll
        for (int k = 0; k < kPre; ++k)
          if (k < pre_nc) merge(pre[k]);
        for (int k = kPre; k < pre_nc; ++k) merge(rs_part[((size_t)k * nbq + pre_qh) * n + pre_row]);
        lpre = pre_row < i_end ? log2_of_scaled(Mx, Ls) : INFINITY;
        if (kb == 0 && pre_row < i_end) {                        // every row once: the merged statistics
          lse2[pre_qh * n + pre_row] = lpre;                     // (nothing reads lse2 in a split sweep)
          if (lse_out) lse_out[pre_qh * n + pre_row] = lpre * kLn2;
        }
      }
      lse_t[u & 1][threadIdx.x] = lpre;                           // rows past the chunk get P = 0
    }
  };
  issue(0);
  commit(0);
  __syncthreads();
  int t_cur = 0;                                                 // row tile of tile u
  for (int u = 0; u < total; ++u) {
    if (u + 1 < total) issue(u + 1);
    const int i0 = i_begin + (ntiles - 1 - t_cur) * kRowTile<RS_SPLIT>;
    const unsigned char* qt = qtile[u & 1];
    const float* lt = lse_t[u & 1];
    if (i0 + kRowTile<RS_SPLIT> - 1 >= j0 && i0 < i_end) {                // wave-uniform: some pair is causal
#pragma unroll
      for (int rh = 0; rh < kRowTile<RS_SPLIT> / 32; ++rh) {              // 32-row slices of the tile
        const int r0 = i0 + 32 * rh;
        if (r0 + 31 < j0 || r0 >= i_end) continue;              // wave-uniform
        op_t a[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) a[kk] = lds_operand<T, D>(qt, 32 * rh + (lane & 31), kk, lane);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          acc[0] = M::mac(a[kk], kop[0][kk], acc[0]);
          acc[1] = M::mac(a[kk], kop[1][kk], acc[1]);
        }
        float lrow[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&lt[32 * rh + 8 * q4 + 4 * (lane >> 5)]);
          lrow[4 * q4 + 0] = v[0]; lrow[4 * q4 + 1] = v[1]; lrow[4 * q4 + 2] = v[2]; lrow[4 * q4 + 3] = v[3];
        }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int jc = j0 + 32 * kc;                          // first key of this column block
          const int key = jc + (lane & 31);
          float p[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(acc[kc][r], c, -lrow[r]));
          // accumulator r holds row r0 + acc_row(r, lane) = r0 + acc_row0(r) + 4 * (lane >> 5), so each
          // mask below is one per-lane threshold against compile-time row offsets
          const int lane_row = 4 * (lane >> 5);
          if (r0 < jc + 31) {                                   // diagonal: rows above the key get 0
            const int th = key - r0 - lane_row;                 // row offset < th: above the key
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (acc_row0(r) < th) p[r] = 0.f;
          }
          const float ts = tree_sum16(p);
          cum_g[kc] += ts;
          if ((r0 + 31) - jc < w_l) {
            band_g[kc] += ts;                                   // every pair of the slice is in the band
          } else if (r0 - (jc + 31) < w_l) {
            const int th = key + w_l - r0 - lane_row;           // row offset < th: inside the band
            float tb = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (acc_row0(r) < th) tb += p[r];
            band_g[kc] += tb;
          }
        }
      }
    }
    if (++t_cur == ntiles) {                                    // end of one query head's rows
      t_cur = 0;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        cum_acc[kc] += cum_g[kc];
        band_acc[kc] += band_g[kc];
        cum_g[kc] = 0.f;
        band_g[kc] = 0.f;
      }
    }
    if (u + 1 < total) commit(u + 1);
    __syncthreads();
  }
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const float cs = cum_acc[kc] + __shfl_xor(cum_acc[kc], 32);
    const float bs = band_acc[kc] + __shfl_xor(band_acc[kc], 32);
    const int key = j0 + 32 * kc + (lane & 31);
    if (lane < 32 && key < n) {
      if (cs_part) {                                      // one row chunk: partial sums for the select pass
        cs_part[((size_t)ch * nbh + bh) * n + key] = make_float2(cs, bs);
      } else {
        cum[(size_t)bh * n + key] = cs;
        band[(size_t)bh * n + key] = bs;
      }
    }
  }
}

template <typename T, int D>
static hipError_t launch_profile_sweeps_t(const ProfileArgs& a, hipStream_t st) {
  const int n_rb = (a.n + kRowsPerWG - 1) / kRowsPerWG;
  const int n_kb = (a.n + kKeysPerWG - 1) / kKeysPerWG;
  const float c = kLog2e / sqrtf((float)D);
  // workgroups per (batch entry, head): key chunks of every row block / row chunks of every key block
  long long rs_groups = 0, cs_groups = 0;
  for (int rb = 0; rb < n_rb; ++rb) rs_groups += split_count(std::min(a.n, (rb + 1) * kRowsPerWG), a.kchunk);
  for (int kb = 0; kb < n_kb; ++kb) cs_groups += split_count(a.n - kb * kKeysPerWG, a.rchunk);
  if (!a.lse_ready) {
    timed_begin(FG_K_ROWSTATS, st);
    rowstats_kernel<T, D><<<dim3((unsigned)(a.Hq * rs_groups), a.B), dim3(256), 0, st>>>(
        (const T*)a.Q, (const T*)a.K, a.lse2, a.lse_out, a.rs_part, a.Hq, a.Hkv, a.n, n_rb, a.kchunk, c);
      const hipError_t e = hipGetLastError();      // a split sweep 1 is merged by the column sweep
    timed_end(st);
    if (e != hipSuccess) return e;
  }
  timed_begin(FG_K_COLSUMS, st);
  const float2* rs_part = a.lse_ready ? nullptr : a.rs_part;
  auto colsums = rs_part ? colsums_kernel<T, D, true> : colsums_kernel<T, D, false>;
  colsums<<<dim3((unsigned)(a.Hkv * cs_groups), a.B), dim3(256), 0, st>>>(
      (const T*)a.Q, (const T*)a.K, a.lse2, a.cum, a.band, a.cs_part, rs_part, a.kchunk, a.lse_out, a.Hq, a.Hkv, a.n,
      n_kb, a.rchunk, a.w_l, c);
  timed_end(st);
  return hipGetLastError();
}

hipError_t launch_profile_sweeps(const ProfileArgs& a, hipStream_t st) {
  if (a.dtype == FG_DTYPE_BF16) {
    return a.D == 128 ? launch_profile_sweeps_t<__bf16, 128>(a, st) : launch_profile_sweeps_t<__bf16, 64>(a, st);
  }
  return a.D == 128 ? launch_profile_sweeps_t<float, 128>(a, st) : launch_profile_sweeps_t<float, 64>(a, st);
}

}  // namespace fg
