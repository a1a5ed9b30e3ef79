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
//   sweep 1 (row statistics): one workgroup per 128 query rows, streaming key
//     tiles through double-buffered LDS (next tile's loads in flight during
//     the current tile's MFMAs), keeps an online max / sum of exp2 per query row and
//     writes lse2_i = log2 sum_j 2^{x_ij} with x_ij = S_ij * log2(e).
//   sweep 2 (column sums): one workgroup per 128 keys (all query heads of the
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
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

constexpr int kRowsPerWG = 128;   // sweep 1: 4 waves x 32 query rows
constexpr int kKeyTile = 64;      // sweep 1: keys staged per LDS tile
constexpr int kKeysPerWG = 128;   // sweep 2: 4 waves x 32 keys
constexpr int kRowTile = 64;      // sweep 2: query rows staged per LDS tile
constexpr int kPadBytes = 16;     // LDS row padding against bank conflicts

// Staging of a tile of ROWS rows x D elements through LDS in two halves so
// that the global loads of tile t+1 are in flight while tile t is computed:
// prefetch() issues 16-byte loads into registers (zeros past row n), commit()
// writes them into an LDS buffer whose rows are padded against bank conflicts.
template <typename T, int D, int ROWS>
struct Stager {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per row
  static constexpr int kRB = kRowBytes + kPadBytes;
  static constexpr int kPer = ROWS * kChunks / 256;       // chunks per thread (256 threads)
  static constexpr int kBytes = ROWS * kRB;
  uint4 r[kPer];

  __device__ __forceinline__ void prefetch(const T* src, int r0, int n) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + i * 256;
      const int row = c / kChunks, q = c % kChunks;
      r[i] = make_uint4(0u, 0u, 0u, 0u);
      if (r0 + row < n)
        r[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(src) +
                                               (size_t)(r0 + row) * kRowBytes + q * 16);
    }
  }
  __device__ __forceinline__ void commit(unsigned char* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = threadIdx.x + i * 256;
      const int row = c / kChunks, q = c % kChunks;
      *reinterpret_cast<uint4*>(lds + row * kRB + q * 16) = r[i];
    }
  }
};

// Pairwise (tree) reductions of an accumulator tile: depth 4 instead of a
// 16-long dependent chain, so a wave keeps several VALU ops in flight.
__device__ __forceinline__ float tree_max16(const f32x16& a) {
  const float b0 = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
  const float b1 = fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7]));
  const float b2 = fmaxf(fmaxf(a[8], a[9]), fmaxf(a[10], a[11]));
  const float b3 = fmaxf(fmaxf(a[12], a[13]), fmaxf(a[14], a[15]));
  return fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
}
__device__ __forceinline__ float tree_sum16(const float* p) {
  const float b0 = (p[0] + p[1]) + (p[2] + p[3]);
  const float b1 = (p[4] + p[5]) + (p[6] + p[7]);
  const float b2 = (p[8] + p[9]) + (p[10] + p[11]);
  const float b3 = (p[12] + p[13]) + (p[14] + p[15]);
  return (b0 + b1) + (b2 + b3);
}

template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::op_t lds_operand(const unsigned char* lds, int row, int kk, int lane) {
  using M = Mfma<T>;
  constexpr int kRB = D * (int)sizeof(T) + kPadBytes;
  const int col = kk * M::KS + (lane >> 5) * M::EPL;
  return *reinterpret_cast<const typename M::op_t*>(lds + row * kRB + col * (int)sizeof(T));
}

template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::op_t global_operand(const T* rowptr, int kk, int lane) {
  using M = Mfma<T>;
  const int col = kk * M::KS + (lane >> 5) * M::EPL;
  return *reinterpret_cast<const typename M::op_t*>(rowptr + col);
}

// ---------------------------------------------------------------- sweep 1: row statistics
template <typename T, int D>
__global__ __launch_bounds__(256) void rowstats_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                       float* __restrict__ lse2, float* __restrict__ lse_out,
                                                       int Hq, int Hkv, int n, int n_rb, float c) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int NK = D / M::KS;
  constexpr int kRB = D * (int)sizeof(T) + kPadBytes;
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][kKeyTile * kRB];

  const int nbh = gridDim.x / n_rb;                      // B * Hq
  const int rb = n_rb - 1 - (int)(blockIdx.x / nbh);     // heaviest row blocks first
  const int bh = blockIdx.x % nbh;
  const int b = bh / Hq, hq = bh % Hq, G = Hq / Hkv;
  const T* Qh = Q + (size_t)bh * n * D;
  const T* Kh = K + ((size_t)b * Hkv + hq / G) * n * D;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int q0 = rb * kRowsPerWG + wave * 32;
  const int qrow = q0 + (lane & 31);

  op_t qop[NK];
  {
    const int qr = qrow < n ? qrow : n - 1;             // clamp: row discarded below
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qop[kk] = global_operand<T, D>(Qh + (size_t)qr * D, kk, lane);
  }

  float m = kNegBig, l = 0.f;
  const int kend = min(n, (rb + 1) * kRowsPerWG);
  const int ntiles = (kend + kKeyTile - 1) / kKeyTile;
  Stager<T, D, kKeyTile> stg;
  stg.prefetch(Kh, 0, n);
  stg.commit(ktile[0]);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kKeyTile;
    if (t + 1 < ntiles) stg.prefetch(Kh, k0 + kKeyTile, n);   // in flight during the MFMAs below
    const unsigned char* kt = ktile[t & 1];
    // both 32-key halves of the tile: MFMAs first, then one max / rescale / exp pass
    const bool act0 = k0 <= q0 + 31 && k0 < n;                  // wave-uniform
    const bool act1 = k0 + 32 <= q0 + 31 && k0 + 32 < n;
    if (act0) {
      // all LDS operand reads of the tile first, so the MFMA chains never wait on LDS latency
      op_t a0[NK], a1[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        a0[kk] = lds_operand<T, D>(kt, (lane & 31), kk, lane);
        a1[kk] = lds_operand<T, D>(kt, 32 + (lane & 31), kk, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 acc0 = {}, acc1 = {};
      if (act1) {                                                // two independent MFMA chains
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          acc0 = M::mac(a0[kk], qop[kk], acc0);
          acc1 = M::mac(a1[kk], qop[kk], acc1);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc0 = M::mac(a0[kk], qop[kk], acc0);
      }
      if (k0 + 63 > q0 || k0 + 64 > n) {                         // diagonal or ragged tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + acc_row(r, lane);
          if (key > qrow || key >= n) acc0[r] = -INFINITY;
          if (!act1 || key + 32 > qrow || key + 32 >= n) acc1[r] = -INFINITY;
        }
      }
      const float tmax = fmaxf(tree_max16(acc0), tree_max16(acc1));
      const float m_new = fmaxf(m, tmax * c);
      float e0[16], e1[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e0[r] = fast_exp2(fmaf(acc0[r], c, -m_new));
        e1[r] = fast_exp2(fmaf(acc1[r], c, -m_new));
      }
      l = fmaf(l, fast_exp2(m - m_new), tree_sum16(e0) + tree_sum16(e1));
      m = m_new;
    }
    if (t + 1 < ntiles) stg.commit(ktile[(t + 1) & 1]);
    __syncthreads();
  }
  // lanes l and l ^ 32 saw disjoint key subsets of the same query row
  const float m_o = __shfl_xor(m, 32), l_o = __shfl_xor(l, 32);
  const float M2 = fmaxf(m, m_o);
  const float L = l * fast_exp2(m - M2) + l_o * fast_exp2(m_o - M2);
  if (lane < 32 && qrow < n) {
    const float v = M2 + fast_log2(L);
    lse2[(size_t)bh * n + qrow] = v;
    if (lse_out) lse_out[(size_t)bh * n + qrow] = v * kLn2;
  }
}

// ---------------------------------------------------------------- sweep 2: column and band sums
template <typename T, int D>
__global__ __launch_bounds__(256) void colsums_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                      const float* __restrict__ lse2, float* __restrict__ cum,
                                                      float* __restrict__ band, int Hq, int Hkv, int n, int n_kb,
                                                      int w_l, float c) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int NK = D / M::KS;
  constexpr int kRB = D * (int)sizeof(T) + kPadBytes;
  __shared__ __attribute__((aligned(16))) unsigned char qtile[2][kRowTile * kRB];
  __shared__ __attribute__((aligned(16))) float lse_t[2][kRowTile];

  const int nbh = gridDim.x / n_kb;                      // B * Hkv
  const int kb = (int)(blockIdx.x / nbh);                // key block 0 (most rows) first
  const int bh = blockIdx.x % nbh;
  const int b = bh / Hkv, h = bh % Hkv, G = Hq / Hkv;
  const T* Kh = K + (size_t)bh * n * D;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int j0 = kb * kKeysPerWG + wave * 32;            // this wave's first key
  const int key = j0 + (lane & 31);

  op_t kop[NK];
  {
    const int kr = key < n ? key : n - 1;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kop[kk] = global_operand<T, D>(Kh + (size_t)kr * D, kk, lane);
  }

  float cum_acc = 0.f, band_acc = 0.f;
  const int i_begin = kb * kKeysPerWG;
  const int ntiles = (n - i_begin + kRowTile - 1) / kRowTile;   // query tiles per query head
  const int total = G * ntiles;
  Stager<T, D, kRowTile> stg;
  float lpre = 0.f;
  auto issue = [&](int u) {                                      // tile u of the (g, tile) sequence
    const int g = u / ntiles, i0 = i_begin + (u % ntiles) * kRowTile;
    const size_t qh = (size_t)b * Hq + (size_t)h * G + g;
    stg.prefetch(Q + qh * n * D, i0, n);
    if (threadIdx.x < kRowTile) lpre = (i0 + (int)threadIdx.x < n) ? lse2[qh * n + i0 + threadIdx.x] : INFINITY;
  };
  auto commit = [&](int buf) {
    stg.commit(qtile[buf]);
    if (threadIdx.x < kRowTile) lse_t[buf][threadIdx.x] = lpre;     // rows past n get P = 0
  };
  issue(0);
  commit(0);
  __syncthreads();
  float cum_g = 0.f, band_g = 0.f;
  for (int u = 0; u < total; ++u) {
    if (u + 1 < total) issue(u + 1);
    const int i0 = i_begin + (u % ntiles) * kRowTile;
    const unsigned char* qt = qtile[u & 1];
    const float* lt = lse_t[u & 1];
    // both 32-row halves of the tile: MFMAs first, then P = 2^(x - lse2) and tree sums
    const bool act0 = i0 + 31 >= j0 && i0 < n;                 // wave-uniform
    const bool act1 = i0 + 63 >= j0 && i0 + 32 < n;
    if (act0 || act1) {
      // all LDS operand reads of the tile first, so the MFMA chains never wait on LDS latency
      op_t a0[NK], a1[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        a0[kk] = lds_operand<T, D>(qt, (lane & 31), kk, lane);
        a1[kk] = lds_operand<T, D>(qt, 32 + (lane & 31), kk, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 acc0 = {}, acc1 = {};
      if (act0 && act1) {                                        // two independent MFMA chains
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          acc0 = M::mac(a0[kk], kop[kk], acc0);
          acc1 = M::mac(a1[kk], kop[kk], acc1);
        }
      } else if (act0) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc0 = M::mac(a0[kk], kop[kk], acc0);
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) acc1 = M::mac(a1[kk], kop[kk], acc1);
      }
      float p0[16], p1[16];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(&lt[8 * a + 4 * (lane >> 5)]);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(&lt[32 + 8 * a + 4 * (lane >> 5)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p0[4 * a + e] = act0 ? fast_exp2(fmaf(acc0[4 * a + e], c, -v0[e])) : 0.f;
          p1[4 * a + e] = act1 ? fast_exp2(fmaf(acc1[4 * a + e], c, -v1[e])) : 0.f;
        }
      }
      if (i0 < j0 + 32) {                                        // diagonal: rows above the key get 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + acc_row(r, lane);
          if (row < key) p0[r] = 0.f;
          if (row + 32 < key) p1[r] = 0.f;
        }
      }
      const float ts0 = tree_sum16(p0), ts1 = tree_sum16(p1);
      cum_g += ts0 + ts1;
      // local band: rows i with 0 <= i - key < w_l, decided per 32-row half
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int r0 = i0 + 32 * h2;
        const float* ph = h2 ? p1 : p0;
        if ((r0 + 31) - j0 < w_l) {
          band_g += h2 ? ts1 : ts0;                              // every pair of the half is inside the band
        } else if (r0 - (j0 + 31) < w_l) {
          float tb = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (r0 + acc_row(r, lane) - key < w_l) tb += ph[r];
          band_g += tb;
        }
      }
    }
    if ((u + 1) % ntiles == 0) {                        // end of one query head's rows
      cum_acc += cum_g;
      band_acc += band_g;
      cum_g = 0.f;
      band_g = 0.f;
    }
    if (u + 1 < total) commit((u + 1) & 1);
    __syncthreads();
  }
  cum_acc += __shfl_xor(cum_acc, 32);
  band_acc += __shfl_xor(band_acc, 32);
  if (lane < 32 && key < n) {
    cum[(size_t)bh * n + key] = cum_acc;
    band[(size_t)bh * n + key] = band_acc;
  }
}

template <typename T, int D>
static hipError_t launch_profile_sweeps_t(const ProfileArgs& a, hipStream_t st) {
  const int n_rb = (a.n + kRowsPerWG - 1) / kRowsPerWG;
  const int n_kb = (a.n + kKeysPerWG - 1) / kKeysPerWG;
  const float c = kLog2e / sqrtf((float)D);
  timed_begin(FG_K_ROWSTATS, st);
  rowstats_kernel<T, D><<<dim3(a.B * a.Hq * n_rb), dim3(256), 0, st>>>(
      (const T*)a.Q, (const T*)a.K, a.lse2, a.lse_out, a.Hq, a.Hkv, a.n, n_rb, c);
  timed_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timed_begin(FG_K_COLSUMS, st);
  colsums_kernel<T, D><<<dim3(a.B * a.Hkv * n_kb), dim3(256), 0, st>>>(
      (const T*)a.Q, (const T*)a.K, a.lse2, a.cum, a.band, a.Hq, a.Hkv, a.n, n_kb, a.w_l, c);
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
