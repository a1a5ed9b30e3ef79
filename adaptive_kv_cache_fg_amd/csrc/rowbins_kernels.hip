// Per-row level bins of the prompt's attention on gfx950: for every query row i
// of every query head, the attention mass A_ij the row puts on keys of each
// shortlist level,
//   bins[i][l] = sum_{j <= i : level(i, j) = l} A_ij,  l = 0 special, 1 punct,
//                2 frequent, 3 local (i - j < w_l), 4 the rest,
// (hyper.ai summary of "Model Tells You What to Discard", Method: the
// constraint equation read per row, and the shortlist equation for the levels).
// Summed over rows and the query heads of a group they give the recovery R_k
// that fg_profile obtains from per-key column sums; per row they show how
// evenly a head's rows are served by its policy (the worst row's kept share).
//
// A third sweep over the causal score matrix with the row sweep's orientation:
// K Q^T MFMA tiles, so a lane owns one query row.  P_ij = 2^(x_ij - lse2_i) from
// the row's log-sum-exp, which the caller passes in (fg_profile's optional lse
// output).  The binning itself is a second product on the matrix cores:
// bins^T = L^T P, with L the key-by-level indicator matrix (one 1 per key in
// the column of its level, plus an all-ones column for the row total), fed
// with P split into two bf16 terms, P = hi + lo, so the products carry about 16
// significant bits of each entry (relative error near 2^-17 per entry).  The
// local level depends on the pair, not the key: it is decided per 32-key unit
// where all pairs agree (every pair local, or none), and per element on the
// vector units only in the few units the band edge i - j = w_l crosses.  Key
// tiles are staged with direct global-to-LDS loads, double-buffered, next to
// the keys' indicator rows (bf16) and level codes (0 special, 1 punct,
// 2 frequent, 3 otherwise -- local or the rest).
#include "fg_common.h"
#include "fg_internal.h"
#include "fg_tiles.h"

namespace fg {

constexpr int kBinRows = 256;       // query rows per workgroup (4 waves x 64)
constexpr int kBinKeyTile = 128;    // keys per staged tile
constexpr uint16_t kBf16One = 0x3F80;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// p[0..7] = hi + lo with hi the bf16 rounding of p and lo the bf16 rounding of
// the (exact) remainder; conversions two at a time.
__device__ __forceinline__ void split_bf16(const float* p, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * e], p[2 * e + 1]}, bf16x2));
    const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xFFFF0000u);
    h[e] = hb;
    l[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p[2 * e] - h0, p[2 * e + 1] - h1}, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void rowbins_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                      const uint8_t* __restrict__ cls,
                                                      const uint32_t* __restrict__ fmask,
                                                      const float* __restrict__ lse, float lse_scale,
                                                      float* __restrict__ bins, int Hq, int Hkv, int n, int n_rb,
                                                      int w_l, float c) {
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int NK = D / M::KS;
  constexpr int kRB = D * (int)sizeof(T) + kPadBytes;
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][kBinKeyTile * kRB];
  // indicator rows: levels 0..3, all ones, all zeros; the row stride is padded by 16 bytes so that the
  // lanes reading the same keys of different rows hit different banks
  __shared__ __attribute__((aligned(16))) uint16_t ind[2][6][kBinKeyTile + 8];
  __shared__ __attribute__((aligned(16))) uint8_t kcode[2][kBinKeyTile];

  const int hq = (int)(blockIdx.x % Hq), rb = n_rb - 1 - (int)(blockIdx.x / Hq);   // heaviest row blocks first
  const int b = blockIdx.y, G = Hq / Hkv, h = hq / G;
  const size_t bh = (size_t)b * Hq + hq;
  const T* Qh = Q + bh * n * D;
  const T* Kh = K + ((size_t)b * Hkv + h) * n * D;
  const uint8_t* cl = cls + (size_t)b * n;
  const uint32_t* fm = fmask + ((size_t)b * Hkv + h) * ((n + 31) / 32);

  const int wave = wave_id(), lane = threadIdx.x & 63, tid = threadIdx.x;
  const int q0 = rb * kBinRows + wave * 64;               // this wave's first query row
  const int qlast = q0 + 63;
  const int kend = min(n, (rb + 1) * kBinRows);           // keys any row of the workgroup sees
  const int ntiles = (kend + kBinKeyTile - 1) / kBinKeyTile;

  op_t qop[2][NK];
  float lse2[2];
  int qrow[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    qrow[cb] = q0 + 32 * cb + (lane & 31);
    const int qr = min(qrow[cb], n - 1);                  // rows past n are computed and dropped
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qop[cb][kk] = global_operand<T, D>(Qh + (size_t)qr * D, kk, lane);
    lse2[cb] = lse[bh * n + qr] * lse_scale;
  }
  // bins^T of this wave's two 32-row blocks: accumulator row = level (0..3 kept
  // levels, 4 row total), column = query row
  f32x16 bacc[2] = {f32x16{}, f32x16{}};
  float s3v[2] = {0.f, 0.f};                              // local mass of the band-edge units

  // indicator row of this lane's A operand: its level (lane % 32) if below 5,
  // else the all-zero row
  const int lev = lane & 31;
  const int row_all = lev < 5 ? lev : 5;
  const int row_mixed = lev == 3 ? 5 : row_all;           // units where the local level is decided per pair

  // level code of key j (threads < kBinKeyTile stage one key of the next tile)
  auto code_of = [&](int j) -> uint32_t {
    if (j >= n) return 3;
    const uint8_t t = cl[j];
    if (t == kSpecial) return 0;
    if (t == kPunct) return 1;
    return ((fm[j >> 5] >> (j & 31)) & 1u) ? 2 : 3;
  };
  auto stage = [&](int buf, uint32_t code) {
#pragma unroll
    for (int l = 0; l < 4; ++l) ind[buf][l][tid] = code == (uint32_t)l ? kBf16One : (uint16_t)0;
    kcode[buf][tid] = (uint8_t)code;
  };
  if (tid < kBinKeyTile) {
#pragma unroll
    for (int buf = 0; buf < 2; ++buf) {
      ind[buf][4][tid] = kBf16One;
      ind[buf][5][tid] = 0;
    }
  }
  LdsLoader<T, D, kBinKeyTile> ldr;
  ldr.init(wave, lane);
  ldr.issue(Kh, 0, n, ktile[0], wave);
  uint32_t code_next = tid < kBinKeyTile ? code_of(tid) : 3u;
  wait_lds_loads();
  if (tid < kBinKeyTile) stage(0, code_next);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kBinKeyTile;
    if (t + 1 < ntiles) {                                 // in flight during this tile's MFMAs
      ldr.issue(Kh, k0 + kBinKeyTile, n, ktile[(t + 1) & 1], wave);
      if (tid < kBinKeyTile) code_next = code_of(k0 + kBinKeyTile + tid);
    }
    const unsigned char* kt = ktile[t & 1];
#pragma unroll
    for (int kh = 0; kh < kBinKeyTile / 32; ++kh) {
      const int key0 = k0 + 32 * kh;
      if (key0 > qlast || key0 >= kend) continue;          // wave-uniform: no causal pair in this unit
      op_t a[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) a[kk] = lds_operand<T, D>(kt, 32 * kh + (lane & 31), kk, lane);
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        acc[0] = M::mac(a[kk], qop[0][kk], acc[0]);
        acc[1] = M::mac(a[kk], qop[1][kk], acc[1]);
      }
      // wave-uniform classes of the unit: every pair causal and in range; every
      // pair within the local window; none within it
      const bool interior = key0 + 31 <= q0 && key0 + 32 <= kend;
      const bool all_local = qlast - key0 < w_l;
      const bool no_local = q0 - (key0 + 31) >= w_l;
      // A operands: indicator rows of the unit's keys in MFMA k order (k index
      // 8 h + e stands for key 16 kb + 8 (e / 4) + 4 h + e % 4, the key of
      // accumulator register 8 kb + e)
      const int row = all_local ? row_all : row_mixed;
      bf16x8 lop[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint16_t* ir = &ind[t & 1][row][32 * kh + 16 * kb + 4 * (lane >> 5)];
        const uint2 x = *reinterpret_cast<const uint2*>(ir);
        const uint2 y = *reinterpret_cast<const uint2*>(ir + 8);
        lop[kb] = __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, y.x, y.y});
      }
      uint32_t cw[4] = {0u, 0u, 0u, 0u};
      if (!all_local && !no_local) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          cw[g4] = *reinterpret_cast<const uint32_t*>(&kcode[t & 1][32 * kh + 8 * g4 + 4 * (lane >> 5)]);
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(acc[cb][r], c, -lse2[cb]));
        if (!interior) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + acc_row(r, lane);
            p[r] = (key <= qrow[cb] && key < kend) ? p[r] : 0.f;
          }
        }
        if (!all_local && !no_local) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + acc_row(r, lane);
            const uint32_t code = (cw[r >> 2] >> (8 * (r & 3))) & 0xFFu;
            s3v[cb] += (code == 3u && qrow[cb] - key < w_l) ? p[r] : 0.f;
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          bf16x8 hi, lo;
          split_bf16(p + 8 * kb, hi, lo);
          bacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lop[kb], hi, bacc[cb], 0, 0, 0);
          bacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lop[kb], lo, bacc[cb], 0, 0, 0);
        }
      }
    }
    wait_lds_loads();
    if (t + 1 < ntiles && tid < kBinKeyTile) stage((t + 1) & 1, code_next);
    __syncthreads();
  }
  // lanes 0..31 hold levels 0..3 of their row in registers 0..3, lanes 32..63
  // the row total in register 0
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float total = __shfl_xor(bacc[cb][0], 32);
    const float s3 = s3v[cb] + __shfl_xor(s3v[cb], 32);
    if (lane < 32 && qrow[cb] < n) {
      const float a0 = bacc[cb][0], a1 = bacc[cb][1], a2 = bacc[cb][2], a3 = bacc[cb][3] + s3;
      float* o = bins + (bh * n + qrow[cb]) * 5;
      o[0] = a0;
      o[1] = a1;
      o[2] = a2;
      o[3] = a3;
      o[4] = fmaxf(0.f, total - (a0 + a1 + a2 + a3));     // the rest: all keys minus the kept levels
    }
  }
}

template <typename T, int D>
static hipError_t launch_rowbins_t(const RowBinsArgs& a, hipStream_t st) {
  const int n_rb = (a.n + kBinRows - 1) / kBinRows;
  const float c = kLog2e / sqrtf((float)D);
  timed_begin(FG_K_ROWBINS, st);
  rowbins_kernel<T, D><<<dim3((unsigned)(a.Hq * n_rb), a.B), dim3(256), 0, st>>>(
      (const T*)a.Q, (const T*)a.K, a.cls, a.fmask, a.lse, a.lse_scale, a.bins, a.Hq, a.Hkv, a.n, n_rb, a.w_l, c);
  timed_end(st);
  return hipGetLastError();
}

// Recovery of the row route: per (b, KV head) hd, whose G query heads' rows are
// the G n consecutive rows [hd G n, (hd + 1) G n) of bins, the per-level sums in
// fp64 (each thread a fixed stride of rows, then a fixed reduction tree),
// R_k = (sum_{l <= k} mass_l) / (G n) for k <= 3 and R_4 = 1 by definition,
// policy = min{k : R_k >= T}, and row_min[k] = the least kept share
// sum_{l <= k} bins[i][l] over the rows (row_min[4]: the least row total).
constexpr int kReduceThreads = 256;
__global__ __launch_bounds__(kReduceThreads) void rowbins_reduce_kernel(const float* __restrict__ bins, int G, int n,
                                                                        double T, float* __restrict__ recovery,
                                                                        uint8_t* __restrict__ policy,
                                                                        float* __restrict__ row_min) {
  __shared__ double s_sum[kReduceThreads / kWave][4];
  __shared__ float s_min[kReduceThreads / kWave][5];
  const int hd = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long rows = (long long)G * n;
  const float* base = bins + (size_t)hd * rows * 5;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  float mn[5] = {INFINITY, INFINITY, INFINITY, INFINITY, INFINITY};
  for (long long r = tid; r < rows; r += kReduceThreads) {
    const float* o = base + r * 5;
    const double b0 = o[0], b1 = o[1], b2 = o[2], b3 = o[3], b4 = o[4];
    s[0] += b0;
    s[1] += b1;
    s[2] += b2;
    s[3] += b3;
    const double c1 = b0 + b1, c2 = c1 + b2, c3 = c2 + b3;
    mn[0] = fminf(mn[0], (float)b0);
    mn[1] = fminf(mn[1], (float)c1);
    mn[2] = fminf(mn[2], (float)c2);
    mn[3] = fminf(mn[3], (float)c3);
    mn[4] = fminf(mn[4], (float)(c3 + b4));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
    for (int l = 0; l < 4; ++l) s[l] += __shfl_xor(s[l], o);
#pragma unroll
    for (int l = 0; l < 5; ++l) mn[l] = fminf(mn[l], __shfl_xor(mn[l], o));
  }
  if (lane == 0) {
#pragma unroll
    for (int l = 0; l < 4; ++l) s_sum[wave][l] = s[l];
#pragma unroll
    for (int l = 0; l < 5; ++l) s_min[wave][l] = mn[l];
  }
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    int pol = 4;
    for (int l = 0; l < 4; ++l) {
      double t = 0.0;
      for (int w = 0; w < kReduceThreads / kWave; ++w) t += s_sum[w][l];
      acc += t;
      const double R = acc / (double)rows;
      recovery[(size_t)hd * 5 + l] = (float)R;
      if (pol == 4 && R >= T) pol = l;
    }
    recovery[(size_t)hd * 5 + 4] = 1.0f;
    policy[hd] = (uint8_t)pol;
    if (row_min) {
      for (int l = 0; l < 5; ++l) {
        float m = s_min[0][l];
        for (int w = 1; w < kReduceThreads / kWave; ++w) m = fminf(m, s_min[w][l]);
        row_min[(size_t)hd * 5 + l] = m;
      }
    }
  }
}

hipError_t launch_rowbins_reduce(const float* bins, int H, int G, int n, double T, float* recovery, uint8_t* policy,
                                 float* row_min, hipStream_t st) {
  timed_begin(FG_K_ROWBINS_REDUCE, st);
  rowbins_reduce_kernel<<<dim3(H), dim3(kReduceThreads), 0, st>>>(bins, G, n, T, recovery, policy, row_min);
  timed_end(st);
  return hipGetLastError();
}

hipError_t launch_rowbins(const RowBinsArgs& a, hipStream_t st) {
  if (a.dtype == FG_DTYPE_BF16)
    return a.D == 128 ? launch_rowbins_t<__bf16, 128>(a, st) : launch_rowbins_t<__bf16, 64>(a, st);
  return a.D == 128 ? launch_rowbins_t<float, 128>(a, st) : launch_rowbins_t<float, 64>(a, st);
}

}  // namespace fg
