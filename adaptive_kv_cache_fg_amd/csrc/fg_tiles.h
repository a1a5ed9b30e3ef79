// LDS tile staging and accumulator-tile reductions shared by the MFMA sweeps
// (gfx950, wave64, 256-thread workgroups of 4 waves).
#pragma once

#include "fg_common.h"

namespace fg {

constexpr int kPadBytes = 16;     // default LDS row padding (one 16-byte slot) against bank conflicts

// Staging of a tile of ROWS rows x D elements into LDS with direct
// global-to-LDS loads (global_load_lds_dwordx4): the data never passes through
// registers, so the loads of tile t+1 run while tile t is computed at no VGPR
// cost.  One wave-wide load writes 64 consecutive 16-byte LDS slots; the tile
// is laid out as rows of kChunks data slots plus PAD_SLOTS pad slots (against
// bank conflicts of the operand reads), so slot s holds row s / kSlotsPerRow and
// the lanes that land on a pad slot load a dummy chunk.  Rows at or past n load
// row n - 1 (finite values the callers mask).  The per-lane byte offsets of the
// kPerWave loads do not depend on the tile and are computed once.
template <typename T, int D, int ROWS, int PAD_SLOTS = 1>
struct LdsLoader {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kSlotsPerRow = kChunks + PAD_SLOTS;
  static constexpr int kWaveLoads = ROWS * kSlotsPerRow / 64;
  static constexpr int kPerWave = (kWaveLoads + 3) / 4;   // 4 waves per workgroup
  static_assert(ROWS * kSlotsPerRow % 64 == 0, "tile must be whole wave loads");
  int row[kPerWave], off[kPerWave];                        // tile row and byte offset within it

  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int s = (4 * j + w) * 64 + lane;
      const int r = s / kSlotsPerRow, pos = s - r * kSlotsPerRow;
      row[j] = r;
      off[j] = r * kRowBytes + (pos < kChunks ? pos : 0) * 16;
    }
  }
  // Issue the loads of rows [r0, r0 + ROWS) of src (n rows) into lds.
  __device__ __forceinline__ void issue(const T* src, int r0, int n, unsigned char* lds, int w) const {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(src) + (size_t)r0 * kRowBytes;
    if (r0 + ROWS <= n) {                                  // wave-uniform: the whole tile exists
#pragma unroll
      for (int j = 0; j < kPerWave; ++j) load(base, (unsigned)off[j], lds, j, w);
    } else {
#pragma unroll
      for (int j = 0; j < kPerWave; ++j)
        load(base, (unsigned)(off[j] - max(0, r0 + row[j] - (n - 1)) * kRowBytes), lds, j, w);
    }
  }
  // base is wave-uniform and o a 32-bit lane offset: the scalar-base + vector-offset form.  The empty
  // asm (no instruction) keeps the compiler from hoisting 64-bit copies of the loop-invariant offsets
  // out of the tile loop, which would hold twice the registers for the whole kernel.
  static __device__ __forceinline__ void load(const unsigned char* base, unsigned o, unsigned char* lds, int j,
                                              int w) {
    if (kWaveLoads % 4 != 0 && j == kPerWave - 1 && 4 * j + w >= kWaveLoads) return;
    asm volatile("" : "+v"(o));
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + o),
                                     reinterpret_cast<__attribute__((address_space(3))) void*>(
                                         reinterpret_cast<uintptr_t>(lds + (4 * j + w) * 1024)),
                                     16, 0, 0);
  }
};

// Completion of this wave's direct LDS loads (their writes are then visible to
// the workgroup after the barrier that follows).
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Pairwise (tree) reductions of an accumulator tile: depth 4 instead of a
// 16-long dependent chain, so a wave keeps several VALU ops in flight.
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }  // v_max3_f32
__device__ __forceinline__ float tree_max16(const f32x16& a) {
  const float m0 = max3(a[0], a[1], a[2]), m1 = max3(a[3], a[4], a[5]), m2 = max3(a[6], a[7], a[8]);
  const float m3 = max3(a[9], a[10], a[11]), m4 = max3(a[12], a[13], a[14]);
  return fmaxf(max3(m0, m1, m2), max3(m3, m4, a[15]));
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

}  // namespace fg
