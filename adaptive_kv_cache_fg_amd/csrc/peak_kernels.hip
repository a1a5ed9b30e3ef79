// Micro-benchmarks of the chip's own ceilings, against which the profiling and
// decode kernels are reported next to the vendor figures.  They take no part
// in the method: bf16 MFMA issue rate, transcendental (v_exp_f32) rate, the MFMA rate beside the
// sweeps' softmax work, a plain 16-byte-vector copy and a read-only stream through HBM.
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

// kChains independent 32x32x16 bf16 accumulator chains per wave, operands in
// registers (random bf16 values loaded once from the caller's buffer), so the
// loop is nothing but MFMAs; the sums are stored so the compiler keeps them.
constexpr int kMfmaChains = 4;
__global__ __launch_bounds__(256) void peak_mfma_kernel(const bf16x8* __restrict__ src, float* __restrict__ out,
                                                        int iters) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const bf16x8 a = src[t & 1023];
  const bf16x8 b = src[(t + 512) & 1023];
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[t] = s;
}

// kExpChains independent chains x <- 2^(-x) per lane (the negation is a free
// source modifier, the values settle near 0.64 and stay finite), so the loop is
// nothing but v_exp_f32.
constexpr int kExpChains = 8;
__global__ __launch_bounds__(256) void peak_exp_kernel(float* __restrict__ out, int iters) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  float x[kExpChains];
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) x[c] = 0.01f * c + 1e-6f * (t & 1023);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) s += x[c];
  out[t] = s;
}

// The profiling sweeps' instruction mix with the two kinds of work in different waves of one SIMD:
// a 512-thread workgroup holds 8 waves, and waves w and w + 4 run on the same SIMD.  Waves 0-3 run
// the 4 MFMA chains of peak_mfma_kernel; waves 4-7 run, per lane and iteration, 8 independent
// score updates of the sweeps' softmax (one FMA, one v_exp_f32, one add each).  One iteration of a
// wave pair is 4 MFMAs (512 score pairs at d = 128) against 8 updates per lane (512 pairs), the ratio
// of a sweep, so the MFMA rate of this kernel is the ceiling of a sweep whose MFMA and VALU work
// overlap as well as the chip lets waves of one SIMD overlap them.
__global__ __launch_bounds__(512) void peak_mfma_softmax_kernel(const bf16x8* __restrict__ src,
                                                                float* __restrict__ out, int iters) {
  const int t = blockIdx.x * 512 + threadIdx.x;
  float s = 0.f;
  if (threadIdx.x < 256) {                                   // waves 0-3: MFMA
    const bf16x8 a = src[t & 1023];
    const bf16x8 b = src[(t + 512) & 1023];
    f32x16 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[c][r];
  } else {                                                   // waves 4-7: x <- 2^(x c - m), sum += x
    float x[kExpChains], sum[kExpChains];
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) {
      x[c] = 0.01f * c + 1e-6f * (t & 1023);
      sum[c] = 0.f;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < kExpChains; ++c) {
        x[c] = __builtin_amdgcn_exp2f(fmaf(x[c], 0.18f, -0.5f));   // stays in (0.7, 0.9)
        sum[c] += x[c];
      }
    }
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) s += sum[c];
  }
  out[t] = s;
}

// Grid-stride copy of 16-byte chunks, kCopyUnroll loads in flight per thread
// before their stores; the stores optionally non-temporal (as the gather's).
constexpr int kCopyUnroll = 4;
template <bool NT>
__global__ __launch_bounds__(256) void peak_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        size_t n16) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t base = (size_t)blockIdx.x * 256 + threadIdx.x; base < n16; base += stride * kCopyUnroll) {
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + u * stride;
      if (i < n16) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + u * stride;
      if (i < n16) {
        if (NT)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v[u]), reinterpret_cast<u32x4*>(dst + i));
        else
          dst[i] = v[u];
      }
    }
  }
}

// A read-only stream: 8 independent 16-byte loads per thread in flight over a grid-stride loop
// (plain or non-temporal), each thread's words folded into one word stored at the end so the
// loads are kept.
constexpr int kReadUnroll = 8;
template <bool NT>
__global__ __launch_bounds__(256) void peak_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                        unsigned* __restrict__ out) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0u;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {   // every load in bounds
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = NT ? __builtin_nontemporal_load(s + i + u * stride) : s[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = s[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_peak_mfma(const void* operands, float* out, int iters, int blocks, hipStream_t st) {
  peak_mfma_kernel<<<dim3(blocks), dim3(256), 0, st>>>(static_cast<const bf16x8*>(operands), out, iters);
  return hipGetLastError();
}

hipError_t launch_peak_exp(float* out, int iters, int blocks, hipStream_t st) {
  peak_exp_kernel<<<dim3(blocks), dim3(256), 0, st>>>(out, iters);
  return hipGetLastError();
}

hipError_t launch_peak_mfma_softmax(const void* operands, float* out, int iters, int blocks, hipStream_t st) {
  peak_mfma_softmax_kernel<<<dim3(blocks), dim3(512), 0, st>>>(static_cast<const bf16x8*>(operands), out, iters);
  return hipGetLastError();
}

hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, bool nontemporal, int blocks, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (nontemporal)
    peak_copy_kernel<true><<<dim3(blocks), dim3(256), 0, st>>>(static_cast<const uint4*>(src),
                                                                static_cast<uint4*>(dst), n16);
  else
    peak_copy_kernel<false><<<dim3(blocks), dim3(256), 0, st>>>(static_cast<const uint4*>(src),
                                                                 static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_peak_read(const void* src, size_t bytes, bool nontemporal, int blocks, unsigned* out,
                            hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (nontemporal)
    peak_read_kernel<true><<<dim3(blocks), dim3(256), 0, st>>>(static_cast<const uint4*>(src), n16, out);
  else
    peak_read_kernel<false><<<dim3(blocks), dim3(256), 0, st>>>(static_cast<const uint4*>(src), n16, out);
  return hipGetLastError();
}

}  // namespace fg
