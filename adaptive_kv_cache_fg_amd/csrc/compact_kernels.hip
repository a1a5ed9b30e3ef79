// Compaction of K/V into ragged head-specific caches (hyper.ai summary of
// "Model Tells You What to Discard", Method, second paragraph:
// K_C, V_C = f(K, V, C)).
//
// The cache of a head holds the prompt keys its first generated token (query
// row n) keeps: {j < n : level(n, j) <= policy}.  Permanent rows -- special,
// punct (policy >= 1), frequent (policy >= 2), everything (policy 4) -- are
// packed in ascending position after a ring of w_l - 1 slots that holds the
// normal keys of the local window (policy 3); slot = position mod (w_l - 1),
// so a new token always lands in the slot of the key leaving the window.
//
// Kernels: a per-head count (plan), one scan over heads for row and work-item
// offsets (one workgroup does both for plans of modest size), and a gather
// over (head, 64-position chunk) whose workgroups rank their kept keys with a
// wave ballot prefix and copy rows with 16-byte loads; the last chunk of a
// head also writes the head's decode work items.
#include "fg_common.h"
#include "fg_internal.h"

namespace fg {

constexpr int kPosChunk = 64;      // positions per gather workgroup (one wave): the most workgroups for the copy
constexpr int kCopyBatch = 4;     // 16-byte chunks of K and of V per thread in flight in the gather's copy
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool fbit(const uint32_t* fm, int j) { return (fm[j >> 5] >> (j & 31)) & 1u; }

__device__ __forceinline__ bool perm_keep(uint8_t c, bool f, int pol) {
  return c == kSpecial || (c == kPunct && pol >= 1) || (f && pol >= 2) || pol == 4;
}

__device__ __forceinline__ int ring_slots(int pol, int w_l) { return (pol == 3 && w_l >= 2) ? w_l - 1 : 0; }

// Permanent-key mask of the 32 positions [32w, 32w + 32) of one head, bit i =
// position 32w + i, from 8 aligned 4-byte words of class bytes (each byte 0, 1
// or 2: bit 0 = special, bit 1 = punct) and the frequent-set word.  The caller
// guarantees that the 32 positions exist and that cl32 is 4-byte aligned.
__device__ __forceinline__ uint32_t perm_mask_word(const uint32_t* cl32, const uint32_t* fm, int w, int pol) {
  if (pol == 4) return 0xffffffffu;
  const uint32_t f = pol >= 2 ? fm[w] : 0u;
  uint32_t m = 0u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t x = cl32[8 * w + k];
    uint32_t keep = x & 0x01010101u;                             // special
    if (pol >= 1) keep |= (x >> 1) & 0x01010101u;                // punct
    keep |= (((f >> (4 * k)) & 0xFu) * 0x00204081u) & 0x01010101u;   // frequent: 4 bits spread to bytes
    m |= ((keep * 0x10204080u) >> 28) << (4 * k);                // byte bits gathered back in order
  }
  return m;
}

__device__ __forceinline__ int block_sum_i(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;   // valid in every thread
}

// Permanent prompt keys (np) and window keys in the ring (nr) of head hd, summed
// over this thread's share: words t0, t0 + stride, ... and the tail positions
// likewise.
__device__ __forceinline__ void head_counts(const uint8_t* __restrict__ cls, const uint8_t* __restrict__ policy,
                                            const uint32_t* __restrict__ fmask, int Hkv, int n, int w_l, int hd,
                                            int t0, int stride, int& np_out, int& nr_out) {
  const int b = hd / Hkv;
  const int nw = (n + 31) / 32;
  const uint8_t* cl = cls + (size_t)b * n;
  const uint32_t* fm = fmask + (size_t)hd * nw;
  const int pol = policy[hd];
  const int R = ring_slots(pol, w_l);
  int np = 0, nr = 0;
  int j0 = 0;                                              // positions below j0 are counted by words
  if ((reinterpret_cast<uintptr_t>(cl) & 3u) == 0) {       // class row 4-byte aligned: 32 positions a step
    const uint32_t* cl32 = reinterpret_cast<const uint32_t*>(cl);
    for (int w = t0; w < n / 32; w += stride) {
      const uint32_t m = perm_mask_word(cl32, fm, w, pol);
      np += __popc(m);
      if (R > 0) {                                         // normal keys of the window [n - R, n)
        const int lo = max(n - R - 32 * w, 0);
        if (lo < 32) nr += __popc(~m & (0xffffffffu << lo));
      }
    }
    j0 = (n / 32) * 32;
  }
  for (int j = j0 + t0; j < n; j += stride) {
    const bool pk = perm_keep(cl[j], fbit(fm, j), pol);
    np += pk;
    nr += (!pk && R > 0 && j >= n - R);
  }
  np_out = np;
  nr_out = nr;
}

__global__ __launch_bounds__(256) void plan_kernel(const uint8_t* __restrict__ cls, const uint8_t* __restrict__ policy,
                                                   const uint32_t* __restrict__ fmask, int Hkv, int n, int w_l,
                                                   int max_new, int max_new_kept, int32_t* __restrict__ kept_count,
                                                   int32_t* __restrict__ ring, int32_t* __restrict__ capacity) {
  __shared__ int red[4];
  const int hd = blockIdx.x;
  int np, nr;
  head_counts(cls, policy, fmask, Hkv, n, w_l, hd, (int)threadIdx.x, (int)blockDim.x, np, nr);
  np = block_sum_i(np, red);
  nr = block_sum_i(nr, red);
  if (threadIdx.x == 0) {
    const int pol = policy[hd];
    const int R = ring_slots(pol, w_l);
    kept_count[hd] = np + nr;
    ring[hd] = R;
    capacity[hd] = R + np + (pol == 4 ? max_new : max_new_kept);
  }
}

// Exclusive prefix sums of the heads' rows and decode work items, one
// workgroup: each thread sums a contiguous segment of heads, the segment totals
// are scanned with wave shuffles and one LDS exchange between the waves, then
// every thread writes its segment's offsets.
// NT threads; capacity may sit in global memory or in LDS.
template <int NT>
__device__ __forceinline__ void scan_heads(const int32_t* capacity, int H, int chunk, int64_t* __restrict__ row_offset,
                                           int64_t* __restrict__ work_offset, int64_t* __restrict__ totals) {
  constexpr int kWaves = NT / kWave;
  __shared__ long long wr[kWaves], ww[kWaves];
  __shared__ int wm[kWaves];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int seg = (H + NT - 1) / NT;
  const int i0 = min(H, t * seg), i1 = min(H, i0 + seg);
  long long sr = 0, sw = 0;
  int mw = 1;
  for (int i = i0; i < i1; ++i) {
    const long long cap = capacity[i];
    const long long w = max(1LL, (cap + chunk - 1) / chunk);   // every head gets an item
    sr += cap;
    sw += w;
    mw = max(mw, (int)w);
  }
  // inclusive scans of the segment totals within the wave
  long long ir = sr, iw = sw;
  for (int o = 1; o < kWave; o <<= 1) {
    const long long ar = __shfl_up(ir, o), aw = __shfl_up(iw, o);
    if (lane >= o) {
      ir += ar;
      iw += aw;
    }
  }
  int m = mw;
  for (int o = 1; o < kWave; o <<= 1) m = max(m, __shfl_xor(m, o));
  if (lane == kWave - 1) {
    wr[wave] = ir;
    ww[wave] = iw;
  }
  if (lane == 0) wm[wave] = m;
  __syncthreads();
  long long cr = 0, cw = 0, tr = 0, tw = 0;
  int mx = 1;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      cr += wr[w];
      cw += ww[w];
    }
    tr += wr[w];
    tw += ww[w];
    mx = max(mx, wm[w]);
  }
  // this segment's exclusive start, then its heads in order
  long long r = cr + ir - sr, w = cw + iw - sw;
  for (int i = i0; i < i1; ++i) {
    const long long cap = capacity[i];
    r += cap;
    w += max(1LL, (cap + chunk - 1) / chunk);
    row_offset[i + 1] = r;
    work_offset[i + 1] = w;
  }
  if (t == 0) {
    row_offset[0] = 0;
    work_offset[0] = 0;
    totals[0] = tr;
    totals[1] = tw;
    totals[2] = mx;
  }
}

constexpr int kScanThreads = 256;
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ capacity, int H, int chunk,
                                                            int64_t* __restrict__ row_offset,
                                                            int64_t* __restrict__ work_offset,
                                                            int64_t* __restrict__ totals) {
  scan_heads<kScanThreads>(capacity, H, chunk, row_offset, work_offset, totals);
}

// Plan and scan in one workgroup (one launch instead of two) for small plans:
// at most kPlanScanMaxWords class words in all (H * ceil(n / 32)); beyond that
// one workgroup counting every head is slower than the per-head launch plus the
// scan.  The heads' counts go to LDS (a power-of-two group of threads per
// head, one LDS atomic per thread and head), the capacities replace them
// there, and the scan reads them from LDS.  Integer sums: the result does not
// depend on the order of the atomics.
constexpr int kPlanScanThreads = 1024;
constexpr int kPlanScanMaxHeads = 2048;
constexpr long long kPlanScanMaxWords = 4096;
__global__ __launch_bounds__(kPlanScanThreads) void plan_scan_kernel(
    const uint8_t* __restrict__ cls, const uint8_t* __restrict__ policy, const uint32_t* __restrict__ fmask, int Hkv,
    int n, int w_l, int max_new, int max_new_kept, int H, int chunk, int32_t* __restrict__ kept_count,
    int32_t* __restrict__ ring, int32_t* __restrict__ capacity, int64_t* __restrict__ row_offset,
    int64_t* __restrict__ work_offset, int64_t* __restrict__ totals) {
  __shared__ int s_np[kPlanScanMaxHeads], s_nr[kPlanScanMaxHeads];
  const int tid = threadIdx.x;
  for (int i = tid; i < H; i += kPlanScanThreads) {
    s_np[i] = 0;
    s_nr[i] = 0;
  }
  __syncthreads();
  int tpg = 1;                                             // threads per head
  while (2 * tpg * H <= kPlanScanThreads) tpg *= 2;
  for (int hd = tid / tpg; hd < H; hd += kPlanScanThreads / tpg) {
    int np, nr;
    head_counts(cls, policy, fmask, Hkv, n, w_l, hd, tid % tpg, tpg, np, nr);
    if (np) atomicAdd(&s_np[hd], np);
    if (nr) atomicAdd(&s_nr[hd], nr);
  }
  __syncthreads();
  for (int hd = tid; hd < H; hd += kPlanScanThreads) {
    const int pol = policy[hd];
    const int R = ring_slots(pol, w_l);
    const int np = s_np[hd], nr = s_nr[hd];
    const int cap = R + np + (pol == 4 ? max_new : max_new_kept);
    kept_count[hd] = np + nr;
    ring[hd] = R;
    capacity[hd] = cap;
    s_np[hd] = cap;                                        // the scan's input
  }
  __syncthreads();
  scan_heads<kPlanScanThreads>(s_np, H, chunk, row_offset, work_offset, totals);
}

template <typename T, int D, int CHUNK>
__global__ __launch_bounds__(CHUNK) void gather_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                     const uint8_t* __restrict__ cls, const uint8_t* __restrict__ policy,
                                                     const uint32_t* __restrict__ fmask,
                                                     const int64_t* __restrict__ row_offset, const int32_t* __restrict__ ring,
                                                     int Hkv, int n, int nch, T* __restrict__ Kc, T* __restrict__ Vc,
                                                     int32_t* __restrict__ pos, int32_t* __restrict__ len,
                                                     uint32_t* __restrict__ error_word, int64_t total_rows,
                                                     const int64_t* __restrict__ work_offset, int chunk,
                                                     int32_t* __restrict__ work, int64_t n_work_cap, int S_cap) {
  constexpr int kCPR = D * (int)sizeof(T) / 16;           // 16-byte chunks per row
  constexpr int kWaves = CHUNK / kWave;
  static_assert(CHUNK % kWave == 0 && CHUNK <= 1024, "one position per thread, whole waves");
  __shared__ int red[kWaves];
  __shared__ int wcnt[kWaves], wrows[kWaves];
  __shared__ int src_j[CHUNK], dst_r[CHUNK], zero_r[CHUNK];
  __shared__ int wzero[kWaves];

  const int hd = blockIdx.x / nch, ch = blockIdx.x % nch, b = hd / Hkv;
  const int nw = (n + 31) / 32;
  const uint8_t* cl = cls + (size_t)b * n;
  const uint32_t* fm = fmask + (size_t)hd * nw;
  const int pol = policy[hd];
  const int R = ring[hd];
  const int64_t off = row_offset[hd];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t w0 = work_offset[hd], w1 = work_offset[hd + 1];
  const bool fits_rows = row_offset[hd + 1] <= total_rows;
  const bool fits = fits_rows && w1 <= n_work_cap && w1 - w0 <= S_cap;
  // Decode work items of this head: chunks of its capacity, each (head, first row, first absolute
  // row, rows in use), written by the head's last chunk once its rows in use are known; the decode
  // keeps the counts current on appends.  A head whose plan exceeds the cache's capacities gets
  // empty items (head -1), as do the items past the plan's total.
  auto write_items = [&](int L, bool real) {
    for (int64_t w = w0 + tid; w < min(w1, n_work_cap); w += blockDim.x) {
      const int start = (int)((w - w0) * chunk);
      work[4 * w] = real ? hd : -1;
      work[4 * w + 1] = real ? start : 0;
      work[4 * w + 2] = real ? (int32_t)(off + start) : 0;
      work[4 * w + 3] = real ? min(chunk, max(0, L - start)) : 0;
    }
  };
  if (blockIdx.x == 0) {                                   // one writer of the error word (uniform branch)
    const int H = (int)(gridDim.x / nch);
    int bad = 0;
    for (int h = tid; h < H; h += blockDim.x) {
      const int64_t a0 = work_offset[h], a1 = work_offset[h + 1];
      bad |= (row_offset[h + 1] > total_rows || a1 > n_work_cap || a1 - a0 > S_cap) ? 1 : 0;
    }
    bad = block_sum_i(bad, red);
    if (tid == 0) *error_word = bad ? 2u : 0u;             // bit 2: a plan that does not fit; bit 1 cleared
    for (int64_t w = work_offset[H] + tid; w < n_work_cap; w += blockDim.x) {   // items past the plan's total
      work[4 * w] = -1;
      work[4 * w + 1] = 0;
      work[4 * w + 2] = 0;
      work[4 * w + 3] = 0;
    }
  }
  if (!fits_rows) {                                        // the plan does not fit the cache: head left empty
    if (ch == nch - 1) {
      if (tid == 0) len[hd] = 0;
      write_items(0, false);
    }
    return;
  }

  // permanent keys at positions before this chunk
  int before = 0;
  if ((reinterpret_cast<uintptr_t>(cl) & 3u) == 0) {       // 32 positions a step (all before this chunk exist)
    const uint32_t* cl32 = reinterpret_cast<const uint32_t*>(cl);
    for (int w = tid; w < ch * (CHUNK / 32); w += blockDim.x) before += __popc(perm_mask_word(cl32, fm, w, pol));
  } else {
    for (int j = tid; j < ch * CHUNK; j += blockDim.x) before += perm_keep(cl[j], fbit(fm, j), pol);
  }
  before = block_sum_i(before, red);

  const int j = ch * CHUNK + tid;
  const bool valid = j < n;
  const bool pf = valid && perm_keep(cl[j], fbit(fm, j), pol);
  const bool win = valid && R > 0 && j >= n - R;          // inside the local window of row n
  const bool rf = win && !pf;
  const bool any = pf || rf;
  const bool zs = win && pf;                               // its ring slot stays empty
  const unsigned long long bp = __ballot(pf), ba = __ballot(any), bz = __ballot(zs);
  if (lane == 0) { wcnt[wave] = __popcll(bp); wrows[wave] = __popcll(ba); wzero[wave] = __popcll(bz); }
  __syncthreads();
  int pbefore = 0, abefore = 0, ptotal = 0, atotal = 0, zbefore = 0, ztotal = 0;
  for (int w = 0; w < kWaves; ++w) {
    pbefore += (w < wave) ? wcnt[w] : 0;
    abefore += (w < wave) ? wrows[w] : 0;
    zbefore += (w < wave) ? wzero[w] : 0;
    ptotal += wcnt[w];
    atotal += wrows[w];
    ztotal += wzero[w];
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  if (any) {
    const int e = abefore + __popcll(ba & below);
    const int64_t dst = pf ? off + R + before + pbefore + __popcll(bp & below) : off + (j % R);
    src_j[e] = j;
    dst_r[e] = (int)(dst - off);
    pos[dst] = j;
  }
  if (zs) {                                               // its slot stays empty; its row is zeroed below
    pos[off + (j % R)] = -1;
    zero_r[zbefore + __popcll(bz & below)] = j % R;
  }
  if (ch == 0 && R > 0) {                                  // window positions before the prompt start
    for (int t = tid; t < R; t += blockDim.x) {
      const int jj = n - R + t;
      if (jj < 0) {
        const int64_t zr = off + (((jj % R) + R) % R);
        pos[zr] = -1;
        for (int q = 0; q < kCPR; ++q) {
          reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(Kc) + zr * D * sizeof(T))[q] = make_uint4(0u, 0u, 0u, 0u);
          reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(Vc) + zr * D * sizeof(T))[q] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  }
  if (ch == nch - 1) {
    if (tid == 0) len[hd] = R + before + ptotal;
    write_items(R + before + ptotal, fits);
  }
  __syncthreads();

  const T* Ks = K + (size_t)hd * n * D;
  const T* Vs = V + (size_t)hd * n * D;
  // rows of empty ring slots get zeros: the decode reads every row in use and weights these by 0
  // (values that were never written could hold NaN bit patterns, and 0 * NaN is NaN)
  for (int idx = tid; idx < ztotal * kCPR; idx += blockDim.x) {
    const int e = idx / kCPR, q = idx % kCPR;
    const size_t d = (size_t)(off + zero_r[e]) * D * sizeof(T) + q * 16;
    *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(Kc) + d) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(Vc) + d) = make_uint4(0u, 0u, 0u, 0u);
  }
  // the copy: kCopyBatch 16-byte chunks of K and of V per thread loaded before any is stored, so
  // a thread has 2 * kCopyBatch loads in flight instead of one chunk per memory round trip
  const int total = atotal * kCPR;
  const unsigned char* ks8 = reinterpret_cast<const unsigned char*>(Ks);
  const unsigned char* vs8 = reinterpret_cast<const unsigned char*>(Vs);
  unsigned char* kc8 = reinterpret_cast<unsigned char*>(Kc);
  unsigned char* vc8 = reinterpret_cast<unsigned char*>(Vc);
  for (int base = 0; base < total; base += kCopyBatch * CHUNK) {
    uint4 kr[kCopyBatch], vr[kCopyBatch];
    size_t dd[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {               // no branches: lanes past the end copy the last
      const int idx = min(base + u * CHUNK + tid, total - 1);   // chunk again (the same bytes, same place)
      const int e = idx / kCPR, q = idx % kCPR;
      const size_t sb = (size_t)src_j[e] * D * sizeof(T) + q * 16;
      dd[u] = (size_t)(off + dst_r[e]) * D * sizeof(T) + q * 16;
      kr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks8 + sb)));
      vr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs8 + sb)));
    }
    // non-temporal loads and stores: the prompt rows are read once and the cache rows are not read
    // again by this launch; streaming both past the caches measured faster than ordinary accesses
    // (stores 10-15 %, loads a further 2-3 % at the Llama-1-65B shape)
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, kr[u]), reinterpret_cast<u32x4*>(kc8 + dd[u]));
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, vr[u]), reinterpret_cast<u32x4*>(vc8 + dd[u]));
    }
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  const int H = a.B * a.Hkv;
  if (H <= kPlanScanMaxHeads && (long long)H * ((a.n + 31) / 32) <= kPlanScanMaxWords) {
    timed_begin(FG_K_PLAN, st);
    plan_scan_kernel<<<dim3(1), dim3(kPlanScanThreads), 0, st>>>(
        a.cls, a.policy, a.fmask, a.Hkv, a.n, a.w_l, a.max_new, a.max_new_kept, H, a.chunk_rows, a.kept_count, a.ring,
        a.capacity, a.row_offset, a.work_offset, a.totals);
    timed_end(st);
    return hipGetLastError();
  }
  timed_begin(FG_K_PLAN, st);
  plan_kernel<<<dim3(H), dim3(256), 0, st>>>(a.cls, a.policy, a.fmask, a.Hkv, a.n, a.w_l, a.max_new, a.max_new_kept,
                                             a.kept_count, a.ring, a.capacity);
  timed_end(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timed_begin(FG_K_SCAN, st);
  scan_kernel<<<dim3(1), dim3(kScanThreads), 0, st>>>(a.capacity, H, a.chunk_rows, a.row_offset, a.work_offset,
                                                       a.totals);
  timed_end(st);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_gather_t(const GatherArgs& a, hipStream_t st) {
  const int H = a.B * a.Hkv;
  const int nch = (a.n + kPosChunk - 1) / kPosChunk;
  timed_begin(FG_K_GATHER, st);
  gather_kernel<T, D, kPosChunk><<<dim3(H * nch), dim3(kPosChunk), 0, st>>>(
      (const T*)a.K, (const T*)a.V, a.cls, a.policy, a.fmask, a.row_offset, a.ring, a.Hkv, a.n, nch, (T*)a.Kc,
      (T*)a.Vc, a.pos, a.len, a.error_word, a.total_rows, a.work_offset, a.chunk_rows, a.work, a.n_work,
      a.items_per_head);
  timed_end(st);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t st) {
  if (a.dtype == FG_DTYPE_BF16)
    return a.D == 128 ? launch_gather_t<__bf16, 128>(a, st) : launch_gather_t<__bf16, 64>(a, st);
  return a.D == 128 ? launch_gather_t<float, 128>(a, st) : launch_gather_t<float, 64>(a, st);
}

}  // namespace fg
