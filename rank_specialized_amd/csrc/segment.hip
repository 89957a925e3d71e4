// Token -> adapter grouping and the tile plan.
//
// Grouping the requests that use the same adapter is the segmented-gather
// idea of "Compress then Serve: Serving Thousands of LoRA Adapters with
// Little Overhead", section 2; the per-token adapter index is the
// `indices` array of its section 13.4.  The result is made unique: adapters
// ascend, tokens keep ascending index inside a group, ids outside [0, n) go
// to a trailing group n.
//
// One workgroup of 1024 threads (16 waves) does the whole job in LDS:
//  1. key[t] = (group << tbits) | t.
//  2. LSD radix sort over the group bits, 4 bits per pass.  Each pass is
//     stable: every wave owns a contiguous block of positions, ranks equal
//     digits inside each 64-position batch with ballots (peer mask =
//     intersection of one ballot per digit bit) and keeps a running count
//     per digit; the per-(digit, wave) counts are scanned in digit-major,
//     wave-minor order, which places earlier waves first.
//  3. perm = low bits of the sorted keys; seg_off[b] = lower_bound(b).
//  4. Tile plan: every adapter group is cut into runs of at most kTile
//     tokens; block-wide exclusive scans over adapters give each run's slot
//     in the large-tile or small-tile list.
#include "device_common.h"
#include "kernels.h"

namespace lora {

constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / kWave;
constexpr int kDigitBits = 4;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kMaxBatches = LORA_SEGMENT_MAX_T / kSegWaves / kWave;  // batches of 64 per wave

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << __lane_id()) - 1ull;
}

// Exclusive scan of one int per thread across the 1024-thread block.
__device__ int block_exclusive_scan(int v, int* s_wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = lane < kSegWaves ? s_wsum[lane] : 0;
#pragma unroll
    for (int d = 1; d < kSegWaves; d <<= 1) {
      int y = __shfl_up(s, d);
      if (lane >= d) s += y;
    }
    if (lane < kSegWaves) s_wsum[lane] = s;
  }
  __syncthreads();
  const int before = w > 0 ? s_wsum[w - 1] : 0;
  *total = s_wsum[kSegWaves - 1];
  __syncthreads();
  return before + x - v;
}

// Tile plan from group offsets held in LDS (so[0..n]).  Every adapter group
// of c tokens is cut into runs of kTile tokens (expand tiles; runs of more
// than kSmallTile tokens go to the "large" list, written first) and into runs
// of kSubTile tokens (shrink sub-tiles).  Each list is ordered by adapter,
// then position (one block scan each).
__device__ void build_tiles(const int32_t* so, int n, void* plan_ws, size_t sub_off, int* s_wsum) {
  const int per = (n + kSegThreads - 1) / kSegThreads;
  const int a0 = threadIdx.x * per;
  const int a1 = min(n, a0 + per);
  int n_large = 0, n_small = 0, n_sub = 0;
  for (int a = a0; a < a1; ++a) {
    const int c = so[a + 1] - so[a];
    const int rem = c % kTile;
    n_large += c / kTile + (rem > kSmallTile ? 1 : 0);
    n_small += (rem > 0 && rem <= kSmallTile) ? 1 : 0;
    n_sub += (c + kSubTile - 1) / kSubTile;
  }
  int total_large, total_small, total_sub;
  int slot_large = block_exclusive_scan(n_large, s_wsum, &total_large);
  int slot_small = block_exclusive_scan(n_small, s_wsum, &total_small) + total_large;
  int slot_sub = block_exclusive_scan(n_sub, s_wsum, &total_sub);
  char* base = reinterpret_cast<char*>(plan_ws);
  int4* tiles = reinterpret_cast<int4*>(base + kPlanHeaderBytes);
  int4* subs = reinterpret_cast<int4*>(base + sub_off);
  for (int a = a0; a < a1; ++a) {
    const int start = so[a], c = so[a + 1] - so[a];
    for (int k = 0; k < c; k += kTile) {
      const int m = min(kTile, c - k);
      const int4 t = make_int4(a, start + k, m, 0);
      if (m > kSmallTile) tiles[slot_large++] = t; else tiles[slot_small++] = t;
    }
    for (int k = 0; k < c; k += kSubTile) subs[slot_sub++] = make_int4(a, start + k, min(kSubTile, c - k), 0);
  }
  if (threadIdx.x == 0) {
    int32_t* hdr = reinterpret_cast<int32_t*>(plan_ws);
    hdr[0] = total_large + total_small;
    hdr[1] = total_large;
    hdr[2] = total_small;
    hdr[3] = total_sub;
  }
}

__global__ void __launch_bounds__(kSegThreads)
segment_kernel(const int32_t* __restrict__ ids, int T, int n, int tbits, int passes, int cap,
               int32_t* __restrict__ seg_off, int32_t* __restrict__ perm,
               int32_t* __restrict__ n_invalid, void* __restrict__ plan_ws, size_t sub_off) {
  extern __shared__ uint32_t dyn[];
  __shared__ int s_cnt[kSegWaves][kDigits];
  __shared__ int s_base[kSegWaves][kDigits];
  __shared__ int s_wsum[kSegWaves];
  __shared__ int s_inval;
  uint32_t* in = dyn;
  uint32_t* out = dyn + cap;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  if (tid == 0) s_inval = 0;
  if (tid < kSegWaves * kDigits) (&s_cnt[0][0])[tid] = 0;
  __syncthreads();

  int inval = 0;
  for (int i = tid; i < T; i += kSegThreads) {
    const int v = ids[i];
    const bool ok = v >= 0 && v < n;
    if (!ok && v != -1) ++inval;
    const uint32_t g = ok ? (uint32_t)v : (uint32_t)n;
    in[i] = (g << tbits) | (uint32_t)i;
  }
  if (inval) atomicAdd(&s_inval, inval);
  __syncthreads();

  // Positions [w * chunk, (w + 1) * chunk) belong to wave w.
  const int chunk = ((T + kSegWaves - 1) / kSegWaves + kWave - 1) / kWave * kWave;
  const int nb = chunk / kWave;
  const int start = w * chunk;
  const uint64_t lt = lanemask_lt();

  for (int p = 0; p < passes; ++p) {
    const int shift = tbits + kDigitBits * p;
    uint32_t key[kMaxBatches];
    int loc[kMaxBatches];
#pragma unroll
    for (int b = 0; b < kMaxBatches; ++b) {
      key[b] = 0;
      loc[b] = -1;
      if (b < nb) {
        const int pos = start + b * kWave + lane;
        const bool valid = pos < T;
        const uint32_t k = valid ? in[pos] : 0u;
        const int d = (int)((k >> shift) & (kDigits - 1));
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < kDigitBits; ++bit) {
          const bool set = (d >> bit) & 1;
          const uint64_t bb = __ballot(valid && set);
          peers &= set ? bb : ~bb;
        }
        const int rank = __popcll(peers & lt);
        const int base = valid ? s_cnt[w][d] : 0;
        if (valid && rank == 0) s_cnt[w][d] = base + __popcll(peers);
        key[b] = k;
        loc[b] = valid ? base + rank : -1;
      }
    }
    __syncthreads();
    if (w == 0) {
      // 256 counts in (digit, wave) order, 4 per lane.
      int v[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = lane * 4 + q;
        v[q] = s_cnt[idx % kSegWaves][idx / kSegWaves];
        sum += v[q];
      }
      int incl = sum;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      int run = incl - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = lane * 4 + q;
        s_base[idx % kSegWaves][idx / kSegWaves] = run;
        s_cnt[idx % kSegWaves][idx / kSegWaves] = 0;
        run += v[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kMaxBatches; ++b) {
      if (b < nb && loc[b] >= 0) {
        const int d = (int)((key[b] >> shift) & (kDigits - 1));
        out[s_base[w][d] + loc[b]] = key[b];
      }
    }
    __syncthreads();
    uint32_t* t = in;
    in = out;
    out = t;
  }

  const uint32_t tmask = (1u << tbits) - 1u;
  for (int i = tid; i < T; i += kSegThreads) perm[i] = (int32_t)(in[i] & tmask);
  int32_t* so = reinterpret_cast<int32_t*>(out);  // cap >= n + 2
  for (int b = tid; b <= n + 1; b += kSegThreads) {
    const uint32_t target = (uint32_t)b << tbits;
    int lo = 0, hi = T;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (in[mid] < target) lo = mid + 1; else hi = mid;
    }
    so[b] = lo;
    seg_off[b] = lo;
  }
  if (tid == 0 && n_invalid != nullptr) *n_invalid = s_inval;
  __syncthreads();
  build_tiles(so, n, plan_ws, sub_off, s_wsum);
}

__global__ void __launch_bounds__(kSegThreads)
plan_from_offsets_kernel(const int32_t* __restrict__ seg_off, int n, void* __restrict__ plan_ws,
                         size_t sub_off) {
  extern __shared__ uint32_t dyn[];
  __shared__ int s_wsum[kSegWaves];
  int32_t* so = reinterpret_cast<int32_t*>(dyn);
  for (int b = threadIdx.x; b <= n; b += kSegThreads) so[b] = seg_off[b];
  __syncthreads();
  build_tiles(so, n, plan_ws, sub_off, s_wsum);
}

static int bits_for(int v) {  // smallest b >= 1 with 2^b > v
  int b = 1;
  while ((1 << b) <= v) ++b;
  return b;
}

size_t segment_lds_bytes(int T, int n) {
  const int cap = T > n + 2 ? T : n + 2;
  return 2 * (size_t)cap * 4;
}

hipError_t launch_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm,
                          int32_t* n_invalid, void* plan_ws, hipStream_t stream) {
  const int tbits = T > 1 ? bits_for(T - 1) : 1;
  const int gbits = bits_for(n);  // group ids 0..n
  const int passes = (gbits + kDigitBits - 1) / kDigitBits;
  const int cap = T > n + 2 ? T : n + 2;
  const size_t lds = segment_lds_bytes(T, n);
  static size_t raised = 64 * 1024;
  if (lds > raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(segment_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    raised = lds;
  }
  hipLaunchKernelGGL(segment_kernel, dim3(1), dim3(kSegThreads), lds, stream, ids, T, n, tbits, passes,
                     cap, seg_off, perm, n_invalid, plan_ws, plan_subtile_offset(T, n));
  return hipGetLastError();
}

hipError_t launch_plan_from_offsets(const int32_t* seg_off, int T, int n, void* plan_ws,
                                    hipStream_t stream) {
  const size_t lds = (size_t)(n + 2) * 4;
  static size_t raised = 64 * 1024;
  if (lds > raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(plan_from_offsets_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    raised = lds;
  }
  hipLaunchKernelGGL(plan_from_offsets_kernel, dim3(1), dim3(kSegThreads), lds, stream, seg_off, n,
                     plan_ws, plan_subtile_offset(T, n));
  return hipGetLastError();
}

}  // namespace lora
