// Token -> adapter grouping and the tile plan.
//
// Grouping the requests that use the same adapter is the segmented-gather
// idea of "Compress then Serve: Serving Thousands of LoRA Adapters with
// Little Overhead", section 2; the per-token adapter index is the
// `indices` array of its section 13.4.  The result is made unique: adapters
// ascend, tokens keep ascending index inside a group, ids outside [0, n) go
// to a trailing group n.
//
// One workgroup does the whole job in LDS (4 waves for T <= 2048, else 16):
//  1. key[t] = (group << tbits) | t.
//  2. LSD radix sort over the group bits, 8 bits per pass (one pass for
//     n < 256, two for n < 65536).  Each pass is stable: every wave owns a
//     contiguous block of positions, ranks equal digits inside each
//     64-position batch with ballots (peer mask = intersection of one ballot
//     per digit bit) and keeps a running count per digit; the per-(digit,
//     wave) counts are scanned in digit-major, wave-minor order, which places
//     earlier waves first.
//  3. perm = low bits of the sorted keys; seg_off[b] = lower_bound(b).
#include "device_common.h"
#include "host_util.h"
#include "kernels.h"

namespace lora {

constexpr int kDigitBits = 8;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kSmallSegT = 2048;  // T up to this uses the 4-wave variant

template <int W>
__global__ void __launch_bounds__(W * 64)
segment_kernel(const int32_t* __restrict__ ids, int T, int n, int tbits, int passes, int cap,
               int32_t* __restrict__ seg_off, int32_t* __restrict__ perm,
               int32_t* __restrict__ n_invalid) {
  constexpr int THREADS = W * 64;
  constexpr int MAXB = (W == 4 ? kSmallSegT : LORA_SEGMENT_MAX_T) / THREADS;  // batches of 64 per wave
  constexpr int PER = kDigits * W / THREADS;                                   // scan entries per thread
  extern __shared__ uint32_t dyn[];
  __shared__ int s_cnt[W][kDigits];
  __shared__ unsigned long long s_wsum[W];
  __shared__ int s_inval;
  uint32_t* in = dyn;
  uint32_t* out = dyn + cap;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  if (tid == 0) s_inval = 0;
  for (int i = tid; i < W * kDigits; i += THREADS) (&s_cnt[0][0])[i] = 0;
  int inval = 0;
  for (int i = tid; i < T; i += THREADS) {
    const int v = ids[i];
    const bool ok = v >= 0 && v < n;
    if (!ok && v != -1) ++inval;
    const uint32_t g = ok ? (uint32_t)v : (uint32_t)n;
    in[i] = (g << tbits) | (uint32_t)i;
  }
  __syncthreads();
  if (inval) atomicAdd(&s_inval, inval);

  // Positions [w * chunk, (w + 1) * chunk) belong to wave w.
  const int chunk = ((T + W - 1) / W + 63) / 64 * 64;
  const int nb = chunk / 64;
  const int start = w * chunk;
  const uint64_t lt = lanemask_lt();

  for (int p = 0; p < passes; ++p) {
    const int shift = tbits + kDigitBits * p;
    uint32_t key[MAXB];
    int loc[MAXB];
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      key[b] = 0;
      loc[b] = -1;
      if (b < nb) {
        const int pos = start + b * 64 + lane;
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
    // Counts in (digit, wave) order, PER consecutive entries per thread.
    int v[PER], sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = tid * PER + q;
      v[q] = s_cnt[idx % W][idx / W];
      sum += v[q];
    }
    unsigned long long tot;
    int run = (int)block_exclusive_scan<W>((unsigned long long)sum, s_wsum, &tot);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = tid * PER + q;
      s_cnt[idx % W][idx / W] = run;  // now the base of (digit, wave)
      run += v[q];
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      if (b < nb && loc[b] >= 0) {
        const int d = (int)((key[b] >> shift) & (kDigits - 1));
        out[s_cnt[w][d] + loc[b]] = key[b];
      }
    }
    __syncthreads();
    // Each wave clears its own counter row; only that wave reads it next pass.
    for (int i = lane; i < kDigits; i += 64) s_cnt[w][i] = 0;
    uint32_t* t = in;
    in = out;
    out = t;
  }

  const uint32_t tmask = (1u << tbits) - 1u;
  for (int i = tid; i < T; i += THREADS) perm[i] = (int32_t)(in[i] & tmask);
  for (int b = tid; b <= n + 1; b += THREADS) {
    const uint32_t target = (uint32_t)b << tbits;
    int lo = 0, hi = T;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (in[mid] < target) lo = mid + 1; else hi = mid;
    }
    seg_off[b] = lo;
  }
  __syncthreads();
  if (tid == 0 && n_invalid != nullptr) *n_invalid = s_inval;
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

size_t segment_static_lds_bytes() { return 16 * kDigits * 4 + 16 * 8 + 16; }

template <int W>
static hipError_t launch_segment_w(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm,
                                   int32_t* n_invalid, hipStream_t stream) {
  const int tbits = T > 1 ? bits_for(T - 1) : 1;
  const int gbits = bits_for(n);  // group ids 0..n
  const int passes = (gbits + kDigitBits - 1) / kDigitBits;
  const int cap = T > n + 2 ? T : n + 2;
  const size_t lds = segment_lds_bytes(T, n);
  static DynLdsLimit lim;
  hipError_t e = ensure_dynamic_lds(lim, reinterpret_cast<const void*>(segment_kernel<W>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(segment_kernel<W>, dim3(1), dim3(W * 64), lds, stream, ids, T, n, tbits, passes, cap,
                     seg_off, perm, n_invalid);
  return hipGetLastError();
}

hipError_t launch_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm,
                          int32_t* n_invalid, hipStream_t stream) {
  if (T <= kSmallSegT) return launch_segment_w<4>(ids, T, n, seg_off, perm, n_invalid, stream);
  return launch_segment_w<16>(ids, T, n, seg_off, perm, n_invalid, stream);
}

}  // namespace lora
