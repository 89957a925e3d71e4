// Token -> adapter grouping and the sub-tile plan, in one launch.
//
// Grouping the requests that use the same adapter is the segmented gather of
// "Compress then Serve: Serving Thousands of LoRA Adapters with Little
// Overhead", section 2; the per-token adapter index is the `indices` array of
// its section 13.4.  The result is unique: adapters ascend, tokens keep
// ascending index inside a group, ids outside [0, n) go to a trailing group
// n (no adapter).
//
// group_kernel: one workgroup of 16 waves (8 where LDS is short), everything in LDS
// (T <= kGroupMaxT, n <= kGroupMaxN).  A stable counting sort:
//  1. wave w owns a contiguous range of tokens; per 64-token batch, the
//     lanes holding equal groups find each other with one ballot per bit of
//     the group id (the peer mask), so each token gets its rank among the
//     batch's equal tokens before it, and the lowest peer adds the count to
//     the wave's own histogram row (no atomics);
//  2. one block scan over (tokens, sub-tiles) per group gives seg_off and
//     the first sub-tile of each adapter; per group the waves' counts give
//     each wave's base position (groups ascending, waves in token order);
//  3. every token lands at base + earlier peers of its batch, in its wave's
//     order, which is token order: the sort is stable;
//  4. one entry per sub-tile (<= 16 consecutive tokens of one adapter):
//     adapter, first position, tokens, index, token indices.
// plan_kernel: the same entries from a caller's (seg_off, perm).
#include "device_common.h"
#include "host_util.h"
#include "kernels.h"

namespace lora {

struct GroupArgs {
  const int32_t* ids;
  int T, n;
  const int32_t* id_map;  // optional: token t is grouped by id_map[ids[t]] (ids outside [0, id_map_n): none)
  int id_map_n;
  int gbits;  // bits of the group ids 0..n
  int32_t* seg_off;  // optional [n + 2]
  int32_t* perm;     // optional [T]
  char* plan;        // optional, plan_bytes(T, n)
  int max_sub;
  int32_t* n_invalid;  // optional
};

// Inclusive prefix sum over the 64 lanes of a wave by DPP: shifts by 1, 2, 4
// and 8 lanes within each row of 16, then row 0's total added into row 1
// and row 2's into row 3 (row_bcast:15), then the first two rows' total
// into rows 2 and 3 (row_bcast:31).  Lanes with no source read 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return (uint32_t)v;
}

// The grouping scans, per group, its tokens and sub-tiles as one 32-bit
// value, tokens << kSubBits | sub-tiles: with T <= kGroupMaxT and n <=
// kGroupMaxN neither field of any prefix overflows.
constexpr int kSubBits = 12;
static_assert(((int64_t)kGroupMaxT + (int64_t)(kSubTile - 1) * kGroupMaxN) / kSubTile < (1 << kSubBits),
              "sub-tile counts fit their field");
static_assert(((int64_t)kGroupMaxT << kSubBits) < (1ll << 32), "token counts fit their field");

// W waves: 16 where the per-wave histograms fit the LDS with the rest, else
// kGroupWaves (8).
template <int W>
size_t group_lds_bytes_w(int T, int n) {
  const size_t n1 = (size_t)n + 1;
  return 4 * (W * n1 + n1 + (n1 + 1) + (size_t)T);
}
size_t group_lds_bytes(int T, int n) { return group_lds_bytes_w<kGroupWaves>(T, n); }

template <int W>
__global__ void __launch_bounds__(W * 64) group_kernel(GroupArgs p) {
  constexpr int kGroupThreads = W * 64;
  constexpr int kGroupBatches = (kGroupMaxT + kGroupThreads - 1) / kGroupThreads;  // 64-token batches per wave
  constexpr int kGroupPerThread = (kGroupMaxN + 1 + kGroupThreads - 1) / kGroupThreads;  // groups per thread
  extern __shared__ __align__(16) int32_t sm[];
  const int T = p.T, n = p.n, n1 = n + 1;
  int32_t* hist = sm;                  // [W][n1]: counts, then base positions
  int32_t* sub0 = hist + W * n1;       // [n1]: first sub-tile of each group
  int32_t* soff = sub0 + n1;           // [n1 + 1]: seg_off
  int32_t* permL = soff + n1 + 1;      // [T]
  __shared__ uint32_t s_wsum[W];
  __shared__ int s_inval;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < W * n1; i += kGroupThreads) hist[i] = 0;
  if (tid == 0) s_inval = 0;
  const int per = ((T + W - 1) / W + 63) & ~63;
  const int t0 = min(T, w * per), t1 = min(T, t0 + per);
  const int nb = (t1 - t0 + 63) >> 6;

  // 1. Group of each token (all loads issued first), its rank among the
  //    equal tokens before it in its batch, and the wave's histogram.
  int gv[kGroupBatches];
#pragma unroll
  for (int b = 0; b < kGroupBatches; ++b) {
    const int t = t0 + b * 64 + lane;
    gv[b] = (b < nb && t < t1) ? p.ids[t] : -1;
  }
  int inval = 0;
  if (p.id_map) {
#pragma unroll
    for (int b = 0; b < kGroupBatches; ++b)
      if (b < nb) gv[b] = (unsigned)gv[b] < (unsigned)p.id_map_n ? p.id_map[gv[b]] : -1;
  }
  __syncthreads();  // hist zeroed
  int rk[kGroupBatches];  // rank | peers << 8 | leader << 16
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int b = 0; b < kGroupBatches; ++b) {
    rk[b] = 0;
    if (b < nb) {  // uniform over the wave
      const int t = t0 + b * 64 + lane;
      const bool in = t < t1;
      const int v = gv[b];
      const bool ok = (unsigned)v < (unsigned)n;
      if (in && !ok && v != -1 && p.id_map == nullptr) ++inval;
      const int g = ok ? v : n;
      gv[b] = in ? g : -1;
      uint64_t peers = __ballot(in);
      for (int bit = 0; bit < p.gbits; ++bit) {
        const bool set = (g >> bit) & 1;
        const uint64_t bb = __ballot(in && set);
        peers &= set ? bb : ~bb;
      }
      if (in) {
        const int below = __popcll(peers & lt);
        const int cnt = __popcll(peers);
        rk[b] = below | (cnt << 8) | ((below == 0) << 16);
        if (below == 0) hist[w * n1 + g] += cnt;  // the wave's own row: one writer per group
      }
    }
  }
  if (inval) atomicAdd(&s_inval, inval);
  __syncthreads();

  // 2. seg_off, first sub-tiles, and each wave's base position per group.
  //    Thread i takes the gpt consecutive groups from i gpt (gpt as small as
  //    the groups allow, so that few threads loop); one 32-bit scan of
  //    (tokens, sub-tiles) over the threads: a DPP scan per wave, the wave
  //    totals through LDS, one barrier.
  const int gpt = (n1 + kGroupThreads - 1) / kGroupThreads;  // 1 .. kGroupPerThread
  const int a0 = tid * gpt;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kGroupPerThread; ++i) {
    const int a = a0 + i;
    if (i < gpt && a < n1) {
      int c = 0;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) c += hist[ww * n1 + a];
      const int st = a < n ? (c + kSubTile - 1) / kSubTile : 0;
      mine += ((uint32_t)c << kSubBits) | (uint32_t)st;
    }
  }
  const uint32_t incl = wave_inclusive_scan(mine);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  uint32_t pre = incl - mine;
#pragma unroll
  for (int ww = 0; ww < W; ++ww) pre += ww < w ? (uint32_t)s_wsum[ww] : 0u;
#pragma unroll
  for (int i = 0; i < kGroupPerThread; ++i) {
    const int a = a0 + i;
    if (i < gpt && a < n1) {
      int pos = (int)(pre >> kSubBits);
      soff[a] = pos;
      sub0[a] = (int)(pre & ((1u << kSubBits) - 1));
      int c = 0;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const int cw = hist[ww * n1 + a];
        hist[ww * n1 + a] = pos + c;
        c += cw;
      }
      const int st = a < n ? (c + kSubTile - 1) / kSubTile : 0;
      pre += ((uint32_t)c << kSubBits) | (uint32_t)st;
    }
  }
  if (tid == 0) soff[n1] = T;
  __syncthreads();

  // 3. Scatter in token order.
#pragma unroll
  for (int b = 0; b < kGroupBatches; ++b) {
    if (b < nb) {
      const int t = t0 + b * 64 + lane;
      const int g = gv[b];
      if (g >= 0) {
        const int pos = hist[w * n1 + g] + (rk[b] & 0xff);
        if ((unsigned)pos < (unsigned)T) {  // always, for a histogram of these tokens
          permL[pos] = t;
          if (p.perm) p.perm[pos] = t;
        }
      }
      // every lane has read its base before the leaders move it
      if (g >= 0 && (rk[b] >> 16)) hist[w * n1 + g] += (rk[b] >> 8) & 0xff;
    }
  }
  if (p.seg_off)
    for (int a = tid; a <= n1; a += kGroupThreads) p.seg_off[a] = soff[a];
  __syncthreads();

  // 4. The plan: one entry per sub-tile.
  if (p.plan) {
    const int n_sub = min(sub0[n], p.max_sub);
    TileEntry* ent = reinterpret_cast<TileEntry*>(p.plan + kPlanHeaderBytes);
    for (int s = tid; s < n_sub; s += kGroupThreads) {
      int lo = 0, hi = n;  // sub0[lo] <= s < sub0[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sub0[mid] <= s) lo = mid; else hi = mid;
      }
      const int a = lo, j = s - sub0[a];
      const int pos0 = soff[a] + j * kSubTile;
      const int m = min(kSubTile, soff[a + 1] - pos0);
      int v[32];
      v[0] = a; v[1] = pos0; v[2] = m; v[3] = j;
#pragma unroll
      for (int i = 4; i < 8; ++i) v[i] = 0;
#pragma unroll
      for (int i = 0; i < kSubTile; ++i) v[8 + i] = i < m ? permL[pos0 + i] : -1;
#pragma unroll
      for (int i = 24; i < 32; ++i) v[i] = 0;
      int4* dst = reinterpret_cast<int4*>(ent + s);
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[q] = make_int4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    if (tid == 0) {
      int32_t* hdr = reinterpret_cast<int32_t*>(p.plan);
      hdr[0] = n_sub;
      hdr[1] = T;
      hdr[2] = n;
      hdr[3] = 0;
    }
  }
  if (tid == 0 && p.n_invalid) *p.n_invalid = s_inval;
}

// ----------------------------------------------------------- plan of a grouping
// The plan of a caller-supplied grouping: one workgroup scans the sub-tile
// counts, then writes the entries in parallel.  With a store, it also writes
// each sub-tile's metadata (h given directly: one partial sum).
template <int APT>
__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t* __restrict__ seg_off, const int32_t* __restrict__ perm, int T, int n, int max_sub,
            char* __restrict__ plan, const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank,
            const float* __restrict__ scale, TileMeta* __restrict__ meta) {
  extern __shared__ int s_sub[];  // [n + 1]: first sub-tile of each adapter
  __shared__ uint64_t s_wsum[16];
  const int tid = threadIdx.x;
  const int a0 = tid * APT;
  int sub_[APT];
  uint64_t mine = 0;
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int a = a0 + i;
    int c = a < n ? seg_off[a + 1] - seg_off[a] : 0;
    c = c > 0 ? (c < T ? c : T) : 0;
    sub_[i] = a < n ? (c + kSubTile - 1) / kSubTile : 0;
    mine += (uint64_t)sub_[i];
  }
  uint64_t tot;
  uint64_t s = block_exclusive_scan<16>(mine, s_wsum, &tot);
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    if (a0 + i < n) s_sub[a0 + i] = (int)s;
    s += sub_[i];
  }
  const int total = min((int)tot, max_sub);
  if (tid == 0) {
    s_sub[n] = (int)tot;
    int32_t* hdr = reinterpret_cast<int32_t*>(plan);
    hdr[0] = total;
    hdr[1] = T;
    hdr[2] = n;
    hdr[3] = 0;
  }
  __syncthreads();
  TileEntry* entries = reinterpret_cast<TileEntry*>(plan + kPlanHeaderBytes);
  for (int st = tid; st < total; st += 1024) {
    int lo = 0, hi = n;  // s_sub[lo] <= st < s_sub[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_sub[mid] <= st) lo = mid; else hi = mid;
    }
    const int a = lo, j = st - s_sub[a];
    const int pos0 = seg_off[a] + j * kSubTile;
    const int m = min(kSubTile, seg_off[a + 1] - pos0);
    TileEntry e;
    e.a = a;
    e.pos0 = pos0;
    e.m = m;
    e.j = j;
#pragma unroll
    for (int i = 0; i < 4; ++i) e.pad0[i] = 0;
#pragma unroll
    for (int i = 0; i < kSubTile; ++i) {
      const int q = pos0 + i;
      const int tk = (i < m && q >= 0 && q < T) ? perm[q] : -1;
      e.tok[i] = (unsigned)tk < (unsigned)T ? tk : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) e.pad1[i] = 0;
    entries[st] = e;
    if (meta) {
      TileMeta tm;
      tm.r = rank[a];
      tm.row_off = row_off[a];
      tm.scale = scale[a];
      tm.S = 1;
      meta[st] = tm;
    }
  }
}

// --------------------------------------------------------------- host
static int bits_for(int v) {  // smallest b >= 1 with 2^b > v
  int b = 1;
  while ((1 << b) <= v) ++b;
  return b;
}

bool group_fits(int T, int n) { return T <= kGroupMaxT && n >= 1 && n <= kGroupMaxN; }

hipError_t launch_group(const int32_t* ids, int T, int n, const int32_t* id_map, int id_map_n, int32_t* seg_off,
                        int32_t* perm, char* plan, int32_t* n_invalid, hipStream_t stream) {
  GroupArgs a;
  a.ids = ids;
  a.T = T;
  a.n = n;
  a.id_map = id_map;
  a.id_map_n = id_map_n;
  a.gbits = bits_for(n);
  a.seg_off = seg_off;
  a.perm = perm;
  a.plan = plan;
  a.max_sub = (int)plan_max_subtiles(T, n);
  a.n_invalid = n_invalid;
  // 16 waves halve each wave's share of the tokens, where their 16
  // histogram rows fit the LDS (n up to about 1500 at T = 8192).
  const size_t lds16 = group_lds_bytes_w<16>(T, n);
  if (lds16 + 1024 <= 160 * 1024) {  // room for the static LDS
    static DynLdsLimit lim16;
    hipError_t e = ensure_dynamic_lds(lim16, reinterpret_cast<const void*>(group_kernel<16>), lds16);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(group_kernel<16>, dim3(1), dim3(16 * 64), lds16, stream, a);
    return hipGetLastError();
  }
  const size_t lds = group_lds_bytes_w<kGroupWaves>(T, n);
  static DynLdsLimit lim;
  hipError_t e = ensure_dynamic_lds(lim, reinterpret_cast<const void*>(group_kernel<kGroupWaves>), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(group_kernel<kGroupWaves>, dim3(1), dim3(kGroupWaves * 64), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* seg_off, const int32_t* perm, int T, int n, char* plan,
                       const lora_store* store, TileMeta* meta, hipStream_t stream) {
  const int max_sub = (int)plan_max_subtiles(T, n);
  const size_t lds = (size_t)(n + 1) * 4;
  const int32_t* ro = store ? store->row_off : nullptr;
  const int32_t* rk = store ? store->rank : nullptr;
  const float* sc = store ? store->scale : nullptr;
  if (n <= 4096) {
    hipLaunchKernelGGL(plan_kernel<4>, dim3(1), dim3(1024), lds, stream, seg_off, perm, T, n, max_sub, plan, ro, rk,
                       sc, meta);
  } else {
    static DynLdsLimit lim;
    hipError_t e = ensure_dynamic_lds(lim, reinterpret_cast<const void*>(plan_kernel<16>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_kernel<16>, dim3(1), dim3(1024), lds, stream, seg_off, perm, T, n, max_sub, plan, ro,
                       rk, sc, meta);
  }
  return hipGetLastError();
}

}  // namespace lora
