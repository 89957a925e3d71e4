// Shrink: h[i, j] = sum_k A_a[j, k] x[perm[i], k]   (j < r_a), float32.
//
// Step 1 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4: A applied with scale
// 1 into a float32 buffer of shape [tokens, R].  Tokens are taken in groups
// of one adapter (the segmented gather of its section 2), so each adapter's
// retained rows are read once per sub-tile of at most 16 of its tokens.
//
// Work item = (sub-tile, K chunk); one workgroup of 8 waves per item, a
// grid-stride loop over the items (two workgroups per CU).  A sub-tile is the skinny GEMM
//   H^T[r_a x m] = A_a[r_a x d_in] . X^T[d_in x m]      (m <= 16)
// on 16x16 MFMA tiles whatever m is.  d_in is cut into S chunks (S <= 8) so
// that a popular or high-rank adapter's rows spread over several CUs; inside
// an item each wave takes `spw` consecutive K steps and issues all of their
// loads before the first MFMA.  The 8 waves' float32 tiles are summed in
// LDS in wave order, and chunk kc's sum is written as partial kc; the
// consumer adds the S partials in chunk order.  No atomics: results are
// deterministic.
//
// Token grouping happens inside every workgroup, so no separate launch and
// no round trip through memory precede the factor loads:
//  * from ids (n <= 4096): a histogram of the ids in LDS, one block scan of
//    (tokens, sub-tiles, items) per adapter, and for each item the
//    sub-tile's tokens by a ballot rank over the ids (tokens keep ascending
//    index);
//  * from a grouping (seg_off, perm): the same scan over seg_off.
// Every adapter's rank, row offset and scale are loaded while the histogram
// forms (one load each per thread), so the item loop finds its adapter's
// metadata in the cache.
// Item 0 of each sub-tile writes the sub-tile's plan entry (adapter,
// position, tokens, rank, row offset, scale) for the expand.
//
// Rank specialization: NG = ceil(r_a / 16) row groups is a template
// parameter; rows j >= r_a and tokens >= m are never loaded.
#include "device_common.h"
#include "host_util.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {


struct ShrinkArgs {
  const int32_t* ids;      // ids mode
  const int32_t* seg_off;  // grouping mode
  const int32_t* perm;     // grouping mode
  int T, n, max_sub;
  const char* x;
  int64_t ldx_bytes;
  const char* a_pack;
  const int32_t* row_off;
  const int32_t* rank;
  const float* scale;
  int d_in, ng_max;
  int spw[5], S[5], kchunk[5];  // by row groups ng = 1..4
  float* part;
  int64_t ldp, pstride;  // floats: row stride, distance between partials
  char* plan;
  // ids mode: when set, token t is grouped by id_map[ids[t]] (ids outside
  // [0, id_map_n) by -1), e.g. the cluster of its adapter.
  const int32_t* id_map;
  int id_map_n;
};

// v[ng] for ng = 1..4 without indexing the argument array at run time
// (which would copy it to private memory).  The four values are taken as
// wave-uniform scalars first: a select between argument fields is otherwise
// turned into one vector load of the selected field, a memory round trip
// (waited for at once) wherever ng differs across lanes.
__device__ __forceinline__ int by_ng(const int (&v)[5], int ng) {
  const int v1 = __builtin_amdgcn_readfirstlane(v[1]), v2 = __builtin_amdgcn_readfirstlane(v[2]);
  const int v3 = __builtin_amdgcn_readfirstlane(v[3]), v4 = __builtin_amdgcn_readfirstlane(v[4]);
  return ng <= 1 ? v1 : ng == 2 ? v2 : ng == 3 ? v3 : v4;
}

// Grouping state in LDS (no per-thread state lives across the item loop):
//   info[a]  = tokens of adapter a | row groups of its rank << 20 (0: rank 0)
//   pref[t]  = exclusive prefix, over the adapters of threads < t, of
//              tokens << 44 | sub-tiles << 24 | items; pref[threads] = total
// Thread t owns adapters [t * APT, (t + 1) * APT).  A workgroup takes items
// blockIdx.x + k * gridDim.x in batches of kMaxItems, and prepares all of a
// batch (owner, sub-tile, K chunk, tokens, metadata) before the first one's
// loads.
constexpr int kMaxItems = 8;

template <typename E, bool kIds, int APT>
__global__ void __launch_bounds__(kShrinkThreads, 4) shrink_kernel(ShrinkArgs p) {
  constexpr int KSTEP = 4 * E::kVec;
  extern __shared__ __align__(16) char dyn[];
  f32x4_t* red = reinterpret_cast<f32x4_t*>(dyn);  // [8 waves][ng_max][64 lanes]
  int* info = reinterpret_cast<int*>(dyn + (size_t)p.ng_max * kShrinkWaves * 64 * 16);  // [n]
  uint16_t* id16 = reinterpret_cast<uint16_t*>(info + ((p.n + 3) & ~3));               // [T] (ids)
  __shared__ uint64_t s_wsum[kShrinkWaves];
  __shared__ uint64_t s_pref[kShrinkThreads + 1];
  // Per item k: adapter, first grouped position, tokens, stored rank, row
  // offset, scale bits, sub-tile index within the adapter, plan sub-tile, K chunk.
  __shared__ int s_it[kMaxItems][9];
  __shared__ int s_tok[kMaxItems][kSubTile];
  __shared__ int s_bc[kMaxItems][kShrinkWaves];
  __shared__ int s_owner[kMaxItems];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = p.n, T = p.T;

  // 1. Tokens per adapter into info[], and the ranks of this thread's
  //    adapters (needed in step 2).
  //    The APT loads are issued before any is used, from indices clamped
  //    into [0, n): a load under a branch, used at once, is waited for before
  //    the next one is issued (APT serial round trips).
  const int a0 = tid * APT;
  int rk_[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) rk_[i] = p.rank[min(a0 + i, n - 1)];  // n >= 1
#pragma unroll
  for (int i = 0; i < APT; ++i) rk_[i] = a0 + i < n ? rk_[i] : 0;
  if (kIds) {
    // ids: 4 per thread per 16-byte load, all loads issued before the
    // histogram consumes them (T <= 16384: at most 8 loads per thread).
    constexpr int kIdLoads = LORA_SEGMENT_MAX_T / (4 * kShrinkThreads);
    int4 iv[kIdLoads];
    const bool vec = ((uintptr_t)p.ids & 15u) == 0;  // same for every thread
#pragma unroll
    for (int q = 0; q < kIdLoads; ++q) {
      const int t = 4 * (q * kShrinkThreads + tid);
      if (vec && t + 3 < T) {
        iv[q] = *reinterpret_cast<const int4*>(p.ids + t);
      } else {
        iv[q].x = t < T ? p.ids[t] : -1;
        iv[q].y = t + 1 < T ? p.ids[t + 1] : -1;
        iv[q].z = t + 2 < T ? p.ids[t + 2] : -1;
        iv[q].w = t + 3 < T ? p.ids[t + 3] : -1;
      }
    }
    if (p.id_map) {  // uniform
      auto mapped = [&](int v) { return (unsigned)v < (unsigned)p.id_map_n ? p.id_map[v] : -1; };
#pragma unroll
      for (int q = 0; q < kIdLoads; ++q) {
        if (4 * q * kShrinkThreads < T) {
          iv[q].x = mapped(iv[q].x);
          iv[q].y = mapped(iv[q].y);
          iv[q].z = mapped(iv[q].z);
          iv[q].w = mapped(iv[q].w);
        }
      }
    }
    for (int i = tid; i < n; i += kShrinkThreads) info[i] = 0;
    __syncthreads();
    // Histogram: a wave instruction whose ids are all equal (a run of one
    // adapter's tokens, as in prefill segments) adds its count with one LDS
    // atomic instead of 64 conflicting ones; otherwise one atomic per lane.
#pragma unroll
    for (int q = 0; q < kIdLoads; ++q) {
      const int t = 4 * (q * kShrinkThreads + tid);
      if (4 * q * kShrinkThreads < T) {  // uniform over the workgroup
        const int v4[4] = {iv[q].x, iv[q].y, iv[q].z, iv[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = t + e < T && (unsigned)v4[e] < (unsigned)n;
          if (t + e < T) id16[t + e] = ok ? (uint16_t)v4[e] : (uint16_t)0xFFFFu;
          const uint64_t valid = __ballot(ok);
          const int leader = valid ? __ffsll((long long)valid) - 1 : 0;
          const int lv = __shfl(v4[e], leader);
          if (valid && __ballot(ok && v4[e] == lv) == valid) {
            if (lane == leader) atomicAdd(&info[lv], __popcll(valid));
          } else if (ok) {
            atomicAdd(&info[v4[e]], 1);
          }
        }
      }
    }
  } else if constexpr (APT <= 8) {
    // Tokens per adapter from the grouping: all the thread's seg_off loads
    // issued first, from indices clamped into the array's n + 2 entries (a
    // loop of dependent load/store pairs waits for each pair in turn).
    int s0[APT], s1[APT];
#pragma unroll
    for (int k = 0; k < APT; ++k) {
      const int i = min(tid + k * kShrinkThreads, n);
      s0[k] = p.seg_off[i];
      s1[k] = p.seg_off[i + 1];
    }
#pragma unroll
    for (int k = 0; k < APT; ++k)
      if (tid + k * kShrinkThreads < n) info[tid + k * kShrinkThreads] = s1[k] - s0[k];
  } else {
    for (int i = tid; i < n; i += kShrinkThreads) info[i] = p.seg_off[i + 1] - p.seg_off[i];
  }
  __syncthreads();
  // 2. Pack (tokens, row groups) per adapter; scan (tokens, sub-tiles, items).
  uint64_t mine = 0;
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int a = a0 + i;
    if (a < n) {
      int c = info[a];
      c = c < 0 ? 0 : (c > T ? T : c);
      const int ng = rk_[i] > 0 ? (rk_[i] + 15) / 16 : 0;
      const int sub = ng ? (c + kSubTile - 1) / kSubTile : 0;
      const int its = ng ? sub * by_ng(p.S, ng) : 0;
      info[a] = c | (ng << 20);
      mine += ((uint64_t)c << 44) | ((uint64_t)sub << 24) | (uint64_t)its;
    }
  }
  uint64_t tot;
  const uint64_t pre = block_exclusive_scan<kShrinkWaves>(mine, s_wsum, &tot);
  s_pref[tid] = pre;
  if (tid == 0) s_pref[kShrinkThreads] = tot;
  const int total_sub = min((int)((tot >> 24) & 0xfffffu), p.max_sub);
  if (blockIdx.x == 0 && tid == 0) *reinterpret_cast<int32_t*>(p.plan) = total_sub;
  const int base_pos = kIds ? 0 : p.seg_off[0];
  const int items = (int)(tot & 0xffffffu);
  // This workgroup's items: first + k G, k < n_mine (G workgroups, at most
  // two per CU, so all are resident); taken in batches of kMaxItems, steps
  // 3 to 5 once per batch on the grouping state of steps 1 and 2.
  const int first = blockIdx.x, G = (int)gridDim.x;
  const int n_mine = first < items ? (items - first + G - 1) / G : 0;
  const int i0 = (int)(pre & 0xffffffu), ni = (int)(mine & 0xffffffu);
  for (int kb = 0; kb < n_mine; kb += kMaxItems) {  // uniform over the workgroup
    const int nk = min(kMaxItems, n_mine - kb);
    // The thread whose item range holds item k of the batch records itself
    // as its owner.
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) {
      const int it = first + (kb + k) * G;
      if (k < nk && it >= i0 && it < i0 + ni) s_owner[k] = tid;
    }
    __syncthreads();

    // 3. Owner, sub-tile and K chunk of each item: lane k of wave 0 takes item
    //    k (the thread that owns it, recorded above, then a walk over that
    //    thread's adapters, whose info entries are read together first).  Its
    //    metadata loads are issued here and written to LDS only after step 4.
    int m_rank = 0, m_ro = 0;
    float m_sc = 0.f;
    if (w == 0 && lane < nk) {
      const int it = first + (kb + lane) * G;
      const int lo = s_owner[lane];
      const uint64_t b = s_pref[lo];
      int iv_[APT];
#pragma unroll
      for (int i = 0; i < APT; ++i) iv_[i] = lo * APT + i < n ? info[lo * APT + i] : 0;
      int s_items = (int)(b & 0xffffffu), s_sub = (int)((b >> 24) & 0xfffffu);
      int pos = base_pos + (int)(b >> 44);
#pragma unroll
      for (int i = 0; i < APT; ++i) {
        const int a = lo * APT + i;
        const int v = iv_[i];
        const int c = v & 0xfffff, ng = v >> 20;
        const int sub = ng ? (c + kSubTile - 1) / kSubTile : 0;
        const int S = by_ng(p.S, ng);
        const int its = ng ? sub * S : 0;
        if (it < s_items + its) {
          const int j = (it - s_items) / S;
          int* q = s_it[lane];
          q[0] = a;
          q[1] = pos + j * kSubTile;
          q[2] = min(kSubTile, c - j * kSubTile);
          q[6] = j;
          q[7] = s_sub + j;
          q[8] = it - s_items - j * S;
          m_rank = p.rank[a];
          m_ro = p.row_off[a];
          m_sc = p.scale[a];
          break;
        }
        s_items += its;
        s_sub += sub;
        pos += c;
      }
    }
    __syncthreads();
    // 4. Each item's tokens: ranks [16 j, 16 j + 16) among the tokens of its
    //    adapter, in token order.  ids: wave w scans a contiguous range of
    //    64-token blocks twice - once to count each item's matches, then, after
    //    a scan of the (item, wave) counts, to place them with ballot ranks.
    if (kIds) {
      const int nb = (T + 63) >> 6;
      const int per = (nb + kShrinkWaves - 1) / kShrinkWaves;
      const int b0 = w * per, b1 = min(nb, b0 + per);
      int ad[kMaxItems], cnt[kMaxItems];
#pragma unroll
      for (int k = 0; k < kMaxItems; ++k) {
        ad[k] = k < nk ? s_it[k][0] : -2;
        cnt[k] = 0;
      }
      for (int b = b0; b < b1; ++b) {
        const int t = b * 64 + lane;
        const int id = t < T ? (int)id16[t] : -1;
#pragma unroll
        for (int k = 0; k < kMaxItems; ++k)
          if (k < nk) cnt[k] += __popcll(__ballot(id == ad[k]));
      }
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kMaxItems; ++k)
          if (k < nk) s_bc[k][w] = cnt[k];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kMaxItems; ++k) {  // tokens of item k before wave w's range
        int before = 0;
        if (k < nk)
          for (int ww = 0; ww < w; ++ww) before += s_bc[k][ww];
        cnt[k] = before - (k < nk ? s_it[k][6] : 0) * kSubTile;
      }
      for (int b = b0; b < b1; ++b) {
        const int t = b * 64 + lane;
        const int id = t < T ? (int)id16[t] : -1;
#pragma unroll
        for (int k = 0; k < kMaxItems; ++k) {
          if (k < nk) {
            const bool hit = id == ad[k];
            const uint64_t bal = __ballot(hit);
            const int rk = cnt[k] + __popcll(bal & lanemask_lt());
            if (hit && rk >= 0 && rk < kSubTile) s_tok[k][rk] = t;
            cnt[k] += __popcll(bal);
          }
        }
      }
    } else {
      for (int idx = tid; idx < nk * kSubTile; idx += kShrinkThreads) {
        const int k = idx / kSubTile, i = idx - k * kSubTile;
        if (i < s_it[k][2]) {
          const int q = s_it[k][1] + i;
          const int tk = (q >= 0 && q < T) ? p.perm[q] : -1;
          s_tok[k][i] = (unsigned)tk < (unsigned)T ? tk : -1;
        }
      }
    }
    if (w == 0 && lane < nk) {
      s_it[lane][3] = m_rank;
      s_it[lane][4] = m_ro;
      s_it[lane][5] = __float_as_int(m_sc);
    }
    __syncthreads();

    TileEntry* entries = reinterpret_cast<TileEntry*>(p.plan + kPlanHeaderBytes);
    for (int k = 0; k < nk; ++k) {
      const int a = __builtin_amdgcn_readfirstlane(s_it[k][0]);
      const int pos0 = __builtin_amdgcn_readfirstlane(s_it[k][1]);
      const int m = __builtin_amdgcn_readfirstlane(s_it[k][2]);
      const int r = __builtin_amdgcn_readfirstlane(s_it[k][3]);
      const int ro = __builtin_amdgcn_readfirstlane(s_it[k][4]);
      const float sc = __int_as_float(__builtin_amdgcn_readfirstlane(s_it[k][5]));
      const int st = __builtin_amdgcn_readfirstlane(s_it[k][7]);
      const int kc = __builtin_amdgcn_readfirstlane(s_it[k][8]);
      const int ng = (r + 15) >> 4;
      // 5. This wave's K steps of chunk kc.
      {
        const int tl = lane & 15;
        const int tk = tl < m ? s_tok[k][tl] : -1;
        const bool tval = tk >= 0;
        const char* xrow = p.x + (int64_t)(tval ? tk : 0) * p.ldx_bytes;
        const char* a_rows = p.a_pack + (size_t)ro * p.d_in * E::kBytes;
        const int spw = by_ng(p.spw, ng);
        const int k0 = kc * by_ng(p.kchunk, ng) + w * spw * KSTEP;
        const int kw = spw * KSTEP;
        f32x4_t* slot = red + w * p.ng_max * 64;
        switch (ng) {
          case 1: shrink_wave<E, 1, 8>(xrow, tval, a_rows, p.d_in, r, k0, kw, slot); break;
          case 2: shrink_wave<E, 2, 5>(xrow, tval, a_rows, p.d_in, r, k0, kw, slot); break;
          case 3: shrink_wave<E, 3, 4>(xrow, tval, a_rows, p.d_in, r, k0, kw, slot); break;
          default: shrink_wave<E, 4, 3>(xrow, tval, a_rows, p.d_in, r, k0, kw, slot); break;
        }
      }
      __syncthreads();
      // 6. Sum the waves' tiles in wave order; write partial kc.  Lane l of
      //    row group q holds token l % 16, ranks 16 q + 4 (l / 16) + 0..3.
      if (tid < ng * 64) {
        const int q = tid >> 6, l = tid & 63;
        f32x4_t s = red[q * 64 + l];
#pragma unroll
        for (int kk = 1; kk < kShrinkWaves; ++kk) s += red[(kk * p.ng_max + q) * 64 + l];
        const int tk = l & 15;
        const int j0 = q * 16 + 4 * (l >> 4);
        const int row = pos0 + tk;
        if (tk < m && row >= 0 && row < T) {
          float* dst = p.part + (int64_t)kc * p.pstride + (int64_t)row * p.ldp + j0;
          if (j0 + 3 < r) {
            *reinterpret_cast<f32x4_t*>(dst) = s;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j0 + e < r) dst[e] = s[e];
          }
        }
      }
      if (kc == 0 && tid < 32) {
        int v = 0;
        if (tid == 0) v = a;
        else if (tid == 1) v = pos0;
        else if (tid == 2) v = m;
        else if (tid == 3) v = r;
        else if (tid == 4) v = ro;
        else if (tid == 5) v = __float_as_int(sc);
        else if (tid == 6) v = by_ng(p.S, ng);
        else if (tid >= 8 && tid < 8 + kSubTile) v = tid - 8 < m ? s_tok[k][tid - 8] : -1;
        reinterpret_cast<int32_t*>(entries + st)[tid] = v;
      }
      __syncthreads();  // red is rewritten by the next item (and s_it, s_tok by the next batch)
    }
  }  // batches
}

// ------------------------------------------------------------- reduce
// h[pos, j] = partial 0 + partial 1 + ... (chunk order, as the expand sums
// them), for every sub-tile of the plan.
__global__ void __launch_bounds__(256)
reduce_partials_kernel(const char* __restrict__ plan, int max_sub, const float* __restrict__ part,
                       int64_t ldp, int64_t pstride, int T, int r_max, int S_max, float* __restrict__ h,
                       int64_t ldh) {
  const int st = blockIdx.x;
  const int count = min(*reinterpret_cast<const int32_t*>(plan), max_sub);
  if (st >= count) return;
  const TileEntry* e = reinterpret_cast<const TileEntry*>(plan + kPlanHeaderBytes) + st;
  const int m = e->m, r = e->r, pos0 = e->pos0, S = e->S;
  if (m <= 0 || m > kSubTile || r <= 0 || r > r_max || S <= 0 || S > S_max) return;
  for (int idx = threadIdx.x; idx < m * r; idx += 256) {
    const int i = idx / r, j = idx - i * r;
    const int row = pos0 + i;
    if (row < 0 || row >= T) continue;
    const float* src = part + (int64_t)row * ldp + j;
    float pk[kMaxChunks];  // S <= kMaxChunks: all loads issued together, summed in chunk order
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) pk[k] = k < S ? src[(int64_t)k * pstride] : 0.f;
    float s = pk[0];
#pragma unroll
    for (int k = 1; k < kMaxChunks; ++k)
      if (k < S) s += pk[k];
    h[(int64_t)row * ldh + j] = s;
  }
}

// --------------------------------------------------------------- plan
// The plan of a caller-supplied grouping, for the standalone expand: one
// workgroup scans the sub-tile counts, then writes the entries in parallel.
template <int APT>
__global__ void __launch_bounds__(1024)
plan_kernel(const int32_t* __restrict__ seg_off, const int32_t* __restrict__ perm, int T, int n,
            const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank,
            const float* __restrict__ scale, int max_sub, char* __restrict__ plan) {
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
    c = c > 0 ? c : 0;
    sub_[i] = (a < n && rank[a] > 0) ? (c + kSubTile - 1) / kSubTile : 0;
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
    *reinterpret_cast<int32_t*>(plan) = total;
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
    e.r = rank[a];
    e.row_off = row_off[a];
    e.scale = scale[a];
    e.S = 1;
    e.pad0 = 0;
#pragma unroll
    for (int i = 0; i < kSubTile; ++i) {
      const int q = pos0 + i;
      const int tk = (i < m && q >= 0 && q < T) ? perm[q] : -1;
      e.tok[i] = (unsigned)tk < (unsigned)T ? tk : -1;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) e.pad1[i] = 0;
    entries[st] = e;
  }
}

// --------------------------------------------------------------- host
static int ng_of(int r_max) { return r_max <= 16 ? 1 : (r_max + 15) / 16; }

size_t shrink_lds_bytes(int T, int n, int r_max, bool with_ids) {
  size_t b = (size_t)ng_of(r_max) * kShrinkWaves * 64 * 16 + (size_t)((n + 3) & ~3) * 4;
  if (with_ids) b += align_up((size_t)T * 2, 16);
  return b;
}

template <typename E, bool kIds, int APT>
static hipError_t launch_shrink_t(const ShrinkArgs& a, int grid, size_t lds, hipStream_t stream) {
  auto fn = shrink_kernel<E, kIds, APT>;
  static DynLdsLimit lim;
  hipError_t e = ensure_dynamic_lds(lim, reinterpret_cast<const void*>(fn), lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kShrinkThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_shrink(const lora_store& s, const int32_t* ids, const int32_t* seg_off, const int32_t* perm,
                         int T, const void* x, int64_t ldx, void* ws, hipStream_t stream, const int32_t* id_map,
                         int id_map_n) {
  const ShrinkSplit sp = shrink_split(s.d_in, s.r_max, s.dtype);
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  char* base = reinterpret_cast<char*>(ws);
  ShrinkArgs a;
  a.ids = ids;
  a.seg_off = seg_off;
  a.perm = perm;
  a.T = T;
  a.n = s.n;
  a.max_sub = (int)max_sub;
  a.x = reinterpret_cast<const char*>(x);
  a.ldx_bytes = ldx * elem_bytes(s.dtype);
  a.a_pack = reinterpret_cast<const char*>(s.A_pack);
  a.row_off = s.row_off;
  a.rank = s.rank;
  a.scale = s.scale;
  a.d_in = s.d_in;
  a.ng_max = ng_of(s.r_max);
  for (int g = 0; g < 5; ++g) {
    a.spw[g] = sp.spw[g];
    a.S[g] = sp.S[g];
    a.kchunk[g] = sp.kchunk[g];
  }
  a.part = reinterpret_cast<float*>(base + L.part);
  a.ldp = partial_ld(s.r_max);
  a.pstride = (int64_t)T * a.ldp;
  a.plan = base + L.plan;
  a.id_map = ids ? id_map : nullptr;
  a.id_map_n = id_map_n;
  const bool with_ids = ids != nullptr;
  const size_t lds = shrink_lds_bytes(T, s.n, s.r_max, with_ids);
  // Two workgroups per CU, all resident (no second round of workgroups),
  // each taking its items in batches of kMaxItems; fewer for fewer items.
  const int64_t items = max_sub * sp.S_max;
  const int64_t g = 2LL * cu_count();
  const int grid = (int)(g < items ? g : items);
  const bool bf = s.dtype == LORA_DTYPE_BF16;
  if (with_ids)
    return bf ? launch_shrink_t<BF16, true, 8>(a, grid, lds, stream)
              : launch_shrink_t<F32, true, 8>(a, grid, lds, stream);
  if (s.n <= kGroupMaxN)
    return bf ? launch_shrink_t<BF16, false, 8>(a, grid, lds, stream)
              : launch_shrink_t<F32, false, 8>(a, grid, lds, stream);
  return bf ? launch_shrink_t<BF16, false, 32>(a, grid, lds, stream)
            : launch_shrink_t<F32, false, 32>(a, grid, lds, stream);
}

hipError_t launch_reduce_partials(const lora_store& s, int T, const void* ws, float* h, int64_t ldh,
                                  hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  const char* base = reinterpret_cast<const char*>(ws);
  const int64_t ldp = partial_ld(s.r_max);
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)max_sub), dim3(256), 0, stream, base + L.plan,
                     (int)max_sub, reinterpret_cast<const float*>(base + L.part), ldp, (int64_t)T * ldp, T,
                     s.r_max, shrink_split(s.d_in, s.r_max, s.dtype).S_max, h, ldh);
  return hipGetLastError();
}

hipError_t launch_plan(const lora_store& s, const int32_t* seg_off, const int32_t* perm, int T, void* ws,
                       hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  char* plan = reinterpret_cast<char*>(ws) + L.plan;
  const size_t lds = (size_t)(s.n + 1) * 4;
  if (s.n <= kGroupMaxN) {
    hipLaunchKernelGGL(plan_kernel<4>, dim3(1), dim3(1024), lds, stream, seg_off, perm, T, s.n, s.row_off,
                       s.rank, s.scale, (int)max_sub, plan);
  } else {
    static DynLdsLimit lim;
    hipError_t e = ensure_dynamic_lds(lim, reinterpret_cast<const void*>(plan_kernel<16>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_kernel<16>, dim3(1), dim3(1024), lds, stream, seg_off, perm, T, s.n, s.row_off,
                       s.rank, s.scale, (int)max_sub, plan);
  }
  return hipGetLastError();
}

}  // namespace lora
