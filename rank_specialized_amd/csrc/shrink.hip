// Shrink: h[i, j] = sum_k A_a[j, k] x[perm[i], k]   (j < r_a), float32.
//
// Step 1 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4: A applied with scale
// 1 into a float32 buffer of shape [tokens, R].  Tokens come in groups of
// one adapter (the segmented gather of its section 2), cut into sub-tiles of
// at most 16 tokens by the plan, so each adapter's retained rows are read
// once per sub-tile.
//
// Work item = (sub-tile, K chunk of 2048 bf16 / 1024 float32 values, or a
// multiple for very wide inputs), one workgroup of 8 waves each (two fit on
// a CU), or of 4 waves in calls of one chunk per sub-tile (four fit on a
// CU).  No grouping work happens here:
// the plan was formed before, once per grouping.  The workgroup reads its
// sub-tile's entry, then the adapter's rank and row offset; each wave
// streams its share of the chunk of the x rows and A rows in batches of
// loads, the waves' float32 sums meet in
// LDS in wave order, and chunk kc's partial sums are written; the consumer
// adds the S partials in chunk order.  No atomics: results are
// deterministic.
//
// Two paths, by the sub-tile's shape:
//  * decode sub-tiles (m <= 4 tokens, rank <= 8 bf16 / 4 f32, r m <= 16):
//    a wavefront reduction.  Lane l takes 8 contiguous bytes of each of the
//    m x rows and r A rows per 64-lane block of K, so every load is fully
//    used; the r x m dot products are summed in float32 per lane and reduced
//    across the wave (a reduce-scatter butterfly).  Instantiated per exact
//    rank and token count.
//  * larger sub-tiles: H^T[r x m] on 16x16 MFMA tiles (bf16 16x16x32, f32
//    16x16x4), one template per 16-rank row group count.
// Item (st, 0) also records the sub-tile's metadata (rank, row offset,
// scale, S) for the expand.
#include "device_common.h"
#include "host_util.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {

struct ShrinkArgs {
  const char* plan;  // the grouping's plan (entries of sub-tiles)
  int max_sub;       // entries the plan buffer holds
  int T, n, R, r_max;
  const char* x;
  int64_t ldx_bytes;
  const char* a_pack;
  const int32_t* row_off;
  const int32_t* rank;
  const float* scale;
  int d_in, kchunk, span, S;
  float* part;
  int64_t ldp, pstride;  // floats: row stride, distance between partials
  TileMeta* meta;
};

// Multi-slice apply: each slice's rank, row offset and scale arrays and hoff
// ([n_sl][n]); the records go to sl_meta[j * max_sub + st].  A separate
// argument of the slice kernel only, so that the ordinary shrink's
// arguments stay small.
struct SliceSet {
  int n_sl;
  const int32_t* rank[LORA_MAX_SLICES];
  const int32_t* row_off[LORA_MAX_SLICES];
  const float* scale[LORA_MAX_SLICES];
  const int32_t* hoff;
  SliceMeta* meta;
};

// The plan's entry st checked against T and the store: every token, row
// and partial it names lies inside the call's buffers.
__device__ __forceinline__ bool entry_ok(int a, int m, int pos0, int n, int T) {
  return (unsigned)a < (unsigned)n && m > 0 && m <= kSubTile && pos0 >= 0 && pos0 <= T - m;
}

// 8 bytes of a row: 4 bf16 or 2 float32 values, widened.
template <typename E>
__device__ __forceinline__ void widen8(const uint2& v, float* f);
template <>
__device__ __forceinline__ void widen8<BF16>(const uint2& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
}
template <>
__device__ __forceinline__ void widen8<F32>(const uint2& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
}

// Wavefront-reduction path, one wave's span: R ranks (exact) x M tokens
// (exact), K range [k0, k0 + kw).  A block of K is 64 lanes x 8 bytes; a
// block's M + R loads are issued together.  On return the wave's R x M sums
// are in red[w][q] (q = t R + j).
template <typename E, int R, int M>
__device__ __forceinline__ void shrink_gemv(const ShrinkArgs& p, int tok_l, int tok_base, int ro, int k0, int kw,
                                            float* red_w) {
  constexpr int HV = 8 / E::kBytes;  // values per lane per block
  constexpr int BLK = 64 * HV;
  const int lane = threadIdx.x & 63;
  // Byte offsets of the token rows: token t of the sub-tile is held by lane
  // tok_base + t of tok_l (the tokens are uniform).
  int64_t xo[M];
#pragma unroll
  for (int t = 0; t < M; ++t) {
    const int tk = __builtin_amdgcn_readlane(tok_l, tok_base + t);
    xo[t] = (int64_t)((unsigned)tk < (unsigned)p.T ? tk : 0) * p.ldx_bytes;
  }
  const char* ar = p.a_pack + (size_t)ro * p.d_in * E::kBytes;
  const int kend = k0 + kw;
  float acc[R][M];
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int t = 0; t < M; ++t) acc[j][t] = 0.f;
  // Two blocks per turn, all their loads issued before either is used: a
  // wave's span is two blocks at most sizes, so the item takes one round
  // trip instead of two (the sums keep their block order).
#pragma nounroll
  for (int kb = k0; kb < kend; kb += 2 * BLK) {
    uint2 xv[2][M], av[2][R];
    bool kv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kb + u * BLK + lane * HV;
      kv[u] = k < kend;
      const size_t kk = (size_t)(kv[u] ? k : k0) * E::kBytes;  // in bounds; masked below
#pragma unroll
      for (int t = 0; t < M; ++t) xv[u][t] = *reinterpret_cast<const uint2*>(p.x + xo[t] + kk);
#pragma unroll
      for (int j = 0; j < R; ++j)
        av[u][j] = *reinterpret_cast<const uint2*>(ar + (size_t)j * p.d_in * E::kBytes + kk);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int t = 0; t < M; ++t)
        if (!kv[u]) xv[u][t] = make_uint2(0, 0);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        float af[HV];
        widen8<E>(av[u][j], af);
#pragma unroll
        for (int t = 0; t < M; ++t) {
          float xf[HV];
          widen8<E>(xv[u][t], xf);
#pragma unroll
          for (int e = 0; e < HV; ++e) acc[j][t] += af[e] * xf[e];
        }
      }
    }
  }
  // The R x M sums across the wave (value t R + j is (j, t)), padded to a
  // power of two; lane l ends with value l >> (6 - log2 Q).
  constexpr int RM = R * M;
  constexpr int Q = RM <= 1 ? 1 : RM <= 2 ? 2 : RM <= 4 ? 4 : RM <= 8 ? 8 : 16;
  constexpr int LOGQ = Q == 1 ? 0 : Q == 2 ? 1 : Q == 4 ? 2 : Q == 8 ? 3 : 4;
  static_assert(RM <= 16, "at most 16 sums per wave");
  float v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) v[q] = q < RM ? acc[q % R][q / R] : 0.f;
  const float sum = wave_reduce_scatter<Q>(v);
  const int q = lane >> (6 - LOGQ);
  if ((lane & ((64 >> LOGQ) - 1)) == 0 && q < RM) red_w[q] = sum;
}

// Token counts m with R m <= kGemvMaxProducts take the wavefront-reduction
// path (their sums and loads stay within the registers of 4 waves per SIMD):
// ranks up to r_cap with up to kGemvMaxTokens tokens, and a single token at
// any rank up to kGemvMaxProducts, which a 16 x 16 matrix tile would fill
// with one row of sixteen.
constexpr int kGemvMaxProducts = 16;
// Items whose entries and metadata a workgroup fetches together.
constexpr int kShrinkBatch = 4;
constexpr int kXcds = 8;    // XCDs of the MI355X, which receive workgroups in turn
constexpr int kXcdRun = 8;  // consecutive items of the plan dealt to one XCD
// (The multi-slice shrink keeps single tokens at r_cap: its slice records
// leave no registers for the wider instances.)
template <bool kWideSingle>
__device__ __forceinline__ bool gemv_fits(int r, int m, int r_cap) {
  if (kWideSingle && m == 1) return r <= kGemvMaxProducts;
  return r <= r_cap && m <= kGemvMaxTokens && r * m <= kGemvMaxProducts;
}

template <typename E, int R>
__device__ __forceinline__ void shrink_gemv_m(const ShrinkArgs& p, int tok_l, int tok_base, int m, int ro, int k0,
                                              int kw, float* red_w) {
  switch (m) {
    case 1: shrink_gemv<E, R, 1>(p, tok_l, tok_base, ro, k0, kw, red_w); break;
    case 2:
      if constexpr (2 * R <= kGemvMaxProducts) shrink_gemv<E, R, 2>(p, tok_l, tok_base, ro, k0, kw, red_w);
      break;
    case 3:
      if constexpr (3 * R <= kGemvMaxProducts) shrink_gemv<E, R, 3>(p, tok_l, tok_base, ro, k0, kw, red_w);
      break;
    default:
      if constexpr (4 * R <= kGemvMaxProducts) shrink_gemv<E, R, 4>(p, tok_l, tok_base, ro, k0, kw, red_w);
      break;
  }
}

// Matrix-core path, one wave's span: NG row groups of 16 ranks; its tile
// goes to red[w][q][lane].
template <typename E, int NG>
__device__ __forceinline__ void shrink_tile(const ShrinkArgs& p, int tok_l, int tok_base, int m, int r, int ro,
                                            int k0, int kw, f32x4_t (*red_w)[64]) {
  constexpr int U = NG == 1 ? 8 : NG == 2 ? 5 : NG == 3 ? 4 : 3;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int tkc = __shfl(tok_l, tok_base + c);  // token c of the sub-tile
  const int tk = c < m ? tkc : -1;
  const bool tval = (unsigned)tk < (unsigned)p.T;
  const char* xrow = p.x + (int64_t)(tval ? tk : 0) * p.ldx_bytes;
  const char* a_rows = p.a_pack + (size_t)ro * p.d_in * E::kBytes;
  f32x4_t acc[NG];
  shrink_mfma<E, NG, U>(xrow, tval, a_rows, p.d_in, r, k0, kw, acc);
#pragma unroll
  for (int q = 0; q < NG; ++q) red_w[q][lane] = acc[q];
}

template <typename E, bool kSl, int W>
__device__ __forceinline__ void shrink_body(const ShrinkArgs& p, const SliceSet& ss) {
  constexpr int kVecRank = kVecMaxRank * 2 / E::kBytes;  // 8 bf16, 4 float32
  __shared__ f32x4_t red[W][4][64];             // matrix path: [wave][row group][lane]
  __shared__ float redg[W][kGemvMaxProducts];   // reduction path: [wave][sum]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n_sub = min(*reinterpret_cast<const int32_t*>(p.plan), p.max_sub);
  const int items = n_sub * p.S;
  const int G = gridDim.x;
  const TileEntry* entries = reinterpret_cast<const TileEntry*>(p.plan + kPlanHeaderBytes);
  // The workgroup's items blockIdx.x + i G, taken kShrinkBatch at a time.
  // Lanes 16 k .. 16 k + 15 of every wave fetch item k's entry, its 16
  // tokens and its adapter's metadata together (two round trips for the
  // batch), so that the items then run back to back on their data loads.
  // Workgroups are dealt to the 8 XCDs in turn (workgroup b to XCD b mod 8).
  // When the grid holds every item, the items go to the XCDs in runs of
  // kXcdRun consecutive items of the plan (run k to XCD k mod 8): an
  // adapter's neighbouring sub-tiles then share one L2, so its A rows are
  // fetched into one or two XCDs instead of each, while the runs of a
  // heavy adapter still spread over the XCDs.
  constexpr int kSpan = kXcds * kXcdRun;
  const bool remap = G % kSpan == 0 && G >= items;
  int first = (int)blockIdx.x;
  if (remap) {
    const int x = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);  // the XCD's j-th workgroup
    first = ((j / kXcdRun) * kXcds + x) * kXcdRun + j % kXcdRun;
  }
  for (int b0 = first; b0 < items; b0 += kShrinkBatch * G) {  // uniform over the workgroup
    const int kl = lane >> 4;
    const int itl = b0 + kl * G;
    const bool vl = kl < kShrinkBatch && itl < items;
    const TileEntry* el = entries + (vl ? itl / p.S : 0);
    const int a_l = vl ? el->a : -1, pos0_l = el->pos0, m_l = el->m;
    const int tok_l = el->tok[lane & 15];
    int r_l = 0, ro_l = 0;
    float sc_l = 0.f;
    // Multi-slice: lane 16 k + j also fetches slice j's record for item k's
    // adapter (read with the metadata; written at the item's end).
    const int jl = lane & 15;
    SliceMeta sm_l{0, 0, 0.f, 0};
    if (vl && entry_ok(a_l, m_l, pos0_l, p.n, p.T)) {
      r_l = p.rank[a_l];
      ro_l = p.row_off[a_l];
      sc_l = p.scale[a_l];
      if (r_l < 0 || r_l > p.r_max || ro_l < 0 || ro_l > p.R - r_l) r_l = 0;  // not this store's metadata
      if (kSl && jl < ss.n_sl) {
        const int32_t* rk = ss.rank[0];
        const int32_t* ok = ss.row_off[0];
        const float* sk = ss.scale[0];
#pragma unroll
        for (int j = 1; j < LORA_MAX_SLICES; ++j)
          if (jl == j) {
            rk = ss.rank[j];
            ok = ss.row_off[j];
            sk = ss.scale[j];
          }
        sm_l.r = rk[a_l];
        sm_l.row_off = ok[a_l];
        sm_l.scale = sk[a_l];
        sm_l.hoff = ss.hoff[(int64_t)jl * p.n + a_l];
      }
    }
    for (int k = 0; k < kShrinkBatch; ++k) {
      const int it = b0 + k * G;
      if (it >= items) break;
      const int st = it / p.S, kc = it - st * p.S;
      const int pos0 = __builtin_amdgcn_readlane(pos0_l, 16 * k);
      const int m = __builtin_amdgcn_readlane(m_l, 16 * k);
      const int r = __builtin_amdgcn_readlane(r_l, 16 * k);
      const int ro = __builtin_amdgcn_readlane(ro_l, 16 * k);
      const float sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc_l), 16 * k));
      const int ng = r <= 16 ? 1 : (r + 15) >> 4;  // 16-rank row groups
      if (kc == 0 && tid == 0) {
        TileMeta tm;
        tm.r = r;
        tm.row_off = ro;
        tm.scale = sc;
        tm.S = p.S;
        p.meta[st] = tm;
      }
      if (kSl && kc == 0 && tid >= 16 * k && tid < 16 * k + ss.n_sl)  // lanes of wave 0 hold item k's records
        ss.meta[(int64_t)(tid - 16 * k) * p.max_sub + st] = sm_l;
      if (r == 0) continue;  // the same in every wave: no barrier is skipped by some only
      const int k0 = kc * p.kchunk + w * p.span;
      const int kw = max(0, min(p.span, p.d_in - k0));
      const bool gemv = gemv_fits<!kSl>(r, m, kVecRank);
      if (gemv) {
        switch (r) {
#define LORA_GEMV_CASE(RR) \
    case RR: shrink_gemv_m<E, RR>(p, tok_l, 16 * k, m, ro, k0, kw, redg[w]); break;
          LORA_GEMV_CASE(1) LORA_GEMV_CASE(2) LORA_GEMV_CASE(3) LORA_GEMV_CASE(4)
          LORA_GEMV_CASE(5) LORA_GEMV_CASE(6) LORA_GEMV_CASE(7) LORA_GEMV_CASE(8)
          default:
            if constexpr (!kSl) {
              switch (r) {
                LORA_GEMV_CASE(9) LORA_GEMV_CASE(10) LORA_GEMV_CASE(11) LORA_GEMV_CASE(12)
                LORA_GEMV_CASE(13) LORA_GEMV_CASE(14) LORA_GEMV_CASE(15) LORA_GEMV_CASE(16)
                default: break;
              }
            }
            break;
#undef LORA_GEMV_CASE
        }
      } else {
        switch ((r + 15) >> 4) {
          case 1: shrink_tile<E, 1>(p, tok_l, 16 * k, m, r, ro, k0, kw, red[w]); break;
          case 2: shrink_tile<E, 2>(p, tok_l, 16 * k, m, r, ro, k0, kw, red[w]); break;
          case 3: shrink_tile<E, 3>(p, tok_l, 16 * k, m, r, ro, k0, kw, red[w]); break;
          default: shrink_tile<E, 4>(p, tok_l, 16 * k, m, r, ro, k0, kw, red[w]); break;
        }
      }
      __syncthreads();
      // The waves' sums added in wave order; chunk kc's partial written.
      float* part = p.part + (int64_t)kc * p.pstride;
      if (gemv) {
        if (tid < r * m) {
          float s = redg[0][tid];
#pragma unroll
          for (int ww = 1; ww < W; ++ww) s += redg[ww][tid];
          const int t = tid / r, j = tid - t * r;
          part[(int64_t)(pos0 + t) * p.ldp + j] = s;
        }
      } else if (tid < ng * 64) {
        const int q = tid >> 6, l = tid & 63;
        f32x4_t s = red[0][q][l];
#pragma unroll
        for (int ww = 1; ww < W; ++ww) s += red[ww][q][l];
        // Lane l of row group q: token l % 16, ranks 16 q + 4 (l / 16) + 0..3.
        const int c = l & 15, j0 = q * 16 + 4 * (l >> 4);
        if (c < m) {
          float* dst = part + (int64_t)(pos0 + c) * p.ldp;
          if (j0 + 3 < r) {
            *reinterpret_cast<f32x4_t*>(dst + j0) = s;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j0 + e < r) dst[j0 + e] = s[e];
          }
        }
      }
      __syncthreads();  // red and redg are rewritten by the next item
    }  // items of the batch
  }  // batches
}

template <typename E, int W>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
shrink_kernel(ShrinkArgs p) {
  shrink_body<E, false, W>(p, SliceSet{});
}

struct ShrinkSliceArgs {
  ShrinkArgs p;
  SliceSet ss;
};

template <typename E, int W>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
shrink_slices_kernel(ShrinkSliceArgs a) {
  shrink_body<E, true, W>(a.p, a.ss);
}

// The kernel of one element type and wave count.
template <int W>
static void launch_shrink_kernel(const lora_store& s, const lora_multi_store* multi, const ShrinkSliceArgs& b, int grid,
                                 hipStream_t stream) {
  const dim3 block(W * 64);
  if (multi) {
    if (s.dtype == LORA_DTYPE_BF16) hipLaunchKernelGGL((shrink_slices_kernel<BF16, W>), dim3(grid), block, 0, stream, b);
    else hipLaunchKernelGGL((shrink_slices_kernel<F32, W>), dim3(grid), block, 0, stream, b);
  } else if (s.dtype == LORA_DTYPE_BF16) {
    hipLaunchKernelGGL((shrink_kernel<BF16, W>), dim3(grid), block, 0, stream, b.p);
  } else {
    hipLaunchKernelGGL((shrink_kernel<F32, W>), dim3(grid), block, 0, stream, b.p);
  }
}

// ------------------------------------------------------------- reduce
// h[pos, j] = partial 0 + partial 1 + ... (chunk order, as the expand sums
// them), for every sub-tile of the plan.
__global__ void __launch_bounds__(256)
reduce_partials_kernel(const char* __restrict__ plan, int max_sub, const TileMeta* __restrict__ meta,
                       const float* __restrict__ part, int64_t ldp, int64_t pstride, int T, int n, int r_max,
                       int S_store, float* __restrict__ h, int64_t ldh) {
  const int st = blockIdx.x;
  const int count = min(*reinterpret_cast<const int32_t*>(plan), max_sub);
  if (st >= count) return;
  const TileEntry* e = reinterpret_cast<const TileEntry*>(plan + kPlanHeaderBytes) + st;
  const int a = e->a, m = e->m, pos0 = e->pos0;
  const TileMeta tm = meta[st];
  const int r = tm.r, S = tm.S;
  if (!entry_ok(a, m, pos0, n, T) || r <= 0 || r > r_max || S <= 0 || S > S_store) return;
  for (int idx = threadIdx.x; idx < m * r; idx += 256) {
    const int i = idx / r, j = idx - i * r;
    const int row = pos0 + i;
    const float* src = part + (int64_t)row * ldp + j;
    const float s = sum_partials(src, pstride, S);
    h[(int64_t)row * ldh + j] = s;
  }
}

// --------------------------------------------------------------- host
static hipError_t shrink_impl(const lora_store& s, const lora_multi_store* multi, void* sl_meta, const char* plan,
                              int T, const void* x, int64_t ldx, void* ws, hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  const ShrinkSplit sp = shrink_split(s.d_in, s.dtype, T, s.n);
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  char* base = reinterpret_cast<char*>(ws);
  ShrinkArgs a;
  a.plan = plan;
  a.max_sub = (int)max_sub;
  a.T = T;
  a.n = s.n;
  a.R = s.R;
  a.r_max = s.r_max;
  a.x = reinterpret_cast<const char*>(x);
  a.ldx_bytes = ldx * elem_bytes(s.dtype);
  a.a_pack = reinterpret_cast<const char*>(s.A_pack);
  a.row_off = s.row_off;
  a.rank = s.rank;
  a.scale = s.scale;
  a.d_in = s.d_in;
  a.kchunk = sp.kchunk;
  a.span = sp.span;
  a.S = sp.S;
  a.part = reinterpret_cast<float*>(base + L.part);
  a.ldp = partial_ld(s.r_max);
  a.pstride = (int64_t)T * a.ldp;
  a.meta = reinterpret_cast<TileMeta*>(base + L.meta);
  // One workgroup per possible item: as workgroups finish, the dispatcher
  // starts the next on the freed CU, which balances items of unequal size
  // better than a fixed assignment to resident workgroups (measured: fleet
  // q 37.6 -> 33.7 us, down 117 -> 107 us).  Workgroups past the plan's
  // count exit at once; past 2^31 items the workgroups loop.
  const int64_t items = max_sub * sp.S;
  const int64_t cap = 1LL << 30;
  // A multiple of 8 XCDs x kXcdRun items, so that the kernel can deal the
  // items to the XCDs in runs.
  constexpr int kSpan = kXcds * kXcdRun;
  const int grid = (int)(((items < cap ? items : cap) + kSpan - 1) / kSpan * kSpan);
  ShrinkSliceArgs b{};
  b.p = a;
  if (multi) {
    b.ss.n_sl = multi->n_slices;
    for (int j = 0; j < LORA_MAX_SLICES; ++j) {
      const bool in = j < multi->n_slices;
      b.ss.rank[j] = in ? multi->slice[j].rank : nullptr;
      b.ss.row_off[j] = in ? multi->slice[j].row_off : nullptr;
      b.ss.scale[j] = in ? multi->slice[j].scale : nullptr;
    }
    b.ss.hoff = multi->hoff;
    b.ss.meta = reinterpret_cast<SliceMeta*>(sl_meta);
  }
  if (sp.waves == 4) launch_shrink_kernel<4>(s, multi, b, grid, stream);
  else launch_shrink_kernel<kShrinkWavesMax>(s, multi, b, grid, stream);
  return hipGetLastError();
}

hipError_t launch_shrink(const lora_store& s, const char* plan, int T, const void* x, int64_t ldx, void* ws,
                         hipStream_t stream) {
  return shrink_impl(s, nullptr, nullptr, plan, T, x, ldx, ws, stream);
}

hipError_t launch_shrink_slices(const lora_multi_store& m, void* sl_meta, const char* plan, int T, const void* x,
                                int64_t ldx, void* ws, hipStream_t stream) {
  return shrink_impl(m.stacked, &m, sl_meta, plan, T, x, ldx, ws, stream);
}

hipError_t launch_reduce_partials(const lora_store& s, const char* plan, int T, const void* ws, float* h,
                                  int64_t ldh, hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  const char* base = reinterpret_cast<const char*>(ws);
  const int64_t ldp = partial_ld(s.r_max);
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)max_sub), dim3(256), 0, stream, plan, (int)max_sub,
                     reinterpret_cast<const TileMeta*>(base + L.meta), reinterpret_cast<const float*>(base + L.part),
                     ldp, (int64_t)T * ldp, T, s.n, s.r_max, shrink_split(s.d_in, s.dtype, T, s.n).S, h, ldh);
  return hipGetLastError();
}

}  // namespace lora
