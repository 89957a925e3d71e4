// Expand: y[perm[i], o] += s_a * sum_{j < r_a} B_a[o, j] h[i, j].
//
// Step 3 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4: B applied with the
// adapter's scale and added into (a slice of) y.  Accumulation in float32,
// one rounding of the new y value to the output type.
//
// Work item = one wave: (tile, run of output features).  Waves are
// independent (no barriers) and walk the items with a grid stride.  Items
// are ordered run-major, so consecutive waves of a workgroup take the same
// run of consecutive tiles: tiles of one popular adapter share that run's
// Bt rows through the CU's cache.
//  * Tiles of more than kSmallTile tokens (prefill segments, popular decode
//    adapters) run on the matrix cores: for a run of 64 features,
//    Y^T[o, t] = Bt^T[o, j] . H^T[j, t] on bf16 16x16x32 MFMA.  h is float32
//    and is fed as the exact sum of two bf16 values (hi = nearest bf16 of h,
//    lo = nearest bf16 of h - hi), so the product keeps about 16 significant
//    bits of h instead of 8.  M rows are permuted so that each lane ends with
//    16 consecutive features of one token: y is read and written with
//    16-byte accesses.
//  * Small tiles (decode: a few tokens per adapter) run on the vector ALUs
//    over a run of 64 x 16 bytes of features: a lane owns 16 bytes of
//    outputs; the tile's y rows and a rank chunk of Bt rows (one coalesced
//    1 KiB run per row) are issued before any arithmetic; h values are
//    wave-uniform scalar loads.
// Every factor byte is read once per tile and every y row of the tile is
// read and written once.
//
// Rank specialization: the vector path is instantiated per rank bucket
// (RB = 4, 8, 16, 32, 64; loads and FMAs fully unrolled, rows j >= r_a never
// loaded); the matrix path per number of 32-deep K steps (1 or 2).
#include "device_common.h"
#include "kernels.h"

namespace lora {

constexpr int kExpandThreads = 256;
constexpr int kLargeRun = 64;  // output features per matrix-path item

// ------------------------------------------------------------ vector path
template <typename E, int RB>
__device__ __forceinline__ void expand_small(const char* __restrict__ bt_rows, int d_out, int r, float s,
                                             const float* __restrict__ hrows, int64_t ldh,
                                             const int32_t* __restrict__ perm, int p0, int m,
                                             char* __restrict__ y, int64_t ldy_bytes, int o) {
  constexpr int V = E::kVec;
  constexpr int MT = kSmallTile;
  constexpr int JN = RB < 16 ? RB : 16;
  const bool active = o < d_out;
  const uint32_t bt_row_bytes = (uint32_t)d_out * E::kBytes;
  // The adapter's Bt rows as one buffer; inactive lanes read zeros.
  const rsrc_t br = make_rsrc(bt_rows, (uint32_t)r * bt_row_bytes);
  const uint32_t boff = active ? (uint32_t)o * E::kBytes : kOutOfRange;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  uint4 yv[MT];
  char* yp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    yp[t] = (t < m) ? y + (int64_t)perm[p0 + t] * ldy_bytes + (size_t)o * E::kBytes : nullptr;
    yv[t] = (active && t < m) ? ld16(yp[t]) : zero;
  }
  float acc[MT][V];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int e = 0; e < V; ++e) acc[t][e] = 0.f;
#pragma unroll 1
  for (int j0 = 0; j0 < RB; j0 += JN) {
    if (j0 >= r) break;
    uint4 b[JN];
#pragma unroll
    for (int jj = 0; jj < JN; ++jj)
      b[jj] = (j0 + jj < r) ? buf_ld16(br, boff, (uint32_t)(j0 + jj) * bt_row_bytes) : zero;
#pragma unroll
    for (int jj = 0; jj < JN; ++jj) {
      if (j0 + jj < r) {
        float bf[V];
        E::widen(b[jj], bf);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < m) {
            const float hv = hrows[(int64_t)t * ldh + j0 + jj];
#pragma unroll
            for (int e = 0; e < V; ++e) acc[t][e] += hv * bf[e];
          }
        }
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t < m) {
      float yf[V];
      E::widen(yv[t], yf);
#pragma unroll
      for (int e = 0; e < V; ++e) yf[e] = yf[e] + s * acc[t][e];
      st16(yp[t], E::narrow(yf));
    }
  }
}

// ------------------------------------------------------------ matrix path
// A-operand fragment of Bt^T for one output feature: Bt[jbase + e][o],
// e = 0..7, from the adapter's Bt buffer (rows j >= r read as zero; voff =
// byte offset of (jbase, o); the row step rides in the uniform offset).
__device__ __forceinline__ uint4 bt_fragment(rsrc_t br, uint32_t voff, uint32_t row_bytes) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(br, voff, (2 * p) * row_bytes, 0);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(br, voff, (2 * p + 1) * row_bytes, 0);
    w[p] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// B-operand fragments of H^T from 8 consecutive float32 h values (columns
// jbase..jbase+7 of one token): columns >= r are zeroed (the shrink leaves
// them unwritten), then each value is split into the exact pair hi + lo of
// bf16 values.
__device__ __forceinline__ void h_fragment(const uint4& q0, const uint4& q1, int r, int jbase, uint4& hi,
                                           uint4& lo) {
  const uint32_t raw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  uint32_t wh[4], wl[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = jbase + 2 * p < r ? __uint_as_float(raw[2 * p]) : 0.f;
    const float b = jbase + 2 * p + 1 < r ? __uint_as_float(raw[2 * p + 1]) : 0.f;
    const uint32_t ah = f32_to_bf16(a), bh = f32_to_bf16(b);
    const float ar = a - __uint_as_float(ah << 16), br = b - __uint_as_float(bh << 16);
    wh[p] = ah | (bh << 16);
    wl[p] = f32_to_bf16(ar) | (f32_to_bf16(br) << 16);
  }
  hi = make_uint4(wh[0], wh[1], wh[2], wh[3]);
  lo = make_uint4(wl[0], wl[1], wl[2], wl[3]);
}

// One wave: 64 output features (4 M-tiles) of one tile, all of its tokens.
// M-tile mm, row i holds output o_w + 16 (i / 4) + 4 mm + (i % 4), so the
// accumulator rows 4 g + v of lane (i, g) are outputs o_w + 16 g + 4 mm + v:
// 16 consecutive features of token i per lane.  The loads of NB token groups
// (y and h) and the Bt fragments are issued before any MFMA, so a wave keeps
// up to ~10 KB in flight.
template <int KS>
__device__ __forceinline__ void expand_large(const uint16_t* __restrict__ bt, int d_out, int r, float s,
                                             const float* __restrict__ hrows, int64_t ldh,
                                             const int32_t* __restrict__ perm, int p0, int m,
                                             char* __restrict__ y, int64_t ldy_bytes, int o_w) {
  constexpr int NB = KS == 1 ? 4 : 2;  // token groups of 16 whose loads are in flight together
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const uint32_t row_bytes = (uint32_t)d_out * 2;
  const rsrc_t br = make_rsrc(bt, (uint32_t)r * row_bytes);
  // The tile's h rows as one buffer: tokens >= m read as zero.
  const uint32_t h_row_bytes = (uint32_t)ldh * 4;
  const rsrc_t hr = make_rsrc(hrows, (uint32_t)m * h_row_bytes);
  const int o_lane = o_w + 16 * g;
  const bool ov0 = o_lane < d_out, ov1 = o_lane + 8 < d_out;
  uint4 af[4][KS];
  for (int u0 = 0; u0 < m; u0 += 16 * NB) {
    // y rows and h of NB token groups.
    int prow[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int tok = u0 + u * 16 + i;
      prow[u] = tok < m ? perm[p0 + tok] : -1;
    }
    uint4 hq[NB][KS][2];
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t voff = (uint32_t)(u0 + u * 16 + i) * h_row_bytes + (uint32_t)(32 * ks + 8 * g) * 4;
        hq[u][ks][0] = buf_ld16(hr, voff, 0);
        hq[u][ks][1] = buf_ld16(hr, voff + 16, 0);
      }
    char* yrow[NB];
    uint4 y0[NB], y1[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool tv = prow[u] >= 0;
      yrow[u] = y + (int64_t)(tv ? prow[u] : 0) * ldy_bytes;
      y0[u] = (tv && ov0) ? ld16(yrow[u] + (size_t)o_lane * 2) : make_uint4(0, 0, 0, 0);
      y1[u] = (tv && ov1) ? ld16(yrow[u] + (size_t)(o_lane + 8) * 2) : make_uint4(0, 0, 0, 0);
    }
    if (u0 == 0) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int o = o_w + 16 * (i >> 2) + 4 * mm + (i & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t voff = o < d_out ? (uint32_t)(32 * ks + 8 * g) * row_bytes + (uint32_t)o * 2
                                          : kOutOfRange;
          af[mm][ks] = bt_fragment(br, voff, row_bytes);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (u0 + u * 16 >= m) break;
      const bool tv = prow[u] >= 0;
      f32x4_t acc[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) acc[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 bh, bl;
        h_fragment(hq[u][ks][0], hq[u][ks][1], r, 32 * ks + 8 * g, bh, bl);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          acc[mm] = mfma_bf16_16x16x32(af[mm][ks], bh, acc[mm]);
          acc[mm] = mfma_bf16_16x16x32(af[mm][ks], bl, acc[mm]);
        }
      }
      if (tv && ov0) {
        float f[8];
        BF16::widen(y0[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] + s * acc[e >> 2][e & 3];
        st16(yrow[u] + (size_t)o_lane * 2, BF16::narrow(f));
      }
      if (tv && ov1) {
        float f[8];
        BF16::widen(y1[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f[e] + s * acc[2 + (e >> 2)][e & 3];
        st16(yrow[u] + (size_t)(o_lane + 8) * 2, BF16::narrow(f));
      }
    }
  }
}

// ------------------------------------------------------------------ kernel
template <typename E>
__global__ void __launch_bounds__(kExpandThreads)
expand_kernel(const float* __restrict__ h, int64_t ldh, const char* __restrict__ bt_pack,
              const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank,
              const float* __restrict__ scale, int d_out, const int32_t* __restrict__ perm,
              const void* __restrict__ plan_ws, char* __restrict__ y, int64_t ldy_bytes) {
  constexpr int V = E::kVec;
  constexpr bool kMatrix = E::kBytes == 2;  // f32 stores always take the vector path
  const Plan pl = plan_view(plan_ws, 0);  // expand tiles only
  const int n_all = pl.count[0];
  const int n_large = kMatrix ? pl.count[1] : 0;
  const int n_small = n_all - n_large;
  const int GL = (d_out + kLargeRun - 1) / kLargeRun;
  const int GS = (d_out + 64 * V - 1) / (64 * V);
  const int64_t large_items = (int64_t)n_large * GL;
  const int64_t items = large_items + (int64_t)n_small * GS;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * (kExpandThreads / 64);
  for (int64_t item = (int64_t)blockIdx.x * (kExpandThreads / 64) + (threadIdx.x >> 6); item < items;
       item += stride) {
    const bool large = item < large_items;
    int t, run;
    if (large) {
      run = (int)(item / n_large);
      t = (int)(item - (int64_t)run * n_large);
    } else {
      const int64_t it = item - large_items;
      run = (int)(it / n_small);
      t = n_large + (int)(it - (int64_t)run * n_small);
    }
    const int4 tile = pl.tiles[t];
    const int a = tile.x, p0 = tile.y, m = tile.z;
    const int r = rank[a];
    if (r <= 0) continue;
    const float sc = scale[a];
    const char* bt_rows = bt_pack + (size_t)row_off[a] * d_out * E::kBytes;
    const float* hrows = h + (int64_t)p0 * ldh;
    if (large) {
      if constexpr (kMatrix) {
        const uint16_t* bt = reinterpret_cast<const uint16_t*>(bt_rows);
        const int o_w = run * kLargeRun;
        if (r <= 32) expand_large<1>(bt, d_out, r, sc, hrows, ldh, perm, p0, m, y, ldy_bytes, o_w);
        else expand_large<2>(bt, d_out, r, sc, hrows, ldh, perm, p0, m, y, ldy_bytes, o_w);
      }
    } else {
      const int o = (run * 64 + lane) * V;
      // f32 stores send every tile here: take the tokens kSmallTile at a time.
      for (int t0 = 0; t0 < m; t0 += kSmallTile) {
        const int mt = min(kSmallTile, m - t0);
        const float* hr = hrows + (int64_t)t0 * ldh;
        const int pt = p0 + t0;
        if (r <= 4) expand_small<E, 4>(bt_rows, d_out, r, sc, hr, ldh, perm, pt, mt, y, ldy_bytes, o);
        else if (r <= 8) expand_small<E, 8>(bt_rows, d_out, r, sc, hr, ldh, perm, pt, mt, y, ldy_bytes, o);
        else if (r <= 16) expand_small<E, 16>(bt_rows, d_out, r, sc, hr, ldh, perm, pt, mt, y, ldy_bytes, o);
        else if (r <= 32) expand_small<E, 32>(bt_rows, d_out, r, sc, hr, ldh, perm, pt, mt, y, ldy_bytes, o);
        else expand_small<E, 64>(bt_rows, d_out, r, sc, hr, ldh, perm, pt, mt, y, ldy_bytes, o);
      }
    }
  }
}

hipError_t launch_expand(const lora_store& s, const float* h, int64_t ldh, int T, const int32_t* perm,
                         const void* plan_ws, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t tiles = plan_max_tiles(T, s.n);
  if (tiles == 0) return hipSuccess;
  const int V = vec_elems(s.dtype);
  const int64_t GL = (s.d_out + kLargeRun - 1) / kLargeRun;
  const int64_t GS = (s.d_out + 64 * V - 1) / (64 * V);
  const int64_t waves = tiles * (GL > GS ? GL : GS);
  const int64_t bound = (waves + 3) / 4;
  const int64_t grid = bound < 4096 ? bound : 4096;
  const int eb = elem_bytes(s.dtype);
  if (s.dtype == LORA_DTYPE_BF16)
    hipLaunchKernelGGL(expand_kernel<BF16>, dim3((unsigned)grid), dim3(kExpandThreads), 0, stream, h, ldh,
                       reinterpret_cast<const char*>(s.Bt_pack), s.row_off, s.rank, s.scale, s.d_out, perm,
                       plan_ws, reinterpret_cast<char*>(y), ldy * eb);
  else
    hipLaunchKernelGGL(expand_kernel<F32>, dim3((unsigned)grid), dim3(kExpandThreads), 0, stream, h, ldh,
                       reinterpret_cast<const char*>(s.Bt_pack), s.row_off, s.rank, s.scale, s.d_out, perm,
                       plan_ws, reinterpret_cast<char*>(y), ldy * eb);
  return hipGetLastError();
}

}  // namespace lora
