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
//    adapters) run on the matrix cores: for a run of 128 features,
//    Y[t, o] = H[t, j] . Bt[j, o] on bf16 16x16x32 MFMA.  h is float32 and
//    is fed as the exact sum of two bf16 values (hi = nearest bf16 of h,
//    lo = nearest bf16 of h - hi), so the product keeps about 16 significant
//    bits of h instead of 8.  N columns are permuted so that each lane ends
//    with 16 consecutive bytes of features of 4 tokens: a y row is read and
//    written as 256 contiguous bytes by 16 lanes.
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
#include "tile_ops.h"

namespace lora {

constexpr int kExpandThreads = 256;
constexpr int kLargeRun = 128;  // output features per matrix-path item (one wave)

// ------------------------------------------------------------ matrix path
// A-operand fragment of H: 8 consecutive float32 h values (columns
// jbase..jbase+7 of one token); columns >= r are zeroed (the shrink leaves
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

// Per-wave LDS slice of Bt: rows j < 64 of 128 features (256 bytes) plus 16
// bytes of padding, so the four lane groups of a transposed read fall in
// different banks.
constexpr int kSliceStride = 272;
constexpr int kSliceBytes = 64 * kSliceStride;

// One wave: 128 output features of one tile, all of its tokens.
//   D[token, feature] = H[token, j] . Bt[j, feature]  on bf16 16x16x32 MFMA,
// eight N-tiles per 16-token M-tile.  N-tile nt, column n is feature
// o_w + 8 n + nt, so lane (n, g) accumulates features o_w + 8n .. o_w + 8n + 7
// (16 bytes) of tokens 4g .. 4g + 3 of the M-tile: a y row is read and written
// as 256 contiguous bytes by 16 lanes.
//   The Bt slice [r x 128] is staged in LDS with coalesced 16-byte loads and
// read back transposed (8 rank indices of one feature per lane).
template <int KS>
__device__ __forceinline__ void expand_large(const char* __restrict__ bt_rows, int d_out, int r, float s,
                                             const float* __restrict__ hrows, int64_t ldh,
                                             const int32_t* __restrict__ perm, int p0, int m,
                                             char* __restrict__ y, int64_t ldy_bytes, int o_w,
                                             char* __restrict__ slice) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const uint32_t row_bytes = (uint32_t)d_out * 2;
  const rsrc_t br = make_rsrc(bt_rows, (uint32_t)r * row_bytes);
  const int col = o_w + 8 * n;  // first feature of this lane's 16 bytes
  const bool cv = col < d_out;
  // Stage Bt rows 0 .. 32 KS - 1 (rows >= r and features >= d_out as zeros).
  {
    uint4 v[8 * KS];
#pragma unroll
    for (int q = 0; q < 8 * KS; ++q) {
      const int j = 4 * q + g;
      v[q] = buf_ld16(br, (j < r && cv) ? (uint32_t)j * row_bytes + (uint32_t)col * 2 : kOutOfRange, 0);
    }
#pragma unroll
    for (int q = 0; q < 8 * KS; ++q)
      *reinterpret_cast<uint4*>(slice + (4 * q + g) * kSliceStride + 16 * n) = v[q];
  }
  __builtin_amdgcn_wave_barrier();
  // B-operand fragments (rebuilt from LDS per M-tile and K step): lane
  // (n, g), N-tile nt holds Bt[32 ks + 8 g + e][col(n) + nt], e = 0..7.
  const uint16_t* sl = reinterpret_cast<const uint16_t*>(slice) + 8 * n;
  auto bfrag = [&](int ks, int nt) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int j = 32 * ks + 8 * g + 2 * p;
      const uint32_t lo = sl[(j * kSliceStride) / 2 + nt];
      const uint32_t hi = sl[((j + 1) * kSliceStride) / 2 + nt];
      w[p] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  // The tile's h rows as one buffer: tokens >= m read as zero.
  const uint32_t h_row_bytes = (uint32_t)ldh * 4;
  const rsrc_t hr = make_rsrc(hrows, (uint32_t)m * h_row_bytes);
  // The y rows this lane touches for NB token groups (tokens 16 u + 4 g + v)
  // are loaded before any matrix work: 16 bytes x 4 NB rows per lane in flight.
  constexpr int NB = KS == 1 ? 4 : 2;
  for (int u0 = 0; u0 < m; u0 += 16 * NB) {
    int prow[NB][4];
    uint4 yv[NB][4];
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = u0 + 16 * u + 4 * g + v;
        prow[u][v] = (tok < m && cv) ? perm[p0 + tok] : -1;
      }
#pragma unroll
    for (int u = 0; u < NB; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        yv[u][v] = prow[u][v] >= 0 ? ld16(y + (int64_t)prow[u][v] * ldy_bytes + (size_t)col * 2)
                                   : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int t0 = u0 + 16 * u;
      if (t0 >= m) break;
      uint4 hq[KS][2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t voff = (uint32_t)(t0 + n) * h_row_bytes + (uint32_t)(32 * ks + 8 * g) * 4;
        hq[ks][0] = buf_ld16(hr, voff, 0);
        hq[ks][1] = buf_ld16(hr, voff + 16, 0);
      }
      f32x4_t acc[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 ah, al;
        h_fragment(hq[ks][0], hq[ks][1], r, 32 * ks + 8 * g, ah, al);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const uint4 b = bfrag(ks, nt);
          acc[nt] = mfma_bf16_16x16x32(ah, b, acc[nt]);
          acc[nt] = mfma_bf16_16x16x32(al, b, acc[nt]);
        }
      }
      // acc[nt][v] = feature col + nt of token t0 + 4 g + v.
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (prow[u][v] >= 0) {
          float f[8];
          BF16::widen(yv[u][v], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = f[e] + s * acc[e][v];
          st16(y + (int64_t)prow[u][v] * ldy_bytes + (size_t)col * 2, BF16::narrow(f));
        }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();  // the slice is rewritten by this wave's next item
}

// ------------------------------------------------------------------ kernel
template <typename E>
__global__ void __launch_bounds__(kExpandThreads)
__attribute__((amdgpu_waves_per_eu(2, 8))) expand_kernel(const float* __restrict__ h, int64_t ldh, const char* __restrict__ bt_pack,
              const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank,
              const float* __restrict__ scale, int d_out, const int32_t* __restrict__ perm,
              const void* __restrict__ plan_ws, char* __restrict__ y, int64_t ldy_bytes) {
  constexpr int V = E::kVec;
  constexpr bool kMatrix = E::kBytes == 2;  // f32 stores always take the vector path
  __shared__ __attribute__((aligned(16))) char slices[kMatrix ? 4 * kSliceBytes : 16];
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
    const bool large = kMatrix && item < large_items;
    int t = 0, run = 0;
    if constexpr (kMatrix) {
      if (large) {
        run = (int)(item / n_large);
        t = (int)(item - (int64_t)run * n_large);
      }
    }
    if (!large) {
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
        const int o_w = run * kLargeRun;
        char* slice = slices + (threadIdx.x >> 6) * kSliceBytes;
        if (r <= 32) expand_large<1>(bt_rows, d_out, r, sc, hrows, ldh, perm, p0, m, y, ldy_bytes, o_w, slice);
        else expand_large<2>(bt_rows, d_out, r, sc, hrows, ldh, perm, p0, m, y, ldy_bytes, o_w, slice);
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
