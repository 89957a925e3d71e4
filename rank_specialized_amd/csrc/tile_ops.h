// Wave-level building blocks shared by the shrink, expand and fused apply
// kernels (gfx950, wave64).
#pragma once
#include "device_common.h"

namespace lora {

// ------------------------------------------------------------ shrink wave
// One wave's share of a sub-tile's shrink: K range [k0, k0 + kc) of
//   H^T[r_a x m] = A_a[r_a x d_in] . X^T[d_in x m]     (m <= 16)
// on 16x16 MFMA tiles.  The wave's float32 partial tile (NG row groups) goes
// to red_slot[q * 64 + lane].  Step s covers K indices [k0 + s * KSTEP,
// +KSTEP); lane group g (lanes 16g..16g+15) takes the g-th 16 bytes of it, so
// the four lane groups of a row read 64 contiguous bytes per instruction and
// two consecutive steps consume whole 128-byte lines.  Both operands of every
// MFMA carry the same K indices (the contraction is a plain sum over K, so
// any K order that is identical for the two operands is exact).  Rows
// j >= r_a read as zero from the adapter's buffer resource and tokens >= m
// are not loaded.
template <typename E, int NG>
__device__ __forceinline__ void shrink_wave(const char* __restrict__ xrow, bool tval,
                                            const char* __restrict__ a_rows, int d_in, int r, int k0,
                                            int kc, f32x4_t* red_slot) {
  constexpr int V = E::kVec;
  constexpr int KSTEP = 4 * V;
  constexpr int U = NG <= 2 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int steps = kc / KSTEP;
  const int kl = k0 + g * V;  // step s covers [k0 + s * KSTEP, +KSTEP): lane group g its g-th 16 bytes
  const uint32_t a_row_bytes = (uint32_t)d_in * E::kBytes;
  // The adapter's retained rows as one buffer: rows j >= r read as zero.
  const rsrc_t ar = make_rsrc(a_rows, (uint32_t)r * a_row_bytes);
  uint32_t aoff[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) aoff[q] = (uint32_t)(q * 16 + i) * a_row_bytes + (uint32_t)kl * E::kBytes;
  f32x4_t acc[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int s0 = 0; s0 < steps; s0 += U) {
    uint4 bx[U], ba[U][NG];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int s = s0 + uu;
      const int k = kl + s * KSTEP;
      const bool kv = s < steps && k < d_in;
      bx[uu] = (tval && kv) ? ld16(xrow + (size_t)k * E::kBytes) : zero;
      const uint32_t so = (uint32_t)(s * KSTEP * E::kBytes);
#pragma unroll
      for (int q = 0; q < NG; ++q) ba[uu][q] = buf_ld16(ar, kv ? aoff[q] + so : kOutOfRange, 0);
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu)
#pragma unroll
      for (int q = 0; q < NG; ++q) acc[q] = mfma_chunk<E>(ba[uu][q], bx[uu], acc[q]);
  }
#pragma unroll
  for (int q = 0; q < NG; ++q) red_slot[q * 64 + lane] = acc[q];
}

// ------------------------------------------------------------ vector path
template <typename E, int RB>
__device__ __forceinline__ void expand_small(const char* __restrict__ bt_rows, int d_out, int r, float s,
                                             const float* __restrict__ hrows, int64_t ldh,
                                             const int32_t* __restrict__ perm, int p0, int m,
                                             char* __restrict__ y, int64_t ldy_bytes, int o) {
  constexpr int V = E::kVec;
  constexpr int MT = kSmallTile;
  constexpr int JN = RB < 8 ? RB : 8;
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

}  // namespace lora
