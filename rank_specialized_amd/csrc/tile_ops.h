// Wave-level building blocks of the shrink and expand kernels (gfx950,
// wave64, 16x16 MFMA tiles).
#pragma once
#include "device_common.h"

namespace lora {

// ------------------------------------------------------------ shrink wave
// One wave's work item of the shrink on the matrix cores: K range
// [k0, k0 + kc) of
//   H^T[r_a x m] = A_a[r_a x d_in] . X^T[d_in x m]     (m <= 16)
// on 16x16 MFMA tiles, NG row groups of 16 ranks.  On return lane l holds, in
// acc[q], token l % 16 and ranks 16 q + 4 (l / 16) + 0..3.  Step s covers K
// indices [k0 + s * KSTEP, +KSTEP); lane group g (lanes 16g..16g+15) takes
// the g-th 16 bytes of it, so the four lane groups of a row read 64
// contiguous bytes per instruction.  Both operands of every MFMA carry the
// same K indices (any K order that is identical for the two operands gives
// the same sum up to rounding order).  Rows j >= r_a read as zero from the
// adapter's buffer resource and tokens >= m are not loaded.  U steps of
// loads are issued before the first MFMA that consumes them.
template <typename E, int NG, int U>
__device__ __forceinline__ void shrink_mfma(const char* __restrict__ xrow, bool tval,
                                            const char* __restrict__ a_rows, int d_in, int r, int k0, int kc,
                                            f32x4_t (&acc)[NG]) {
  constexpr int V = E::kVec;
  constexpr int KSTEP = 4 * V;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  const int steps = (kc + KSTEP - 1) / KSTEP;
  const int kl = k0 + g * V;
  const uint32_t a_row_bytes = (uint32_t)d_in * E::kBytes;
  // The adapter's retained rows as one buffer: rows j >= r read as zero.
  const rsrc_t ar = make_rsrc(a_rows, (uint32_t)r * a_row_bytes);
  uint32_t aoff[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) aoff[q] = (uint32_t)(q * 16 + i) * a_row_bytes + (uint32_t)kl * E::kBytes;
#pragma unroll
  for (int q = 0; q < NG; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = make_uint4(0, 0, 0, 0);
  const int kend = k0 + kc;
  for (int s0 = 0; s0 < steps; s0 += U) {
    uint4 bx[U], ba[U][NG];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int s = s0 + uu;
      const int k = kl + s * KSTEP;
      const bool kv = s < steps && k < kend;
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
}

// ------------------------------------------------------------ expand helpers
// Zero the elements of a 16-byte chunk at index >= nvalid (0 <= nvalid).
template <typename E>
__device__ __forceinline__ uint4 keep_first(uint4 v, int nvalid);
template <>
__device__ __forceinline__ uint4 keep_first<BF16>(uint4 v, int nvalid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t m = 2 * p + 1 < nvalid ? 0xffffffffu : (2 * p < nvalid ? 0x0000ffffu : 0u);
    w[p] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 keep_first<F32>(uint4 v, int nvalid) {
  return make_uint4(nvalid > 0 ? v.x : 0u, nvalid > 1 ? v.y : 0u, nvalid > 2 ? v.z : 0u,
                    nvalid > 3 ? v.w : 0u);
}

// A-operand chunk of H for the expand MFMA: V float32 values h[j0 .. j0+V)
// of one token.  bf16: each value is split into the exact pair hi + lo of
// bf16 values (hi = nearest bf16 of h, lo = nearest bf16 of h - hi), so the
// matrix core sees about 16 significant bits of h instead of 8.  f32: the
// values as they are.
template <typename E>
struct HChunk;
template <>
struct HChunk<BF16> {
  uint4 hi, lo;
  __device__ __forceinline__ void set(const float* f) {
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t ah = f32_to_bf16(f[2 * p]), bh = f32_to_bf16(f[2 * p + 1]);
      const float ar = f[2 * p] - __uint_as_float(ah << 16);
      const float br = f[2 * p + 1] - __uint_as_float(bh << 16);
      wh[p] = ah | (bh << 16);
      wl[p] = f32_to_bf16(ar) | (f32_to_bf16(br) << 16);
    }
    hi = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    lo = make_uint4(wl[0], wl[1], wl[2], wl[3]);
  }
  __device__ __forceinline__ f32x4_t mma(const uint4& b, f32x4_t c) const {
    c = mfma_bf16_16x16x32(hi, b, c);
    return mfma_bf16_16x16x32(lo, b, c);
  }
};
template <>
struct HChunk<F32> {
  uint4 v;
  __device__ __forceinline__ void set(const float* f) {
    v = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                   __float_as_uint(f[3]));
  }
  __device__ __forceinline__ f32x4_t mma(const uint4& b, f32x4_t c) const { return mfma_chunk<F32>(v, b, c); }
};

}  // namespace lora
