// Device-side helpers shared by the kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace lora {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
// bfloat16 is the top half of a binary32 word: widening is a 16-bit shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// binary32 -> bfloat16 bits, round to nearest, ties to even: add 0x7fff plus
// the lowest kept bit, then drop the low 16 bits.  NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ------------------------------------------------------------ element types
// Each lane moves 16 bytes at a time: 8 bf16 or 4 f32 values.
struct BF16 {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  typedef uint16_t storage;
  __device__ static __forceinline__ void widen(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ uint4 narrow(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
};
struct F32 {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
  typedef float storage;
  __device__ static __forceinline__ void widen(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 narrow(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
// Streaming (nontemporal) forms, for data touched exactly once (the y rows of
// the expand, the x rows of the shrink): they do not displace the factor rows
// and partial sums that other waves read again from L2.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16_stream(void* p, const uint4& v) {
  u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// ----------------------------------------------------------- buffer loads
// A buffer resource (base address and size in bytes) lets a load carry a
// 32-bit offset instead of a 64-bit address, and an offset at or beyond the
// size reads as zero.  Used for the per-adapter factor blocks (a few MB at
// most), where rows past the retained rank then need no predicate.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset that always reads as zero

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_ld4(rsrc_t r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ uint32_t buf_ld2(rsrc_t r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

// ------------------------------------------------------------------- MFMA
// 16x16 output tile, float32 accumulate.  Operand convention (both
// operands): lane l supplies row/column (l % 16) of its matrix and the
// K-slice owned by lane group (l / 16).  Output: lane l holds column l % 16,
// rows 4 * (l / 16) + 0..3.
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32_16x16x4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One 16-byte K-chunk of both operands: 1 bf16 MFMA (K = 32 over the wave)
// or 4 f32 MFMAs (K = 4 each).
template <typename E>
__device__ __forceinline__ f32x4_t mfma_chunk(const uint4& a, const uint4& b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma_chunk<BF16>(const uint4& a, const uint4& b, f32x4_t c) {
  return mfma_bf16_16x16x32(a, b, c);
}
template <>
__device__ __forceinline__ f32x4_t mfma_chunk<F32>(const uint4& a, const uint4& b, f32x4_t c) {
  c = mfma_f32_16x16x4(__uint_as_float(a.x), __uint_as_float(b.x), c);
  c = mfma_f32_16x16x4(__uint_as_float(a.y), __uint_as_float(b.y), c);
  c = mfma_f32_16x16x4(__uint_as_float(a.z), __uint_as_float(b.z), c);
  c = mfma_f32_16x16x4(__uint_as_float(a.w), __uint_as_float(b.w), c);
  return c;
}

// ------------------------------------------------------------ partial sums
// src[0] + src[stride] + ... + src[(S - 1) stride], added in chunk order; the
// loads are issued kMaxChunks at a time.
__device__ __forceinline__ float sum_partials(const float* src, int64_t stride, int S) {
  float s = 0.f;
  for (int k0 = 0; k0 < S; k0 += kMaxChunks) {
    float pk[kMaxChunks];
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) pk[k] = k0 + k < S ? src[(int64_t)(k0 + k) * stride] : 0.f;
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k)
      if (k0 + k < S) s = (k0 + k == 0) ? pk[k] : s + pk[k];
  }
  return s;
}

// ------------------------------------------------------------ wave sum
// Sum of v over the 64 lanes of the wave, the same in every lane: sums of 2,
// 4, 8 and 16 lanes by DPP, then the four rows' sums read from lanes 0, 16,
// 32 and 48 and added in row order.
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// Sums over the 64 lanes of Q values per lane (Q a power of two, 1..64), by
// a reduce-scatter butterfly: at the exchange across lane bit d (32, 16,
// ...) each lane keeps one half of its values and adds the partner's copy of
// that half, so the values a lane holds halve at every step; once one is
// left, plain exchanges finish the sum.  On return v[0] of lane l is the sum
// of value l >> (6 - log2 Q) over all lanes (a fixed order, the same in
// every lane).  Q + 6 - log2 Q - 1 exchanges in all.
template <int Q, int D, int CNT>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[Q], int lane) {
  if constexpr (D >= 1) {
    if constexpr (CNT > 1) {
      constexpr int H = CNT / 2;
      const bool upper = (lane & D) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = upper ? v[i] : v[i + H];
        const float keep = upper ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, D);
      }
      reduce_scatter_step<Q, D / 2, H>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], D);
      reduce_scatter_step<Q, D / 2, 1>(v, lane);
    }
  }
}

template <int Q>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[Q]) {
  static_assert(Q >= 1 && Q <= 64 && (Q & (Q - 1)) == 0, "Q is a power of two up to 64");
  reduce_scatter_step<Q, 32, Q>(v, threadIdx.x & 63);
  return v[0];
}

// ------------------------------------------------------------ block scan
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << __lane_id()) - 1ull; }

// Exclusive scan of one value per thread across a workgroup of W waves;
// *total receives the sum over the workgroup.  Contains barriers: every
// thread of the workgroup must call it.
template <int W, typename V>
__device__ V block_exclusive_scan(V v, V* s_wsum, V* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  V x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    V y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    V s = lane < W ? s_wsum[lane] : V(0);
#pragma unroll
    for (int d = 1; d < W; d <<= 1) {
      V y = __shfl_up(s, d);
      if (lane >= d) s += y;
    }
    if (lane < W) s_wsum[lane] = s;
  }
  __syncthreads();
  const V before = w > 0 ? s_wsum[w - 1] : V(0);
  *total = s_wsum[W - 1];
  __syncthreads();
  return before + x - v;
}

}  // namespace lora
