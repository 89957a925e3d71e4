// Shrink: h[i, j] = sum_k A_a[j, k] x[perm[i], k]   (j < r_a), float32.
//
// Step 1 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4 (A applied with scale
// 1 into a float32 buffer of shape [tokens, R]).  Rows of h follow the
// grouped order, so one tile's rows are contiguous.
//
// One workgroup (4 waves) per tile (<= 64 tokens of one adapter).  The tile
// is a skinny GEMM  H^T[r_a x m] = A_a[r_a x d_in] . X^T[d_in x m]  and runs
// on 16x16 MFMA tiles whatever m is: the matrix core performs the d_in
// reduction, so a one-token decode segment needs no cross-lane reduction;
// rows j >= r_a and tokens >= m are never loaded (zero operands), so memory
// traffic is exactly the retained rows plus the tile's x rows.
//
// Rank specialization: NG = ceil(r_a / 16) row groups is a template
// parameter, so each instantiation keeps exactly its accumulators and
// issues its loads for several K-steps back to back.
//
// K split: the 4 waves take consecutive quarters of d_in; inside a wave,
// lane group g (lanes 16g..16g+15) owns a contiguous quarter of the wave's
// range and walks it 16 bytes per step, so both operands of every MFMA
// carry the same K indices (the contraction is a plain sum over K, so any
// assignment of K indices to lane groups that is identical for the two
// operands is exact).  The 4 partial tiles are summed in LDS in wave order
// (deterministic).
#include "device_common.h"
#include "kernels.h"

namespace lora {

template <typename E, int NG>
__device__ __forceinline__ void shrink_tile(const char* __restrict__ x, int64_t ldx_bytes,
                                            const char* __restrict__ a_rows, int d_in, int r,
                                            const int32_t* __restrict__ perm, int p0, int m,
                                            float* __restrict__ h, int64_t ldh, f32x4_t* red) {
  constexpr int V = E::kVec;
  constexpr int KSTEP = 4 * V;              // K covered by one 16-byte chunk over the wave
  constexpr int U = NG <= 1 ? 8 : (NG == 2 ? 4 : 2);  // K-steps issued back to back
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int steps_total = (d_in + KSTEP - 1) / KSTEP;
  const int steps_w = (steps_total + 3) / 4;
  const int k_lane0 = (w * steps_w * 4 + g * steps_w) * V;
  const size_t a_row_bytes = (size_t)d_in * E::kBytes;

  const char* arow[NG];
  bool aval[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int j = q * 16 + i;
    aval[q] = j < r;
    arow[q] = a_rows + (size_t)(aval[q] ? j : 0) * a_row_bytes;
  }
  const uint4 zero = make_uint4(0, 0, 0, 0);
  const int nt = (m + 15) >> 4;
  for (int u = 0; u < nt; ++u) {
    const int tl = u * 16 + i;
    const bool tval = tl < m;
    const char* xrow = x + (int64_t)(tval ? perm[p0 + tl] : 0) * ldx_bytes;
    f32x4_t acc[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < steps_w; s0 += U) {
      uint4 bx[U], ba[U][NG];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int s = s0 + uu;
        const int k = k_lane0 + s * V;
        const bool kv = s < steps_w && k < d_in;
        bx[uu] = (tval && kv) ? ld16(xrow + (size_t)k * E::kBytes) : zero;
#pragma unroll
        for (int q = 0; q < NG; ++q)
          ba[uu][q] = (aval[q] && kv) ? ld16(arow[q] + (size_t)k * E::kBytes) : zero;
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu)
#pragma unroll
        for (int q = 0; q < NG; ++q) acc[q] = mfma_chunk<E>(ba[uu][q], bx[uu], acc[q]);
    }
    if (w > 0) {
#pragma unroll
      for (int q = 0; q < NG; ++q) red[((w - 1) * NG + q) * 64 + lane] = acc[q];
    }
    __syncthreads();
    if (w == 0) {
      const int tok = u * 16 + i;  // output column of this lane
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        f32x4_t s = acc[q];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) s += red[((ww - 1) * NG + q) * 64 + lane];
        const int j0 = q * 16 + 4 * g;
        if (tok < m && j0 < r) {
          float* hr = h + (int64_t)(p0 + tok) * ldh + j0;
          if (j0 + 0 < r) hr[0] = s[0];
          if (j0 + 1 < r) hr[1] = s[1];
          if (j0 + 2 < r) hr[2] = s[2];
          if (j0 + 3 < r) hr[3] = s[3];
        }
      }
    }
    __syncthreads();
  }
}

template <typename E>
__global__ void __launch_bounds__(256)
shrink_kernel(const char* __restrict__ x, int64_t ldx_bytes, const char* __restrict__ a_pack,
              const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank, int d_in,
              const int32_t* __restrict__ perm, const void* __restrict__ plan_ws,
              float* __restrict__ h, int64_t ldh) {
  __shared__ f32x4_t red[3 * 4 * 64];
  const Plan pl = plan_view(plan_ws);
  const int t = blockIdx.x;
  if (t >= *pl.count) return;
  const int4 tile = pl.tiles[t];
  const int a = tile.x, p0 = tile.y, m = tile.z;
  const int r = rank[a];
  if (r <= 0) return;
  const char* a_rows = a_pack + (size_t)row_off[a] * d_in * E::kBytes;
  switch ((r + 15) >> 4) {
    case 1: shrink_tile<E, 1>(x, ldx_bytes, a_rows, d_in, r, perm, p0, m, h, ldh, red); break;
    case 2: shrink_tile<E, 2>(x, ldx_bytes, a_rows, d_in, r, perm, p0, m, h, ldh, red); break;
    case 3: shrink_tile<E, 3>(x, ldx_bytes, a_rows, d_in, r, perm, p0, m, h, ldh, red); break;
    default: shrink_tile<E, 4>(x, ldx_bytes, a_rows, d_in, r, perm, p0, m, h, ldh, red); break;
  }
}

hipError_t launch_shrink(const lora_store& s, const void* x, int64_t ldx, int T, const int32_t* perm,
                         const void* plan_ws, float* h, int64_t ldh, hipStream_t stream) {
  const int64_t grid = plan_max_tiles(T, s.n);
  if (grid == 0) return hipSuccess;
  const int eb = elem_bytes(s.dtype);
  if (s.dtype == LORA_DTYPE_BF16)
    hipLaunchKernelGGL(shrink_kernel<BF16>, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const char*>(x), ldx * eb,
                       reinterpret_cast<const char*>(s.A_pack), s.row_off, s.rank, s.d_in, perm,
                       plan_ws, h, ldh);
  else
    hipLaunchKernelGGL(shrink_kernel<F32>, dim3((unsigned)grid), dim3(256), 0, stream,
                       reinterpret_cast<const char*>(x), ldx * eb,
                       reinterpret_cast<const char*>(s.A_pack), s.row_off, s.rank, s.d_in, perm,
                       plan_ws, h, ldh);
  return hipGetLastError();
}

}  // namespace lora
