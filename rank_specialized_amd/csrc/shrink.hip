// Shrink: h[i, j] = sum_k A_a[j, k] x[perm[i], k]   (j < r_a), float32.
//
// Step 1 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4 (A applied with scale
// 1 into a float32 buffer of shape [tokens, R]).  Rows of h follow the
// grouped order, so one tile's rows are contiguous.
//
// One workgroup of 16 waves per sub-tile (<= 16 tokens of one adapter).  A
// sub-tile is the skinny GEMM  H^T[r_a x m] = A_a[r_a x d_in] . X^T[d_in x m]
// on 16x16 MFMA tiles whatever m is: the matrix core does the d_in
// reduction, so a one-token decode segment needs no cross-lane reduction.
// Rows j >= r_a and tokens >= m are never loaded (zero operands): memory
// traffic is the retained rows (once per sub-tile) plus the tile's x rows.
// The 16 waves split d_in into 16 chunks, so even a decode batch of a few
// hundred tokens spreads over thousands of waves, and a popular adapter's
// tokens spread over several CUs (a CU's own bandwidth is the limit
// otherwise).  The waves' float32 partial tiles are summed in LDS in a fixed
// order (deterministic, no atomics) and written to h once.
//
// Rank specialization: NG = ceil(r_a / 16) row groups is a template
// parameter; each instantiation keeps exactly its accumulators and issues U
// K-steps of loads back to back (U sized so the loads in flight fit the
// register budget of a 1024-thread workgroup).
//
// Inside a wave, step s covers K indices [k0 + s * 32, +32) (bf16): lane
// group g (lanes 16g..16g+15) takes the g-th 16 bytes of it, so the four lane
// groups of a row read 64 contiguous bytes per instruction and two
// consecutive steps consume whole 128-byte lines.  Both operands of every
// MFMA carry the same K indices (the contraction is a plain sum over K, so
// any K order that is identical for the two operands is exact).
#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {

constexpr int kShrinkWaves = 16;
constexpr int kShrinkThreads = kShrinkWaves * kWave;

// red: [16 slots][ng_max][64 lanes] of f32x4; slot = wave = K chunk.
template <typename E>
__global__ void __launch_bounds__(kShrinkThreads)
shrink_kernel(const char* __restrict__ x, int64_t ldx_bytes, const char* __restrict__ a_pack,
              const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank, int d_in, int ng_max,
              const int32_t* __restrict__ perm, const void* __restrict__ plan_ws, size_t sub_off,
              float* __restrict__ h, int64_t ldh) {
  extern __shared__ f32x4_t red[];
  constexpr int KSTEP = 4 * E::kVec;
  const Plan pl = plan_view(plan_ws, sub_off);
  const int t = blockIdx.x;  // grid = sub-tile capacity, so subtiles[t] is in bounds
  const int4 tile = pl.subtiles[t];
  const int count = pl.count[3];
  if (t >= count) return;
  const int a = tile.x, p0 = tile.y, m = tile.z;  // m <= kSubTile
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tl = lane & 15;
  const bool tval = tl < m;
  const int tok = tval ? perm[p0 + tl] : 0;
  const int r = rank[a];
  const int ro = row_off[a];
  if (r <= 0) return;  // uniform over the workgroup
  const int ng = (r + 15) >> 4;
  int kc = (d_in + kShrinkWaves - 1) / kShrinkWaves;
  kc = (kc + KSTEP - 1) / KSTEP * KSTEP;
  const int k0 = w * kc;
  const char* xrow = x + (int64_t)tok * ldx_bytes;
  const char* a_rows = a_pack + (size_t)ro * d_in * E::kBytes;
  f32x4_t* slot = red + w * ng_max * 64;
  switch (ng) {
    case 1: shrink_wave<E, 1>(xrow, tval, a_rows, d_in, r, k0, kc, slot); break;
    case 2: shrink_wave<E, 2>(xrow, tval, a_rows, d_in, r, k0, kc, slot); break;
    case 3: shrink_wave<E, 3>(xrow, tval, a_rows, d_in, r, k0, kc, slot); break;
    default: shrink_wave<E, 4>(xrow, tval, a_rows, d_in, r, k0, kc, slot); break;
  }
  __syncthreads();
  // Sum the 16 slots of each (row group, lane, accumulator row) in slot order
  // and write h.  Lane l of a partial tile holds token l % 16 and rank rows
  // 4 * (l / 16) + 0..3 of its row group.
  const float* redf = reinterpret_cast<const float*>(red);
  for (int c = threadIdx.x; c < ng * 256; c += kShrinkThreads) {
    const int v = c & 3, l = (c >> 2) & 63, q = c >> 8;
    const int tk = l & 15;
    const int j = q * 16 + 4 * (l >> 4) + v;
    if (tk >= m || j >= r) continue;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kShrinkWaves; ++k) s += redf[((k * ng_max + q) * 64 + l) * 4 + v];
    h[(int64_t)(p0 + tk) * ldh + j] = s;
  }
}

size_t shrink_lds_bytes(int r_max) {
  const int ng_max = r_max <= 0 ? 1 : (r_max + 15) / 16;
  return (size_t)kShrinkWaves * ng_max * 64 * sizeof(float) * 4;
}

hipError_t launch_shrink(const lora_store& s, const void* x, int64_t ldx, int T, const int32_t* perm,
                         const void* plan_ws, float* h, int64_t ldh, hipStream_t stream) {
  const int64_t subs = plan_max_subtiles(T, s.n);
  if (subs == 0) return hipSuccess;
  const int ng_max = s.r_max <= 0 ? 1 : (s.r_max + 15) / 16;
  const size_t lds = shrink_lds_bytes(s.r_max);
  const size_t sub_off = plan_subtile_offset(T, s.n);
  const int eb = elem_bytes(s.dtype);
  if (s.dtype == LORA_DTYPE_BF16)
    hipLaunchKernelGGL(shrink_kernel<BF16>, dim3((unsigned)subs), dim3(kShrinkThreads), lds, stream,
                       reinterpret_cast<const char*>(x), ldx * eb,
                       reinterpret_cast<const char*>(s.A_pack), s.row_off, s.rank, s.d_in, ng_max, perm,
                       plan_ws, sub_off, h, ldh);
  else
    hipLaunchKernelGGL(shrink_kernel<F32>, dim3((unsigned)subs), dim3(kShrinkThreads), lds, stream,
                       reinterpret_cast<const char*>(x), ldx * eb,
                       reinterpret_cast<const char*>(s.A_pack), s.row_off, s.rank, s.d_in, ng_max, perm,
                       plan_ws, sub_off, h, ldh);
  return hipGetLastError();
}

}  // namespace lora
