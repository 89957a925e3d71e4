// Fused apply for decode-shaped batches (few tokens per adapter):
//   y[t] += s_a * B_a (A_a x[t])  for the tokens of one sub-tile, in one
// workgroup, with the float32 intermediate kept in LDS.
//
// The two steps are those of "Compress then Serve: Serving Thousands of LoRA
// Adapters with Little Overhead", section 13.4 (A applied with scale 1 into
// a float32 buffer, then B applied with the scale and added into y); fusing
// them removes the intermediate's round trip through memory and one launch,
// which dominate when every adapter has only a handful of tokens.
//
// One workgroup of 16 waves per sub-tile (<= 16 tokens of one adapter):
//  1. shrink: the 16 waves split d_in exactly as the standalone shrink does
//     (same chunks, same in-LDS summation order), so h is bit-identical;
//  2. expand: the waves take (run of 64 x 16 bytes of output features,
//     group of kSmallTile tokens) items with the same vector code as the
//     standalone expand's decode path, reading h from LDS.
// The result equals lora_shrink followed by lora_expand bit for bit.
#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {

constexpr int kFusedWaves = 16;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kHlStride = 68;  // floats per token row of h in LDS

template <typename E>
__global__ void __launch_bounds__(kFusedThreads)
apply_fused_kernel(const char* __restrict__ x, int64_t ldx_bytes, const char* __restrict__ a_pack,
                   const char* __restrict__ bt_pack, const int32_t* __restrict__ row_off,
                   const int32_t* __restrict__ rank, const float* __restrict__ scale, int d_in, int d_out,
                   int ng_max, const int32_t* __restrict__ perm, const void* __restrict__ plan_ws,
                   size_t sub_off, char* __restrict__ y, int64_t ldy_bytes) {
  extern __shared__ f32x4_t red[];
  __shared__ float hl[kSubTile * kHlStride];
  constexpr int V = E::kVec;
  constexpr int KSTEP = 4 * V;
  const Plan pl = plan_view(plan_ws, sub_off);
  const int t = blockIdx.x;  // grid = sub-tile capacity
  const int4 tile = pl.subtiles[t];
  const int count = pl.count[3];
  if (t >= count) return;
  const int a = tile.x, p0 = tile.y, m = tile.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tl = lane & 15;
  const bool tval = tl < m;
  const int tok = tval ? perm[p0 + tl] : 0;
  const int r = rank[a];
  const int ro = row_off[a];
  if (r <= 0) return;  // uniform over the workgroup
  const float sc = scale[a];
  const int ng = (r + 15) >> 4;
  // 1. shrink (identical split to the standalone shrink kernel)
  {
    int kc = (d_in + kFusedWaves - 1) / kFusedWaves;
    kc = (kc + KSTEP - 1) / KSTEP * KSTEP;
    const char* xrow = x + (int64_t)tok * ldx_bytes;
    const char* a_rows = a_pack + (size_t)ro * d_in * E::kBytes;
    f32x4_t* slot = red + w * ng_max * 64;
    switch (ng) {
      case 1: shrink_wave<E, 1>(xrow, tval, a_rows, d_in, r, w * kc, kc, slot); break;
      case 2: shrink_wave<E, 2>(xrow, tval, a_rows, d_in, r, w * kc, kc, slot); break;
      case 3: shrink_wave<E, 3>(xrow, tval, a_rows, d_in, r, w * kc, kc, slot); break;
      default: shrink_wave<E, 4>(xrow, tval, a_rows, d_in, r, w * kc, kc, slot); break;
    }
  }
  __syncthreads();
  {
    const float* redf = reinterpret_cast<const float*>(red);
    for (int c = threadIdx.x; c < ng * 256; c += kFusedThreads) {
      const int v = c & 3, l = (c >> 2) & 63, q = c >> 8;
      const int tk = l & 15;
      const int j = q * 16 + 4 * (l >> 4) + v;
      if (tk >= m || j >= r) continue;
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < kFusedWaves; ++k) s += redf[((k * ng_max + q) * 64 + l) * 4 + v];
      hl[tk * kHlStride + j] = s;
    }
  }
  __syncthreads();
  // 2. expand
  const char* bt_rows = bt_pack + (size_t)ro * d_out * E::kBytes;
  const int runs = (d_out + 64 * V - 1) / (64 * V);
  const int groups = (m + kSmallTile - 1) / kSmallTile;
  for (int item = w; item < runs * groups; item += kFusedWaves) {
    const int run = item % runs, tg = item / runs;
    const int t0 = tg * kSmallTile;
    const int mt = min(kSmallTile, m - t0);
    const int o = (run * 64 + lane) * V;
    const float* hr = hl + t0 * kHlStride;
    if (r <= 4) expand_small<E, 4>(bt_rows, d_out, r, sc, hr, kHlStride, perm, p0 + t0, mt, y, ldy_bytes, o);
    else if (r <= 8) expand_small<E, 8>(bt_rows, d_out, r, sc, hr, kHlStride, perm, p0 + t0, mt, y, ldy_bytes, o);
    else if (r <= 16) expand_small<E, 16>(bt_rows, d_out, r, sc, hr, kHlStride, perm, p0 + t0, mt, y, ldy_bytes, o);
    else if (r <= 32) expand_small<E, 32>(bt_rows, d_out, r, sc, hr, kHlStride, perm, p0 + t0, mt, y, ldy_bytes, o);
    else expand_small<E, 64>(bt_rows, d_out, r, sc, hr, kHlStride, perm, p0 + t0, mt, y, ldy_bytes, o);
  }
}

hipError_t launch_apply_fused(const lora_store& s, const void* x, int64_t ldx, int T, const int32_t* perm,
                              const void* plan_ws, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t subs = plan_max_subtiles(T, s.n);
  if (subs == 0) return hipSuccess;
  const int ng_max = s.r_max <= 0 ? 1 : (s.r_max + 15) / 16;
  const size_t lds = (size_t)kFusedWaves * ng_max * 64 * 16;
  const size_t sub_off = plan_subtile_offset(T, s.n);
  const int eb = elem_bytes(s.dtype);
  if (s.dtype == LORA_DTYPE_BF16)
    hipLaunchKernelGGL(apply_fused_kernel<BF16>, dim3((unsigned)subs), dim3(kFusedThreads), lds, stream,
                       reinterpret_cast<const char*>(x), ldx * eb, reinterpret_cast<const char*>(s.A_pack),
                       reinterpret_cast<const char*>(s.Bt_pack), s.row_off, s.rank, s.scale, s.d_in, s.d_out,
                       ng_max, perm, plan_ws, sub_off, reinterpret_cast<char*>(y), ldy * eb);
  else
    hipLaunchKernelGGL(apply_fused_kernel<F32>, dim3((unsigned)subs), dim3(kFusedThreads), lds, stream,
                       reinterpret_cast<const char*>(x), ldx * eb, reinterpret_cast<const char*>(s.A_pack),
                       reinterpret_cast<const char*>(s.Bt_pack), s.row_off, s.rank, s.scale, s.d_in, s.d_out,
                       ng_max, perm, plan_ws, sub_off, reinterpret_cast<char*>(y), ldy * eb);
  return hipGetLastError();
}

}  // namespace lora
