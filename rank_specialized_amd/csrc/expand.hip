// Expand: y[perm[i], o] += s_a * sum_{j < r_a} B_a[o, j] h[i, j].
//
// Step 3 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4: B applied with the
// adapter's scale and added into (a slice of) y.  Accumulation in float32,
// one rounding of the new y value to the output type.
//
// Work unit: one wave per (tile, 64 x 16-byte run of output features).  A
// lane owns one 16-byte run of outputs (8 bf16 / 4 f32); for each retained
// rank index j the wave reads one contiguous 1 KiB run of Bt_pack row j, so
// every factor byte is read once per tile with fully coalesced loads, and
// every y row of the tile is read and written once with 16-byte accesses.
// h values are wave-uniform (scalar loads).
//
// Rank specialization: RB (rank bucket) is a template parameter; all of a
// bucket's Bt loads (up to 32 rows) are issued back to back before the FMAs,
// and rows j >= r_a are never loaded.
#include "device_common.h"
#include "kernels.h"

namespace lora {

constexpr int kExpandTokens = 4;  // tokens accumulated per pass

template <typename E, int RB>
__device__ __forceinline__ void expand_run(const char* __restrict__ bt_rows, int d_out, int r, float s,
                                           const float* __restrict__ h, int64_t ldh,
                                           const int32_t* __restrict__ perm, int p0, int m,
                                           char* __restrict__ y, int64_t ldy_bytes, int o) {
  constexpr int V = E::kVec;
  constexpr int MT = kExpandTokens;
  constexpr int JN = RB < 16 ? RB : 16;
  const bool active = o < d_out;
  const size_t bt_row_bytes = (size_t)d_out * E::kBytes;
  const char* bcol = bt_rows + (size_t)o * E::kBytes;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int t0 = 0; t0 < m; t0 += MT) {
    const int mt = min(MT, m - t0);
    float acc[MT][V];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < V; ++e) acc[t][e] = 0.f;
    const float* hrow = h + (int64_t)(p0 + t0) * ldh;
#pragma unroll 1
    for (int j0 = 0; j0 < RB; j0 += JN) {
      uint4 b[JN];
#pragma unroll
      for (int jj = 0; jj < JN; ++jj) {
        const int j = j0 + jj;
        b[jj] = (active && j < r) ? ld16(bcol + (size_t)j * bt_row_bytes) : zero;
      }
#pragma unroll
      for (int jj = 0; jj < JN; ++jj) {
        const int j = j0 + jj;
        if (j < r) {
          float bf[V];
          E::widen(b[jj], bf);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < mt) {
              const float hv = hrow[(int64_t)t * ldh + j];
#pragma unroll
              for (int e = 0; e < V; ++e) acc[t][e] += hv * bf[e];
            }
          }
        }
      }
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t < mt) {
          const int tok = perm[p0 + t0 + t];
          char* yp = y + (int64_t)tok * ldy_bytes + (size_t)o * E::kBytes;
          float yf[V];
          E::widen(ld16(yp), yf);
#pragma unroll
          for (int e = 0; e < V; ++e) yf[e] = yf[e] + s * acc[t][e];
          st16(yp, E::narrow(yf));
        }
      }
    }
  }
}

template <typename E>
__global__ void __launch_bounds__(256)
expand_kernel(const float* __restrict__ h, int64_t ldh, const char* __restrict__ bt_pack,
              const int32_t* __restrict__ row_off, const int32_t* __restrict__ rank,
              const float* __restrict__ scale, int d_out, int n_runs, int groups_per_tile,
              const int32_t* __restrict__ perm, const void* __restrict__ plan_ws,
              char* __restrict__ y, int64_t ldy_bytes) {
  const Plan pl = plan_view(plan_ws);
  const int t = blockIdx.x / groups_per_tile;
  const int run = (blockIdx.x % groups_per_tile) * 4 + (threadIdx.x >> 6);
  if (t >= *pl.count || run >= n_runs) return;
  const int4 tile = pl.tiles[t];
  const int a = tile.x, p0 = tile.y, m = tile.z;
  const int r = rank[a];
  if (r <= 0) return;
  const float s = scale[a];
  const char* bt_rows = bt_pack + (size_t)row_off[a] * d_out * E::kBytes;
  const int o = (run * 64 + (threadIdx.x & 63)) * E::kVec;
#define LORA_EXPAND_CASE(RB) \
  expand_run<E, RB>(bt_rows, d_out, r, s, h, ldh, perm, p0, m, y, ldy_bytes, o)
  if (r <= 4) LORA_EXPAND_CASE(4);
  else if (r <= 8) LORA_EXPAND_CASE(8);
  else if (r <= 16) LORA_EXPAND_CASE(16);
  else if (r <= 24) LORA_EXPAND_CASE(24);
  else if (r <= 32) LORA_EXPAND_CASE(32);
  else if (r <= 48) LORA_EXPAND_CASE(48);
  else LORA_EXPAND_CASE(64);
#undef LORA_EXPAND_CASE
}

hipError_t launch_expand(const lora_store& s, const float* h, int64_t ldh, int T, const int32_t* perm,
                         const void* plan_ws, void* y, int64_t ldy, hipStream_t stream) {
  const int64_t tiles = plan_max_tiles(T, s.n);
  if (tiles == 0) return hipSuccess;
  const int V = vec_elems(s.dtype);
  const int n_runs = (s.d_out + 64 * V - 1) / (64 * V);
  const int groups = (n_runs + 3) / 4;
  const int64_t grid = tiles * groups;
  const int eb = elem_bytes(s.dtype);
  if (s.dtype == LORA_DTYPE_BF16)
    hipLaunchKernelGGL(expand_kernel<BF16>, dim3((unsigned)grid), dim3(256), 0, stream, h, ldh,
                       reinterpret_cast<const char*>(s.Bt_pack), s.row_off, s.rank, s.scale, s.d_out,
                       n_runs, groups, perm, plan_ws, reinterpret_cast<char*>(y), ldy * eb);
  else
    hipLaunchKernelGGL(expand_kernel<F32>, dim3((unsigned)grid), dim3(256), 0, stream, h, ldh,
                       reinterpret_cast<const char*>(s.Bt_pack), s.row_off, s.rank, s.scale, s.d_out,
                       n_runs, groups, perm, plan_ws, reinterpret_cast<char*>(y), ldy * eb);
  return hipGetLastError();
}

}  // namespace lora
