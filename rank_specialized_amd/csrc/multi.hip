// Multi-slice apply: the projections that read the same input (q, k and v;
// gate and up) applied with one read of x.
//
// "Compress then Serve: Serving Thousands of LoRA Adapters with Little
// Overhead", section 13.4: the expand step adds into a slice of y given by
// an offset and a width, so several projections' deltas can land in one
// fused output.  Here the slices' A factors are stacked per adapter
// (A_q,a; A_k,a; A_v,a) into one store, so that one shrink reads each x row
// once for every slice; each slice's expand then reads its own columns of
// the stacked h (from hoff[s][a]) with its own B, rank and scale.
#include "device_common.h"
#include "kernels.h"

namespace lora {

struct StackArgs {
  int n, n_slices;
  int64_t row_bytes;            // d_in * element bytes (a multiple of 16)
  const int32_t* stk_row_off;   // [n + 1]: the stacked store's row offsets
  const int32_t* hoff;          // [n_slices][n]
  const char* src_a[kMaxSlices];
  const int32_t* src_row_off[kMaxSlices];
  const int32_t* src_rank[kMaxSlices];
  char* dst;
};

// One workgroup per stacked row g: its adapter a (the last with
// row_off[a] <= g), its slice s (hoff[s][a] <= j < hoff[s][a] + rank_s[a]
// for j = g - row_off[a]), then a copy of the slice's row.
__global__ void __launch_bounds__(256) stack_rows_kernel(StackArgs p) {
  const int g = blockIdx.x;
  int lo = 0, hi = p.n;  // row_off[lo] <= g < row_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.stk_row_off[mid] <= g) lo = mid;
    else hi = mid;
  }
  const int a = lo, j = g - p.stk_row_off[a];
  const char* src = nullptr;
  for (int s = 0; s < p.n_slices; ++s) {
    const int h = p.hoff[(size_t)s * p.n + a], rk = p.src_rank[s][a];
    if (j >= h && j < h + rk) src = p.src_a[s] + (size_t)(p.src_row_off[s][a] + j - h) * p.row_bytes;
  }
  if (src == nullptr) return;  // not reached for a consistent stacking
  char* dst = p.dst + (size_t)g * p.row_bytes;
  for (int64_t off = 16 * (int64_t)threadIdx.x; off < p.row_bytes; off += 16 * 256) st16(dst + off, ld16(src + off));
}

hipError_t launch_stack_rows(int n, int d_in, int dtype, int n_slices, int R, const int32_t* stk_row_off,
                             const int32_t* hoff, const lora_store* slices, void* dst, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  StackArgs a;
  a.n = n;
  a.n_slices = n_slices;
  a.row_bytes = (int64_t)d_in * elem_bytes(dtype);
  a.stk_row_off = stk_row_off;
  a.hoff = hoff;
  for (int s = 0; s < kMaxSlices; ++s) {
    const bool in = s < n_slices;
    a.src_a[s] = in ? reinterpret_cast<const char*>(slices[s].A_pack) : nullptr;
    a.src_row_off[s] = in ? slices[s].row_off : nullptr;
    a.src_rank[s] = in ? slices[s].rank : nullptr;
  }
  a.dst = reinterpret_cast<char*>(dst);
  hipLaunchKernelGGL(stack_rows_kernel, dim3((unsigned)R), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lora
