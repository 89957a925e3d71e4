// Retained-rank store packing.
//
// Lays every adapter's retained factors end to end at its own rank (or at a
// common padded rank for the comparison variant): the explicit retained-rank
// representation of "LoRAForge: Co-Designing Compression and Execution for
// More Efficient Multi-LoRA Serving" (section "LoRAForge's Core Design").
//   A_pack: rows row_off[a] .. row_off[a] + stored - 1 are the rows of A_a
//           ([r_a, d_in] row-major), then zero rows up to the stored rank;
//   B_pack: elements row_off[a] * d_out .. are B_a in its own [d_out, r_a]
//           row-major orientation, each row widened with zeros to the
//           stored rank.
// Both factors keep the orientation the adapter was trained in, so packing
// is a copy, and the expand reads a run of consecutive rows of B_a (all
// ranks of 128 output features) as one contiguous block.
#include "device_common.h"
#include "kernels.h"

namespace lora {

// Binary search: adapter owning stored row rr (row_off is non-decreasing).
__device__ __forceinline__ int owner_of_row(const int32_t* row_off, int n, int rr) {
  int lo = 0, hi = n;  // invariant: row_off[lo] <= rr < row_off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (row_off[mid] <= rr) lo = mid; else hi = mid;
  }
  return lo;
}

// One block per stored row of A_pack.
template <typename E>
__global__ void __launch_bounds__(256) pack_a_kernel(const int32_t* __restrict__ row_off,
                                                     const int32_t* __restrict__ true_rank,
                                                     const void* const* __restrict__ a_ptrs, int n,
                                                     int d_in, void* __restrict__ a_pack) {
  __shared__ int s_owner;
  const int rr = blockIdx.x;
  if (threadIdx.x == 0) s_owner = owner_of_row(row_off, n, rr);
  __syncthreads();
  const int a = s_owner;
  const int j = rr - row_off[a];
  typedef typename E::storage S;
  S* dst = reinterpret_cast<S*>(a_pack) + (size_t)rr * d_in;
  const S* src = j < true_rank[a] ? reinterpret_cast<const S*>(a_ptrs[a]) + (size_t)j * d_in : nullptr;
  constexpr int V = E::kVec;
  if (src != nullptr && ((reinterpret_cast<uintptr_t>(src) & 15u) == 0)) {
    for (int k = threadIdx.x * V; k < d_in; k += blockDim.x * V) st16(dst + k, ld16(src + k));
  } else if (src != nullptr) {
    for (int k = threadIdx.x; k < d_in; k += blockDim.x) dst[k] = src[k];
  } else {
    for (int k = threadIdx.x * V; k < d_in; k += blockDim.x * V) st16(dst + k, make_uint4(0, 0, 0, 0));
  }
}

// One block per (adapter, run of kPackRows rows of B_a): element (o, j) of
// the adapter's block is B_a[o, j] for j < r_a and zero for the padded
// columns r_a <= j < stored rank.
constexpr int kPackRows = 256;

template <typename E>
__global__ void __launch_bounds__(256) pack_b_kernel(const int32_t* __restrict__ row_off,
                                                     const int32_t* __restrict__ true_rank,
                                                     const void* const* __restrict__ b_ptrs,
                                                     int d_out, void* __restrict__ b_pack) {
  typedef typename E::storage S;
  const int a = blockIdx.y;
  const int o0 = blockIdx.x * kPackRows;
  const int r = true_rank[a];
  const int stored = row_off[a + 1] - row_off[a];
  if (stored == 0 || o0 >= d_out) return;
  const int rows = min(kPackRows, d_out - o0);
  const S* src = r > 0 ? reinterpret_cast<const S*>(b_ptrs[a]) + (size_t)o0 * r : nullptr;
  S* dst = reinterpret_cast<S*>(b_pack) + (size_t)row_off[a] * d_out + (size_t)o0 * stored;
  for (int idx = threadIdx.x; idx < rows * stored; idx += blockDim.x) {
    const int o = idx / stored, j = idx - o * stored;
    dst[idx] = j < r ? src[(size_t)o * r + j] : S(0);
  }
}

hipError_t launch_pack(int dtype, const void* meta, int n, int d_in, int d_out, int rows,
                       void* a_pack, void* b_pack, hipStream_t stream) {
  const char* m = reinterpret_cast<const char*>(meta);
  const int32_t* row_off = reinterpret_cast<const int32_t*>(m);
  const int32_t* true_rank = row_off + (n + 1) + 2 * n;
  const void* const* a_ptrs = reinterpret_cast<const void* const*>(m + meta_ptr_offset(n));
  const void* const* b_ptrs = a_ptrs + n;
  if (rows > 0) {
    if (dtype == LORA_DTYPE_BF16)
      hipLaunchKernelGGL(pack_a_kernel<BF16>, dim3(rows), dim3(256), 0, stream, row_off, true_rank,
                         a_ptrs, n, d_in, a_pack);
    else
      hipLaunchKernelGGL(pack_a_kernel<F32>, dim3(rows), dim3(256), 0, stream, row_off, true_rank,
                         a_ptrs, n, d_in, a_pack);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((d_out + kPackRows - 1) / kPackRows, n);
    if (dtype == LORA_DTYPE_BF16)
      hipLaunchKernelGGL(pack_b_kernel<BF16>, grid, dim3(256), 0, stream, row_off, true_rank, b_ptrs,
                         d_out, b_pack);
    else
      hipLaunchKernelGGL(pack_b_kernel<F32>, grid, dim3(256), 0, stream, row_off, true_rank, b_ptrs,
                         d_out, b_pack);
  }
  return hipGetLastError();
}

}  // namespace lora
