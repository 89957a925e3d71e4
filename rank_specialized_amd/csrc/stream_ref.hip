// Bandwidth references for the benchmark, built as their own small library
// (libstream_ref.so), apart from the LoRA library: a plain device copy and a
// plain read of a buffer.  One 16-byte element per thread, 256 threads per
// workgroup, streaming (nontemporal) loads and stores: the simplest form that
// keeps the most loads in flight.  They measure what a read-and-write stream
// and a read-only stream reach on this GPU, the practical ceilings beside the
// published HBM peak that the expand (y read and written) and the shrink
// (reads only) are compared with.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr size_t kMaxBlocks = 1u << 30;  // beyond, the workgroups loop

__global__ void __launch_bounds__(kThreads) copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                        size_t n) {
  const size_t step = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += step)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Every element is read; the xor of the words is written only when it equals
// a value no caller passes (the store keeps the loads from being dropped).
__global__ void __launch_bounds__(kThreads) read_kernel(const u32x4_t* __restrict__ src, size_t n,
                                                        unsigned* __restrict__ sink) {
  const size_t step = (size_t)gridDim.x * kThreads;
  unsigned s = 0;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += step) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    s ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (s == 0x9e3779b9u) sink[0] = s;
}

dim3 grid_of(size_t n) {
  const size_t blocks = (n + kThreads - 1) / kThreads;
  return dim3((unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks));
}

}  // namespace

// dst[0, bytes) = src[0, bytes).  bytes a multiple of 16, both buffers 16-byte
// aligned device memory that do not overlap.  Returns 0, 1 for bad arguments,
// 2 for a launch error.
extern "C" int stream_ref_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0 || (bytes && (!src || !dst)) || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return 1;
  const size_t n = bytes / 16;
  if (n == 0) return 0;
  hipLaunchKernelGGL(copy_kernel, grid_of(n), dim3(kThreads), 0, stream, reinterpret_cast<const u32x4_t*>(src),
                     reinterpret_cast<u32x4_t*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads src[0, bytes); sink (4 bytes of device memory) is written only for a
// value of the data that callers do not use.  Same arguments and returns as
// stream_ref_copy.
extern "C" int stream_ref_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  if (bytes % 16 != 0 || (bytes && (!src || !sink)) || (uintptr_t)src % 16 != 0) return 1;
  const size_t n = bytes / 16;
  if (n == 0) return 0;
  hipLaunchKernelGGL(read_kernel, grid_of(n), dim3(kThreads), 0, stream, reinterpret_cast<const u32x4_t*>(src), n,
                     reinterpret_cast<unsigned*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
