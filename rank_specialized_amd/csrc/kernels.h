// Kernel launchers (one per .hip file); called by the C ABI in api.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace lora {

hipError_t launch_pack(int dtype, const void* meta, int n, int d_in, int d_out, int rows, void* a_pack,
                       void* bt_pack, hipStream_t stream);

// Single-workgroup stable grouping of T tokens over n adapters + tile plan.
size_t segment_lds_bytes(int T, int n);
size_t segment_static_lds_bytes();
hipError_t launch_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm,
                          int32_t* n_invalid, void* plan_ws, hipStream_t stream);
hipError_t launch_plan_from_offsets(const int32_t* seg_off, int T, int n, void* plan_ws,
                                    hipStream_t stream);

hipError_t launch_shrink(const lora_store& s, const void* x, int64_t ldx, int T, const int32_t* perm,
                         const void* plan_ws, float* h, int64_t ldh, hipStream_t stream);
hipError_t launch_expand(const lora_store& s, const float* h, int64_t ldh, int T, const int32_t* perm,
                         const void* plan_ws, void* y, int64_t ldy, hipStream_t stream);
// Shrink and expand of every shrink sub-tile in one workgroup (h in LDS).
hipError_t launch_apply_fused(const lora_store& s, const void* x, int64_t ldx, int T, const int32_t* perm,
                              const void* plan_ws, void* y, int64_t ldy, hipStream_t stream);

// Decode-shaped batches (a few tokens per adapter on average) take the fused
// path; prefill-shaped ones the separate shrink and expand kernels.
inline bool use_fused_apply(int T, int n) { return (int64_t)T <= 8 * (int64_t)n; }

}  // namespace lora
