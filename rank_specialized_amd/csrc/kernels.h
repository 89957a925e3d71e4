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
hipError_t launch_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm,
                          int32_t* n_invalid, void* plan_ws, hipStream_t stream);
hipError_t launch_plan_from_offsets(const int32_t* seg_off, int T, int n, void* plan_ws,
                                    hipStream_t stream);

hipError_t launch_shrink(const lora_store& s, const void* x, int64_t ldx, int T, const int32_t* perm,
                         const void* plan_ws, float* h, int64_t ldh, hipStream_t stream);
hipError_t launch_expand(const lora_store& s, const float* h, int64_t ldh, int T, const int32_t* perm,
                         const void* plan_ws, void* y, int64_t ldy, hipStream_t stream);

}  // namespace lora
