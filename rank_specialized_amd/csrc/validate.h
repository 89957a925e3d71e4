// Argument checks of the C ABI.  Pure host C++ (no HIP calls), so every
// error path can be exercised without a GPU.
#pragma once
#include "plan.h"

namespace lora {

int check_store_shape(int n, int d_in, int d_out, int dtype, const int32_t* ranks_host, int pad_to,
                      int* r_max_out, int64_t* rows_out);
int check_store(const lora_store* s);
int check_segment_args(const int32_t* ids, int T, int n, const int32_t* seg_off, const int32_t* perm);
int check_grouping(const lora_store* s, int T, const int32_t* seg_off, const int32_t* perm);
size_t workspace_bytes(const lora_store* s, int T);
int check_ws(const lora_store* s, int T, const void* ws, size_t ws_bytes);
int check_rows(const void* p, int64_t ld, int d, int dtype, int T);
int check_h(const float* h, int64_t ldh, const lora_store* s, int T);

}  // namespace lora
