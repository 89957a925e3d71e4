// Kernel launchers (one group per .hip file); called by the C ABI in api.hip.
// Every launcher only enqueues work on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace lora {

hipError_t launch_pack(int dtype, const void* meta, int n, int d_in, int d_out, int rows, void* a_pack,
                       void* b_pack, hipStream_t stream);

// Single-workgroup stable grouping of T tokens over n adapters.
size_t segment_lds_bytes(int T, int n);
size_t segment_static_lds_bytes();
hipError_t launch_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm,
                          int32_t* n_invalid, hipStream_t stream);

// Grouping and plan in one workgroup (group_fits: T <= kGroupMaxT, n <=
// kGroupMaxN): seg_off, perm and the plan are each optional.  With id_map,
// token t is grouped by id_map[ids[t]] (the cluster of its adapter).
bool group_fits(int T, int n);
size_t group_lds_bytes(int T, int n);
hipError_t launch_group(const int32_t* ids, int T, int n, const int32_t* id_map, int id_map_n, int32_t* seg_off,
                        int32_t* perm, char* plan, int32_t* n_invalid, hipStream_t stream);
// Plan of a caller-supplied grouping; with a store, also each sub-tile's
// metadata (for the expand from a caller's h).
hipError_t launch_plan(const int32_t* seg_off, const int32_t* perm, int T, int n, char* plan,
                       const lora_store* store, TileMeta* meta, hipStream_t stream);

// Shrink of every sub-tile of `plan` into the float32 partial sums of ws
// (ws_layout), recording each sub-tile's metadata there too.
hipError_t launch_shrink(const lora_store& s, const char* plan, int T, const void* x, int64_t ldx, void* ws,
                         hipStream_t stream);
// The whole apply in one launch for decode-sized calls with ids
// (decode_apply_fits): one workgroup per (token, slice of output features).
bool decode_apply_fits(const lora_store& s, int T, bool with_ids);
hipError_t launch_decode_apply(const lora_store& s, const int32_t* ids, int T, const void* x, int64_t ldx, void* y,
                               int64_t ldy, hipStream_t stream);
// Shared-basis apply: per token of each planned sub-tile (grouped by the
// cluster of its adapter), g = s_a Sigma_a (sum of the partials) into h.
hipError_t launch_jd_sigma(const lora_store& basis, const char* plan, int T, const void* ws, const int32_t* ids,
                           int n, const int32_t* cluster_of, const float* sigma, int diag, const float* scale,
                           float* h, int64_t ldh, hipStream_t stream);
// h (grouped rows) = sum of the partials, in chunk order.
hipError_t launch_reduce_partials(const lora_store& s, const char* plan, int T, const void* ws, float* h,
                                  int64_t ldh, hipStream_t stream);
// Expand over the plan and the metadata in ws: from h (grouped rows) or,
// with h == nullptr, from the shrink's partial sums in ws.
hipError_t launch_expand(const lora_store& s, const char* plan, int T, const void* ws, const float* h, int64_t ldh,
                         void* y, int64_t ldy, hipStream_t stream);

// The base layer with the branch in its epilogue (bf16 store):
// y = x W0^T + s_a B_a h over tiles of 256 outputs x 256 tokens, tokens in
// grouped order through perm (nullptr: identity); with ids == nullptr the
// base product alone.  h comes from the shrink's partial sums in ws.
size_t base_fused_lds_bytes();
hipError_t launch_base_fused(const lora_store& s, const void* w, int64_t ldw, const void* x, int64_t ldx, void* y,
                             int64_t ldy, int T, const int32_t* perm, const int32_t* ids, const void* ws,
                             hipStream_t stream);

// Retained-factor construction (r-SVD): per adapter, the Grams of B and A^T
// (float64 MFMA), Cholesky and the core C, its Jacobi SVD, W_B and W_A, in
// ws; the write forms B W_B and W_A^T A into a store's buffers.
size_t rsvd_workspace_bytes(int n);
// phases: bit 0 the Gram kernel, bit 1 Cholesky + core, bit 2 Jacobi, bit 3
// W_B / W_A.
hipError_t launch_rsvd_factor(int n, int d_in, int d_out, int dtype, int r, const void* A, const void* B,
                              float* sigma, int32_t* status, void* ws, hipStream_t stream, int phases);
hipError_t launch_rsvd_write(const lora_store& s, int r, const void* A, const void* B, const void* ws,
                             hipStream_t stream);

// Multi-slice apply: the stacked A rows (one workgroup per stacked row).
constexpr int kMaxSlices = LORA_MAX_SLICES;
hipError_t launch_stack_rows(int n, int d_in, int dtype, int n_slices, int R, const int32_t* stk_row_off,
                             const int32_t* hoff, const lora_store* slices, void* dst, hipStream_t stream);
// Multi-slice apply: the stacked store's shrink, which also writes every
// slice's per-sub-tile records (SliceMeta, [n_slices][plan_max_subtiles])
// to sl_meta; then one expand launch for all slices, each reading its records.
hipError_t launch_shrink_slices(const lora_multi_store& m, void* sl_meta, const char* plan, int T, const void* x,
                                int64_t ldx, void* ws, hipStream_t stream);
hipError_t launch_expand_slices(const lora_multi_store& m, const SliceMeta* sl_meta, const char* plan, int T,
                                const void* ws, void* const* y_host, const int64_t* ldy_host, hipStream_t stream);

}  // namespace lora
