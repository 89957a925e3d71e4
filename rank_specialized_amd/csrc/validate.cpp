// Argument validation for the C ABI (host only, no HIP calls).
#include "validate.h"

namespace lora {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_store_shape(int n, int d_in, int d_out, int dtype, const int32_t* ranks_host, int pad_to,
                      int* r_max_out, int64_t* rows_out) {
  if (n < 0 || d_in <= 0 || d_out <= 0 || pad_to < 0) return LORA_ERR_INVALID_ARG;
  if (n > 0 && ranks_host == nullptr) return LORA_ERR_INVALID_ARG;
  if (dtype != LORA_DTYPE_BF16 && dtype != LORA_DTYPE_F32) return LORA_ERR_UNSUPPORTED;
  int r_max = 0;
  for (int a = 0; a < n; ++a) {
    if (ranks_host[a] < 0) return LORA_ERR_INVALID_ARG;
    if (ranks_host[a] > r_max) r_max = ranks_host[a];
  }
  if (pad_to > 0 && pad_to < r_max) return LORA_ERR_INVALID_ARG;
  int stored_max = pad_to > 0 ? pad_to : r_max;
  if (stored_max > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  int64_t rows = 0;
  for (int a = 0; a < n; ++a) rows += pad_to > 0 ? pad_to : ranks_host[a];
  if (rows > INT32_MAX) return LORA_ERR_INVALID_ARG;
  int v = vec_elems(dtype);
  if (d_in % v != 0 || d_out % v != 0) return LORA_ERR_UNSUPPORTED;
  if (r_max_out) *r_max_out = stored_max;
  if (rows_out) *rows_out = rows;
  return LORA_OK;
}

int check_store(const lora_store* s) {
  if (s == nullptr) return LORA_ERR_INVALID_ARG;
  if (s->n < 1 || s->d_in <= 0 || s->d_out <= 0 || s->R < 0 || s->r_max < 0 || s->pad_to < 0)
    return LORA_ERR_INVALID_ARG;
  if (s->dtype != LORA_DTYPE_BF16 && s->dtype != LORA_DTYPE_F32) return LORA_ERR_UNSUPPORTED;
  if (s->r_max > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
  if (s->row_off == nullptr || s->rank == nullptr || s->scale == nullptr) return LORA_ERR_INVALID_ARG;
  if (s->R > 0 && (s->A_pack == nullptr || s->B_pack == nullptr)) return LORA_ERR_INVALID_ARG;
  int v = vec_elems(s->dtype);
  if (s->d_in % v != 0 || s->d_out % v != 0) return LORA_ERR_UNSUPPORTED;
  if ((s->A_pack && !aligned16(s->A_pack)) || (s->B_pack && !aligned16(s->B_pack)))
    return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int check_segment_args(const int32_t* ids, int T, int n, const int32_t* seg_off, const int32_t* perm) {
  if (T < 0 || n < 1) return LORA_ERR_INVALID_ARG;
  if (seg_off == nullptr) return LORA_ERR_INVALID_ARG;
  if (T > 0 && (ids == nullptr || perm == nullptr)) return LORA_ERR_INVALID_ARG;
  if (T > LORA_SEGMENT_MAX_T || n > LORA_SEGMENT_MAX_N) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int check_grouping(const lora_store* s, int T, const int32_t* seg_off, const int32_t* perm) {
  if (T < 0) return LORA_ERR_INVALID_ARG;
  if (seg_off == nullptr) return LORA_ERR_INVALID_ARG;
  if (T > 0 && perm == nullptr) return LORA_ERR_INVALID_ARG;
  if (s->n > LORA_SEGMENT_MAX_N) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

size_t workspace_bytes(const lora_store* s, int T) {
  if (s == nullptr || T < 0 || s->n < 1 || s->d_in <= 0 || s->r_max < 0) return 0;
  return ws_layout(T, s->n, s->d_in, s->r_max, s->dtype).total;
}

int check_ws(const lora_store* s, int T, const void* ws, size_t ws_bytes) {
  if (T == 0) return LORA_OK;  // nothing is launched
  if (ws == nullptr) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < workspace_bytes(s, T)) return LORA_ERR_INVALID_ARG;
  if (ws && !aligned16(ws)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int check_rows(const void* p, int64_t ld, int d, int dtype, int T) {
  if (T > 0 && p == nullptr) return LORA_ERR_INVALID_ARG;
  if (ld < d) return LORA_ERR_INVALID_ARG;
  if (p && !aligned16(p)) return LORA_ERR_UNSUPPORTED;
  if (ld % vec_elems(dtype) != 0) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int check_h(const float* h, int64_t ldh, const lora_store* s, int T) {
  if (T > 0 && h == nullptr) return LORA_ERR_INVALID_ARG;
  if (ldh < s->r_max || ldh < 1) return LORA_ERR_INVALID_ARG;
  if (h && ((uintptr_t)h & 3u)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

}  // namespace lora
