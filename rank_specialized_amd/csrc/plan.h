// Internal sizes shared by the host dispatcher and the validation code.
// No HIP types: this header is also compiled by the host-only validator.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/lora.h"

namespace lora {

constexpr int kTile = LORA_TILE_TOKENS;  // tokens per work tile

// Tiles of more than kSmallTile tokens take the matrix-core expand path;
// smaller ones (decode) take the vector path.
constexpr int kSmallTile = 4;
// The shrink works on sub-tiles of at most kSubTile tokens (one MFMA column
// block), so that every shrink workgroup moves a similar amount of data.
constexpr int kSubTile = 16;

// Upper bound on the number of runs of at most `len` tokens that T tokens
// over n adapters cut into: each non-empty group of c tokens gives
// ceil(c / len) runs and at most min(n, T) groups are non-empty.
inline int64_t plan_max_runs(int T, int n, int len) {
  if (T <= 0 || n <= 0) return 0;
  int64_t k = n < T ? n : T;
  return ((int64_t)T + (int64_t)(len - 1) * k) / len;
}
inline int64_t plan_max_tiles(int T, int n) { return plan_max_runs(T, n, kTile); }
inline int64_t plan_max_subtiles(int T, int n) { return plan_max_runs(T, n, kSubTile); }

// Plan layout: int32 header[16], then the expand tiles, then the shrink
// sub-tiles; every entry is int4 {adapter, first grouped position, tokens, 0}.
//   header[0] = expand tiles, header[1] = large ones (tokens > kSmallTile,
//   listed first), header[2] = small ones, header[3] = shrink sub-tiles.
constexpr size_t kPlanHeaderBytes = 64;
inline size_t plan_subtile_offset(int T, int n) {
  return kPlanHeaderBytes + 16 * (size_t)plan_max_tiles(T, n);
}
inline size_t plan_bytes(int T, int n) {
  if (T < 0 || n < 0) return 0;
  return plan_subtile_offset(T, n) + 16 * (size_t)plan_max_subtiles(T, n);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int elem_bytes(int dtype) { return dtype == LORA_DTYPE_BF16 ? 2 : 4; }
inline int vec_elems(int dtype) { return dtype == LORA_DTYPE_BF16 ? 8 : 4; }  // 16-byte vectors

// Meta buffer of a store: row_off[n+1] | rank[n] (stored) | scale[n] |
// true_rank[n] (before padding) | (16-aligned) A pointers[n] | B pointers[n].
inline size_t meta_ptr_offset(int n) { return align_up((size_t)(4 * (size_t)n + 1) * 4, 16); }
inline size_t meta_bytes(int n) { return meta_ptr_offset(n) + 16 * (size_t)n; }

// h leading dimension used inside lora_apply_batched.
inline int64_t apply_ldh(int r_max) { return r_max < 4 ? 4 : (int64_t)align_up((size_t)r_max, 4); }

}  // namespace lora
