// Internal sizes and layouts shared by the host dispatcher, the validation
// code and the kernels.  No HIP types: also compiled by the host-only
// validator.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/lora.h"

namespace lora {

// A sub-tile is a run of at most kSubTile tokens of one adapter in grouped
// order: one 16-wide block of a matrix-core tile.
constexpr int kSubTile = 16;

// The shrink's workgroup: 8 waves share one (sub-tile, K chunk) item; two
// workgroups fit on a CU, so one's grouping and reduction overlap the
// other's loads.
constexpr int kShrinkWaves = 8;
constexpr int kShrinkThreads = kShrinkWaves * 64;

// The shrink groups tokens itself (histogram of the ids in LDS) when
// n <= kGroupMaxN; beyond that the apply first runs the single-workgroup sort.
constexpr int kGroupMaxN = 4096;

// The expand's wave covers kExpandCols output features of one sub-tile.
constexpr int kExpandCols = 128;
constexpr int kExpandWaves = 4;  // waves per expand workgroup
// Feature blocks one matrix-path expand wave takes in turn (a run): its
// sub-tile's tokens and h are read once, and each block's y rows are
// issued before the previous block is computed.  Measured against 4 and 8
// (prefill, fleet): 2 is as fast or faster.
constexpr int kExpandRun = 2;
// One-block items (sub-tiles x feature blocks) from which a call uses runs:
// about 16 times the waves the GPU holds at 3 per SIMD.
constexpr int64_t kExpandRunMinItems = 48 * 1024;
// Sub-tiles of at most kVecMaxTokens tokens and rank at most kVecMaxRank
// (bf16; half that for float32) take the vector path of the expand: one wave
// per (sub-tile, kVecCols output features, group of kVecTokens tokens); the
// others its matrix-core path.
constexpr int kVecMaxRank = 8;
constexpr int kVecMaxTokens = 8;
constexpr int kVecTokens = 4;
constexpr int kVecCols = 512;

// A batched apply with ids of at most kDecodeMaxT tokens over a store of
// rank <= kVecMaxRank whose d_in is one 16-byte chunk per thread of a
// 512-thread workgroup runs as one launch, a workgroup per token (the
// adapter's A and B are then read once per token, from cache after the
// first: worth it while tokens per adapter stay few).
constexpr int kDecodeMaxT = 512;

// Upper bound on the number of runs of at most `len` tokens that T tokens
// over n adapters cut into: each non-empty group of c tokens gives
// ceil(c / len) runs and at most min(n, T) groups are non-empty.
inline int64_t plan_max_runs(int T, int n, int len) {
  if (T <= 0 || n <= 0) return 0;
  int64_t k = n < T ? n : T;
  return ((int64_t)T + (int64_t)(len - 1) * k) / len;
}
inline int64_t plan_max_subtiles(int T, int n) { return plan_max_runs(T, n, kSubTile); }

// The work plan: a 256-byte header (int32 [0] = number of sub-tiles), then
// one 128-byte entry per sub-tile, in adapter order.  Written by the shrink
// (or by the plan kernel) and read by the expand and the partial-sum reduce.
struct TileEntry {
  int32_t a;        // adapter
  int32_t pos0;     // grouped position of the first token
  int32_t m;        // tokens (1..kSubTile)
  int32_t r;        // stored rank
  int32_t row_off;  // first row of the adapter in the store
  float scale;      // s_a
  int32_t S;        // K chunks of the shrink (partial sums to add)
  int32_t pad0;
  int32_t tok[kSubTile];  // token indices, ascending
  int32_t pad1[8];
};
static_assert(sizeof(TileEntry) == 128, "entry is one 128-byte line");
constexpr size_t kPlanHeaderBytes = 256;
inline size_t plan_bytes(int T, int n) {
  return kPlanHeaderBytes + sizeof(TileEntry) * (size_t)plan_max_subtiles(T, n);
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int elem_bytes(int dtype) { return dtype == LORA_DTYPE_BF16 ? 2 : 4; }
inline int vec_elems(int dtype) { return dtype == LORA_DTYPE_BF16 ? 8 : 4; }  // 16-byte vectors

// The shrink splits d_in into S <= kMaxChunks chunks; each of the 8 waves of an item
// takes `spw` consecutive K steps (a step is 4 x 16 bytes of K: 32 bf16 or
// 16 f32 values), issued as one batch of loads.  The batch depends on the
// adapter's number of 16-rank row groups (ng): 8, 5, 4, 3 steps for ng =
// 1..4, about 60 registers of loads either way.  S is at most 8; very wide
// inputs give more steps per wave (several batches).  Indexed by ng (1..4).
constexpr int kMaxChunks = 8;
struct ShrinkSplit {
  int spw[5];     // K steps per wave
  int S[5];       // K chunks (partial sums per output)
  int kchunk[5];  // K elements per chunk = 8 * spw * step
  int S_max;      // largest S over the row groups the store needs
};
inline int shrink_batch_steps(int ng) { return ng <= 1 ? 8 : ng == 2 ? 5 : ng == 3 ? 4 : 3; }
inline int rank_groups(int r) { return r <= 16 ? 1 : (r + 15) / 16; }
inline ShrinkSplit shrink_split(int d_in, int r_max, int dtype) {
  const int step = 4 * vec_elems(dtype);
  const int steps = (d_in + step - 1) / step;
  ShrinkSplit sp;
  sp.spw[0] = sp.S[0] = sp.kchunk[0] = 0;
  sp.S_max = 1;
  for (int ng = 1; ng <= 4; ++ng) {
    int spw = shrink_batch_steps(ng);
    int S = (steps + kShrinkWaves * spw - 1) / (kShrinkWaves * spw);
    if (S > kMaxChunks) {
      spw = (steps + kShrinkWaves * kMaxChunks - 1) / (kShrinkWaves * kMaxChunks);
      S = (steps + kShrinkWaves * spw - 1) / (kShrinkWaves * spw);
    }
    sp.spw[ng] = spw;
    sp.S[ng] = S;
    sp.kchunk[ng] = kShrinkWaves * spw * step;
    if (ng <= rank_groups(r_max) && S > sp.S_max) sp.S_max = S;
  }
  return sp;
}

// Row stride (floats) of the float32 partial sums: r_max rounded up to 8 so
// that every 8-value rank chunk a lane reads lies inside its row.
inline int64_t partial_ld(int r_max) { return (int64_t)align_up((size_t)(r_max < 1 ? 1 : r_max), 8); }

// Workspace of shrink / expand / apply, each part 256-byte aligned:
//   plan | partial sums [S][T][ldp] float32 | seg_off [n+2] | perm [T]
// (the last two only when the apply has to sort: n > kGroupMaxN).
struct WsLayout {
  size_t plan, part, seg_off, perm, total;
};
inline WsLayout ws_layout(int T, int n, int d_in, int r_max, int dtype) {
  WsLayout L;
  const ShrinkSplit sp = shrink_split(d_in, r_max, dtype);
  L.plan = 0;
  L.part = align_up(plan_bytes(T, n), 256);
  L.seg_off = L.part + align_up((size_t)sp.S_max * (size_t)T * (size_t)partial_ld(r_max) * 4, 256);
  L.perm = L.seg_off + (n > kGroupMaxN ? align_up((size_t)(n + 2) * 4, 256) : 0);
  L.total = L.perm + (n > kGroupMaxN ? align_up((size_t)T * 4, 256) : 0);
  return L;
}

// Meta buffer of a store: row_off[n+1] | rank[n] (stored) | scale[n] |
// true_rank[n] (before padding) | (16-aligned) A pointers[n] | B pointers[n].
inline size_t meta_ptr_offset(int n) { return align_up((size_t)(4 * (size_t)n + 1) * 4, 16); }
inline size_t meta_bytes(int n) { return meta_ptr_offset(n) + 16 * (size_t)n; }

}  // namespace lora
