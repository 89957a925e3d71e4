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

// The shrink's workgroup: W waves share one work item (a sub-tile and a chunk
// of d_in), each wave taking an equal span of the chunk, and their float32
// sums meet in LDS.  W = 8 (two workgroups per CU, so one's reduction
// overlaps the other's loads), or 4 in the calls that shrink_split gives one
// chunk per sub-tile for their size or their shape.  Measured on the
// fleet's decode step, whose projections run on concurrent streams: 4 waves
// took the step from 13.91 to 13.59 ms, while each shrink timed alone on one
// stream stayed at 29.1 us on average; the smaller workgroups fit beside the
// other streams' kernels.  In smaller calls (decode spectral, two chunks per
// sub-tile) 4 waves were slower, 25.6 -> 28.2 us per shrink: each wave's span
// doubles, and so do its batches of loads.
constexpr int kShrinkWavesMax = 8;

// The grouping kernel (one workgroup: a stable counting sort of the ids and
// the sub-tile plan, in LDS) handles T <= kGroupMaxT and n <= kGroupMaxN;
// larger groupings use the radix sort and a plan kernel.
constexpr int kGroupMaxN = 2048;
constexpr int kGroupMaxT = 8192;
constexpr int kGroupWaves = 8;

// The expand's wave covers kExpandCols output features of one sub-tile.
constexpr int kExpandCols = 128;
// Waves per expand workgroup.  The waves share nothing (no LDS, no
// barriers), so this only sets the dispatch granularity.  Measured with 4,
// 2 and 1: the fleet's 5S step took 13.59, 13.08 and 14.28 ms, the expand
// averaged 45.4, 42.8 and 49.7 us over its 196 modules, and decode
// spectral's expand took 28.8, 27.7 and 26.8 us.  Two waves are kept.
constexpr int kExpandWaves = 2;
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
// In the expand's run form (calls of kExpandRunMinItems items or more, 3
// waves per SIMD), bf16 sub-tiles up to rank kVecMaxRankRun take the vector
// path too: its registers fit there (at 4 waves per SIMD they would spill),
// and ranks 9..16 of few tokens then stop filling 16 x 16 matrix tiles
// with one or two rows (fleet step 14.79 -> 14.15 ms).
constexpr int kVecMaxRankRun = 16;
constexpr int kVecMaxTokens = 8;
constexpr int kVecTokens = 4;
constexpr int kVecCols = 512;
// Sub-tiles of at most kGemvMaxTokens tokens and rank at most kVecMaxRank
// (bf16; half that for float32) take the shrink's wavefront-reduction path:
// lanes split d_in, every load is a fully used 16-byte chunk of x or A, and
// the r x m dot products are reduced across the wave at the end.  The
// others take its matrix-core path (16x16 tiles of ranks x tokens).
constexpr int kGemvMaxTokens = 4;

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

// The plan of a grouping: its sub-tiles in grouped order (adapters
// ascending, tokens ascending inside an adapter).  It depends on the
// grouping only, so one plan serves every store of the same adapters (all
// the projections of a decode step).  A 256-byte header (int32 [0] = number
// of sub-tiles, [1] = T, [2] = n), then one 128-byte entry per sub-tile.
struct TileEntry {
  int32_t a;     // adapter
  int32_t pos0;  // grouped position of the first token
  int32_t m;     // tokens (1..kSubTile)
  int32_t j;     // index of the sub-tile among its adapter's
  int32_t pad0[4];
  int32_t tok[kSubTile];  // token indices, ascending; -1 past m
  int32_t pad1[8];
};
static_assert(sizeof(TileEntry) == 128, "entry is one 128-byte line");
constexpr size_t kPlanHeaderBytes = 256;
inline size_t plan_bytes(int T, int n) {
  return kPlanHeaderBytes + sizeof(TileEntry) * (size_t)plan_max_subtiles(T, n);
}

// A call's own view of each sub-tile: the store's values for its adapter
// (written by the shrink, read by the expand, so that the expand's loads of
// B, h and y need no dependent metadata load).
struct TileMeta {
  int32_t r;        // stored rank (0: the adapter adds nothing)
  int32_t row_off;  // first row of the adapter in the store
  float scale;      // s_a
  int32_t S;        // partial sums of h (K chunks of the shrink)
};
static_assert(sizeof(TileMeta) == 16, "one 16-byte load");

// Multi-slice apply: per sub-tile and slice, the slice's rank, row offset and
// scale for the sub-tile's adapter and the first column of its h among the
// stacked ranks, written by the stacked store's shrink, so that a slice's
// expand reads them with the plan entry (one round trip) instead of after it.
struct SliceMeta {
  int32_t r, row_off;
  float scale;
  int32_t hoff;
};
static_assert(sizeof(SliceMeta) == 16, "one 16-byte load");

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int elem_bytes(int dtype) { return dtype == LORA_DTYPE_BF16 ? 2 : 4; }
inline int vec_elems(int dtype) { return dtype == LORA_DTYPE_BF16 ? 8 : 4; }  // 16-byte vectors

// The shrink cuts d_in into S <= kMaxChunks chunks, one workgroup item per
// (sub-tile, chunk).  A unit is 8 waves x 8 matrix-core K steps of 64
// bytes per row (256 bf16, 128 float32 values per wave); with 8 waves one
// batch of loads covers a unit at ranks up to 16 (two or three batches
// above).  Smaller chunks for
// higher ranks, to even out the items' bytes, were measured slower (decode
// spectral and prefill: more partial sums for the expand, no better
// balance).  A call that can hold kOneChunkMinSubtiles sub-tiles or more
// has items enough to fill the GPU with one chunk per sub-tile: an input of
// up to two units then goes in one chunk (half the items, one partial sum
// per h value; the fleet's decode step 15.36 -> 14.75 ms), while a smaller
// call keeps two chunks for more items in flight (decode spectral: 64.5
// against 68.2 us with one).  S depends on d_in, T and n only, so it is the
// same for every sub-tile of a call.  The last chunk may be shorter.
constexpr int kMaxChunks = 8;
struct ShrinkSplit {
  int kchunk;  // K elements per chunk
  int waves;   // waves per workgroup (8, or 4 for one chunk per sub-tile)
  int span;    // K elements per wave (kchunk / waves)
  int S;       // chunks (partial sums per h value)
};
constexpr int64_t kOneChunkMinSubtiles = 1024;
inline ShrinkSplit shrink_split(int d_in, int dtype, int T, int n) {
  const int unit = kShrinkWavesMax * 8 * 4 * vec_elems(dtype);  // 2048 bf16, 1024 float32
  const int units = (d_in + unit - 1) / unit;
  int mult = (units + kMaxChunks - 1) / kMaxChunks;
  // Large calls, and calls with at least a full sub-tile per adapter on
  // average (prefill: its sub-tiles are full, so its items are too): measured
  // on prefill (T = 8192, 32 adapters), one chunk and 4 waves took the call
  // from 159.0 to 153.3 us (the expand sums one partial, not two: 110.8 ->
  // 106.4 us); on decode spectral (T = 2048, 512 adapters, mostly partial
  // sub-tiles) the same split was slower, 61.9 -> 66.0 us.
  const bool large = plan_max_subtiles(T, n) >= kOneChunkMinSubtiles || (int64_t)T >= (int64_t)kSubTile * n;
  if (units <= 2 && large) mult = units;
  if (mult < 1) mult = 1;
  ShrinkSplit sp;
  sp.kchunk = mult * unit;
  sp.waves = large ? 4 : kShrinkWavesMax;
  sp.span = sp.kchunk / sp.waves;
  sp.S = (d_in + sp.kchunk - 1) / sp.kchunk;
  if (sp.S < 1) sp.S = 1;
  return sp;
}

// Row stride (floats) of the float32 partial sums: r_max rounded up to 8 so
// that every 8-value rank chunk a lane reads lies inside its row.
inline int64_t partial_ld(int r_max) { return (int64_t)align_up((size_t)(r_max < 1 ? 1 : r_max), 8); }

// Workspace of shrink / expand / apply, each part 256-byte aligned:
//   tile meta [max_sub] | partial sums [S][T][ldp] float32 | plan |
//   seg_off [n+2] | perm [T]
// The plan, seg_off and perm parts hold the grouping a call forms itself
// (from ids, or a plan from a caller's seg_off / perm); a call given a plan
// leaves them unused.
struct WsLayout {
  size_t meta, part, plan, seg_off, perm, hs, total;
};
inline WsLayout ws_layout(int T, int n, int d_in, int r_max, int dtype) {
  WsLayout L;
  const ShrinkSplit sp = shrink_split(d_in, dtype, T, n);
  L.meta = 0;
  L.part = align_up(sizeof(TileMeta) * (size_t)plan_max_subtiles(T, n), 256);
  L.plan = L.part + align_up((size_t)sp.S * (size_t)T * (size_t)partial_ld(r_max) * 4, 256);
  L.seg_off = L.plan + align_up(plan_bytes(T, n), 256);
  L.perm = L.seg_off + align_up((size_t)(n + 2) * 4, 256);
  L.hs = L.perm + align_up((size_t)T * 4, 256);
  // The base-fused apply's s h as bf16 pairs hi, lo: [T][2][ldp].
  L.total = L.hs + align_up((size_t)T * (size_t)partial_ld(r_max) * 4, 256);
  return L;
}

// The multi-slice apply's workspace: the stacked store's, then the slice
// records [n_slices][plan_max_subtiles].
inline size_t slice_meta_bytes(int T, int n, int n_slices) {
  return align_up(sizeof(SliceMeta) * (size_t)plan_max_subtiles(T, n) * (size_t)n_slices, 256);
}

// Meta buffer of a store: row_off[n+1] | rank[n] (stored) | scale[n] |
// true_rank[n] (before padding) | (16-aligned) A pointers[n] | B pointers[n].
inline size_t meta_ptr_offset(int n) { return align_up((size_t)(4 * (size_t)n + 1) * 4, 16); }
inline size_t meta_bytes(int n) { return meta_ptr_offset(n) + 16 * (size_t)n; }

}  // namespace lora
