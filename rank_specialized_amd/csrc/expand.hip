// Expand: y[t, o] += s_a * sum_{j < r_a} B_a[o, j] h[t, j].
//
// Step 3 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4: B applied with the
// adapter's scale and added into (a slice of) y.  Accumulation in float32,
// one rounding of the new y value to the output type.
//
// Work item = one wave: (sub-tile, 128 output features).  Waves are
// independent (no barriers); every wave issues its y rows and its B rows
// before any arithmetic, so an item costs one memory round trip (two for
// bf16 ranks above 32, whose second K chunk of B is read after the first).
// In calls of at least kExpandRunMinItems such items a wave takes a run of
// kExpandRun consecutive feature blocks of its sub-tile instead: tokens and
// h are read once, and each block's y rows are issued before the previous
// block's products, so the next block's loads overlap this block's work.  In
// that form two consecutive sub-tiles of one adapter (ranks of one K chunk)
// pair up: their waves take one feature block each, for both sub-tiles, so
// B's rows are read once for the two (prefill expand 120 -> 114 us).
//   D[token, feature] = H[token, j] . B_a^T[j, feature]
// on 16x16 MFMA tiles (bf16: 16x16x32, f32: 16x16x4), eight N blocks per
// wave.  Column c of N block b is feature o0 + 8 c + b, so lane (c, g) ends
// with features o0 + 8c .. o0 + 8c + 7 of tokens 4g .. 4g + 3: a y row is
// read and written as 256 contiguous bytes by 16 lanes.  The B operand of
// lane (c, g) in block b is 16 contiguous bytes of row o0 + 8c + b of B_a
// (ranks 32 q + 8 g ..), read straight from the store: B_a is kept in its
// own [d_out, r_a] orientation, so a wave reads 128 consecutive rows of B_a,
// one contiguous run of the store.  Ranks >= r_a are masked to zero (a lane
// whose chunk starts at or past r_a loads nothing).
//   h is float32 and enters the bf16 matrix core as the exact sum of two bf16
// values (hi + lo), keeping about 16 significant bits; with the shrink's
// partial sums (S chunks of d_in) added first, in chunk order.
//
// Rank specialization: the number of 32-deep (bf16) or 16-deep (f32) K
// chunks is a template parameter; a tile of rank r_a issues exactly the loads
// and MFMAs of ceil(r_a / 32) chunks.
//
// Decode sub-tiles (at most 8 tokens, rank at most 8 in bf16 or 4 in
// float32) take the vector path
// instead: one wave per (sub-tile, 512 output features, 4 tokens).  Lane l
// owns features o .. o + 7 (o = 512 fb + 8 l); in the [d_out, r] layout their
// B values are 16 r contiguous bytes, read as r fully used 16-byte loads.
// h[t, j] is held by lane t r + j and broadcast with a lane read; each output
// is y + s * sum_j h[t, j] B[o + f, j] in float32 (h exact, no bf16 split).
// The path is instantiated per exact rank, so the unpacking of the B block
// is static.  Both paths live in one kernel: a sub-tile owns `slots`
// consecutive waves and its entry decides which path they take (waves a path
// does not need return at once), so the plan is read in one launch.  A
// sub-tile's rank, row offset, scale and partial count come from the
// metadata the shrink recorded beside the plan, read with the entry.
#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {

struct ExpandArgs {
  // The plan and the metadata first: a wave's first loads need both.
  const char* plan;
  const TileMeta* meta;  // per sub-tile: rank, row offset, scale, partial count (from the shrink)
  const char* b_pack;
  int d_out, T, max_sub;
  int slots;  // waves per sub-tile: max(fbn, (kVecMaxTokens / kVecTokens) fbv)
  int fbn;    // kExpandCols-feature blocks (matrix path)
  int fbv;    // kVecCols-feature blocks (vector path)
  int n, r_max, R, S_max;  // the store's bounds: plan entries outside them are skipped
  const float* hsrc;      // partial sums (kPart) or h
  int64_t ldh, hstride;   // floats
  char* y;
  int64_t ldy_bytes;
  // Slice mode (multi-slice apply): the plan and partial sums come from the
  // shrink of a stacked store (the bounds above are that store's); B comes
  // from the slice's store, and its rank, row offset, scale and h column
  // (among the stacked ranks) from the records the stacked shrink wrote,
  // checked against the slice store's bounds.
  const SliceMeta* sl_meta;  // [max_sub]: this slice's records
  int sl_r_max, sl_R;
};

// The H operand chunk of one lane: h[hrow, j0 .. j0 + V) of the rows the
// expand reads (the S partial sums added in chunk order, or h), zero past
// the rank and for a row that is not valid.
template <typename E, bool kPart>
__device__ __forceinline__ HChunk<E> h_chunk(const ExpandArgs& p, int hrow, bool valid, int j0, int r, int S, int hoff) {
  constexpr int V = E::kVec;
  float f[V];
#pragma unroll
  for (int e = 0; e < V; ++e) f[e] = 0.f;
  if (valid && hrow >= 0 && hrow < p.T && j0 < r) {
    const float* src = p.hsrc + (int64_t)hrow * p.ldh + hoff + j0;
    // A slice's columns (multi-slice apply) may start off a 16-byte
    // boundary, or end so that a whole vector would run past the row of
    // partial sums: those are read column by column, only below the rank.
    const bool whole = (hoff & 3) == 0 && hoff + j0 + V <= p.ldh;
    if (kPart && !whole) {
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = j0 + e < r ? src[e] : 0.f;
#pragma unroll 4
      for (int k = 1; k < S; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (j0 + e < r) f[e] += src[(int64_t)k * p.hstride + e];
    } else if (kPart) {
#pragma unroll
      for (int v = 0; v < V / 4; ++v) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 4 * v);
        f[4 * v] = x[0]; f[4 * v + 1] = x[1]; f[4 * v + 2] = x[2]; f[4 * v + 3] = x[3];
      }
#pragma unroll 4
      for (int k = 1; k < S; ++k) {
#pragma unroll
        for (int v = 0; v < V / 4; ++v) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + (int64_t)k * p.hstride + 4 * v);
          f[4 * v] += x[0]; f[4 * v + 1] += x[1]; f[4 * v + 2] += x[2]; f[4 * v + 3] += x[3];
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (j0 + e >= r) f[e] = 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = j0 + e < r ? src[e] : 0.f;
    }
  }
  HChunk<E> h;
  h.set(f);
  return h;
}

template <typename E, bool kPart, int NQ, int RUN>
__device__ __forceinline__ void expand_run(const ExpandArgs& p, const int4& tk4, int m, int r, int pos0,
                                           int ro, float sc, int S, int fb0, int nb, int hoff) {
  constexpr int V = E::kVec;
  constexpr int KSTEP = 4 * V;  // ranks per K chunk
  constexpr int YV = 8 / V;     // 16-byte vectors per 8 features: bf16 1, f32 2
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // Rows of tokens 4g .. 4g + 3 (nullptr: no token), the same for every
  // feature block of the run.
  // tk4: tokens 4g .. 4g + 3 of the sub-tile, read with the entry.
  const int tkv[4] = {tk4.x, tk4.y, tk4.z, tk4.w};
  const char* yrow[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int tok = 4 * g + e < m ? tkv[e] : -1;
    yrow[e] = (unsigned)tok < (unsigned)p.T ? p.y + (int64_t)tok * p.ldy_bytes : nullptr;
  }
  auto feat = [&](int k) { return (fb0 + k) * kExpandCols + 8 * c; };  // first feature of the lane in block k
  auto load_y = [&](int o, uint4(&yv)[4][YV]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int v = 0; v < YV; ++v)
        yv[e][v] = (yrow[e] && o + v * V < p.d_out) ? ld16_stream(yrow[e] + (size_t)(o + v * V) * E::kBytes) : zero;
  };
  // B rows o .. o + 7 (one per N block), ranks of this lane's K chunks.
  // bf16 rows of an odd rank start on 2-byte boundaries, and a 16-byte
  // buffer load must start on a 4-byte one: such a chunk (row o + b odd,
  // i.e. N block b odd, the same for every lane) is read from the dword below
  // plus one more dword, and shifted down by 16 bits.
  const uint32_t row_bytes = (uint32_t)r * E::kBytes;
  const rsrc_t br = make_rsrc(p.b_pack + (size_t)ro * p.d_out * E::kBytes, (uint32_t)p.d_out * row_bytes);
  const bool odd_rows = E::kBytes == 2 && (r & 1);
  auto load_b = [&](int q, int o, uint4(&bb)[8]) {
    const int j0 = q * KSTEP + g * V;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool ok = j0 < r && o + b < p.d_out;
      const uint32_t off = (uint32_t)(o + b) * row_bytes + (uint32_t)j0 * E::kBytes;
      if ((b & 1) && odd_rows) {
        const uint32_t lo = ok ? off - 2 : kOutOfRange;
        const uint4 d = buf_ld16(br, lo, 0);
        const uint32_t t = buf_ld4(br, ok ? lo + 16 : kOutOfRange);
        bb[b] = make_uint4(__builtin_amdgcn_alignbit(d.y, d.x, 16), __builtin_amdgcn_alignbit(d.z, d.y, 16),
                           __builtin_amdgcn_alignbit(d.w, d.z, 16), __builtin_amdgcn_alignbit(t, d.w, 16));
      } else {
        bb[b] = buf_ld16(br, ok ? off : kOutOfRange, 0);
      }
    }
  };
  // First block's y rows, B rows, then the H chunks (read once for the
  // whole run).  One block per wave issues its y rows first (the longest
  // wait); a run issues them after B and h instead, so that its first
  // products need not wait for them (prefill's expand 122.4 -> 119.0 us; one
  // block per wave was slower that way).
  uint4 ya[4][YV], yb[4][YV];
  if constexpr (RUN == 1) load_y(feat(0), ya);
  // bf16 ranks above 32 take two K chunks.  The second chunk's B rows are
  // loaded after the first chunk's products, into the same registers: the
  // kernel then fits the registers of 4 waves per SIMD, for one more (mostly
  // L2) round trip on those sub-tiles only.
  constexpr int NB = (E::kBytes == 2 && NQ > 1) ? 1 : NQ;  // chunks loaded up front
  uint4 bq[NB][8];
#pragma unroll
  for (int q = 0; q < NB; ++q) load_b(q, feat(0), bq[q]);
  // H chunks: token c of the sub-tile, ranks j0 .. j0 + V.
  HChunk<E> hc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) hc[q] = h_chunk<E, kPart>(p, pos0 + c, c < m, q * KSTEP + g * V, r, S, hoff);
  if constexpr (RUN > 1) load_y(feat(0), ya);
  // The run: block k's products and stores, with block k + 1's y rows
  // issued before block k is waited for (its B rows first: waits are in
  // issue order, so the next block's y loads must come after what block k
  // needs).
#pragma unroll
  for (int k = 0; k < RUN; ++k) {
    if (k >= nb) break;
    const int o = feat(k);
    uint4(&ycur)[4][YV] = (k & 1) ? yb : ya;
    uint4(&ynxt)[4][YV] = (k & 1) ? ya : yb;
    if (k > 0) {
#pragma unroll
      for (int q = 0; q < NB; ++q) load_b(q, o, bq[q]);
    }
    if (k + 1 < nb) load_y(feat(k + 1), ynxt);
    f32x4_t acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q >= NB) {
        __builtin_amdgcn_sched_barrier(0);  // not above the previous chunk's products
        load_b(q, o, bq[NB - 1]);
      }
      const int nvalid = r - (q * KSTEP + g * V);
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[b] = hc[q].mma(keep_first<E>(bq[q < NB ? q : NB - 1][b], nvalid), acc[b]);
    }
    // acc[b][e] = feature o + b of token 4g + e.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (yrow[e] == nullptr) continue;
      char* yp = const_cast<char*>(yrow[e]) + (size_t)o * E::kBytes;
#pragma unroll
      for (int v = 0; v < YV; ++v) {
        if (o + v * V >= p.d_out) continue;
        float f[V];
        E::widen(ycur[e][v], f);
#pragma unroll
        for (int kk = 0; kk < V; ++kk) f[kk] = f[kk] + sc * acc[v * V + kk][e];
        st16_stream(yp + 16 * v, E::narrow(f));
      }
    }
  }
}

// Run form, a pair: consecutive sub-tiles a and b of one adapter (ranks of
// one K chunk) over one block of kExpandCols features.  B's rows of the block
// are read once for both sub-tiles; the lane layout, the order of operations
// and the results are those of the one-sub-tile form.
template <typename E, bool kPart>
__device__ __forceinline__ void expand_pair(const ExpandArgs& p, const int4& tka, const int4& tkb, int ma, int pa,
                                            int mb, int pb, int r, int ro, float sc, int S, int fb) {
  constexpr int V = E::kVec;
  constexpr int YV = 8 / V;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  const int o = fb * kExpandCols + 8 * c;
  const int tkv[2][4] = {{tka.x, tka.y, tka.z, tka.w}, {tkb.x, tkb.y, tkb.z, tkb.w}};
  const int mk[2] = {ma, mb};
  const char* yrow[2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = 4 * g + e < mk[k] ? tkv[k][e] : -1;
      yrow[k][e] = (unsigned)tok < (unsigned)p.T ? p.y + (int64_t)tok * p.ldy_bytes : nullptr;
    }
  // Both sub-tiles' y rows first (the longest wait), then B, then h.
  uint4 yv[2][4][YV];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int v = 0; v < YV; ++v)
        yv[k][e][v] = (yrow[k][e] && o + v * V < p.d_out) ? ld16_stream(yrow[k][e] + (size_t)(o + v * V) * E::kBytes)
                                                          : zero;
  const uint32_t row_bytes = (uint32_t)r * E::kBytes;
  const rsrc_t br = make_rsrc(p.b_pack + (size_t)ro * p.d_out * E::kBytes, (uint32_t)p.d_out * row_bytes);
  const bool odd_rows = E::kBytes == 2 && (r & 1);
  const int j0 = g * V;
  uint4 bq[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool ok = j0 < r && o + b < p.d_out;
    const uint32_t off = (uint32_t)(o + b) * row_bytes + (uint32_t)j0 * E::kBytes;
    if ((b & 1) && odd_rows) {
      const uint32_t lo = ok ? off - 2 : kOutOfRange;
      const uint4 d = buf_ld16(br, lo, 0);
      const uint32_t t = buf_ld4(br, ok ? lo + 16 : kOutOfRange);
      bq[b] = make_uint4(__builtin_amdgcn_alignbit(d.y, d.x, 16), __builtin_amdgcn_alignbit(d.z, d.y, 16),
                         __builtin_amdgcn_alignbit(d.w, d.z, 16), __builtin_amdgcn_alignbit(t, d.w, 16));
    } else {
      bq[b] = buf_ld16(br, ok ? off : kOutOfRange, 0);
    }
  }
  const HChunk<E> hc[2] = {h_chunk<E, kPart>(p, pa + c, c < ma, j0, r, S, 0),
                           h_chunk<E, kPart>(p, pb + c, c < mb, j0, r, S, 0)};
  const int nvalid = r - j0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    f32x4_t acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = hc[k].mma(keep_first<E>(bq[b], nvalid), f32x4_t{0.f, 0.f, 0.f, 0.f});
    // acc[b][e] = feature o + b of token 4g + e of sub-tile k.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (yrow[k][e] == nullptr) continue;
      char* yp = const_cast<char*>(yrow[k][e]) + (size_t)o * E::kBytes;
#pragma unroll
      for (int v = 0; v < YV; ++v) {
        if (o + v * V >= p.d_out) continue;
        float f[V];
        E::widen(yv[k][e][v], f);
#pragma unroll
        for (int kk = 0; kk < V; ++kk) f[kk] = f[kk] + sc * acc[v * V + kk][e];
        st16_stream(yp + 16 * v, E::narrow(f));
      }
    }
  }
}

// Sub-tile st checked against T and the store (metadata left in the
// workspace by a call on another store is skipped): every token, B row and
// partial sum it names then lies inside the call's buffers.
__device__ __forceinline__ bool entry_fits(const ExpandArgs& p, int a, int m, int pos0, const TileMeta& tm) {
  return (unsigned)a < (unsigned)p.n && m > 0 && m <= kSubTile && pos0 >= 0 && pos0 <= p.T - m && tm.r > 0 &&
         tm.r <= p.r_max && tm.row_off >= 0 && tm.row_off <= p.R - tm.r && tm.S > 0 && tm.S <= p.S_max;
}

// Whether sub-tiles s and s + 1 (heads e0, e1, metadata t0, t1) make a pair
// for the run form's matrix path: the adapter's sub-tiles j and j + 1 with j
// even, both valid with the same metadata, both on the matrix path at rank r
// of one K chunk.  The waves of both evaluate it on the same plan, so the
// pair's feature blocks are split between them without overlap.
template <typename E, int RUN>
__device__ __forceinline__ bool pair_ok(const ExpandArgs& p, int lim, int s, const int4& e0, const int4& e1,
                                        const TileMeta& t0, const TileMeta& t1, int r);

// ------------------------------------------------------------ vector path
// float32 B blocks are twice as large: that path stops at rank kVecMaxRank / 2.
template <typename E, int RUN>
constexpr int vec_rank_cap() {
  return (RUN > 1 && E::kBytes == 2) ? kVecMaxRankRun : kVecMaxRank * 2 / E::kBytes;
}
template <typename E, int RUN>
__device__ __forceinline__ bool vector_expand(int r, int m) {
  return r <= vec_rank_cap<E, RUN>() && m <= kVecMaxTokens;
}

template <typename E, int RUN>
__device__ __forceinline__ bool pair_ok(const ExpandArgs& p, int lim, int s, const int4& e0, const int4& e1,
                                        const TileMeta& t0, const TileMeta& t1, int r) {
  if (s < 0 || s + 1 >= lim) return false;
  if (e1.x != e0.x || (e0.w & 1) || e1.w != e0.w + 1) return false;
  if (!entry_fits(p, e0.x, e0.z, e0.y, t0) || !entry_fits(p, e1.x, e1.z, e1.y, t1)) return false;
  if (t0.r != t1.r || t0.row_off != t1.row_off || t0.S != t1.S || __float_as_int(t0.scale) != __float_as_int(t1.scale))
    return false;
  return r <= 4 * E::kVec && !vector_expand<E, RUN>(r, e0.z) && !vector_expand<E, RUN>(r, e1.z);
}

template <typename E, bool kPart, int R>
__device__ __forceinline__ void expand_vec_item(const ExpandArgs& p, const int4& tk4, int m, int t0,
                                                int pos0, int ro, float sc, int S, int o, int hoff) {
  constexpr int V = E::kVec;
  constexpr int YV = 8 / V;                   // 16-byte vectors per 8 features
  constexpr int BV = 8 * R * E::kBytes / 16;  // 16-byte vectors of the lane's 8 x R block of B
  const int lane = threadIdx.x & 63;
  const int mt = min(kVecTokens, m - t0);
  const int nf = min(8, p.d_out - o);  // 8; 4 for a float32 row of 4 (mod 8) features; <= 0 past the row
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // y rows of tokens t0 .. t0 + 3 and the B block, issued first.  The four
  // token indices were read with the entry: lane group t0 / 4 holds them.
  static_assert(kVecTokens == 4, "tokens t0 .. t0 + 3 are one lane group's");
  const int src = 16 * (t0 / 4);
  int tk[kVecTokens] = {__builtin_amdgcn_readlane(tk4.x, src), __builtin_amdgcn_readlane(tk4.y, src),
                        __builtin_amdgcn_readlane(tk4.z, src), __builtin_amdgcn_readlane(tk4.w, src)};  // -1: no row
  uint4 yv[kVecTokens][YV];
#pragma unroll
  for (int t = 0; t < kVecTokens; ++t) {
    tk[t] = (t < mt && (unsigned)tk[t] < (unsigned)p.T && nf > 0) ? tk[t] : -1;
    const char* yr = p.y + (int64_t)max(tk[t], 0) * p.ldy_bytes + (size_t)max(o, 0) * E::kBytes;
#pragma unroll
    for (int v = 0; v < YV; ++v) yv[t][v] = (tk[t] >= 0 && v * V < nf) ? ld16_stream(yr + 16 * v) : zero;
  }
  const char* bb = p.b_pack + ((size_t)ro * p.d_out + (size_t)o * R) * E::kBytes;
  uint4 bv[BV];
#pragma unroll
  for (int i = 0; i < BV; ++i) bv[i] = (16 * i < nf * R * E::kBytes) ? ld16(bb + 16 * i) : zero;
  // h[t, j] in lane t R + j (t < 4): the S partial sums in chunk order, or h.
  float hv = 0.f;
  {
    const int t = lane / R, j = lane - t * R;
    if (t < mt) {
      const int row = pos0 + t0 + t;
      if (row >= 0 && row < p.T) {
        const float* src = p.hsrc + (int64_t)row * p.ldh + hoff + j;
        // The S partial sums in chunk order (their loads issued together,
        // eight at a time), or h.
        hv = kPart ? sum_partials(src, p.hstride, S) : src[0];
      }
    }
  }
  float acc[kVecTokens][8];
#pragma unroll
  for (int t = 0; t < kVecTokens; ++t)
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[t][f] = 0.f;
  const uint32_t* bw = reinterpret_cast<const uint32_t*>(bv);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float bj[8];  // B[o + f, j]: element f R + j of the lane's block
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int e = f * R + j;
      if constexpr (E::kBytes == 2)
        bj[f] = (e & 1) ? bf16_hi(bw[e >> 1]) : bf16_lo(bw[e >> 1]);
      else
        bj[f] = __uint_as_float(bw[e]);
    }
#pragma unroll
    for (int t = 0; t < kVecTokens; ++t) {
      const float h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hv), t * R + j));
#pragma unroll
      for (int f = 0; f < 8; ++f) acc[t][f] += h * bj[f];
    }
  }
#pragma unroll
  for (int t = 0; t < kVecTokens; ++t) {
    if (tk[t] < 0) continue;
    char* yr = p.y + (int64_t)tk[t] * p.ldy_bytes + (size_t)o * E::kBytes;
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      if (v * V >= nf) continue;
      float f[V];
      E::widen(yv[t][v], f);
#pragma unroll
      for (int k = 0; k < V; ++k) f[k] = f[k] + sc * acc[t][v * V + k];
      st16_stream(yr + 16 * v, E::narrow(f));
    }
  }
}

// ------------------------------------------------------------ the kernel
template <typename E, bool kPart, bool kSlice, int RUN>
__device__ __forceinline__ void expand_wave(const ExpandArgs& p) {
  constexpr int KSTEP = 4 * E::kVec;
  constexpr int kGroups = kVecMaxTokens / kVecTokens;
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * kExpandWaves + (threadIdx.x >> 6));
  const int st = item / p.slots, slot = item - st * p.slots;
  // The plan's count, the entry's head and the metadata are all read before
  // the first test, so that they take one round trip (the index clamped into
  // the plan; the tests decide what is used).
  const int sc0 = min(st, p.max_sub - 1);
  const TileEntry* ent = reinterpret_cast<const TileEntry*>(p.plan + kPlanHeaderBytes) + sc0;
  const int count = *reinterpret_cast<const int32_t*>(p.plan);
  const int4 head = *reinterpret_cast<const int4*>(ent);  // a, pos0, m, j
  const TileMeta tm = p.meta[sc0];
  SliceMeta sm{0, 0, 0.f, 0};
  if constexpr (kSlice) sm = p.sl_meta[sc0];
  // Tokens 4g .. 4g + 3 in lane group g (an entry always holds 16).
  const int g4 = 4 * ((threadIdx.x & 63) >> 4);
  const int4 tk4 = *reinterpret_cast<const int4*>(ent->tok + g4);
  // Run form: the neighbours' heads, metadata and tokens too (a pair of
  // sub-tiles needs its partner's), in the same round trip.
  constexpr bool kPairs = RUN > 1 && !kSlice && E::kBytes == 2;
  int4 hp{}, hn{}, tkp{}, tkn{};
  TileMeta tp{}, tn{};
  if constexpr (kPairs) {
    const int sp = sc0 > 0 ? sc0 - 1 : sc0, sn = sc0 + 1 < p.max_sub ? sc0 + 1 : sc0;
    const TileEntry* ep = ent + (sp - sc0);
    const TileEntry* en = ent + (sn - sc0);
    hp = *reinterpret_cast<const int4*>(ep);
    hn = *reinterpret_cast<const int4*>(en);
    tp = p.meta[sp];
    tn = p.meta[sn];
    tkp = *reinterpret_cast<const int4*>(ep->tok + g4);
    tkn = *reinterpret_cast<const int4*>(en->tok + g4);
  }
  const int m = head.z, pos0 = head.y;
  if ((st >= p.max_sub) | (st >= count) | !entry_fits(p, head.x, m, pos0, tm)) return;
  const int S = kPart ? tm.S : 1;
  int r = tm.r, ro = tm.row_off, hoff = 0;
  float sc = tm.scale;
  if constexpr (kSlice) {  // slice mode: this slice's rank, B rows, scale and h columns
    const int r2 = sm.r, ro2 = sm.row_off, h2 = sm.hoff;
    if (r2 <= 0 || r2 > p.sl_r_max || ro2 < 0 || ro2 > p.sl_R - r2 || h2 < 0 || h2 > r - r2) return;
    r = r2;
    ro = ro2;
    hoff = h2;
    sc = sm.scale;
  }
  if (vector_expand<E, RUN>(r, m)) {
    const int fb = slot / kGroups, tg = slot - fb * kGroups;
    if (fb >= p.fbv || tg * kVecTokens >= m) return;
    // Every lane stays: lanes past d_out load and store nothing but may hold h.
    const int o = fb * kVecCols + 8 * (threadIdx.x & 63);
    const int t0 = tg * kVecTokens;
    switch (r) {
#define LORA_VEC_CASE(RR) \
  case RR: expand_vec_item<E, kPart, RR>(p, tk4, m, t0, pos0, ro, sc, S, o, hoff); break;
      LORA_VEC_CASE(1) LORA_VEC_CASE(2) LORA_VEC_CASE(3) LORA_VEC_CASE(4)
      LORA_VEC_CASE(5) LORA_VEC_CASE(6) LORA_VEC_CASE(7) LORA_VEC_CASE(8)
      default:
        if constexpr (vec_rank_cap<E, RUN>() > 8) {
          switch (r) {
            LORA_VEC_CASE(9) LORA_VEC_CASE(10) LORA_VEC_CASE(11) LORA_VEC_CASE(12)
            LORA_VEC_CASE(13) LORA_VEC_CASE(14) LORA_VEC_CASE(15) LORA_VEC_CASE(16)
            default: break;
          }
        }
        break;
#undef LORA_VEC_CASE
    }
    return;
  }
  const int runs = (p.fbn + RUN - 1) / RUN;
  if (slot >= runs) return;
  if constexpr (kPairs) {
    // Sub-tiles j and j + 1 (j even) of an adapter pair up: their 2 runs
    // waves take one block each, for both, so that B's rows are read once.
    const int lim = min(count, p.max_sub);
    const bool odd = head.w & 1;
    if (odd ? pair_ok<E, RUN>(p, lim, st - 1, hp, head, tp, tm, r) : pair_ok<E, RUN>(p, lim, st, head, hn, tm, tn, r)) {
      const int fb = odd ? runs + slot : slot;
      if (fb >= p.fbn) return;
      if (odd) expand_pair<E, kPart>(p, tkp, tk4, hp.z, hp.y, m, pos0, r, ro, sc, S, fb);
      else expand_pair<E, kPart>(p, tk4, tkn, m, pos0, hn.z, hn.y, r, ro, sc, S, fb);
      return;
    }
  }
  const int fb0 = slot * RUN, nb = min(RUN, p.fbn - fb0);
  const int nq = (r + KSTEP - 1) / KSTEP;
  if (nq <= 1) {
    expand_run<E, kPart, 1, RUN>(p, tk4, m, r, pos0, ro, sc, S, fb0, nb, hoff);
  } else if constexpr (KSTEP == 32) {  // bf16: ranks <= 64 take at most 2 chunks
    expand_run<E, kPart, 2, RUN>(p, tk4, m, r, pos0, ro, sc, S, fb0, nb, hoff);
  } else {
    if (nq == 2) expand_run<E, kPart, 2, RUN>(p, tk4, m, r, pos0, ro, sc, S, fb0, nb, hoff);
    else if (nq == 3) expand_run<E, kPart, 3, RUN>(p, tk4, m, r, pos0, ro, sc, S, fb0, nb, hoff);
    else expand_run<E, kPart, 4, RUN>(p, tk4, m, r, pos0, ro, sc, S, fb0, nb, hoff);
  }
}

// bf16 runs 4 waves per SIMD with one feature block per wave, 3 with runs
// (the second y buffer; spilling at 4 was slower); float32, a small-shape
// type here, is left to the compiler.  At 3 waves per SIMD the one-block
// form was slower (the y rows in flight matter more).
template <typename E, bool kPart, bool kSlice, int RUN>
__global__ void __launch_bounds__(kExpandWaves * 64)
__attribute__((amdgpu_waves_per_eu(E::kBytes == 2 ? (RUN > 1 ? 3 : 4) : 1))) expand_kernel(ExpandArgs p) {
  expand_wave<E, kPart, kSlice, RUN>(p);
}

template <int RUN>
static hipError_t launch_expand_kernel(int dtype, bool part, dim3 grid, dim3 block, hipStream_t stream,
                                       const ExpandArgs& a) {
  if (dtype == LORA_DTYPE_BF16) {
    if (part) hipLaunchKernelGGL((expand_kernel<BF16, true, false, RUN>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expand_kernel<BF16, false, false, RUN>), grid, block, 0, stream, a);
  } else {
    if (part) hipLaunchKernelGGL((expand_kernel<F32, true, false, RUN>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expand_kernel<F32, false, false, RUN>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

// Whether a call uses the run form: the one-block form would launch many
// times the waves the GPU holds.
static bool expand_run_form(int64_t one_block_items) { return one_block_items >= kExpandRunMinItems; }

// The arguments of one expand (slice: the multi-slice apply's slice store,
// whose B is applied, with its records); `run`: the form the launch uses.
static ExpandArgs expand_args(const lora_store& s, const lora_store* slice, const SliceMeta* sl_meta, const char* plan,
                              int T, const void* ws, const float* h, int64_t ldh, void* y, int64_t ldy, bool run) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  const char* base = reinterpret_cast<const char*>(ws);
  const lora_store& out = slice ? *slice : s;  // the store whose B is applied
  ExpandArgs a;
  a.b_pack = reinterpret_cast<const char*>(out.B_pack);
  a.d_out = out.d_out;
  a.T = T;
  a.max_sub = (int)max_sub;
  a.fbn = (out.d_out + kExpandCols - 1) / kExpandCols;
  a.plan = plan;
  a.meta = reinterpret_cast<const TileMeta*>(base + L.meta);
  a.n = s.n;
  a.r_max = s.r_max;
  a.R = s.R;
  a.S_max = shrink_split(s.d_in, s.dtype, T, s.n).S;
  a.y = reinterpret_cast<char*>(y);
  a.ldy_bytes = ldy * elem_bytes(s.dtype);
  a.sl_meta = sl_meta;
  a.sl_r_max = slice ? slice->r_max : 0;
  a.sl_R = slice ? slice->R : 0;
  if (h == nullptr) {
    a.hsrc = reinterpret_cast<const float*>(base + L.part);
    a.ldh = partial_ld(s.r_max);
    a.hstride = (int64_t)T * a.ldh;
  } else {
    a.hsrc = h;
    a.ldh = ldh;
    a.hstride = 0;
  }
  a.fbv = (out.d_out + kVecCols - 1) / kVecCols;
  const int vec_waves = (kVecMaxTokens / kVecTokens) * a.fbv;
  const int run_len = run ? kExpandRun : 1;
  const int runs = (a.fbn + run_len - 1) / run_len;
  a.slots = runs > vec_waves ? runs : vec_waves;
  return a;
}

static dim3 expand_grid(const ExpandArgs& a) {
  const int64_t items = (int64_t)a.max_sub * a.slots;
  return dim3((unsigned)((items + kExpandWaves - 1) / kExpandWaves));
}

hipError_t launch_expand(const lora_store& s, const char* plan, int T, const void* ws, const float* h, int64_t ldh,
                         void* y, int64_t ldy, hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  const bool run = expand_run_form(max_sub * (int64_t)((s.d_out + kExpandCols - 1) / kExpandCols));
  const ExpandArgs a = expand_args(s, nullptr, nullptr, plan, T, ws, h, ldh, y, ldy, run);
  const dim3 block(kExpandWaves * 64);
  return run ? launch_expand_kernel<kExpandRun>(s.dtype, h == nullptr, expand_grid(a), block, stream, a)
             : launch_expand_kernel<1>(s.dtype, h == nullptr, expand_grid(a), block, stream, a);
}

// Every slice of a multi-slice apply in one launch: grid dimension y picks
// the slice (one launch's ramp and tail instead of one per slice).
struct ExpandSlices {
  ExpandArgs s[LORA_MAX_SLICES];
};

template <typename E, int RUN>
__global__ void __launch_bounds__(kExpandWaves * 64)
__attribute__((amdgpu_waves_per_eu(E::kBytes == 2 ? (RUN > 1 ? 3 : 4) : 1))) expand_slices_kernel(ExpandSlices a) {
  expand_wave<E, true, true, RUN>(a.s[blockIdx.y]);
}

hipError_t launch_expand_slices(const lora_multi_store& m, const SliceMeta* sl_meta, const char* plan, int T,
                                const void* ws, void* const* y_host, const int64_t* ldy_host, hipStream_t stream) {
  const lora_store& s = m.stacked;
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  // One form for the launch: the one-block items of all slices together.
  int64_t one_block = 0;
  for (int k = 0; k < m.n_slices; ++k) one_block += max_sub * (int64_t)((m.slice[k].d_out + kExpandCols - 1) / kExpandCols);
  const bool run = expand_run_form(one_block);
  ExpandSlices a;
  unsigned gx = 0;
  for (int k = 0; k < m.n_slices; ++k) {
    a.s[k] = expand_args(s, &m.slice[k], sl_meta + (size_t)k * max_sub, plan, T, ws, nullptr, 0, y_host[k], ldy_host[k],
                         run);
    gx = expand_grid(a.s[k]).x > gx ? expand_grid(a.s[k]).x : gx;
  }
  const dim3 grid(gx, (unsigned)m.n_slices), block(kExpandWaves * 64);
  if (s.dtype == LORA_DTYPE_BF16) {
    if (run) hipLaunchKernelGGL((expand_slices_kernel<BF16, kExpandRun>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expand_slices_kernel<BF16, 1>), grid, block, 0, stream, a);
  } else {
    if (run) hipLaunchKernelGGL((expand_slices_kernel<F32, kExpandRun>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expand_slices_kernel<F32, 1>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lora
