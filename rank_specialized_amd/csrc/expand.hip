// Expand: y[t, o] += s_a * sum_{j < r_a} B_a[o, j] h[t, j].
//
// Step 3 of the two-step branch in "Compress then Serve: Serving Thousands
// of LoRA Adapters with Little Overhead", section 13.4: B applied with the
// adapter's scale and added into (a slice of) y.  Accumulation in float32,
// one rounding of the new y value to the output type.
//
// Work item = one wave: (sub-tile, 128 output features).  Waves are
// independent (no barriers); every wave issues its y rows and its B rows
// before any arithmetic, so an item costs one memory round trip.
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
#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {

struct ExpandArgs {
  const char* b_pack;
  int d_out, T, max_sub, fbn;
  int n, r_max, R, S_max;  // the store's bounds: plan entries outside them are skipped
  const float* hsrc;      // partial sums (kPart) or h
  int64_t ldh, hstride;   // floats
  const char* plan;
  char* y;
  int64_t ldy_bytes;
};

template <typename E, bool kPart, int NQ>
__device__ __forceinline__ void expand_item(const ExpandArgs& p, const TileEntry* ent, int m, int r, int pos0,
                                            int ro, float sc, int S, int o) {
  constexpr int V = E::kVec;
  constexpr int KSTEP = 4 * V;  // ranks per K chunk
  constexpr int YV = 8 / V;     // 16-byte vectors per 8 features: bf16 1, f32 2
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // y rows of tokens 4g .. 4g + 3 (issued first: the longest wait).
  char* yp[4];
  uint4 yv[4][YV];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = 4 * g + e;
    const int tok = t < m ? ent->tok[t] : -1;
    yp[e] = ((unsigned)tok < (unsigned)p.T && o < p.d_out)
                ? p.y + (int64_t)tok * p.ldy_bytes + (size_t)o * E::kBytes
                : nullptr;
#pragma unroll
    for (int v = 0; v < YV; ++v) yv[e][v] = (yp[e] && o + v * V < p.d_out) ? ld16(yp[e] + 16 * v) : zero;
  }
  // B rows o .. o + 7 (one per N block), ranks of this lane's K chunks.
  // bf16 rows of an odd rank start on 2-byte boundaries, and a 16-byte
  // buffer load must start on a 4-byte one: such a chunk (row o + b odd,
  // i.e. N block b odd, the same for every lane) is read from the dword below
  // plus one more dword, and shifted down by 16 bits.
  const uint32_t row_bytes = (uint32_t)r * E::kBytes;
  const rsrc_t br = make_rsrc(p.b_pack + (size_t)ro * p.d_out * E::kBytes, (uint32_t)p.d_out * row_bytes);
  const bool odd_rows = E::kBytes == 2 && (r & 1);
  uint4 bq[NQ][8];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int j0 = q * KSTEP + g * V;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool ok = j0 < r && o + b < p.d_out;
      const uint32_t off = (uint32_t)(o + b) * row_bytes + (uint32_t)j0 * E::kBytes;
      if ((b & 1) && odd_rows) {
        const uint32_t lo = ok ? off - 2 : kOutOfRange;
        const uint4 d = buf_ld16(br, lo, 0);
        const uint32_t t = buf_ld4(br, ok ? lo + 16 : kOutOfRange);
        bq[q][b] = make_uint4(__builtin_amdgcn_alignbit(d.y, d.x, 16), __builtin_amdgcn_alignbit(d.z, d.y, 16),
                              __builtin_amdgcn_alignbit(d.w, d.z, 16), __builtin_amdgcn_alignbit(t, d.w, 16));
      } else {
        bq[q][b] = buf_ld16(br, ok ? off : kOutOfRange, 0);
      }
    }
  }
  // H chunks: token c of the sub-tile, ranks j0 .. j0 + V.
  HChunk<E> hc[NQ];
  const int hrow = pos0 + c;
  const bool hv = c < m && hrow >= 0 && hrow < p.T;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int j0 = q * KSTEP + g * V;
    float f[V];
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = 0.f;
    if (hv && j0 < r) {
      const float* src = p.hsrc + (int64_t)hrow * p.ldh + j0;
      if (kPart) {
#pragma unroll
        for (int v = 0; v < V / 4; ++v) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + 4 * v);
          f[4 * v] = x[0]; f[4 * v + 1] = x[1]; f[4 * v + 2] = x[2]; f[4 * v + 3] = x[3];
        }
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
    hc[q].set(f);
  }
  f32x4_t acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int nvalid = r - (q * KSTEP + g * V);
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = hc[q].mma(keep_first<E>(bq[q][b], nvalid), acc[b]);
  }
  // acc[b][e] = feature o + b of token 4g + e.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (yp[e] == nullptr) continue;
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      if (o + v * V >= p.d_out) continue;
      float f[V];
      E::widen(yv[e][v], f);
#pragma unroll
      for (int k = 0; k < V; ++k) f[k] = f[k] + sc * acc[v * V + k][e];
      st16(yp[e] + 16 * v, E::narrow(f));
    }
  }
}

template <typename E, bool kPart>
__global__ void __launch_bounds__(kExpandWaves * 64) expand_kernel(ExpandArgs p) {
  constexpr int KSTEP = 4 * E::kVec;
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * kExpandWaves + (threadIdx.x >> 6));
  const int st = item / p.fbn, fb = item - st * p.fbn;
  if (st >= p.max_sub) return;
  const int count = *reinterpret_cast<const int32_t*>(p.plan);
  if (st >= count) return;
  const TileEntry* ent = reinterpret_cast<const TileEntry*>(p.plan + kPlanHeaderBytes) + st;
  const int a = ent->a, m = ent->m, r = ent->r, pos0 = ent->pos0, ro = ent->row_off;
  const float sc = ent->scale;
  const int S = kPart ? ent->S : 1;
  // An entry must describe this store (a plan left in the workspace by a
  // call on another store is skipped): every B row and partial sum it names
  // then lies inside the store's and the workspace's buffers.
  if ((unsigned)a >= (unsigned)p.n || m <= 0 || m > kSubTile || r <= 0 || r > p.r_max || ro < 0 ||
      ro > p.R - r || S <= 0 || S > p.S_max)
    return;
  const int o = fb * kExpandCols + 8 * (threadIdx.x & 15);
  const int nq = (r + KSTEP - 1) / KSTEP;
  if (nq <= 1) {
    expand_item<E, kPart, 1>(p, ent, m, r, pos0, ro, sc, S, o);
  } else if constexpr (KSTEP == 32) {  // bf16: ranks <= 64 take at most 2 chunks
    expand_item<E, kPart, 2>(p, ent, m, r, pos0, ro, sc, S, o);
  } else {
    if (nq == 2) expand_item<E, kPart, 2>(p, ent, m, r, pos0, ro, sc, S, o);
    else if (nq == 3) expand_item<E, kPart, 3>(p, ent, m, r, pos0, ro, sc, S, o);
    else expand_item<E, kPart, 4>(p, ent, m, r, pos0, ro, sc, S, o);
  }
}

hipError_t launch_expand(const lora_store& s, int T, const void* ws, const float* h, int64_t ldh, void* y,
                         int64_t ldy, hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, s.n);
  if (max_sub == 0) return hipSuccess;
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  const char* base = reinterpret_cast<const char*>(ws);
  ExpandArgs a;
  a.b_pack = reinterpret_cast<const char*>(s.B_pack);
  a.d_out = s.d_out;
  a.T = T;
  a.max_sub = (int)max_sub;
  a.fbn = (s.d_out + kExpandCols - 1) / kExpandCols;
  a.plan = base + L.plan;
  a.n = s.n;
  a.r_max = s.r_max;
  a.R = s.R;
  a.S_max = shrink_split(s.d_in, s.r_max, s.dtype).S_max;
  a.y = reinterpret_cast<char*>(y);
  a.ldy_bytes = ldy * elem_bytes(s.dtype);
  const bool part = h == nullptr;
  if (part) {
    a.hsrc = reinterpret_cast<const float*>(base + L.part);
    a.ldh = partial_ld(s.r_max);
    a.hstride = (int64_t)T * a.ldh;
  } else {
    a.hsrc = h;
    a.ldh = ldh;
    a.hstride = 0;
  }
  const int64_t items = max_sub * a.fbn;
  const dim3 grid((unsigned)((items + kExpandWaves - 1) / kExpandWaves));
  const dim3 block(kExpandWaves * 64);
  if (s.dtype == LORA_DTYPE_BF16) {
    if (part) hipLaunchKernelGGL((expand_kernel<BF16, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expand_kernel<BF16, false>), grid, block, 0, stream, a);
  } else {
    if (part) hipLaunchKernelGGL((expand_kernel<F32, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((expand_kernel<F32, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace lora
