// Decode apply: y[t] += s_a B_a (A_a x[t]) for a decode-sized batch, in one
// launch, one workgroup per (token, slice of output features).
//
// "Compress then Serve: Serving Thousands of LoRA Adapters with Little
// Overhead", section 13.4: each step of the two-step branch is a batched
// call that takes the per-token adapter indices; with about one token per
// adapter (decode) the grouping buys no reuse of A or B, so the token's
// adapter is read from its index directly.  The arithmetic is the same as
// the shrink and expand: products and sums in float32, one rounding of the
// new y value.
//
// Workgroup (token t, feature group fg), 512 threads, each with one 16-byte
// chunk of K and one group of 8 output features (kDecodeChunks):
//   1. ids[t] (a scalar load) and, for n <= 64, lane l's copy of adapter l's
//      rank, row offset and scale, loaded together.
//   2. The adapter's rank, row offset and scale (a cross-lane read of the
//      copies, else loads); then the thread's chunks of the x row (K = d_in
//      fits the workgroup's 512 chunks), of each of the R rows of A, the
//      8 x R blocks of B (rows o .. o + 7 of B_a in its [d_out, r_a] layout:
//      16 R contiguous bytes) and, last, of the y row (features o .. o + 7 of
//      each group): y is needed only at the end, and issued after A the A
//      rows arrive sooner (6.0 against 6.4 us per call, cold decode-uniform).
//   3. h[j] = sum over the threads' chunks: per lane, then across the wave
//      (DPP steps and lane reads), then over the waves in order (LDS).
//   4. y[o + f] += s_a sum_j h[j] B_a[o + f, j], written back.
// Every load is issued unconditionally, from an address clamped into the
// buffer; the lanes past d_in zero their partial sums, and the features past
// d_out are not stored.  Loads under a branch made the compiler wait for them
// right after their issue, one memory round trip in the middle of the loads.
// The kernel is instantiated per exact rank 1..kVecMaxRank (bf16) or
// 1..kVecMaxRank / 2 (float32), so the unpacking of the B block is static.
#include "device_common.h"
#include "kernels.h"

namespace lora {

// 16-byte chunks of K (and 8-feature groups) per thread.  One chunk (8 waves)
// is fastest: with two or four per thread and the same bytes per workgroup,
// the call took 1.09x and 1.21x as long (cold decode-uniform).
constexpr int kDecodeChunks = 1;
constexpr int kDecodeThreads = 512 / kDecodeChunks;
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kDecodeKChunks = kDecodeThreads * kDecodeChunks;  // 512 chunks: d_in <= 4096 bf16, 2048 float32
constexpr int kDecodeFeatures = kDecodeKChunks * 8;             // output features per workgroup

struct DecodeArgs {
  const int32_t* ids;
  int T, n, nf;  // nf: feature groups of kDecodeFeatures
  const char* x;
  int64_t ldx_bytes;
  const char* a_pack;
  const char* b_pack;
  const int32_t* row_off;
  const int32_t* rank;
  const float* scale;
  int d_in, d_out, R;  // R: rows of the store
  char* y;
  int64_t ldy_bytes;
};

// Element e of a 16-byte chunk as float32.
template <typename E>
__device__ __forceinline__ float chunk_elem(const uint4& v, int e) {
  const uint32_t w = e < E::kVec / 2 ? (e < E::kVec / 4 ? v.x : v.y) : (e < 3 * E::kVec / 4 ? v.z : v.w);
  if constexpr (E::kBytes == 2) return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  else return __uint_as_float(w);
}

template <typename E, int R>
__device__ __forceinline__ void decode_token(const DecodeArgs& p, const bool (&kv)[kDecodeChunks],
                                             const int (&kc)[kDecodeChunks], const uint4 (&xv)[kDecodeChunks],
                                             char* yrow,
                                             const int (&oc)[kDecodeChunks], const int (&nfe)[kDecodeChunks], int ro,
                                             float sc, float* s_h) {
  constexpr int V = E::kVec;
  constexpr int YV = 8 / V;
  constexpr int BV = 8 * R * E::kBytes / 16;
  constexpr int C = kDecodeChunks;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // A rows ro .. ro + R - 1 at K elements kc[c] .. kc[c] + V; the B blocks of
  // rows oc[c] .. oc[c] + 7 (chunks past the last feature re-read the first).
  uint4 av[C][R], bv[C][BV];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const char* ar = p.a_pack + ((size_t)ro * p.d_in + (size_t)kc[c]) * E::kBytes;
#pragma unroll
    for (int j = 0; j < R; ++j) av[c][j] = ld16(ar + (size_t)j * p.d_in * E::kBytes);
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const char* bb = p.b_pack + ((size_t)ro * p.d_out + (size_t)oc[c] * R) * E::kBytes;
    const int b_valid = nfe[c] * R * E::kBytes;  // bytes of the block that belong to features < d_out
#pragma unroll
    for (int i = 0; i < BV; ++i) bv[c][i] = ld16(bb + (16 * i < b_valid ? 16 * i : 0));
  }
  uint4 yv[C][YV];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int v = 0; v < YV; ++v)
      yv[c][v] = ld16_stream(yrow + (size_t)(v * V < nfe[c] ? oc[c] + v * V : oc[c]) * E::kBytes);
  // h: this thread's chunks, the wave, the waves in order.
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float sc_ = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) sc_ += chunk_elem<E>(xv[c], e) * chunk_elem<E>(av[c][j], e);
      s += kv[c] ? sc_ : 0.f;
    }
    acc[j] = s;
  }
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = wave_sum(acc[j]);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < R; ++j) s_h[w * kVecMaxRank + j] = acc[j];
  }
  __syncthreads();
  float h[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float v = s_h[j];
#pragma unroll
    for (int ww = 1; ww < kDecodeWaves; ++ww) v += s_h[ww * kVecMaxRank + j];
    h[j] = v;
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (nfe[c] <= 0) continue;
    const uint32_t* bw = reinterpret_cast<const uint32_t*>(bv[c]);
    float ay[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) ay[f] = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int e = f * R + j;  // B[o + f, j] in the block
        float b;
        if constexpr (E::kBytes == 2) b = (e & 1) ? bf16_hi(bw[e >> 1]) : bf16_lo(bw[e >> 1]);
        else b = __uint_as_float(bw[e]);
        ay[f] += h[j] * b;
      }
    char* yp = yrow + (size_t)oc[c] * E::kBytes;
#pragma unroll
    for (int v = 0; v < YV; ++v) {
      if (v * V >= nfe[c]) continue;
      float f[V];
      E::widen(yv[c][v], f);
#pragma unroll
      for (int kk = 0; kk < V; ++kk) f[kk] = f[kk] + sc * ay[v * V + kk];
      st16_stream(yp + 16 * v, E::narrow(f));
    }
  }
}

template <typename E>
__global__ void __launch_bounds__(kDecodeThreads) decode_apply_kernel(DecodeArgs p) {
  constexpr int V = E::kVec;
  constexpr int YV = 8 / V;
  constexpr int C = kDecodeChunks;
  __shared__ float s_h[kDecodeWaves * kVecMaxRank];
  const int tid = threadIdx.x, lane = tid & 63;
  const int t = blockIdx.x / p.nf, fg = blockIdx.x - t * p.nf;
  if (t >= p.T) return;
  const int a = p.ids[t];  // uniform over the workgroup
  // The adapter's rank, row offset and scale.  For n <= 64 every wave loads
  // adapter l's into lane l together with the index (no second dependent
  // round trip) and reads lane a's; otherwise they are loaded at a.
  int r, ro;
  float sc;
  if (p.n <= 64) {
    const int li = min(lane, p.n - 1);  // n >= 1 here
    const int m_rank = p.rank[li], m_row = p.row_off[li];
    const float m_scale = p.scale[li];
    const int ac = (unsigned)a < (unsigned)p.n ? a : 0;
    r = __builtin_amdgcn_readfirstlane(__shfl(m_rank, ac));
    ro = __builtin_amdgcn_readfirstlane(__shfl(m_row, ac));
    sc = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(__shfl(m_scale, ac))));
  } else {
    if ((unsigned)a >= (unsigned)p.n) return;
    r = p.rank[a];
    ro = p.row_off[a];
    sc = p.scale[a];
  }
  if ((unsigned)a >= (unsigned)p.n) return;      // no adapter (-1 or out of range): y unchanged
  if (r <= 0 || ro < 0 || ro > p.R - r) return;  // rank 0: a zero delta
  // x chunks (issued with the A and B loads; y after them).  Chunk c of the thread:
  // K elements (c T + tid) V and output features 8 (fg 512 + c T + tid),
  // T the workgroup's threads.
  bool kv[C];
  int kc[C], oc[C], nfe[C];
  uint4 xv[C];
  const char* xrow = p.x + (int64_t)t * p.ldx_bytes;
  char* yrow = p.y + (int64_t)t * p.ldy_bytes;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int k = (c * kDecodeThreads + tid) * V;
    kv[c] = k < p.d_in;
    kc[c] = kv[c] ? k : 0;
    xv[c] = ld16(xrow + (size_t)kc[c] * E::kBytes);
    const int o = (fg * kDecodeKChunks + c * kDecodeThreads + tid) * 8;
    nfe[c] = min(8, p.d_out - o);
    oc[c] = nfe[c] > 0 ? o : 0;
  }
  switch (r) {  // uniform over the workgroup
#define LORA_TOKEN_CASE(RR) \
  case RR: decode_token<E, RR>(p, kv, kc, xv, yrow, oc, nfe, ro, sc, s_h); break;
    LORA_TOKEN_CASE(1) LORA_TOKEN_CASE(2) LORA_TOKEN_CASE(3) LORA_TOKEN_CASE(4)
    default:
      if constexpr (E::kBytes == 2) {
        switch (r) {
          LORA_TOKEN_CASE(5) LORA_TOKEN_CASE(6) LORA_TOKEN_CASE(7) LORA_TOKEN_CASE(8)
          default: break;  // ranks above kVecMaxRank are not sent here
        }
      }
      break;
#undef LORA_TOKEN_CASE
  }
}

bool decode_apply_fits(const lora_store& s, int T, bool with_ids) {
  const int r_cap = s.dtype == LORA_DTYPE_BF16 ? kVecMaxRank : kVecMaxRank / 2;  // float32 blocks: twice the bytes
  return with_ids && s.n >= 1 && s.r_max >= 1 && s.r_max <= r_cap && s.d_in <= kDecodeKChunks * vec_elems(s.dtype) &&
         T <= kDecodeMaxT;
}

hipError_t launch_decode_apply(const lora_store& s, const int32_t* ids, int T, const void* x, int64_t ldx, void* y,
                               int64_t ldy, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  DecodeArgs a;
  a.ids = ids;
  a.T = T;
  a.n = s.n;
  a.nf = (s.d_out + kDecodeFeatures - 1) / kDecodeFeatures;
  a.x = reinterpret_cast<const char*>(x);
  a.ldx_bytes = ldx * elem_bytes(s.dtype);
  a.a_pack = reinterpret_cast<const char*>(s.A_pack);
  a.b_pack = reinterpret_cast<const char*>(s.B_pack);
  a.row_off = s.row_off;
  a.rank = s.rank;
  a.scale = s.scale;
  a.d_in = s.d_in;
  a.d_out = s.d_out;
  a.R = s.R;
  a.y = reinterpret_cast<char*>(y);
  a.ldy_bytes = ldy * elem_bytes(s.dtype);
  const dim3 grid((unsigned)((int64_t)T * a.nf)), block(kDecodeThreads);
  if (s.dtype == LORA_DTYPE_BF16) hipLaunchKernelGGL(decode_apply_kernel<BF16>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(decode_apply_kernel<F32>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace lora
