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
// Workgroup (token t, feature group fg), 512 threads:
//   1. ids[t] (a scalar load), and meanwhile the thread's 16-byte chunk of the
//      x row (K = d_in fits one chunk per thread) and of the y row (features
//      o .. o + 7, o = 8 (512 fg + thread)).
//   2. The adapter's rank, row offset and scale; then the thread's chunk of
//      each of the R rows of A and the 8 x R block of B (rows o .. o + 7 of
//      B_a in its [d_out, r_a] layout: 16 R contiguous bytes).
//   3. h[j] = sum over the threads' chunks: per lane, then a butterfly over
//      the lanes, then over the waves in order (LDS).
//   4. y[o + f] += s_a sum_j h[j] B_a[o + f, j], written back.
// The kernel is instantiated per exact rank 1..kVecMaxRank (bf16) or
// 1..kVecMaxRank / 2 (float32), so the unpacking of the B block is static.
#include "device_common.h"
#include "kernels.h"

namespace lora {

constexpr int kDecodeThreads = 512;
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kDecodeFeatures = kDecodeThreads * 8;  // output features per workgroup

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
__device__ __forceinline__ void decode_token(const DecodeArgs& p, int k, const uint4& xv, const uint4 (&yv)[8 / E::kVec],
                                             char* yp, int o, int nfe, int ro, float sc, float* s_h) {
  constexpr int V = E::kVec;
  constexpr int YV = 8 / V;
  constexpr int BV = 8 * R * E::kBytes / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // A rows ro .. ro + R - 1 at K elements k .. k + V; the B block of o .. o + 7.
  const bool kv = k < p.d_in;
  const char* ar = p.a_pack + ((size_t)ro * p.d_in + (size_t)(kv ? k : 0)) * E::kBytes;
  uint4 av[R], bv[BV];
#pragma unroll
  for (int j = 0; j < R; ++j) av[j] = kv ? ld16(ar + (size_t)j * p.d_in * E::kBytes) : zero;
  const char* bb = p.b_pack + ((size_t)ro * p.d_out + (size_t)(nfe > 0 ? o : 0) * R) * E::kBytes;
#pragma unroll
  for (int i = 0; i < BV; ++i) bv[i] = 16 * i < nfe * R * E::kBytes ? ld16(bb + 16 * i) : zero;
  // h: this thread's chunk, the lanes (butterfly), the waves in order.
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) s += chunk_elem<E>(xv, e) * chunk_elem<E>(av[j], e);
    acc[j] = s;
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    float v = acc[j];
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) v += __shfl_xor(v, sh);
    acc[j] = v;
  }
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
  if (nfe <= 0 || yp == nullptr) return;
  const uint32_t* bw = reinterpret_cast<const uint32_t*>(bv);
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
#pragma unroll
  for (int v = 0; v < YV; ++v) {
    if (v * V >= nfe) continue;
    float f[V];
    E::widen(yv[v], f);
#pragma unroll
    for (int kk = 0; kk < V; ++kk) f[kk] = f[kk] + sc * ay[v * V + kk];
    st16_stream(yp + 16 * v, E::narrow(f));
  }
}

template <typename E>
__global__ void __launch_bounds__(kDecodeThreads) decode_apply_kernel(DecodeArgs p) {
  constexpr int V = E::kVec;
  constexpr int YV = 8 / V;
  __shared__ float s_h[kDecodeWaves * kVecMaxRank];
  const int tid = threadIdx.x;
  const int t = blockIdx.x / p.nf, fg = blockIdx.x - t * p.nf;
  if (t >= p.T) return;
  const int a = p.ids[t];  // uniform over the workgroup
  // x and y chunks, issued with the index.
  const uint4 zero = make_uint4(0, 0, 0, 0);
  const int k = tid * V;
  const uint4 xv = k < p.d_in ? ld16(p.x + (int64_t)t * p.ldx_bytes + (size_t)k * E::kBytes) : zero;
  const int o = (fg * kDecodeThreads + tid) * 8;
  const int nfe = min(8, p.d_out - o);
  char* yp = nfe > 0 ? p.y + (int64_t)t * p.ldy_bytes + (size_t)o * E::kBytes : nullptr;
  uint4 yv[YV];
#pragma unroll
  for (int v = 0; v < YV; ++v) yv[v] = (yp && v * V < nfe) ? ld16_stream(yp + 16 * v) : zero;
  if ((unsigned)a >= (unsigned)p.n) return;  // no adapter (-1 or out of range): y unchanged
  const int r = p.rank[a], ro = p.row_off[a];
  const float sc = p.scale[a];
  if (r <= 0 || ro < 0 || ro > p.R - r) return;  // rank 0: a zero delta
  switch (r) {  // uniform over the workgroup
#define LORA_TOKEN_CASE(RR) \
  case RR: decode_token<E, RR>(p, k, xv, yv, yp, o, nfe, ro, sc, s_h); break;
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
  return with_ids && s.r_max >= 1 && s.r_max <= r_cap && s.d_in <= kDecodeThreads * vec_elems(s.dtype) &&
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
