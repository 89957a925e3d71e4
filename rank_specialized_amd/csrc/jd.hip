// Shared-basis (joint-diagonalization) apply: the steps around the shrink
// and the expand.
//
// "Compress then Serve: Serving Thousands of LoRA Adapters with Little
// Overhead", section 3.1: adapter i's product B_i A_i is held as
// U Sigma_i V^T (Sigma_i full r x r, or diagonal); section 3.2: each cluster
// j of adapters has its own U_j, V_j; section 11: the branch is served as
// U (Sigma (V^T x)), V^T x and the U product shared by a cluster's tokens;
// section 13.4: the three steps (A, Sigma, B) take a per-token index.
//
// Here the clusters are the "adapters" of an ordinary store (A rows = V_j^T,
// B block = U_j, every rank r, scale 1): the shrink groups the tokens by the
// cluster of their adapter (the grouping kernel maps the ids through
// cluster_of) and the expand runs unchanged; between them, jd_sigma_kernel takes each token of
// each planned sub-tile: h = the shrink's partial sums (chunk order), then
// g = s_a Sigma_a h, written as the expand's h.
#include "device_common.h"
#include "kernels.h"

namespace lora {

struct SigmaArgs {
  const char* plan;
  const TileMeta* meta;  // per sub-tile, from the shrink
  int max_sub, k, r, S_max;  // the basis store's bounds: entries outside them are skipped
  const float* part;
  int64_t ldp, pstride;
  const int32_t* ids;
  int T, n;
  const int32_t* cluster_of;
  const float* sigma;  // full: [n][r][r] row-major; diagonal: [n][r]
  int diag;
  const float* scale;
  float* h;
  int64_t ldh;
};

// g[lane] = s * sum_j Sigma[lane][j] h[j] for lanes < r <= RP: the row's loads
// issued together, h[j] broadcast from lane j.
template <int RP>
__device__ __forceinline__ float sigma_full(const float* srow, float h, int r, float s) {
  const int lane = threadIdx.x & 63;
  float sv[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) sv[j] = (lane < r && j < r) ? srow[j] : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const float hj = __shfl(h, j);
    if (j < r) acc += sv[j] * hj;
  }
  return s * acc;
}

// One wave per (sub-tile, token slot of it); lane j < r owns rank j.
__global__ void __launch_bounds__(256) jd_sigma_kernel(SigmaArgs p) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int st = item / kSubTile, i = item - st * kSubTile;
  if (st >= p.max_sub) return;
  if (st >= *reinterpret_cast<const int32_t*>(p.plan)) return;
  const TileEntry* e = reinterpret_cast<const TileEntry*>(p.plan + kPlanHeaderBytes) + st;
  const TileMeta tm = p.meta[st];
  const int c = e->a, m = e->m, r = tm.r, S = tm.S, pos0 = e->pos0;
  if ((unsigned)c >= (unsigned)p.k || m <= 0 || m > kSubTile || r != p.r || S <= 0 || S > p.S_max || i >= m)
    return;
  const int row = pos0 + i, t = e->tok[i];
  if (row < 0 || row >= p.T || (unsigned)t >= (unsigned)p.T) return;
  const int a = p.ids[t];
  if ((unsigned)a >= (unsigned)p.n || p.cluster_of[a] != c) return;  // as the grouping assigned it
  // h[lane]: the S partial sums, loads issued together, added in chunk order.
  float h = 0.f;
  if (lane < r) {
    const float* src = p.part + (int64_t)row * p.ldp + lane;
    h = sum_partials(src, p.pstride, S);
  }
  const float s = p.scale[a];
  float g;
  if (p.diag) {
    g = lane < r ? s * (p.sigma[(int64_t)a * r + lane] * h) : 0.f;
  } else {
    const float* srow = p.sigma + ((int64_t)a * r + (lane < r ? lane : 0)) * r;
    g = r <= 8 ? sigma_full<8>(srow, h, r, s)
        : r <= 16 ? sigma_full<16>(srow, h, r, s)
        : r <= 32 ? sigma_full<32>(srow, h, r, s)
                  : sigma_full<LORA_MAX_RANK>(srow, h, r, s);
  }
  if (lane < r) p.h[(int64_t)row * p.ldh + lane] = g;
}

hipError_t launch_jd_sigma(const lora_store& basis, const char* plan, int T, const void* ws, const int32_t* ids,
                           int n,
                           const int32_t* cluster_of, const float* sigma, int diag, const float* scale, float* h,
                           int64_t ldh, hipStream_t stream) {
  const int64_t max_sub = plan_max_subtiles(T, basis.n);
  if (max_sub == 0) return hipSuccess;
  const WsLayout L = ws_layout(T, basis.n, basis.d_in, basis.r_max, basis.dtype);
  const char* base = reinterpret_cast<const char*>(ws);
  SigmaArgs a;
  a.plan = plan;
  a.meta = reinterpret_cast<const TileMeta*>(base + L.meta);
  a.max_sub = (int)max_sub;
  a.k = basis.n;
  a.r = basis.r_max;
  a.S_max = shrink_split(basis.d_in, basis.dtype, T, basis.n).S;
  a.part = reinterpret_cast<const float*>(base + L.part);
  a.ldp = partial_ld(basis.r_max);
  a.pstride = (int64_t)T * a.ldp;
  a.ids = ids;
  a.T = T;
  a.n = n;
  a.cluster_of = cluster_of;
  a.sigma = sigma;
  a.diag = diag;
  a.scale = scale;
  a.h = h;
  a.ldh = ldh;
  const int64_t waves = max_sub * kSubTile;
  hipLaunchKernelGGL(jd_sigma_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lora
