// Retained-factor construction: the rank-k SVD of each adapter's B A through
// tall-and-skinny QRs of B and A^T, batched over the adapters of a module.
//
// "LoRAForge: Co-Designing Compression and Execution for More Efficient
// Multi-LoRA Serving", section "FlashTSQR: An Accelerator for Batched Factor
// Construction" and the glossary before it: post-hoc compression decomposes
// the original factors; a tall-and-skinny QR works on row blocks and then
// merges them, parallel across modules and row blocks.  "Compress then
// Serve", section 4: alone, an adapter's best rank-k replacement is the
// rank-k SVD of B A (Eckart-Young).
//
// For B (d_out x r) and A (r x d_in), with B = Q_B R_B and A^T = Q_A R_A:
// B A = Q_B (R_B R_A^T) Q_A^T, and the SVD of the r x r core C = U S V^T
// gives B' = Q_B U_k = B (R_B^-1 U_k) and A' = S_k V_k^T Q_A^T =
// (R_A^-1 V_k S_k)^T A.  Q is never formed.
//
//   rsvd_gram_kernel   R's Gram matrix M^T M of a factor (M = B, or A^T),
//                      one row block per workgroup, float64 (bf16 and f32
//                      products are exact in float64): the blocks' parts
//                      are merged by the core kernel, summed in block order.
//                      R^T R = M^T M, so R is the Cholesky factor: this is
//                      the Cholesky form of the tall-skinny QR (one pass over
//                      the rows; its R loses accuracy as cond(M)^2, which the
//                      core kernel reports when a pivot collapses).
//   rsvd_core_kernel   per adapter, in LDS: Cholesky of both Grams, the core
//                      C = R_B R_A^T, its SVD by one-sided Jacobi (column
//                      pairs in a round-robin order, rotations until every
//                      pair is orthogonal to 1e-15), the singular values in
//                      descending order, and W_B = R_B^-1 U, W_A = R_A^-1 V S
//                      by back substitution.
//   rsvd_write_kernel  B'[o, c] = sum_i B[o, i] W_B[i, c] and
//                      A'[c, k] = sum_i W_A[i, c] A[i, k] for c < k_a, written
//                      straight into a store's A and B buffers at the store's
//                      row offsets and ranks (k_a), rounded once.
#include "device_common.h"
#include "kernels.h"

namespace lora {

constexpr int kRsvdThreads = 256;
constexpr int kRsvdR = LORA_MAX_RANK;  // largest original rank
constexpr int kRsvdTile = 64;          // rows of a Gram tile
constexpr int kRsvdMaxBlocks = 4;      // row blocks per factor

template <typename E>
__device__ __forceinline__ double load_elem(const char* base, int64_t i) {
  if constexpr (E::kBytes == 2) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
  else return (double)reinterpret_cast<const float*>(base)[i];
}

struct RsvdArgs {
  int n, d_in, d_out, r, nblk;
  const char* A;  // [n][r][d_in]
  const char* B;  // [n][d_out][r]
  double* part;   // [n][2][nblk][kRsvdR][kRsvdR]
  double* WB;     // [n][kRsvdR][kRsvdR]
  double* WA;     // [n][kRsvdR][kRsvdR]
  float* sigma;   // [n][r]
  int32_t* status;
};

// Workgroup (adapter, side, row block): side 0 = B (rows of length r, d_out
// of them), side 1 = A^T (the columns of A).
template <typename E>
__global__ void __launch_bounds__(kRsvdThreads) rsvd_gram_kernel(RsvdArgs p) {
  __shared__ double t[kRsvdTile][kRsvdR + 1];
  const int b = blockIdx.x;
  const int blk = b % p.nblk, side = (b / p.nblk) & 1, a = b / (2 * p.nblk);
  const int tid = threadIdx.x, r = p.r;
  const int D = side == 0 ? p.d_out : p.d_in;
  const int per = ((D + p.nblk - 1) / p.nblk + kRsvdTile - 1) / kRsvdTile * kRsvdTile;
  const int k0 = blk * per, k1 = min(D, k0 + per);
  const int i0 = 4 * (tid / 16), j0 = 4 * (tid % 16);
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  const char* base = side == 0 ? p.B + (size_t)a * p.d_out * r * E::kBytes : p.A + (size_t)a * r * p.d_in * E::kBytes;
  for (int kt = k0; kt < k1; kt += kRsvdTile) {
    const int rows = min(kRsvdTile, k1 - kt);
    // Stage rows kt .. kt + rows of M (row kk holds M[kt + kk][0 .. r)).
    for (int e = tid; e < kRsvdTile * kRsvdR; e += kRsvdThreads) {
      int kk, i;
      if (side == 0) {
        kk = e / kRsvdR;
        i = e - kk * kRsvdR;
      } else {
        i = e / kRsvdTile;
        kk = e - i * kRsvdTile;
      }
      double v = 0.0;
      if (kk < rows && i < r)
        v = side == 0 ? load_elem<E>(base, (int64_t)(kt + kk) * r + i) : load_elem<E>(base, (int64_t)i * p.d_in + kt + kk);
      t[kk][i] = v;
    }
    __syncthreads();
    if (i0 < r && j0 < r) {
      for (int kk = 0; kk < rows; ++kk) {
        double x[4], y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          x[u] = t[kk][i0 + u];
          y[u] = t[kk][j0 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] += x[u] * y[v];
      }
    }
    __syncthreads();
  }
  double* out = p.part + ((((size_t)a * 2 + side) * p.nblk + blk) * kRsvdR) * kRsvdR;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[(size_t)(i0 + u) * kRsvdR + j0 + v] = acc[u][v];
}

// Upper Cholesky factor of the r x r matrix g in place (R in the upper
// triangle, R^T R = g; the lower triangle is left as it was).  A pivot at or
// below 1e-14 of the largest diagonal entry (cond(M) above about 1e7, where
// the Cholesky form of the QR stops being accurate) sets *bad; a pivot at or
// below 1e-30 of it, or not positive, is raised to that floor so that the
// factorization finishes (a zero column gives a zero row of R but for a tiny
// diagonal).
__device__ void cholesky_upper(double (*g)[kRsvdR + 1], int r, double* s_d, int* bad) {
  const int tid = threadIdx.x;
  double dmax = 0.0;
  for (int j = 0; j < r; ++j) dmax = fmax(dmax, g[j][j]);
  __syncthreads();  // every thread has read the diagonal before it changes
  const double warn = 1e-14 * dmax, floor_v = fmax(1e-30 * dmax, 1e-300);
  for (int j = 0; j < r; ++j) {
    if (tid == 0) {
      double d = g[j][j];
      if (!(d > warn)) *bad = 1;
      if (!(d > floor_v)) d = floor_v;
      *s_d = sqrt(d);
      g[j][j] = *s_d;
    }
    __syncthreads();
    const double d = *s_d;
    for (int c = j + 1 + tid; c < r; c += kRsvdThreads) g[j][c] /= d;
    __syncthreads();
    const int m = r - j - 1;
    for (int e = tid; e < m * m; e += kRsvdThreads) {
      const int c1 = j + 1 + e / m, c2 = j + 1 + e % m;
      if (c2 >= c1) g[c1][c2] -= g[j][c1] * g[j][c2];
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kRsvdThreads) rsvd_core_kernel(RsvdArgs p) {
  extern __shared__ double lds[];
  double (*gb)[kRsvdR + 1] = reinterpret_cast<double (*)[kRsvdR + 1]>(lds);
  double (*ga)[kRsvdR + 1] = gb + kRsvdR;
  double (*c)[kRsvdR + 1] = ga + kRsvdR;
  double (*v)[kRsvdR + 1] = c + kRsvdR;
  __shared__ double s_d;
  __shared__ double s_sig[kRsvdR];
  __shared__ int s_pos[kRsvdR];
  __shared__ int s_rot, s_bad;
  const int a = blockIdx.x, tid = threadIdx.x, r = p.r;
  if (tid == 0) s_bad = 0;
  // 1. The Grams: the row blocks' parts summed in block order.
  for (int e = tid; e < kRsvdR * kRsvdR; e += kRsvdThreads) {
    const int i = e / kRsvdR, j = e % kRsvdR;
    double sb = 0.0, sa = 0.0;
    for (int blk = 0; blk < p.nblk; ++blk) {
      sb += p.part[((((size_t)a * 2 + 0) * p.nblk + blk) * kRsvdR + i) * kRsvdR + j];
      sa += p.part[((((size_t)a * 2 + 1) * p.nblk + blk) * kRsvdR + i) * kRsvdR + j];
    }
    gb[i][j] = sb;
    ga[i][j] = sa;
  }
  __syncthreads();
  // 2. R_B, R_A (upper triangles of gb, ga).
  cholesky_upper(gb, r, &s_d, &s_bad);
  cholesky_upper(ga, r, &s_d, &s_bad);
  // 3. C = R_B R_A^T, V = I.
  for (int e = tid; e < kRsvdR * kRsvdR; e += kRsvdThreads) {
    const int i = e / kRsvdR, j = e % kRsvdR;
    double s = 0.0;
    if (i < r && j < r)
      for (int k = max(i, j); k < r; ++k) s += gb[i][k] * ga[j][k];
    c[i][j] = s;
    v[i][j] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();
  // 4. One-sided Jacobi: rotate column pairs of C (and V) until orthogonal.
  //    Round-robin pairing of m = r rounded up to even players: each round,
  //    m / 2 disjoint pairs, 8 threads per pair; m - 1 rounds per sweep.
  const int m = (r + 1) & ~1;
  const int grp = tid >> 3, l = tid & 7;
  for (int sweep = 0; sweep < 40; ++sweep) {
    if (tid == 0) s_rot = 0;
    __syncthreads();
    for (int rnd = 0; rnd < m - 1; ++rnd) {
      for (int pr = grp; pr < m / 2; pr += kRsvdThreads / 8) {
        int pp, qq;
        if (pr == 0) {
          pp = m - 1;
          qq = rnd;
        } else {
          pp = (rnd + pr) % (m - 1);
          qq = (rnd - pr + m - 1) % (m - 1);
        }
        const int P = min(pp, qq), Q = max(pp, qq);
        double al = 0.0, be = 0.0, ga_ = 0.0;
        if (Q < r) {
          for (int i = l; i < r; i += 8) {
            const double x = c[i][P], y = c[i][Q];
            al += x * x;
            be += y * y;
            ga_ += x * y;
          }
        }
#pragma unroll
        for (int sh = 1; sh < 8; sh <<= 1) {
          al += __shfl_xor(al, sh, 8);
          be += __shfl_xor(be, sh, 8);
          ga_ += __shfl_xor(ga_, sh, 8);
        }
        if (Q < r && fabs(ga_) > 1e-15 * sqrt(al * be) && ga_ != 0.0) {
          const double zeta = (be - al) / (2.0 * ga_);
          const double tt = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
          const double cs = 1.0 / sqrt(1.0 + tt * tt), sn = cs * tt;
          for (int i = l; i < r; i += 8) {
            const double x = c[i][P], y = c[i][Q];
            c[i][P] = cs * x - sn * y;
            c[i][Q] = sn * x + cs * y;
            const double vx = v[i][P], vy = v[i][Q];
            v[i][P] = cs * vx - sn * vy;
            v[i][Q] = sn * vx + cs * vy;
          }
          if (l == 0) s_rot = 1;
        }
      }
      __syncthreads();
    }
    const bool more = s_rot != 0;
    __syncthreads();
    if (!more) break;
  }
  // 5. Singular values (column norms) and their descending order.
  if (tid < r) {
    double s = 0.0;
    for (int i = 0; i < r; ++i) s += c[i][tid] * c[i][tid];
    s_sig[tid] = sqrt(s);
  }
  __syncthreads();
  if (tid < r) {
    int pos = 0;
    const double me = s_sig[tid];
    for (int k = 0; k < r; ++k) pos += (s_sig[k] > me || (s_sig[k] == me && k < tid)) ? 1 : 0;
    s_pos[tid] = pos;
  }
  __syncthreads();
  // 6. Thread j: u_j = C[:, j] / sigma_j, then W_B[:, pos_j] = R_B^-1 u_j and
  //    W_A[:, pos_j] = R_A^-1 (sigma_j v_j), by back substitution in place.
  if (tid < r) {
    const int j = tid, pos = s_pos[j];
    const double sg = s_sig[j];
    const double inv = sg > 0.0 ? 1.0 / sg : 0.0;
    for (int i = 0; i < r; ++i) {
      c[i][j] *= inv;
      v[i][j] *= sg;
    }
    for (int i = r - 1; i >= 0; --i) {
      double sb = c[i][j], sa = v[i][j];
      for (int k = i + 1; k < r; ++k) {
        sb -= gb[i][k] * c[k][j];
        sa -= ga[i][k] * v[k][j];
      }
      c[i][j] = sb / gb[i][i];
      v[i][j] = sa / ga[i][i];
    }
    double* wb = p.WB + (size_t)a * kRsvdR * kRsvdR;
    double* wa = p.WA + (size_t)a * kRsvdR * kRsvdR;
    for (int i = 0; i < r; ++i) {
      wb[(size_t)i * kRsvdR + pos] = c[i][j];
      wa[(size_t)i * kRsvdR + pos] = v[i][j];
    }
    p.sigma[(size_t)a * r + pos] = (float)sg;
  }
  if (tid == 0) p.status[a] = s_bad;
}

struct RsvdWriteArgs {
  int n, d_in, d_out, r, R, nbo;  // nbo: row blocks of B' (kRsvdThreads rows each)
  const char* A;
  const char* B;
  const double* WB;
  const double* WA;
  const int32_t* row_off;
  const int32_t* rank;       // stored rank
  const int32_t* true_rank;  // retained rank k_a
  char* A_pack;
  char* B_pack;
};

template <typename E>
__device__ __forceinline__ void store_elem(typename E::storage* out, size_t i, double v) {
  if constexpr (E::kBytes == 2) out[i] = (uint16_t)f32_to_bf16((float)v);
  else out[i] = (float)v;
}

// Workgroup (adapter, block): blocks [0, nbo) write kRsvdThreads rows of B'
// each (a thread per row), the rest kRsvdThreads columns of A' each (a
// thread per column).  Components c < min(k_a, r) come from W; the others
// (a retained rank above r, or padding up to the stored rank) are zero.
template <typename E>
__global__ void __launch_bounds__(kRsvdThreads) rsvd_write_kernel(RsvdWriteArgs p) {
  __shared__ double w[kRsvdR][kRsvdR];
  const int nb = p.nbo + (p.d_in + kRsvdThreads - 1) / kRsvdThreads;
  const int a = blockIdx.x / nb, blk = blockIdx.x - a * nb;
  const int tid = threadIdx.x, r = p.r;
  const int ro = p.row_off[a], stored = p.rank[a];
  const int k = min(p.true_rank[a], r);
  if (stored <= 0 || ro < 0 || ro > p.R - stored) return;  // uniform per workgroup
  const bool bside = blk < p.nbo;
  const double* W = (bside ? p.WB : p.WA) + (size_t)a * kRsvdR * kRsvdR;
  for (int e = tid; e < kRsvdR * kRsvdR; e += kRsvdThreads) w[e / kRsvdR][e % kRsvdR] = e / kRsvdR < r ? W[e] : 0.0;
  __syncthreads();
  typename E::storage* outA = reinterpret_cast<typename E::storage*>(p.A_pack);
  typename E::storage* outB = reinterpret_cast<typename E::storage*>(p.B_pack);
  if (bside) {
    const int o = blk * kRsvdThreads + tid;
    if (o >= p.d_out) return;
    const char* brow = p.B + ((size_t)a * p.d_out + o) * r * E::kBytes;
    double x[kRsvdR];
#pragma unroll
    for (int i = 0; i < kRsvdR; ++i) x[i] = i < r ? load_elem<E>(brow, i) : 0.0;
    const size_t base = (size_t)ro * p.d_out + (size_t)o * stored;
    for (int cc = 0; cc < stored; ++cc) {
      double s = 0.0;
      if (cc < k) {
#pragma unroll
        for (int i = 0; i < kRsvdR; ++i) s += x[i] * w[i][cc];
      }
      store_elem<E>(outB, base + cc, s);
    }
  } else {
    const int col = (blk - p.nbo) * kRsvdThreads + tid;
    if (col >= p.d_in) return;
    const char* abase = p.A + (size_t)a * r * p.d_in * E::kBytes;
    double x[kRsvdR];
#pragma unroll
    for (int i = 0; i < kRsvdR; ++i) x[i] = i < r ? load_elem<E>(abase, (int64_t)i * p.d_in + col) : 0.0;
    for (int cc = 0; cc < stored; ++cc) {
      double s = 0.0;
      if (cc < k) {
#pragma unroll
        for (int i = 0; i < kRsvdR; ++i) s += w[i][cc] * x[i];
      }
      store_elem<E>(outA, (size_t)(ro + cc) * p.d_in + col, s);
    }
  }
}

int rsvd_blocks(int d_in, int d_out) {
  const int d = d_in > d_out ? d_in : d_out;
  const int b = (d + kRsvdTile - 1) / kRsvdTile;
  return b < kRsvdMaxBlocks ? b : kRsvdMaxBlocks;
}

size_t rsvd_workspace_bytes(int n, int d_in, int d_out) {
  const size_t m = (size_t)kRsvdR * kRsvdR * sizeof(double);
  return (size_t)n * (2 * (size_t)rsvd_blocks(d_in, d_out) + 2) * m;
}

static RsvdArgs rsvd_args(int n, int d_in, int d_out, int r, const void* A, const void* B, float* sigma,
                          int32_t* status, void* ws) {
  RsvdArgs a;
  a.n = n;
  a.d_in = d_in;
  a.d_out = d_out;
  a.r = r;
  a.nblk = rsvd_blocks(d_in, d_out);
  a.A = reinterpret_cast<const char*>(A);
  a.B = reinterpret_cast<const char*>(B);
  const size_t m = (size_t)kRsvdR * kRsvdR;
  a.part = reinterpret_cast<double*>(ws);
  a.WB = a.part + (size_t)n * 2 * a.nblk * m;
  a.WA = a.WB + (size_t)n * m;
  a.sigma = sigma;
  a.status = status;
  return a;
}

hipError_t launch_rsvd_factor(int n, int d_in, int d_out, int dtype, int r, const void* A, const void* B,
                              float* sigma, int32_t* status, void* ws, hipStream_t stream) {
  const RsvdArgs a = rsvd_args(n, d_in, d_out, r, A, B, sigma, status, ws);
  const dim3 blk(kRsvdThreads);
  if (dtype == LORA_DTYPE_BF16)
    hipLaunchKernelGGL(rsvd_gram_kernel<BF16>, dim3((unsigned)(n * 2 * a.nblk)), blk, 0, stream, a);
  else
    hipLaunchKernelGGL(rsvd_gram_kernel<F32>, dim3((unsigned)(n * 2 * a.nblk)), blk, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)4 * kRsvdR * (kRsvdR + 1) * sizeof(double);
  static bool raised = false;
  if (!raised) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(rsvd_core_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL(rsvd_core_kernel, dim3((unsigned)n), blk, lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_rsvd_write(const lora_store& s, int r, const void* A, const void* B, const void* ws,
                             hipStream_t stream) {
  const RsvdArgs f = rsvd_args(s.n, s.d_in, s.d_out, r, A, B, nullptr, nullptr, const_cast<void*>(ws));
  RsvdWriteArgs a;
  a.n = s.n;
  a.d_in = s.d_in;
  a.d_out = s.d_out;
  a.r = r;
  a.R = s.R;
  a.nbo = (s.d_out + kRsvdThreads - 1) / kRsvdThreads;
  a.A = reinterpret_cast<const char*>(A);
  a.B = reinterpret_cast<const char*>(B);
  a.WB = f.WB;
  a.WA = f.WA;
  a.row_off = s.row_off;
  a.rank = s.rank;
  a.true_rank = s.rank + 2 * s.n;  // meta: row_off | rank | scale | true_rank
  a.A_pack = reinterpret_cast<char*>(const_cast<void*>(s.A_pack));
  a.B_pack = reinterpret_cast<char*>(const_cast<void*>(s.B_pack));
  const int nb = a.nbo + (s.d_in + kRsvdThreads - 1) / kRsvdThreads;
  const dim3 grid((unsigned)((int64_t)s.n * nb)), blk(kRsvdThreads);
  if (s.dtype == LORA_DTYPE_BF16) hipLaunchKernelGGL(rsvd_write_kernel<BF16>, grid, blk, 0, stream, a);
  else hipLaunchKernelGGL(rsvd_write_kernel<F32>, grid, blk, 0, stream, a);
  return hipGetLastError();
}

}  // namespace lora
