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
// B A = Q_B C Q_A^T with the r x r core C = R_B R_A^T.  With C = U S V^T,
// B' = Q_B U_k = B (R_B^-1 U_k) and A' = S_k V_k^T Q_A^T = U_k^T C Q_A^T =
// U_k^T R_B A, so W_B = R_B^-1 U and W_A = R_B^T U (V is never needed, nor Q).
//
//   rsvd_gram_kernel    the Gram matrix M^T M of one factor (M = B, or A^T):
//                       four waves each take every fourth block of rows,
//                       float64 MFMA (16x16x4) on the ten upper 16 x 16 tiles,
//                       the waves' parts summed in wave order.  R^T R = M^T M:
//                       this is the Cholesky form of the tall-skinny QR (one
//                       pass over the rows, the row blocks merged by a sum).
//                       bf16 and f32 inputs are exact in float64.
//   rsvd_prep_kernel    per adapter, two waves: the Cholesky factors R_B and
//                       R_A (a pivot at 1e-14 of the largest diagonal entry or
//                       below flags the adapter), then C = R_B R_A^T.
//   rsvd_jacobi_kernel  per adapter, two waves, lane j holding column j of C
//                       (half of its rows per wave) in registers:
//                       one-sided Jacobi, column pairs (j, j^m) for
//                       m = 1 .. 2^ceil(log2 r) - 1 (every pair once per
//                       sweep), partner rows fetched across lanes, column
//                       norms carried through each sweep's rotations, until
//                       every pair is orthogonal to 1e-15 or a sweep's
//                       rotations all had |tan| < 1e-4; then sigma_j = |C_j|,
//                       their descending order, U.
//   rsvd_post_kernel    per adapter, two waves: W_A = R_B^T U and
//                       W_B = R_B^-1 U (back substitution), columns in sigma
//                       order.
//   rsvd_write_kernel   B'[o, c] = sum_i B[o, i] W_B[i, c] and
//                       A'[c, k] = sum_i W_A[i, c] A[i, k] (float64) for
//                       c < k_a, into a store's A and B buffers at the store's
//                       row offsets and ranks.
#include "device_common.h"
#include "kernels.h"

namespace lora {

constexpr int kRsvdR = LORA_MAX_RANK;  // largest original rank
constexpr int kRsvdMat = kRsvdR * kRsvdR;
constexpr int kGramWaves = 4;
constexpr int kGramTiles = 10;  // upper 16 x 16 tiles of a 64 x 64 Gram
// Workspace, float64 matrices per adapter (64 x 64 each): the Grams of B and
// of A^T, the core C, R_B, U, W_B, W_A (W_B and W_A transposed).
constexpr int kWsGramB = 0, kWsGramA = 1, kWsC = 2, kWsRB = 3, kWsU = 4, kWsWB = 5, kWsWA = 6, kWsMats = 7;
constexpr int kJacobiWaves = 2;

typedef double f64x4_t __attribute__((ext_vector_type(4)));

struct RsvdArgs {
  int n, d_in, d_out, r;
  const char* A;  // [n][r][d_in]
  const char* B;  // [n][d_out][r]
  double* ws;     // [n][kWsMats][64][64]
  float* sigma;   // [n][r]
  int32_t* status;
};

__device__ __forceinline__ double* ws_mat(const RsvdArgs& p, int a, int m) {
  return p.ws + ((size_t)a * kWsMats + m) * kRsvdMat;
}

template <typename E>
__device__ __forceinline__ double load_elem(const char* base, int64_t i) {
  if constexpr (E::kBytes == 2) return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
  else return (double)reinterpret_cast<const float*>(base)[i];
}

// ------------------------------------------------------------------ Gram
// Wait for this wave's LDS writes before its lanes read each other's: LDS
// operations of one wave complete in order, so only the wave itself waits.
__device__ __forceinline__ void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup (adapter, side): side 0 = B (rows of r elements), side 1 = A^T
// (the columns of A).  A sub-chunk is E::kVec rows of M: side 0 reads it as r
// contiguous 16-byte vectors of B (lane l < r the l-th), side 1 as one
// 16-byte vector per row of A (lane l < r: A[l][k0 .. k0 + kVec)).  Wave w
// takes every fourth group of kGramSub sub-chunks, stages it in float64 in
// its own LDS tile (zero outside the r columns) and feeds 16 x 16 x 4 MFMAs:
// lane l holds M[k0 + l/16][16 b + l%16] as the A operand of tile row b and
// the B operand of tile column b.
constexpr int kGramSub = 2;
template <typename E, int NB>
__global__ void __launch_bounds__(kGramWaves * 64) rsvd_gram_kernel(RsvdArgs p) {
  constexpr int KV = E::kVec;                // rows per sub-chunk
  constexpr int kRows = kGramSub * KV;       // rows per group
  constexpr int kStage = kGramWaves * kRows * kRsvdR;         // doubles
  constexpr int kRed = (kGramWaves - 1) * kGramTiles * 256;   // doubles
  __shared__ __align__(16) double lds[kStage > kRed ? kStage : kRed];
  const int a = blockIdx.x >> 1, side = blockIdx.x & 1;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = p.r;
  const int D = side == 0 ? p.d_out : p.d_in;
  const int nsub = D / KV;
  const int ngroups = (nsub + kGramSub - 1) / kGramSub;
  double* tile = lds + (size_t)w * kRows * kRsvdR;
  for (int e = l; e < kRows * kRsvdR; e += 64) tile[e] = 0.0;
  const char* base = side == 0 ? p.B + (size_t)a * p.d_out * r * E::kBytes
                               : p.A + (size_t)a * r * p.d_in * E::kBytes;
  // Side 0: the kVec elements of lane l's vector sit at flat offsets
  // l * KV + t of the sub-chunk, i.e. (row, col) = divmod(l * KV + t, r).
  const int e0 = l * KV, row0 = e0 / r, col0 = e0 - row0 * r;
  const bool whole = r % KV == 0;  // side 0: a vector never crosses a row
  f64x4_t acc[kGramTiles];
#pragma unroll
  for (int t = 0; t < kGramTiles; ++t) acc[t] = (f64x4_t){0.0, 0.0, 0.0, 0.0};
  auto load = [&](int c) -> uint4 {
    if (c >= nsub || l >= r) return make_uint4(0u, 0u, 0u, 0u);
    const size_t off = side == 0 ? ((size_t)c * KV * r + (size_t)l * KV) : ((size_t)l * p.d_in + (size_t)c * KV);
    return ld16(base + off * E::kBytes);
  };
  // Groups in flight: the one being staged and the next.
  uint4 q[2][kGramSub];
#pragma unroll
  for (int u = 0; u < kGramSub; ++u) {
    q[0][u] = load(w * kGramSub + u);
    q[1][u] = load((w + kGramWaves) * kGramSub + u);
  }
  for (int g = w; g < ngroups; g += kGramWaves) {
#pragma unroll
    for (int u = 0; u < kGramSub; ++u) {
      if (l < r) {
        float f[KV];
        E::widen(q[0][u], f);
        double* sub = tile + u * KV * kRsvdR;
        if (side == 1) {
#pragma unroll
          for (int t = 0; t < KV; ++t) sub[t * kRsvdR + l] = (double)f[t];
        } else if (whole) {
#pragma unroll
          for (int t = 0; t < KV; t += 2) {
            double2 v2;
            v2.x = (double)f[t];
            v2.y = (double)f[t + 1];
            *reinterpret_cast<double2*>(&sub[row0 * kRsvdR + col0 + t]) = v2;
          }
        } else {
          int row = row0, col = col0;
#pragma unroll
          for (int t = 0; t < KV; ++t) {
            sub[row * kRsvdR + col] = (double)f[t];
            if (++col == r) {
              col = 0;
              ++row;
            }
          }
        }
      }
      q[0][u] = q[1][u];
      q[1][u] = load((g + 2 * kGramWaves) * kGramSub + u);
    }
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < kRows / 4; ++s) {
      double x[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) x[b] = b < NB ? tile[(4 * s + (l >> 4)) * kRsvdR + 16 * b + (l & 15)] : 0.0;
      int t = 0;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = ib; jb < 4; ++jb, ++t)
          if (jb < NB) acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(x[ib], x[jb], acc[t], 0, 0, 0);
    }
    // The MFMAs consumed this wave's reads before the next group's writes
    // (which cover every (row, column < r) of the tile, with zeros past the
    // end of M).
    wave_lds_sync();
  }
  __syncthreads();  // every wave is done with its staging tile
  if (w > 0) {
#pragma unroll
    for (int t = 0; t < kGramTiles; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) lds[((w - 1) * kGramTiles + t) * 256 + v * 64 + l] = acc[t][v];
  }
  __syncthreads();
  if (w == 0) {
    double* G = ws_mat(p, a, side == 0 ? kWsGramB : kWsGramA);
    int t = 0;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = ib; jb < 4; ++jb, ++t) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          double s = acc[t][v];
#pragma unroll
          for (int ww = 0; ww < kGramWaves - 1; ++ww) s += lds[(ww * kGramTiles + t) * 256 + v * 64 + l];
          // MFMA result layout: lane l, element v holds row 4 v + l / 16,
          // column l % 16 of the tile.
          const int i = 16 * ib + 4 * v + (l >> 4), j = 16 * jb + (l & 15);
          G[i * kRsvdR + j] = s;
          if (ib != jb) G[j * kRsvdR + i] = s;
        }
      }
  }
}

// ------------------------------------------------------------------ prep
// Upper Cholesky factor of m (lane c owns column c; R in the upper triangle,
// the lower triangle zeroed), left-looking: step j forms row j of R from the
// rows above it, R[j][c] = (G[j][c] - sum_{k<j} R[k][j] R[k][c]) / R[j][j],
// with only reads in its sums (every lane also forms the pivot, in the same
// order, so all agree on it), then one write per lane and one barrier.
// Pivot rules as in the file comment; a pivot at or below 1e-30 of the
// largest diagonal entry, or not positive, is raised to that floor so the
// factorization finishes (a zero column gives a zero row of R but for a tiny
// diagonal).
__device__ void cholesky_lanes(double (*m)[kRsvdR + 1], int r, int c, int* bad) {
  double dmax = 0.0;
  for (int j = 0; j < r; ++j) dmax = fmax(dmax, m[j][j]);
  const double warn = 1e-14 * dmax, floor_v = fmax(1e-30 * dmax, 1e-300);
  __syncthreads();  // every lane has read the diagonal before it changes
  for (int j = 0; j < r; ++j) {
    double dg[4] = {0.0, 0.0, 0.0, 0.0}, ac[4] = {0.0, 0.0, 0.0, 0.0};
    int k = 0;
    for (; k + 3 < j; k += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double rkj = m[k + u][j];
        dg[u] = fma(rkj, rkj, dg[u]);
        ac[u] = fma(rkj, m[k + u][c], ac[u]);
      }
    }
    for (; k < j; ++k) {
      const double rkj = m[k][j];
      dg[0] = fma(rkj, rkj, dg[0]);
      ac[0] = fma(rkj, m[k][c], ac[0]);
    }
    double d2 = m[j][j] - ((dg[0] + dg[1]) + (dg[2] + dg[3]));
    const double g = m[j][c] - ((ac[0] + ac[1]) + (ac[2] + ac[3]));
    if (!(d2 > warn) && c == 0) *bad = 1;
    if (!(d2 > floor_v)) d2 = floor_v;
    const double d = sqrt(d2);
    if (c == j) m[j][j] = d;
    else if (c > j && c < r) m[j][c] = g / d;
    __syncthreads();
  }
  for (int i = c + 1; i < kRsvdR; ++i) m[i][c] = 0.0;
  __syncthreads();
}

// Workgroup per adapter: wave 0 factors B's Gram, wave 1 A^T's; then wave w
// forms rows 32 w .. 32 w + 31 of C = R_B R_A^T (lane j: column j).
__global__ void __launch_bounds__(128) rsvd_prep_kernel(RsvdArgs p) {
  __shared__ double m[2][kRsvdR][kRsvdR + 1];
  __shared__ int s_bad;
  const int a = blockIdx.x, tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = p.r;
  if (tid == 0) s_bad = 0;
  const double* G = ws_mat(p, a, w == 0 ? kWsGramB : kWsGramA);
  for (int i = 0; i < kRsvdR; ++i) m[w][i][l] = G[i * kRsvdR + l];
  __syncthreads();
  cholesky_lanes(m[w], r, l, &s_bad);
  double c[32];
#pragma unroll
  for (int ii = 0; ii < 32; ++ii) c[ii] = 0.0;
  for (int k = 0; k < r; ++k) {
    const double raj = m[1][l][k];  // R_A[j][k], j = l
#pragma unroll
    for (int ii = 0; ii < 32; ++ii) c[ii] = fma(m[0][32 * w + ii][k], raj, c[ii]);
  }
  double* C = ws_mat(p, a, kWsC);
#pragma unroll
  for (int ii = 0; ii < 32; ++ii) C[(32 * w + ii) * kRsvdR + l] = c[ii];
  if (w == 0) {
    double* RB = ws_mat(p, a, kWsRB);
    for (int i = 0; i < kRsvdR; ++i) RB[i * kRsvdR + l] = m[0][i][l];
  }
  __syncthreads();
  if (tid == 0) p.status[a] = s_bad;
}

// ---------------------------------------------------------------- Jacobi
// 1 / x and 1 / sqrt(x) for the rotation: the hardware estimates refined by
// two Newton steps each (to within an ulp or so; the rotation only needs
// cos^2 + sin^2 = 1 to working precision, not correct rounding).
__device__ __forceinline__ double rcp_nr(double x) {
  double y = __builtin_amdgcn_rcp(x);
  y = fma(y, fma(-x, y, 1.0), y);
  return fma(y, fma(-x, y, 1.0), y);
}
__device__ __forceinline__ double rsq_nr(double x) {
  double y = __builtin_amdgcn_rsq(x);
  const double hx = 0.5 * x;
  y = y * fma(-hx * y, y, 1.5);
  return y * fma(-hx * y, y, 1.5);
}

// Workgroup of two waves per adapter; RB = the rank rounded up to a power of
// two (>= 8), rows and pairings beyond it all zero.  Lane j of wave h holds
// rows h RB/2 .. (h + 1) RB/2 - 1 of column j in registers.  In the round of
// m, column j meets column j ^ m: the partner's rows come from lane j ^ m of
// the same wave; each wave's partial dot product C_j . C_p goes through LDS
// and every wave adds the parts in wave order, so both lanes of a
// pair, in both waves, take the same rotation.
template <int RB>
__global__ void __launch_bounds__(kJacobiWaves * 64) rsvd_jacobi_kernel(RsvdArgs p) {
  constexpr int RPW = RB / kJacobiWaves;  // rows per wave
  __shared__ double part[2][kJacobiWaves][64];
  const int a = blockIdx.x, tid = threadIdx.x, h = tid >> 6, j = tid & 63, r = p.r;
  const double* C = ws_mat(p, a, kWsC);
  double* U = ws_mat(p, a, kWsU);
  double c[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) c[i] = C[(h * RPW + i) * kRsvdR + j];
  int buf = 0;
  // |C_j|^2 over the four waves' rows, summed in wave order (the same bits in
  // every wave).
  auto column_norm = [&](double* nrm) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < RPW; ++i) s = fma(c[i], c[i], s);
    part[buf][h][j] = s;
    __syncthreads();
    s = 0.0;
#pragma unroll
    for (int hh = 0; hh < kJacobiWaves; ++hh) s += part[buf][hh][j];
    buf ^= 1;
    *nrm = s;
  };
  for (int sweep = 0; sweep < 40; ++sweep) {
    // Squared norms are computed exactly once a sweep and carried through
    // its rotations (a rotation by tan = t moves t * gamma from the lower
    // column's norm to the upper's).
    double nrm;
    column_norm(&nrm);
    bool rot = false;  // a rotation with |tan| >= 1e-4 this sweep
    for (int mm = 1; mm < RB; ++mm, buf ^= 1) {
      const bool lower = j < (j ^ mm);
      double y[RPW];
      double g4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        y[i] = __shfl_xor(c[i], mm);
        g4[i & 3] = fma(c[i], y[i], g4[i & 3]);
      }
      double g = (g4[0] + g4[1]) + (g4[2] + g4[3]);
      const double pn = __shfl_xor(nrm, mm);
      if constexpr (kJacobiWaves > 1) {
        part[buf][h][j] = g;
        __syncthreads();
        g = 0.0;
#pragma unroll
        for (int hh = 0; hh < kJacobiWaves; ++hh) g += part[buf][hh][j];
      }
      // Both lanes of a pair see the same alpha (lower column), beta, gamma.
      const double al = lower ? nrm : pn, be = lower ? pn : nrm;
      if (g != 0.0 && g * g > 1e-30 * (al * be)) {
        const double zeta = (be - al) * rcp_nr(2.0 * g);
        const double z2 = fma(zeta, zeta, 1.0);
        const double t = copysign(rcp_nr(fabs(zeta) + z2 * rsq_nr(z2)), zeta);
        const double cs = rsq_nr(fma(t, t, 1.0)), sn = cs * t;
        // Lower column: cs c - sn c_partner; upper: cs c + sn c_partner.
        const double ssn = lower ? -sn : sn;
#pragma unroll
        for (int i = 0; i < RPW; ++i) c[i] = fma(ssn, y[i], cs * c[i]);
        nrm = fma(lower ? -t : t, g, nrm);
        rot = rot || fabs(t) >= 1e-4;
      }
    }
    // Every wave took the same decisions, so every wave leaves together.  A
    // sweep whose rotations all had |tan| < 1e-4 leaves off-diagonal terms of
    // about that order squared (quadratic convergence; about 1e-12 relative
    // on rank-64 cores): no further sweep.  Large rotations (close singular
    // values) never stop it early.
    if (!__any(rot)) break;
  }
  double s2;
  column_norm(&s2);
  const double sg = sqrt(s2);
  // Descending order, ties (and a NaN, ranked last) by lane: a permutation.
  const double key = sg == sg ? sg : -1.0;
  int pos = 0;
  for (int k = 0; k < 64; ++k) {
    const double o = __shfl(key, k);
    pos += (o > key || (o == key && k < j)) ? 1 : 0;
  }
  const double inv = sg > 0.0 ? 1.0 / sg : 0.0;
#pragma unroll
  for (int i = 0; i < RPW; ++i) U[(h * RPW + i) * kRsvdR + pos] = c[i] * inv;
  for (int i = RB + h; i < kRsvdR; i += kJacobiWaves) U[i * kRsvdR + pos] = 0.0;
  if (h == 0 && j < r) p.sigma[(size_t)a * r + pos] = (float)sg;
}

// ------------------------------------------------------------------ post
// Two waves per adapter, lane c of each holding column c of U: wave 0 forms
// column c of W_A = R_B^T U, wave 1 column c of W_B = R_B^-1 U (row-oriented
// back substitution in LDS); each is written as row c of the transposed
// matrix, with rows past r zero.
__global__ void __launch_bounds__(128) rsvd_post_kernel(RsvdArgs p) {
  __shared__ double rb[kRsvdR][kRsvdR + 1];
  __shared__ double x[kRsvdR][kRsvdR + 1];
  const int a = blockIdx.x, tid = threadIdx.x, w = tid >> 6, c = tid & 63, r = p.r;
  const double* RB = ws_mat(p, a, kWsRB);
  const double* U = ws_mat(p, a, kWsU);
  for (int k = w; k < kRsvdR; k += 2) rb[k][c] = RB[k * kRsvdR + c];
  if (w == 1)
    for (int k = 0; k < kRsvdR; ++k) x[k][c] = U[k * kRsvdR + c];
  __syncthreads();
  if (w == 0) {
    double* WA = ws_mat(p, a, kWsWA);
    double u[kRsvdR];
#pragma unroll
    for (int k = 0; k < kRsvdR; ++k) u[k] = U[k * kRsvdR + c];
    for (int i = 0; i < kRsvdR; ++i) {  // rb and u are zero past r
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int k = 0; k < kRsvdR; ++k) s4[k & 3] = fma(rb[k][i], u[k], s4[k & 3]);  // rb is zero below the diagonal
      WA[c * kRsvdR + i] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
  } else {
    double* WB = ws_mat(p, a, kWsWB);
    for (int i = r; i < kRsvdR; ++i) WB[c * kRsvdR + i] = 0.0;
    for (int i = r - 1; i >= 0; --i) {
      double s4[4] = {0.0, 0.0, 0.0, 0.0};
      int k = i + 1;
      for (; k + 3 < r; k += 4)
#pragma unroll
        for (int q = 0; q < 4; ++q) s4[q] = fma(rb[i][k + q], x[k + q][c], s4[q]);
      for (; k < r; ++k) s4[0] = fma(rb[i][k], x[k][c], s4[0]);
      const double s = (x[i][c] - ((s4[0] + s4[1]) + (s4[2] + s4[3]))) / rb[i][i];
      x[i][c] = s;
      WB[c * kRsvdR + i] = s;
    }
  }
}

// ----------------------------------------------------------------- write
struct RsvdWriteArgs {
  int n, d_in, d_out, r, R, nbo;  // nbo: row blocks of B' (256 rows each)
  const int32_t* row_off;
  const int32_t* rank;       // stored rank
  const int32_t* true_rank;  // retained rank k_a
};

template <typename E>
__device__ __forceinline__ void store_elem(typename E::storage* out, size_t i, double v) {
  if constexpr (E::kBytes == 2) out[i] = (uint16_t)f32_to_bf16((float)v);
  else out[i] = (float)v;
}

// Workgroup (adapter, block): blocks [0, nbo) write 256 rows of B' each, the
// rest 256 columns of A' each.  The workgroup first copies its tile of B
// (256 whole rows) or of A (all r rows, 256 columns) into LDS with coalesced
// 16-byte loads (element by element when B's rows are not 16-byte
// multiples).  Then float64 MFMA (16 x 16 x 4), K = the original rank:
//   B side: D[row][c] = sum_i B[row][i] W_B[i][c]   (M = 16 rows, N = 16 components)
//   A side: D[c][col] = sum_i W_A[i][c] A[i][col]   (M = 16 components, N = 16 columns)
// W operand: lane l holds W[4 s + l/16][c0 + l%16] (zero for components at or
// past min(k_a, r), so that padding up to the stored rank comes out zero);
// tile operand: lane l holds the tile value at (row or column l%16, rank
// 4 s + l/16), zero past r.  Wave w takes the tile's 16-row (16-column) blocks
// w, w + 4, w + 8, w + 12.  Result layout: lane l, element v holds row 4 v +
// l/16, column l%16 of the 16 x 16 block.
template <typename E, int RB>
__global__ void __launch_bounds__(256) rsvd_write_kernel(RsvdWriteArgs p, const char* __restrict__ A,
                                                         const char* __restrict__ B, const double* __restrict__ ws,
                                                         typename E::storage* __restrict__ outA,
                                                         typename E::storage* __restrict__ outB) {
  typedef typename E::storage S;
  constexpr int KV = E::kVec;
  constexpr int KS = RB / 4;       // K steps
  constexpr int kRowB = RB + KV;  // padded B row in LDS (elements), 16-byte multiple
  constexpr int kTileB = 256 * kRowB, kTileA = RB * 256;
  __shared__ __align__(16) S tile[kTileB > kTileA ? kTileB : kTileA];
  const int nb = p.nbo + (p.d_in + 255) / 256;
  const int a = blockIdx.x / nb, blk = blockIdx.x - a * nb;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = p.r;
  const int ro = p.row_off[a], stored = p.rank[a];
  const int k = min(p.true_rank[a], r);
  if (stored <= 0 || ro < 0 || ro > p.R - stored) return;  // uniform per workgroup
  const bool bside = blk < p.nbo;
  const double* __restrict__ Wt = ws + ((size_t)a * kWsMats + (bside ? kWsWB : kWsWA)) * kRsvdMat;
  auto widen1 = [](S v) -> double {
    if constexpr (E::kBytes == 2) return (double)__uint_as_float((uint32_t)v << 16);
    else return (double)v;
  };
  const int li = l >> 4, lj = l & 15;
  int n0 = 0, nrows = 0;  // the tile's first row (B) or column (A), and how many
  if (bside) {
    n0 = blk * 256;
    nrows = min(256, p.d_out - n0);
    const char* bblk = B + ((size_t)a * p.d_out + n0) * r * E::kBytes;
    if (r % KV == 0) {
      const int vpr = r / KV;  // 16-byte vectors per row
      for (int v = tid; v < nrows * vpr; v += 256) {
        const int row = v / vpr, c0 = (v - row * vpr) * KV;
        *reinterpret_cast<uint4*>(&tile[row * kRowB + c0]) = ld16(bblk + (size_t)v * 16);
      }
    } else {
      const S* src = reinterpret_cast<const S*>(bblk);
      for (int e = tid; e < nrows * r; e += 256) tile[(e / r) * kRowB + e % r] = src[e];
    }
  } else {
    n0 = (blk - p.nbo) * 256;
    nrows = min(256, p.d_in - n0);
    const char* ablk = A + ((size_t)a * r * p.d_in + n0) * E::kBytes;
    const int vpr = 256 / KV;  // 16-byte vectors per tile row
    for (int v = tid; v < r * vpr; v += 256) {
      const int i = v / vpr, c0 = (v - i * vpr) * KV;
      if (c0 < nrows)  // d_in is a multiple of KV: a vector is wholly in or out
        *reinterpret_cast<uint4*>(&tile[i * 256 + c0]) = ld16(ablk + ((size_t)i * p.d_in + c0) * E::kBytes);
    }
  }
  __syncthreads();
  const int nblocks = (nrows + 15) / 16;
  for (int c0 = 0; c0 < stored; c0 += 16) {  // 16 components at a time
    const int cw = c0 + lj;                  // this lane's component in the W operand
    double wv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int i = 4 * s + li;
      wv[s] = (cw < k && i < r) ? Wt[cw * kRsvdR + i] : 0.0;
    }
    for (int b = w; b < nblocks; b += 4) {
      const int m0 = b * 16;  // first row (B) or column (A) of the block in the tile
      f64x4_t acc = (f64x4_t){0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int i = 4 * s + li;
        const double tv = i < r ? widen1(bside ? tile[(m0 + lj) * kRowB + i] : tile[i * 256 + m0 + lj]) : 0.0;
        acc = bside ? __builtin_amdgcn_mfma_f64_16x16x4f64(tv, wv[s], acc, 0, 0, 0)
                    : __builtin_amdgcn_mfma_f64_16x16x4f64(wv[s], tv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = 4 * v + li;  // row of the 16 x 16 result
        if (bside) {
          const int row = m0 + rr, c = c0 + lj;
          if (row < nrows && c < stored)
            store_elem<E>(outB, (size_t)ro * p.d_out + (size_t)(n0 + row) * stored + c, acc[v]);
        } else {
          const int c = c0 + rr, col = m0 + lj;
          if (c < stored && col < nrows) store_elem<E>(outA, (size_t)(ro + c) * p.d_in + n0 + col, acc[v]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host
size_t rsvd_workspace_bytes(int n) { return (size_t)n * kWsMats * kRsvdMat * sizeof(double); }

static RsvdArgs rsvd_args(int n, int d_in, int d_out, int r, const void* A, const void* B, float* sigma,
                          int32_t* status, void* ws) {
  RsvdArgs a;
  a.n = n;
  a.d_in = d_in;
  a.d_out = d_out;
  a.r = r;
  a.A = reinterpret_cast<const char*>(A);
  a.B = reinterpret_cast<const char*>(B);
  a.ws = reinterpret_cast<double*>(ws);
  a.sigma = sigma;
  a.status = status;
  return a;
}

template <typename E>
static void launch_gram(const RsvdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(2 * a.n)), blk(kGramWaves * 64);
  if (a.r <= 16) hipLaunchKernelGGL((rsvd_gram_kernel<E, 1>), grid, blk, 0, stream, a);
  else if (a.r <= 32) hipLaunchKernelGGL((rsvd_gram_kernel<E, 2>), grid, blk, 0, stream, a);
  else hipLaunchKernelGGL((rsvd_gram_kernel<E, 4>), grid, blk, 0, stream, a);
}

hipError_t launch_rsvd_factor(int n, int d_in, int d_out, int dtype, int r, const void* A, const void* B,
                              float* sigma, int32_t* status, void* ws, hipStream_t stream, int phases) {
  const RsvdArgs a = rsvd_args(n, d_in, d_out, r, A, B, sigma, status, ws);
  hipError_t e;
  if (phases & 1) {
    if (dtype == LORA_DTYPE_BF16) launch_gram<BF16>(a, stream);
    else launch_gram<F32>(a, stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 2) {
    hipLaunchKernelGGL(rsvd_prep_kernel, dim3((unsigned)n), dim3(128), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 4) {
    const dim3 grid((unsigned)n), blk(kJacobiWaves * 64);
    if (r <= 8) hipLaunchKernelGGL(rsvd_jacobi_kernel<8>, grid, blk, 0, stream, a);
    else if (r <= 16) hipLaunchKernelGGL(rsvd_jacobi_kernel<16>, grid, blk, 0, stream, a);
    else if (r <= 32) hipLaunchKernelGGL(rsvd_jacobi_kernel<32>, grid, blk, 0, stream, a);
    else hipLaunchKernelGGL(rsvd_jacobi_kernel<64>, grid, blk, 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (phases & 8) {
    hipLaunchKernelGGL(rsvd_post_kernel, dim3((unsigned)n), dim3(128), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename E>
static void launch_write(const RsvdWriteArgs& a, dim3 grid, const void* A, const void* B, const void* ws,
                         const lora_store& s, hipStream_t stream) {
  const char* pa = reinterpret_cast<const char*>(A);
  const char* pb = reinterpret_cast<const char*>(B);
  const double* w = reinterpret_cast<const double*>(ws);
  auto* oa = reinterpret_cast<typename E::storage*>(const_cast<void*>(s.A_pack));
  auto* ob = reinterpret_cast<typename E::storage*>(const_cast<void*>(s.B_pack));
  const dim3 blk(256);
  if (a.r <= 8) hipLaunchKernelGGL((rsvd_write_kernel<E, 8>), grid, blk, 0, stream, a, pa, pb, w, oa, ob);
  else if (a.r <= 16) hipLaunchKernelGGL((rsvd_write_kernel<E, 16>), grid, blk, 0, stream, a, pa, pb, w, oa, ob);
  else if (a.r <= 32) hipLaunchKernelGGL((rsvd_write_kernel<E, 32>), grid, blk, 0, stream, a, pa, pb, w, oa, ob);
  else hipLaunchKernelGGL((rsvd_write_kernel<E, 64>), grid, blk, 0, stream, a, pa, pb, w, oa, ob);
}

hipError_t launch_rsvd_write(const lora_store& s, int r, const void* A, const void* B, const void* ws,
                             hipStream_t stream) {
  RsvdWriteArgs a;
  a.n = s.n;
  a.d_in = s.d_in;
  a.d_out = s.d_out;
  a.r = r;
  a.R = s.R;
  a.nbo = (s.d_out + 255) / 256;
  a.row_off = s.row_off;
  a.rank = s.rank;
  a.true_rank = s.rank + 2 * s.n;  // meta: row_off | rank | scale | true_rank
  const int nb = a.nbo + (s.d_in + 255) / 256;
  const dim3 grid((unsigned)((int64_t)s.n * nb));
  if (s.dtype == LORA_DTYPE_BF16) launch_write<BF16>(a, grid, A, B, ws, s, stream);
  else launch_write<F32>(a, grid, A, B, ws, s, stream);
  return hipGetLastError();
}

}  // namespace lora
