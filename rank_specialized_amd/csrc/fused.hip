// The base layer with the adapter branch fused into its epilogue:
//
//   y[t] = W0 x[t] + s_a B_a h[t],   h[t] = A_a x[t]  (a = the token's adapter)
//
// "Compress then Serve" section 3: the adapted layer computes (W0 + B A) x;
// section 11: the base product W0 x is shared by every request of a batch and
// each request adds its own branch.  Here the branch enters the base
// product's float32 accumulators before y is rounded, so y is written once,
// instead of written by the base product and then read and written again by
// the expand.
//
// Tiles of 256 outputs x 256 tokens; 8 waves, each 128 x 64 (2 x 4); K
// staged 64 values at a time into LDS by buffer loads that write LDS
// directly (no registers in between), two buffers of 64 KiB (W0 rows and x
// rows, 128 bytes per row, its eight 16-byte chunks permuted by row & 7 so
// that the MFMA reads of 8 consecutive rows hit distinct banks).
// Products on v_mfma_f32_32x32x16_bf16 with W0 on the output side and x on
// the token side: a lane's accumulators hold 4 consecutive outputs of one
// token.  Tokens are taken in grouped order (adapters ascending, from the
// grouping), rows of x and y gathered through perm, so a 32-token block
// holds few adapters where adapters have many tokens.
//
// The branch: per 32-token block, the distinct adapters of its tokens, each
// rank range cut into groups of 8 ranks, are appended to the products as
// extra K: the output side is B_a[o][j0 .. j0+8), the token side
// s_a h[t][j0 .. j0+8) for the tokens of that adapter and 0 for the others.
// h is the sum of the shrink's float32 partial sums, entering as the exact
// pair hi + lo of bf16 values (about 16 significant bits), as in the expand.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "host_util.h"
#include "kernels.h"
#include "tile_ops.h"

namespace lora {
namespace {

constexpr int kFT = 256;                                // outputs and tokens per tile
constexpr int kFK = 64;                                 // K values per stage
constexpr int kFNB = 2;                                 // stage buffers: loads run kFNB - 1 stages ahead
constexpr int kFWaves = 8;                              // 2 (outputs) x 4 (tokens), two per SIMD
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFTokW = kFT / (kFWaves / 2);             // tokens per wave
constexpr int kFTB = kFTokW / 32;                       // 32-token blocks per wave
constexpr int kFRowsPerWave = kFT / kFWaves;            // rows of each operand one wave loads
constexpr int kFChunks = kFK / 8;                       // 16-byte chunks per row of a stage
constexpr int kFRowBytes = kFK * 2;
constexpr int kFOperandBytes = kFT * kFRowBytes;
constexpr int kFStageBytes = 2 * kFOperandBytes;        // W0 rows, then x rows
constexpr int kFRowsPerLoad = 64 / kFChunks;            // rows one wave-wide 16-byte load fills
constexpr int kFLoads = kFRowsPerWave / kFRowsPerLoad;  // such loads per wave, operand and stage
constexpr int kFKSub = kFK / 16;                        // MFMA K steps per stage
constexpr int kFBlockGroups = 32 * (LORA_MAX_RANK / 8);  // rank groups of one 32-token block, at most
constexpr int kFTableBytes = kFTB * kFBlockGroups * 8;       // one wave's rank-group tables
constexpr int kFLdsBytes = kFNB * kFStageBytes + kFWaves * kFTableBytes;
constexpr int kFGroupT = 4;  // token tiles per group of the tile order

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// 32 x 32 output block, float32 accumulate: lane l supplies row (l % 32) of
// each operand and the K-slice of lane group l / 32; it holds column l % 32,
// rows 8 (v / 4) + 4 (l / 32) + v % 4 of the result (v = 0..15).
__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

struct FusedArgs {
  const char* w;  // W0 [d_out] rows of ldw_bytes
  int64_t ldw_bytes;
  const char* x;  // x [T] rows of ldx_bytes (T * ldx_bytes < 2^31)
  int64_t ldx_bytes;
  char* y;
  int64_t ldy_bytes;
  int T, d_in, d_out;
  const int32_t* perm;  // grouped position -> token; nullptr: identity
  const int32_t* ids;   // nullptr: no branch
  int n;
  const char* b_pack;  // the store's B, b_bytes < 2^31
  uint32_t b_bytes;
  const int32_t* row_off;
  const int32_t* rank;
  const float* scale;
  const uint16_t* hs;  // s h per grouped position: [T][2][ldp] bf16 (hi, lo)
  int64_t ldp;
  int tiles_o, tiles_t;
};

// Block b -> tile.  Workgroups are dealt to the 8 XCDs in turn (b % 8); the
// remap gives each XCD a run of consecutive tiles, and the order walks
// groups of kFGroupT token tiles across all output tiles, so the tiles an
// XCD holds at once share their x and W0 rows in its L2.
__device__ __forceinline__ void tile_of(int b, int nb, int tiles_o, int tiles_t, int& to, int& tt) {
  const int q = nb >> 3, rem = nb & 7, xcd = b & 7;
  const int g = xcd * q + (xcd < rem ? xcd : rem) + (b >> 3);
  const int width = kFGroupT * tiles_o;
  const int grp = g / width, first = grp * kFGroupT;
  const int gt = tiles_t - first < kFGroupT ? tiles_t - first : kFGroupT;
  const int in = g - grp * width;
  tt = first + in % gt;
  to = in / gt;
}

__device__ __forceinline__ uint4 lds16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// LDS slot of 16-byte chunk c of stage row r.  An MFMA read has 16 lanes in
// flight per cycle (64 banks of 4 bytes), rows r .. r + 15 at one chunk: the
// slot permutation spreads them over all banks (rows of 128 bytes: row
// pairs share a slot, the two rows of a pair sit on opposite bank halves;
// rows of 64 bytes: each 4-row group on its own quarter).
__device__ __forceinline__ int chunk_slot(int r, int c) {
  if constexpr (kFChunks == 8) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);
}

// 16 bytes per lane from a buffer into LDS at dst + 16 * lane (dst the same
// for the whole wave); an offset out of the buffer's range writes zeros.
__device__ __forceinline__ void lds_dma16(rsrc_t r, char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}
// Wait until at most N of this wave's buffer loads are outstanding (they
// complete in issue order); the other counters left at their maxima.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}


// Where a lane's loads of a stage come from: the two buffers (W0 rows of the
// tile, all x rows) and per load the offset of the lane's row and chunk.
struct StageLoader {
  rsrc_t rw, rx;
  uint32_t vw[kFLoads], vx[kFLoads];
  int k8[kFLoads];  // first K value of the lane's chunk of each load
};

// The loads of one stage (K values k0 .. k0 + kFK) into `dst`, the wave's
// first row of the W0 half of a stage buffer.
__device__ __forceinline__ void issue_stage(const StageLoader& L, char* dst, int k0, int d_in) {
#pragma unroll
  for (int q = 0; q < kFLoads; ++q) {
    const bool kv = k0 + L.k8[q] < d_in;  // chunks past d_in read as zero
    lds_dma16(L.rw, dst + q * kFRowsPerLoad * kFRowBytes, kv ? L.vw[q] : kOutOfRange, (uint32_t)(2 * k0));
    lds_dma16(L.rx, dst + kFOperandBytes + q * kFRowsPerLoad * kFRowBytes, kv ? L.vx[q] : kOutOfRange,
              (uint32_t)(2 * k0));
  }
}

// One stage of the loop: the loads of a later stage into `wr` (when `load`),
// `mid`, and the products of the stage at `wa` (W0 rows of the wave) and `xa`
// (its x rows).  The pointers are restrict: the buffers differ, so the
// compiler need not hold the LDS reads until the loads into `wr` land (the
// loop orders buffers and loads with its own waits and barriers).
template <typename Mid>
__device__ __forceinline__ void stage_step(const char* __restrict__ wa, const char* __restrict__ xa,
                                           char* __restrict__ wr, bool load, int k0, const StageLoader& L,
                                           int d_in, const uint32_t (&ra)[kFKSub], f32x16_t (&acc)[kFTB][4],
                                           Mid&& mid) {
  if (load) issue_stage(L, wr, k0, d_in);
  mid();  // work between the loads and the products (the branch)
  // Fragments of K step kk + 1 are read while the products of step kk run.
  uint4 a[2][4], b[2][kFTB];
#pragma unroll
  for (int ob = 0; ob < 4; ++ob) a[0][ob] = lds16(wa + ob * 32 * kFRowBytes + ra[0]);
#pragma unroll
  for (int tb = 0; tb < kFTB; ++tb) b[0][tb] = lds16(xa + tb * 32 * kFRowBytes + ra[0]);
#pragma unroll
  for (int kk = 0; kk < kFKSub; ++kk) {
    const int c = kk & 1, nx = c ^ 1;
    if (kk + 1 < kFKSub) {
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) a[nx][ob] = lds16(wa + ob * 32 * kFRowBytes + ra[kk + 1]);
#pragma unroll
      for (int tb = 0; tb < kFTB; ++tb) b[nx][tb] = lds16(xa + tb * 32 * kFRowBytes + ra[kk + 1]);
    }
#pragma unroll
    for (int tb = 0; tb < kFTB; ++tb)
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) acc[tb][ob] = mfma32(a[c][ob], b[c][tb], acc[tb][ob]);
  }
  // Issue order: the first step's reads, then each step's products with the
  // next step's reads spread between them, so the matrix core does not wait
  // for LDS after the first step.
  constexpr int kReads = 4 + kFTB, kProducts = 4 * kFTB;
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
  for (int kk = 0; kk + 1 < kFKSub; ++kk) {
#pragma unroll
    for (int i = 0; i < kReads; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kProducts - kReads, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kProducts, 0);
}

// s_a h[t] of every grouped position as the exact pair hi + lo of bf16
// values, for the fused kernel's branch: hs[pos][0][j] = hi, hs[pos][1][j] =
// lo, zero at j >= r_a (h = the sum of the shrink's partial sums, in chunk
// order).  One thread per position and 8 ranks.
__global__ __launch_bounds__(256) void branch_h_kernel(const int32_t* __restrict__ perm, const int32_t* __restrict__ ids,
                                                      int T, int n, const int32_t* __restrict__ rank,
                                                      const float* __restrict__ scale, const float* __restrict__ part,
                                                      int64_t ldp, int64_t pstride, int S, uint16_t* __restrict__ hs) {
  const int chunks = (int)(ldp / 8);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * chunks) return;
  const int pos = (int)(i / chunks), j0 = (int)(i % chunks) * 8;
  int r = 0;
  float sc = 0.f;
  const int tok = perm[pos];
  if ((unsigned)tok < (unsigned)T) {
    const int id = ids[tok];
    if ((unsigned)id < (unsigned)n) {
      r = rank[id];
      sc = scale[id];
    }
  }
  float f[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) f[k] = 0.f;
  if (j0 < r) {
    const float* src = part + (int64_t)pos * ldp + j0;
    for (int c = 0; c < S; ++c) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const f32x4_t x4 = *reinterpret_cast<const f32x4_t*>(src + (int64_t)c * pstride + 4 * v);
        f[4 * v] += x4[0]; f[4 * v + 1] += x4[1]; f[4 * v + 2] += x4[2]; f[4 * v + 3] += x4[3];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] = j0 + k < r ? sc * f[k] : 0.f;
  }
  HChunk<BF16> hc;
  hc.set(f);
  uint16_t* dst = hs + (int64_t)pos * 2 * ldp + j0;
  *reinterpret_cast<uint4*>(dst) = hc.hi;
  *reinterpret_cast<uint4*>(dst + ldp) = hc.lo;
}

__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(kFWaves / 4, kFWaves / 4)))
void base_fused_kernel(const FusedArgs p) {
  extern __shared__ __align__(16) char lds[];
  int to, tt;
  tile_of((int)blockIdx.x, (int)gridDim.x, p.tiles_o, p.tiles_t, to, tt);
  const int o0 = to * kFT, p0 = tt * kFT;
  const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wo = w & 1, wt = w >> 1;
  const int lr = lane & 31, lh = lane >> 5;

  // ---- loader: buffer loads straight into LDS.  One load of a wave fills
  // 1 KiB of LDS, 16 bytes per lane in lane order: kFRowsPerLoad rows of a
  // stage.  Wave w fills rows 64 w .. 64 w + 63 of both operands; lane i
  // lands in chunk slot i % kFChunks of its row, so it loads the chunk whose
  // slot that is (the permutation is its own inverse).
  const int lrow = lane / kFChunks;
  const int rows_o = p.d_out - o0 < kFT ? p.d_out - o0 : kFT;
  const rsrc_t rw = make_rsrc(p.w + (int64_t)o0 * p.ldw_bytes, (uint32_t)((int64_t)rows_o * p.ldw_bytes));
  const rsrc_t rx = make_rsrc(p.x, (uint32_t)((int64_t)p.T * p.ldx_bytes));
  StageLoader ld;
  ld.rw = rw;
  ld.rx = rx;
#pragma unroll
  for (int q = 0; q < kFLoads; ++q) {
    const int row = kFRowsPerWave * w + kFRowsPerLoad * q + lrow;
    const int ch = chunk_slot(row, lane % kFChunks);
    ld.k8[q] = 8 * ch;
    ld.vw[q] = row < rows_o ? (uint32_t)(row * p.ldw_bytes) + 16u * ch : kOutOfRange;
    const int pos = p0 + row;
    int tok = -1;
    if (pos < p.T) tok = p.perm ? p.perm[pos] : pos;
    ld.vx[q] = (unsigned)tok < (unsigned)p.T ? (uint32_t)((int64_t)tok * p.ldx_bytes) + 16u * ch : kOutOfRange;
  }
  // MFMA reads: row lr of a 32-row block, chunk 2 kk + lh of the stage.
  uint32_t ra[kFKSub];
#pragma unroll
  for (int kk = 0; kk < kFKSub; ++kk)
    ra[kk] = (uint32_t)(lr * kFRowBytes + (chunk_slot(lr, 2 * kk + lh) << 4));

  f32x16_t acc[kFTB][4];  // [token block][output block]
#pragma unroll
  for (int tb = 0; tb < kFTB; ++tb)
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tb][ob][v] = 0.f;

  // ---- the branch.  Per 32-token block of the wave, a table in LDS of its
  // rank groups (8 bytes each: head lane | j0 << 8 | r << 16, row offset).
  // A step is one group per lane half of one block: 8 products (4 output
  // blocks, hi and lo).  One step runs per stage of the main loop, its B
  // rows and s h loaded a stage ahead, so their latency hides behind the
  // stage's products.
  int2* table = reinterpret_cast<int2*>(lds + kFNB * kFStageBytes) + w * kFTB * kFBlockGroups;
  int my_head[kFTB], my_pos[kFTB], steps[kFTB], groups[kFTB];
#pragma unroll
  for (int tb = 0; tb < kFTB; ++tb) {
    my_head[tb] = -1;
    my_pos[tb] = 0;
    steps[tb] = 0;
    groups[tb] = 0;
  }
  if (p.ids != nullptr) {
#pragma unroll
    for (int tb = 0; tb < kFTB; ++tb) {
      const int pos = p0 + kFTokW * wt + 32 * tb + lr;
      int a = -1, r = 0, ro = 0;
      if (pos < p.T) {
        const int tok = p.perm[pos];
        if ((unsigned)tok < (unsigned)p.T) {
          const int id = p.ids[tok];
          if ((unsigned)id < (unsigned)p.n) {
            const int rr = p.rank[id];
            if (rr > 0) {
              a = id;
              r = rr;
              ro = p.row_off[id];
            }
          }
        }
      }
      // Heads: the block's first token of each adapter (both lane halves
      // hold the same 32 tokens and compute the same flags).
      const int a_prev = __shfl(a, (lane + 63) & 63);
      const bool head = a >= 0 && (lr == 0 || a_prev != a);
      const uint32_t heads = (uint32_t)__ballot(head);
      const int ng = head ? (r + 7) >> 3 : 0;
      int incl = ng;
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) {
        const int v = __shfl_up(incl, d, 32);
        if (lr >= d) incl += v;
      }
      groups[tb] = __shfl(incl, 31);  // wave-uniform
      steps[tb] = (groups[tb] + 1) >> 1;
      const uint32_t below = heads & (lr == 31 ? 0xffffffffu : ((2u << lr) - 1u));
      my_head[tb] = (a >= 0 && below != 0u) ? 31 - __clz((int)below) : -1;
      my_pos[tb] = pos;
      if (lh == 0 && head)
        for (int g = 0; g < ng; ++g) table[tb * kFBlockGroups + incl - ng + g] = make_int2(lr | (8 * g) << 8 | r << 16, ro);
    }
    __syncthreads();  // tables written (each wave reads only its own)
  }
  int nbs = 0;
#pragma unroll
  for (int tb = 0; tb < kFTB; ++tb) nbs += steps[tb];

  const rsrc_t rb = make_rsrc(p.b_pack, p.b_bytes);
  const rsrc_t rh = make_rsrc(p.hs, (uint32_t)((int64_t)p.T * p.ldp * 4));
  const uint32_t hs_row = (uint32_t)(4 * p.ldp);  // bytes per position: hi then lo
  // A step's operands: B_a rows o .. of the 8 ranks j0 .. (16 bytes from the
  // dword at or below their start, plus the next dword, shifted down by 16
  // bits when the start is odd), and s h hi / lo of the lane's token (zero
  // unless the token's adapter is the group's).
  uint4 sb[4], sh_hi, sh_lo;
  uint32_t st[4];
  int s_tb = 0, s_nvalid = 0, s_shift = 0;
  auto load_step = [&](int bs) {
    int tb = 0, pair = bs;
#pragma unroll
    for (int k = 0; k + 1 < kFTB; ++k)
      if (tb == k && pair >= steps[k]) {
        pair -= steps[k];
        tb = k + 1;
      }
    int ng = groups[0];
#pragma unroll
    for (int k = 1; k < kFTB; ++k)
      if (tb == k) ng = groups[k];
    const int gi = 2 * pair + lh;
    const int2 e = gi < ng ? table[tb * kFBlockGroups + gi] : make_int2(255, 0);
    const int head = e.x & 255, j0 = (e.x >> 8) & 255, r = e.x >> 16;
    const bool valid = head != 255;
    const uint32_t ebase = (uint32_t)e.y * (uint32_t)p.d_out + (uint32_t)j0;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      const int o = o0 + 128 * wo + 32 * ob + lr;
      const bool ok = valid && o < p.d_out;
      const uint32_t off = 2u * (ebase + (uint32_t)o * (uint32_t)r);
      sb[ob] = buf_ld16(rb, ok ? (off & ~3u) : kOutOfRange, 0);
      st[ob] = buf_ld4(rb, ok ? (off & ~3u) + 16u : kOutOfRange);
    }
    s_shift = (r & lr & 1) ? 16 : 0;  // o = lr modulo 2; the row starts odd when o r is odd
    s_nvalid = r - j0;
    s_tb = tb;
    int mh = my_head[0], mp = my_pos[0];
#pragma unroll
    for (int k = 1; k < kFTB; ++k)
      if (tb == k) {
        mh = my_head[k];
        mp = my_pos[k];
      }
    const bool match = valid && head == mh;
    const uint32_t hv = match ? (uint32_t)mp * hs_row + 2u * (uint32_t)j0 : kOutOfRange;
    sh_hi = buf_ld16(rh, hv, 0);
    sh_lo = buf_ld16(rh, match ? hv + 2u * (uint32_t)p.ldp : kOutOfRange, 0);
  };
  auto run_step = [&]() {
    uint4 bv[4];
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      const uint4 d = sb[ob];
      const uint4 v = make_uint4(__builtin_amdgcn_alignbit(d.y, d.x, s_shift), __builtin_amdgcn_alignbit(d.z, d.y, s_shift),
                                 __builtin_amdgcn_alignbit(d.w, d.z, s_shift), __builtin_amdgcn_alignbit(st[ob], d.w, s_shift));
      bv[ob] = keep_first<BF16>(v, s_nvalid);
    }
#pragma unroll
    for (int tb = 0; tb < kFTB; ++tb)
      if (s_tb == tb) {
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
          acc[tb][ob] = mfma32(bv[ob], sh_hi, acc[tb][ob]);
          acc[tb][ob] = mfma32(bv[ob], sh_lo, acc[tb][ob]);
        }
      }
  };
  int bs = 0;
  if (nbs > 0) load_step(0);

  const int nk = (p.d_in + kFK - 1) / kFK;
  // The first kFNB - 1 stages, then per stage: wait for it, the loads of
  // the stage kFNB - 1 ahead, the products, one step of the branch.
#pragma unroll
  for (int s0 = 0; s0 < kFNB - 1; ++s0)
    if (s0 < nk) issue_stage(ld, lds + s0 * kFStageBytes + kFRowsPerWave * w * kFRowBytes, s0 * kFK, p.d_in);
  for (int ks = 0; ks < nk; ++ks) {
    // Stage ks is in LDS once at most the loads of the stages issued after
    // it are outstanding, in every wave (a branch step's loads, issued
    // after those of stage ks, may still be in flight).
    if (ks + kFNB - 2 < nk)
      wait_loads<(kFNB - 2) * 2 * kFLoads>();
    else
      wait_loads<0>();
    // A bare barrier: __syncthreads() would also wait for every load in
    // flight (its fence), which is the prefetch this loop is built for.
    __builtin_amdgcn_s_barrier();
    // The buffer refilled here was last read in iteration ks - 1, which every
    // wave has finished.
    const int nx = ks + kFNB - 1;
    const char* rd = lds + (ks % kFNB) * kFStageBytes;
    char* wr = lds + (nx % kFNB) * kFStageBytes + kFRowsPerWave * w * kFRowBytes;
    // The branch step between the stage's loads and its products: its
    // operands were loaded right after the previous stage's loads, and the
    // next step's go out now, each with a whole stage to arrive.
    stage_step(rd + 128 * wo * kFRowBytes, rd + kFOperandBytes + kFTokW * wt * kFRowBytes, wr, nx < nk, nx * kFK,
               ld, p.d_in, ra, acc, [&]() {
                 if (bs < nbs) {
                   run_step();
                   if (++bs < nbs) load_step(bs);
                 }
               });
  }
  // Blocks with more steps than the loop has stages.
  while (bs < nbs) {
    run_step();
    if (++bs < nbs) load_step(bs);
  }

  // ---- y: round once and store, 4 consecutive outputs per lane and value group
#pragma unroll
  for (int tb = 0; tb < kFTB; ++tb) {
    const int pos = p0 + kFTokW * wt + 32 * tb + lr;
    if (pos >= p.T) continue;
    const int tok = p.perm ? p.perm[pos] : pos;
    if ((unsigned)tok >= (unsigned)p.T) continue;
    char* yrow = p.y + (int64_t)tok * p.ldy_bytes;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int o = o0 + 128 * wo + 32 * ob + 8 * g + 4 * lh;
        if (o < p.d_out) {
          const f32x16_t& v = acc[tb][ob];
          uint2 out;
          out.x = pack_bf16x2(v[4 * g], v[4 * g + 1]);
          out.y = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
          *reinterpret_cast<uint2*>(yrow + 2 * (int64_t)o) = out;
        }
      }
  }
}

}  // namespace

size_t base_fused_lds_bytes() { return kFLdsBytes; }

hipError_t launch_base_fused(const lora_store& s, const void* w, int64_t ldw, const void* x, int64_t ldx, void* y,
                             int64_t ldy, int T, const int32_t* perm, const int32_t* ids, const void* ws,
                             hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  FusedArgs a{};
  a.w = reinterpret_cast<const char*>(w);
  a.ldw_bytes = ldw * 2;
  a.x = reinterpret_cast<const char*>(x);
  a.ldx_bytes = ldx * 2;
  a.y = reinterpret_cast<char*>(y);
  a.ldy_bytes = ldy * 2;
  a.T = T;
  a.d_in = s.d_in;
  a.d_out = s.d_out;
  a.perm = perm;
  a.ids = ids;
  a.n = s.n;
  a.b_pack = reinterpret_cast<const char*>(s.B_pack);
  a.b_bytes = (uint32_t)((int64_t)s.R * s.d_out * 2);
  a.row_off = s.row_off;
  a.rank = s.rank;
  a.scale = s.scale;
  if (ids != nullptr) {
    const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
    const char* base = reinterpret_cast<const char*>(ws);
    uint16_t* hs = reinterpret_cast<uint16_t*>(const_cast<char*>(base) + L.hs);
    a.hs = hs;
    a.ldp = partial_ld(s.r_max);
    const int64_t work = (int64_t)T * (a.ldp / 8);
    hipLaunchKernelGGL(branch_h_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, stream, perm, ids, T, s.n,
                       s.rank, s.scale, reinterpret_cast<const float*>(base + L.part), a.ldp, (int64_t)T * a.ldp,
                       shrink_split(s.d_in, s.dtype, T, s.n).S, hs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.tiles_o = (s.d_out + kFT - 1) / kFT;
  a.tiles_t = (T + kFT - 1) / kFT;
  const int64_t grid = (int64_t)a.tiles_o * a.tiles_t;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  static DynLdsLimit lim;
  hipError_t e = ensure_dynamic_lds(lim, reinterpret_cast<const void*>(base_fused_kernel), kFLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(base_fused_kernel, dim3((unsigned)grid), dim3(kFThreads), kFLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace lora
