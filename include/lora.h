/*
 * lora.h - C ABI of the batched, rank-specialized LoRA-delta apply on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  A batch of T tokens x[t] (rows of d_in values) each names
 * an adapter a = ids[t]; every adapter keeps its own retained rank r_a.  The
 * library adds the LoRA branch of each token's adapter into the output:
 *
 *     y[t] += s_a * B_a (A_a x[t])        A_a: r_a x d_in,  B_a: d_out x r_a
 *
 * Sources:
 *  - "Compress then Serve: Serving Thousands of LoRA Adapters with Little
 *    Overhead" (arXiv 2407.00066): section 3 defines the LoRA-updated layer
 *    (W0 + B A) x with B of shape d_B x r and A of shape r x d_A; section 11
 *    computes W0 x once and adds the per-request branch B_i A_i x; section 2
 *    describes grouping the requests that use the same adapter (segmented
 *    gather); section 13.4 gives the two-step form used here: A applied with
 *    scale 1 into a float32 buffer of shape [tokens, R], then B applied with
 *    the scale and added into a slice (offset, width) of y.
 *  - "LoRAForge: Co-Designing Compression and Execution for More Efficient
 *    Multi-LoRA Serving", section "LoRAForge's Core Design: Explicit
 *    Retained-Rank Representation and Dual Strategies": execution runs on
 *    each adapter's retained factors at its own rank, without padding or
 *    re-expansion; rank-specialized kernels are compiled for specific rank
 *    values.  The abstract page of the same title names padding, factor
 *    access and generic kernels as what hides the retained low rank.
 *
 * Conventions shared by every entry point.
 *  - Pointers are DEVICE pointers unless the parameter name ends in _host.
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device memory.  Only lora_pack_retained synchronizes (its stream, once,
 *    at the end, so the host staging it used can be released).
 *  - Every call enqueues work on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns; results are visible after the stream reaches that
 *    point.  Calls are stateless; concurrent calls on different streams are
 *    safe when their outputs (and workspaces) are disjoint.
 *  - Return value: LORA_OK, or an error code.  On LORA_ERR_INVALID_ARG and
 *    LORA_ERR_UNSUPPORTED nothing has been enqueued.  On LORA_ERR_HIP a HIP
 *    call failed; lora_last_hip_error() returns its hipError_t (per thread).
 *  - dtype: LORA_DTYPE_BF16 (x, factors and y are bfloat16) or
 *    LORA_DTYPE_F32 (all float32).  Accumulation is float32 in both.
 *  - Row strides (ldx, ldy, ldh) are in elements.  x and y rows must start on
 *    16-byte boundaries: base pointers 16-byte aligned, strides a multiple of
 *    8 elements (bf16) or 4 elements (f32).  d_in and d_out must be
 *    multiples of 8 (bf16) or 4 (f32).  Violations: LORA_ERR_UNSUPPORTED.
 *  - Aliasing: x, y, h and the workspaces must not overlap one another.
 */
#ifndef RANK_SPECIALIZED_LORA_H
#define RANK_SPECIALIZED_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lora_status {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARG = 1, /* a null pointer, negative size, inconsistent sizes */
  LORA_ERR_UNSUPPORTED = 2, /* valid, but outside the kernels' envelope */
  LORA_ERR_HIP = 3          /* a HIP runtime call failed; see lora_last_hip_error */
};

enum lora_dtype { LORA_DTYPE_F32 = 0, LORA_DTYPE_BF16 = 1 };

/* Largest retained (or padded) rank the kernels accept. */
#define LORA_MAX_RANK 64
#define LORA_MAX_SLICES 4
/* Largest T and n that lora_segment accepts (single-workgroup sort); the
 * batched apply with ids accepts the same T. */
#define LORA_SEGMENT_MAX_T 16384
#define LORA_SEGMENT_MAX_N 16382

/*
 * The retained-rank store: every adapter's factors laid end to end at its
 * own rank (pad_to = 0), or every adapter padded with zeros to pad_to (the
 * rank-padded comparison variant, the stacked [b, r, n] / [b, m, r] layout
 * of "Compress then Serve" section 11).  Both factors keep the orientation
 * of the section-3 definition (B: d_B x r, A: r x d_A):
 *
 *   A_pack  [R, d_in]   rows row_off[a] .. row_off[a] + rank[a] - 1: A_a
 *                       (row-major), zero rows past r_a
 *   B_pack  elements row_off[a] * d_out .. (row_off[a] + rank[a]) * d_out - 1:
 *                       B_a as a [d_out, rank[a]] row-major block, zero
 *                       columns past r_a
 *   row_off [n + 1]     int32, exclusive scan of the stored ranks
 *   rank    [n]         int32, stored rank of each adapter (r_a, or pad_to)
 *   scale   [n]         float32, s_a
 *
 * A plain struct filled by lora_pack_retained.  Its device pointers point
 * into the caller's buffers; its lifetime is the caller's.
 */
typedef struct lora_store {
  int32_t n;           /* adapters */
  int32_t d_in;        /* input features */
  int32_t d_out;       /* output features */
  int32_t dtype;       /* enum lora_dtype */
  int32_t r_max;       /* largest stored rank */
  int32_t R;           /* total stored rank = row_off[n] */
  int32_t pad_to;      /* 0 = rank-specialized; otherwise every rank padded to this */
  int32_t reserved;
  const void* A_pack;
  const void* B_pack;
  const int32_t* row_off;
  const int32_t* rank;
  const float* scale;
} lora_store;

/* Human-readable name of a status code (static string). */
const char* lora_status_string(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int lora_last_hip_error(void);

/* ABI version; bumps on any incompatible change of this header. */
int lora_abi_version(void);

/*
 * Size query for a store (host only, nothing enqueued).
 *   n, d_in, d_out, dtype : as in lora_store.
 *   ranks_host [n]        : retained rank of each adapter, 0 <= r_a.
 *   pad_to                : 0 for the rank-specialized store; otherwise every
 *                           adapter is stored at rank pad_to (pad_to >= max r_a).
 * Out (host): bytes needed for A_pack, B_pack and meta.
 * Errors: INVALID_ARG (null outputs, n < 0, d <= 0, r_a < 0, pad_to below a
 * rank, total rank overflowing int32); UNSUPPORTED (stored rank above
 * LORA_MAX_RANK, d not a multiple of 8 (bf16) / 4 (f32), unknown dtype).
 */
int lora_store_bytes(int n, int d_in, int d_out, int dtype, const int32_t* ranks_host, int pad_to,
                     size_t* a_bytes_host, size_t* b_bytes_host, size_t* meta_bytes_host);

/*
 * Pack retained factors into a store.
 *   A_ptrs_host [n] : host array of device pointers; A_a is r_a x d_in,
 *                     row-major (rows of d_in contiguous elements).
 *   B_ptrs_host [n] : host array of device pointers; B_a is d_out x r_a,
 *                     row-major.  Either pointer may be NULL when r_a = 0.
 *   scales_host [n] : s_a.
 *   A_pack, B_pack, meta : caller buffers of at least the sizes that
 *                     lora_store_bytes returns, 16-byte aligned.
 *   out_host        : filled on success (references A_pack, B_pack, meta).
 * Copies the factors (bit-exact), writes zeros where pad_to pads, and
 * writes row_off / rank / scale into meta.  With A_ptrs_host and B_ptrs_host
 * both NULL, only meta and *out_host are written and A_pack / B_pack are left
 * as they are (for lora_rsvd_write to fill).  Synchronizes `stream` before
 * returning.  Errors: as lora_store_bytes, plus INVALID_ARG for null buffers,
 * one pointer array NULL and not the other, or a null factor pointer with
 * r_a > 0.
 */
int lora_pack_retained(lora_store* out_host, int n, int d_in, int d_out, int dtype,
                       const int32_t* ranks_host, const float* scales_host,
                       const void* const* A_ptrs_host, const void* const* B_ptrs_host,
                       void* A_pack, void* B_pack, void* meta, int pad_to, void* stream);

/*
 * Group tokens by adapter: a stable counting sort of ids (the grouping of
 * requests that use the same adapter, "Compress then Serve" section 2).
 *   ids [T]         : int32 adapter id per token.  -1 = no adapter; any other
 *                     id outside [0, n) is treated as -1 and counted.
 *   seg_off [n + 2] : out.  Adapter a's tokens occupy grouped positions
 *                     seg_off[a] .. seg_off[a+1]-1; group n holds the tokens
 *                     without an adapter; seg_off[n+1] = T.
 *   perm [T]        : out.  perm[i] = original token index at grouped
 *                     position i.  Adapters ascend; inside a group tokens
 *                     keep ascending index (unique result).
 *   n_invalid       : optional (NULL) device int32; receives the count of
 *                     ids that are neither -1 nor in [0, n).
 * T = 0 writes seg_off (all zero).  Errors: INVALID_ARG (null pointers,
 * T < 0, n < 1); UNSUPPORTED (T > LORA_SEGMENT_MAX_T or n > LORA_SEGMENT_MAX_N).
 */
int lora_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm, int32_t* n_invalid,
                 void* stream);

/*
 * The plan of a grouping: its sub-tiles (runs of at most 16 tokens of one
 * adapter, in grouped order), each with its adapter, first grouped
 * position, token count and token indices.  It depends on the grouping only
 * (not on a store), so one plan serves every store over the same adapters,
 * e.g. all the projections of a decode step, which then skip forming it
 * ("Compress then Serve" section 2: the requests of one adapter are grouped
 * once).
 * lora_plan_bytes: bytes of a plan for T tokens over n adapters (host only;
 *   0 on invalid arguments).
 * lora_group: lora_segment plus the plan, in one launch where T <= 8192 and
 *   n <= 2048 (else the sort, then a plan launch).  plan: caller buffer of
 *   at least lora_plan_bytes(T, n) bytes, 16-byte aligned.  Other arguments
 *   and errors as lora_segment, plus INVALID_ARG for a null or small plan
 *   buffer and UNSUPPORTED for a misaligned one.
 */
size_t lora_plan_bytes(int T, int n);
int lora_group(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm, void* plan, size_t plan_bytes,
               int32_t* n_invalid, void* stream);

/*
 * Workspace of lora_shrink, lora_expand and the applies for T tokens on this
 * store (host only; 0 on invalid arguments).  It holds each sub-tile's
 * metadata for this store, the shrink's float32 partial sums, and the plan
 * (and, beyond the one-launch grouping's size, seg_off and perm) of a call
 * that forms its own grouping; the contents need no initialization and are
 * scratch after the call.  One workspace must not be shared by calls in
 * flight together.
 */
size_t lora_workspace_bytes(const lora_store* store_host, int T);

/*
 * Shrink (step 1 of "Compress then Serve" section 13.4):
 *   h[i, j] = sum_k A_a[j, k] * x[perm[i], k]    for j < r_a, a = adapter of
 *                                                grouped position i
 *   x   [T, ldx] : dtype of the store, token order.
 *   seg_off, perm: a grouping as lora_segment writes it (for store->n).
 *   h   [T, ldh] : float32, GROUPED order (row i = grouped position i),
 *                  ldh >= r_max.  Columns >= r_a and rows of tokens without
 *                  an adapter (or with r_a = 0) are not written.  Products
 *                  are accumulated in float32 (bf16 products are exact in
 *                  float32); the sum over d_in is formed in a fixed order,
 *                  so results are deterministic.
 *   ws           : lora_workspace_bytes(store, T) bytes, 16-byte aligned.
 * Errors: INVALID_ARG (null pointers, T < 0, ldx < d_in, ldh < r_max, ws too
 * small); UNSUPPORTED (alignment, see conventions; n > LORA_SEGMENT_MAX_N).
 */
int lora_shrink(const lora_store* store_host, const void* x, int64_t ldx, int T, const int32_t* seg_off,
                const int32_t* perm, float* h, int64_t ldh, void* ws, size_t ws_bytes, void* stream);

/*
 * Expand (step 3 of "Compress then Serve" section 13.4):
 *   y[perm[i], o] += s_a * sum_{j < r_a} B_a[o, j] * h[i, j]
 * accumulated in float32 and rounded once to the output dtype (bf16: round
 * to nearest, ties to even).  h [T, ldh] float32 in grouped order (as
 * lora_shrink writes it; columns >= r_a are not read).  y [T, ldy] in token
 * order, ldy >= d_out; y may be a column slice of a wider buffer (pass the
 * slice's first column and the wider row stride) - the y_offset /
 * y_slice_size of the same section.  Rows of tokens without an adapter (and
 * of adapters with r_a = 0) are left untouched.  Errors as lora_shrink.
 */
int lora_expand(const lora_store* store_host, const float* h, int64_t ldh, int T, const int32_t* seg_off,
                const int32_t* perm, void* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/*
 * The batched apply:  y[t] += s_a * B_a (A_a x[t])  for every token.
 * Either ids, or ids = NULL and seg_off / perm from lora_segment.  (To reuse
 * one grouping across many stores, form its plan once with lora_group and
 * call lora_apply_planned.)
 * Decode-sized calls with ids (lora_apply_launches returns 1) run as one
 * kernel, a workgroup per (token, slice of the output features): it reads
 * the token's adapter from ids, reduces h over all of d_in (float32, a fixed
 * order) and adds the delta into that slice of the token's y row (the
 * per-token indexed form of the same two steps: section 13.4 of the Compress
 * then Serve page).  Other calls run as three kernels: the grouping (the plan
 * of sub-tiles, into the workspace), the shrink (float32 partial sums over
 * chunks of d_in) and the expand (partials summed in chunk order, then y
 * updated); their result equals lora_segment + lora_shrink + lora_expand bit
 * for bit.  The two forms sum h in different orders, so on float data they
 * agree to float32 rounding.
 * Errors: union of those calls'.
 */
int lora_apply_batched(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy,
                       int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * The batched apply without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory or pass one: code under HIP
 * graph capture that must not call hipMalloc, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, same kernels and the same result
 * as lora_apply_batched (bit for bit); the workspace is the library's own
 * array of LORA_NOALLOC_SCRATCH_BYTES bytes, one per device, held from the
 * first call on that device until the process ends.
 *  - No hipMalloc, hipFree or allocating library call is made.
 *  - Every call on a device shares that device's array, and the array keeps
 *    the last call's contents (nothing in it needs to start at zero): calls
 *    that overlap on one device (several streams, several host threads) race
 *    on it and give wrong results.  Serialize them, or use lora_apply_batched
 *    with a workspace each.
 * Errors: those of lora_apply_batched (the workspace's aside), checked before
 * any HIP call; UNSUPPORTED when lora_workspace_bytes(store, T) exceeds
 * LORA_NOALLOC_SCRATCH_BYTES; HIP_ERROR if the array's address cannot be
 * looked up on the current device.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (32 << 20)
int lora_apply_batched_noalloc(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy,
                               int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm,
                               void* stream);

/*
 * The base layer with the adapter branch in its epilogue ("Compress then
 * Serve" section 3: the adapted layer computes (W0 + B A) x; section 11: the
 * base product is shared by the batch and each request adds its branch):
 *   y[t] = W0 x[t] + s_a B_a (A_a x[t])   for a = ids[t] in [0, n), r_a > 0,
 *   y[t] = W0 x[t]                        for every other token.
 * y is overwritten, and written once: the branch is added to the base
 * product's float32 accumulators before y is rounded to bf16.
 *   W0 [d_out, ldw] : device, bf16, row-major, the layer's [out, in]
 *                     orientation (y = x W0^T); ldw >= d_in, ldw % 8 == 0,
 *                     16-byte aligned.
 *   x [T, ldx], y [T, ldy] : device bf16 rows as in lora_apply_batched; y
 *                     must not overlap x or W0.
 *   ids [T]         : device int32 adapter ids (-1 or any id outside [0, n):
 *                     base only), or NULL for the base product alone.
 *   ws              : lora_workspace_bytes(store, T) bytes when ids is given
 *                     (the grouping, plan and partial sums); may be NULL
 *                     without ids.
 * Enqueues the grouping and the shrink (with ids) and one GEMM kernel.
 * Accuracy: float32 accumulation of the bf16 products; h enters the branch
 * as the exact pair hi + lo of bf16 values (about 16 significant bits).
 * Errors: INVALID_ARG (null pointers, ldw < d_in, T < 0, ws too small);
 * UNSUPPORTED (a float32 store, rows not 16-byte aligned, T above
 * LORA_SEGMENT_MAX_T or n above LORA_SEGMENT_MAX_N with ids; 256 * ldw * 2,
 * T * ldx * 2 or R * d_out * 2 bytes at or above 2^31).
 */
int lora_apply_base_fused(const lora_store* store_host, const void* W0, int64_t ldw, const void* x, int64_t ldx,
                          void* y, int64_t ldy, int T, const int32_t* ids, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * One kernel of lora_apply_batched at a time, for measuring each alone:
 * phases = 1 forms the plan and runs the shrink (partial sums and each
 * sub-tile's metadata into ws), 2 the expand only (from the plan, metadata
 * and partial sums a previous phase-1 call left in ws, for the same store, T
 * and grouping; metadata that does not fit this store is skipped, so a
 * mismatched workspace gives wrong values, never an access outside the
 * store's buffers), 3 = lora_apply_batched (the one-kernel form for
 * decode-sized calls with ids).  Phases 1 and 2 always run the two-kernel
 * form.
 * Errors: as lora_apply_batched; INVALID_ARG for phases outside 1..3.
 */
int lora_apply_batched_phases(const lora_store* store_host, const void* x, int64_t ldx, void* y,
                              int64_t ldy, int T, const int32_t* ids, const int32_t* seg_off,
                              const int32_t* perm, void* ws, size_t ws_bytes, void* stream, int phases);

/*
 * The batched apply on a plan from lora_group (same T, and n = store->n):
 * the shrink and the expand only, so that a grouping formed once serves many
 * stores (every projection of a decode step).  plan_bytes: the plan buffer's
 * size.  lora_apply_planned_phases runs one of them at a time, as
 * lora_apply_batched_phases (3 = both).  A plan of another grouping gives
 * wrong values, never an access outside the call's buffers (its entries are
 * checked against T and the store).  Errors: as lora_apply_batched, plus
 * INVALID_ARG for a null or small plan buffer, UNSUPPORTED for a misaligned
 * one.
 */
int lora_apply_planned(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                       const void* plan, size_t plan_bytes, void* ws, size_t ws_bytes, void* stream);
int lora_apply_planned_phases(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                              const void* plan, size_t plan_bytes, void* ws, size_t ws_bytes, void* stream,
                              int phases);

/*
 * Kernel launches an apply enqueues for this store, T and kind of grouping
 * (host only, nothing enqueued).  with_ids: 1 ids (lora_apply_batched), 0 a
 * caller's seg_off / perm (lora_apply_batched), 2 a plan
 * (lora_apply_planned).  Returns 1 for the one-kernel decode form (ids
 * given, T <= 512, r_max <= 8 for bf16 or <= 4 for f32, d_in <= 4096 for
 * bf16 or <= 2048 for f32), 2 for the shrink and the expand on a plan, 3 for
 * the grouping (or the plan of a given grouping), the shrink and the expand,
 * 4 when the sort precedes them (ids given, T > 8192 or n > 2048), 0 for
 * T = 0.  A negative value is -(the status the apply would return): an
 * invalid store, T or with_ids, or UNSUPPORTED sizes.
 */
int lora_apply_launches(const lora_store* store_host, int T, int with_ids);

/*
 * Shared-basis (joint-diagonalization) adapters.  "Compress then Serve"
 * section 3.1 holds adapter i's product B_i A_i as U Sigma_i V^T, with U
 * (d_out x r) and V (d_in x r) shared and Sigma_i a full r x r matrix
 * (JD-Full) or diagonal (JD-Diag); section 3.2 splits the adapters into
 * clusters, cluster j with its own U_j, V_j; section 11 serves the branch as
 * U (Sigma (V^T x)).  The apply is
 *
 *     y[t] += s_a * U_c (Sigma_a (V_c^T x[t]))     a = ids[t], c = cluster_of[a]
 *
 * The store:
 *   basis      : an ordinary store (lora_pack_retained) whose n = k entries
 *                are the clusters, every one at rank r: A_j = V_j^T (r x
 *                d_in), B_j = U_j (d_out x r), scale 1.
 *   n_adapters : adapters.
 *   r          : the shared rank (= basis.r_max; basis.R must be k * r).
 *   diag       : 1: Sigma_a is a vector of r values (JD-Diag); 0: r x r
 *                row-major (JD-Full).
 *   cluster_of : device int32 [n_adapters]; a value outside [0, k) means the
 *                adapter adds nothing.
 *   sigma      : device float32, [n_adapters][r] or [n_adapters][r][r].
 *   scale      : device float32 [n_adapters] (s_a).
 * The caller owns every buffer; the struct only points at them.
 */
typedef struct lora_jd_store {
  lora_store basis;
  int32_t n_adapters;
  int32_t r;
  int32_t diag;
  int32_t reserved;
  const int32_t* cluster_of;
  const float* sigma;
  const float* scale;
} lora_jd_store;

/* Workspace of lora_jd_apply for T tokens (host only; 0 on invalid
 * arguments): the float32 h buffer (Sigma applied) and the basis store's
 * lora_workspace_bytes. */
size_t lora_jd_workspace_bytes(const lora_jd_store* store_host, int T);

/*
 * The shared-basis apply (section 13.4's three steps with a per-token index:
 * V^T, then Sigma with the scale, then U, added into y).  Three kernels: the
 * shrink of the basis store with the tokens grouped by the cluster of their
 * adapter (h = V_c^T x, float32); per token g = s_a Sigma_a h (float32, a
 * fixed order); the expand of the basis store from g (y updated, one
 * rounding).  x [T, ldx], y [T, ldy] in token order as for
 * lora_apply_batched; ids as for lora_apply_batched (ids outside [0,
 * n_adapters) add nothing).  Errors: INVALID_ARG (null pointers, T < 0,
 * r != basis.r_max, basis.R != basis.n * r, diag not 0 or 1, workspace too
 * small); UNSUPPORTED (those of lora_apply_batched for the basis store, more
 * than 2048 clusters, T > 8192: the grouping by cluster runs in one workgroup).
 */
int lora_jd_apply(const lora_jd_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                  const int32_t* ids, void* ws, size_t ws_bytes, void* stream);

/*
 * Multi-slice apply: several projections that read the same input (q, k and
 * v; gate and up) applied with one read of x.  "Compress then Serve"
 * section 13.4 adds the B step into a slice of y given by an offset and a
 * width; here each slice is an ordinary store of the same adapters (same n,
 * d_in and dtype; each slice with its own d_out, ranks, row offsets and
 * scales), and its y may be a column slice of one fused output (a pointer
 * into the row plus the fused row stride).
 *
 *     y_s[t] += s_{s,a} * B_{s,a} (A_{s,a} x[t])     for every slice s,  a = ids[t]
 *
 * The multi store:
 *   slice[s]  : the slices' stores (their B, ranks, row offsets and scales are
 *               used; their A rows are copied into `stacked`).
 *   stacked   : per adapter, the A rows of slice 0, then slice 1, ... (stored
 *               ranks); rank = the sum of the slices' stored ranks, at most
 *               LORA_MAX_RANK.  Not an ordinary store: its B_pack aliases its
 *               A_pack and its d_out is d_in, so that no call reads outside
 *               its buffers, but only lora_apply_multi gives it a meaning.
 *   hoff      : device int32 [n_slices][n]: the first stacked row (and h
 *               column) of slice s of adapter a.
 * The caller owns every buffer; the struct only points at them.
 */
typedef struct lora_multi_store {
  int32_t n_slices;
  int32_t reserved;
  lora_store stacked;
  lora_store slice[LORA_MAX_SLICES];
  const int32_t* hoff;
} lora_multi_store;

/*
 * Size query (host only): bytes of the stacked A buffer, of its metadata and
 * of hoff for these slices.  Errors: INVALID_ARG (null pointers, n_slices
 * outside 1..LORA_MAX_SLICES, an invalid slice store, slices whose n, d_in or
 * dtype differ).
 */
int lora_multi_bytes(int n_slices, const lora_store* slices_host, size_t* a_bytes_host, size_t* meta_bytes_host,
                     size_t* hoff_bytes_host);

/*
 * Build a multi store from the slices' stores: reads their ranks back (the
 * stream is synchronized), writes the stacked metadata and hoff, and copies
 * every slice's A rows into A_stacked (bit-exact).  A_stacked, meta and hoff:
 * caller buffers of lora_multi_bytes' sizes, 16-byte aligned.  The slices'
 * stores must stay alive (their B and metadata are used by the apply).
 * Errors: as lora_multi_bytes; INVALID_ARG for null buffers; UNSUPPORTED
 * when an adapter's stacked rank exceeds LORA_MAX_RANK.
 */
int lora_pack_multi(lora_multi_store* out_host, int n_slices, const lora_store* slices_host, void* A_stacked,
                    void* meta, int32_t* hoff, void* stream);

/* Workspace of lora_apply_multi for T tokens (host only; 0 on invalid
 * arguments): that of the stacked store, then 16 bytes per slice and
 * possible sub-tile (each slice's rank, row offset, scale and h column for
 * the sub-tile's adapter, written by the stacked shrink for the slices'
 * expands), 256-byte aligned. */
size_t lora_multi_workspace_bytes(const lora_multi_store* store_host, int T);

/*
 * The multi-slice apply: one shrink of the stacked store (x read once for
 * every slice; tokens grouped from ids, or from a grouping as for
 * lora_apply_batched), then one expand per slice into y_host[s] (device
 * pointers, row stride ldy_host[s] elements, [T, d_out of slice s]).  Each
 * y_s is updated once, rounded once.  Errors: those of lora_apply_batched
 * for the stacked store and each slice's y; INVALID_ARG for an inconsistent
 * multi store.
 */
int lora_apply_multi(const lora_multi_store* store_host, const void* x, int64_t ldx, void* const* y_host,
                     const int64_t* ldy_host, int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm,
                     void* ws, size_t ws_bytes, void* stream);
/* The same on a plan from lora_group (n = the multi store's n), as
 * lora_apply_planned. */
int lora_apply_multi_planned(const lora_multi_store* store_host, const void* x, int64_t ldx, void* const* y_host,
                             const int64_t* ldy_host, int T, const void* plan, size_t plan_bytes, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Retained-rank allocation (host only, nothing enqueued): how many ranks each
 * of m units (one adapter of one module: a factor pair of original rank
 * r_orig[u]) keeps after compression.  "LoRAForge" core design section: a
 * uniform ratio with a floor, or a spectral budget that keeps the
 * components carrying the most energy (sigma^2).
 *
 * lora_ranks_uniform:  r[u] = min(r_orig[u], max(floor, ceil(ratio r_orig[u]))),
 *   0 <= ratio <= 1.
 * lora_ranks_spectral: every unit first keeps min(floor, r_orig[u]); the rest
 *   of `budget` (total ranks over all units) goes one rank at a time to the
 *   unit whose next singular value is largest (ties: the lower unit), never
 *   beyond r_orig[u].  sigma: the units' singular values end to end, unit u
 *   at sigma[sigma_off[u] .. sigma_off[u+1]) with sigma_off[u+1] -
 *   sigma_off[u] = r_orig[u], each unit's values finite, >= 0 and
 *   non-increasing (as an SVD gives them).
 * Errors: INVALID_ARG (null pointers with m > 0, negative sizes, ratio
 * outside [0, 1], sigma inconsistent with r_orig or not non-increasing).
 */
int lora_ranks_uniform(int m, const int32_t* r_orig_host, double ratio, int floor_rank, int32_t* r_out_host);
int lora_ranks_spectral(int m, const int32_t* r_orig_host, const float* sigma_host, const int64_t* sigma_off_host,
                        int floor_rank, int64_t budget, int32_t* r_out_host);

/*
 * Retained-factor construction (r-SVD), batched over the n adapters of one
 * module that share an original rank r.  "LoRAForge" post-hoc compression
 * decomposes each adapter's original factors into retained ones, with a
 * tall-and-skinny QR of row blocks merged afterwards, parallel over adapters
 * and row blocks (section "FlashTSQR: An Accelerator for Batched Factor
 * Construction"); "Compress then Serve" section 4: alone, an adapter's best
 * rank-k replacement is the rank-k SVD of B A.  With B = Q_B R_B, A^T = Q_A
 * R_A and the core C = R_B R_A^T = U S V^T, the retained factors are
 * B' = Q_B U_k = B (R_B^-1 U_k) and A' = S_k V_k^T Q_A^T = U_k^T R_B A:
 * B' has orthonormal columns and B' A' is the best rank-k approximation of
 * B A.  R comes from the Gram matrix M^T M in float64 (the Cholesky form of
 * the QR: one pass over the rows; accurate while cond(B), cond(A) stay well
 * below 1e7); the core's SVD is a one-sided Jacobi iteration in float64.
 *
 * lora_rsvd_workspace_bytes: bytes of ws for n adapters (host only; 0 on
 *   invalid arguments): 7 float64 64 x 64 matrices per adapter, holding W_B
 *   and W_A between the two calls below.
 * lora_rsvd_factor: stage 1, enqueued on `stream` (four kernels).
 *   A_all  : device [n][r][d_in] (each A_a row-major), dtype elements.
 *   B_all  : device [n][d_out][r] (each B_a row-major).
 *   sigma  : out, device float32 [n][r]: the singular values of each B_a A_a,
 *            descending.
 *   status : out, device int32 [n]: 0, or 1 when a pivot of the Cholesky of
 *            B_a^T B_a or A_a A_a^T fell to 1e-14 of its largest diagonal
 *            entry or below (a numerically rank-deficient factor; zero
 *            factors give sigma = 0 and zero retained factors).
 *   ws     : device, at least lora_rsvd_workspace_bytes.
 *   A_all, B_all and ws 16-byte aligned; d_in and d_out multiples of 8
 *   (bf16) / 4 (f32), as for a store.
 * lora_rsvd_write: stage 2.  Writes the retained factors of the same adapters
 *   (A_all, B_all and ws as given to lora_rsvd_factor) into `store`, a store
 *   of n = the same adapters, built by lora_pack_retained with both factor
 *   pointer arrays NULL and each adapter's retained rank k_a (chosen, e.g.,
 *   by lora_ranks_uniform or lora_ranks_spectral from sigma).  Adapter a gets
 *   A' (k_a x d_in) and B' (d_out x k_a) at its row offset, rounded from
 *   float64 through float32 to the store's dtype; components past r (k_a > r)
 *   and padding up to the stored rank are zero.
 * Errors: INVALID_ARG (null pointers, n < 0, d < 1, r < 1, workspace too
 * small, an invalid store); UNSUPPORTED (r above LORA_MAX_RANK, d_in < r or
 * d_out < r, d not a multiple of 8 / 4, unknown dtype, unaligned pointers, n
 * too large for one grid).
 */
size_t lora_rsvd_workspace_bytes(int n, int d_in, int d_out);
int lora_rsvd_factor(int n, int d_in, int d_out, int dtype, int r, const void* A_all, const void* B_all,
                     float* sigma, int32_t* status, void* ws, size_t ws_bytes, void* stream);
int lora_rsvd_write(const lora_store* store_host, int r, const void* A_all, const void* B_all, const void* ws,
                    size_t ws_bytes, void* stream);

/*
 * Some kernels of lora_rsvd_factor, for measuring each alone: phases is a
 * bit mask, 1 the Grams, 2 the Cholesky factors and the core C, 4 the
 * core's SVD (sigma, U), 8 W_B and W_A; each reads what the earlier ones
 * left in ws (from a call for the same A_all, B_all, n, d_in, d_out, r).
 * 15 = lora_rsvd_factor.
 * Errors: as lora_rsvd_factor; INVALID_ARG for phases outside 1..15.
 */
int lora_rsvd_factor_phases(int n, int d_in, int d_out, int dtype, int r, const void* A_all, const void* B_all,
                            float* sigma, int32_t* status, void* ws, size_t ws_bytes, void* stream, int phases);

#ifdef __cplusplus
}
#endif

#endif /* RANK_SPECIALIZED_LORA_H */
