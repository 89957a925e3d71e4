// C ABI of the batched, rank-specialized LoRA-delta apply (include/lora.h).
// Host dispatch only: validate, size grids, launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <vector>

#include "host_util.h"
#include "kernels.h"
#include "validate.h"

namespace lora {
static thread_local int g_last_hip = 0;
static int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return LORA_ERR_HIP;
}
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
}  // namespace lora

using namespace lora;

extern "C" {

const char* lora_status_string(int status) {
  switch (status) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARG: return "invalid argument";
    case LORA_ERR_UNSUPPORTED: return "unsupported (outside the kernels' envelope)";
    case LORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int lora_last_hip_error(void) { return g_last_hip; }

int lora_abi_version(void) { return 5; }

int lora_store_bytes(int n, int d_in, int d_out, int dtype, const int32_t* ranks_host, int pad_to,
                     size_t* a_bytes_host, size_t* b_bytes_host, size_t* meta_bytes_host) {
  if (!a_bytes_host || !b_bytes_host || !meta_bytes_host) return LORA_ERR_INVALID_ARG;
  int r_max = 0;
  int64_t rows = 0;
  int st = check_store_shape(n, d_in, d_out, dtype, ranks_host, pad_to, &r_max, &rows);
  if (st != LORA_OK) return st;
  const size_t eb = (size_t)elem_bytes(dtype);
  *a_bytes_host = (size_t)rows * d_in * eb;
  *b_bytes_host = (size_t)rows * d_out * eb;
  *meta_bytes_host = meta_bytes(n);
  return LORA_OK;
}

int lora_pack_retained(lora_store* out_host, int n, int d_in, int d_out, int dtype,
                       const int32_t* ranks_host, const float* scales_host,
                       const void* const* A_ptrs_host, const void* const* B_ptrs_host, void* A_pack,
                       void* B_pack, void* meta, int pad_to, void* stream) {
  if (!out_host || !scales_host || !meta) return LORA_ERR_INVALID_ARG;
  if (n < 1) return LORA_ERR_INVALID_ARG;
  int r_max = 0;
  int64_t rows = 0;
  int st = check_store_shape(n, d_in, d_out, dtype, ranks_host, pad_to, &r_max, &rows);
  if (st != LORA_OK) return st;
  // Both pointer arrays NULL: metadata only, the factors are written later
  // (lora_rsvd_write).
  const bool meta_only = !A_ptrs_host && !B_ptrs_host;
  if (!meta_only && (!A_ptrs_host || !B_ptrs_host)) return LORA_ERR_INVALID_ARG;
  if (rows > 0 && (!A_pack || !B_pack)) return LORA_ERR_INVALID_ARG;
  if (!aligned16(meta) || (A_pack && !aligned16(A_pack)) || (B_pack && !aligned16(B_pack)))
    return LORA_ERR_UNSUPPORTED;
  if (!meta_only)
    for (int a = 0; a < n; ++a)
      if (ranks_host[a] > 0 && (!A_ptrs_host[a] || !B_ptrs_host[a])) return LORA_ERR_INVALID_ARG;

  // Host image of the meta buffer.
  std::vector<char> img(meta_bytes(n), 0);
  int32_t* row_off = reinterpret_cast<int32_t*>(img.data());
  int32_t* rank = row_off + (n + 1);
  float* scale = reinterpret_cast<float*>(rank + n);
  int32_t* true_rank = reinterpret_cast<int32_t*>(scale + n);
  const void** ptrs = reinterpret_cast<const void**>(img.data() + meta_ptr_offset(n));
  row_off[0] = 0;
  for (int a = 0; a < n; ++a) {
    const int stored = pad_to > 0 ? pad_to : ranks_host[a];
    rank[a] = stored;
    true_rank[a] = ranks_host[a];
    scale[a] = scales_host[a];
    row_off[a + 1] = row_off[a] + stored;
    ptrs[a] = meta_only ? nullptr : A_ptrs_host[a];
    ptrs[n + a] = meta_only ? nullptr : B_ptrs_host[a];
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(meta, img.data(), img.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e);
  if (!meta_only) {
    e = launch_pack(dtype, meta, n, d_in, d_out, (int)rows, A_pack, B_pack, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);

  lora_store st_out;
  std::memset(&st_out, 0, sizeof(st_out));
  st_out.n = n;
  st_out.d_in = d_in;
  st_out.d_out = d_out;
  st_out.dtype = dtype;
  st_out.r_max = r_max;
  st_out.R = (int32_t)rows;
  st_out.pad_to = pad_to;
  st_out.A_pack = A_pack;
  st_out.B_pack = B_pack;
  st_out.row_off = reinterpret_cast<const int32_t*>(meta);
  st_out.rank = st_out.row_off + (n + 1);
  st_out.scale = reinterpret_cast<const float*>(st_out.rank + n);
  *out_host = st_out;
  return LORA_OK;
}

int lora_segment(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm, int32_t* n_invalid,
                 void* stream) {
  int st = check_segment_args(ids, T, n, seg_off, perm);
  if (st != LORA_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (group_fits(T, n)) {
    e = launch_group(ids, T, n, nullptr, 0, seg_off, perm, nullptr, n_invalid, strm);
  } else {
    int max_lds = 0;  // of the current device
    e = device_attribute<hipDeviceAttributeMaxSharedMemoryPerBlock>(&max_lds);
    if (e != hipSuccess) return hip_fail(e);
    if (segment_lds_bytes(T, n) + segment_static_lds_bytes() > (size_t)max_lds) return LORA_ERR_UNSUPPORTED;
    e = launch_segment(ids, T, n, seg_off, perm, n_invalid, strm);
  }
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

size_t lora_plan_bytes(int T, int n) {
  if (T < 0 || n < 1) return 0;
  return plan_bytes(T, n);
}

static int check_plan(const void* plan, size_t plan_bytes_, int T, int n) {
  if (T == 0) return LORA_OK;
  if (plan == nullptr || plan_bytes_ < plan_bytes(T, n)) return LORA_ERR_INVALID_ARG;
  if (!aligned16(plan)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int lora_group(const int32_t* ids, int T, int n, int32_t* seg_off, int32_t* perm, void* plan, size_t plan_bytes_,
               int32_t* n_invalid, void* stream) {
  int st = check_segment_args(ids, T, n, seg_off, perm);
  if (st != LORA_OK) return st;
  if ((st = check_plan(plan, plan_bytes_, T, n)) != LORA_OK) return st;
  if (T == 0) return lora_segment(ids, T, n, seg_off, perm, n_invalid, stream);
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (group_fits(T, n)) {
    e = launch_group(ids, T, n, nullptr, 0, seg_off, perm, reinterpret_cast<char*>(plan), n_invalid, strm);
  } else {
    st = lora_segment(ids, T, n, seg_off, perm, n_invalid, stream);
    if (st != LORA_OK) return st;
    e = launch_plan(seg_off, perm, T, n, reinterpret_cast<char*>(plan), nullptr, nullptr, strm);
  }
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

size_t lora_workspace_bytes(const lora_store* store_host, int T) {
  if (check_store(store_host) != LORA_OK) return 0;
  return workspace_bytes(store_host, T);
}

// The plan of a call's grouping, formed in ws when the caller did not pass
// one: from ids (the grouping kernel; beyond its size, the sort and the plan
// kernel), or from a caller's (seg_off, perm).  groups_n is the number of
// groups (adapters, or clusters with id_map).
static hipError_t form_plan(const lora_store& s, int groups_n, int T, const int32_t* ids, const int32_t* id_map,
                            int id_map_n, const int32_t* seg_off, const int32_t* perm, void* ws, const char** plan,
                            hipStream_t strm) {
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  char* base = reinterpret_cast<char*>(ws);
  char* pl = base + L.plan;
  *plan = pl;
  if (ids == nullptr) return launch_plan(seg_off, perm, T, groups_n, pl, nullptr, nullptr, strm);
  if (group_fits(T, groups_n))
    return launch_group(ids, T, groups_n, id_map, id_map_n, nullptr, nullptr, pl, nullptr, strm);
  int32_t* so = reinterpret_cast<int32_t*>(base + L.seg_off);
  int32_t* pm = reinterpret_cast<int32_t*>(base + L.perm);
  hipError_t e = launch_segment(ids, T, groups_n, so, pm, nullptr, strm);
  if (e != hipSuccess) return e;
  return launch_plan(so, pm, T, groups_n, pl, nullptr, nullptr, strm);
}

int lora_shrink(const lora_store* store_host, const void* x, int64_t ldx, int T, const int32_t* seg_off,
                const int32_t* perm, float* h, int64_t ldh, void* ws, size_t ws_bytes, void* stream) {
  int st = check_store(store_host);
  if (st != LORA_OK) return st;
  if ((st = check_grouping(store_host, T, seg_off, perm)) != LORA_OK) return st;
  if ((st = check_rows(x, ldx, store_host->d_in, store_host->dtype, T)) != LORA_OK) return st;
  if ((st = check_h(h, ldh, store_host, T)) != LORA_OK) return st;
  if ((st = check_ws(store_host, T, ws, ws_bytes)) != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const char* plan = nullptr;
  hipError_t e = form_plan(*store_host, store_host->n, T, nullptr, nullptr, 0, seg_off, perm, ws, &plan, strm);
  if (e == hipSuccess) e = launch_shrink(*store_host, plan, T, x, ldx, ws, strm);
  if (e == hipSuccess) e = launch_reduce_partials(*store_host, plan, T, ws, h, ldh, strm);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

int lora_expand(const lora_store* store_host, const float* h, int64_t ldh, int T, const int32_t* seg_off,
                const int32_t* perm, void* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int st = check_store(store_host);
  if (st != LORA_OK) return st;
  if ((st = check_grouping(store_host, T, seg_off, perm)) != LORA_OK) return st;
  if ((st = check_rows(y, ldy, store_host->d_out, store_host->dtype, T)) != LORA_OK) return st;
  if ((st = check_h(h, ldh, store_host, T)) != LORA_OK) return st;
  if ((st = check_ws(store_host, T, ws, ws_bytes)) != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const lora_store& s = *store_host;
  const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
  char* base = reinterpret_cast<char*>(ws);
  char* plan = base + L.plan;
  // The plan and each sub-tile's metadata from the store (h is given: one
  // partial sum).
  hipError_t e = launch_plan(seg_off, perm, T, s.n, plan, &s, reinterpret_cast<TileMeta*>(base + L.meta), strm);
  if (e == hipSuccess) e = launch_expand(s, plan, T, ws, h, ldh, y, ldy, strm);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

// The apply's argument checks other than the workspace's (host only).
static int check_apply_args(const lora_store* store_host, const void* x, int64_t ldx, const void* y, int64_t ldy,
                            int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm) {
  int st = check_store(store_host);
  if (st != LORA_OK) return st;
  const lora_store& s = *store_host;
  if (T < 0) return LORA_ERR_INVALID_ARG;
  if ((st = check_rows(x, ldx, s.d_in, s.dtype, T)) != LORA_OK) return st;
  if ((st = check_rows(y, ldy, s.d_out, s.dtype, T)) != LORA_OK) return st;
  if (ids != nullptr && (T > LORA_SEGMENT_MAX_T || s.n > LORA_SEGMENT_MAX_N)) return LORA_ERR_UNSUPPORTED;
  if (T > 0 && ids == nullptr && (st = check_grouping(store_host, T, seg_off, perm)) != LORA_OK) return st;
  return LORA_OK;
}

// phases: 1 = plan (unless given) + shrink, 2 = expand (from the plan and the
// metadata and partial sums of a phase-1 call in ws), 3 = the apply (the
// one-kernel decode form when it fits).  `given_plan`: a caller's plan
// (lora_group); otherwise the grouping comes from ids or (seg_off, perm).
static int apply_impl(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                      const int32_t* ids, const int32_t* seg_off, const int32_t* perm, const void* given_plan,
                      void* ws, size_t ws_bytes, void* stream, int phases) {
  int st = check_store(store_host);
  if (st != LORA_OK) return st;
  const lora_store& s = *store_host;
  if (T < 0) return LORA_ERR_INVALID_ARG;
  if (phases < 1 || phases > 3) return LORA_ERR_INVALID_ARG;
  if ((st = check_rows(x, ldx, s.d_in, s.dtype, T)) != LORA_OK) return st;
  if ((st = check_rows(y, ldy, s.d_out, s.dtype, T)) != LORA_OK) return st;
  if ((st = check_ws(store_host, T, ws, ws_bytes)) != LORA_OK) return st;
  if (ids != nullptr && (T > LORA_SEGMENT_MAX_T || s.n > LORA_SEGMENT_MAX_N)) return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;  // nothing to group or apply
  if (given_plan == nullptr && ids == nullptr && (st = check_grouping(store_host, T, seg_off, perm)) != LORA_OK)
    return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (phases == 3 && given_plan == nullptr && decode_apply_fits(s, T, ids != nullptr)) {
    e = launch_decode_apply(s, ids, T, x, ldx, y, ldy, strm);
    return e == hipSuccess ? LORA_OK : hip_fail(e);
  }
  const char* plan = reinterpret_cast<const char*>(given_plan);
  if (plan == nullptr) {
    const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
    plan = reinterpret_cast<const char*>(ws) + L.plan;
    if (phases & 1) e = form_plan(s, s.n, T, ids, nullptr, 0, seg_off, perm, ws, &plan, strm);
  }
  if (e == hipSuccess && (phases & 1)) e = launch_shrink(s, plan, T, x, ldx, ws, strm);
  if (e == hipSuccess && (phases & 2)) e = launch_expand(s, plan, T, ws, nullptr, 0, y, ldy, strm);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

int lora_apply_batched(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy,
                       int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm, void* ws,
                       size_t ws_bytes, void* stream) {
  return apply_impl(store_host, x, ldx, y, ldy, T, ids, seg_off, perm, nullptr, ws, ws_bytes, stream, 3);
}

int lora_apply_planned_phases(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                              const void* plan, size_t plan_bytes_, void* ws, size_t ws_bytes, void* stream,
                              int phases) {
  const int st = check_store(store_host);
  if (st != LORA_OK) return st;
  if (T < 0) return LORA_ERR_INVALID_ARG;
  const int sp = check_plan(plan, plan_bytes_, T, store_host->n);
  if (sp != LORA_OK) return sp;
  return apply_impl(store_host, x, ldx, y, ldy, T, nullptr, nullptr, nullptr, T > 0 ? plan : nullptr, ws, ws_bytes,
                    stream, phases);
}

int lora_apply_planned(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                       const void* plan, size_t plan_bytes_, void* ws, size_t ws_bytes, void* stream) {
  return lora_apply_planned_phases(store_host, x, ldx, y, ldy, T, plan, plan_bytes_, ws, ws_bytes, stream, 3);
}

// ------------------------------------------------------------ no allocation
// The workspace of lora_apply_batched_noalloc: one array per device, resident
// for the life of the process.  Host code never uses its name as an address
// (in host code it is a stand-in, not device memory): the device address is
// looked up once per device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];
static std::atomic<void*> g_scratch[kMaxDevices];  // per device; null until looked up

// The scratch array's address on the current device (looked up on first use
// there; two threads racing both look it up and store the same address).
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

int lora_apply_batched_noalloc(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy,
                               int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm,
                               void* stream) {
  // Every argument check before any HIP call; then the size the call needs
  // against the scratch array's.
  const int st = check_apply_args(store_host, x, ldx, y, ldy, T, ids, seg_off, perm);
  if (st != LORA_OK) return st;
  if (workspace_bytes(store_host, T) > (size_t)LORA_NOALLOC_SCRATCH_BYTES) return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  return apply_impl(store_host, x, ldx, y, ldy, T, ids, seg_off, perm, nullptr, ws,
                    (size_t)LORA_NOALLOC_SCRATCH_BYTES, stream, 3);
}

// ------------------------------------------------------- base layer fused
int lora_apply_base_fused(const lora_store* store_host, const void* W0, int64_t ldw, const void* x, int64_t ldx,
                          void* y, int64_t ldy, int T, const int32_t* ids, void* ws, size_t ws_bytes,
                          void* stream) {
  int st = check_store(store_host);
  if (st != LORA_OK) return st;
  const lora_store& s = *store_host;
  if (T < 0) return LORA_ERR_INVALID_ARG;
  if (s.dtype != LORA_DTYPE_BF16) return LORA_ERR_UNSUPPORTED;
  if ((st = check_rows(x, ldx, s.d_in, s.dtype, T)) != LORA_OK) return st;
  if ((st = check_rows(y, ldy, s.d_out, s.dtype, T)) != LORA_OK) return st;
  if (W0 == nullptr) return LORA_ERR_INVALID_ARG;
  if ((st = check_rows(W0, ldw, s.d_in, s.dtype, s.d_out)) != LORA_OK) return st;
  constexpr int64_t kLimit = (int64_t)1 << 31;  // 32-bit buffer offsets
  if (256 * ldw * 2 >= kLimit || (int64_t)T * ldx * 2 >= kLimit) return LORA_ERR_UNSUPPORTED;
  if (ids != nullptr) {
    if (T > LORA_SEGMENT_MAX_T || s.n > LORA_SEGMENT_MAX_N) return LORA_ERR_UNSUPPORTED;
    if ((int64_t)s.R * s.d_out * 2 >= kLimit) return LORA_ERR_UNSUPPORTED;
    if ((st = check_ws(store_host, T, ws, ws_bytes)) != LORA_OK) return st;
  }
  if (T == 0) return LORA_OK;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  const int32_t* perm = nullptr;
  if (ids != nullptr) {
    // The grouping with its permutation kept in ws (the GEMM takes tokens in
    // grouped order), the plan, then the shrink's partial sums.
    const WsLayout L = ws_layout(T, s.n, s.d_in, s.r_max, s.dtype);
    char* base = reinterpret_cast<char*>(ws);
    int32_t* so = reinterpret_cast<int32_t*>(base + L.seg_off);
    int32_t* pm = reinterpret_cast<int32_t*>(base + L.perm);
    char* pl = base + L.plan;
    if (group_fits(T, s.n)) {
      e = launch_group(ids, T, s.n, nullptr, 0, so, pm, pl, nullptr, strm);
    } else {
      e = launch_segment(ids, T, s.n, so, pm, nullptr, strm);
      if (e == hipSuccess) e = launch_plan(so, pm, T, s.n, pl, nullptr, nullptr, strm);
    }
    if (e == hipSuccess) e = launch_shrink(s, pl, T, x, ldx, ws, strm);
    perm = pm;
  }
  if (e == hipSuccess) e = launch_base_fused(s, W0, ldw, x, ldx, y, ldy, T, perm, ids, ws, strm);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

// Shared-basis workspace: h [T][ldp] | the basis store's workspace.
static size_t jd_h_bytes(const lora_store& b, int T) {
  return align_up((size_t)(T > 0 ? T : 0) * (size_t)partial_ld(b.r_max) * 4, 256);
}

static int check_jd_store(const lora_jd_store* s) {
  if (!s) return LORA_ERR_INVALID_ARG;
  const int st = check_store(&s->basis);
  if (st != LORA_OK) return st;
  if (s->n_adapters < 1 || s->r < 1 || s->r != s->basis.r_max || (int64_t)s->basis.R != (int64_t)s->basis.n * s->r ||
      (s->diag != 0 && s->diag != 1) || !s->cluster_of || !s->sigma || !s->scale)
    return LORA_ERR_INVALID_ARG;
  if (s->basis.n > kGroupMaxN || s->n_adapters > LORA_SEGMENT_MAX_N) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

size_t lora_jd_workspace_bytes(const lora_jd_store* store_host, int T) {
  if (check_jd_store(store_host) != LORA_OK || T < 0) return 0;
  return jd_h_bytes(store_host->basis, T) + workspace_bytes(&store_host->basis, T);
}

int lora_jd_apply(const lora_jd_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy, int T,
                  const int32_t* ids, void* ws, size_t ws_bytes, void* stream) {
  int st = check_jd_store(store_host);
  if (st != LORA_OK) return st;
  const lora_jd_store& j = *store_host;
  const lora_store& b = j.basis;
  if (T < 0) return LORA_ERR_INVALID_ARG;
  if ((st = check_rows(x, ldx, b.d_in, b.dtype, T)) != LORA_OK) return st;
  if ((st = check_rows(y, ldy, b.d_out, b.dtype, T)) != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  if (!ids || !ws) return LORA_ERR_INVALID_ARG;
  if (!aligned16(ws)) return LORA_ERR_UNSUPPORTED;
  if (!group_fits(T, b.n)) return LORA_ERR_UNSUPPORTED;  // the grouping by cluster runs in one workgroup
  if (ws_bytes < lora_jd_workspace_bytes(store_host, T)) return LORA_ERR_INVALID_ARG;
  char* base = reinterpret_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(base);
  void* bws = base + jd_h_bytes(b, T);
  const int64_t ldh = partial_ld(b.r_max);
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  const char* plan = nullptr;
  hipError_t e = form_plan(b, b.n, T, ids, j.cluster_of, j.n_adapters, nullptr, nullptr, bws, &plan, strm);
  if (e == hipSuccess) e = launch_shrink(b, plan, T, x, ldx, bws, strm);
  if (e == hipSuccess)
    e = launch_jd_sigma(b, plan, T, bws, ids, j.n_adapters, j.cluster_of, j.sigma, j.diag, j.scale, h, ldh, strm);
  if (e == hipSuccess) e = launch_expand(b, plan, T, bws, h, ldh, y, ldy, strm);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

int lora_apply_launches(const lora_store* store_host, int T, int with_ids) {
  const int st = check_store(store_host);
  if (st != LORA_OK) return -st;
  if (T < 0) return -LORA_ERR_INVALID_ARG;
  const lora_store& s = *store_host;
  if (with_ids == 1 && (T > LORA_SEGMENT_MAX_T || s.n > LORA_SEGMENT_MAX_N)) return -LORA_ERR_UNSUPPORTED;
  if (with_ids < 0 || with_ids > 2) return -LORA_ERR_INVALID_ARG;
  if (T == 0) return 0;
  if (with_ids == 2) return 2;  // a plan: shrink, expand
  if (decode_apply_fits(s, T, with_ids != 0)) return 1;
  return (with_ids && !group_fits(T, s.n)) ? 4 : 3;
}

int lora_apply_batched_phases(const lora_store* store_host, const void* x, int64_t ldx, void* y, int64_t ldy,
                              int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm, void* ws,
                              size_t ws_bytes, void* stream, int phases) {
  return apply_impl(store_host, x, ldx, y, ldy, T, ids, seg_off, perm, nullptr, ws, ws_bytes, stream, phases);
}

size_t lora_rsvd_workspace_bytes(int n, int d_in, int d_out) {
  if (n < 0 || d_in < 1 || d_out < 1) return 0;
  return rsvd_workspace_bytes(n);
}

static int check_rsvd(int n, int d_in, int d_out, int dtype, int r) {
  if (n < 0 || d_in < 1 || d_out < 1 || r < 1) return LORA_ERR_INVALID_ARG;
  if (dtype != LORA_DTYPE_BF16 && dtype != LORA_DTYPE_F32) return LORA_ERR_UNSUPPORTED;
  if (r > LORA_MAX_RANK || d_in < r || d_out < r) return LORA_ERR_UNSUPPORTED;
  const int v = dtype == LORA_DTYPE_BF16 ? 8 : 4;  // rows are read as 16-byte vectors
  if (d_in % v != 0 || d_out % v != 0) return LORA_ERR_UNSUPPORTED;
  // Grids (workgroups of 256 threads) stay below 2^32 threads.
  const int64_t wgs = (int64_t)n * (2 + (d_in + 255) / 256 + (d_out + 255) / 256);
  if (wgs * 256 >= ((int64_t)1 << 32)) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

int lora_rsvd_factor_phases(int n, int d_in, int d_out, int dtype, int r, const void* A_all, const void* B_all,
                            float* sigma, int32_t* status, void* ws, size_t ws_bytes, void* stream, int phases) {
  if (phases < 1 || phases > 15) return LORA_ERR_INVALID_ARG;
  int st = check_rsvd(n, d_in, d_out, dtype, r);
  if (st != LORA_OK) return st;
  if (n == 0) return LORA_OK;
  if (!A_all || !B_all || !sigma || !status || !ws) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < rsvd_workspace_bytes(n)) return LORA_ERR_INVALID_ARG;
  if (!aligned16(ws) || !aligned16(A_all) || !aligned16(B_all)) return LORA_ERR_UNSUPPORTED;
  hipError_t e = launch_rsvd_factor(n, d_in, d_out, dtype, r, A_all, B_all, sigma, status, ws,
                                    reinterpret_cast<hipStream_t>(stream), phases);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

int lora_rsvd_factor(int n, int d_in, int d_out, int dtype, int r, const void* A_all, const void* B_all,
                     float* sigma, int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  return lora_rsvd_factor_phases(n, d_in, d_out, dtype, r, A_all, B_all, sigma, status, ws, ws_bytes, stream, 15);
}

int lora_rsvd_write(const lora_store* store_host, int r, const void* A_all, const void* B_all, const void* ws,
                    size_t ws_bytes, void* stream) {
  int st = check_store(store_host);
  if (st != LORA_OK) return st;
  const lora_store& s = *store_host;
  st = check_rsvd(s.n, s.d_in, s.d_out, s.dtype, r);
  if (st != LORA_OK) return st;
  if (s.n == 0 || s.R == 0) return LORA_OK;
  if (!A_all || !B_all || !ws) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < rsvd_workspace_bytes(s.n)) return LORA_ERR_INVALID_ARG;
  if (!aligned16(ws) || !aligned16(A_all) || !aligned16(B_all)) return LORA_ERR_UNSUPPORTED;
  hipError_t e = launch_rsvd_write(s, r, A_all, B_all, ws, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

static int check_slices(int n_slices, const lora_store* sl) {
  if (!sl || n_slices < 1 || n_slices > LORA_MAX_SLICES) return LORA_ERR_INVALID_ARG;
  for (int k = 0; k < n_slices; ++k) {
    const int st = check_store(&sl[k]);
    if (st != LORA_OK) return st;
    if (sl[k].n != sl[0].n || sl[k].d_in != sl[0].d_in || sl[k].dtype != sl[0].dtype) return LORA_ERR_INVALID_ARG;
  }
  return LORA_OK;
}

int lora_multi_bytes(int n_slices, const lora_store* slices_host, size_t* a_bytes_host, size_t* meta_bytes_host,
                     size_t* hoff_bytes_host) {
  if (!a_bytes_host || !meta_bytes_host || !hoff_bytes_host) return LORA_ERR_INVALID_ARG;
  const int st = check_slices(n_slices, slices_host);
  if (st != LORA_OK) return st;
  int64_t R = 0;  // the stacked total rank is the sum of the slices' totals
  for (int k = 0; k < n_slices; ++k) R += slices_host[k].R;
  if (R > INT32_MAX) return LORA_ERR_INVALID_ARG;
  const lora_store& s0 = slices_host[0];
  *a_bytes_host = (size_t)R * s0.d_in * elem_bytes(s0.dtype);
  *meta_bytes_host = meta_bytes(s0.n);
  *hoff_bytes_host = (size_t)n_slices * s0.n * sizeof(int32_t);
  return LORA_OK;
}

int lora_pack_multi(lora_multi_store* out_host, int n_slices, const lora_store* slices_host, void* A_stacked,
                    void* meta, int32_t* hoff, void* stream) {
  size_t ab = 0, mb = 0, hb = 0;
  int st = lora_multi_bytes(n_slices, slices_host, &ab, &mb, &hb);
  if (st != LORA_OK) return st;
  if (!out_host || !meta || !hoff || (ab > 0 && !A_stacked)) return LORA_ERR_INVALID_ARG;
  if (!aligned16(meta) || !aligned16(hoff) || (A_stacked && !aligned16(A_stacked))) return LORA_ERR_UNSUPPORTED;
  const lora_store& s0 = slices_host[0];
  const int n = s0.n;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // The slices' stored ranks, read back.
  std::vector<int32_t> rk((size_t)n_slices * n);
  for (int k = 0; k < n_slices; ++k) {
    hipError_t e = hipMemcpyAsync(rk.data() + (size_t)k * n, slices_host[k].rank, (size_t)n * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  std::vector<char> img(mb, 0);
  int32_t* row_off = reinterpret_cast<int32_t*>(img.data());
  int32_t* rank = row_off + (n + 1);
  float* scale = reinterpret_cast<float*>(rank + n);
  int32_t* true_rank = reinterpret_cast<int32_t*>(scale + n);
  std::vector<int32_t> ho((size_t)n_slices * n);
  int r_max = 0;
  row_off[0] = 0;
  for (int a = 0; a < n; ++a) {
    int r = 0;
    for (int k = 0; k < n_slices; ++k) {
      const int v = rk[(size_t)k * n + a];
      if (v < 0 || v > LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;  // not a store's metadata
      ho[(size_t)k * n + a] = r;
      r += v;
    }
    if (r > LORA_MAX_RANK) return LORA_ERR_UNSUPPORTED;
    rank[a] = true_rank[a] = r;
    scale[a] = 1.f;
    row_off[a + 1] = row_off[a] + r;
    r_max = r > r_max ? r : r_max;
  }
  const int R = row_off[n];
  if ((size_t)R * s0.d_in * elem_bytes(s0.dtype) != ab) return LORA_ERR_INVALID_ARG;  // ranks disagree with R
  e = hipMemcpyAsync(meta, img.data(), img.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(hoff, ho.data(), hb, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = launch_stack_rows(n, s0.d_in, s0.dtype, n_slices, R, reinterpret_cast<const int32_t*>(meta), hoff,
                          slices_host, A_stacked, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  lora_multi_store m;
  std::memset(&m, 0, sizeof(m));
  m.n_slices = n_slices;
  for (int k = 0; k < n_slices; ++k) m.slice[k] = slices_host[k];
  lora_store& t = m.stacked;
  t.n = n;
  t.d_in = s0.d_in;
  t.d_out = s0.d_in;  // B_pack aliases A_pack: bounded by A's size
  t.dtype = s0.dtype;
  t.r_max = r_max;
  t.R = R;
  t.pad_to = 0;
  t.A_pack = A_stacked;
  t.B_pack = A_stacked;
  t.row_off = reinterpret_cast<const int32_t*>(meta);
  t.rank = t.row_off + (n + 1);
  t.scale = reinterpret_cast<const float*>(t.rank + n);
  m.hoff = hoff;
  *out_host = m;
  return LORA_OK;
}

static int check_multi(const lora_multi_store* m) {
  if (!m || !m->hoff) return LORA_ERR_INVALID_ARG;
  int st = check_slices(m->n_slices, m->slice);
  if (st != LORA_OK) return st;
  if ((st = check_store(&m->stacked)) != LORA_OK) return st;
  const lora_store& t = m->stacked;
  if (t.n != m->slice[0].n || t.d_in != m->slice[0].d_in || t.dtype != m->slice[0].dtype) return LORA_ERR_INVALID_ARG;
  return LORA_OK;
}

size_t lora_multi_workspace_bytes(const lora_multi_store* store_host, int T) {
  if (check_multi(store_host) != LORA_OK || T < 0) return 0;
  const size_t base = workspace_bytes(&store_host->stacked, T);
  return base ? base + slice_meta_bytes(T, store_host->stacked.n, store_host->n_slices) : 0;
}

static int multi_impl(const lora_multi_store* store_host, const void* x, int64_t ldx, void* const* y_host,
                      const int64_t* ldy_host, int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm,
                      const void* given_plan, void* ws, size_t ws_bytes, void* stream) {
  int st = check_multi(store_host);
  if (st != LORA_OK) return st;
  const lora_multi_store& m = *store_host;
  const lora_store& s = m.stacked;
  if (T < 0 || !y_host || !ldy_host) return LORA_ERR_INVALID_ARG;
  if ((st = check_rows(x, ldx, s.d_in, s.dtype, T)) != LORA_OK) return st;
  for (int k = 0; k < m.n_slices; ++k)
    if ((st = check_rows(y_host[k], ldy_host[k], m.slice[k].d_out, s.dtype, T)) != LORA_OK) return st;
  if ((st = check_ws(&s, T, ws, ws_bytes)) != LORA_OK) return st;
  if (T > 0 && ws_bytes < lora_multi_workspace_bytes(store_host, T)) return LORA_ERR_INVALID_ARG;
  if (ids != nullptr && (T > LORA_SEGMENT_MAX_T || s.n > LORA_SEGMENT_MAX_N)) return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;
  if (given_plan == nullptr && ids == nullptr && (st = check_grouping(&s, T, seg_off, perm)) != LORA_OK) return st;
  hipStream_t strm = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  const char* plan = reinterpret_cast<const char*>(given_plan);
  if (plan == nullptr) e = form_plan(s, s.n, T, ids, nullptr, 0, seg_off, perm, ws, &plan, strm);
  // The slice records follow the stacked store's workspace.
  SliceMeta* sl_meta = reinterpret_cast<SliceMeta*>(reinterpret_cast<char*>(ws) + workspace_bytes(&s, T));
  if (e == hipSuccess) e = launch_shrink_slices(m, sl_meta, plan, T, x, ldx, ws, strm);
  if (e == hipSuccess) e = launch_expand_slices(m, sl_meta, plan, T, ws, y_host, ldy_host, strm);
  return e == hipSuccess ? LORA_OK : hip_fail(e);
}

int lora_apply_multi(const lora_multi_store* store_host, const void* x, int64_t ldx, void* const* y_host,
                     const int64_t* ldy_host, int T, const int32_t* ids, const int32_t* seg_off, const int32_t* perm,
                     void* ws, size_t ws_bytes, void* stream) {
  return multi_impl(store_host, x, ldx, y_host, ldy_host, T, ids, seg_off, perm, nullptr, ws, ws_bytes, stream);
}

int lora_apply_multi_planned(const lora_multi_store* store_host, const void* x, int64_t ldx, void* const* y_host,
                             const int64_t* ldy_host, int T, const void* plan, size_t plan_bytes_, void* ws,
                             size_t ws_bytes, void* stream) {
  const int st = check_multi(store_host);
  if (st != LORA_OK) return st;
  if (T < 0) return LORA_ERR_INVALID_ARG;
  const int sp = check_plan(plan, plan_bytes_, T, store_host->stacked.n);
  if (sp != LORA_OK) return sp;
  return multi_impl(store_host, x, ldx, y_host, ldy_host, T, nullptr, nullptr, nullptr, T > 0 ? plan : nullptr, ws,
                    ws_bytes, stream);
}

}  // extern "C"
