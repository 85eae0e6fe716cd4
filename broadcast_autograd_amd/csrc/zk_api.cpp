// zk_api.cpp -- the extern "C" boundary (include/zk.h).
//
// Every argument is validated and the whole launch plan is built on the host
// before the first HIP call; an error returns with nothing launched and no
// output written.  The library keeps no state between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "zk.h"
#include "zk_kernels.h"
#include "zk_plan.h"

using namespace zk;

namespace {

bool valid_op(zk_op op) { return op >= ZK_ADD && op <= ZK_DIV; }
bool valid_epi(zk_epi e) {
  return e == ZK_EPI_NONE || e == ZK_EPI_GELU || e == ZK_EPI_RELU;
}

int64_t numel(const zk_desc &d) {
  int64_t m = 1;
  for (int k = 0; k < d.rank; ++k) m *= d.sizes[k];
  return m;
}

// The operand is dense row-major with exactly `n` elements in the broadcast
// layout (sizes equal to the trailing out sizes, dense strides).
bool dense_full(const zk_desc &d, int64_t out_numel) {
  if (numel(d) != out_numel) return false;
  int64_t s = 1;
  for (int k = d.rank - 1; k >= 0; --k) {
    if (d.sizes[k] != 1 && d.strides[k] != s) return false;
    s *= d.sizes[k];
  }
  return true;
}

struct Ext {
  uintptr_t lo = 0, hi = 0;
};
Ext ext_of(const void *p, const zk_desc &d) {
  Ext e;
  if (p) byte_extent(p, d, &e.lo, &e.hi);
  return e;
}
Ext ext_dense(const void *p, int64_t n) {
  Ext e;
  if (p) byte_extent_dense(p, n, &e.lo, &e.hi);
  return e;
}
bool ov(const Ext &a, const Ext &b) { return overlaps(a.lo, a.hi, b.lo, b.hi); }

zk_status hip_status(hipError_t e) { return e == hipSuccess ? ZK_OK : ZK_ERR_HIP; }

// Workspace a backward call needs, as a function of the shapes (and of which
// gradients are requested) only: the larger of the plans for 16-byte aligned
// and for misaligned pointers, since alignment picks between them.
size_t bwd_workspace(zk_op op, zk_epi epi, const zk_desc &da,
                     const zk_desc &db, bool wa, bool wb) {
  size_t m = 0;
  for (uintptr_t q : {(uintptr_t)0, (uintptr_t)4}) {
    BwdPlan p;
    if (plan_bwd(op, epi, da, db, wa, wb, q, q, q, q, q, q, q, &p) == ZK_OK)
      m = p.workspace > m ? p.workspace : m;
  }
  return m;
}

bool valid_op2(zk_op op) { return op == ZK_ADD || op == ZK_SUB; }

// Dense row-major descriptor of a shape.
zk_desc dense_desc(int r, const int64_t *n) {
  zk_desc d{};
  d.rank = r;
  int64_t s = 1;
  for (int k = r - 1; k >= 0; --k) {
    d.sizes[k] = n[k];
    d.strides[k] = s;
    s *= n[k];
  }
  return d;
}

bool same_view(const zk_desc &x, const zk_desc &y) {
  if (x.rank != y.rank) return false;
  for (int k = 0; k < x.rank; ++k)
    if (x.sizes[k] != y.sizes[k] || (x.sizes[k] != 1 && x.strides[k] != y.strides[k]))
      return false;
  return true;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// The kernels keep binary64 partials in the workspace: 8-byte alignment
// (hipMalloc and torch allocations are 256-byte aligned).
bool ws_aligned(const void *ws, size_t need) {
  return need == 0 || ((uintptr_t)ws & 7u) == 0;
}

size_t reduce_workspace(const zk_desc &din, int rout, const int64_t *nout);

// Layout of the fused backward's workspace (shapes only):
//   [op1 backward][c reduction][t gradient buffer][t reduction]
struct Bwd2Layout {
  size_t op1 = 0, cred = 0, tbuf = 0, tred = 0;
  size_t total() const { return op1 + cred + tbuf + tred; }
};
Bwd2Layout bwd2_layout(zk_op op1, const zk_desc &da, const zk_desc &db,
                       const zk_desc &dc, int r, const int64_t *n, bool wa, bool wb,
                       bool wc) {
  Bwd2Layout L;
  int rab;
  int64_t nab[kMaxDims];
  broadcast_shape(da.rank, da.sizes, db.rank, db.sizes, &rab, nab);
  const zk_desc ds = dense_desc(r, n);
  const int64_t ns = numel(ds), nab_el = numel(dense_desc(rab, nab));
  L.op1 = round256(bwd_workspace(op1, ZK_EPI_NONE, da, db, wa, wb));
  if (wc && numel(dc) < ns) L.cred = round256(reduce_workspace(ds, dc.rank, dc.sizes));
  if (nab_el < ns && (wa || wb)) {
    L.tbuf = round256((size_t)nab_el * 4u);
    L.tred = round256(reduce_workspace(ds, rab, nab));
  }
  return L;
}

size_t reduce_workspace(const zk_desc &din, int rout, const int64_t *nout) {
  size_t m = 0;
  for (uintptr_t q : {(uintptr_t)0, (uintptr_t)4}) {
    BwdPlan p;
    if (plan_reduce(din, rout, nout, q, q, &p) == ZK_OK)
      m = p.workspace > m ? p.workspace : m;
  }
  return m;
}

// ------------------------------------------------ debug pointer checks
// -1: not decided yet (ZK_DEBUG is read at the first consultation).
std::atomic<int32_t> g_debug{-1};

int32_t debug_mode() {
  int32_t d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char *e = std::getenv("ZK_DEBUG");
    int32_t want = (e && std::strcmp(e, "1") == 0) ? 1 : 0, expect = -1;
    g_debug.compare_exchange_strong(expect, want, std::memory_order_relaxed);
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d;
}

// With debug checks on: ZK_OK only when every non-NULL pointer is device
// memory of the stream's device (or managed memory); no launch otherwise.
zk_status debug_check_list(void *stream, const void *const *ptrs, size_t n) {
  if (debug_mode() != 1) return ZK_OK;
  int dev = -1;
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // leave no error for the caller's next call
    return ZK_ERR_DEVICE;
  }
  std::vector<PtrRecord> recs;
  recs.reserve(n);
  for (size_t i = 0; i < n; ++i) {
    if (!ptrs[i]) continue;
    hipPointerAttribute_t a{};
    PtrRecord r{0, kMemUnregistered, -1};
    if (hipPointerGetAttributes(&a, ptrs[i]) == hipSuccess) {
      r.known = 1;
      r.mem_type = a.isManaged ? kMemManaged : (int32_t)a.type;
      r.device = a.device;
    } else {
      (void)hipGetLastError();
    }
    recs.push_back(r);
  }
  return check_ptr_records(recs.data(), (int)recs.size(), dev);
}

zk_status debug_check(void *stream, std::initializer_list<const void *> ptrs) {
  return debug_check_list(stream, ptrs.begin(), ptrs.size());
}

// ------------------------------------------------ optional kernel timing
struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> start, end;
  std::vector<int32_t> ids;
  int next = 0;
};
Profiler &prof() {
  static Profiler p;
  return p;
}

}  // namespace

namespace zk {
ProfScope::ProfScope(int32_t kernel) : slot(-1), ev_start(nullptr), ev_end(nullptr) {
  Profiler &p = prof();
  if (!p.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> g(p.mu);
  if (p.next >= (int)p.start.size()) return;
  slot = p.next++;
  p.ids[slot] = kernel;
  ev_start = p.start[slot];
  ev_end = p.end[slot];
}
}  // namespace zk

extern "C" {

zk_status zk_profile_start(int32_t capacity) {
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = false;
  for (auto e : p.start) (void)hipEventDestroy(e);
  for (auto e : p.end) (void)hipEventDestroy(e);
  p.start.clear();
  p.end.clear();
  p.ids.assign(capacity > 0 ? capacity : 0, -1);
  p.next = 0;
  for (int i = 0; i < capacity; ++i) {
    // No system-scope fence: the events only time device work.
    const unsigned fl = hipEventDisableSystemFence;
    hipEvent_t a, b;
    if (hipEventCreateWithFlags(&a, fl) != hipSuccess) return ZK_ERR_HIP;
    if (hipEventCreateWithFlags(&b, fl) != hipSuccess) {
      (void)hipEventDestroy(a);
      return ZK_ERR_HIP;
    }
    p.start.push_back(a);
    p.end.push_back(b);
  }
  p.on = true;
  return ZK_OK;
}

zk_status zk_profile_stop(void) {
  prof().on = false;
  return ZK_OK;
}

zk_status zk_profile_read(int32_t max, int32_t *kernel_ids, float *ms,
                          int32_t *count) {
  if (!count || (max > 0 && (!kernel_ids || !ms))) return ZK_ERR_NULL;
  Profiler &p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  int n = p.next < max ? p.next : max;
  for (int i = 0; i < n; ++i) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.start[i], p.end[i]) != hipSuccess) return ZK_ERR_HIP;
    kernel_ids[i] = p.ids[i];
    ms[i] = t;
  }
  *count = n;
  return ZK_OK;
}

const char *zk_status_string(zk_status s) {
  switch (s) {
    case ZK_OK: return "ok";
    case ZK_ERR_NULL: return "a required pointer is NULL";
    case ZK_ERR_RANK: return "rank out of range [0, 8]";
    case ZK_ERR_BAD_SIZE: return "negative size";
    case ZK_ERR_BAD_STRIDE: return "negative stride";
    case ZK_ERR_BROADCAST: return "shapes do not broadcast";
    case ZK_ERR_ALIAS: return "an output overlaps an input or another output";
    case ZK_ERR_WORKSPACE:
      return "workspace too small or not 8-byte aligned (zk_binary_bwd_noalloc: the call "
             "needs more than ZK_SCRATCH_BYTES)";
    case ZK_ERR_UNSUPPORTED: return "unsupported op or epilogue";
    case ZK_ERR_HIP: return "HIP launch failed";
    case ZK_ERR_SHAPE: return "target shape does not broadcast to the input";
    case ZK_ERR_DEVICE: return "a pointer is not device memory of the stream's device";
  }
  return "unknown status";
}

const char *zk_kernel_name(int32_t k) { return kernel_name(k); }

int32_t zk_set_debug(int32_t mode) {
  const int32_t before = debug_mode();
  if (mode == 0 || mode == 1) g_debug.store(mode, std::memory_order_relaxed);
  return before;
}

zk_status zk_broadcast_shape(int32_t rank_a, const int64_t *sizes_a,
                             int32_t rank_b, const int64_t *sizes_b,
                             int32_t *rank_out, int64_t sizes_out[ZK_MAX_DIMS]) {
  if (!rank_out || !sizes_out) return ZK_ERR_NULL;
  int r = 0;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape(rank_a, sizes_a, rank_b, sizes_b, &r, n);
  if (s) return s;
  *rank_out = r;
  for (int k = 0; k < r; ++k) sizes_out[k] = n[k];
  return ZK_OK;
}

zk_status zk_binary_fwd(zk_op op, zk_epi epi, const float *a, const zk_desc *da,
                        const float *b, const zk_desc *db, float *out,
                        void *stream) {
  if (!valid_op(op) || !valid_epi(epi)) return ZK_ERR_UNSUPPORTED;
  zk_status s;
  if ((s = check_desc(da)) || (s = check_desc(db))) return s;
  FwdPlan p;
  if ((s = plan_fwd(op, epi, *da, *db, (uintptr_t)a, (uintptr_t)b,
                    (uintptr_t)out, &p)))
    return s;
  if (p.empty) return ZK_OK;
  if (!a || !b || !out) return ZK_ERR_NULL;
  const int64_t n = p.c.numel;
  Ext eo = ext_dense(out, n), ea = ext_of(a, *da), eb = ext_of(b, *db);
  if (ov(eo, ea) && !(out == a && dense_full(*da, n))) return ZK_ERR_ALIAS;
  if (ov(eo, eb) && !(out == b && dense_full(*db, n))) return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {a, b, out}))) return s;
  return hip_status(launch_fwd(p, op, epi, a, b, out, (hipStream_t)stream));
}

}  // extern "C"

namespace {
// zk_binary_bwd; lib_ws: the workspace is the library's own scratch array
// (left out of the debug pointer check, which asks about caller memory).
zk_status binary_bwd_impl(zk_op op, zk_epi epi, const float *grad, const float *a,
                          const zk_desc *da, const float *b, const zk_desc *db,
                          float *grad_a, const float *acc_a, float *grad_b,
                          const float *acc_b, void *workspace, size_t *workspace_bytes,
                          void *stream, bool lib_ws) {
  if (!valid_op(op) || !valid_epi(epi)) return ZK_ERR_UNSUPPORTED;
  if (!workspace_bytes) return ZK_ERR_NULL;
  zk_status s;
  if ((s = check_desc(da)) || (s = check_desc(db))) return s;
  BwdPlan p;
  if ((s = plan_bwd(op, epi, *da, *db, grad_a != nullptr, grad_b != nullptr,
                    (uintptr_t)grad, (uintptr_t)a, (uintptr_t)b,
                    (uintptr_t)grad_a, (uintptr_t)grad_b, (uintptr_t)acc_a,
                    (uintptr_t)acc_b, &p)))
    return s;
  const size_t need = bwd_workspace(op, epi, *da, *db, grad_a != nullptr,
                                    grad_b != nullptr);
  if (!workspace) {
    *workspace_bytes = need;
    return ZK_OK;
  }
  if (*workspace_bytes < need || !ws_aligned(workspace, need)) return ZK_ERR_WORKSPACE;
  const int64_t n = p.c.numel;
  const int64_t na = numel(*da), nb = numel(*db);
  if (n > 0 && (!grad || !a || !b)) return ZK_ERR_NULL;
  // Extents of everything written and read.
  Ext eg = ext_dense(grad, n), ea = ext_of(a, *da), eb = ext_of(b, *db);
  Ext ega = ext_dense(grad_a, na), egb = ext_dense(grad_b, nb);
  Ext exa = ext_dense(acc_a, na), exb = ext_dense(acc_b, nb);
  Ext ews;
  if (need) ews = Ext{(uintptr_t)workspace, (uintptr_t)workspace + need};
  const Ext outs[2] = {ega, egb};
  const float *gp[2] = {grad_a, grad_b};
  const float *accp[2] = {acc_a, acc_b};
  const Ext accs[2] = {exa, exb};
  if (ov(ega, egb)) return ZK_ERR_ALIAS;
  for (int w = 0; w < 2; ++w) {
    if (!gp[w]) continue;
    const Ext &o = outs[w];
    if (ov(o, eg) || ov(o, ea) || ov(o, eb) || ov(o, ews)) return ZK_ERR_ALIAS;
    if (ov(o, accs[w]) && accp[w] != gp[w]) return ZK_ERR_ALIAS;
    if (ov(o, accs[1 - w])) return ZK_ERR_ALIAS;
  }
  if (need && (ov(ews, eg) || ov(ews, ea) || ov(ews, eb) || ov(ews, exa) ||
                      ov(ews, exb)))
    return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {grad, a, b, grad_a, acc_a, grad_b, acc_b,
                                need && !lib_ws ? workspace : nullptr})))
    return s;
  return hip_status(launch_bwd(p, op, epi, grad, a, b, grad_a, acc_a, grad_b,
                               acc_b, workspace, (hipStream_t)stream));
}
}  // namespace

extern "C" {

zk_status zk_binary_bwd(zk_op op, zk_epi epi, const float *grad, const float *a,
                        const zk_desc *da, const float *b, const zk_desc *db,
                        float *grad_a, const float *acc_a, float *grad_b,
                        const float *acc_b, void *workspace,
                        size_t *workspace_bytes, void *stream) {
  return binary_bwd_impl(op, epi, grad, a, da, b, db, grad_a, acc_a, grad_b, acc_b, workspace,
                         workspace_bytes, stream, false);
}

zk_status zk_binary_bwd_noalloc(zk_op op, zk_epi epi, const float *grad, const float *a,
                                const zk_desc *da, const float *b, const zk_desc *db,
                                float *grad_a, const float *acc_a, float *grad_b,
                                const float *acc_b, void *stream) {
  // the workspace need, from the shapes alone (host planning, nothing launched)
  size_t need = 0;
  zk_status s = zk_binary_bwd(op, epi, grad, a, da, b, db, grad_a, acc_a, grad_b, acc_b,
                              nullptr, &need, nullptr);
  if (s) return s;
  if (need > ZK_SCRATCH_BYTES) return ZK_ERR_WORKSPACE;
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return ZK_ERR_DEVICE;
  }
  if (stream) {
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return ZK_ERR_DEVICE;
    }
    if (sdev != dev) return ZK_ERR_DEVICE;
  }
  void *ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) {
    (void)hipGetLastError();
    return ZK_ERR_HIP;
  }
  size_t cap = ZK_SCRATCH_BYTES;
  return binary_bwd_impl(op, epi, grad, a, da, b, db, grad_a, acc_a, grad_b, acc_b, ws, &cap,
                         stream, true);
}

}  // extern "C"

namespace {
// Product of in's sizes over the dims where the target is 1 or missing:
// the number of input elements each target element sums.
int64_t reduced_count(int rin, const int64_t *nin, int rout, const int64_t *nout) {
  int64_t c = 1;
  for (int k = 0; k < rin; ++k) {
    const int ko = k - (rin - rout);
    if (ko < 0 || nout[ko] == 1) c *= nin[k];
  }
  return c;
}

zk_status reduce_common(const float *in, const zk_desc *din, int32_t rank_out,
                        const int64_t *sizes_out, float *out, void *workspace,
                        size_t *workspace_bytes, void *stream, bool mean) {
  if (!workspace_bytes) return ZK_ERR_NULL;
  zk_status s;
  if ((s = check_desc(din))) return s;
  if (rank_out < 0 || rank_out > kMaxDims) return ZK_ERR_RANK;
  if (rank_out > 0 && !sizes_out) return ZK_ERR_NULL;
  for (int k = 0; k < rank_out; ++k)
    if (sizes_out[k] < 0) return ZK_ERR_BAD_SIZE;
  BwdPlan p;
  if ((s = plan_reduce(*din, rank_out, sizes_out, (uintptr_t)in, (uintptr_t)out, &p)))
    return s;
  const size_t need = reduce_workspace(*din, rank_out, sizes_out);
  if (!workspace) {
    *workspace_bytes = need;
    return ZK_OK;
  }
  if (*workspace_bytes < need || !ws_aligned(workspace, need)) return ZK_ERR_WORKSPACE;
  int64_t nout = 1;
  for (int k = 0; k < rank_out; ++k) nout *= sizes_out[k];
  if (p.c.numel > 0 && !in) return ZK_ERR_NULL;
  if (nout > 0 && !out) return ZK_ERR_NULL;
  Ext ei = ext_of(in, *din), eo = ext_dense(out, nout);
  Ext ews;
  if (need) ews = Ext{(uintptr_t)workspace, (uintptr_t)workspace + need};
  if (ov(eo, ei) || ov(eo, ews) || ov(ews, ei)) return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {p.c.numel > 0 ? in : nullptr, nout > 0 ? out : nullptr,
                                need ? workspace : nullptr})))
    return s;
  const double count =
      mean ? (double)reduced_count(din->rank, din->sizes, rank_out, sizes_out) : -1.0;
  return hip_status(launch_reduce(p, in, out, workspace, (hipStream_t)stream, nullptr, false,
                                  count));
}

// Tensor list of zk_grad_norm / zk_clip_grad_norm: sizes non-negative;
// with `ptrs`, pointers present for non-empty tensors and no two tensors
// overlapping.
zk_status check_grad_list(int32_t count, const void *const *grads, const int64_t *numels,
                          bool ptrs) {
  if (count < 0) return ZK_ERR_BAD_SIZE;
  if (count > 0 && !numels) return ZK_ERR_NULL;
  int64_t total = 0;
  for (int t = 0; t < count; ++t) {
    if (numels[t] < 0 || numels[t] > kMaxExtent) return ZK_ERR_BAD_SIZE;
    if (__builtin_add_overflow(total, numels[t], &total) || total > kMaxExtent)
      return ZK_ERR_BAD_SIZE;
  }
  if (!ptrs) return ZK_OK;
  if (count > 0 && !grads) return ZK_ERR_NULL;
  std::vector<std::pair<uintptr_t, uintptr_t>> ext;
  ext.reserve(count);
  for (int t = 0; t < count; ++t) {
    if (numels[t] == 0) continue;
    if (!grads[t]) return ZK_ERR_NULL;
    Ext e = ext_dense(grads[t], numels[t]);
    ext.emplace_back(e.lo, e.hi);
  }
  std::sort(ext.begin(), ext.end());
  for (size_t k = 1; k < ext.size(); ++k)
    if (ext[k].first < ext[k - 1].second) return ZK_ERR_ALIAS;
  return ZK_OK;
}

zk_status norm_common(int32_t count, float *const *grads, const int64_t *numels, bool clip,
                      float max_norm, float *norm_out, void *workspace,
                      size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes) return ZK_ERR_NULL;
  zk_status s;
  if ((s = check_grad_list(count, (const void *const *)grads, numels, workspace != nullptr)))
    return s;
  if (clip && !(max_norm >= 0.0f)) return ZK_ERR_UNSUPPORTED;  // NaN or negative
  const size_t need = norm_workspace(count, numels);
  if (!workspace) {
    *workspace_bytes = need;
    return ZK_OK;
  }
  if (*workspace_bytes < need || !ws_aligned(workspace, need)) return ZK_ERR_WORKSPACE;
  if (!norm_out) return ZK_ERR_NULL;
  const Ext ew{(uintptr_t)workspace, (uintptr_t)workspace + need};
  const Ext en = ext_dense(norm_out, 1);
  if (ov(ew, en)) return ZK_ERR_ALIAS;
  for (int t = 0; t < count; ++t) {
    if (numels[t] == 0) continue;
    const Ext e = ext_dense(grads[t], numels[t]);
    if (ov(e, ew) || ov(e, en)) return ZK_ERR_ALIAS;
  }
  if (debug_mode() == 1) {
    std::vector<const void *> ptrs{norm_out, need ? workspace : nullptr};
    for (int t = 0; t < count; ++t)
      if (numels[t] > 0) ptrs.push_back(grads[t]);
    if ((s = debug_check_list(stream, ptrs.data(), ptrs.size()))) return s;
  }
  return hip_status(launch_grad_norm(count, grads, numels, norm_out, workspace, clip,
                                     (double)max_norm, (hipStream_t)stream));
}
}  // namespace

extern "C" {

zk_status zk_reduce_to_shape(const float *in, const zk_desc *din,
                             int32_t rank_out, const int64_t *sizes_out,
                             float *out, void *workspace,
                             size_t *workspace_bytes, void *stream) {
  return reduce_common(in, din, rank_out, sizes_out, out, workspace, workspace_bytes, stream,
                       false);
}

zk_status zk_mean_to_shape(const float *in, const zk_desc *din, int32_t rank_out,
                           const int64_t *sizes_out, float *out, void *workspace,
                           size_t *workspace_bytes, void *stream) {
  return reduce_common(in, din, rank_out, sizes_out, out, workspace, workspace_bytes, stream,
                       true);
}

zk_status zk_mean_bwd(const float *grad, int32_t rank_out, const int64_t *sizes_out,
                      int32_t rank_in, const int64_t *sizes_in, float *grad_in,
                      void *stream) {
  if (rank_out < 0 || rank_out > kMaxDims || rank_in < 0 || rank_in > kMaxDims)
    return ZK_ERR_RANK;
  if ((rank_out > 0 && !sizes_out) || (rank_in > 0 && !sizes_in)) return ZK_ERR_NULL;
  for (int k = 0; k < rank_out; ++k)
    if (sizes_out[k] < 0) return ZK_ERR_BAD_SIZE;
  for (int k = 0; k < rank_in; ++k)
    if (sizes_in[k] < 0) return ZK_ERR_BAD_SIZE;
  int r;
  int64_t n[kMaxDims];
  zk_status s = broadcast_shape(rank_in, sizes_in, rank_out, sizes_out, &r, n);
  if (s == ZK_ERR_BROADCAST) return ZK_ERR_SHAPE;
  if (s) return s;
  if (r != rank_in) return ZK_ERR_SHAPE;
  for (int k = 0; k < r; ++k)
    if (n[k] != sizes_in[k]) return ZK_ERR_SHAPE;
  // grad read as a view of the input's shape: stride 0 on the reduced dims
  const zk_desc dout = dense_desc(rank_out, sizes_out);
  zk_desc dg{};
  dg.rank = rank_in;
  for (int k = 0; k < rank_in; ++k) {
    const int ko = k - (rank_in - rank_out);
    dg.sizes[k] = sizes_in[k];
    dg.strides[k] = (ko < 0 || sizes_out[ko] == 1) ? 0 : dout.strides[ko];
  }
  const int64_t nin = numel(dg);
  if (nin == 0) return ZK_OK;
  if (!grad || !grad_in) return ZK_ERR_NULL;
  if (ov(ext_dense(grad_in, nin), ext_dense(grad, numel(dout)))) return ZK_ERR_ALIAS;
  const float c32 = (float)reduced_count(rank_in, sizes_in, rank_out, sizes_out);
  return zk_scalar_fwd(ZK_DIV, ZK_EPI_NONE, grad, &dg, c32, 0, grad_in, stream);
}

zk_status zk_grad_norm(int32_t count, const float *const *grads, const int64_t *numels,
                       float *norm_out, void *workspace, size_t *workspace_bytes,
                       void *stream) {
  return norm_common(count, const_cast<float *const *>(grads), numels, false, 0.0f, norm_out,
                     workspace, workspace_bytes, stream);
}

zk_status zk_clip_grad_norm(int32_t count, float *const *grads, const int64_t *numels,
                            float max_norm, float *norm_out, void *workspace,
                            size_t *workspace_bytes, void *stream) {
  return norm_common(count, grads, numels, true, max_norm, norm_out, workspace,
                     workspace_bytes, stream);
}

namespace {
zk_status row_stats_common(int mode, const float *x, int64_t rows, int64_t cols, int64_t ld,
                           float *o1, float *o2, void *stream) {
  if (rows < 0 || cols < 0 || rows > kMaxExtent || cols > kMaxExtent) return ZK_ERR_BAD_SIZE;
  if (ld < cols || (rows > 1 && ld < 1)) return ZK_ERR_BAD_STRIDE;
  if (rows == 0) return ZK_OK;
  int64_t last = 0;  // one past the last element read
  if (cols > 0 && (__builtin_mul_overflow(rows - 1, ld, &last) ||
                   __builtin_add_overflow(last, cols, &last) || last > kMaxExtent))
    return ZK_ERR_BAD_STRIDE;
  if (!o1 || !o2) return ZK_ERR_NULL;
  if (cols > 0 && !x) return ZK_ERR_NULL;
  const Ext e1 = ext_dense(o1, rows), e2 = ext_dense(o2, rows);
  Ext ex;
  if (cols > 0) ex = ext_dense(x, (rows - 1) * ld + cols);
  if (ov(e1, e2) || ov(e1, ex) || ov(e2, ex)) return ZK_ERR_ALIAS;
  if (zk_status s = debug_check(stream, {cols > 0 ? x : nullptr, o1, o2})) return s;
  return hip_status(launch_row_stats(mode, x, rows, cols, ld, o1, o2, (hipStream_t)stream));
}
}  // namespace

zk_status zk_row_moments(const float *x, int64_t rows, int64_t cols, int64_t ld, float *mean,
                         float *var, void *stream) {
  return row_stats_common(0, x, rows, cols, ld, mean, var, stream);
}

zk_status zk_row_softmax_stats(const float *x, int64_t rows, int64_t cols, int64_t ld,
                               float *rowmax, float *sumexp, void *stream) {
  return row_stats_common(1, x, rows, cols, ld, rowmax, sumexp, stream);
}

zk_status zk_scalar_fwd(zk_op op, zk_epi epi, const float *t, const zk_desc *dt,
                        float sv, int32_t scalar_first, float *out, void *stream) {
  if (!valid_op(op) || !valid_epi(epi)) return ZK_ERR_UNSUPPORTED;
  zk_status s;
  if ((s = check_desc(dt))) return s;
  const zk_desc d0{};  // the scalar as a rank-0 operand
  const bool sf = scalar_first != 0;
  const zk_desc &da = sf ? d0 : *dt, &db = sf ? *dt : d0;
  const float *pa = sf ? nullptr : t, *pb = sf ? t : nullptr;
  FwdPlan p;
  if ((s = plan_fwd(op, epi, da, db, (uintptr_t)pa, (uintptr_t)pb, (uintptr_t)out, &p)))
    return s;
  if (p.empty) return ZK_OK;
  if (!t || !out) return ZK_ERR_NULL;
  if (p.kernel == K_FWD_ROW) {
    p.small_mode = SM_ARG;  // the tensor is the dense operand
  } else if (p.kernel != K_FWD_GENERIC) {
    p.kernel = K_FWD_GENERIC;
    p.vec = ((uintptr_t)out & 15u) == 0 ? 4 : 1;
  }
  const int64_t n = p.c.numel;
  if (ov(ext_dense(out, n), ext_of(t, *dt)) && !(out == t && dense_full(*dt, n)))
    return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {t, out}))) return s;
  const ScalarArg sa{sf ? 0 : 1, sv};
  return hip_status(launch_fwd(p, op, epi, pa, pb, out, (hipStream_t)stream, &sa));
}

zk_status zk_scalar_bwd(zk_op op, zk_epi epi, const float *grad, const float *t,
                        const zk_desc *dt, float sv, int32_t scalar_first,
                        float *grad_t, const float *acc_t, void *stream) {
  if (!valid_op(op) || !valid_epi(epi)) return ZK_ERR_UNSUPPORTED;
  zk_status s;
  if ((s = check_desc(dt))) return s;
  const zk_desc d0{};
  const bool sf = scalar_first != 0;
  const zk_desc &da = sf ? d0 : *dt, &db = sf ? *dt : d0;
  const float *pa = sf ? nullptr : t, *pb = sf ? t : nullptr;
  float *ga = sf ? nullptr : grad_t, *gb = sf ? grad_t : nullptr;
  const float *xa = sf ? nullptr : acc_t, *xb = sf ? acc_t : nullptr;
  BwdPlan p;
  if ((s = plan_bwd(op, epi, da, db, !sf && grad_t, sf && grad_t, (uintptr_t)grad,
                    (uintptr_t)pa, (uintptr_t)pb, (uintptr_t)ga, (uintptr_t)gb,
                    (uintptr_t)xa, (uintptr_t)xb, &p)))
    return s;
  const int64_t n = p.c.numel;
  if (!grad_t || n == 0) return ZK_OK;
  if (!grad || !t) return ZK_ERR_NULL;
  // The tensor has the full shape: one element-wise pass.  The scalar needs
  // no layout, so the flat kernel applies whenever the tensor is dense.
  if (canon_is_flat(p.c, sf ? 2 : 1)) {
    p.ew_kernel = K_BWD_EW_FLAT;
    auto al = [](const void *q) { return ((uintptr_t)q & 15u) == 0; };
    p.vec = al(grad) && al(t) && al(grad_t) && al(acc_t) ? 4 : 1;
  }
  Ext eg = ext_dense(grad, n), et = ext_of(t, *dt), eo = ext_dense(grad_t, n);
  Ext ex = ext_dense(acc_t, n);
  if (ov(eo, eg) || ov(eo, et)) return ZK_ERR_ALIAS;
  if (ov(eo, ex) && acc_t != grad_t) return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {grad, t, grad_t, acc_t}))) return s;
  const ScalarArg sa{sf ? 0 : 1, sv};
  return hip_status(launch_bwd(p, op, epi, grad, pa, pb, ga, xa, gb, xb, nullptr,
                               (hipStream_t)stream, nullptr, nullptr, 1.f, &sa));
}

zk_status zk_unary_fwd(zk_epi f, const float *x, const zk_desc *dx, float *out,
                       void *stream) {
  if (f != ZK_EPI_GELU && f != ZK_EPI_RELU) return ZK_ERR_UNSUPPORTED;
  return zk_scalar_fwd(ZK_SUB, f, x, dx, 0.0f, 0, out, stream);  // x - 0 == x
}

zk_status zk_unary_bwd(zk_epi f, const float *grad, const float *x, const zk_desc *dx,
                       float *grad_x, const float *acc_x, void *stream) {
  if (f != ZK_EPI_GELU && f != ZK_EPI_RELU) return ZK_ERR_UNSUPPORTED;
  return zk_scalar_bwd(ZK_SUB, f, grad, x, dx, 0.0f, 0, grad_x, acc_x, stream);
}

zk_status zk_materialize(const float *in, const zk_desc *din, int32_t rank_out,
                         const int64_t *sizes_out, float *out, void *stream) {
  zk_status s;
  if ((s = check_desc(din))) return s;
  if (rank_out < 0 || rank_out > kMaxDims) return ZK_ERR_RANK;
  if (rank_out > 0 && !sizes_out) return ZK_ERR_NULL;
  for (int k = 0; k < rank_out; ++k)
    if (sizes_out[k] < 0) return ZK_ERR_BAD_SIZE;
  CopyPlan p;
  if ((s = plan_copy(*din, rank_out, sizes_out, (uintptr_t)in, (uintptr_t)out, &p))) return s;
  if (p.empty) return ZK_OK;
  if (!in || !out) return ZK_ERR_NULL;
  if (ov(ext_dense(out, p.c.numel), ext_of(in, *din))) return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {in, out}))) return s;
  return hip_status(launch_copy(p, in, out, (hipStream_t)stream));
}

zk_status zk_binary2_fwd(zk_op op1, zk_op op2, const float *a, const zk_desc *da,
                         const float *b, const zk_desc *db, const float *c,
                         const zk_desc *dc, float *out, void *stream) {
  if (!valid_op(op1) || !valid_op2(op2)) return ZK_ERR_UNSUPPORTED;
  zk_status s;
  if ((s = check_desc(da)) || (s = check_desc(db)) || (s = check_desc(dc))) return s;
  Fwd2Plan p;
  if ((s = plan_fwd2(*da, *db, *dc, (uintptr_t)a, (uintptr_t)b, (uintptr_t)c,
                     (uintptr_t)out, &p)))
    return s;
  if (p.empty) return ZK_OK;
  if (!a || !b || !c || !out) return ZK_ERR_NULL;
  const int64_t n = p.c.numel;
  Ext eo = ext_dense(out, n);
  const float *in[3] = {a, b, c};
  const zk_desc *din[3] = {da, db, dc};
  for (int x = 0; x < 3; ++x)
    if (ov(eo, ext_of(in[x], *din[x])) && !(out == in[x] && dense_full(*din[x], n)))
      return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {a, b, c, out}))) return s;
  return hip_status(launch_fwd2(p, op1, op2, a, b, c, out, (hipStream_t)stream));
}

zk_status zk_binary2_bwd(zk_op op1, zk_op op2, const float *grad, const float *a,
                         const zk_desc *da, const float *b, const zk_desc *db,
                         const float *c, const zk_desc *dc, float *grad_a,
                         const float *acc_a, float *grad_b, const float *acc_b,
                         float *grad_c, const float *acc_c, void *workspace,
                         size_t *workspace_bytes, void *stream) {
  if (!valid_op(op1) || !valid_op2(op2)) return ZK_ERR_UNSUPPORTED;
  if (!workspace_bytes) return ZK_ERR_NULL;
  zk_status s;
  if ((s = check_desc(da)) || (s = check_desc(db)) || (s = check_desc(dc))) return s;
  int r, rab;
  int64_t n[kMaxDims], nab[kMaxDims];
  if ((s = broadcast_shape3(*da, *db, *dc, &r, n))) return s;
  if ((s = broadcast_shape(da->rank, da->sizes, db->rank, db->sizes, &rab, nab))) return s;
  const zk_desc ds = dense_desc(r, n), dab = dense_desc(rab, nab);
  const int64_t ns = numel(ds), nt = numel(dab);
  const int64_t na = numel(*da), nb = numel(*db), nc = numel(*dc);
  // A tensor used twice: c is a (or b) and one buffer takes both paths.
  int tie = -1;
  if (grad_c && grad_c == grad_a) tie = 0;
  else if (grad_c && grad_c == grad_b) tie = 1;
  if (tie >= 0) {
    const zk_desc &dt = tie == 0 ? *da : *db;
    const float *pt = tie == 0 ? a : b;
    const float *acct = tie == 0 ? acc_a : acc_b;
    if (op2 != ZK_ADD || c != pt || !same_view(*dc, dt) || numel(dt) != ns || acct || acc_c)
      return ZK_ERR_UNSUPPORTED;
  }
  const bool wa = grad_a != nullptr, wb = grad_b != nullptr;
  const bool wc = grad_c != nullptr && tie < 0;
  const bool split = nt < ns;  // t = a op1 b is repeated into out
  const Bwd2Layout L = bwd2_layout(op1, *da, *db, *dc, r, n, wa, wb, wc);
  const size_t need = L.total();
  if (!workspace) {
    *workspace_bytes = need;
    return ZK_OK;
  }
  if (*workspace_bytes < need || !ws_aligned(workspace, need)) return ZK_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
  float *tbuf = split && (wa || wb) ? reinterpret_cast<float *>(ws + L.op1 + L.cred) : nullptr;
  const float *up = tbuf ? tbuf : grad;  // upstream gradient of t
  const float *acc_a1 = tie == 0 ? up : acc_a;
  const float *acc_b1 = tie == 1 ? up : acc_b;
  BwdPlan p1, pc, pt;
  if ((wa || wb) &&
      (s = plan_bwd(op1, ZK_EPI_NONE, *da, *db, wa, wb, (uintptr_t)up, (uintptr_t)a,
                    (uintptr_t)b, (uintptr_t)grad_a, (uintptr_t)grad_b,
                    (uintptr_t)acc_a1, (uintptr_t)acc_b1, &p1)))
    return s;
  if (wc && nc < ns &&
      (s = plan_reduce(ds, dc->rank, dc->sizes, (uintptr_t)grad, (uintptr_t)grad_c, &pc)))
    return s;
  if (tbuf && (s = plan_reduce(ds, rab, nab, (uintptr_t)grad, (uintptr_t)tbuf, &pt)))
    return s;
  if (ns > 0 && (!grad || !a || !b || !c)) return ZK_ERR_NULL;
  // Aliasing: outputs against each other, the inputs, the accs and the
  // workspace (an output may be its own acc; a tied pair is one output).
  Ext eg = ext_dense(grad, ns), ea = ext_of(a, *da), eb = ext_of(b, *db), ec = ext_of(c, *dc);
  Ext ews;
  if (need) ews = Ext{(uintptr_t)workspace, (uintptr_t)workspace + need};
  float *outs[3] = {grad_a, grad_b, tie < 0 ? grad_c : nullptr};
  const float *accs[3] = {acc_a, acc_b, acc_c};
  const int64_t cnt[3] = {na, nb, nc};
  Ext eo[3], ex[3];
  for (int w = 0; w < 3; ++w) {
    eo[w] = ext_dense(outs[w], cnt[w]);
    ex[w] = ext_dense(accs[w], cnt[w]);
  }
  for (int w = 0; w < 3; ++w) {
    if (!outs[w]) continue;
    if (ov(eo[w], eg) || ov(eo[w], ea) || ov(eo[w], eb) || ov(eo[w], ec) || ov(eo[w], ews))
      return ZK_ERR_ALIAS;
    for (int v = 0; v < 3; ++v) {
      if (v != w && outs[v] && ov(eo[w], eo[v])) return ZK_ERR_ALIAS;
      if (ov(eo[w], ex[v]) && !(v == w && accs[v] == outs[w])) return ZK_ERR_ALIAS;
    }
  }
  if (need)
    for (int w = 0; w < 3; ++w)
      if (ov(ews, eg) || ov(ews, ea) || ov(ews, eb) || ov(ews, ec) || ov(ews, ex[w]))
        return ZK_ERR_ALIAS;
  if ((s = debug_check(stream, {grad, a, b, c, grad_a, acc_a, grad_b, acc_b, grad_c, acc_c,
                                need ? workspace : nullptr})))
    return s;
  const hipStream_t st = (hipStream_t)stream;
  const float sign = op2 == ZK_SUB ? -1.f : 1.f;
  hipError_t e = hipSuccess;
  if (ns == 0) {
    // Sums over nothing: each requested gradient is its acc, or zeros.
    const zk_desc *dw[3] = {da, db, dc};
    float *gw[3] = {grad_a, grad_b, wc ? grad_c : nullptr};
    const float *aw[3] = {acc_a, acc_b, acc_c};
    for (int w = 0; w < 3; ++w) {
      if (!gw[w] || cnt[w] == 0) continue;
      BwdPlan pz;
      if ((s = plan_reduce(ds, dw[w]->rank, dw[w]->sizes, 0, 0, &pz))) return s;
      e = launch_reduce(pz, grad, gw[w], ws, st, aw[w]);
      if (e != hipSuccess) return ZK_ERR_HIP;
    }
    return ZK_OK;
  }
  if (tbuf) {
    e = launch_reduce(pt, grad, tbuf, ws + L.op1 + L.cred + L.tbuf, st);
    if (e != hipSuccess) return ZK_ERR_HIP;
  }
  // c's gradient rides with the op1 backward when both walk the full layout
  const bool gc_in_op1 = wc && nc == ns && !split && (wa || wb);
  if (wa || wb) {
    e = launch_bwd(p1, op1, ZK_EPI_NONE, up, a, b, grad_a, acc_a1, grad_b, acc_b1, ws, st,
                   gc_in_op1 ? grad_c : nullptr, acc_c, sign);
    if (e != hipSuccess) return ZK_ERR_HIP;
  }
  if (wc && !gc_in_op1) {
    if (nc == ns) e = launch_signed(grad, ns, grad_c, acc_c, sign, st);
    else e = launch_reduce(pc, grad, grad_c, ws + L.op1, st, acc_c, op2 == ZK_SUB);
    if (e != hipSuccess) return ZK_ERR_HIP;
  }
  return ZK_OK;
}

zk_status zk_plan_describe(int32_t kind, zk_op op, zk_epi epi, const zk_desc *da,
                           const zk_desc *db, zk_plan_info *info) {
  if (!info) return ZK_ERR_NULL;
  if (!valid_op(op) || !valid_epi(epi)) return ZK_ERR_UNSUPPORTED;
  zk_status s;
  if ((s = check_desc(da)) || (s = check_desc(db))) return s;
  std::memset(info, 0, sizeof(*info));
  info->kernel2 = K_NONE;
  const Canon *c = nullptr;
  if (kind == 0) {
    static thread_local FwdPlan p;
    p = FwdPlan();
    if ((s = plan_fwd(op, epi, *da, *db, 0, 0, 0, &p))) return s;
    info->kernel = p.kernel;
    info->index64 = p.idx64;
    info->vec = p.vec;
    c = &p.c;
    info->rank = c->rank;
    for (int k = 0; k < c->rank; ++k) {
      info->sizes[k] = c->n[k];
      for (int o = 0; o < 3; ++o) info->strides[o][k] = c->s[o][k];
    }
    return ZK_OK;
  }
  static thread_local BwdPlan p;
  p = BwdPlan();
  if (kind == 1) {
    if ((s = plan_bwd(op, epi, *da, *db, true, true, 0, 0, 0, 0, 0, 0, 0, &p))) return s;
  } else if (kind == 2) {
    if ((s = plan_reduce(*da, db->rank, db->sizes, 0, 0, &p))) return s;
  } else {
    return ZK_ERR_UNSUPPORTED;
  }
  c = &p.c;
  info->kernel = p.ew_kernel;
  if (p.nred > 0) {
    if (info->kernel == K_NONE) info->kernel = p.red[0].kernel;
    else info->kernel2 = p.red[0].kernel;
    info->partials = p.red[0].partials;
  }
  if (p.nred > 1) info->kernel2 = p.red[1].kernel;
  info->index64 = p.idx64;
  info->vec = p.vec;
  info->workspace_bytes = kind == 1 ? bwd_workspace(op, epi, *da, *db, true, true)
                                    : reduce_workspace(*da, db->rank, db->sizes);
  info->rank = c->rank;
  for (int k = 0; k < c->rank; ++k) {
    info->sizes[k] = c->n[k];
    if (kind == 1) {
      for (int o = 0; o < 3; ++o) info->strides[o][k] = c->s[o][k];
    } else {  // [0] dense input layout, [1] input strides, [2] target
      info->strides[0][k] = c->s[1][k];
      info->strides[1][k] = c->s[0][k];
      info->strides[2][k] = c->s[4][k];
    }
  }
  return ZK_OK;
}

}  // extern "C"
