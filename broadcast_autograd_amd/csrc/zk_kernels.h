// zk_kernels.h -- kernel argument blocks (passed by value, like the book's
// fixed 8-dim DimsArg in the GPU chapter, "kernel dispatch") and the host
// launchers implemented in the .hip files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zk.h"
#include "zk_plan.h"

namespace zk {

// Canonical iteration space handed to a kernel.
struct Space {
  int32_t rank;
  int64_t n[kMaxDims];
  int64_t s[kMaxOps][kMaxDims];
  FastDiv fd[kMaxDims];  // divisors n[k] (used when 32-bit indexing)
  int64_t numel;
};

// A reduction's split of the canonical dims into kept (K) and reduced (R)
// dims for the gather kernel; dims listed outer -> inner.
struct RedDims {
  int32_t nk, nr;
  int32_t kdim[kMaxDims], rdim[kMaxDims];
  FastDiv kfd[kMaxDims], rfd[kMaxDims];
};

Space make_space(const Canon &c);

// A host scalar operand passed by value: side 0 = operand a, 1 = operand b.
struct ScalarArg {
  int32_t side;
  float value;
};

// Reserves a HIP event pair for the one kernel launched in its scope while
// zk_profile_start() is in effect (slot < 0 otherwise).  ZK_LAUNCH hands the
// pair to hipExtLaunchKernel, so the events carry the kernel's own begin and
// end timestamps from its dispatch packet, not those of separate markers.
struct ProfScope {
  explicit ProfScope(int32_t kernel);
  int slot;
  hipEvent_t ev_start, ev_end;
};

#define ZK_LAUNCH(ps, kernel, grid, block, shmem, st, ...)                    \
  do {                                                                     \
    if ((ps).slot >= 0)                                                    \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, (ps).ev_start,   \
                            (ps).ev_end, 0, __VA_ARGS__);                  \
    else                                                                   \
      hipLaunchKernelGGL(kernel, grid, block, shmem, st, __VA_ARGS__);      \
  } while (0)

// sa (optional): one operand is a host scalar; its pointer is unused.
hipError_t launch_fwd(const FwdPlan &p, zk_op op, zk_epi epi, const float *a,
                      const float *b, float *out, hipStream_t st,
                      const ScalarArg *sa = nullptr);

hipError_t launch_copy(const CopyPlan &p, const float *in, float *out, hipStream_t st);

hipError_t launch_fwd2(const Fwd2Plan &p, zk_op op1, zk_op op2, const float *a,
                       const float *b, const float *c, float *out, hipStream_t st);

// grad_c (optional): also write c_sign * g (+ acc_c) over the dense output
// layout, the gradient of a fused expression's second operand c.
hipError_t launch_bwd(const BwdPlan &p, zk_op op, zk_epi epi, const float *g,
                      const float *a, const float *b, float *grad_a,
                      const float *acc_a, float *grad_b, const float *acc_b,
                      void *ws, hipStream_t st, float *grad_c = nullptr,
                      const float *acc_c = nullptr, float c_sign = 1.f,
                      const ScalarArg *sa = nullptr);

// gc[i] = sign * g[i] (+ acc[i]) for i < n.
hipError_t launch_signed(const float *g, int64_t n, float *gc, const float *acc,
                         float sign, hipStream_t st);

// acc (optional) is added to each sum; neg negates the sum first; a
// mean_count >= 0 divides each sum by it in binary64 (the mean).
hipError_t launch_reduce(const BwdPlan &p, const float *in, float *out,
                         void *ws, hipStream_t st, const float *acc = nullptr,
                         bool neg = false, double mean_count = -1.0);

// ---- global L2 norm / ClipGradNorm (zk_norm.hip)
constexpr int kNormTab = 128;  // tensors per launch, passed in the kernel arguments
// Up to kNormTab non-empty dense tensors and the first block of each
// (2.5 KB of kernel arguments).
struct NormTab {
  float *p[kNormTab];
  int64_t n[kNormTab];
  uint32_t b0[kNormTab + 1];  // b0[nt] = blocks of this launch
  int32_t nt;
  int64_t part0;  // index of this launch's first partial
};
// Workspace: one binary64 partial per block of the tensor list.
struct NormFinArgs {
  int64_t P;  // partials
  double max_norm;
};
// Most blocks one launch of a table may hold (b0 is 32-bit).
constexpr int64_t kNormMaxTableBlocks = (int64_t)1 << 30;
size_t norm_workspace(int count, const int64_t *numels);
// norm_out: device float.  clip: also scale every tensor in place when the
// norm exceeds max_norm.
hipError_t launch_grad_norm(int count, float *const *g, const int64_t *numels, float *norm_out,
                            void *ws, bool clip, double max_norm, hipStream_t st);

// ---- the library-owned scratch array (zk_scratch.hip): the device address of
// the current device's copy, looked up on its first use.
hipError_t scratch_on_current_device(void **ptr);

// ---- per-row statistics (zk_rows.hip): mode 0 mean / variance, mode 1
// row max / sum of exponentials; rows of `cols` elements at a pitch of ld.
hipError_t launch_row_stats(int mode, const float *x, int64_t rows, int64_t cols, int64_t ld,
                            float *o1, float *o2, hipStream_t st);

}  // namespace zk
