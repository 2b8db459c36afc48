// Checks of the caller contracts that only the device can see, run before a
// call's kernels when the environment sets GLA_DEBUG (a non-empty value other
// than 0): slot indices in range and distinct, log-decays not positive and
// not NaN, packed-sequence offsets in order and within their bounds.  Each
// check sets bits of one flag word; the host reads it back after the checks
// and fails the call before its kernels run.  Off the hot path: the checks
// synchronise the stream, so a call under GLA_DEBUG cannot be captured in a
// graph.
#include "gla_common.h"
#include "gla_debug.h"

namespace gla {

__global__ void debug_zero_kernel(int* flag) {
  if (threadIdx.x == 0) *flag = 0;
}

// Slot i: in [0, n_slots) and different from every earlier slot.
__global__ void __launch_bounds__(256) debug_slots_kernel(const int32_t* idx, int64_t n, int64_t n_slots,
                                                          int* flag) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t v = idx[i];
  if (v < 0 || v >= n_slots) atomicOr(flag, DBG_SLOT_RANGE);
  for (int64_t j = 0; j < i; ++j)
    if (idx[j] == v) {
      atomicOr(flag, DBG_SLOT_DUP);
      break;
    }
}

// g[b, t, h] <= 0 (not positive, not NaN) over a strided [B, T, H] view.
__global__ void __launch_bounds__(256) debug_decay_kernel(const float* g, int64_t B, int64_t T, int64_t H,
                                                          int64_t sb, int64_t st, int64_t sh, int* flag) {
  const int64_t n = B * T * H;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t h = i % H, bt = i / H, t = bt % T, b = bt / T;
    if (!(g[b * sb + t * st + h * sh] <= 0.f)) {
      atomicOr(flag, DBG_DECAY);
      return;
    }
  }
}

// Sequence i of a packed batch: 0 <= cu[i] <= cu[i+1] <= total and
// cu[i+1] - cu[i] <= max_len.
__global__ void __launch_bounds__(256) debug_offsets_kernel(const int32_t* cu, int64_t n, int64_t total,
                                                            int64_t max_len, int* flag) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t a = cu[i], b = cu[i + 1];
  if (a < 0 || b < a || b > total || b - a > max_len) atomicOr(flag, DBG_OFFSETS);
}

static unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t debug_zero(int* flag, hipStream_t st) {
  hipLaunchKernelGGL(debug_zero_kernel, dim3(1), dim3(64), 0, st, flag);
  return hipGetLastError();
}

hipError_t debug_slots(const int32_t* idx, int64_t n, int64_t n_slots, int* flag, hipStream_t st) {
  if (n <= 0 || !idx) return hipSuccess;
  hipLaunchKernelGGL(debug_slots_kernel, dim3(blocks(n)), dim3(256), 0, st, idx, n, n_slots, flag);
  return hipGetLastError();
}

hipError_t debug_decay(const float* g, int64_t B, int64_t T, int64_t H, int64_t sb, int64_t st_, int64_t sh,
                       int* flag, hipStream_t st) {
  const int64_t n = B * T * H;
  if (n <= 0) return hipSuccess;
  const unsigned grid = blocks(n) < 4096u ? blocks(n) : 4096u;
  hipLaunchKernelGGL(debug_decay_kernel, dim3(grid), dim3(256), 0, st, g, B, T, H, sb, st_, sh, flag);
  return hipGetLastError();
}

hipError_t debug_offsets(const int32_t* cu, int64_t n, int64_t total, int64_t max_len, int* flag, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(debug_offsets_kernel, dim3(blocks(n)), dim3(256), 0, st, cu, n, total, max_len, flag);
  return hipGetLastError();
}

}  // namespace gla
