// Batched single-token decode step of the Simple GLA mixer for gfx950.
//
// For each sequence and head: S <- e^{g} S + k^T v in place on the float32
// state pool, then o = q S.  The per-sequence state has a fixed size that does
// not grow with the context ("AWS serve Laplace 3B di i14 con uno stato fisso
// di 29,5 MB", section "Lo stato di Laplace 3B resta fisso durante
// l'inferenza"), so the step is one read and one write of the state: a purely
// HBM-bound kernel (0.62 flop per byte).
//
// One workgroup of 192 threads handles one (sequence, head): thread t owns
// columns 4*(t%48)..+3 of rows 24*(t/48)..+23, loads all 24 rows before any
// arithmetic (24 x 16 bytes in flight per lane), updates them, writes them
// back, and the four row groups reduce o through LDS.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

template <class TIn, class TOut>
__global__ void __launch_bounds__(192) step_kernel(StepArgs a) {
  constexpr int ROWS = DK / 4;  // rows per thread
  __shared__ float sk[DK];
  __shared__ float sq[DK];
  __shared__ f32x4 red[4][48];
  const int64_t item = blockIdx.x;
  const int64_t b = item / a.H;
  const int h = (int)(item % a.H);
  const int64_t slot = a.slot_idx ? (int64_t)a.slot_idx[b] : b;
  float* S = a.pool + (slot * a.H + h) * (int64_t)(DK * DV);
  const int t = threadIdx.x;
  const int c4 = t % 48, rg = t / 48;

  f32x4 s[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
    s[r] = __builtin_nontemporal_load((const f32x4*)(S + (rg * ROWS + r) * DV) + c4);

  const TIn* qp = (const TIn*)a.q + item * DK;
  const TIn* kp = (const TIn*)a.k + item * DK;
  if (t < DK) sk[t] = (float)kp[t];
  else sq[t - DK] = (float)qp[t - DK];
  const f32x4 v = load4f((const TIn*)a.v + item * DV + 4 * c4);
  const float gam = exp2f(fmaxf(a.g[item], G_MIN) * LOG2E);
  __syncthreads();

  f32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int d = rg * ROWS + r;
    s[r] = gam * s[r] + sk[d] * v;
    acc += sq[d] * s[r];
    __builtin_nontemporal_store(s[r], (f32x4*)(S + d * DV) + c4);
  }
  red[rg][c4] = acc;
  __syncthreads();
  if (rg == 0) {
    const f32x4 o = red[0][c4] + red[1][c4] + red[2][c4] + red[3][c4];
    store4((TOut*)a.o + item * DV + 4 * c4, o);
  }
}

hipError_t launch_step(const StepArgs& a, int in_bf16, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H)), block(192);
  if (in_bf16) {
    if (out_bf16) hipLaunchKernelGGL((step_kernel<bf16, bf16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((step_kernel<bf16, float>), grid, block, 0, st, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((step_kernel<float, bf16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((step_kernel<float, float>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace gla
