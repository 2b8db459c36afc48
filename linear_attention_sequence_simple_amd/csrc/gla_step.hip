// Batched single-token decode step of the Simple GLA mixer for gfx950.
//
// For each sequence and head: S <- e^{g} S + k^T v in place on the float32
// state pool, then o = q S.  The per-sequence state has a fixed size that does
// not grow with the context ("AWS serve Laplace 3B di i14 con uno stato fisso
// di 29,5 MB", section "Lo stato di Laplace 3B resta fisso durante
// l'inferenza"), so the step is one read and one write of the state: a purely
// HBM-bound kernel (0.62 flop per byte).
//
// One workgroup of 384 threads handles one (sequence, head): thread t owns
// columns 4*(t%48)..+3 of rows 12*(t/48)..+11, loads all 12 rows before any
// arithmetic (12 x 16 bytes in flight per lane), updates them, writes them
// back, and the eight row groups reduce o through LDS.  192 threads of 24
// rows each ran 1% slower (543 against 538 us per layer-step of 1,280 x 16
// slots) and 768 threads of 6 rows 0.3% slower: the smaller per-thread share
// lets more waves stay resident.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

template <class TIn, class TOut>
__global__ void __launch_bounds__(384) step_kernel(StepArgs a) {
  constexpr int RG = 8, ROWS = DK / RG;  // rows per thread
  __shared__ float sk[DK];
  __shared__ float sq[DK];
  __shared__ f32x4 red[RG][48];
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
  else if (t < 2 * DK) sq[t - DK] = (float)qp[t - DK];
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
    f32x4 o = red[0][c4];
#pragma unroll
    for (int i = 1; i < RG; ++i) o += red[i][c4];
    store4((TOut*)a.o + item * DV + 4 * c4, o);
  }
}

hipError_t launch_step(const StepArgs& a, int in_bf16, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H)), block(384);
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
