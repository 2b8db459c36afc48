// 16-bit decode state for gfx950.
//
// The HEAL summary ("Resumo Técnico: Desmistificando a Instabilidade
// Numérica na Inferência de LLMs com HEAL", section "A. Mitigando o
// Truncamento de Atenção via Quantização INT16") keeps tensors in 16-bit
// integers, holding memory at 16 bits per element with less truncation than
// a 16-bit float, and rescales rare outlier channels.  The decode step's
// state is stored that way here: column d (a value channel) of a state holds
// int16 mantissas m[c][d] and one int32 exponent e[d], value m * 2^e.  The
// exponent puts the column's largest magnitude M at [2^14, 2^15) quanta (one
// step higher when M would round up to 2^15), so the largest entry keeps 15
// bits and rounding costs at most half a quantum, 2^-15 M.  A column that
// holds a non-finite value is stored as the reserved mantissa -32768
// throughout, which reads back as NaN.
//
// The step reads 2 bytes per state element instead of 4: one (sequence,
// head) moves 2 x 37,632 B instead of 2 x 73,728 B.  It decodes the stored
// state, updates it in fp32 exactly like the float32 step, reads o from the
// updated fp32 values, and encodes them.  The exponent needs the column's
// maximum over all 96 rows, which the four row groups of a column exchange
// through LDS next to the partial sums of o.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

constexpr int Q16_NAN = -32768;
constexpr int ROWS = DK / 4;   // rows per thread (4 row groups of a column)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Exponent of a column whose largest magnitude is M (finite, >= 0): with
// M = f 2^x, f in [1/2, 1), e = x - 15; one more when M / 2^e >= 32767.5.
// M = 0 gives e = -15.
__device__ __forceinline__ int q16_exponent(float M) {
  int x;
  (void)frexpf(M, &x);
  int e = x - 15;
  if (ldexpf(M, -e) >= 32767.5f) ++e;
  return e;
}

// |s| for the column maximum, infinite for a non-finite s (NaN included).
__device__ __forceinline__ f32x4 q16_mag(f32x4 s) {
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = fabsf(s[j]);
    r[j] = a <= 3.402823466e38f ? a : __builtin_inff();
  }
  return r;
}

__device__ __forceinline__ f32x4 max4(f32x4 a, f32x4 b) {
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = fmaxf(a[j], b[j]);
  return r;
}

__device__ __forceinline__ f32x4 q16_decode(i16x4 m, i32x4 e) {
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = m[j] == Q16_NAN ? __builtin_nanf("") : ldexpf((float)m[j], e[j]);
  return r;
}

// Exponents of four columns from their maxima (infinite: the column is
// stored as the NaN code, exponent 0).
__device__ __forceinline__ i32x4 q16_exponents(f32x4 colmax) {
  i32x4 e;
#pragma unroll
  for (int j = 0; j < 4; ++j) e[j] = colmax[j] <= 3.402823466e38f ? q16_exponent(colmax[j]) : 0;
  return e;
}

// Mantissas, rounded half to even (|m| <= 32767 by the exponent rule).
__device__ __forceinline__ i16x4 q16_encode(f32x4 s, f32x4 colmax, i32x4 e) {
  i16x4 m;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    m[j] = colmax[j] <= 3.402823466e38f ? (short)__builtin_rintf(ldexpf(s[j], -e[j])) : (short)Q16_NAN;
  return m;
}

// Maxima of the four columns 4*c4.. over the four row groups (after the
// barrier that follows each group's store of its own maxima).
__device__ __forceinline__ f32x4 column_max(const f32x4 (*cmax)[48], int c4) {
  return max4(max4(cmax[0][c4], cmax[1][c4]), max4(cmax[2][c4], cmax[3][c4]));
}

// One workgroup of 192 threads per (sequence, head): thread t owns columns
// 4*(t%48)..+3 of rows 24*(t/48)..+23, as in the float32 step.
template <class TIn, class TOut>
__global__ void __launch_bounds__(192) step_q16_kernel(StepQ16Args a) {
  __shared__ float sk[DK];
  __shared__ float sq[DK];
  __shared__ f32x4 red[4][48];
  __shared__ f32x4 cmax[4][48];
  const int64_t item = blockIdx.x;
  const int64_t b = item / a.H;
  const int h = (int)(item % a.H);
  const int64_t slot = a.slot_idx ? (int64_t)a.slot_idx[b] : b;
  int16_t* M = a.pool.mant + (slot * a.H + h) * (int64_t)(DK * DV);
  int32_t* E = a.pool.expo + (slot * a.H + h) * (int64_t)DV;
  const int t = threadIdx.x;
  const int c4 = t % 48, rg = t / 48;

  i16x4 raw[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
    raw[r] = __builtin_nontemporal_load((const i16x4*)(M + (rg * ROWS + r) * DV) + c4);
  const i32x4 ex = *(const i32x4*)(E + 4 * c4);

  const TIn* qp = (const TIn*)a.q + item * DK;
  const TIn* kp = (const TIn*)a.k + item * DK;
  if (t < DK) sk[t] = (float)kp[t];
  else sq[t - DK] = (float)qp[t - DK];
  const f32x4 v = load4f((const TIn*)a.v + item * DV + 4 * c4);
  const float gam = exp2f(fmaxf(a.g[item], G_MIN) * LOG2E);
  __syncthreads();

  f32x4 s[ROWS];
  f32x4 acc = {0, 0, 0, 0}, lmax = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int d = rg * ROWS + r;
    s[r] = gam * q16_decode(raw[r], ex) + sk[d] * v;
    acc += sq[d] * s[r];
    lmax = max4(lmax, q16_mag(s[r]));
  }
  red[rg][c4] = acc;
  cmax[rg][c4] = lmax;
  __syncthreads();
  if (rg == 0) {
    const f32x4 o = red[0][c4] + red[1][c4] + red[2][c4] + red[3][c4];
    store4((TOut*)a.o + item * DV + 4 * c4, o);
  }
  const f32x4 colmax = column_max(cmax, c4);
  const i32x4 e = q16_exponents(colmax);
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
    __builtin_nontemporal_store(q16_encode(s[r], colmax, e), (i16x4*)(M + (rg * ROWS + r) * DV) + c4);
  if (rg == 0) *(i32x4*)(E + 4 * c4) = e;
}

// States [n][H][DK][DV] float32 to or from pool slots (slot_idx[i] or i):
// MODE 0 writes a float32 pool, 1 reads it, 2 encodes into a 16-bit pool,
// 3 decodes from it.  Same thread layout as the step.
template <int MODE>
__global__ void __launch_bounds__(192) state_io_kernel(StateIoArgs a) {
  __shared__ f32x4 cmax[4][48];
  const int64_t item = blockIdx.x;
  const int64_t i = item / a.H;
  const int h = (int)(item % a.H);
  const int64_t slot = a.slot_idx ? (int64_t)a.slot_idx[i] : i;
  const int64_t sh = slot * a.H + h;
  float* S = a.S + item * (int64_t)(DK * DV);
  const int t = threadIdx.x;
  const int c4 = t % 48, rg = t / 48;
  auto row = [&](int r) { return (int64_t)(rg * ROWS + r) * DV + 4 * c4; };
  if constexpr (MODE == 0 || MODE == 1) {
    float* P = a.pool_f32 + sh * (int64_t)(DK * DV);
    const float* src = MODE == 0 ? S : P;
    float* dst = MODE == 0 ? P : S;
    f32x4 x[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) x[r] = *(const f32x4*)(src + row(r));
#pragma unroll
    for (int r = 0; r < ROWS; ++r) *(f32x4*)(dst + row(r)) = x[r];
  } else if constexpr (MODE == 3) {
    const int16_t* M = a.q16.mant + sh * (int64_t)(DK * DV);
    const i32x4 e = *(const i32x4*)(a.q16.expo + sh * DV + 4 * c4);
    i16x4 m[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) m[r] = *(const i16x4*)(M + row(r));
#pragma unroll
    for (int r = 0; r < ROWS; ++r) *(f32x4*)(S + row(r)) = q16_decode(m[r], e);
  } else {
    int16_t* M = a.q16.mant + sh * (int64_t)(DK * DV);
    f32x4 x[ROWS];
    f32x4 lmax = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      x[r] = *(const f32x4*)(S + row(r));
      lmax = max4(lmax, q16_mag(x[r]));
    }
    cmax[rg][c4] = lmax;
    __syncthreads();
    const f32x4 colmax = column_max(cmax, c4);
    const i32x4 e = q16_exponents(colmax);
#pragma unroll
    for (int r = 0; r < ROWS; ++r) *(i16x4*)(M + row(r)) = q16_encode(x[r], colmax, e);
    if (rg == 0) *(i32x4*)(a.q16.expo + sh * DV + 4 * c4) = e;
  }
}

hipError_t launch_step_q16(const StepQ16Args& a, int in_bf16, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H)), block(192);
  if (in_bf16) {
    if (out_bf16) hipLaunchKernelGGL((step_q16_kernel<bf16, bf16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((step_q16_kernel<bf16, float>), grid, block, 0, st, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((step_q16_kernel<float, bf16>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((step_q16_kernel<float, float>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_state_io(const StateIoArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.n * a.H)), block(192);
  const bool q16 = a.q16.mant != nullptr;
  if (a.write) {
    if (q16) hipLaunchKernelGGL((state_io_kernel<2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((state_io_kernel<0>), grid, block, 0, st, a);
  } else {
    if (q16) hipLaunchKernelGGL((state_io_kernel<3>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((state_io_kernel<1>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace gla
