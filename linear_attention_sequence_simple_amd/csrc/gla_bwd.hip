// Backward of the Simple GLA mixer for gfx950: the finishing kernels.
//
// The pages run the backward sequentially over the chunk steps ("Adaptaciones
// para AWS Trainium2", item 3, of the page "Cómo i14 llevó Laplace 3B a AWS
// Trainium2").  Here the gradients come from three walks of the chunk kernel
// (gla_walk.hip), each the forward recurrence with other operand roles:
//   dq_t = sum_{s<=t} e^{b_t-b_s} (dO_t.v_s) k_s + ...      forward in time,
//   dv_t = sum_{s>=t} e^{b_s-b_t} (k_t.q_s) dO_s + ...      backward in time,
//   dk_t = sum_{s>=t} e^{b_s-b_t} (v_t.dO_s) q_s + ...      backward in time,
// where the contraction over the 192 value columns (dq, dk) is split into two
// halves whose fp32 partial sums are added here.  The log-decay gradient uses
//     dg_t = sum_{u >= t} (q_u.dq_u - k_u.dk_u) + <dS_T, S_T>
// (derivative through the running sum of the log-decay): bwd_finish writes
// the in-chunk suffix sums and the chunk totals, dg_finish adds the rest.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

// One workgroup per (batch, head, chunk).  Threads walk the chunk's 128 x 96
// gradient rows as 16-byte pieces of 8 columns (row-contiguous accesses).
template <class TOut>
__global__ void __launch_bounds__(256) bwd_finish_kernel(BwdFinishArgs a) {
  __shared__ float part[CH][13];            // per token: r of each 8-column piece
  const int N = a.n_chunks;
  const int64_t item = blockIdx.x;
  const int n = (int)(item % N);
  const int64_t bh = item / N;
  const int h = (int)(bh % a.H);
  const int64_t b = bh / a.H;
  const int64_t T = a.T;
  const int64_t plane = a.B * T * a.H * DK;   // distance between the two partial sums
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int p = threadIdx.x + 256 * i, row = p / 12, cp = p % 12;
    const int64_t t = (int64_t)n * CH + row;
    float r = 0.f;
    if (t < T) {
      const int64_t off = ((b * T + t) * a.H + h) * DK + cp * 8;
      const f32x4 qa = *(const f32x4*)(a.dq_part + off), qb = *(const f32x4*)(a.dq_part + off + 4);
      const f32x4 qc = *(const f32x4*)(a.dq_part + plane + off), qd = *(const f32x4*)(a.dq_part + plane + off + 4);
      const f32x4 ka = *(const f32x4*)(a.dk_part + off), kb = *(const f32x4*)(a.dk_part + off + 4);
      const f32x4 kc = *(const f32x4*)(a.dk_part + plane + off), kd = *(const f32x4*)(a.dk_part + plane + off + 4);
      const bf16x8 qv = *(const bf16x8*)((const bf16*)a.q + off);
      const bf16x8 kv = *(const bf16x8*)((const bf16*)a.k + off);
      const f32x4 dq0 = qa + qc, dq1 = qb + qd, dk0 = ka + kc, dk1 = kb + kd;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r += (float)qv[e] * dq0[e] - (float)kv[e] * dk0[e];
        r += (float)qv[e + 4] * dq1[e] - (float)kv[e + 4] * dk1[e];
      }
      store4((TOut*)a.dq + off, dq0);
      store4((TOut*)a.dq + off + 4, dq1);
      store4((TOut*)a.dk + off, dk0);
      store4((TOut*)a.dk + off + 4, dk1);
    }
    part[row][cp] = r;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // r of tokens 2l, 2l+1 (pieces summed in a fixed order), then in-chunk
    // suffix sums
    const int l = threadIdx.x;
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int cp = 0; cp < 12; ++cp) {
      r0 += part[2 * l][cp];
      r1 += part[2 * l + 1][cp];
    }
    const float suf = wave_incl_rscan(r0 + r1);     // sum over tokens >= 2l
    float* dgb = a.dg + b * T * a.H + h;
    const int64_t ta = (int64_t)n * CH + 2 * l, tb = ta + 1;
    if (ta < T) dgb[ta * a.H] = suf;
    if (tb < T) dgb[tb * a.H] = suf - r0;
    if (l == 0) a.chunk_r[bh * N + n] = suf;
  }
}

// dg += (sum of the chunk totals after this chunk) + <dS_T, S_T>, and
// dS0 = e^{g_0} dS_{-1}: the state gradient leaving the first token, carried
// through that token's decay.  One workgroup per (batch, head).
__global__ void __launch_bounds__(256) dg_finish_kernel(float* dg, const float* chunk_r, const float* dS_T,
                                                        const float* S_T, float* dS0, const float* g, int64_t T,
                                                        int H, int N) {
  __shared__ float red[256];
  __shared__ float suffix[1025];
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / H;
  const int h = (int)(bh % H);
  float c = 0.f;
  if (dS_T) {
    const float* x = dS_T + bh * (int64_t)(DK * DV);
    const float* y = S_T + bh * (int64_t)(DK * DV);
    for (int e = threadIdx.x; e < DK * DV; e += 256) c += x[e] * y[e];
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const float cst = red[0];
  if (threadIdx.x == 0) {
    float acc = cst;
    suffix[N] = acc;
    for (int n = N - 1; n >= 0; --n) {
      suffix[n] = acc;            // chunks after n, plus the constant
      acc += chunk_r[bh * N + n];
    }
  }
  __syncthreads();
  float* dgb = dg + b * T * H + h;
  for (int64_t t = threadIdx.x; t < T; t += 256) dgb[t * H] += suffix[t / CH];
  if (dS0) {
    const float gam0 = __expf(fmaxf(g[b * T * H + h], G_MIN));
    float* x = dS0 + bh * (int64_t)(DK * DV);
    for (int e = threadIdx.x; e < DK * DV; e += 256) x[e] *= gam0;
  }
}

hipError_t launch_bwd_finish(const BwdFinishArgs& a, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H * a.n_chunks)), block(256);
  if (out_bf16) hipLaunchKernelGGL((bwd_finish_kernel<bf16>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_finish_kernel<float>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dg_finish(float* dg, const float* chunk_r, const float* dS_T, const float* S_T, float* dS0,
                            const float* g, int64_t B, int64_t T, int H, int n_chunks, hipStream_t st) {
  if (n_chunks > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dg_finish_kernel, dim3((unsigned)(B * H)), dim3(256), 0, st, dg, chunk_r, dS_T, S_T, dS0, g,
                     T, H, n_chunks);
  return hipGetLastError();
}

}  // namespace gla
