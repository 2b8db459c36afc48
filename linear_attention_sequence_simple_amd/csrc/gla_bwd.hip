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
// halves: the walk of the second half adds the first half's fp32 partial sums
// and writes q_t.dq_t (k_t.dk_t).  The log-decay gradient uses
//     dg_t = sum_{u >= t} (q_u.dq_u - k_u.dk_u) + <dS_T, S_T>
// (derivative through the running sum of the log-decay): bwd_finish writes
// the in-chunk suffix sums and the chunk totals, dg_const and dg_carry add
// the rest.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

// r_t = q_t.dq_t - k_t.dk_t (both dot products written by the last walks of
// dq and dk), its in-chunk suffix sums into dg and the chunk totals.  One
// wave per (batch, head, chunk), four per workgroup; two tokens per lane.
__global__ void __launch_bounds__(256) bwd_finish_kernel(BwdFinishArgs a) {
  const int N = a.n_chunks;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.B * a.H * N) return;
  const int n = (int)(item % N);
  const int64_t bh = item / N;
  const int h = (int)(bh % a.H);
  const int64_t b = bh / a.H;
  const int64_t T = a.T;
  const int l = threadIdx.x & 63;
  const int64_t ta = (int64_t)n * CH + 2 * l, tb = ta + 1;
  const int64_t base = b * T * a.H + h;
  const float r0 = ta < T ? a.rq[base + ta * a.H] - a.rk[base + ta * a.H] : 0.f;
  const float r1 = tb < T ? a.rq[base + tb * a.H] - a.rk[base + tb * a.H] : 0.f;
  const float suf = wave_incl_rscan(r0 + r1);     // sum over tokens >= 2l
  if (ta < T) a.dg[base + ta * a.H] = suf;
  if (tb < T) a.dg[base + tb * a.H] = suf - r0;
  if (l == 0) a.chunk_r[bh * N + n] = suf;
}

// dg_carry reads and writes [B, T, H] as (batch, chunk) tiles: the 128
// tokens x H heads of one chunk are contiguous, so whole tiles move as
// coalesced rows.  (The scan above keeps one wave per (batch, head, chunk):
// a tiled scan with the same coalescing ran slower, 9.6 against 6.2 us at
// B=4, T=4096, for want of workgroups.)
constexpr int HG = 16;         // heads per tile pass

// Per (batch, head): cst = <dS_T, S_T> (zero without dS_T) into cst[bh], and
// dS0 = e^{g_0} dS_{-1}, the state gradient leaving the first token carried
// through that token's decay.
__global__ void __launch_bounds__(256) dg_const_kernel(float* cst, const float* dS_T, const float* S_T, float* dS0,
                                                       const float* g, int64_t T, int H) {
  __shared__ float red[256];
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
  if (threadIdx.x == 0) cst[bh] = red[0];
  if (dS0) {
    const float gam0 = __expf(fmaxf(g[b * T * H + h], G_MIN));
    float* x = dS0 + bh * (int64_t)(DK * DV);
    for (int e = threadIdx.x; e < DK * DV; e += 256) x[e] *= gam0;
  }
}

// dg += (sum of the chunk totals after this chunk) + cst, per head.  One
// workgroup per (batch, chunk): 16 threads per head add the later chunks'
// totals (a fixed order, so results are deterministic), then the tile is
// updated as coalesced rows.
__global__ void __launch_bounds__(256) dg_carry_kernel(float* dg, const float* chunk_r, const float* cst, int64_t T,
                                                       int H, int N) {
  __shared__ float part[HG][16];
  __shared__ float carry[HG];
  const int64_t b = blockIdx.x / N;
  const int n = (int)(blockIdx.x % N);
  const int64_t t0 = (int64_t)n * CH;
  for (int hg = 0; hg < H; hg += HG) {
    const int G = min(HG, H - hg);
    const int hh = threadIdx.x >> 4, j = threadIdx.x & 15;
    if (hh < G) {
      const float* r = chunk_r + (b * H + hg + hh) * N;
      float s = 0.f;
      for (int m = n + 1 + j; m < N; m += 16) s += r[m];
      part[hh][j] = s;
    }
    __syncthreads();
    if (threadIdx.x < G) {
      float s = cst ? cst[b * H + hg + threadIdx.x] : 0.f;
      for (int i = 0; i < 16; ++i) s += part[threadIdx.x][i];
      carry[threadIdx.x] = s;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < CH * G; i += 256) {
      const int tok = i / G, k = i % G;
      if (t0 + tok < T) dg[(b * T + t0 + tok) * H + hg + k] += carry[k];
    }
    __syncthreads();
  }
}

// The fp32 backward's dot products rq_t = q_t.dq_t and rk_t = k_t.dk_t from
// the float32 gradients (the walks' own sums), and, for bf16 outputs, those
// gradients rounded into the outputs.  32 lanes per (batch, token, head) row,
// three of its 96 columns each, so that a wave reads two whole rows.
__global__ void __launch_bounds__(256) row_dots_kernel(RowDotsArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= a.rows) return;
  const int l = threadIdx.x & 31;
  const int64_t off = row * DK + 3 * l;
  float rq = 0.f, rk = 0.f;
#pragma unroll
  for (int e = 0; e < 3; ++e) {
    rq += a.q[off + e] * a.dq[off + e];
    rk += a.k[off + e] * a.dk[off + e];
  }
#pragma unroll
  for (int m = 16; m > 0; m >>= 1) {
    rq += __shfl_xor(rq, m, 32);
    rk += __shfl_xor(rk, m, 32);
  }
  if (l == 0) {
    a.rq[row] = rq;
    a.rk[row] = rk;
  }
  if (a.dq_bf16) {
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      a.dq_bf16[off + e] = (bf16)a.dq[off + e];
      a.dk_bf16[off + e] = (bf16)a.dk[off + e];
    }
  }
}

hipError_t launch_row_dots(const RowDotsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(row_dots_kernel, dim3((unsigned)((a.rows + 7) / 8)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const BwdFinishArgs& a, hipStream_t st) {
  const int64_t items = a.B * a.H * a.n_chunks;
  hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// chunk_r holds [B*H][n_chunks] chunk totals followed by B*H constants (not
// formed when neither dS_T nor dS0 is given: the constant is then zero).
hipError_t launch_dg_finish(float* dg, const float* chunk_r, const float* dS_T, const float* S_T, float* dS0,
                            const float* g, int64_t B, int64_t T, int H, int n_chunks, hipStream_t st) {
  float* cst = nullptr;
  if (dS_T || dS0) {
    cst = const_cast<float*>(chunk_r) + B * H * (int64_t)n_chunks;
    hipLaunchKernelGGL(dg_const_kernel, dim3((unsigned)(B * H)), dim3(256), 0, st, cst, dS_T, S_T, dS0, g, T, H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(dg_carry_kernel, dim3((unsigned)(B * n_chunks)), dim3(256), 0, st, dg, chunk_r, cst, T, H,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace gla
