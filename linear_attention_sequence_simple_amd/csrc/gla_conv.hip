// Causal depth-wise convolution of width 4 with SiLU, ahead of the mixer, for
// gfx950.
//
// Every residual vector goes through a causal depth-wise Conv1d of width 4
// and a SiLU before the fused projection that produces the mixer's inputs
// ("Cómo i14 llevó Laplace 3B a AWS Trainium2", section "Diseño esencial de
// Laplace 3B"):
//     a_t[c] = bias[c] + sum_{j<4} w[c][j] x_{t-3+j}[c],   y_t[c] = a_t[c] / (1 + e^{-a_t[c]})
// Tokens before a sequence's first come from its history (the last three
// inputs of the previous call, kept per pool slot) or are zero.
//
// Plain streaming work: 2 bytes read and 2 written per bf16 token-channel, 9
// flops.  Each thread owns 8 channels (one 16-byte piece of a bf16 row) of a
// run of 32 tokens of one sequence; consecutive threads own consecutive
// pieces of a row, so every token row is read and written as whole
// contiguous lines.  The three previous inputs stay in registers; each run
// reads its three predecessors again (from L2: the neighbouring run just read
// them), 3/32 of its loads.  Loads are issued eight tokens ahead.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

constexpr int CONV_RUN = 32;   // tokens per thread
constexpr int CONV_AHEAD = 8;  // tokens loaded before their arithmetic

struct Row8 {
  float v[8];
};

__device__ __forceinline__ Row8 load8(const bf16* p) {
  const bf16x8 b = *(const bf16x8*)p;
  Row8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.v[e] = (float)b[e];
  return r;
}
__device__ __forceinline__ Row8 load8(const float* p) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  Row8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.v[e] = a[e];
    r.v[4 + e] = b[e];
  }
  return r;
}
__device__ __forceinline__ void store8(bf16* p, const Row8& r) {
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (bf16)r.v[e];
  *(bf16x8*)p = b;
}
__device__ __forceinline__ void store8(float* p, const Row8& r) {
  *(f32x4*)p = f32x4{r.v[0], r.v[1], r.v[2], r.v[3]};
  *(f32x4*)(p + 4) = f32x4{r.v[4], r.v[5], r.v[6], r.v[7]};
}
// A row piece as loaded: packed bf16 (4 registers) or fp32 (8), converted
// where it is used.
template <class T> struct Raw8;
template <> struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const f32x4*)p;
    b = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

__device__ __forceinline__ Row8 zero8() {
  Row8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.v[e] = 0.f;
  return r;
}

// First row and length of sequence b: packed offsets clamped into the
// tensor and the length bound, or b*T and T.
__device__ __forceinline__ void conv_span(const ConvArgs& a, int64_t b, int64_t& t0, int64_t& L) {
  if (a.cu) {
    t0 = min(max((int64_t)a.cu[b], (int64_t)0), a.total);
    const int64_t end = min(max((int64_t)a.cu[b + 1], t0), min(a.total, t0 + a.T));
    L = end - t0;
  } else {
    t0 = b * a.T;
    L = a.T;
  }
}

template <class TIn, class TOut>
__global__ void __launch_bounds__(256) conv_kernel(ConvArgs a) {
  const int cgs = a.D / 8;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cg = (int)(item % cgs);
  const int64_t rest = item / cgs;
  const int run = (int)(rest % a.runs);
  const int64_t b = rest / a.runs;
  if (b >= a.B) return;
  int64_t t0, L;
  conv_span(a, b, t0, L);
  const int64_t tb = (int64_t)run * CONV_RUN;
  if (tb >= L) return;
  const int n = (int)min((int64_t)CONV_RUN, L - tb);
  const int c0 = 8 * cg;
  const int64_t D = a.D;
  const TIn* xs = (const TIn*)a.x + t0 * D + c0;
  TOut* ys = (TOut*)a.y + t0 * D + c0;

  float w[8][4], bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const f32x4 we = *(const f32x4*)(a.w + (int64_t)(c0 + e) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[e][j] = we[j];
    bias[e] = 0.f;
  }
  if (a.bias) {
    const Row8 bb = load8(a.bias + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) bias[e] = bb.v[e];
  }
  // x_{tb-3}, x_{tb-2}, x_{tb-1}: earlier tokens of the sequence, else its
  // history row (t + 3), else zero
  Row8 h[3];
  const TIn* hist = (a.state && a.init) ? (const TIn*)a.state + (a.slot ? (int64_t)a.slot[b] : b) * 3 * D + c0 : nullptr;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int64_t t = tb - 3 + m;
    h[m] = t >= 0 ? load8(xs + t * D) : hist ? load8(hist + (t + 3) * D) : zero8();
  }

  Raw8<TIn> xin[CONV_AHEAD];
  for (int i0 = 0; i0 < n; i0 += CONV_AHEAD) {
#pragma unroll
    for (int i = 0; i < CONV_AHEAD; ++i)
      if (i0 + i < n) xin[i].load(xs + (tb + i0 + i) * D);
#pragma unroll
    for (int i = 0; i < CONV_AHEAD; ++i) {
      if (i0 + i < n) {
        Row8 out, cur;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cur.v[e] = xin[i][e];
          const float acc = bias[e] + w[e][0] * h[0].v[e] + w[e][1] * h[1].v[e] + w[e][2] * h[2].v[e] +
                            w[e][3] * cur.v[e];
          out.v[e] = acc / (1.f + __expf(-acc));
        }
        store8(ys + (tb + i0 + i) * D, out);
        h[0] = h[1];
        h[1] = h[2];
        h[2] = cur;
      }
    }
  }
}

// New history of every sequence: the last three inputs of its old history
// followed by its tokens.  Runs after conv_kernel (which reads the old
// history); each thread reads its three old rows before writing them.
template <class TIn>
__global__ void __launch_bounds__(256) conv_state_kernel(ConvArgs a) {
  const int cgs = a.D / 8;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cg = (int)(item % cgs);
  const int64_t b = item / cgs;
  if (b >= a.B) return;
  int64_t t0, L;
  conv_span(a, b, t0, L);
  const int64_t D = a.D;
  const int c0 = 8 * cg;
  TIn* st = (TIn*)a.state + (a.slot ? (int64_t)a.slot[b] : b) * 3 * D + c0;
  const TIn* xs = (const TIn*)a.x + t0 * D + c0;
  constexpr int W = sizeof(TIn) * 8 / 16;   // 16-byte pieces per 8 channels
  uint4 r[3][W];
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const int64_t z = L + m;                 // index into history (3 rows) + tokens
    const TIn* src = z >= 3 ? xs + (z - 3) * D : a.init ? st + z * D : nullptr;
#pragma unroll
    for (int p = 0; p < W; ++p) r[m][p] = src ? ((const uint4*)src)[p] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int p = 0; p < W; ++p) ((uint4*)(st + m * D))[p] = r[m][p];
}

template <class TIn, class TOut>
static hipError_t launch_conv_t(const ConvArgs& a, hipStream_t st) {
  const int64_t threads = a.B * a.runs * (a.D / 8);
  hipLaunchKernelGGL((conv_kernel<TIn, TOut>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.state) return e;
  const int64_t sthreads = a.B * (a.D / 8);
  hipLaunchKernelGGL((conv_state_kernel<TIn>), dim3((unsigned)((sthreads + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs& a, bool in_bf16, bool out_bf16, hipStream_t st) {
  if (in_bf16) return out_bf16 ? launch_conv_t<bf16, bf16>(a, st) : launch_conv_t<bf16, float>(a, st);
  return out_bf16 ? launch_conv_t<float, bf16>(a, st) : launch_conv_t<float, float>(a, st);
}

}  // namespace gla
