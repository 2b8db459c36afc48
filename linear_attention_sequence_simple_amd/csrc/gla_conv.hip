// Causal depth-wise convolution of width 4 with SiLU, ahead of the mixer, for
// gfx950.
//
// Every residual vector goes through a causal depth-wise Conv1d of width 4
// and a SiLU before the fused projection that produces the mixer's inputs
// ("Cómo i14 llevó Laplace 3B a AWS Trainium2", section "Diseño esencial de
// Laplace 3B"):
//     a_t[c] = bias[c] + sum_{j<4} w[c][j] x_{t-3+j}[c],   y_t[c] = a_t[c] / (1 + e^{-a_t[c]})
// Tokens before a sequence's first come from its window (the last four
// inputs of the previous call, float32, kept per pool slot; the newest three
// are read) or are zero.
//
// Plain streaming work: 2 bytes read and 2 written per bf16 token-channel, 9
// flops.  Each thread owns 8 channels (one 16-byte piece of a bf16 row) of a
// run of 32 tokens of one sequence; consecutive threads own consecutive
// pieces of a row, so every token row is read and written as whole
// contiguous lines.  The three previous inputs stay in registers; each run
// reads its three predecessors again (from L2: the neighbouring run just read
// them), 3/32 of its loads.  A whole run keeps eight loads in flight: token
// i + 8 is requested as token i is used.  Measured at 0.87 of a plain device
// copy of the same tensors (about 4.6 against 5.2 TB/s).  The thread
// of a sequence's first run (per 8 channels) is the only reader of its old
// window, so it also writes the new one, after reading the old.
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
// The same for the streamed outputs, which nothing reads back soon.
__device__ __forceinline__ void store8_stream(bf16* p, const Row8& r) {
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (bf16)r.v[e];
  __builtin_nontemporal_store(b, (bf16x8*)p);
}
__device__ __forceinline__ void store8_stream(float* p, const Row8& r) {
  __builtin_nontemporal_store(f32x4{r.v[0], r.v[1], r.v[2], r.v[3]}, (f32x4*)p);
  __builtin_nontemporal_store(f32x4{r.v[4], r.v[5], r.v[6], r.v[7]}, (f32x4*)(p + 4));
}
// A streamed row piece as loaded (non-temporal: each token row is read by
// its run and, three rows of it, by the next): packed bf16 (4 registers) or
// fp32 (8), converted where it is used.
template <class T> struct Raw8;
template <> struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = __builtin_nontemporal_load((const bf16x8*)p); }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load((const f32x4*)p);
    b = __builtin_nontemporal_load((const f32x4*)(p + 4));
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

__device__ __forceinline__ Row8 zero8() {
  Row8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.v[e] = 0.f;
  return r;
}

// x_{t-3}, x_{t-2}, x_{t-1} of the token being computed.
struct Window {
  Row8 r0, r1, r2;
};

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

// Outputs of tokens tb..tb+n-1 of one sequence for channels c0..c0+7, from
// xs (the sequence's first row at channel c0) to ys; h holds x_{tb-3..tb-1}.
template <class TIn, class TOut>
__device__ __forceinline__ void conv_tokens(const ConvArgs& a, int c0, const TIn* xs, TOut* ys, int64_t tb, int n,
                                            Window& h) {
  const int64_t D = a.D;
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
  auto step = [&](const Raw8<TIn>& x, int64_t t) {
    Row8 out, cur;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cur.v[e] = x[e];
      const float acc = bias[e] + w[e][0] * h.r0.v[e] + w[e][1] * h.r1.v[e] + w[e][2] * h.r2.v[e] +
                        w[e][3] * cur.v[e];
      out.v[e] = acc / (1.f + __expf(-acc));
    }
    store8_stream(ys + t * D, out);
    h.r0 = h.r1;
    h.r1 = h.r2;
    h.r2 = cur;
  };
  Raw8<TIn> xin[CONV_AHEAD];
  if (n == CONV_RUN) {
    // a whole run: token i + CONV_AHEAD is requested as token i is used, so
    // CONV_AHEAD loads stay in flight throughout
#pragma unroll
    for (int i = 0; i < CONV_AHEAD; ++i) xin[i].load(xs + (tb + i) * D);
#pragma unroll
    for (int i = 0; i < CONV_RUN; ++i) {
      const Raw8<TIn> x = xin[i % CONV_AHEAD];
      if (i + CONV_AHEAD < CONV_RUN) xin[i % CONV_AHEAD].load(xs + (tb + i + CONV_AHEAD) * D);
      step(x, tb + i);
    }
    return;
  }
  // the last, shorter run of a sequence: CONV_AHEAD tokens at a time
  for (int i0 = 0; i0 < n; i0 += CONV_AHEAD) {
#pragma unroll
    for (int i = 0; i < CONV_AHEAD; ++i)
      if (i0 + i < n) xin[i].load(xs + (tb + i0 + i) * D);
#pragma unroll
    for (int i = 0; i < CONV_AHEAD; ++i)
      if (i0 + i < n) step(xin[i], tb + i0 + i);
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
  const int c0 = 8 * cg;
  const int64_t D = a.D;
  const TIn* xs = (const TIn*)a.x + t0 * D + c0;
  float* hist = a.state ? a.state + (a.slot ? (int64_t)a.slot[b] : b) * CONV_WIN * D + c0 : nullptr;
  const bool keeper = run == 0 && hist;        // writes the sequence's new window
  if (tb >= L && !keeper) return;
  // x_{tb-3}, x_{tb-2}, x_{tb-1}: earlier tokens of the sequence, else its
  // window row t + 4 (row m holds x_{m-4}), else zero
  auto before = [&](int64_t t) {
    return t >= 0 ? load8(xs + t * D) : (hist && a.init) ? load8(hist + (t + CONV_WIN) * D) : zero8();
  };
  Window h{before(tb - 3), before(tb - 2), before(tb - 1)};
  if (keeper && !(L == 0 && a.init)) {
    // rows L..L+3 of (old window, tokens), with h holding old rows 1..3 (or
    // zeros without init) since tb = 0; row 0 of the old window is needed
    // only when L = 0, where the window stays as it is (with init) or is the
    // zero window (without).  Every source is read before the writes.
    const Row8 n0 = L >= 4 ? load8(xs + (L - 4) * D) : L == 3 ? h.r2 : L == 2 ? h.r1 : L == 1 ? h.r0 : zero8();
    const Row8 n1 = L >= 3 ? load8(xs + (L - 3) * D) : L == 2 ? h.r2 : L == 1 ? h.r1 : h.r0;
    const Row8 n2 = L >= 2 ? load8(xs + (L - 2) * D) : L == 1 ? h.r2 : h.r1;
    const Row8 n3 = L >= 1 ? load8(xs + (L - 1) * D) : h.r2;
    store8(hist, n0);
    store8(hist + D, n1);
    store8(hist + 2 * D, n2);
    store8(hist + 3 * D, n3);
  }
  if (tb < L) conv_tokens<TIn, TOut>(a, c0, xs, (TOut*)a.y + t0 * D + c0, tb, (int)min((int64_t)CONV_RUN, L - tb), h);
}

template <class TIn, class TOut>
static hipError_t launch_conv_t(ConvArgs a, hipStream_t st) {
  a.runs = (int)((a.T + CONV_RUN - 1) / CONV_RUN);
  const int64_t threads = a.B * a.runs * (a.D / 8);
  hipLaunchKernelGGL((conv_kernel<TIn, TOut>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs& a, bool in_bf16, bool out_bf16, hipStream_t st) {
  if (in_bf16) return out_bf16 ? launch_conv_t<bf16, bf16>(a, st) : launch_conv_t<bf16, float>(a, st);
  return out_bf16 ? launch_conv_t<float, bf16>(a, st) : launch_conv_t<float, float>(a, st);
}

}  // namespace gla
