// Chunk-parallel part of the Simple GLA backward for gfx950.
//
// The pages run the backward sequentially over the chunk steps ("Adaptaciones
// para AWS Trainium2", item 3, of the page "Cómo i14 llevó Laplace 3B a AWS
// Trainium2").  Here the two sequential parts -- the forward states S_n
// entering each chunk and the state gradients dS_{n+1} leaving it -- come from
// the chunk walks; with those in hand every chunk's gradients are independent:
//     P  = (Q K^T) (.) M,   dP = (dO V^T) (.) M
//     dQ = dP K + diag(Lambda) dO S_n^T
//     dK = dP^T Q + diag(kappa) V dS_{n+1}^T
//     dV = P^T dO + diag(kappa) K dS_{n+1}
// (chain rule of the chunk form O = (QK^T (.) M)V + diag(Lambda) Q S_n,
// S_{n+1} = Gamma S_n + (diag(kappa) K)^T V).  The log-decay gradient uses
//     dg_t = sum_{u >= t} (q_u.dq_u - k_u.dk_u) + <dS_T, S_T>
// (derivative through the running sum of the log-decay): this kernel writes
// the in-chunk suffix sums and the chunk totals; dg_finish adds the rest.
//
// One workgroup (4 waves) per (batch, head, chunk).  Wave w owns the 32
// tokens 32w..32w+31 as the column block of its result tiles:
//   dV^T[:, w], dQ^T[:, w], dK^T[:, w]  (c or d rows, tokens in columns),
// so each lane ends up with one token and the q.dq / k.dk dot products need
// only a sum over its registers and one exchange with the other lane group.
// The masked scores and the stored states enter the products as compensated
// bf16 pairs (value + residual, two MFMAs); q, k, v, dO are exact bf16.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

struct BwdSmem {
  static constexpr int PX = DK + 8;
  static constexpr int PY = DV + 8;
  bf16 q[CH * PX];
  bf16 k[CH * PX];
  bf16 v[CH * PY];
  bf16 dO[CH * PY];
  DecayLds dec;
  float r[CH];
};

__device__ __forceinline__ void load_tile_lds(bf16* lds, int pitch, const bf16* base, int64_t row_stride,
                                              int width, int64_t t0, int64_t T) {
  const int ppr = width / 8;
  const int np = CH * ppr;
  for (int p = threadIdx.x; p < np; p += 256) {
    const int row = p / ppr, cp = p % ppr;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t0 + row < T) val = *(const uint4*)(base + (t0 + row) * row_stride + cp * 8);
    *(uint4*)(lds + row * pitch + cp * 8) = val;
  }
}

__device__ __forceinline__ bf16x8 gfrag(const bf16* base, int f) {
  return *(const bf16x8*)(base + ((int64_t)f * 64 + lane_id()) * 8);
}

// Masked score tiles of one column block: rows in [32*R0, 128) (or [0, 32*(W+1))),
// held as compensated bf16 operand pairs for the next contraction over rows.
struct PairFrag {
  bf16x8 hi[2], lo[2];
};

template <class TOut, int W>
__device__ __forceinline__ void bwd_wave(const BwdArgs& a, BwdSmem& sm, int64_t bh, int64_t b, int h, int n) {
  constexpr int PX = BwdSmem::PX, PY = BwdSmem::PY;
  const int lane = lane_id();
  const int g2 = lane >> 5;
  const int tl = 32 * W + (lane & 31);            // this lane's token inside the chunk
  const int64_t T = a.T;
  const int64_t trow = (int64_t)n * CH + tl;
  const bool valid = trow < T;
  const float b_t = sm.dec.b2[tl];
  // per chunk: [hi fragments | lo fragments]
  const int64_t frag_base = (bh * a.n_chunks + n) * (int64_t)(2 * DK * DV);
  const bf16* Sdc = (const bf16*)a.s_dc + frag_base;
  const bf16* dSdc = (const bf16*)a.ds_dc + frag_base;
  const bf16* dScd = (const bf16*)a.ds_cd + frag_base;
  const float kap = sm.dec.kap[tl];
  const float lam = sm.dec.lam[tl];
  const int64_t tok = ((int64_t)b * T + trow) * a.H + h;

  // ---- phase 1: P (query rows i >= 32W, key column tl) and dV^T[:, W]
  {
    PairFrag P[4];
#pragma unroll
    for (int I = W; I < 4; ++I) {
      f32x16 ap = {};
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          ap = mfma(frag_kcN(sm.q, PX, 32 * I, 32 * kb, s), frag_kcN(sm.k, PX, 32 * W, 32 * kb, s), ap);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * I + out_row(r);
        const float w = exp2f(fminf(sm.dec.b2[i] - b_t, 0.f));
        ap[r] = ((I > W) || (tl <= i)) ? ap[r] * w : 0.f;
      }
      regs_to_frag_split(ap, 0, P[I].hi[0], P[I].lo[0]);
      regs_to_frag_split(ap, 1, P[I].hi[1], P[I].lo[1]);
    }
#pragma unroll
    for (int cb = 0; cb < 6; ++cb) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 bk = frag_kcN(sm.k, PX, 32 * W, 32 * kb, s);
          const int f = cb * 6 + kb * 2 + s;
          acc = mfma(gfrag(dScd, f), bk, acc);
          acc = mfma(gfrag(dScd + DK * DV, f), bk, acc);
        }
      acc *= kap;
#pragma unroll
      for (int I = W; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ad = frag_kr(sm.dO, PY, 32 * I, 32 * cb, s);
          acc = mfma(ad, P[I].hi[s], acc);
          acc = mfma(ad, P[I].lo[s], acc);
        }
      if (valid) {
        TOut* p = (TOut*)a.dv + tok * DV + 32 * cb + 4 * g2;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          store4(p + 8 * qq, f32x4{acc[4 * qq], acc[4 * qq + 1], acc[4 * qq + 2], acc[4 * qq + 3]});
      }
    }
  }

  // ---- phase 2: dP^T (key rows j <= block W, query column tl) and dQ^T[:, W]
  float rq = 0.f;
  {
    PairFrag D[4];
#pragma unroll
    for (int J = 0; J <= W; ++J) {
      f32x16 ad = {};
#pragma unroll
      for (int kb = 0; kb < 6; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          ad = mfma(frag_kcN(sm.v, PY, 32 * J, 32 * kb, s), frag_kcN(sm.dO, PY, 32 * W, 32 * kb, s), ad);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = 32 * J + out_row(r);
        const float w = exp2f(fminf(b_t - sm.dec.b2[j], 0.f));
        ad[r] = ((J < W) || (j <= tl)) ? ad[r] * w : 0.f;
      }
      regs_to_frag_split(ad, 0, D[J].hi[0], D[J].lo[0]);
      regs_to_frag_split(ad, 1, D[J].hi[1], D[J].lo[1]);
    }
#pragma unroll
    for (int db = 0; db < 3; ++db) {
      f32x16 aq = {};
#pragma unroll
      for (int kc = 0; kc < 12; ++kc) {
        const bf16x8 bo = frag_kcN(sm.dO, PY, 32 * W, 32 * (kc >> 1), kc & 1);
        aq = mfma(gfrag(Sdc, db * 12 + kc), bo, aq);
        aq = mfma(gfrag(Sdc + DK * DV, db * 12 + kc), bo, aq);
      }
      aq *= lam;
#pragma unroll
      for (int J = 0; J <= W; ++J)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ak = frag_kr(sm.k, PX, 32 * J, 32 * db, s);
          aq = mfma(ak, D[J].hi[s], aq);
          aq = mfma(ak, D[J].lo[s], aq);
        }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 qv = load4f(sm.q + tl * PX + 32 * db + 8 * qq + 4 * g2);
#pragma unroll
        for (int e = 0; e < 4; ++e) rq += qv[e] * aq[4 * qq + e];
      }
      if (valid) {
        TOut* pq = (TOut*)a.dq + tok * DK + 32 * db + 4 * g2;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          store4(pq + 8 * qq, f32x4{aq[4 * qq], aq[4 * qq + 1], aq[4 * qq + 2], aq[4 * qq + 3]});
      }
    }
  }

  // ---- phase 3: dP (query rows i >= 32W, key column tl) and dK^T[:, W]
  float rk = 0.f;
  {
    PairFrag D[4];
#pragma unroll
    for (int I = W; I < 4; ++I) {
      f32x16 ad = {};
#pragma unroll
      for (int kb = 0; kb < 6; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          ad = mfma(frag_kcN(sm.dO, PY, 32 * I, 32 * kb, s), frag_kcN(sm.v, PY, 32 * W, 32 * kb, s), ad);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * I + out_row(r);
        const float w = exp2f(fminf(sm.dec.b2[i] - b_t, 0.f));
        ad[r] = ((I > W) || (tl <= i)) ? ad[r] * w : 0.f;
      }
      regs_to_frag_split(ad, 0, D[I].hi[0], D[I].lo[0]);
      regs_to_frag_split(ad, 1, D[I].hi[1], D[I].lo[1]);
    }
#pragma unroll
    for (int db = 0; db < 3; ++db) {
      f32x16 ak = {};
#pragma unroll
      for (int kc = 0; kc < 12; ++kc) {
        const bf16x8 bv = frag_kcN(sm.v, PY, 32 * W, 32 * (kc >> 1), kc & 1);
        ak = mfma(gfrag(dSdc, db * 12 + kc), bv, ak);
        ak = mfma(gfrag(dSdc + DK * DV, db * 12 + kc), bv, ak);
      }
      ak *= kap;
#pragma unroll
      for (int I = W; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 aq = frag_kr(sm.q, PX, 32 * I, 32 * db, s);
          ak = mfma(aq, D[I].hi[s], ak);
          ak = mfma(aq, D[I].lo[s], ak);
        }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 kv = load4f(sm.k + tl * PX + 32 * db + 8 * qq + 4 * g2);
#pragma unroll
        for (int e = 0; e < 4; ++e) rk += kv[e] * ak[4 * qq + e];
      }
      if (valid) {
        TOut* pk = (TOut*)a.dk + tok * DK + 32 * db + 4 * g2;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          store4(pk + 8 * qq, f32x4{ak[4 * qq], ak[4 * qq + 1], ak[4 * qq + 2], ak[4 * qq + 3]});
      }
    }
  }
  float r = rq - rk;
  r += __shfl_xor(r, 32, 64);
  if (lane < 32) sm.r[tl] = valid ? r : 0.f;
}

template <class TOut>
__global__ void __launch_bounds__(256, 1) bwd_chunk_kernel(BwdArgs a) {
  __shared__ BwdSmem sm;
  const int N = a.n_chunks;
  const int64_t item = blockIdx.x;
  const int n = (int)(item % N);
  const int64_t bh = item / N;
  const int h = (int)(bh % a.H);
  const int64_t b = bh / a.H;
  const int64_t T = a.T;
  const int64_t t0 = (int64_t)n * CH;
  const int64_t rsx = (int64_t)a.H * DK, rsy = (int64_t)a.H * DV;
  load_tile_lds(sm.q, BwdSmem::PX, (const bf16*)a.q + b * T * rsx + h * DK, rsx, DK, t0, T);
  load_tile_lds(sm.k, BwdSmem::PX, (const bf16*)a.k + b * T * rsx + h * DK, rsx, DK, t0, T);
  load_tile_lds(sm.v, BwdSmem::PY, (const bf16*)a.v + b * T * rsy + h * DV, rsy, DV, t0, T);
  load_tile_lds(sm.dO, BwdSmem::PY, (const bf16*)a.dO + b * T * rsy + h * DV, rsy, DV, t0, T);
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const float* gb = a.g + b * T * a.H + h;
    const int64_t ta = t0 + 2 * l, tb = ta + 1, tc = t0 + 127 - 2 * l, td = tc - 1;
    build_decay(&sm.dec, ta < T ? gb[ta * a.H] : 0.f, tb < T ? gb[tb * a.H] : 0.f, tc < T ? gb[tc * a.H] : 0.f,
                td < T ? gb[td * a.H] : 0.f);
  }
  __syncthreads();
  switch (threadIdx.x >> 6) {
    case 0: bwd_wave<TOut, 0>(a, sm, bh, b, h, n); break;
    case 1: bwd_wave<TOut, 1>(a, sm, bh, b, h, n); break;
    case 2: bwd_wave<TOut, 2>(a, sm, bh, b, h, n); break;
    default: bwd_wave<TOut, 3>(a, sm, bh, b, h, n); break;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // in-chunk suffix sums of r (two tokens per lane)
    const int l = threadIdx.x;
    const float r0 = sm.r[2 * l], r1 = sm.r[2 * l + 1];
    const float suf = wave_incl_rscan(r0 + r1);     // sum over tokens >= 2l
    const float d0 = suf, d1 = suf - r0;
    float* dgb = a.dg + b * T * a.H + h;
    const int64_t ta = t0 + 2 * l, tb = ta + 1;
    if (ta < T) dgb[ta * a.H] = d0;
    if (tb < T) dgb[tb * a.H] = d1;
    if (l == 0) a.chunk_r[bh * N + n] = suf;
  }
}

// dg += (sum of the chunk totals after this chunk) + <dS_T, S_T>; one
// workgroup per (batch, head).
__global__ void __launch_bounds__(256) dg_finish_kernel(float* dg, const float* chunk_r, const float* dS_T,
                                                        const float* S_T, int64_t T, int H, int N) {
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
}

hipError_t launch_bwd_chunks(const BwdArgs& a, int out_bf16, hipStream_t st) {
  const dim3 grid((unsigned)(a.B * a.H * a.n_chunks)), block(256);
  if (out_bf16) hipLaunchKernelGGL((bwd_chunk_kernel<bf16>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((bwd_chunk_kernel<float>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dg_finish(float* dg, const float* chunk_r, const float* dS_T, const float* S_T, int64_t B,
                            int64_t T, int H, int n_chunks, hipStream_t st) {
  if (n_chunks > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dg_finish_kernel, dim3((unsigned)(B * H)), dim3(256), 0, st, dg, chunk_r, dS_T, S_T, T, H,
                     n_chunks);
  return hipGetLastError();
}

}  // namespace gla
