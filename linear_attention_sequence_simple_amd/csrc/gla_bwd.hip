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
// One workgroup (8 waves) per (batch, head, chunk).  Token block w (32
// tokens) is the column block of the result tiles dV^T[:, w] (wave w) and
// dQ^T[:, w], dK^T[:, w] (wave 4+w), so each lane ends up with one token and
// the q.dq / k.dk dot products need only a sum over its registers and one
// exchange with the other lane group.
// The masked scores and the stored states enter the products as compensated
// bf16 pairs (value + residual, two MFMAs); q, k, v, dO are exact bf16.
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

// Chunk tiles in LDS: q, k [128][96] and the two 96-wide halves of v, dO,
// all in the swizzled unpadded layout (swz96), so the row reads and the
// transposed reads are free of bank conflicts.
struct BwdSmem {
  bf16 q[CH * 96];
  bf16 k[CH * 96];
  bf16 v[2][CH * 96];
  bf16 dO[2][CH * 96];
  DecayLds dec;
  float r[CH];
};

// One chunk tile [128][W] of a [B,T,H,D] tensor into LDS (as 96-wide halves),
// rows past T as zero; all 512 threads.
template <int WIDTH>
__device__ __forceinline__ void stage_tile(bf16* lds, const bf16* base, int64_t row_stride, int64_t t0, int64_t T) {
  constexpr int PPR = WIDTH / 8, NP = CH * PPR, PER = NP / 512;
  uint4 r[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = threadIdx.x + 512 * i, row = p / PPR, cp = p % PPR;
    r[i] = (t0 + row < T) ? *(const uint4*)(base + (t0 + row) * row_stride + cp * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = threadIdx.x + 512 * i, row = p / PPR, cp = p % PPR;
    *(uint4*)(lds + (cp / 12) * (CH * 96) + swz96(row, (cp % 12) * 8)) = r[i];
  }
}

__device__ __forceinline__ bf16x8 gfrag(const bf16* base, int f) {
  return *(const bf16x8*)(base + ((int64_t)f * 64 + lane_id()) * 8);
}
// 32-column blocks of a 192-wide tile stored as two swizzled halves
__device__ __forceinline__ const bf16* half_of(const bf16 (*t)[CH * 96], int col0) { return t[col0 / 96]; }

// Masked score tile rows in register order, as compensated operand pairs.
struct PairFrag {
  bf16x8 hi[2], lo[2];
};

// ---- dV wave: P (query rows i >= 32W, key column tl) and dV^T[:, W]
template <class TOut, int W>
__device__ __forceinline__ void bwd_dv_wave(const BwdArgs& a, BwdSmem& sm, const bf16* dScd, int64_t tok, bool valid) {
  const int lane = lane_id(), g2 = lane >> 5;
  const int tl = 32 * W + (lane & 31);
  const float b_t = sm.dec.b2[tl];
  const float kap = sm.dec.kap[tl];
  PairFrag P[4];
#pragma unroll
  for (int I = W; I < 4; ++I) {
    f32x16 ap = {};
#pragma unroll
    for (int k = 0; k < 6; ++k)
      ap = mfma(sfrag_kcN(sm.q, 32 * I, 32 * (k >> 1), k & 1), sfrag_kcN(sm.k, 32 * W, 32 * (k >> 1), k & 1), ap);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * I + out_row(r);
      const float w = exp2f(fminf(sm.dec.b2[i] - b_t, 0.f));
      ap[r] = ((I > W) || (tl <= i)) ? ap[r] * w : 0.f;
    }
    split_tile(ap, 0, P[I].hi[0], P[I].lo[0]);
    split_tile(ap, 1, P[I].hi[1], P[I].lo[1]);
  }
  // keys of this block as B operands of the state term (plain order over d)
  bf16x8 kB[6];
#pragma unroll
  for (int k = 0; k < 6; ++k) kB[k] = sfrag_kcN(sm.k, 32 * W, 32 * (k >> 1), k & 1);
  // state-gradient fragments, 4 steps ahead over the 36 (c-block, d-step) pairs
  constexpr int L = 4;
  bf16x8 fh[36], fl[36];
#pragma unroll
  for (int f = 0; f < L; ++f) { fh[f] = gfrag(dScd, f); fl[f] = gfrag(dScd + DK * DV, f); }
#pragma unroll
  for (int cb = 0; cb < 6; ++cb) {
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int f = cb * 6 + k;
      if (f + L < 36) { fh[f + L] = gfrag(dScd, f + L); fl[f + L] = gfrag(dScd + DK * DV, f + L); }
      acc = mfma(fh[f], kB[k], acc);
      acc = mfma(fl[f], kB[k], acc);
    }
    acc *= kap;
    const bf16* dOh = half_of(sm.dO, 32 * cb);
#pragma unroll
    for (int I = W; I < 4; ++I)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ad = sfrag_kr(dOh, 32 * I, (32 * cb) % 96, s);
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

// State terms of dQ^T or dK^T for the three d-blocks: sum over the 12
// 16-wide c steps of fragments (hi, lo) from the workspace times a 192-wide
// LDS operand (rows of this wave's tokens), with the global fragments 4 steps
// ahead over the 36 (d-block, c-step) pairs.
__device__ __forceinline__ void state_terms(const bf16* frag, const bf16 (*y)[CH * 96], int row0, f32x16 (&acc)[3]) {
  constexpr int L = 4;
  bf16x8 fh[36], fl[36];
#pragma unroll
  for (int f = 0; f < L; ++f) { fh[f] = gfrag(frag, f); fl[f] = gfrag(frag + DK * DV, f); }
#pragma unroll
  for (int db = 0; db < 3; ++db) {
    acc[db] = f32x16{};
#pragma unroll
    for (int k = 0; k < 12; ++k) {
      const int f = db * 12 + k;
      if (f + L < 36) { fh[f + L] = gfrag(frag, f + L); fl[f + L] = gfrag(frag + DK * DV, f + L); }
      const int c0 = 32 * (k >> 1);
      const bf16x8 bo = sfrag_kcN(half_of(y, c0), row0, c0 % 96, k & 1);
      acc[db] = mfma(fh[f], bo, acc[db]);
      acc[db] = mfma(fl[f], bo, acc[db]);
    }
  }
}

// Masked dP^T tile (key rows of block J, query column tl) when TRANSPOSED,
// else the masked dP tile (query rows of block J, key column tl), as a
// compensated operand pair.
template <bool TRANSPOSED>
__device__ __forceinline__ PairFrag dp_tile(const BwdSmem& sm, int J, int W, int tl, float b_t) {
  const bf16(*ra)[CH * 96] = TRANSPOSED ? sm.v : sm.dO;
  const bf16(*rb)[CH * 96] = TRANSPOSED ? sm.dO : sm.v;
  f32x16 ad = {};
#pragma unroll
  for (int k = 0; k < 12; ++k) {
    const int c0 = 32 * (k >> 1);
    ad = mfma(sfrag_kcN(half_of(ra, c0), 32 * J, c0 % 96, k & 1), sfrag_kcN(half_of(rb, c0), 32 * W, c0 % 96, k & 1), ad);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 32 * J + out_row(r);
    // dP^T[j][tl] needs j <= tl, weight 2^(b_tl - b_j); dP[j][tl] needs tl <= j
    const float w = TRANSPOSED ? exp2f(fminf(b_t - sm.dec.b2[j], 0.f)) : exp2f(fminf(sm.dec.b2[j] - b_t, 0.f));
    const bool keep = TRANSPOSED ? ((J < W) || (j <= tl)) : ((J > W) || (tl <= j));
    ad[r] = keep ? ad[r] * w : 0.f;
  }
  PairFrag D;
  split_tile(ad, 0, D.hi[0], D.lo[0]);
  split_tile(ad, 1, D.hi[1], D.lo[1]);
  return D;
}

// ---- dQ/dK wave: dP^T -> dQ^T[:, W], dP -> dK^T[:, W], and q.dq - k.dk
template <class TOut, int W>
__device__ __forceinline__ void bwd_dqk_wave(const BwdArgs& a, BwdSmem& sm, const bf16* Sdc, const bf16* dSdc,
                                             int64_t tok, bool valid) {
  const int lane = lane_id(), g2 = lane >> 5;
  const int tl = 32 * W + (lane & 31);
  const float b_t = sm.dec.b2[tl];
  float r = 0.f;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    // part 0: dQ^T = diag(Lambda) (S_n dO^T-term) + K^T dP^T;  part 1: dK^T = diag(kappa) (...) + Q^T dP
    const bool isq = part == 0;
    f32x16 acc[3];
    state_terms(isq ? Sdc : dSdc, isq ? sm.dO : sm.v, 32 * W, acc);
    const float sc = isq ? sm.dec.lam[tl] : sm.dec.kap[tl];
#pragma unroll
    for (int db = 0; db < 3; ++db) acc[db] *= sc;
    const bf16* xo = isq ? sm.k : sm.q;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (isq ? (J > W) : (J < W)) continue;
      const PairFrag D = isq ? dp_tile<true>(sm, J, W, tl, b_t) : dp_tile<false>(sm, J, W, tl, b_t);
#pragma unroll
      for (int db = 0; db < 3; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ax = sfrag_kr(xo, 32 * J, 32 * db, s);
          acc[db] = mfma(ax, D.hi[s], acc[db]);
          acc[db] = mfma(ax, D.lo[s], acc[db]);
        }
    }
    const bf16* xs = isq ? sm.q : sm.k;
    TOut* out = (TOut*)(isq ? a.dq : a.dk) + tok * DK + 4 * g2;
    float rr = 0.f;
#pragma unroll
    for (int db = 0; db < 3; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const bf16x4 xv = *(const LDS_AS bf16x4*)(to_lds(xs) + swz96(tl, 32 * db + 8 * qq + 4 * g2));
#pragma unroll
        for (int e = 0; e < 4; ++e) rr += (float)xv[e] * acc[db][4 * qq + e];
      }
      if (valid) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          store4(out + 32 * db + 8 * qq,
                 f32x4{acc[db][4 * qq], acc[db][4 * qq + 1], acc[db][4 * qq + 2], acc[db][4 * qq + 3]});
      }
    }
    r += isq ? rr : -rr;
  }
  r += __shfl_xor(r, 32, 64);
  if (lane < 32) sm.r[tl] = valid ? r : 0.f;
}

template <class TOut, int WV>
__device__ __forceinline__ void bwd_wave(const BwdArgs& a, BwdSmem& sm, int64_t bh, int64_t b, int h, int n) {
  constexpr int W = WV & 3;                        // token block
  const int lane = lane_id();
  const int64_t T = a.T;
  const int64_t trow = (int64_t)n * CH + 32 * W + (lane & 31);
  const bool valid = trow < T;
  const int64_t tok = ((int64_t)b * T + trow) * a.H + h;
  // per chunk: [hi fragments | lo fragments]
  const int64_t frag_base = (bh * a.n_chunks + n) * (int64_t)(2 * DK * DV);
  if constexpr (WV < 4)
    bwd_dv_wave<TOut, W>(a, sm, (const bf16*)a.ds_cd + frag_base, tok, valid);
  else
    bwd_dqk_wave<TOut, W>(a, sm, (const bf16*)a.s_dc + frag_base, (const bf16*)a.ds_dc + frag_base, tok, valid);
}

template <class TOut>
__global__ void __launch_bounds__(512, 1) bwd_chunk_kernel(BwdArgs a) {
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
  stage_tile<DK>(sm.q, (const bf16*)a.q + b * T * rsx + h * DK, rsx, t0, T);
  stage_tile<DK>(sm.k, (const bf16*)a.k + b * T * rsx + h * DK, rsx, t0, T);
  stage_tile<DV>(sm.v[0], (const bf16*)a.v + b * T * rsy + h * DV, rsy, t0, T);
  stage_tile<DV>(sm.dO[0], (const bf16*)a.dO + b * T * rsy + h * DV, rsy, t0, T);
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
    case 3: bwd_wave<TOut, 3>(a, sm, bh, b, h, n); break;
    case 4: bwd_wave<TOut, 4>(a, sm, bh, b, h, n); break;
    case 5: bwd_wave<TOut, 5>(a, sm, bh, b, h, n); break;
    case 6: bwd_wave<TOut, 6>(a, sm, bh, b, h, n); break;
    default: bwd_wave<TOut, 7>(a, sm, bh, b, h, n); break;
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
  const dim3 grid((unsigned)(a.B * a.H * a.n_chunks)), block(512);
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
