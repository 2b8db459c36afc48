// Chunk walk kernels of the Simple GLA mixer for gfx950.
//
// One workgroup (4 waves) walks the chunks of one (batch, head, dv-slice,
// segment) in order, keeping the recurrent state in matrix-core accumulators.
// Chunk formulation (chunks of 128 tokens, "Adaptaciones para AWS Trainium2",
// item 1, of the page "Cómo i14 llevó Laplace 3B a AWS Trainium2"): with b_i
// the running sum of the log-decay inside the chunk, Lambda_i = e^{b_i},
// Gamma = e^{b_last}, kappa_j = e^{b_last - b_j}, M_ij = e^{b_i - b_j} (j <= i),
//     O   = (Q K^T (.) M) V + diag(Lambda) Q S_n
//     S_n+1 = Gamma S_n + (diag(kappa) K)^T V
// which follows from unrolling S_t = e^{g_t} S_{t-1} + k_t^T v_t over the
// chunk.  The reverse walk of the backward carries the state gradient
//     dS_n = Gamma dS_n+1 + (diag(Lambda) Q)^T dO
// with the same code (X = Q, Y = dO, weights Lambda, chunks in reverse).
//
// The state is held transposed, Z^T[c][d], as 32x32 tiles (c rows, d cols)
// spread over the 4 waves.  Wave w owns the output rows (tokens) 32w..32w+31
// of each chunk.
//
// With bf16 inputs the inputs themselves are exact MFMA operands, but the
// intermediates (decay-masked scores, the bf16 copy of the fp32 state, the
// decay-weighted keys) are not: each is split into a bf16 value and its bf16
// residual and multiplied as two MFMAs (error-compensated 16-bit products, as
// the HEAL page "Problema" / "HEAL-B" sections describe for bf16 inference).
#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

template <int NC, bool OUT>
struct Own {
  // Z tiles t = cb*3 + db, contiguous ranges per wave.  With the output on,
  // waves with fewer causal score tiles take more state tiles.
  static constexpr int count(int w) {
    if (OUT) {
      if (NC == 3) return w == 0 ? 5 : w == 1 ? 3 : w == 2 ? 1 : 0;
      if (NC == 2) return w == 0 ? 3 : w == 1 ? 2 : w == 2 ? 1 : 0;
      if (NC == 1) return w == 0 ? 2 : w == 1 ? 1 : 0;
    } else {
      if (NC == 3) return w == 0 ? 3 : 2;
      if (NC == 2) return w < 2 ? 2 : 1;
      if (NC == 1) return w < 3 ? 1 : 0;
    }
    return 0;
  }
  static constexpr int first(int w) {
    int f = 0;
    for (int i = 0; i < w; ++i) f += count(i);
    return f;
  }
  static_assert(first(4) == 3 * NC, "every state tile needs an owner");
};

template <class T> struct Pad { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

template <class TIn, int NC, bool OUT>
struct WalkSmem {
  static constexpr int DVS = 32 * NC;
  static constexpr int PX = DK + Pad<TIn>::v;
  static constexpr int PY = DVS + (sizeof(TIn) == 2 ? 8 : 0);
  static constexpr int PZ = DVS + (sizeof(TIn) == 2 ? 8 : 0);
  TIn x[CH * PX];
  TIn y[CH * PY];
  TIn q[OUT ? CH * PX : 16];
  TIn z[DK * PZ];
  TIn zl[sizeof(TIn) == 2 ? DK * PZ : 16];   // residual of the bf16 state copy
  DecayLds dec;
};

// Rows [t0, t0+128) of a [B,T,H,D] tensor, columns [col0, col0+W), as 16-byte
// pieces held in registers; rows past T read as zero.
template <class T, int WCOLS>
struct TileRegs {
  static constexpr int EPP = 16 / sizeof(T);           // elements per piece
  static constexpr int PPR = WCOLS / EPP;              // pieces per row
  static constexpr int NP = CH * PPR;
  static constexpr int PER = (NP + 255) / 256;
  uint4 r[PER];
  __device__ __forceinline__ void load(const T* base, int64_t row_stride, int t0, int64_t T_len) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = threadIdx.x + 256 * i;
      const int row = p / PPR, cp = p % PPR;
      if (p < NP && t0 + row < T_len)
        r[i] = *(const uint4*)(base + (int64_t)(t0 + row) * row_stride + cp * EPP);
      else
        r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = threadIdx.x + 256 * i;
      if (p < NP) {
        const int row = p / PPR, cp = p % PPR;
        *(uint4*)(lds + row * PITCH + cp * EPP) = r[i];
      }
    }
  }
};

template <class TIn, class TOut, int NC, int MODE, int W>
__device__ __forceinline__ void walk_wave(const WalkArgs& a, WalkSmem<TIn, NC, MODE == WALK_FWD_OUT>& sm,
                                          int b, int h, int slice, int seg) {
  constexpr bool OUT = MODE == WALK_FWD_OUT;
  constexpr bool REV = MODE == WALK_REV;
  using S = WalkSmem<TIn, NC, OUT>;
  using FT = typename Frag<TIn>::type;
  constexpr int SUB = Frag<TIn>::SUB;
  constexpr int NT = Own<NC, OUT>::count(W);
  constexpr int T0 = Own<NC, OUT>::first(W);
  constexpr int DVS = 32 * NC;
  constexpr bool COMP = sizeof(TIn) == 2;

  const int lane = lane_id();
  const int g2 = lane >> 5;
  const int c0 = slice * DVS;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t T = a.T;
  const TIn* Xb = (const TIn*)a.X + (int64_t)b * T * a.H * DK + (int64_t)h * DK;
  const TIn* Yb = (const TIn*)a.Y + (int64_t)b * T * a.H * DV + (int64_t)h * DV + c0;
  const TIn* Qb = OUT ? (const TIn*)a.Q + (int64_t)b * T * a.H * DK + (int64_t)h * DK : nullptr;
  const float* gb = a.g + (int64_t)b * T * a.H + h;

  const int gseg = seg + a.seg_offset;
  const int n_begin = gseg * a.cps;
  const int n_end = min(a.n_chunks, n_begin + a.cps);
  const int nloc = n_end - n_begin;

  // ---- state tiles: load the initial state or start from zero
  f32x16 z[NT > 0 ? NT : 1];
  {
    const float* zi = a.zinit ? a.zinit + bh * a.zinit_bh_stride + (int64_t)gseg * a.zinit_seg_stride : nullptr;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        f32x4 v = zi ? load4f(zi + (int64_t)d * DV + c0 + 32 * cb + 8 * qq + 4 * g2) : f32x4{0, 0, 0, 0};
        z[t][4 * qq + 0] = v[0]; z[t][4 * qq + 1] = v[1];
        z[t][4 * qq + 2] = v[2]; z[t][4 * qq + 3] = v[3];
      }
    }
  }

  TileRegs<TIn, DK> px;
  TileRegs<TIn, DVS> py;
  TileRegs<TIn, OUT ? DK : 8> pq;
  float gx0 = 0.f, gx1 = 0.f;
  auto prefetch = [&](int n) {
    const int t0 = n * CH;
    px.load(Xb, (int64_t)a.H * DK, t0, T);
    py.load(Yb, (int64_t)a.H * DV, t0, T);
    if constexpr (OUT) pq.load(Qb, (int64_t)a.H * DK, t0, T);
    if (W == 0) {
      const int64_t ta = t0 + 2 * lane, tb = ta + 1;
      gx0 = ta < T ? gb[ta * a.H] : 0.f;
      gx1 = tb < T ? gb[tb * a.H] : 0.f;
    }
  };
  if (nloc > 0) prefetch(REV ? n_end - 1 : n_begin);

  float decay_sum = 0.f;
  const bool store_dc = a.st_dc != nullptr, store_cd = a.st_cd != nullptr;

  for (int it = 0; it < nloc; ++it) {
    const int n = REV ? n_end - 1 - it : n_begin + it;
    __syncthreads();
    px.template store<S::PX>(sm.x);
    py.template store<S::PY>(sm.y);
    if constexpr (OUT) pq.template store<S::PX>(sm.q);
    if (W == 0) build_decay(&sm.dec, gx0, gx1);
    if (OUT || store_dc || store_cd) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
        const int d = 32 * db + (lane & 31);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int off = d * S::PZ + 32 * cb + 8 * qq + 4 * g2;
          const f32x4 v4 = f32x4{z[t][4 * qq], z[t][4 * qq + 1], z[t][4 * qq + 2], z[t][4 * qq + 3]};
          if constexpr (COMP) store4_split((bf16*)sm.z + off, (bf16*)sm.zl + off, v4);
          else store4(sm.z + off, v4);
        }
      }
    }
    __syncthreads();
    decay_sum += sm.dec.blast;

    if constexpr (sizeof(TIn) == 2) {
      // Per-chunk state export for the backward, bf16 MFMA-operand order.
      if (store_dc || store_cd) {
        // per chunk: [hi fragments | lo fragments], DK*DV bf16 each
        const int64_t base = (bh * a.n_chunks + n) * (int64_t)(2 * DK * DV);
        if (store_dc) {  // fragments (db, kc): S[d = 32db + l%32][c = 16kc + 8g + e]
          constexpr int NF = 3 * (DVS / 16);
          for (int f = W; f < NF; f += 4) {
            const int db = f / (DVS / 16), kcl = f % (DVS / 16);
            const int kc = c0 / 16 + kcl;
            bf16* dst = (bf16*)a.st_dc + base + ((int64_t)(db * (DV / 16) + kc) * 64 + lane) * 8;
            *(bf16x8*)dst = frag_kcN((const bf16*)sm.z, S::PZ, 32 * db, 16 * kcl, 0);
            *(bf16x8*)(dst + DK * DV) = frag_kcN((const bf16*)sm.zl, S::PZ, 32 * db, 16 * kcl, 0);
          }
        }
        if (store_cd) {  // fragments (cb, kb, s): S[d = 32kb + k(s,e)][c = 32cb + l%32]
          constexpr int NF = NC * 6;
          for (int f = W; f < NF; f += 4) {
            const int cbl = f / 6, kb = (f % 6) / 2, s = f % 2;
            const int cb = c0 / 32 + cbl;
            bf16* dst = (bf16*)a.st_cd + base + ((int64_t)((cb * 3 + kb) * 2 + s) * 64 + lane) * 8;
            *(bf16x8*)dst = frag_kr((const bf16*)sm.z, S::PZ, 32 * kb, 32 * cbl, s);
            *(bf16x8*)(dst + DK * DV) = frag_kr((const bf16*)sm.zl, S::PZ, 32 * kb, 32 * cbl, s);
          }
        }
      }
    }

    if (it + 1 < nloc) prefetch(REV ? n - 1 : n + 1);

    if constexpr (OUT) {
      const int il = 32 * W + (lane & 31);          // this lane's token inside the chunk
      const float bi = sm.dec.b2[il];
      FT qn[3][SUB], qp[3][SUB];
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          qn[kb][s] = frag_kcN(sm.q, S::PX, 32 * W, 32 * kb, s);
          qp[kb][s] = frag_kcP(sm.q, S::PX, 32 * W, 32 * kb, s);
        }
      // Decay-masked scores P^T (keys j in rows, queries i in columns).
      FT pf[W + 1][SUB];
      FT pl[COMP ? W + 1 : 1][SUB];
#pragma unroll
      for (int J = 0; J <= W; ++J) {
        f32x16 acc = {};
#pragma unroll
        for (int kb = 0; kb < 3; ++kb)
#pragma unroll
          for (int s = 0; s < SUB; ++s)
            acc = mfma(frag_kcN(sm.x, S::PX, 32 * J, 32 * kb, s), qn[kb][s], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = 32 * J + out_row(r);
          const float w = exp2f(fminf(bi - sm.dec.b2[j], 0.f));
          acc[r] = (J < W || j <= il) ? acc[r] * w : 0.f;
        }
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          if constexpr (COMP) regs_to_frag_split(acc, s, pf[J][s], pl[J][s]);
          else pf[J][s] = acc[s];
        }
      }
      const float lam = sm.dec.lam[il];
      const int64_t trow = (int64_t)n * CH + il;
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        f32x16 o = {};
#pragma unroll
        for (int kb = 0; kb < 3; ++kb)
#pragma unroll
          for (int s = 0; s < SUB; ++s) {
            o = mfma(frag_kr(sm.z, S::PZ, 32 * kb, 32 * cb, s), qp[kb][s], o);
            if constexpr (COMP) o = mfma(frag_kr(sm.zl, S::PZ, 32 * kb, 32 * cb, s), qp[kb][s], o);
          }
        o *= lam;
#pragma unroll
        for (int J = 0; J <= W; ++J)
#pragma unroll
          for (int s = 0; s < SUB; ++s) {
            const FT ay = frag_kr(sm.y, S::PY, 32 * J, 32 * cb, s);
            o = mfma(ay, pf[J][s], o);
            if constexpr (COMP) o = mfma(ay, pl[J][s], o);
          }
        if (trow < T) {
          TOut* op = (TOut*)a.O + (((int64_t)b * T + trow) * a.H + h) * DV + c0 + 32 * cb + 4 * g2;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            store4(op + 8 * qq, f32x4{o[4 * qq], o[4 * qq + 1], o[4 * qq + 2], o[4 * qq + 3]});
        }
      }
    }

    // State update: Z^T = Gamma Z^T + Y^T (w X), contraction over the chunk's tokens.
    if constexpr (NT > 0) {
      const float gam = sm.dec.gam;
      const float* wts = REV ? sm.dec.lam : sm.dec.kap;
#pragma unroll
      for (int t = 0; t < NT; ++t) z[t] *= gam;
      constexpr int DB_LO = (NT >= 3) ? 0 : (T0 % 3);
      constexpr int DB_N = (NT >= 3) ? 3 : NT;   // contiguous db range (mod 3) when NT < 3
#pragma unroll
      for (int J = 0; J < 4; ++J) {
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          FT bx[3], bl[3];
#pragma unroll
          for (int k = 0; k < DB_N; ++k) {
            const int db = (DB_LO + k) % 3;
            if constexpr (COMP)
              scale_k_split(frag_kr(sm.x, S::PX, 32 * J, 32 * db, s), wts + 32 * J, s, bx[db], bl[db]);
            else
              bx[db] = scale_k(frag_kr(sm.x, S::PX, 32 * J, 32 * db, s), wts + 32 * J, s);
          }
          FT ay = {};
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
            if (t == 0 || db == 0) ay = frag_kr(sm.y, S::PY, 32 * J, 32 * cb, s);
            z[t] = mfma(ay, bx[db], z[t]);
            if constexpr (COMP) z[t] = mfma(ay, bl[db], z[t]);
          }
        }
      }
    }
  }

  // ---- final state
  if (a.zfin && (a.zfin_only_seg < 0 || a.zfin_only_seg == gseg)) {
    float* zo = a.zfin + bh * a.zfin_bh_stride + (int64_t)gseg * a.zfin_seg_stride;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        store4(zo + (int64_t)d * DV + c0 + 32 * cb + 8 * qq + 4 * g2,
               f32x4{z[t][4 * qq], z[t][4 * qq + 1], z[t][4 * qq + 2], z[t][4 * qq + 3]});
    }
  }
  if (a.seg_decay && slice == 0 && threadIdx.x == 0)
    a.seg_decay[bh * a.seg_decay_bh_stride + gseg] = decay_sum;
}

template <class TIn, class TOut, int NC, int MODE>
__global__ void __launch_bounds__(256, 1) walk_kernel(WalkArgs a) {
  __shared__ WalkSmem<TIn, NC, MODE == WALK_FWD_OUT> sm;
  // Work item order: slice fastest, then segment, head, batch.  Consecutive
  // items are placed on the same XCD (the dispatcher deals workgroups to the
  // 8 XCDs round-robin), so the dv-slices of one head and neighbouring heads
  // share that XCD's L2.
  const int nwg = gridDim.x;
  int wid = blockIdx.x;
  if ((nwg & 7) == 0) wid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int slice = wid % a.ns;
  int rest = wid / a.ns;
  const int seg = rest % a.nseg_launch;
  rest /= a.nseg_launch;
  const int h = rest % a.H;
  const int b = rest / a.H;
  switch (threadIdx.x >> 6) {
    case 0: walk_wave<TIn, TOut, NC, MODE, 0>(a, sm, b, h, slice, seg); break;
    case 1: walk_wave<TIn, TOut, NC, MODE, 1>(a, sm, b, h, slice, seg); break;
    case 2: walk_wave<TIn, TOut, NC, MODE, 2>(a, sm, b, h, slice, seg); break;
    default: walk_wave<TIn, TOut, NC, MODE, 3>(a, sm, b, h, slice, seg); break;
  }
}

// Segment scan: buf[bh][s] holds the state change of segment s from a zero
// state (pass 1); replace it by the state entering segment s.  decay[bh][s] is
// the segment's total log2-decay.  Forward order starts from Z0, reverse order
// (rev != 0) from the last segment.
__global__ void __launch_bounds__(256) seg_scan_kernel(float* buf, const float* decay, const float* Z0,
                                                       int nseg, int rev) {
  const int64_t bh = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= DK * DV) return;
  f32x4 z = Z0 ? *(const f32x4*)(Z0 + bh * DK * DV + e) : f32x4{0, 0, 0, 0};
  for (int it = 0; it < nseg; ++it) {
    const int s = rev ? nseg - 1 - it : it;
    float* p = buf + (bh * nseg + s) * (int64_t)(DK * DV) + e;
    const f32x4 d = *(const f32x4*)p;
    *(f32x4*)p = z;
    if (it + 1 < nseg) z = exp2f(decay[bh * nseg + s]) * z + d;
  }
}

// ---------------------------------------------------------------------------
template <class TIn, class TOut, int NC, int MODE>
static hipError_t launch_one(const WalkArgs& a, int nwg, hipStream_t st) {
  hipLaunchKernelGGL((walk_kernel<TIn, TOut, NC, MODE>), dim3(nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, int variant, int nwg, hipStream_t st) {
  switch (variant) {
    case WV_FWD_OUT_BF16_BF16: return launch_one<bf16, bf16, 3, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_OUT_BF16_F32: return launch_one<bf16, float, 3, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_OUT_F32_F32: return launch_one<float, float, 2, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_OUT_F32_BF16: return launch_one<float, bf16, 2, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_STATE_BF16: return launch_one<bf16, float, 3, WALK_FWD_STATE>(a, nwg, st);
    case WV_FWD_STATE_F32: return launch_one<float, float, 2, WALK_FWD_STATE>(a, nwg, st);
    case WV_REV_BF16: return launch_one<bf16, float, 3, WALK_REV>(a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

int walk_slices(int variant) {
  switch (variant) {
    case WV_FWD_OUT_F32_F32: case WV_FWD_OUT_F32_BF16: case WV_FWD_STATE_F32: return DV / 64;
    default: return DV / 96;
  }
}

hipError_t launch_seg_scan(float* buf, const float* decay, const float* Z0, int64_t BH, int nseg, int rev,
                           hipStream_t st) {
  hipLaunchKernelGGL(seg_scan_kernel, dim3((DK * DV / 4 + 255) / 256, (unsigned)BH), dim3(256), 0, st, buf,
                     decay, Z0, nseg, rev);
  return hipGetLastError();
}

}  // namespace gla
