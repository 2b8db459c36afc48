// Chunk walk kernels of the Simple GLA mixer for gfx950.
//
// One workgroup walks the chunks of one (batch, head, dv-slice, segment) in
// order, keeping the recurrent state in matrix-core accumulators.
// Chunk formulation (chunks of 128 tokens, "Adaptaciones para AWS Trainium2",
// item 1, of the page "Cómo i14 llevó Laplace 3B a AWS Trainium2"): with b_i
// the running sum of the log-decay inside the chunk, Lambda_i = e^{b_i},
// Gamma = e^{b_last}, kappa_j = e^{b_last - b_j}, M_ij = e^{b_i - b_j} (j <= i),
//     O   = (Q K^T (.) M) V + diag(Lambda) Q S_n
//     S_n+1 = Gamma S_n + (diag(kappa) K)^T V
// which follows from unrolling S_t = e^{g_t} S_{t-1} + k_t^T v_t over the
// chunk.  The walks read their tensors through strided views (batch, head,
// token and slice strides), so the backward runs the same kernels on other
// operand roles and, with negative token strides, backwards in time.
//
// The state is held transposed, Z^T[c][d], as 32x32 tiles (c rows, d cols)
// spread over the "state" waves.  The prefill with output runs 8 waves, two
// per SIMD: output wave w (0..3) owns the tokens 32w..32w+31 of each chunk
// (scores, state read-out, P V) and state wave 4+u updates a share of the
// state tiles; the shares are uneven so that each SIMD's pair of waves has
// about the same matrix-core work.  The state-only walks run 4 state waves.
//
// With bf16 inputs the inputs themselves are exact MFMA operands, but the
// intermediates (decay-masked scores, the bf16 copy of the fp32 state, the
// decay-weighted keys) are not: each is split into a bf16 value and its bf16
// residual and multiplied as two MFMAs (the error-compensated 16-bit products
// of section "B. Mitigando o Truncamento de GEMM via Compensação de Erro
// Algébrica" on the page "Resumo Técnico: Desmistificando a Instabilidade
// Numérica na Inferência de LLMs com HEAL").
#include <type_traits>

#include "gla_common.h"
#include "gla_kernels.h"

namespace gla {

template <int MODE>
struct WalkShape {
  static constexpr bool OUT = MODE == WALK_FWD_OUT;
  static constexpr int WAVES = OUT ? 8 : 4;
  static constexpr int THREADS = 64 * WAVES;
};

template <int NC, bool OUT>
struct Own {
  // State tiles t = cb*3 + db owned by state wave u, contiguous ranges.  With
  // the output on, state wave u shares a SIMD with output wave u, whose work
  // grows with u.
  static constexpr int count(int u) {
    if (OUT) {
      // bf16: output wave w's products grow with w, so the state tiles go
      // 3, 3, 2, 1 over the SIMDs (measured best); fp32: every SIMD gets a
      // second active wave to overlap the output wave's stalls
      if (NC == 3) return u < 2 ? 3 : u == 2 ? 2 : 1;
      if (NC == 2) return u == 0 ? 3 : u == 1 ? 2 : u == 2 ? 1 : 0;
      if (NC == 1) return u < 3 ? 1 : 0;
    } else {
      if (NC == 3) return u == 0 ? 3 : 2;
      if (NC == 2) return u < 2 ? 2 : 1;
      if (NC == 1) return u < 3 ? 1 : 0;
    }
    return 0;
  }
  static constexpr int first(int u) {
    int f = 0;
    for (int i = 0; i < u; ++i) f += count(i);
    return f;
  }
  static_assert(first(4) == 3 * NC, "every state tile needs an owner");
};

template <class T> struct Pad { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

template <class TIn, int NC, bool OUT>
struct WalkSmem {
  static constexpr bool COMP = sizeof(TIn) == 2;   // bf16 inputs: compensated intermediates
  static constexpr int DVS = 32 * NC;
  // bf16 tiles use the swizzled unpadded [rows][96] layout (swz96); fp32
  // tiles are padded row-major.
  static_assert(!COMP || DVS == 96, "the swizzled bf16 layout assumes 96 columns");
  static constexpr int PX = COMP ? DK : DK + Pad<TIn>::v;
  static constexpr int PY = DVS;
  static constexpr int PZ = DVS;
  static constexpr int PQ = DK;                    // fp32 queries: unpadded (LDS budget)
  // The bf16 state-only walks read only the weighted keys and the values, so
  // they keep no raw keys and no state copy: about 76 KB, two workgroups per
  // compute unit.
  static constexpr bool RAWX = OUT || !COMP;
  TIn x[RAWX ? CH * PX : 8];              // keys, as loaded
  TIn xh[COMP ? CH * PX : 8];             // decay-weighted keys: bf16 value ...
  TIn xl[COMP ? CH * PX : 8];             // ... and bf16 residual
  TIn y[CH * PY];                         // values (reverse walk: dO), this dv-slice
  TIn q[(OUT && COMP) ? CH * PQ : 8];     // queries (the fp32 output waves read theirs from memory)
  TIn z[OUT ? DK * PZ : 8];               // state entering the chunk, [d][c]
  TIn zl[(OUT && COMP) ? DK * PZ : 8];    // residual of its bf16 copy
  // Decay tables of the current chunk and of the next one (built a chunk
  // ahead).
  static constexpr int NDEC = 2;
  DecayLds dec[NDEC];
  // utab[U(I) + j] = 2^{b_{32I} - b_j} for j < 32I (I = 1, 2, 3; U = 0, 32, 96):
  // the key-side factor of the decay between token blocks.
  float utab[NDEC][OUT ? 192 : 4];
};

__device__ __forceinline__ int utab_off(int I) { return I == 1 ? 0 : I == 2 ? 32 : 96; }

// Rows [t0, t0+nrows) of a strided token view start, in memory order, at
// tile_base = base + (t0 + rref) * stride with rref = nrows-1 for a negative
// stride (time read backwards) and 0 otherwise; row r, column c then sits at
// the non-negative byte offset row_offset from it.  The base is the same for
// the whole workgroup and the offset fits 32 bits, which keeps the per-lane
// address in one register.
template <class T>
__device__ __forceinline__ const char* tile_base(const T* base, int64_t stride, int64_t t0, int nrows) {
  return (const char*)(base + (t0 + (stride < 0 ? nrows - 1 : 0)) * stride);
}
template <class T>
__device__ __forceinline__ uint32_t row_offset(int r, int c, int64_t stride, int nrows) {
  return (uint32_t)(((r - (stride < 0 ? nrows - 1 : 0)) * (int)stride + c) * (int)sizeof(T));
}

// Rows [t0, t0+128) of a token view, as 16-byte pieces held in registers;
// rows past T read as zero.
template <class T, int WCOLS, int NTHR>
struct TileRegs {
  // loader threads are numbered 0..NTHR-1 (the state waves of the workgroup)
  static constexpr int EPP = 16 / sizeof(T);           // elements per piece
  static constexpr int PPR = WCOLS / EPP;              // pieces per row
  static constexpr int NP = CH * PPR;
  static constexpr int PER = (NP + NTHR - 1) / NTHR;
  uint4 r[PER];
  // The pieces with index i of all threads cover rows (NTHR i)/PPR onwards, a
  // group of at most GROWS rows.  Each load takes a workgroup-uniform address
  // (the group's first row in memory order) and a 32-bit lane offset that is
  // the same in every chunk, so no per-chunk 64-bit address arithmetic runs
  // on the vector units; GROWS <= 32 keeps the offset within the 32-row bound
  // the views guarantee.
  static constexpr int group_rows() {
    int m = 0;
    for (int i = 0; i < PER; ++i) {
      const int rows = (NTHR * i + NTHR - 1) / PPR - (NTHR * i) / PPR + 1;
      m = rows > m ? rows : m;
    }
    return m;
  }
  static constexpr int GROWS = group_rows();
  static_assert(GROWS <= 32, "a piece group must stay within 32 rows");
  __device__ __forceinline__ void load_piece(int i, const T* base, int64_t row_stride, int t0, int64_t T_len) {
    const int p = (threadIdx.x & (NTHR - 1)) + NTHR * i;
    const int row = p / PPR, cp = p % PPR;
    const int g0 = (NTHR * i) / PPR;
    const char* gb = tile_base(base, row_stride, (int64_t)t0 + g0, GROWS);
    const uint32_t off = row_offset<T>(row - g0, cp * EPP, row_stride, GROWS);
    r[i] = (p < NP && t0 + row < T_len) ? *(const uint4*)(gb + off) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void load(const T* base, int64_t row_stride, int t0, int64_t T_len) {
#pragma unroll
    for (int i = 0; i < PER; ++i) load_piece(i, base, row_stride, t0, T_len);
  }
  template <int PITCH>
  __device__ __forceinline__ void store(T* lds) const {
    const int tid = threadIdx.x & (NTHR - 1);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = tid + NTHR * i;
      if (p < NP) {
        const int row = p / PPR, cp = p % PPR;
        const int off = (sizeof(T) == 2) ? swz96(row, cp * EPP) : row * PITCH + cp * EPP;
        *(uint4*)(lds + off) = r[i];
      }
    }
  }
  // bf16 rows scaled by w[row], stored as compensated hi/lo copies.
  template <int PITCH>
  __device__ __forceinline__ void store_weighted(bf16* hi, bf16* lo, const float* w) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) store_weighted_piece(i, hi, lo, w);
  }
  __device__ __forceinline__ void store_weighted_piece(int i, bf16* hi, bf16* lo, const float* w) const {
    {
      const int p = (threadIdx.x & (NTHR - 1)) + NTHR * i;
      if (p < NP) {
        const int row = p / PPR, cp = p % PPR;
        const float s = w[row];
        const uint32_t u[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
        float f[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[2 * k] = bf16_lo_f(u[k]) * s;
          f[2 * k + 1] = bf16_hi_f(u[k]) * s;
        }
        bf16x8 h8, l8;
        split8(f, h8, l8);
        *(bf16x8*)(hi + swz96(row, cp * EPP)) = h8;
        *(bf16x8*)(lo + swz96(row, cp * EPP)) = l8;
      }
    }
  }
};

// The tokens of walk b: first token, length and chunk count.  PACKED walks
// take them from the sequence offsets, the others from the launch.
struct SeqSpan {
  int64_t t0, T;
  int n_chunks;
};
template <bool PACKED>
__device__ __forceinline__ SeqSpan seq_span(const WalkArgs& a, int b) {
  if constexpr (!PACKED) {
    return SeqSpan{0, a.T, a.n_chunks};
  } else {
    const int64_t t0 = min(max((int64_t)a.cu[b], (int64_t)0), a.cu_total);
    const int64_t end = min(max((int64_t)a.cu[b + 1], t0), min(a.cu_total, t0 + a.T));
    const int64_t T = end - t0;
    return SeqSpan{t0, T, (int)((T + CH - 1) / CH)};
  }
}
// Row of batch-head (b, h) in a state view, through the slot indices idx of
// packed walks.
template <bool PACKED>
__device__ __forceinline__ int64_t state_row(const int32_t* idx, int b, int h, int H) {
  if constexpr (PACKED) return (int64_t)(idx ? idx[b] : b) * H + h;
  return (int64_t)b * H + h;
}

template <class TIn, class TOut, int NC, int MODE, int W, bool PACKED, bool GATED>
__device__ __forceinline__ void walk_wave(const WalkArgs& a, WalkSmem<TIn, NC, MODE == WALK_FWD_OUT>& sm,
                                          int b, int h, int slice, int seg) {
  constexpr bool OUT = MODE == WALK_FWD_OUT;
  using S = WalkSmem<TIn, NC, OUT>;
  using FT = typename Frag<TIn>::type;
  constexpr int SUB = Frag<TIn>::SUB;
  constexpr bool OUTW = OUT && W < 4;                // output wave (else: state wave)
  constexpr int U = OUT ? W - 4 : W;                  // index among the state waves
  constexpr int NT = OUTW ? 0 : Own<NC, OUT>::count(U);
  constexpr int T0 = OUTW ? 0 : Own<NC, OUT>::first(U);
  constexpr int DVS = 32 * NC;
  constexpr bool COMP = S::COMP;
  constexpr int NTHR = 256;                           // loader threads: the 4 state waves
  constexpr bool LOADER = !OUTW;
  static_assert(!(OUT && COMP), "the bf16 walks with output run prefill_wave");

  const int lane = lane_id();
  const int g2 = lane >> 5;
  const int64_t bh = (int64_t)b * a.H + h;
  const SeqSpan sq = seq_span<PACKED>(a, b);
  const int64_t T = sq.T;
  const TIn* Xb = (const TIn*)a.X.p + b * a.X.sb + sq.t0 * a.X.st + h * a.X.sh + slice * a.X.ss;
  const TIn* Yb = (const TIn*)a.Y.p + b * a.Y.sb + sq.t0 * a.Y.st + h * a.Y.sh + slice * a.Y.ss;
  const TIn* Qb = OUT ? (const TIn*)a.Q.p + b * a.Q.sb + sq.t0 * a.Q.st + h * a.Q.sh + slice * a.Q.ss : nullptr;
  const float* gb = a.g + b * a.gsb + sq.t0 * a.gst + h * a.gsh;

  const int gseg = seg + a.seg_offset;
  const int n_begin = a.chunk0 + gseg * a.cps;
  const int n_end = min(sq.n_chunks, n_begin + a.cps);
  const int nloc = PACKED ? max(0, n_end - n_begin) : n_end - n_begin;   // packed: past a sequence's end, 0

  // ---- state tiles Z^T (c rows, d columns): initial state or zero
  f32x16 z[NT > 0 ? NT : 1];
  {
    const StateView& zv = a.zinit;
    const float* zi = zv.p ? zv.p + state_row<PACKED>(a.zinit_idx, b, h, a.H) * zv.sbh + (int64_t)gseg * zv.sseg + slice * zv.ss : nullptr;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = 32 * cb + 8 * qq + 4 * g2;
        if (!zi) {
          for (int e = 0; e < 4; ++e) z[t][4 * qq + e] = 0.f;
        } else if (zv.sy == 1) {              // 4 consecutive y: one 16-byte access
          const f32x4 v = load4f(zi + d * zv.sx + c);
          for (int e = 0; e < 4; ++e) z[t][4 * qq + e] = v[e];
        } else {                              // consecutive lanes are consecutive in memory
          for (int e = 0; e < 4; ++e) z[t][4 * qq + e] = zi[d * zv.sx + (c + e) * zv.sy];
        }
      }
    }
  }

  // DEPTH register buffers of chunk tiles: chunk it+DEPTH is requested while
  // chunk it is processed.  The state-only bf16 walks have little arithmetic
  // to hide memory behind and the registers for two buffers; the others keep
  // one.  The chunk loop is unrolled by two so that each buffer keeps its
  // registers (copies would force early waits).
  constexpr int DEPTH = (!OUT && COMP) ? 2 : 1;
  TileRegs<TIn, DK, NTHR> px[DEPTH];
  TileRegs<TIn, DVS, NTHR> py[DEPTH];
  auto prefetch = [&](auto bc, int n) {
    constexpr int B = decltype(bc)::value % DEPTH;
    const int t0 = n * CH;
    if constexpr (LOADER) {
      px[B].load(Xb, a.X.st, t0, T);
      py[B].load(Yb, a.Y.st, t0, T);
    }
  };
  constexpr std::integral_constant<int, 0> I0{};
  constexpr std::integral_constant<int, 1> I1{};
  // log-decay of chunk n for wave 0: tokens 2l, 2l+1 and the mirrored
  // 127-2l, 126-2l; zero past T
  float gx0 = 0.f, gx1 = 0.f, gm0 = 0.f, gm1 = 0.f;
  auto load_g = [&](int n) {
    if (W == 0) {
      const int64_t t0 = (int64_t)n * CH;
      const int64_t ta = t0 + 2 * lane, tb = ta + 1, tc = t0 + 127 - 2 * lane, td = tc - 1;
      const int sh = a.gshift;
      gx0 = (ta < T && ta >= sh) ? gb[(ta - sh) * a.gst] : 0.f;
      gx1 = (tb < T && tb >= sh) ? gb[(tb - sh) * a.gst] : 0.f;
      gm0 = (tc < T && tc >= sh) ? gb[(tc - sh) * a.gst] : 0.f;
      gm1 = (td < T && td >= sh) ? gb[(td - sh) * a.gst] : 0.f;
    }
  };
  // An fp32 output wave's 32 query rows as MFMA B operands in register order
  // (sub-step s of block kb: column 32 kb + 8 (s/4) + 4 g + s%4), read from
  // memory a chunk ahead, four consecutive contraction values per 16-byte
  // load; rows past T read as zero.
  float qn[OUTW ? 3 : 1][16];
  auto load_qn = [&](int n) {
    if constexpr (OUTW) {
      const int64_t t = (int64_t)n * CH + 32 * W + (lane & 31);
      const bool live = t < T;
      const float* p = (const float*)Qb + (live ? t : 0) * a.Q.st + 4 * g2;
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 v = live ? load4f(p + 32 * kb + 8 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) qn[kb][4 * i + e] = v[e];
        }
    }
  };
  auto step_of = [&](int i) { return n_begin + i; };
  if (nloc > 0) {
    prefetch(I0, step_of(0));
    load_qn(step_of(0));
    if (DEPTH == 2 && nloc > 1) prefetch(I1, step_of(1));
    load_g(step_of(0));
    if (W == 0) build_decay(&sm.dec[0], gx0, gx1, gm0, gm1, OUT ? sm.utab[0] : nullptr);
    if (nloc > 1) load_g(step_of(1));
  }

  float decay_sum = 0.f;

  auto body = [&](auto bc, int it) {
    constexpr int B = decltype(bc)::value % DEPTH;    // register buffer of this chunk
    const int n = step_of(it);
    const int cur = it & 1;                            // decay-table buffer of this chunk
    DecayLds& dc = sm.dec[cur];
    __syncthreads();            // previous chunk's LDS reads done; this chunk's decay tables visible
    if constexpr (LOADER) {
      if constexpr (S::RAWX) px[B].template store<S::PX>(sm.x);
      py[B].template store<S::PY>(sm.y);
      if constexpr (COMP)
        px[B].template store_weighted<S::PX>((bf16*)sm.xh, (bf16*)sm.xl, dc.kap);
    }
    // chunk it+DEPTH goes into this buffer now that it is staged
    if (it + DEPTH < nloc) prefetch(bc, step_of(it + DEPTH));
    if constexpr (OUT) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
        const int d = 32 * db + (lane & 31);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const f32x4 v4 = f32x4{z[t][4 * qq], z[t][4 * qq + 1], z[t][4 * qq + 2], z[t][4 * qq + 3]};
          store4(sm.z + d * S::PZ + 32 * cb + 8 * qq + 4 * g2, v4);
        }
      }
    }
    __syncthreads();                                   // tiles and state copy visible
    decay_sum += dc.blast;


    if constexpr (OUTW) {
      const int il = 32 * W + (lane & 31);          // this lane's token inside the chunk
      const float bi = dc.b2[il];
      // Decay-masked scores P^T (keys j in rows, queries i in columns), all
      // key blocks at once.  Off the diagonal 2^{b_i - b_j} =
      // 2^{b_i - b_{32W}} 2^{b_{32W} - b_j}, both factors <= 1.
      // The fp32 products run in groups of 4 contraction sub-steps (48 steps
      // over the 96-wide keys, 16 per 32-token block of P), the operands of
      // group i+1 requested before the products of group i and the schedule
      // fenced between groups: unfenced, the compiler requests every operand
      // of a loop up front and spills.
      static_assert(SUB == 16, "the walk with output here is the fp32 one");
      f32x16 acc[W + 1];
#pragma unroll
      for (int J = 0; J <= W; ++J) acc[J] = f32x16{};
      {
        // the 4 sub-steps of a group are 4 consecutive key columns: one
        // 16-byte read per key block
        f32x4 xa[2][W + 1];
        const LDS_AS float* xl = (const LDS_AS float*)sm.x + (lane & 31) * S::PX + 4 * g2;
        auto load_x = [&](int buf, int grp) {
#pragma unroll
          for (int J = 0; J <= W; ++J)
            xa[buf][J] = *(const LDS_AS f32x4*)(xl + 32 * J * S::PX + 32 * (grp >> 2) + 8 * (grp & 3));
        };
        load_x(0, 0);
#pragma unroll
        for (int grp = 0; grp < 12; ++grp) {
          if (grp + 1 < 12) load_x((grp + 1) & 1, grp + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int J = 0; J <= W; ++J) acc[J] = mfma(xa[grp & 1][J][e], qn[grp >> 2][4 * (grp & 3) + e], acc[J]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      FT pf[W + 1][SUB];
      const float ri = W > 0 ? exp2f(bi - dc.b2[32 * W]) : 1.f;
#pragma unroll
      for (int J = 0; J <= W; ++J) {
        if (J < W) {
          const float* u = sm.utab[cur] + utab_off(W) + 32 * J + 4 * g2;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x4 uu = *(const f32x4*)(u + 8 * qq);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[J][4 * qq + e] *= uu[e] * ri;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * J + out_row(r);
            const float w = exp2f(fminf(bi - dc.b2[j], 0.f));
            acc[J][r] = j <= il ? acc[J][r] * w : 0.f;
          }
        }
#pragma unroll
        for (int s = 0; s < SUB; ++s) pf[J][s] = acc[J][s];
      }
      // Outputs of all dv blocks at once: O^T = diag(Lambda) (Z^T Q^T) + V^T P^T.
      f32x16 o[NC];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) o[cb] = f32x16{};
      {
        float za[2][NC][4];
        auto load_z = [&](int buf, int grp) {
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) za[buf][cb][e] = frag_kr(sm.z, S::PZ, 32 * (grp >> 2), 32 * cb, 4 * (grp & 3) + e);
        };
        load_z(0, 0);
#pragma unroll
        for (int grp = 0; grp < 12; ++grp) {
          if (grp + 1 < 12) load_z((grp + 1) & 1, grp + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) o[cb] = mfma(za[grp & 1][cb][e], qn[grp >> 2][4 * (grp & 3) + e], o[cb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the queries are dead: request the next chunk's
      if (it + 1 < nloc) load_qn(step_of(it + 1));
      const float lam = exp2f(dc.b2[il]);
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) o[cb] *= lam;
      {
        constexpr int NG = 4 * (W + 1);                  // groups of 4 sub-steps over the key blocks
        float ya[2][NC][4];
        auto load_y = [&](int buf, int grp) {
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) ya[buf][cb][e] = frag_kr(sm.y, S::PY, 32 * (grp >> 2), 32 * cb, 4 * (grp & 3) + e);
        };
        load_y(0, 0);
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) {
          if (grp + 1 < NG) load_y((grp + 1) & 1, grp + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) o[cb] = mfma(ya[grp & 1][cb][e], pf[grp >> 2][4 * (grp & 3) + e], o[cb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int64_t trow = (int64_t)n * CH + il;
      if (a.acc.p && trow < T) {
        // add a partial sum of the same outputs (fp32, computed by another
        // walk over the other half of a contraction)
        const float* ap = (const float*)a.acc.p + b * a.acc.sb + sq.t0 * a.acc.st + h * a.acc.sh + trow * a.acc.st +
                          slice * a.acc.ss + 4 * g2;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x4 v = load4f(ap + 32 * cb + 8 * qq);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[cb][4 * qq + e] += v[e];
          }
      }
      if (GATED && trow < T) {
        // output gate: this lane's token row, the same columns as its outputs
        const TIn* gp = (const TIn*)a.G.p + b * a.G.sb + sq.t0 * a.G.st + h * a.G.sh + trow * a.G.st +
                        slice * a.G.ss + 4 * g2;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x4 gv = load4f(gp + 32 * cb + 8 * qq);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[cb][4 * qq + e] = gate_silu(o[cb][4 * qq + e], gv[e]);
          }
      }
      if (trow < T) {
        TOut* op = (TOut*)a.O.p + b * a.O.sb + sq.t0 * a.O.st + h * a.O.sh + trow * a.O.st + slice * a.O.ss + 4 * g2;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            store4(op + 32 * cb + 8 * qq,
                   f32x4{o[cb][4 * qq], o[cb][4 * qq + 1], o[cb][4 * qq + 2], o[cb][4 * qq + 3]});
      }
    }

    // State update: Z^T = Gamma Z^T + Y^T (w X), contraction over the chunk's tokens.
    if constexpr (NT > 0) {
      const float gam = dc.gam;
      const float* wts = dc.kap;
#pragma unroll
      for (int t = 0; t < NT; ++t) z[t] *= gam;
      constexpr int DB_LO = (NT >= 3) ? 0 : (T0 % 3);
      constexpr int DB_N = (NT >= 3) ? 3 : NT;   // contiguous db range (mod 3) when NT < 3
      if constexpr (COMP) {
        // Software-pipelined over the 8 (J, s) contraction steps.
        constexpr int CB_LO = T0 / 3, NCB = (T0 + NT - 1) / 3 - CB_LO + 1;
        bf16x8 bx[2][3], bl[2][3], ay[2][NCB];
        auto load_ops = [&](int buf, int k) {
          const int J = k >> 1, s = k & 1;
#pragma unroll
          for (int q = 0; q < DB_N; ++q) {
            const int db = (DB_LO + q) % 3;
            bx[buf][db] = sfrag_kr((const bf16*)sm.xh, 32 * J, 32 * db, s);
            bl[buf][db] = sfrag_kr((const bf16*)sm.xl, 32 * J, 32 * db, s);
          }
#pragma unroll
          for (int c = 0; c < NCB; ++c) ay[buf][c] = sfrag_kr((const bf16*)sm.y, 32 * J, 32 * (CB_LO + c), s);
        };
        load_ops(0, 0);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int cur = k & 1;
          if (k + 1 < 8) load_ops(cur ^ 1, k + 1);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
            z[t] = mfma(ay[cur][cb - CB_LO], bx[cur][db], z[t]);
            z[t] = mfma(ay[cur][cb - CB_LO], bl[cur][db], z[t]);
          }
        }
      } else {
        // fp32: 4 groups of 4 sub-steps per 32-token block J, pipelined and
        // fenced like the output products; the J loop is not unrolled, so
        // the fragment addresses are formed once per block (unrolled, their
        // base registers alone spill).
        constexpr int CB_LO = T0 / 3, NCB = (T0 + NT - 1) / 3 - CB_LO + 1;
        float bxa[2][3][4], aya[2][NCB][4];
        auto load_s = [&](int buf, int J, int grp) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int s = 4 * grp + e;
#pragma unroll
            for (int k = 0; k < DB_N; ++k) {
              const int db = (DB_LO + k) % 3;
              bxa[buf][db][e] = scale_k(frag_kr(sm.x, S::PX, 32 * J, 32 * db, s), wts + 32 * J, s);
            }
#pragma unroll
            for (int c = 0; c < NCB; ++c) aya[buf][c][e] = frag_kr(sm.y, S::PY, 32 * J, 32 * (CB_LO + c), s);
          }
        };
        load_s(0, 0, 0);
#pragma unroll 1
        for (int J = 0; J < 4; ++J) {
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            if (grp + 1 < 4) load_s((grp + 1) & 1, J, grp + 1);
            else if (J + 1 < 4) load_s(0, J + 1, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
                z[t] = mfma(aya[grp & 1][cb - CB_LO][e], bxa[grp & 1][db][e], z[t]);
              }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    // Decay tables of the next chunk, after this wave's arithmetic so that
    // its log-decay loads (issued an iteration ago) have arrived; they are
    // published by the next iteration's first barrier.
    if (W == 0 && it + 1 < nloc) {
      build_decay(&sm.dec[cur ^ 1], gx0, gx1, gm0, gm1, OUT ? sm.utab[cur ^ 1] : nullptr);
      if (it + 2 < nloc) load_g(step_of(it + 2));
    }
  };
  if constexpr (DEPTH == 2) {
    for (int it = 0; it < nloc; it += 2) {
      body(I0, it);
      if (it + 1 < nloc) body(I1, it + 1);
    }
  } else {
    for (int it = 0; it < nloc; ++it) body(I0, it);
  }

  // ---- final state
  if (a.zfin.p && (a.zfin_only_seg < 0 || a.zfin_only_seg == gseg)) {
    const StateView& zv = a.zfin;
    float* zo = zv.p + state_row<PACKED>(a.zfin_idx, b, h, a.H) * zv.sbh + (int64_t)gseg * zv.sseg + slice * zv.ss;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = 32 * cb + 8 * qq + 4 * g2;
        if (zv.sy == 1) {
          store4(zo + d * zv.sx + c, f32x4{z[t][4 * qq], z[t][4 * qq + 1], z[t][4 * qq + 2], z[t][4 * qq + 3]});
        } else {
          for (int e = 0; e < 4; ++e) zo[d * zv.sx + (c + e) * zv.sy] = z[t][4 * qq + e];
        }
      }
    }
  }
  if (a.seg_decay && slice == 0 && threadIdx.x == 0)
    a.seg_decay[bh * a.seg_decay_bh_stride + gseg] = decay_sum;
}

// bf16 prefill with output: 8 waves.  For chunk n (decay tables dec[n&1]):
//   phase 1  output waves: decay-masked scores P from their 32 queries (in
//                          registers, read from memory a chunk ahead) and
//                          the keys, and
//                          O = diag(Lambda) (Q S_n) from the published bf16
//                          value/residual copy of S_n; wave 0 then builds
//                          the decay tables of chunk n+1 in the other buffer
//            state waves:  stage the values and the decay-weighted keys of
//                          chunk n and request chunk n+1's values and keys
//   barrier
//   phase 2  output waves: O += P V, request their queries of chunk n+1,
//                          store O
//            state waves:  S_n+1 = Gamma S_n + (diag(kappa) K)^T V, publish
//                          S_n+1, stage the keys of chunk n+1
//   barrier
// Every LDS tile is read in one phase only and rewritten in the other, so
// one buffer of each suffices (the decay tables, read in phase 1 and built
// there for the next chunk, have two) and the staging
// overlaps the products.  All tiles are read from memory with row-contiguous
// 16-byte accesses, spread over both phases so that the workgroups on the
// chip keep the memory busy instead of all loading at the same moment.  The
// query rows of the LDS tile serve only the bf16 output's transpose.
template <class TOut, int W, bool PACKED, bool GATED, bool ACC>
__device__ __forceinline__ void prefill_wave(const WalkArgs& a, WalkSmem<bf16, 3, true>& sm, int b, int h,
                                             int slice, int seg) {
  using S = WalkSmem<bf16, 3, true>;
  constexpr int NC = 3;
  constexpr int DVS = 96;
  constexpr bool OUTW = W < 4;                        // output wave (else: state wave)
  constexpr int U = OUTW ? 0 : W - 4;                 // index among the state waves
  constexpr int NT = OUTW ? 0 : Own<NC, true>::count(U);
  constexpr int T0 = OUTW ? 0 : Own<NC, true>::first(U);
  constexpr int NTHR = 256;                           // loader threads: the 4 state waves

  const int lane = lane_id();
  const int g2 = lane >> 5;
  const int64_t bh = (int64_t)b * a.H + h;
  const SeqSpan sq = seq_span<PACKED>(a, b);
  const int64_t T = sq.T;
  const bf16* Xb = (const bf16*)a.X.p + b * a.X.sb + sq.t0 * a.X.st + h * a.X.sh + slice * a.X.ss;
  const bf16* Yb = (const bf16*)a.Y.p + b * a.Y.sb + sq.t0 * a.Y.st + h * a.Y.sh + slice * a.Y.ss;
  const bf16* Qb = (const bf16*)a.Q.p + b * a.Q.sb + sq.t0 * a.Q.st + h * a.Q.sh + slice * a.Q.ss;
  const float* gb = a.g + b * a.gsb + sq.t0 * a.gst + h * a.gsh;
  const int gseg = seg + a.seg_offset;
  const int n_begin = a.chunk0 + gseg * a.cps;
  const int n_end = min(sq.n_chunks, n_begin + a.cps);
  const int nloc = PACKED ? max(0, n_end - n_begin) : n_end - n_begin;   // packed: past a sequence's end, 0

  // ---- state tiles Z^T (c rows, d columns): initial state or zero
  f32x16 z[NT > 0 ? NT : 1];
  {
    const StateView& zv = a.zinit;
    const float* zi = zv.p ? zv.p + state_row<PACKED>(a.zinit_idx, b, h, a.H) * zv.sbh + (int64_t)gseg * zv.sseg + slice * zv.ss : nullptr;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = 32 * cb + 8 * qq + 4 * g2;
        if (!zi) {
          for (int e = 0; e < 4; ++e) z[t][4 * qq + e] = 0.f;
        } else if (zv.sy == 1) {              // 4 consecutive y: one 16-byte access
          const f32x4 v = load4f(zi + d * zv.sx + c);
          for (int e = 0; e < 4; ++e) z[t][4 * qq + e] = v[e];
        } else {                              // consecutive lanes are consecutive in memory
          for (int e = 0; e < 4; ++e) z[t][4 * qq + e] = zi[d * zv.sx + (c + e) * zv.sy];
        }
      }
    }
  }

  TileRegs<bf16, DK, NTHR> px;                          // keys of the chunk being staged
  TileRegs<bf16, DVS, NTHR> py;                         // and its values
  // an output wave's 32 query rows, read from memory a chunk ahead straight
  // into the plain-order MFMA B operands (lane l: row l%32, columns
  // 32 kb + 16 s + 8 (l/32) .. +7): 6 pieces of 16 bytes at immediate offsets
  // from one 32-bit lane offset, under one row check (per-piece offsets would
  // be held as 64-bit values across the chunk loop and spilled)
  bf16x8 qcur[OUTW ? 3 : 1][2];
  auto load_q = [&](int n) {
    if constexpr (OUTW) {
      const int64_t t0 = (int64_t)n * CH + 32 * W;
      const char* p = tile_base(Qb, a.Q.st, t0, 32) + row_offset<bf16>(lane & 31, 8 * g2, a.Q.st, 32);
      const bool live = t0 + (lane & 31) < T;
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s) qcur[kb][s] = live ? *(const bf16x8*)(p + 2 * (32 * kb + 16 * s)) : bf16x8{};
    }
  };
  // publish the state as a bf16 value/residual pair
  auto publish = [&]() {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int off = swz96(d, 32 * cb + 8 * qq + 4 * g2);
        store4_split((bf16*)sm.z + off, (bf16*)sm.zl + off,
                     f32x4{z[t][4 * qq], z[t][4 * qq + 1], z[t][4 * qq + 2], z[t][4 * qq + 3]});
      }
    }
  };
  // log-decay of chunk n for wave 0: tokens 2l, 2l+1 and the mirrored
  // 127-2l, 126-2l; zero past T
  float gx0 = 0.f, gx1 = 0.f, gm0 = 0.f, gm1 = 0.f;
  auto load_g = [&](int n) {
    if (W == 0) {
      const int64_t t0 = (int64_t)n * CH;
      const int64_t ta = t0 + 2 * lane, tb = ta + 1, tc = t0 + 127 - 2 * lane, td = tc - 1;
      const int sh = a.gshift;
      gx0 = (ta < T && ta >= sh) ? gb[(ta - sh) * a.gst] : 0.f;
      gx1 = (tb < T && tb >= sh) ? gb[(tb - sh) * a.gst] : 0.f;
      gm0 = (tc < T && tc >= sh) ? gb[(tc - sh) * a.gst] : 0.f;
      gm1 = (td < T && td >= sh) ? gb[(td - sh) * a.gst] : 0.f;
    }
  };

  if (nloc > 0) {
    if constexpr (!OUTW) {
      px.load(Xb, a.X.st, n_begin * CH, T);
      py.load(Yb, a.Y.st, n_begin * CH, T);
    }
    load_q(n_begin);
    load_g(n_begin);
    if (W == 0) build_decay(&sm.dec[0], gx0, gx1, gm0, gm1, sm.utab[0]);
    if (nloc > 1) load_g(n_begin + 1);
    publish();
    if constexpr (!OUTW) px.template store<S::PX>(sm.x);
  }
  __syncthreads();

  float decay_sum = 0.f;
  for (int it = 0; it < nloc; ++it) {
    const int n = n_begin + it;
    const int cur = it & 1;
    const DecayLds& dc = sm.dec[cur];
    decay_sum += dc.blast;

    // ================= phase 1
    f32x16 o[NC];
    bf16x8 pf[OUTW ? W + 1 : 1][2], pl[OUTW ? W + 1 : 1][2];
    float gam = 0.f;
    if constexpr (OUTW) {
      const int il = 32 * W + (lane & 31);            // this lane's token inside the chunk
      const float bi = dc.b2[il];
      // O^T = diag(Lambda) (Z^T Q^T), operands of step k+1 requested before
      // the products of step k
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) o[cb] = f32x16{};
      bf16x8 zh[2][NC], zlo[2][NC];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) {
        zh[0][cb] = sfrag_krN((const bf16*)sm.z, 0, 32 * cb, 0);
        zlo[0][cb] = sfrag_krN((const bf16*)sm.zl, 0, 32 * cb, 0);
      }
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const int bf = k & 1, kb = k >> 1, s = k & 1;
        if (k + 1 < 6) {
#pragma unroll
          for (int cb = 0; cb < NC; ++cb) {
            zh[bf ^ 1][cb] = sfrag_krN((const bf16*)sm.z, 32 * ((k + 1) >> 1), 32 * cb, (k + 1) & 1);
            zlo[bf ^ 1][cb] = sfrag_krN((const bf16*)sm.zl, 32 * ((k + 1) >> 1), 32 * cb, (k + 1) & 1);
          }
        }
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
          o[cb] = mfma(zh[bf][cb], qcur[kb][s], o[cb]);
          o[cb] = mfma(zlo[bf][cb], qcur[kb][s], o[cb]);
        }
        __builtin_amdgcn_sched_barrier(0);   // one step of operands in flight
      }
      const float lam = exp2f(dc.b2[il]);
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) o[cb] *= lam;
      // wave 0 has the least product work: it builds the next chunk's decay
      // tables here (that buffer's readers finished in the previous chunk)
      if (W == 0 && it + 1 < nloc) {
        build_decay(&sm.dec[cur ^ 1], gx0, gx1, gm0, gm1, sm.utab[cur ^ 1]);
        if (it + 2 < nloc) load_g(n + 2);
      }
      // Decay-masked scores P^T (keys j in rows, queries i in columns).  Off
      // the diagonal 2^{b_i - b_j} = 2^{b_i - b_{32W}} 2^{b_{32W} - b_j}.
      f32x16 acc[W + 1];
#pragma unroll
      for (int J = 0; J <= W; ++J) acc[J] = f32x16{};
      {
        bf16x8 xk[2][W + 1];
#pragma unroll
        for (int J = 0; J <= W; ++J) xk[0][J] = sfrag_kcN(sm.x, 32 * J, 0, 0);
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          const int bf = k & 1, kb = k >> 1, s = k & 1;
          if (k + 1 < 6) {
#pragma unroll
            for (int J = 0; J <= W; ++J) xk[bf ^ 1][J] = sfrag_kcN(sm.x, 32 * J, 32 * ((k + 1) >> 1), (k + 1) & 1);
          }
#pragma unroll
          for (int J = 0; J <= W; ++J) acc[J] = mfma(xk[bf][J], qcur[kb][s], acc[J]);
          __builtin_amdgcn_sched_barrier(0);   // one step of operands in flight
        }
      }
      const float ri = W > 0 ? exp2f(bi - dc.b2[32 * W]) : 1.f;
#pragma unroll
      for (int J = 0; J <= W; ++J) {
        if (J < W) {
          const float* u = sm.utab[cur] + utab_off(W) + 32 * J + 4 * g2;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x4 uu = *(const f32x4*)(u + 8 * qq);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[J][4 * qq + e] *= uu[e] * ri;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = 32 * J + out_row(r);
            const float w = exp2f(fminf(bi - dc.b2[j], 0.f));
            acc[J][r] = j <= il ? acc[J][r] * w : 0.f;
          }
        }
        split_tile(acc[J], 0, pf[J][0], pl[J][0]);
        split_tile(acc[J], 1, pf[J][1], pl[J][1]);
      }
    } else {
      gam = dc.gam;
      py.template store<S::PY>(sm.y);
      if (it + 1 < nloc) py.load(Yb, a.Y.st, (n + 1) * CH, T);
#pragma unroll
      for (int i = 0; i < decltype(px)::PER; ++i) {
        px.store_weighted_piece(i, (bf16*)sm.xh, (bf16*)sm.xl, dc.kap);
        if (it + 1 < nloc) px.load_piece(i, Xb, a.X.st, (n + 1) * CH, T);
      }
    }
    __syncthreads();                                   // weighted keys and values visible; queries, keys, state copy and tables read

    // ================= phase 2
    if constexpr (OUTW) {
      // O^T += V^T P^T.  A gated walk requests this lane's gate (its token
      // row, the same columns as its outputs) before the last key block's
      // products, once the earlier blocks' P operands are dead (requested
      // earlier, the gate's registers spill).
      constexpr int NK = 2 * (W + 1);                   // (J, s) steps
      bf16x8 yv[2][NC];
      bf16x4 gt[GATED ? NC : 1][4];
      const int64_t grow = (int64_t)n * CH + 32 * W + (lane & 31);
      // ACC walks add a partial sum of the same outputs (fp32, computed by
      // another walk over the other half of a contraction): this lane's row
      // is requested before the last key block's products (any earlier, its
      // 48 registers spill)
      f32x4 av[ACC ? NC : 1][4];
#pragma unroll
      for (int cb = 0; cb < NC; ++cb) yv[0][cb] = sfrag_kr(sm.y, 0, 32 * cb, 0);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const int bf = k & 1, J = k >> 1, s = k & 1;
        if (ACC && k == NK - 1) {
          const bool live = grow < T;
          const float* ap = (const float*)a.acc.p + b * a.acc.sb + sq.t0 * a.acc.st + h * a.acc.sh +
                            (live ? grow : 0) * a.acc.st + 4 * g2;
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) av[cb][qq] = live ? load4f(ap + 32 * cb + 8 * qq) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (GATED && k == NK - 2) {
          const bool live = grow < T;
          const bf16* gp = (const bf16*)a.G.p + b * a.G.sb + sq.t0 * a.G.st + h * a.G.sh +
                           (live ? grow : 0) * a.G.st + slice * a.G.ss + 4 * g2;
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) gt[cb][qq] = live ? *(const bf16x4*)(gp + 32 * cb + 8 * qq) : bf16x4{};
        }
        if (k + 1 < NK) {
#pragma unroll
          for (int cb = 0; cb < NC; ++cb) yv[bf ^ 1][cb] = sfrag_kr(sm.y, 32 * ((k + 1) >> 1), 32 * cb, (k + 1) & 1);
        }
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
          o[cb] = mfma(yv[bf][cb], pf[J][s], o[cb]);
          o[cb] = mfma(yv[bf][cb], pl[J][s], o[cb]);
        }
      }
      if constexpr (ACC) {
        // add the partial sum and, when asked, write the dot product of each
        // output row with a row of D
        const int64_t trow = grow;
        const bool live = trow < T;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[cb][4 * qq + e] += av[cb][qq][e];
        if (a.rdot.p) {
          const bf16* dp = (const bf16*)a.D.p + b * a.D.sb + sq.t0 * a.D.st + h * a.D.sh + trow * a.D.st + 4 * g2;
          float r = 0.f;
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const bf16x4 dv = live ? *(const bf16x4*)(dp + 32 * cb + 8 * qq) : bf16x4{};
#pragma unroll
              for (int e = 0; e < 4; ++e) r += (float)dv[e] * o[cb][4 * qq + e];
            }
          r += __shfl_xor(r, 32, 64);
          if (g2 == 0 && live)
            ((float*)a.rdot.p)[b * a.rdot.sb + (sq.t0 + trow) * a.rdot.st + h * a.rdot.sh] = r;
        }
      }
      if constexpr (GATED) {
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[cb][4 * qq + e] = gate_silu(o[cb][4 * qq + e], (float)gt[cb][qq][e]);
      }
      if constexpr (std::is_same<TOut, bf16>::value) {
        // Through this wave's own rows of the query tile (free until the
        // next phase 1; the wave's LDS accesses execute in order): written
        // in the accumulator layout, read back and stored as row-contiguous
        // 16-byte pieces.
        bf16* ot = sm.q + 32 * W * 96;
        const bf16* ob = (const bf16*)a.O.p + b * a.O.sb + sq.t0 * a.O.st + h * a.O.sh + slice * a.O.ss;
        const int64_t t0 = (int64_t)n * CH + 32 * W;
        char* tile = const_cast<char*>(tile_base(ob, a.O.st, t0, 32));
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            store4(ot + swz96(lane & 31, 32 * cb + 8 * qq + 4 * g2),
                   f32x4{o[cb][4 * qq], o[cb][4 * qq + 1], o[cb][4 * qq + 2], o[cb][4 * qq + 3]});
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          const int p = lane + 64 * i, row = p / 12, cp = p % 12;
          const uint4 v = *(const uint4*)(ot + swz96(row, cp * 8));
          if (t0 + row < T) *(uint4*)(tile + row_offset<bf16>(row, cp * 8, a.O.st, 32)) = v;
        }
      } else {
        const int64_t trow = (int64_t)n * CH + 32 * W + (lane & 31);
        if (trow < T) {
          TOut* op = (TOut*)a.O.p + b * a.O.sb + sq.t0 * a.O.st + h * a.O.sh + trow * a.O.st + slice * a.O.ss + 4 * g2;
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              store4(op + 32 * cb + 8 * qq,
                     f32x4{o[cb][4 * qq], o[cb][4 * qq + 1], o[cb][4 * qq + 2], o[cb][4 * qq + 3]});
        }
      }
      // the next chunk's query loads (24 registers) after the products and stores
      __builtin_amdgcn_sched_barrier(0);
      if (it + 1 < nloc) load_q(n + 1);
    } else {
      // Z^T = Gamma Z^T + V^T (kappa K), over the 8 (token block, half) steps
#pragma unroll
      for (int t = 0; t < NT; ++t) z[t] *= gam;
      constexpr int DB_LO = (NT >= 3) ? 0 : (T0 % 3);
      constexpr int DB_N = (NT >= 3) ? 3 : NT;        // contiguous db range (mod 3) when NT < 3
      constexpr int CB_LO = T0 / 3, NCB = (T0 + NT - 1) / 3 - CB_LO + 1;
      bf16x8 bx[2][3], bl[2][3], ay[2][NCB];
      auto load_ops = [&](int buf, int k) {
        const int J = k >> 1, s = k & 1;
#pragma unroll
        for (int q = 0; q < DB_N; ++q) {
          const int db = (DB_LO + q) % 3;
          bx[buf][db] = sfrag_kr((const bf16*)sm.xh, 32 * J, 32 * db, s);
          bl[buf][db] = sfrag_kr((const bf16*)sm.xl, 32 * J, 32 * db, s);
        }
#pragma unroll
        for (int c = 0; c < NCB; ++c) ay[buf][c] = sfrag_kr(sm.y, 32 * J, 32 * (CB_LO + c), s);
      };
      load_ops(0, 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int bf = k & 1;
        if (k + 1 < 8) load_ops(bf ^ 1, k + 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
          z[t] = mfma(ay[bf][cb - CB_LO], bx[bf][db], z[t]);
          z[t] = mfma(ay[bf][cb - CB_LO], bl[bf][db], z[t]);
        }
      }
      if (it + 1 < nloc) {
        publish();
        px.template store<S::PX>(sm.x);
      }
    }
    __syncthreads();                                   // next chunk's keys, tables and state copy visible
  }

  // ---- final state
  if (a.zfin.p && (a.zfin_only_seg < 0 || a.zfin_only_seg == gseg)) {
    const StateView& zv = a.zfin;
    float* zo = zv.p + state_row<PACKED>(a.zfin_idx, b, h, a.H) * zv.sbh + (int64_t)gseg * zv.sseg + slice * zv.ss;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb = (T0 + t) / 3, db = (T0 + t) % 3;
      const int d = 32 * db + (lane & 31);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = 32 * cb + 8 * qq + 4 * g2;
        if (zv.sy == 1) {
          store4(zo + d * zv.sx + c, f32x4{z[t][4 * qq], z[t][4 * qq + 1], z[t][4 * qq + 2], z[t][4 * qq + 3]});
        } else {
          for (int e = 0; e < 4; ++e) zo[d * zv.sx + (c + e) * zv.sy] = z[t][4 * qq + e];
        }
      }
    }
  }
  if (a.seg_decay && slice == 0 && threadIdx.x == 0)
    a.seg_decay[bh * a.seg_decay_bh_stride + gseg] = decay_sum;
}

// Packed launches of at most 64 sequences walk the longest sequences first:
// the dispatcher starts workgroups in launch order, so a long sequence left
// to the end of the launch would still run after the rest of the chip has
// gone idle.  Returns the sequence of rank i in decreasing length (ties in
// index order), computed by every wave from the offsets: lane c holds
// sequence c's length and counts the sequences that precede it.
__device__ __forceinline__ int longest_first(const WalkArgs& a, int i) {
  if (a.B > 64) return i;
  const int lane = threadIdx.x & 63;
  const bool live = lane < a.B;
  const long long len = live ? (long long)a.cu[lane + 1] - a.cu[lane] : -1;
  int rank = 0;
  for (int j = 0; j < 64; ++j) {
    const long long lj = __shfl(len, j, 64);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  const unsigned long long pick = __ballot(live && rank == i);
  return __ffsll(pick) - 1;
}

// The walk of workgroup `local` of a launch of `nwg` workgroups.
template <class TIn, class TOut, int NC, int MODE, bool PACKED = false, bool GATED = false, bool ACC = false>
__device__ __forceinline__ void walk_block(const WalkArgs& a, WalkSmem<TIn, NC, MODE == WALK_FWD_OUT>& sm, int local,
                                           int nwg) {
  // Work item order: slice fastest, then segment, head, batch.  Equal-length
  // walks place consecutive items on the same XCD (the dispatcher deals
  // workgroups to the 8 XCDs round-robin), so the dv-slices of one head and
  // neighbouring heads share that XCD's L2.
  int wid = local;
  if constexpr (PACKED) {
    // Sequences of different lengths: the dv-slices of one head stay on one
    // XCD (workgroups l and l+8 share one) and consecutive heads go to
    // consecutive XCDs, so every XCD gets an even share of every sequence
    // and starts its work in launch order (longest sequences first).
    const int y = local >> 3;
    if (nwg % (8 * a.ns) == 0) wid = ((y / a.ns) * 8 + (local & 7)) * a.ns + y % a.ns;
  } else if ((nwg & 7) == 0) {
    wid = (local & 7) * (nwg >> 3) + (local >> 3);
  }
  const int slice = wid % a.ns;
  int rest = wid / a.ns;
  const int seg = rest % a.nseg_launch;
  rest /= a.nseg_launch;
  const int h = rest % a.H;
  int b = rest / a.H;
  if constexpr (PACKED) b = longest_first(a, b);
  if constexpr (MODE == WALK_FWD_OUT && std::is_same<TIn, bf16>::value) {
    switch (threadIdx.x >> 6) {
      case 0: prefill_wave<TOut, 0, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      case 1: prefill_wave<TOut, 1, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      case 2: prefill_wave<TOut, 2, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      case 3: prefill_wave<TOut, 3, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      case 4: prefill_wave<TOut, 4, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      case 5: prefill_wave<TOut, 5, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      case 6: prefill_wave<TOut, 6, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
      default: prefill_wave<TOut, 7, PACKED, GATED, ACC>(a, sm, b, h, slice, seg); break;
    }
    return;
  } else {
  switch (threadIdx.x >> 6) {
    case 0: walk_wave<TIn, TOut, NC, MODE, 0, PACKED, GATED>(a, sm, b, h, slice, seg); break;
    case 1: walk_wave<TIn, TOut, NC, MODE, 1, PACKED, GATED>(a, sm, b, h, slice, seg); break;
    case 2: walk_wave<TIn, TOut, NC, MODE, 2, PACKED, GATED>(a, sm, b, h, slice, seg); break;
    case 3: walk_wave<TIn, TOut, NC, MODE, 3, PACKED, GATED>(a, sm, b, h, slice, seg); break;
    default:
      if constexpr (WalkShape<MODE>::WAVES == 8) {
        switch (threadIdx.x >> 6) {
          case 4: walk_wave<TIn, TOut, NC, MODE, 4, PACKED, GATED>(a, sm, b, h, slice, seg); break;
          case 5: walk_wave<TIn, TOut, NC, MODE, 5, PACKED, GATED>(a, sm, b, h, slice, seg); break;
          case 6: walk_wave<TIn, TOut, NC, MODE, 6, PACKED, GATED>(a, sm, b, h, slice, seg); break;
          default: walk_wave<TIn, TOut, NC, MODE, 7, PACKED, GATED>(a, sm, b, h, slice, seg); break;
        }
      }
      break;
  }
  }
}


// The bf16 state-only walks fit two workgroups per compute unit (LDS), so
// they are built for two waves per SIMD (256 registers each).
template <class TIn, int MODE>
constexpr int walk_waves_per_eu() { return (MODE == WALK_FWD_STATE && sizeof(TIn) == 2) ? 2 : 1; }

template <class TIn, class TOut, int NC, int MODE, bool PACKED, bool GATED>
__global__ void __launch_bounds__(WalkShape<MODE>::THREADS, (walk_waves_per_eu<TIn, MODE>())) walk_kernel(WalkArgs a) {
  __shared__ WalkSmem<TIn, NC, MODE == WALK_FWD_OUT> sm;
  walk_block<TIn, TOut, NC, MODE, PACKED, GATED>(a, sm, (int)blockIdx.x, (int)gridDim.x);
}

// Two independent state walks of one kind side by side: workgroups [0, nwg0)
// run a0, the rest a1.  Each walk orders its own workgroups; the XCD
// placement matches the dispatcher's when nwg0 is a multiple of 8.
template <class TIn, int NC>
__global__ void __launch_bounds__(WalkShape<WALK_FWD_STATE>::THREADS, (walk_waves_per_eu<TIn, WALK_FWD_STATE>()))
    walk_pair_kernel(WalkArgs a0, WalkArgs a1, int nwg0) {
  __shared__ WalkSmem<TIn, NC, false> sm;
  if ((int)blockIdx.x < nwg0)
    walk_block<TIn, float, NC, WALK_FWD_STATE>(a0, sm, (int)blockIdx.x, nwg0);
  else
    walk_block<TIn, float, NC, WALK_FWD_STATE>(a1, sm, (int)blockIdx.x - nwg0, (int)gridDim.x - nwg0);
}

// Segment scan: buf[bh][s] holds the state change of segment s from a zero
// state (pass 1); replace it by the state entering segment s.  decay[bh][s] is
// the segment's total log2-decay.  Forward order starts from Z0, reverse order
// (rev != 0) from the last segment.
__global__ void __launch_bounds__(256) seg_scan_kernel(float* buf, const float* decay, const float* Z0,
                                                       const int32_t* z0_idx, int H, int nseg, int rev) {
  const int64_t bh = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= DK * DV) return;
  const int64_t zrow = z0_idx ? (int64_t)z0_idx[bh / H] * H + bh % H : bh;
  f32x4 z = Z0 ? *(const f32x4*)(Z0 + zrow * DK * DV + e) : f32x4{0, 0, 0, 0};
  // Entries in groups of 8: the group's state changes and decays are all
  // requested before its first store (each entry is read before it is
  // overwritten), instead of one memory latency per entry.
  constexpr int G = 8;
  for (int it0 = 0; it0 < nseg; it0 += G) {
    f32x4 d[G];
    float dec[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int it = it0 + j;
      if (it < nseg) {
        const int s = rev ? nseg - 1 - it : it;
        d[j] = *(const f32x4*)(buf + (bh * nseg + s) * (int64_t)(DK * DV) + e);
        dec[j] = decay[bh * nseg + s];
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int it = it0 + j;
      if (it < nseg) {
        const int s = rev ? nseg - 1 - it : it;
        *(f32x4*)(buf + (bh * nseg + s) * (int64_t)(DK * DV) + e) = z;
        if (it + 1 < nseg) z = exp2f(dec[j]) * z + d[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Packed walks and walks with an output gate are compile-time variants, so
// that the plain walks keep their registers.
template <class TIn, class TOut, int NC, int MODE>
static hipError_t launch_one(const WalkArgs& a, int nwg, hipStream_t st) {
  const dim3 grid(nwg), block(WalkShape<MODE>::THREADS);
  if (a.cu && a.G.p) return hipErrorInvalidValue;        // not a combination the library launches
  if constexpr (NC == 1) {                               // the fp32 backward's walks: plain views only
    if (a.cu || a.G.p) return hipErrorInvalidValue;
    hipLaunchKernelGGL((walk_kernel<TIn, TOut, NC, MODE, false, false>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  if (a.cu)
    hipLaunchKernelGGL((walk_kernel<TIn, TOut, NC, MODE, true, false>), grid, block, 0, st, a);
  else if (MODE == WALK_FWD_OUT && a.G.p)
    hipLaunchKernelGGL((walk_kernel<TIn, TOut, NC, MODE, false, MODE == WALK_FWD_OUT>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((walk_kernel<TIn, TOut, NC, MODE, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, int variant, int nwg, hipStream_t st) {
  // the bf16 walks add partial sums only in the pair launch built for it
  if (a.acc.p && (variant == WV_FWD_OUT_BF16_BF16 || variant == WV_FWD_OUT_BF16_F32)) return hipErrorInvalidValue;
  switch (variant) {
    case WV_FWD_OUT_BF16_BF16: return launch_one<bf16, bf16, 3, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_OUT_BF16_F32: return launch_one<bf16, float, 3, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_OUT_F32_F32: return launch_one<float, float, 2, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_OUT_F32_BF16: return launch_one<float, bf16, 2, WALK_FWD_OUT>(a, nwg, st);
    case WV_FWD_STATE_BF16: return launch_one<bf16, float, 3, WALK_FWD_STATE>(a, nwg, st);
    case WV_FWD_STATE_F32: return launch_one<float, float, 2, WALK_FWD_STATE>(a, nwg, st);
    case WV_OUT_F32_NC1: return launch_one<float, float, 1, WALK_FWD_OUT>(a, nwg, st);
    default: return hipErrorInvalidValue;
  }
}

template <class TOut, bool ACC>
__global__ void __launch_bounds__(WalkShape<WALK_FWD_OUT>::THREADS, 1)
    walk_out_pair_kernel(WalkArgs a0, WalkArgs a1, int nwg0) {
  __shared__ WalkSmem<bf16, 3, true> sm;
  if ((int)blockIdx.x < nwg0)
    walk_block<bf16, TOut, 3, WALK_FWD_OUT, false, false, ACC>(a0, sm, (int)blockIdx.x, nwg0);
  else
    walk_block<bf16, TOut, 3, WALK_FWD_OUT, false, false, ACC>(a1, sm, (int)blockIdx.x - nwg0, (int)gridDim.x - nwg0);
}

hipError_t launch_out_walk_pair(const WalkArgs& a0, int nwg0, const WalkArgs& a1, int nwg1, int out_bf16,
                                hipStream_t st) {
  const dim3 grid(nwg0 + nwg1), block(WalkShape<WALK_FWD_OUT>::THREADS);
  // both walks add partial sums (a compile-time variant), or neither
  if ((a0.acc.p != nullptr) != (a1.acc.p != nullptr)) return hipErrorInvalidValue;
  const bool acc = a0.acc.p != nullptr;
  if (out_bf16) {
    if (acc) hipLaunchKernelGGL((walk_out_pair_kernel<bf16, true>), grid, block, 0, st, a0, a1, nwg0);
    else hipLaunchKernelGGL((walk_out_pair_kernel<bf16, false>), grid, block, 0, st, a0, a1, nwg0);
  } else {
    if (acc) hipLaunchKernelGGL((walk_out_pair_kernel<float, true>), grid, block, 0, st, a0, a1, nwg0);
    else hipLaunchKernelGGL((walk_out_pair_kernel<float, false>), grid, block, 0, st, a0, a1, nwg0);
  }
  return hipGetLastError();
}

// Up to four bf16 walks with output in one launch, in two groups of two
// compile-time variants: workgroups [o[i], o[i+1]) run a[i]; a[0], a[1] as
// (TA, ACCA), a[2], a[3] as (TB, ACCB).  Walks with no workgroups are skipped.
struct WalkQuad {
  WalkArgs a[4];
  int o[5];
};

template <class TA, bool ACCA, class TB, bool ACCB>
__global__ void __launch_bounds__(WalkShape<WALK_FWD_OUT>::THREADS, 1) walk_out_quad_kernel(WalkQuad w) {
  __shared__ WalkSmem<bf16, 3, true> sm;
  const int x = (int)blockIdx.x;
  const int i = (x >= w.o[1]) + (x >= w.o[2]) + (x >= w.o[3]);
  const int local = x - w.o[i], nwg = w.o[i + 1] - w.o[i];
  // the walk's arguments read in place from the kernel-argument segment (the
  // parameter is its first and only explicit argument): indexing the
  // parameter itself would copy all four argument sets to scratch memory
  using KArgs = const __attribute__((address_space(4))) WalkQuad;
  const WalkArgs& a = *(const WalkArgs*)&((KArgs*)__builtin_amdgcn_kernarg_segment_ptr())->a[i];
  if (i < 2)
    walk_block<bf16, TA, 3, WALK_FWD_OUT, false, false, ACCA>(a, sm, local, nwg);
  else
    walk_block<bf16, TB, 3, WALK_FWD_OUT, false, false, ACCB>(a, sm, local, nwg);
}

hipError_t launch_out_walk_quad(const WalkArgs* a, const int* nwg, int kind, hipStream_t st) {
  WalkQuad w;
  w.o[0] = 0;
  for (int i = 0; i < 4; ++i) {
    if (nwg[i] < 0) return hipErrorInvalidValue;
    w.a[i] = a[i];
    w.o[i + 1] = w.o[i] + nwg[i];
  }
  // the walks of group A add partial sums exactly in the ACC kinds; group B never does
  const bool acc_a = kind == QUAD_ACC_F32_F32 || kind == QUAD_ACC_BF16_F32 || kind == QUAD_ACC_BF16_BF16;
  for (int i = 0; i < 4; ++i)
    if (nwg[i] > 0 && (a[i].acc.p != nullptr) != (i < 2 && acc_a)) return hipErrorInvalidValue;
  if (w.o[4] == 0) return hipSuccess;
  const dim3 grid(w.o[4]), block(WalkShape<WALK_FWD_OUT>::THREADS);
  switch (kind) {
    case QUAD_F32_F32: hipLaunchKernelGGL((walk_out_quad_kernel<float, false, float, false>), grid, block, 0, st, w); break;
    case QUAD_F32_BF16: hipLaunchKernelGGL((walk_out_quad_kernel<float, false, bf16, false>), grid, block, 0, st, w); break;
    case QUAD_ACC_F32_F32: hipLaunchKernelGGL((walk_out_quad_kernel<float, true, float, false>), grid, block, 0, st, w); break;
    case QUAD_ACC_BF16_F32: hipLaunchKernelGGL((walk_out_quad_kernel<bf16, true, float, false>), grid, block, 0, st, w); break;
    case QUAD_ACC_BF16_BF16: hipLaunchKernelGGL((walk_out_quad_kernel<bf16, true, bf16, false>), grid, block, 0, st, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_state_walk_pair(const WalkArgs& a0, int nwg0, const WalkArgs& a1, int nwg1, hipStream_t st) {
  hipLaunchKernelGGL((walk_pair_kernel<bf16, 3>), dim3(nwg0 + nwg1), dim3(WalkShape<WALK_FWD_STATE>::THREADS), 0,
                     st, a0, a1, nwg0);
  return hipGetLastError();
}

int walk_slices(int variant) {
  switch (variant) {
    case WV_FWD_OUT_F32_F32: case WV_FWD_OUT_F32_BF16: case WV_FWD_STATE_F32: return DV / 64;
    case WV_OUT_F32_NC1: return DK / 32;
    default: return DV / 96;
  }
}

hipError_t launch_seg_scan(float* buf, const float* decay, const float* Z0, const int32_t* z0_idx, int H,
                           int64_t BH, int nseg, int rev, hipStream_t st) {
  hipLaunchKernelGGL(seg_scan_kernel, dim3((DK * DV / 4 + 255) / 256, (unsigned)BH), dim3(256), 0, st, buf,
                     decay, Z0, z0_idx, H, nseg, rev);
  return hipGetLastError();
}

}  // namespace gla
