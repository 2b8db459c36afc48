// Device helpers shared by the gfx950 kernels of the Simple GLA mixer.
//
// Matrix-core conventions (checked on gfx950 with a lane-layout probe):
//  * v_mfma_f32_32x32x16_bf16: lane l holds 8 bf16 of A at row m = l%32 and of
//    B at column n = l%32; the 16 contraction values are split 8/8 between
//    the lane groups g = l/32.  The 16 fp32 results of lane l sit in column
//    n = l%32, rows m(r) = 8*(r/4) + 4*g + (r%4), r = 0..15.
//  * v_mfma_f32_32x32x2f32: one fp32 of A (row l%32) and of B (column l%32),
//    contraction index g = l/32; results laid out as above.
//  * ds_read_b64_tr_b16: within each 16-lane group, lanes 4r..4r+3 give the
//    address of 4 consecutive bf16 of row r (r = 0..3); lane L receives the
//    4 values of column L, one from each row.
//
// Because the contraction order inside an MFMA is free as long as A and B
// agree, a result tile held in registers can feed the next MFMA directly
// with its row index m as the contraction index.  All operands below use the
// same "register order" for a 32-wide contraction block:
//    bf16, sub-step s (0..1), element e (0..7): k = 16s + 8(e/4) + 4g + e%4
//    fp32, sub-step s (0..15):                   k = 8(s/4) + 4g + s%4
// which is exactly the row order of the 16 result registers.  Operands that
// both come from LDS in their natural layout use the plain order
//    bf16: k = 16s + 8g + e           (one 16-byte read).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_kernels.h"

namespace gla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float G_MIN = -60.0f;

#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Operand type of one MFMA sub-step and sub-steps per 32-wide contraction block.
template <class T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; static constexpr int SUB = 2; };
template <> struct Frag<float> { typedef float type; static constexpr int SUB = 16; };

typedef const LDS_AS bf16* lds_cptr;
// A generic pointer into shared memory as an LDS-address-space pointer, so
// that constant offsets fold into the DS instructions' offset field.
__device__ __forceinline__ lds_cptr to_lds(const bf16* p) { return (lds_cptr)(p); }
__device__ __forceinline__ bf16x4 lds_tr4(lds_cptr p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p));
}
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) { return lds_tr4(to_lds(p)); }
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// --- fragments of a row-major LDS matrix M[row][col] (pitch in elements) ---
// "kr": the contraction index runs along rows, the lane index along columns
//       (lane <-> col0 + l%32), register order.
// "kc": the lane index runs along rows (row0 + l%32), contraction along
//       columns; kcP in register order, kcN in the plain order.

__device__ __forceinline__ bf16x8 frag_kr(const bf16* M, int pitch, int row0, int col0, int s) {
  const int l = lane_id(), G = l >> 4, g = G >> 1, h = G & 1, L = l & 15;
  const bf16* p = M + (row0 + 16 * s + 4 * g + (L >> 2)) * pitch + col0 + 16 * h + 4 * (L & 3);
  return cat(lds_tr4(p), lds_tr4(p + 8 * pitch));
}
// (M in LDS: through an LDS-space pointer the constant part of the index
// folds into the DS instruction's offset, so all fragments of a tile share one
// per-lane address register.)
__device__ __forceinline__ float frag_kr(const float* M, int pitch, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5;
  return ((const LDS_AS float*)M)[(row0 + 8 * (s >> 2) + 4 * g + (s & 3)) * pitch + col0 + (l & 31)];
}

// As frag_kr, in the plain contraction order (k = 16s + 8g + e).
__device__ __forceinline__ bf16x8 frag_krN(const bf16* M, int pitch, int row0, int col0, int s) {
  const int l = lane_id(), G = l >> 4, g = G >> 1, h = G & 1, L = l & 15;
  const bf16* p = M + (row0 + 16 * s + 8 * g + (L >> 2)) * pitch + col0 + 16 * h + 4 * (L & 3);
  return cat(lds_tr4(p), lds_tr4(p + 4 * pitch));
}

__device__ __forceinline__ bf16x8 frag_kcP(const bf16* M, int pitch, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5;
  const bf16* p = M + (row0 + (l & 31)) * pitch + col0 + 16 * s + 4 * g;
  return cat(*(const bf16x4*)p, *(const bf16x4*)(p + 8));
}
__device__ __forceinline__ float frag_kcP(const float* M, int pitch, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5;
  return ((const LDS_AS float*)M)[(row0 + (l & 31)) * pitch + col0 + 8 * (s >> 2) + 4 * g + (s & 3)];
}

__device__ __forceinline__ bf16x8 frag_kcN(const bf16* M, int pitch, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5;
  return *(const bf16x8*)(M + (row0 + (l & 31)) * pitch + col0 + 16 * s + 8 * g);
}
__device__ __forceinline__ float frag_kcN(const float* M, int pitch, int row0, int col0, int s) {
  return frag_kcP(M, pitch, row0, col0, s);
}

// --- bf16 tiles [rows][96] without padding, 16-byte units XOR-swizzled by
// (row >> 2) & 3.  With 64 banks of 4 bytes this makes the transposed reads
// (4 rows x 64 bytes per 32 lanes) and the row reads (16 rows x 16 bytes per
// 16 lanes) free of bank conflicts.
__device__ __forceinline__ int swz96(int row, int col) {
  return row * 96 + ((((col >> 3) ^ ((row >> 2) & 3))) << 3) + (col & 7);
}
// Hot-loop loaders for row0, col0 multiples of 32: the swizzle key then
// depends on the lane only, so each access is a per-lane offset (computed once)
// plus a compile-time offset.
__device__ __forceinline__ bf16x8 sfrag_kr(const bf16* M, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5, h = (l >> 4) & 1, L = l & 15;
  const int rowl = 4 * g + (L >> 2), ul = 2 * h + ((L & 3) >> 1), hl = 4 * (L & 1);
  const int off1 = rowl * 96 + ((ul ^ g) << 3) + hl;
  const int off2 = (rowl + 8) * 96 + ((ul ^ (g + 2)) << 3) + hl;
  const lds_cptr base = to_lds(M) + (row0 + 16 * s) * 96 + col0;
  return cat(lds_tr4(base + off1), lds_tr4(base + off2));
}
__device__ __forceinline__ bf16x8 sfrag_krN(const bf16* M, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5, h = (l >> 4) & 1, L = l & 15;
  const int rowl = 8 * g + (L >> 2), ul = 2 * h + ((L & 3) >> 1), hl = 4 * (L & 1);
  const int off1 = rowl * 96 + ((ul ^ (2 * g)) << 3) + hl;
  const int off2 = (rowl + 4) * 96 + ((ul ^ (2 * g + 1)) << 3) + hl;
  const lds_cptr base = to_lds(M) + (row0 + 16 * s) * 96 + col0;
  return cat(lds_tr4(base + off1), lds_tr4(base + off2));
}
__device__ __forceinline__ bf16x8 sfrag_kcN(const bf16* M, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5, r = l & 31, key = (r >> 2) & 3;
  const int off = r * 96 + (((2 * s + g) ^ key) << 3);
  return *(const LDS_AS bf16x8*)(to_lds(M) + row0 * 96 + col0 + off);
}
// General (any row0, col0) versions for cold paths.
__device__ __forceinline__ bf16x8 sfrag_kcN_any(const bf16* M, int row0, int col0, int s) {
  const int l = lane_id(), g = l >> 5;
  return *(const bf16x8*)(M + swz96(row0 + (l & 31), col0 + 16 * s + 8 * g));
}
__device__ __forceinline__ bf16x8 sfrag_krN_any(const bf16* M, int row0, int col0, int s) {
  const int l = lane_id(), G = l >> 4, g = G >> 1, h = G & 1, L = l & 15;
  const int r = row0 + 16 * s + 8 * g + (L >> 2), c = col0 + 16 * h + 4 * (L & 3);
  return cat(lds_tr4(M + swz96(r, c)), lds_tr4(M + swz96(r + 4, c)));
}

// Contraction row (within a 32-block) of register/element e of sub-step s.
__device__ __forceinline__ int kidx_bf16(int s, int e) {
  return 16 * s + 8 * (e >> 2) + 4 * (lane_id() >> 5) + (e & 3);
}
__device__ __forceinline__ int kidx_f32(int s) {
  return 8 * (s >> 2) + 4 * (lane_id() >> 5) + (s & 3);
}
// Row (within a 32x32 result tile) held by result register r.
__device__ __forceinline__ int out_row(int r) { return 8 * (r >> 2) + 4 * (lane_id() >> 5) + (r & 3); }

// Scale the 8 contraction values of a bf16 operand by per-k weights w[k]
// (w indexed by contraction row inside the block), rounding back to bf16.
__device__ __forceinline__ bf16x8 scale_k(bf16x8 a, const float* w, int s) {
  const int g = lane_id() >> 5;
  const f32x4 w0 = *(const f32x4*)(w + 16 * s + 4 * g);
  const f32x4 w1 = *(const f32x4*)(w + 16 * s + 8 + 4 * g);
  bf16x8 r;
  r[0] = (bf16)((float)a[0] * w0[0]); r[1] = (bf16)((float)a[1] * w0[1]);
  r[2] = (bf16)((float)a[2] * w0[2]); r[3] = (bf16)((float)a[3] * w0[3]);
  r[4] = (bf16)((float)a[4] * w1[0]); r[5] = (bf16)((float)a[5] * w1[1]);
  r[6] = (bf16)((float)a[6] * w1[2]); r[7] = (bf16)((float)a[7] * w1[3]);
  return r;
}
__device__ __forceinline__ float scale_k(float a, const float* w, int s) {   // w in LDS
  return a * ((const LDS_AS float*)w)[kidx_f32(s)];
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float bf16_lo_f(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf16_hi_f(uint32_t p) { return __builtin_bit_cast(float, p & 0xffff0000u); }

// hi = bf16(x), lo = bf16(x - hi) for a pair of floats.
__device__ __forceinline__ void split_pk(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pk_bf16(a, b);
  lo = pk_bf16(a - bf16_lo_f(hi), b - bf16_hi_f(hi));
}

// Split 8 floats (as 4 pairs) into compensated bf16x8 hi/lo operands.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split_pk(x[2 * i], x[2 * i + 1], h[i], l[i]);
  hi = __builtin_bit_cast(bf16x8, *(uint4*)h);
  lo = __builtin_bit_cast(bf16x8, *(uint4*)l);
}

// The compensated operand pair for sub-step s of a result tile's registers.
__device__ __forceinline__ void split_tile(const f32x16& t, int s, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split_pk(t[8 * s + 2 * i], t[8 * s + 2 * i + 1], h[i], l[i]);
  hi = __builtin_bit_cast(bf16x8, *(uint4*)h);
  lo = __builtin_bit_cast(bf16x8, *(uint4*)l);
}

// Error-compensated bf16 operands: x ~= hi + lo with hi = bf16(x) and
// lo = bf16(x - hi), so a product with an exact bf16 operand, done as two
// MFMAs, keeps about 16 significant bits of x instead of 8.
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

__device__ __forceinline__ void scale_k_split(bf16x8 a, const float* w, int s, bf16x8& hi, bf16x8& lo) {
  const int g = lane_id() >> 5;
  const f32x4 w0 = *(const f32x4*)(w + 16 * s + 4 * g);
  const f32x4 w1 = *(const f32x4*)(w + 16 * s + 8 + 4 * g);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (float)a[e] * (e < 4 ? w0[e & 3] : w1[e & 3]);
    bf16 h, l;
    split_bf16(x, h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

__device__ __forceinline__ void regs_to_frag_split(const f32x16& t, int s, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16 h, l;
    split_bf16(t[8 * s + e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

__device__ __forceinline__ void store4_split(bf16* hi, bf16* lo, f32x4 v) {
  uint32_t h[2], l[2];
  split_pk(v[0], v[1], h[0], l[0]);
  split_pk(v[2], v[3], h[1], l[1]);
  *(uint2*)hi = make_uint2(h[0], h[1]);
  *(uint2*)lo = make_uint2(l[0], l[1]);
}

// The bf16 operand for sub-step s taken from result registers of a tile.
__device__ __forceinline__ bf16x8 regs_to_frag(const f32x16& t, int s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)t[8 * s + e];
  return r;
}

// Converting stores of 4 consecutive values.
__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *(bf16x4*)p = b;
}
__device__ __forceinline__ f32x4 load4f(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load4f(const bf16* p) {
  bf16x4 b = *(const bf16x4*)p;
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// x * silu(a) = x * a / (1 + e^-a): the output gate (e^-a overflows to inf
// for a below about -88, which gives -0).
__device__ __forceinline__ float gate_silu(float x, float a) { return x * (a / (1.0f + __expf(-a))); }

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

// Inclusive suffix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_rscan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_down(x, off, 64);
    if (l + off < 64) x += y;
  }
  return x;
}

// DPP lane moves (gfx9 encodings): row_shr:n = 0x110+n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143, wave_shr:1 = 0x138.  Lanes without a source read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true));
}
// Inclusive prefix sum over the 64 lanes: shifts 1, 2, 4, 8 inside each row
// of 16 lanes, then the row totals are broadcast into the later rows.
__device__ __forceinline__ float wave_scan_dpp(float x) {
  x += dpp_mov<0x111, 0xf>(x);
  x += dpp_mov<0x112, 0xf>(x);
  x += dpp_mov<0x114, 0xf>(x);
  x += dpp_mov<0x118, 0xf>(x);
  x += dpp_mov<0x142, 0xa>(x);
  x += dpp_mov<0x143, 0xc>(x);
  return x;
}
// Value of the previous lane (0 for lane 0).
__device__ __forceinline__ float wave_shr1(float x) { return dpp_mov<0x138, 0xf>(x); }

// Chunk decay tables in LDS, from the chunk's log-decay.  With b_i the
// inclusive running sum of the clamped log-decay (in log2 units):
//   b2[i]  = b_i (so Lambda_i = 2^{b_i}),  kap[i] = 2^{b_last - b_i},  gam = 2^{b_last}
struct DecayLds {
  float b2[CH];
  float kap[CH];
  float gam;
  float blast;
};

// Called by one whole wave.  x0, x1: log-decays of tokens 2l and 2l+1;
// m0, m1: of tokens 127-2l and 126-2l (0 for padded tokens).  kappa comes
// from a prefix sum over the mirrored tokens (a suffix sum), so it does not
// inherit the rounding of b_last - b_j; kappa of the last real token is 1.
// If utab is given, also utab[U(I) + j] = 2^{b_{32I} - b_j} for j < 32I,
// I = 1..3, U = 0, 32, 96 (decay factors between 32-token blocks).
__device__ __forceinline__ void build_decay(DecayLds* d, float x0, float x1, float m0, float m1,
                                            float* utab = nullptr) {
  const int l = lane_id();
  x0 = fmaxf(x0, G_MIN) * LOG2E;
  x1 = fmaxf(x1, G_MIN) * LOG2E;
  m0 = fmaxf(m0, G_MIN) * LOG2E;
  m1 = fmaxf(m1, G_MIN) * LOG2E;
  const float pr = wave_scan_dpp(x0 + x1);            // sum over tokens <= 2l+1
  const float pr_ex = wave_shr1(pr);                  // sum over tokens < 2l
  const float sr = wave_scan_dpp(m0 + m1);            // sum over tokens >= 126-2l
  const float sr_ex = wave_shr1(sr);                  // sum over tokens > 127-2l
  const float b0 = pr_ex + x0, b1 = pr;
  const float blast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr), 63));
  d->b2[2 * l] = b0;
  d->b2[2 * l + 1] = b1;
  d->kap[127 - 2 * l] = exp2f(sr_ex);
  d->kap[126 - 2 * l] = exp2f(sr_ex + m0);
  if (l == 0) { d->gam = exp2f(blast); d->blast = blast; }
  if (utab) {
#pragma unroll
    for (int I = 1; I < 4; ++I) {
      // b_{32I} is b0 of lane 16I
      const float bref = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b0), 16 * I));
      const int off = I == 1 ? 0 : I == 2 ? 32 : 96;
      if (2 * l < 32 * I) utab[off + 2 * l] = exp2f(bref - b0);
      if (2 * l + 1 < 32 * I) utab[off + 2 * l + 1] = exp2f(bref - b1);
    }
  }
}

}  // namespace gla
