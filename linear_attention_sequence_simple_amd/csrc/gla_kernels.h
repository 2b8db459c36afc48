// Launch interface between the host library and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr int CH = 128;   // chunk length (tokens)
constexpr int DK = 96;    // key/query width per head
constexpr int DV = 192;   // value width per head

enum WalkMode { WALK_FWD_OUT = 0, WALK_FWD_STATE = 1 };

enum WalkVariant {
  WV_FWD_OUT_BF16_BF16 = 0,
  WV_FWD_OUT_BF16_F32 = 1,
  WV_FWD_OUT_F32_F32 = 2,
  WV_FWD_OUT_F32_BF16 = 3,
  WV_FWD_STATE_BF16 = 4,
  WV_FWD_STATE_F32 = 5,
  // fp32 in and out, 32-column value slices (three over a 96-wide value
  // tile): the fp32 backward's walks whose values are k or q
  WV_OUT_F32_NC1 = 6,
};

// A token tensor as one walk sees it: column j of dv-slice s of token t (in
// walk order), batch b, head h is at
//     p + b*sb + h*sh + t*st + s*ss + j        (elements)
// A negative st walks a [B,T,H,D] tensor backwards in time.
struct TokView {
  const void* p;
  int64_t sb, sh, st, ss;
};

// A state block: element (x index i, y index j) of dv-slice s of (batch-head
// bh, segment seg) is at p + bh*sbh + seg*sseg + s*ss + i*sx + j*sy, where x
// indexes the key-side width and y the value-side width of the walk.
struct StateView {
  float* p;
  int64_t sbh, sseg, ss, sx, sy;
};

// Arguments of one walk launch: the recurrence Z_t = e^{g_t} Z_{t-1} + x_t^T y_t
// over the walk's tokens, optionally with the outputs
// o_t = q_t Z_t (queries Q, written to O).
struct WalkArgs {
  TokView X;            // keys            (width 96)
  TokView Y;            // values          (width 96 per slice; 64 for fp32 inputs)
  TokView Q;            // queries         (width 96), with output only
  TokView O;            // outputs         (width of Y), with output only
  TokView G;            // with output: gate in the input dtype, same columns as O
                        // (p null: none); o_t <- o_t * silu(gate_t) before the store
  const float* g;       // log-decay of walk token t: g[b*gsb + h*gsh + (t - gshift)*gst],
  int64_t gsb, gsh, gst;  // zero for t < gshift
  int gshift;
  TokView acc;          // with output: fp32 partial sums added to the outputs (p null: none),
                        // the layout of O (fp32)
  TokView D;            // with acc: rows dotted with the final outputs (bf16, width of Y)
  TokView rdot;         // with acc: those dot products, one float per token (p null: none)
  StateView zinit;      // initial state (p null: zero)
  StateView zfin;       // final state (p null: not written)
  int zfin_only_seg;    // -1: every segment writes; else only that segment
  float* seg_decay;     // per-segment total log2-decay or null
  int64_t seg_decay_bh_stride;
  int64_t B, T;
  int H, n_chunks, cps, ns, nseg_launch, seg_offset;
  int chunk0;           // segment s of the walk covers chunks chunk0 + s*cps onwards (cps of them)
  // Packed sequences (null: B sequences of T tokens): sequence b is tokens
  // [cu[b], cu[b+1]) of a token axis of cu_total rows, the batch strides are
  // zero, and T and n_chunks bound its length in tokens and chunks.  Offsets
  // are clamped into [0, cu_total] and lengths to [0, T].
  const int32_t* cu;
  int64_t cu_total;
  // Packed sequences only: the batch index of sequence b's initial (final)
  // state is zinit_idx[b] (zfin_idx[b]), a slot of a pool; null: b.
  const int32_t* zinit_idx;
  const int32_t* zfin_idx;
};

hipError_t launch_walk(const WalkArgs& a, int variant, int nwg, hipStream_t st);
// Two bf16 walks with output in one launch (nwg0 + nwg1 workgroups).
hipError_t launch_out_walk_pair(const WalkArgs& a0, int nwg0, const WalkArgs& a1, int nwg1, int out_bf16,
                                hipStream_t st);
// Two independent bf16 state-only walks in one launch (nwg0 + nwg1
// workgroups).
hipError_t launch_state_walk_pair(const WalkArgs& a0, int nwg0, const WalkArgs& a1, int nwg1, hipStream_t st);
// Up to four bf16 walks with output in one launch (nwg[i] workgroups each,
// zero to skip one), in two groups of compile-time variants named by `kind`
// (group A: walks 0 and 1, output type and partial sums; group B: walks 2 and
// 3, output type, no partial sums).
enum WalkQuadKind {
  QUAD_F32_F32 = 0,        // A: float out;                B: float out
  QUAD_F32_BF16 = 1,       // A: float out;                B: bf16 out
  QUAD_ACC_F32_F32 = 2,    // A: float out, partial sums;  B: float out
  QUAD_ACC_BF16_F32 = 3,   // A: bf16 out, partial sums;   B: float out
  QUAD_ACC_BF16_BF16 = 4,  // A: bf16 out, partial sums;   B: bf16 out
};
hipError_t launch_out_walk_quad(const WalkArgs* a, const int* nwg, int kind, hipStream_t st);
int walk_slices(int variant);
// Z0 row of batch-head bh: z0_idx[bh / H] * H + bh % H when z0_idx is set.
hipError_t launch_seg_scan(float* buf, const float* decay, const float* Z0, const int32_t* z0_idx, int H,
                           int64_t BH, int nseg, int rev, hipStream_t st);

// Decode step: see gla_step.hip.
// The convolution ahead of the mixer (gla_conv.hip): sequence b is rows
// cu[b]..cu[b+1] of x (cu null: rows b*T..(b+1)*T), at most T tokens; its
// window (when state is set) is the CONV_WIN rows of slot slot[b] (slot
// null: b), row m holding x_{m-4}.
constexpr int CONV_WIN = 4;
struct ConvArgs {
  const void* x;
  const float* w;       // [D, 4]
  const float* bias;    // [D] or null
  float* state;         // [slots, CONV_WIN, D] float32, or null
  const int32_t* slot;
  const int32_t* cu;
  int64_t B, T, total;
  int D, runs, init;    // runs: token runs per sequence, set by the launcher
  void* y;
};
hipError_t launch_conv(const ConvArgs& a, bool in_bf16, bool out_bf16, hipStream_t st);

struct StepArgs {
  const void* q; const void* k; const void* v; const float* g;
  float* pool; const int32_t* slot_idx; void* o;
  int64_t B; int H;
};
hipError_t launch_step(const StepArgs& a, int in_bf16, int out_bf16, hipStream_t st);

// 16-bit decode state (gla_state16.hip): int16 mantissas [slot][H][DK][DV]
// and one int32 exponent per state column [slot][H][DV].
struct Q16Pool {
  int16_t* mant; int32_t* expo;
};
struct StepQ16Args {
  const void* q; const void* k; const void* v; const float* g;
  Q16Pool pool; const int32_t* slot_idx; void* o;
  int64_t B; int H;
};
hipError_t launch_step_q16(const StepQ16Args& a, int in_bf16, int out_bf16, hipStream_t st);
// n float32 states S [n][H][DK][DV] into (write != 0) or out of pool slots
// slot_idx[i] (or i): pool_f32 for a float32 pool, q16 (mant set) for a
// 16-bit one.
struct StateIoArgs {
  float* S; float* pool_f32; Q16Pool q16; const int32_t* slot_idx;
  int64_t n; int H; int write;
};
hipError_t launch_state_io(const StateIoArgs& a, hipStream_t st);

// Backward finish: see gla_bwd.hip.
struct BwdFinishArgs {
  const float* rq;                    // [B,T,H] q_t.dq_t
  const float* rk;                    // [B,T,H] k_t.dk_t
  float* dg;                          // [B,T,H] in-chunk suffix sums of rq - rk
  float* chunk_r;                     // [BH][N] per-chunk totals
  int64_t B, T; int H, n_chunks;
};
hipError_t launch_bwd_finish(const BwdFinishArgs& a, hipStream_t st);
// fp32 backward: rq = q.dq and rk = k.dk per [B,T,H] row from float32
// q, k, dq, dk ([rows][DK]); with dq_bf16 set, dq and dk rounded into
// dq_bf16 and dk_bf16.
struct RowDotsArgs {
  const float* q; const float* k; const float* dq; const float* dk;
  float* rq; float* rk;
  __bf16* dq_bf16; __bf16* dk_bf16;
  int64_t rows;
};
hipError_t launch_row_dots(const RowDotsArgs& a, hipStream_t st);
hipError_t launch_dg_finish(float* dg, const float* chunk_r, const float* dS_T, const float* S_T, float* dS0,
                            const float* g, int64_t B, int64_t T, int H, int n_chunks, hipStream_t st);

}  // namespace gla
