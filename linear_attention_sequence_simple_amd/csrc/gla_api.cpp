// Host side of libgla: the C ABI declared in include/gla.h.
//
// Every call validates its arguments before touching the HIP runtime, picks a
// launch plan, carves the caller's workspace, and enqueues kernels on the
// caller's stream without synchronising.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "gla.h"
#include "gla_debug.h"
#include "gla_kernels.h"

using namespace gla;

struct gla_state {
  float* data;                 // float32 states (GLA_STATE_F32), else NULL
  int64_t n_slots;
  int32_t H, dk, dv;
  int device;
  int32_t format;              // gla_state_fmt
  int16_t* mant;               // GLA_STATE_Q16: mantissas [n_slots][H][dk][dv]
  int32_t* expo;               // and exponents [n_slots][H][dv]
  float* conv;                 // the convolution's window [n_slots][4][conv_D] float32, or NULL
  int32_t conv_D;              // its channels (0: no window)
  void* base;                  // the allocation
};

namespace {

thread_local std::string g_err;

gla_status fail(gla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

gla_status ok() { return GLA_OK; }

gla_status device_err(hipError_t e, const char* where) {
  if (e == hipSuccess) return GLA_OK;
  return fail(GLA_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- GLA_DEBUG: device-side checks of the caller contracts (gla_debug.hip)
bool debug_on() {
  const char* s = std::getenv("GLA_DEBUG");
  return s && *s && std::strcmp(s, "0") != 0;
}

// One flag word per device, allocated on first use under GLA_DEBUG.
int* debug_flag() {
  static std::mutex mu;
  static std::map<int, int*> flags;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  auto it = flags.find(dev);
  if (it != flags.end()) return it->second;
  int* p = nullptr;
  if (hipMalloc(&p, sizeof(int)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  flags[dev] = p;
  return p;
}

// Held from clearing a device's flag to reading it back, so that calls from
// several host threads under GLA_DEBUG never share a flag's contents.
std::mutex& debug_mutex() {
  static std::mutex mu;
  return mu;
}

// Under GLA_DEBUG: clears the flag, runs checks(flag) (launches on st), reads
// the flag back (synchronising st) and fails the call when a check found a
// violation, before any of the call's own kernels is launched.
template <class F>
gla_status debug_checks(hipStream_t st, const char* call, F&& checks) {
  if (!debug_on()) return GLA_OK;
  std::lock_guard<std::mutex> lock(debug_mutex());
  int* flag = debug_flag();
  if (!flag) return fail(GLA_ERR_OUT_OF_MEMORY, "%s: the GLA_DEBUG flag could not be allocated", call);
  hipError_t e = debug_zero(flag, st);
  if (e == hipSuccess) e = checks(flag);
  int h = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&h, flag, sizeof h, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_err(e, "GLA_DEBUG checks");
  if (!h) return GLA_OK;
  std::string what;
  if (h & DBG_SLOT_RANGE) what += " a slot index is out of range;";
  if (h & DBG_SLOT_DUP) what += " a slot index is repeated;";
  if (h & DBG_DECAY) what += " a log-decay is positive or NaN;";
  if (h & DBG_OFFSETS) what += " sequence offsets are out of order or beyond their bounds;";
  return fail(GLA_ERR_INVALID_ARGUMENT, "%s (GLA_DEBUG):%s", call, what.c_str());
}

gla_status check_ptr(const void* p, const char* name, bool nullable) {
  if (!p) return nullable ? GLA_OK : fail(GLA_ERR_INVALID_ARGUMENT, "%s must not be NULL", name);
  if (!aligned16(p)) return fail(GLA_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return GLA_OK;
}

#define TRY(x)                       \
  do {                               \
    gla_status s_ = (x);             \
    if (s_ != GLA_OK) return s_;     \
  } while (0)

bool valid_dtype(int32_t d) { return d == GLA_F32 || d == GLA_BF16; }

gla_status check_heads(int32_t H, int32_t dk, int32_t dv) {
  if (H < 1) return fail(GLA_ERR_INVALID_ARGUMENT, "H must be >= 1 (got %d)", H);
  if (dk != DK || dv != DV)
    return fail(GLA_ERR_UNSUPPORTED, "only dk=%d, dv=%d are implemented (got dk=%d, dv=%d)", DK, DV, dk, dv);
  return GLA_OK;
}

gla_status check_dims(const gla_dims* d) {
  if (!d) return fail(GLA_ERR_INVALID_ARGUMENT, "dims must not be NULL");
  if (d->B < 1 || d->T < 1) return fail(GLA_ERR_INVALID_ARGUMENT, "B and T must be >= 1 (got B=%lld, T=%lld)",
                                        (long long)d->B, (long long)d->T);
  TRY(check_heads(d->H, d->dk, d->dv));
  if (d->chunk != CH) return fail(GLA_ERR_UNSUPPORTED, "only chunk=%d is implemented (got %d)", CH, d->chunk);
  if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype))
    return fail(GLA_ERR_INVALID_ARGUMENT, "in_dtype/out_dtype must be GLA_F32 or GLA_BF16");
  if (d->B * d->H > (int64_t)1 << 24) return fail(GLA_ERR_UNSUPPORTED, "B*H too large");
  // the walks address 32 token rows of a [B,T,H,dv] fp32 tensor with 32-bit offsets
  if ((int64_t)d->H * DV * 4 * 32 >= (int64_t)1 << 31) return fail(GLA_ERR_UNSUPPORTED, "H too large");
  if ((d->T + CH - 1) / CH > (1 << 20)) return fail(GLA_ERR_UNSUPPORTED, "T too large");
  if (d->segments < 0) return fail(GLA_ERR_INVALID_ARGUMENT, "segments must be >= 0 (got %d)", d->segments);
  return GLA_OK;
}

constexpr int64_t kStateElems = (int64_t)DK * DV;
constexpr int kTargetWorkgroups = 256;   // one per compute unit

// Segments per (batch, head, slice) walk: as many as the chip runs in one
// round of workgroups (one per compute unit), at least two chunks per segment;
// or the caller's count (dims->segments > 0), at most one segment per chunk.
// A count that overflows the round leaves its last workgroups to walk their
// whole segments on a nearly idle chip: 48 fp32 walks run 4 segments (192
// workgroups) faster than 6 (288), and a bf16 prefill of 5 x 16 heads runs
// unsegmented (160 workgroups) in 0.70 of the time of 2 segments (320).
int plan_segments(int64_t walkers, int n_chunks, int32_t forced) {
  int nseg = (int)std::max<int64_t>(1, kTargetWorkgroups / walkers);
  nseg = std::min(nseg, std::max(1, n_chunks / 2));
  if (forced > 0) nseg = std::min<int>(forced, n_chunks);
  return std::max(1, nseg);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// float32 states of a packed prefill into a 16-bit pool, one per sequence and
// head, staged in the workspace after the forward's own part
size_t stage_bytes(const gla_dims* d) { return align256((size_t)d->B * d->H * kStateElems * sizeof(float)); }

struct FwdPlan {
  int variant, ns, nseg, cps, n_chunks, fine;
  size_t ws_seg_states, ws_seg_decay, ws_total;
};

// Pass 1 may split each segment into `fine` parts: more, shorter state walks.
// The bf16 state walk fits two workgroups per compute unit, so it splits
// while that keeps at most two per unit and the parts stay whole chunks.
int fine_factor(int64_t pass1_workgroups, int cps, bool bf16) {
  int f = 1;
  if (!bf16) return f;
  while (f < 4 && cps % (2 * f) == 0 && pass1_workgroups * 2 * f <= 2 * kTargetWorkgroups) f *= 2;
  return f;
}

// Segment-state entries: the states entering every fine part of every
// segment but the last, and the state entering the last segment.
int seg_entries(int nseg, int fine) { return (nseg - 1) * fine + 1; }

FwdPlan plan_fwd(const gla_dims* d) {
  FwdPlan p{};
  const bool in_bf16 = d->in_dtype == GLA_BF16, out_bf16 = d->out_dtype == GLA_BF16;
  p.variant = in_bf16 ? (out_bf16 ? WV_FWD_OUT_BF16_BF16 : WV_FWD_OUT_BF16_F32)
                      : (out_bf16 ? WV_FWD_OUT_F32_BF16 : WV_FWD_OUT_F32_F32);
  p.ns = walk_slices(p.variant);
  p.n_chunks = (int)((d->T + CH - 1) / CH);
  const int64_t walkers = d->B * d->H * p.ns;
  p.nseg = plan_segments(walkers, p.n_chunks, d->segments);
  p.cps = (p.n_chunks + p.nseg - 1) / p.nseg;
  p.nseg = (p.n_chunks + p.cps - 1) / p.cps;
  const int64_t BH = d->B * d->H;
  p.fine = fine_factor(BH * p.ns * (p.nseg - 1), p.cps, in_bf16);
  if (p.nseg > 1) {
    const int ne = seg_entries(p.nseg, p.fine);
    p.ws_seg_states = align256((size_t)BH * ne * kStateElems * sizeof(float));
    p.ws_seg_decay = align256((size_t)BH * ne * sizeof(float));
  }
  p.ws_total = p.ws_seg_states + p.ws_seg_decay;
  return p;
}

// A [B,T,H,cols] row-major tensor of `esize`-byte elements, read forwards or
// backwards in time, in dv-slices of `slice_w` columns.
TokView tok_view(const void* p, size_t esize, const gla_dims* d, int cols, int slice_w, bool backwards) {
  TokView v;
  const int64_t row = (int64_t)d->H * cols;
  v.sb = d->T * row;
  v.sh = cols;
  v.ss = slice_w;
  v.st = backwards ? -row : row;
  v.p = backwards ? (const void*)((const char*)p + (d->T - 1) * row * (int64_t)esize) : p;
  return v;
}

// [BH][DK][DV] fp32 states.  A walk's state element (x index i, y index j) of
// slice s is S[i][s*w + j] when the walk's keys span dk (plain), or
// S[j][s*w + i] when its keys span a dv-slice (transposed).
StateView state_plain(float* p, int w) { return StateView{p, kStateElems, 0, w, DV, 1}; }
StateView state_transposed(float* p, int w) { return StateView{p, kStateElems, 0, w, 1, DV}; }

// The same layout for the per-segment states [BH][entries][DK][DV].
StateView seg_view(float* p, StateView lay, int entries) {
  lay.p = p;
  lay.sbh = (int64_t)entries * kStateElems;
  lay.sseg = kStateElems;
  return lay;
}

struct SegPlan {
  int ns, nseg, cps, n_chunks, fine;
  int entries() const { return seg_entries(nseg, fine); }
};

// The states entering the (coarse) segments inside the fine-part entries.
StateView coarse(StateView seg, const SegPlan& sp) {
  seg.sseg *= sp.fine;
  return seg;
}

void set_plan(WalkArgs& a, const SegPlan& sp) {
  a.ns = sp.ns;
  a.n_chunks = sp.n_chunks;
  a.cps = sp.cps;
}

// Segment pass 1: the walk of every fine part of every segment but the last
// from a zero state, writing each part's state change into `seg` and its
// total decay into seg_decay.
int pass1_workgroups(const SegPlan& sp, int64_t BH) { return (int)(BH * sp.ns * (sp.nseg - 1) * sp.fine); }

WalkArgs pass1_args(WalkArgs a, const SegPlan& sp, StateView seg, float* seg_decay) {
  set_plan(a, sp);
  a.cps = sp.cps / sp.fine;
  a.zinit = StateView{};
  a.zfin = seg;                                   // rows of the workspace: by sequence, never by slot
  a.zinit_idx = a.zfin_idx = nullptr;
  a.zfin_only_seg = -1;
  a.seg_decay = seg_decay;
  a.seg_decay_bh_stride = sp.entries();
  a.nseg_launch = (sp.nseg - 1) * sp.fine;
  a.seg_offset = 0;
  return a;
}

// Pass 1 and a scan over the parts from z0, which leaves in `seg` the state
// entering every part.  z0 and seg share one layout; z0_idx (or null) maps
// batch indices to rows of z0.
hipError_t segment_states(WalkArgs a, int state_variant, const SegPlan& sp, const float* z0, const int32_t* z0_idx,
                          int H, StateView seg, float* seg_decay, int64_t BH, hipStream_t st) {
  hipError_t e = launch_walk(pass1_args(a, sp, seg, seg_decay), state_variant, pass1_workgroups(sp, BH), st);
  if (e != hipSuccess) return e;
  return launch_seg_scan(seg.p, seg_decay, z0, z0_idx, H, BH, sp.entries(), 0, st);
}

// The walk of every segment from its entering state (zinit: the segment
// states, or the initial state when there is one segment); the final state
// comes from the last segment.
WalkArgs segments_args(WalkArgs a, const SegPlan& sp, StateView zinit, StateView zfin) {
  set_plan(a, sp);
  a.zinit = zinit;
  a.zfin = zfin;
  a.zfin.sseg = 0;
  a.zfin_only_seg = sp.nseg > 1 ? sp.nseg - 1 : -1;
  a.seg_decay = nullptr;
  a.nseg_launch = sp.nseg;
  a.seg_offset = 0;
  return a;
}

hipError_t walk_segments(WalkArgs a, int variant, const SegPlan& sp, StateView zinit, StateView zfin, int64_t BH,
                         hipStream_t st) {
  return launch_walk(segments_args(a, sp, zinit, zfin), variant, (int)(BH * sp.ns * sp.nseg), st);
}

// A view moved by `elems` elements of `esize` bytes (a dv-half of a tensor).
TokView shifted(TokView v, int64_t elems, size_t esize) {
  if (v.p) v.p = (const char*)v.p + elems * (int64_t)esize;
  return v;
}
StateView shifted(StateView v, int64_t elems) {
  if (v.p) v.p += elems;
  return v;
}
// One [B,T,H] float per token, read forwards or backwards in time.
TokView token_floats(float* p, const gla_dims* d, bool backwards) {
  TokView v = tok_view(p, 4, d, 1, 0, backwards);
  return v;
}

// Backward workspace: fp32 sums of dq and dk over the first dv-half
// ([B,T,H,DK] each), the dot products q.dq and k.dk ([B,T,H] each), the final
// forward state, per-chunk sums of the log-decay gradient, and the segment
// states and decays of the forward and the backward-in-time recurrences.
struct BwdPlan {
  SegPlan sp;
  size_t off_dq, off_dk, off_rq, off_rk, off_st, off_r, off_segf, off_segr, off_decf, off_decr, ws_total;
};

BwdPlan plan_bwd(const gla_dims* d) {
  BwdPlan p{};
  p.sp.n_chunks = (int)((d->T + CH - 1) / CH);
  p.sp.ns = DV / 96;
  const int64_t BH = d->B * d->H;
  p.sp.nseg = plan_segments(BH * p.sp.ns, p.sp.n_chunks, d->segments);
  p.sp.cps = (p.sp.n_chunks + p.sp.nseg - 1) / p.sp.nseg;
  p.sp.nseg = (p.sp.n_chunks + p.sp.cps - 1) / p.sp.cps;
  p.sp.fine = fine_factor(2 * BH * p.sp.ns * (p.sp.nseg - 1), p.sp.cps, true);   // two recurrences
  const size_t part = align256((size_t)d->B * d->T * d->H * DK * sizeof(float));
  const size_t tok = align256((size_t)d->B * d->T * d->H * sizeof(float));
  size_t off = 0;
  p.off_dq = off; off += part;
  p.off_dk = off; off += part;
  p.off_rq = off; off += tok;
  p.off_rk = off; off += tok;
  p.off_st = off; off += align256((size_t)BH * kStateElems * sizeof(float));
  p.off_r = off; off += align256((size_t)BH * (p.sp.n_chunks + 1) * sizeof(float));   // chunk totals, constants
  const size_t seg = p.sp.nseg > 1 ? align256((size_t)BH * p.sp.entries() * kStateElems * sizeof(float)) : 0;
  const size_t dec = p.sp.nseg > 1 ? align256((size_t)BH * p.sp.entries() * sizeof(float)) : 0;
  p.off_segf = off; off += seg;
  p.off_segr = off; off += seg;
  p.off_decf = off; off += dec;
  p.off_decr = off; off += dec;
  p.ws_total = off;
  return p;
}

// fp32 backward workspace: the first dv-half's sums of dq and dk
// ([B,T,H,DK] each), the float32 gradients when the outputs are bf16, q.dq
// and k.dk ([B,T,H] each), the final forward state, the per-chunk sums of the
// log-decay gradient, and the segment states and decays of both recurrences
// when the walks are split.  Every walk has three slices (32 value columns
// for dq and dk, 64 for dv), so one segment plan serves them all.
struct BwdF32Plan {
  int n_chunks;
  SegPlan sp;
  size_t off_adq, off_adk, off_fdq, off_fdk, off_rq, off_rk, off_st, off_r, off_segf, off_segr, off_decf, off_decr,
      ws_total;
};

BwdF32Plan plan_bwd_f32(const gla_dims* d) {
  BwdF32Plan p{};
  p.n_chunks = (int)((d->T + CH - 1) / CH);
  const int64_t BH = d->B * d->H;
  p.sp.n_chunks = p.n_chunks;
  p.sp.ns = 3;
  p.sp.nseg = plan_segments(BH * p.sp.ns, p.n_chunks, d->segments);
  p.sp.cps = (p.n_chunks + p.sp.nseg - 1) / p.sp.nseg;
  p.sp.nseg = (p.n_chunks + p.sp.cps - 1) / p.sp.cps;
  p.sp.fine = fine_factor(2 * BH * p.sp.ns * (p.sp.nseg - 1), p.sp.cps, false);
  const size_t part = align256((size_t)d->B * d->T * d->H * DK * sizeof(float));
  const size_t tok = align256((size_t)d->B * d->T * d->H * sizeof(float));
  const bool bf16_out = d->out_dtype == GLA_BF16;
  size_t off = 0;
  p.off_adq = off; off += part;
  p.off_adk = off; off += part;
  p.off_fdq = off; off += bf16_out ? part : 0;
  p.off_fdk = off; off += bf16_out ? part : 0;
  p.off_rq = off; off += tok;
  p.off_rk = off; off += tok;
  p.off_st = off; off += align256((size_t)BH * kStateElems * sizeof(float));
  p.off_r = off; off += align256((size_t)BH * (p.n_chunks + 1) * sizeof(float));
  const size_t seg = p.sp.nseg > 1 ? align256((size_t)BH * p.sp.entries() * kStateElems * sizeof(float)) : 0;
  const size_t dec = p.sp.nseg > 1 ? align256((size_t)BH * p.sp.entries() * sizeof(float)) : 0;
  p.off_segf = off; off += seg;
  p.off_segr = off; off += seg;
  p.off_decf = off; off += dec;
  p.off_decr = off; off += dec;
  p.ws_total = off;
  return p;
}

// A view with caller strides (elements), in dv-slices of `slice_w` columns.
TokView strided_view(const void* p, const gla_strides& s, int slice_w) {
  TokView v;
  v.p = p;
  v.sb = s.batch;
  v.sh = s.head;
  v.st = s.token;
  v.ss = slice_w;
  return v;
}

// Strides of a view: 16-byte rows steps, positive, and 32 token rows within
// the 32-bit tile offsets of the walks.
gla_status check_strides(const gla_strides* s, size_t esize, bool rows16, const char* name) {
  if (!s) return GLA_OK;
  if (s->batch < 1 || s->token < 1 || s->head < 1)
    return fail(GLA_ERR_INVALID_ARGUMENT, "%s strides must be positive (got %lld, %lld, %lld)", name,
                (long long)s->batch, (long long)s->token, (long long)s->head);
  const int64_t q = rows16 ? (int64_t)(16 / esize) : 1;
  if (s->batch % q || s->token % q || s->head % q)
    return fail(GLA_ERR_INVALID_ARGUMENT, "%s strides must be multiples of 16 bytes", name);
  const int64_t lim = ((int64_t)1 << 31) / (32 * (int64_t)esize);
  if (s->token >= lim || s->head >= lim) return fail(GLA_ERR_INVALID_ARGUMENT, "%s strides too large", name);
  return GLA_OK;
}

// The forward's walk arguments over [B,T,H,cols] tensors (T of dims), with
// sequences of at most max_len tokens.
WalkArgs fwd_args(const gla_dims* dims, const FwdPlan& p, const void* q, const void* k, const void* v,
                  const float* g, void* o, int64_t max_len) {
  const size_t isz = dims->in_dtype == GLA_BF16 ? 2 : 4, osz = dims->out_dtype == GLA_BF16 ? 2 : 4;
  const int w = DV / p.ns;                        // dv-slice width
  WalkArgs a{};
  a.X = tok_view(k, isz, dims, DK, 0, false);
  a.Y = tok_view(v, isz, dims, DV, w, false);
  a.Q = tok_view(q, isz, dims, DK, 0, false);
  a.O = tok_view(o, osz, dims, DV, w, false);
  a.g = g;
  a.gsb = dims->T * dims->H;
  a.gsh = 1;
  a.gst = dims->H;
  a.B = dims->B;
  a.T = max_len;
  a.H = dims->H;
  return a;
}

// The forward's launches: one walk per (sequence, head, slice), or pass 1,
// the segment scan and the walks of all segments.  z0 (p null: zero) and
// zfin (p null: not written) may be the same memory; a packed walk reaches
// them through a.zinit_idx and a.zfin_idx.
hipError_t run_fwd(const gla_dims* dims, const FwdPlan& p, WalkArgs a, StateView z0, StateView zfin, void* ws,
                   hipStream_t st) {
  const int64_t BH = dims->B * dims->H;
  const SegPlan sp{p.ns, p.nseg, p.cps, p.n_chunks, p.fine};
  if (p.nseg == 1) return walk_segments(a, p.variant, sp, z0, zfin, BH, st);
  char* wsb = (char*)ws;
  const StateView seg = seg_view((float*)wsb, z0, sp.entries());
  const int state_variant = dims->in_dtype == GLA_BF16 ? WV_FWD_STATE_BF16 : WV_FWD_STATE_F32;
  const int32_t* z0_idx = a.zinit_idx;
  a.zinit_idx = nullptr;                          // the segment states are indexed by sequence
  hipError_t e = segment_states(a, state_variant, sp, z0.p, z0_idx, dims->H, seg,
                                (float*)(wsb + p.ws_seg_states), BH, st);
  if (e == hipSuccess) e = walk_segments(a, p.variant, sp, coarse(seg, sp), zfin, BH, st);
  return e;
}


gla_status check_conv_D(int32_t D) {
  if (D < 8 || D % 8 != 0 || D > (1 << 16))
    return fail(GLA_ERR_UNSUPPORTED, "D must be a multiple of 8 in [8, 65536] (got %d)", D);
  return GLA_OK;
}

// Bytes of one slot: the mixer state in `format` and the convolution's
// window of conv_D channels (conv_D = 0: none).
size_t slot_bytes(int32_t H, int32_t dk, int32_t dv, int32_t format, int32_t conv_D) {
  const size_t mixer = format == GLA_STATE_Q16 ? (size_t)H * (dk * dv * sizeof(int16_t) + dv * sizeof(int32_t))
                                               : (size_t)H * dk * dv * sizeof(float);
  return mixer + (size_t)CONV_WIN * conv_D * sizeof(float);
}

// A pool of n_slots states in `format` (and, with conv_D > 0, a float32
// convolution window [4][conv_D] per slot), zero-filled in stream order (zero
// mantissas and exponents read as zero states too).
gla_status alloc_pool(int64_t n_slots, int32_t H, int32_t dk, int32_t dv, int32_t format, int32_t conv_D,
                      void* stream, gla_state** out) {
  if (!out) return fail(GLA_ERR_INVALID_ARGUMENT, "out must not be NULL");
  *out = nullptr;
  if (n_slots < 1) return fail(GLA_ERR_INVALID_ARGUMENT, "n_slots must be >= 1 (got %lld)", (long long)n_slots);
  TRY(check_heads(H, dk, dv));
  if (format != GLA_STATE_F32 && format != GLA_STATE_Q16)
    return fail(GLA_ERR_INVALID_ARGUMENT, "format must be GLA_STATE_F32 or GLA_STATE_Q16 (got %d)", format);
  if (conv_D != 0) TRY(check_conv_D(conv_D));
  const bool q16 = format == GLA_STATE_Q16;
  const size_t slot = q16 ? (size_t)H * dk * dv * sizeof(int16_t) : gla_state_slot_bytes(H, dk, dv);
  if ((size_t)n_slots > ((size_t)1 << 46) / slot_bytes(H, dk, dv, format, conv_D))
    return fail(GLA_ERR_OUT_OF_MEMORY, "pool of %lld slots is too large", (long long)n_slots);
  const size_t mant_bytes = (size_t)n_slots * slot;
  const size_t expo_off = q16 ? align256(mant_bytes) : mant_bytes;
  const size_t mixer_bytes = q16 ? expo_off + (size_t)n_slots * H * dv * sizeof(int32_t) : mant_bytes;
  const size_t conv_off = align256(mixer_bytes);
  const size_t bytes = conv_D ? conv_off + (size_t)n_slots * CONV_WIN * conv_D * sizeof(float) : mixer_bytes;
  int dev = 0;
  TRY(device_err(hipGetDevice(&dev), "hipGetDevice"));
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return fail(GLA_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
  }
  e = hipMemsetAsync(p, 0, bytes, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return device_err(e, "hipMemsetAsync");
  }
  gla_state* s = new gla_state{q16 ? nullptr : (float*)p, n_slots, H, dk, dv, dev, format,
                               q16 ? (int16_t*)p : nullptr, q16 ? (int32_t*)((char*)p + expo_off) : nullptr,
                               conv_D ? (float*)((char*)p + conv_off) : nullptr, conv_D, p};
  *out = s;
  return ok();
}



gla_status state_io(const gla_state* pool, int64_t n, const int32_t* slot_idx, float* S, int write, void* stream,
                    const char* what) {
  if (!pool) return fail(GLA_ERR_INVALID_ARGUMENT, "pool must not be NULL");
  if (n < 0) return fail(GLA_ERR_INVALID_ARGUMENT, "n must be >= 0 (got %lld)", (long long)n);
  if (!slot_idx && n > pool->n_slots)
    return fail(GLA_ERR_INVALID_ARGUMENT, "n=%lld exceeds the pool's %lld slots", (long long)n,
                (long long)pool->n_slots);
  if (n * pool->H > ((int64_t)1 << 31) - 1) return fail(GLA_ERR_UNSUPPORTED, "n*H too large");
  if (n == 0) return ok();
  TRY(check_ptr(S, "S", false));
  if (slot_idx && ((uintptr_t)slot_idx & 3u)) return fail(GLA_ERR_INVALID_ARGUMENT, "slot_idx must be 4-byte aligned");
  TRY(debug_checks((hipStream_t)stream, what, [&](int* f) {
    return debug_slots(slot_idx, n, pool->n_slots, f, (hipStream_t)stream);
  }));
  StateIoArgs a{S, pool->data, Q16Pool{pool->mant, pool->expo}, slot_idx, n, pool->H, write};
  return device_err(launch_state_io(a, (hipStream_t)stream), what);
}


gla_status check_fwd_args(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g,
                          const float* S0, const void* o, const float* S_T) {
  TRY(check_dims(dims));
  TRY(check_ptr(q, "q", false));
  TRY(check_ptr(k, "k", false));
  TRY(check_ptr(v, "v", false));
  TRY(check_ptr(g, "g", false));
  TRY(check_ptr(S0, "S0", true));
  TRY(check_ptr(o, "o", false));
  TRY(check_ptr(S_T, "S_T", true));
  return GLA_OK;
}

// The forward over dense [B,T,H,d] tensors with the plan's workspace at ws.
hipError_t launch_fwd_dense(const gla_dims* dims, const FwdPlan& p, const void* q, const void* k, const void* v,
                            const float* g, const float* S0, void* o, float* S_T, void* ws, hipStream_t st) {
  WalkArgs a = fwd_args(dims, p, q, k, v, g, o, dims->T);
  const int w = DV / p.ns;
  return run_fwd(dims, p, a, state_plain(const_cast<float*>(S0), w), state_plain(S_T, w), ws, st);
}

// ---- Scratch of gla_chunk_fwd_noalloc: the segment plan's workspace in a
// static device array, one copy per device, never allocated by the library.
// Every call on a device shares its copy, so calls that overlap on one device
// race; nothing in it needs to start at zero (pass 1 writes every segment
// entry before the scan and the walks read it).
constexpr size_t kScratchBytes = (size_t)GLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address on the current device, resolved once per
// device with that device current (the array's name in host code is only a
// stand-in for the symbol, never an address to pass to a kernel).
gla_status scratch_ptr(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  TRY(device_err(hipGetDevice(&dev), "hipGetDevice"));
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *out = it->second;
    return GLA_OK;
  }
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    return fail(GLA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
  }
  addr[dev] = p;
  *out = p;
  return GLA_OK;
}

// The backward with fp32 inputs: the bf16 path's walks on the fp32 matrix
// cores.  dq and dk contract over the 192 value columns as two 96-column
// halves (the walk's key width), the second adding the first's sums; their
// values (k for dq, q for dk) are walked in three 32-column slices, and dv in
// three 64-column slices.  Whole sequences, no segment plan.
gla_status bwd_f32(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g, const float* S0,
                   const void* dO, const float* dS_T, void* dq, void* dk, void* dv, float* dg, float* dS0, void* ws,
                   size_t ws_bytes, void* stream) {
  const BwdF32Plan p = plan_bwd_f32(dims);
  const SegPlan& sp = p.sp;
  if (ws_bytes < p.ws_total) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, p.ws_total);
  TRY(check_ptr(ws, "ws", false));
  if (p.n_chunks > 1024) return fail(GLA_ERR_UNSUPPORTED, "the backward supports at most 1024 chunks (T <= 131072)");
  hipStream_t st = (hipStream_t)stream;
  TRY(debug_checks(st, "gla_chunk_bwd", [&](int* f) {
    return debug_decay(g, dims->B, dims->T, dims->H, dims->T * dims->H, dims->H, 1, f, st);
  }));
  char* w = (char*)ws;
  const int64_t BH = dims->B * dims->H;
  const bool bf16_out = dims->out_dtype == GLA_BF16;
  float* adq = (float*)(w + p.off_adq);
  float* adk = (float*)(w + p.off_adk);
  float* fdq = bf16_out ? (float*)(w + p.off_fdq) : (float*)dq;
  float* fdk = bf16_out ? (float*)(w + p.off_fdk) : (float*)dk;
  float* rq = (float*)(w + p.off_rq);
  float* rk = (float*)(w + p.off_rk);
  float* S_T = (float*)(w + p.off_st);
  constexpr int hw = 96, sw = 32, dw = 64;       // dv-half, dq/dk value-slice and dv value-slice widths
  // states of the dq and dk walks: element (x = column of a dv-half, y =
  // row of S) of value slice s, i.e. S[32 s + y][half + x]
  auto tview = [&](const float* base) { return StateView{const_cast<float*>(base), kStateElems, 0, (int64_t)sw * DV, 1, DV}; };
  auto common = [&](WalkArgs& a, bool backwards) {
    a.g = backwards ? g + (dims->T - 1) * dims->H : g;
    a.gsb = dims->T * dims->H;
    a.gsh = 1;
    a.gst = backwards ? -(int64_t)dims->H : dims->H;
    a.gshift = backwards ? 1 : 0;
    a.B = dims->B;
    a.T = dims->T;
    a.H = dims->H;
  };
  hipError_t e = hipSuccess;
  // With segments: the state entering every segment, of the forward
  // recurrence S (keys k, values v) and of the backward-in-time one U (keys
  // q, values dO, log-decay shifted), from state-only walks over 64-column
  // value slices and a scan, in the plain [dk][dv] layout of S0 and dS_T; the
  // walks below read them through their own views.
  float* seg_f = sp.nseg > 1 ? (float*)(w + p.off_segf) : nullptr;
  float* seg_r = sp.nseg > 1 ? (float*)(w + p.off_segr) : nullptr;
  if (sp.nseg > 1) {
    WalkArgs fs{};
    fs.X = tok_view(k, 4, dims, DK, 0, false);
    fs.Y = tok_view(v, 4, dims, DV, dw, false);
    common(fs, false);
    WalkArgs rs{};
    rs.X = tok_view(q, 4, dims, DK, 0, true);
    rs.Y = tok_view(dO, 4, dims, DV, dw, true);
    common(rs, true);
    e = segment_states(fs, WV_FWD_STATE_F32, sp, S0, nullptr, dims->H, seg_view(seg_f, state_plain(nullptr, dw), sp.entries()),
                       (float*)(w + p.off_decf), BH, st);
    if (e == hipSuccess)
      e = segment_states(rs, WV_FWD_STATE_F32, sp, dS_T, nullptr, dims->H,
                         seg_view(seg_r, state_plain(nullptr, dw), sp.entries()), (float*)(w + p.off_decr), BH, st);
    if (e != hipSuccess) return device_err(e, "gla_chunk_bwd segment states");
  }
  // a walk's entering states: the segment states through the walk's view, or
  // the initial state itself (or none) with one segment
  auto entering = [&](StateView lay, float* seg, const float* z0) {
    if (sp.nseg > 1) return coarse(seg_view(seg, lay, sp.entries()), sp);
    lay.p = const_cast<float*>(z0);
    return z0 ? lay : StateView{};
  };
  for (int hh = 0; hh < 2 && e == hipSuccess; ++hh) {
    // dq: forward recurrence with keys a dv-half of v, values k, queries the
    // same half of dO; its state is S^T restricted to the half
    WalkArgs f{};
    f.X = shifted(tok_view(v, 4, dims, DV, 0, false), (int64_t)hh * hw, 4);
    f.Y = tok_view(k, 4, dims, DK, sw, false);
    f.Q = shifted(tok_view(dO, 4, dims, DV, 0, false), (int64_t)hh * hw, 4);
    f.O = tok_view(hh == 0 ? adq : fdq, 4, dims, DK, sw, false);
    if (hh == 1) f.acc = tok_view(adq, 4, dims, DK, sw, false);
    common(f, false);
    const StateView fzT = shifted(tview(dS_T ? S_T : nullptr), (int64_t)hh * hw);
    e = walk_segments(f, WV_OUT_F32_NC1, sp, shifted(entering(tview(nullptr), seg_f, S0), (int64_t)hh * hw),
                      dS_T ? fzT : StateView{}, BH, st);
    if (e != hipSuccess) break;
    // dk: backward in time, keys the half of dO, values q, queries the same
    // half of v; its state is the state gradient's transpose
    WalkArgs r{};
    r.X = shifted(tok_view(dO, 4, dims, DV, 0, true), (int64_t)hh * hw, 4);
    r.Y = tok_view(q, 4, dims, DK, sw, true);
    r.Q = shifted(tok_view(v, 4, dims, DV, 0, true), (int64_t)hh * hw, 4);
    r.O = tok_view(hh == 0 ? adk : fdk, 4, dims, DK, sw, true);
    if (hh == 1) r.acc = tok_view(adk, 4, dims, DK, sw, true);
    common(r, true);
    e = walk_segments(r, WV_OUT_F32_NC1, sp, shifted(entering(tview(nullptr), seg_r, dS_T), (int64_t)hh * hw),
                      StateView{}, BH, st);
  }
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd dq/dk walks");
  // dv: backward in time, keys q, values dO (64-column slices), queries k;
  // the final state is the gradient leaving the first token
  {
    WalkArgs a{};
    a.X = tok_view(q, 4, dims, DK, 0, true);
    a.Y = tok_view(dO, 4, dims, DV, dw, true);
    a.Q = tok_view(k, 4, dims, DK, 0, true);
    a.O = tok_view(dv, bf16_out ? 2 : 4, dims, DV, dw, true);
    common(a, true);
    e = walk_segments(a, bf16_out ? WV_FWD_OUT_F32_BF16 : WV_FWD_OUT_F32_F32, sp,
                      entering(state_plain(nullptr, dw), seg_r, dS_T), state_plain(dS0, dw), BH, st);
    if (e != hipSuccess) return device_err(e, "gla_chunk_bwd dv walk");
  }
  RowDotsArgs rd{(const float*)q, (const float*)k, fdq, fdk, rq, rk, bf16_out ? (__bf16*)dq : nullptr,
                 bf16_out ? (__bf16*)dk : nullptr, dims->B * dims->T * dims->H};
  e = launch_row_dots(rd, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd row dots");
  BwdFinishArgs fa{};
  fa.rq = rq;
  fa.rk = rk;
  fa.dg = dg;
  fa.chunk_r = (float*)(w + p.off_r);
  fa.B = dims->B;
  fa.T = dims->T;
  fa.H = dims->H;
  fa.n_chunks = p.n_chunks;
  e = launch_bwd_finish(fa, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd finish");
  e = launch_dg_finish(dg, fa.chunk_r, dS_T, S_T, dS0, g, dims->B, dims->T, dims->H, p.n_chunks, st);
  return device_err(e, "gla_chunk_bwd dg finish");
}

}  // namespace

extern "C" {

const char* gla_status_str(gla_status s) {
  switch (s) {
    case GLA_OK: return "GLA_OK";
    case GLA_ERR_INVALID_ARGUMENT: return "GLA_ERR_INVALID_ARGUMENT";
    case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED";
    case GLA_ERR_OUT_OF_MEMORY: return "GLA_ERR_OUT_OF_MEMORY";
    case GLA_ERR_DEVICE: return "GLA_ERR_DEVICE";
  }
  return "GLA_ERR_UNKNOWN";
}

const char* gla_last_error(void) { return g_err.c_str(); }

size_t gla_state_slot_bytes(int32_t H, int32_t dk, int32_t dv) {
  if (H < 1 || dk < 1 || dv < 1) return 0;
  return (size_t)H * dk * dv * sizeof(float);
}


gla_status gla_state_alloc(int64_t n_slots, int32_t H, int32_t dk, int32_t dv, void* stream, gla_state** out) {
  return alloc_pool(n_slots, H, dk, dv, GLA_STATE_F32, 0, stream, out);
}

gla_status gla_state_alloc_q16(int64_t n_slots, int32_t H, int32_t dk, int32_t dv, void* stream, gla_state** out) {
  return alloc_pool(n_slots, H, dk, dv, GLA_STATE_Q16, 0, stream, out);
}

gla_status gla_state_alloc_conv(int64_t n_slots, int32_t H, int32_t dk, int32_t dv, int32_t format, int32_t conv_D,
                                void* stream, gla_state** out) {
  if (!out) return fail(GLA_ERR_INVALID_ARGUMENT, "out must not be NULL");
  *out = nullptr;
  TRY(check_conv_D(conv_D));
  return alloc_pool(n_slots, H, dk, dv, format, conv_D, stream, out);
}

int32_t gla_state_conv_channels(const gla_state* pool) { return pool ? pool->conv_D : 0; }

float* gla_state_conv_ptr(const gla_state* pool, int64_t slot) {
  if (!pool || !pool->conv || slot < 0 || slot >= pool->n_slots) return nullptr;
  return pool->conv + slot * (int64_t)CONV_WIN * pool->conv_D;
}

size_t gla_state_seq_bytes(int32_t H, int32_t dk, int32_t dv, int32_t format, int32_t conv_D) {
  if (H < 1 || dk < 1 || dv < 1 || conv_D < 0 || (format != GLA_STATE_F32 && format != GLA_STATE_Q16)) return 0;
  return slot_bytes(H, dk, dv, format, conv_D);
}

int32_t gla_state_format(const gla_state* pool) { return pool ? pool->format : -1; }

gla_status gla_state_q16_ptrs(const gla_state* pool, int64_t slot, int16_t** mant, int32_t** expo) {
  if (!pool || !mant || !expo) return fail(GLA_ERR_INVALID_ARGUMENT, "pool, mant and expo must not be NULL");
  if (pool->format != GLA_STATE_Q16) return fail(GLA_ERR_INVALID_ARGUMENT, "the pool does not hold 16-bit states");
  if (slot < 0 || slot >= pool->n_slots)
    return fail(GLA_ERR_INVALID_ARGUMENT, "slot %lld out of range [0, %lld)", (long long)slot, (long long)pool->n_slots);
  *mant = pool->mant + slot * (int64_t)pool->H * pool->dk * pool->dv;
  *expo = pool->expo + slot * (int64_t)pool->H * pool->dv;
  return ok();
}


gla_status gla_state_write(gla_state* pool, int64_t n, const int32_t* slot_idx, const float* S, void* stream) {
  return state_io(pool, n, slot_idx, const_cast<float*>(S), 1, stream, "gla_state_write launch");
}

gla_status gla_state_read(const gla_state* pool, int64_t n, const int32_t* slot_idx, float* S, void* stream) {
  return state_io(pool, n, slot_idx, S, 0, stream, "gla_state_read launch");
}

gla_status gla_state_free(gla_state* pool) {
  if (!pool) return GLA_OK;
  int cur = 0;
  (void)hipGetDevice(&cur);
  (void)hipSetDevice(pool->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipFree(pool->base);
  (void)hipSetDevice(cur);
  delete pool;
  return device_err(e, "gla_state_free");
}

float* gla_state_ptr(const gla_state* pool, int64_t slot) {
  if (!pool || !pool->data || slot < 0 || slot >= pool->n_slots) return nullptr;
  return pool->data + slot * (int64_t)pool->H * pool->dk * pool->dv;
}

int64_t gla_state_slots(const gla_state* pool) { return pool ? pool->n_slots : 0; }

gla_status gla_workspace_size(int32_t op, const gla_dims* dims, size_t* bytes) {
  if (!bytes) return fail(GLA_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  TRY(check_dims(dims));
  if (op == GLA_OP_FWD) {
    *bytes = plan_fwd(dims).ws_total;
    return ok();
  }
  if (op == GLA_OP_BWD) {
    *bytes = dims->in_dtype == GLA_F32 ? plan_bwd_f32(dims).ws_total : plan_bwd(dims).ws_total;
    return ok();
  }
  if (op == GLA_OP_FWD_VARLEN_Q16) {
    *bytes = plan_fwd(dims).ws_total + stage_bytes(dims);
    return ok();
  }
  return fail(GLA_ERR_INVALID_ARGUMENT, "op must be GLA_OP_FWD, GLA_OP_BWD or GLA_OP_FWD_VARLEN_Q16 (got %d)", op);
}

gla_status gla_chunk_fwd(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g,
                         const float* S0, void* o, float* S_T, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_fwd_args(dims, q, k, v, g, S0, o, S_T));
  const FwdPlan p = plan_fwd(dims);
  if (ws_bytes < p.ws_total) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, p.ws_total);
  if (p.ws_total > 0) TRY(check_ptr(ws, "ws", false));
  TRY(debug_checks((hipStream_t)stream, "gla_chunk_fwd", [&](int* f) {
    return debug_decay(g, dims->B, dims->T, dims->H, dims->T * dims->H, dims->H, 1, f, (hipStream_t)stream);
  }));
  return device_err(launch_fwd_dense(dims, p, q, k, v, g, S0, o, S_T, ws, (hipStream_t)stream), "gla_chunk_fwd launch");
}

gla_status gla_chunk_fwd_noalloc(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g,
                                 const float* S0, void* o, float* S_T, void* stream) {
  TRY(check_fwd_args(dims, q, k, v, g, S0, o, S_T));
  const FwdPlan p = plan_fwd(dims);
  if (p.ws_total > kScratchBytes)
    return fail(GLA_ERR_UNSUPPORTED,
                "gla_chunk_fwd_noalloc: this plan needs %zu bytes of scratch, more than the library's static "
                "%zu-byte array; call gla_chunk_fwd with a workspace",
                p.ws_total, kScratchBytes);
  void* ws = nullptr;
  if (p.ws_total > 0) TRY(scratch_ptr(&ws));
  return device_err(launch_fwd_dense(dims, p, q, k, v, g, S0, o, S_T, ws, (hipStream_t)stream),
                    "gla_chunk_fwd_noalloc launch");
}

gla_status gla_chunk_fwd_strided(const gla_dims* dims, const void* q, const gla_strides* sq, const void* k,
                                 const gla_strides* sk, const void* v, const gla_strides* sv, const float* g,
                                 const gla_strides* sg, const void* gate, const gla_strides* sgate,
                                 const float* S0, void* o, const gla_strides* so, float* S_T, void* ws,
                                 size_t ws_bytes, void* stream) {
  TRY(check_dims(dims));
  TRY(check_ptr(q, "q", false));
  TRY(check_ptr(k, "k", false));
  TRY(check_ptr(v, "v", false));
  if (!g || ((uintptr_t)g & 3u)) return fail(GLA_ERR_INVALID_ARGUMENT, "g must be a non-NULL, 4-byte aligned pointer");
  TRY(check_ptr(S0, "S0", true));
  TRY(check_ptr(o, "o", false));
  TRY(check_ptr(S_T, "S_T", true));
  const size_t isz = dims->in_dtype == GLA_BF16 ? 2 : 4, osz = dims->out_dtype == GLA_BF16 ? 2 : 4;
  TRY(check_strides(sq, isz, true, "q"));
  TRY(check_strides(sk, isz, true, "k"));
  TRY(check_strides(sv, isz, true, "v"));
  TRY(check_strides(so, osz, true, "o"));
  TRY(check_strides(sg, 4, false, "g"));
  TRY(check_ptr(gate, "gate", true));
  if (!gate && sgate) return fail(GLA_ERR_INVALID_ARGUMENT, "gate strides given without a gate");
  TRY(check_strides(sgate, isz, true, "gate"));
  const FwdPlan p = plan_fwd(dims);
  if (ws_bytes < p.ws_total) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, p.ws_total);
  if (p.ws_total > 0) TRY(check_ptr(ws, "ws", false));
  TRY(debug_checks((hipStream_t)stream, "gla_chunk_fwd_strided", [&](int* f) {
    return sg ? debug_decay(g, dims->B, dims->T, dims->H, sg->batch, sg->token, sg->head, f, (hipStream_t)stream)
              : debug_decay(g, dims->B, dims->T, dims->H, dims->T * dims->H, dims->H, 1, f, (hipStream_t)stream);
  }));
  WalkArgs a = fwd_args(dims, p, q, k, v, g, o, dims->T);
  const int w = DV / p.ns;
  if (sq) a.Q = strided_view(q, *sq, 0);
  if (sk) a.X = strided_view(k, *sk, 0);
  if (sv) a.Y = strided_view(v, *sv, w);
  if (so) a.O = strided_view(o, *so, w);
  if (gate) a.G = sgate ? strided_view(gate, *sgate, w) : tok_view(gate, isz, dims, DV, w, false);
  if (sg) {
    a.gsb = sg->batch;
    a.gst = sg->token;
    a.gsh = sg->head;
  }
  const hipError_t e = run_fwd(dims, p, a, state_plain(const_cast<float*>(S0), w), state_plain(S_T, w), ws,
                               (hipStream_t)stream);
  return device_err(e, "gla_chunk_fwd_strided launch");
}

gla_status gla_chunk_fwd_varlen(const gla_dims* dims, int64_t total_tokens, const int32_t* cu_seqlens, const void* q,
                                const void* k, const void* v, const float* g, gla_state* pool,
                                const int32_t* slot_idx, int32_t init_from_pool, void* o, void* ws, size_t ws_bytes,
                                void* stream) {
  TRY(check_dims(dims));
  if (total_tokens < 0 || total_tokens > INT32_MAX)
    return fail(GLA_ERR_INVALID_ARGUMENT, "total_tokens must be in [0, 2^31) (got %lld)", (long long)total_tokens);
  if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u))
    return fail(GLA_ERR_INVALID_ARGUMENT, "cu_seqlens must be a non-NULL, 4-byte aligned device array");
  if (slot_idx && ((uintptr_t)slot_idx & 3u)) return fail(GLA_ERR_INVALID_ARGUMENT, "slot_idx must be 4-byte aligned");
  if (!pool) return fail(GLA_ERR_INVALID_ARGUMENT, "pool must not be NULL");
  if (pool->H != dims->H || pool->dk != dims->dk || pool->dv != dims->dv)
    return fail(GLA_ERR_INVALID_ARGUMENT, "pool holds H=%d dk=%d dv=%d, call has H=%d dk=%d dv=%d", pool->H,
                pool->dk, pool->dv, dims->H, dims->dk, dims->dv);
  if (!slot_idx && dims->B > pool->n_slots)
    return fail(GLA_ERR_INVALID_ARGUMENT, "B=%lld sequences exceed the pool's %lld slots", (long long)dims->B,
                (long long)pool->n_slots);
  if (init_from_pool != 0 && init_from_pool != 1)
    return fail(GLA_ERR_INVALID_ARGUMENT, "init_from_pool must be 0 or 1 (got %d)", init_from_pool);
  const bool no_tokens = total_tokens == 0;      // every sequence empty: token tensors may be NULL
  TRY(check_ptr(q, "q", no_tokens));
  TRY(check_ptr(k, "k", no_tokens));
  TRY(check_ptr(v, "v", no_tokens));
  TRY(check_ptr(g, "g", no_tokens));
  TRY(check_ptr(o, "o", no_tokens));
  const FwdPlan p = plan_fwd(dims);
  const bool q16 = pool->format == GLA_STATE_Q16;
  const size_t need = p.ws_total + (q16 ? stage_bytes(dims) : 0);
  if (ws_bytes < need) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, need);
  if (need > 0) TRY(check_ptr(ws, "ws", false));
  TRY(debug_checks((hipStream_t)stream, "gla_chunk_fwd_varlen", [&](int* f) {
    hipStream_t s_ = (hipStream_t)stream;
    hipError_t e_ = debug_offsets(cu_seqlens, dims->B, total_tokens, dims->T, f, s_);
    if (e_ == hipSuccess) e_ = debug_slots(slot_idx, dims->B, pool->n_slots, f, s_);
    if (e_ == hipSuccess && total_tokens > 0) e_ = debug_decay(g, 1, total_tokens, dims->H, 0, dims->H, 1, f, s_);
    return e_;
  }));
  // packed [total_tokens, H, cols] tensors: one "batch" row holding every token
  gla_dims packed = *dims;
  packed.B = 1;
  packed.T = total_tokens;
  WalkArgs a = fwd_args(&packed, p, q, k, v, g, o, dims->T);
  a.X.sb = a.Y.sb = a.Q.sb = a.O.sb = 0;
  a.gsb = 0;
  a.B = dims->B;
  a.cu = cu_seqlens;
  a.cu_total = total_tokens;
  const int w = DV / p.ns;
  if (!q16) {
    a.zinit_idx = a.zfin_idx = slot_idx;
    const StateView zfin = state_plain(pool->data, w);
    const StateView z0 = init_from_pool ? zfin : state_plain(nullptr, w);
    const hipError_t e = run_fwd(dims, p, a, z0, zfin, ws, (hipStream_t)stream);
    return device_err(e, "gla_chunk_fwd_varlen launch");
  }
  // 16-bit pool: sequence b's float32 state is row b of the staging area
  float* stage = (float*)((char*)ws + p.ws_total);
  const Q16Pool qp{pool->mant, pool->expo};
  hipError_t e = hipSuccess;
  if (init_from_pool) e = launch_state_io(StateIoArgs{stage, nullptr, qp, slot_idx, dims->B, dims->H, 0}, (hipStream_t)stream);
  a.zinit_idx = a.zfin_idx = nullptr;
  const StateView zfin = state_plain(stage, w);
  const StateView z0 = init_from_pool ? zfin : state_plain(nullptr, w);
  if (e == hipSuccess) e = run_fwd(dims, p, a, z0, zfin, ws, (hipStream_t)stream);
  if (e == hipSuccess)
    e = launch_state_io(StateIoArgs{stage, nullptr, qp, slot_idx, dims->B, dims->H, 1}, (hipStream_t)stream);
  return device_err(e, "gla_chunk_fwd_varlen launch");
}

gla_status gla_recurrent_step(int64_t B, int32_t H, int32_t dk, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                              const void* q, const void* k, const void* v, const float* g, gla_state* pool,
                              const int32_t* slot_idx, void* o, void* stream) {
  if (B < 1) return fail(GLA_ERR_INVALID_ARGUMENT, "B must be >= 1 (got %lld)", (long long)B);
  TRY(check_heads(H, dk, dv));
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(GLA_ERR_INVALID_ARGUMENT, "in_dtype/out_dtype must be GLA_F32 or GLA_BF16");
  if (!pool) return fail(GLA_ERR_INVALID_ARGUMENT, "pool must not be NULL");
  if (pool->H != H || pool->dk != dk || pool->dv != dv)
    return fail(GLA_ERR_INVALID_ARGUMENT, "pool holds H=%d dk=%d dv=%d, call has H=%d dk=%d dv=%d", pool->H,
                pool->dk, pool->dv, H, dk, dv);
  if (!slot_idx && B > pool->n_slots)
    return fail(GLA_ERR_INVALID_ARGUMENT, "B=%lld exceeds the pool's %lld slots", (long long)B,
                (long long)pool->n_slots);
  if (B * H > ((int64_t)1 << 31) - 1) return fail(GLA_ERR_UNSUPPORTED, "B*H too large");
  TRY(check_ptr(q, "q", false));
  TRY(check_ptr(k, "k", false));
  TRY(check_ptr(v, "v", false));
  if (!g) return fail(GLA_ERR_INVALID_ARGUMENT, "g must not be NULL");
  if (slot_idx && ((uintptr_t)slot_idx & 3u)) return fail(GLA_ERR_INVALID_ARGUMENT, "slot_idx must be 4-byte aligned");
  TRY(check_ptr(o, "o", false));
  TRY(debug_checks((hipStream_t)stream, "gla_recurrent_step", [&](int* f) {
    hipError_t e_ = debug_slots(slot_idx, B, pool->n_slots, f, (hipStream_t)stream);
    if (e_ == hipSuccess) e_ = debug_decay(g, B, 1, H, H, 0, 1, f, (hipStream_t)stream);
    return e_;
  }));
  if (pool->format == GLA_STATE_Q16) {
    StepQ16Args a{q, k, v, g, Q16Pool{pool->mant, pool->expo}, slot_idx, o, B, H};
    return device_err(launch_step_q16(a, in_dtype == GLA_BF16, out_dtype == GLA_BF16, (hipStream_t)stream),
                      "gla_recurrent_step launch");
  }
  StepArgs a{q, k, v, g, pool->data, slot_idx, o, B, H};
  return device_err(launch_step(a, in_dtype == GLA_BF16, out_dtype == GLA_BF16, (hipStream_t)stream),
                    "gla_recurrent_step launch");
}

namespace {

// The convolution over [B,T,D] or packed rows, with the window rows of
// `window` ([slots][4][D] float32, or null) addressed through slot_idx.
gla_status conv_call(int64_t B, int64_t T, int32_t D, int32_t in_dtype, int32_t out_dtype, const int32_t* cu_seqlens,
                     int64_t total_tokens, const void* x, const float* w, const float* bias, float* window,
                     int64_t n_slots, const int32_t* slot_idx, int32_t init, void* y, void* stream,
                     const char* name) {
  if (B < 1 || T < 1) return fail(GLA_ERR_INVALID_ARGUMENT, "B and T must be >= 1 (got B=%lld, T=%lld)",
                                  (long long)B, (long long)T);
  TRY(check_conv_D(D));
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(GLA_ERR_INVALID_ARGUMENT, "in_dtype/out_dtype must be GLA_F32 or GLA_BF16");
  if (cu_seqlens) {
    if ((uintptr_t)cu_seqlens & 3u) return fail(GLA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
    if (total_tokens < 0 || total_tokens > INT32_MAX)
      return fail(GLA_ERR_INVALID_ARGUMENT, "total_tokens must be in [0, 2^31) (got %lld)", (long long)total_tokens);
  } else if (B > INT64_MAX / T) {
    return fail(GLA_ERR_UNSUPPORTED, "B*T too large");
  }
  if (B > ((int64_t)1 << 36) / (T * (D / 8))) return fail(GLA_ERR_UNSUPPORTED, "B*T*D too large");
  if (init != 0 && init != 1) return fail(GLA_ERR_INVALID_ARGUMENT, "%s: the init flag must be 0 or 1 (got %d)", name, init);
  TRY(check_ptr(x, "x", false));
  TRY(check_ptr(w, "w", false));
  TRY(check_ptr(bias, "bias", true));
  if (slot_idx && ((uintptr_t)slot_idx & 3u)) return fail(GLA_ERR_INVALID_ARGUMENT, "slot_idx must be 4-byte aligned");
  TRY(check_ptr(y, "y", false));
  TRY(debug_checks((hipStream_t)stream, name, [&](int* f) {
    hipError_t e_ = cu_seqlens ? debug_offsets(cu_seqlens, B, total_tokens, T, f, (hipStream_t)stream) : hipSuccess;
    if (e_ == hipSuccess && window) e_ = debug_slots(slot_idx, B, n_slots, f, (hipStream_t)stream);
    return e_;
  }));
  ConvArgs a{};
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.state = window;
  a.slot = slot_idx;
  a.cu = cu_seqlens;
  a.B = B;
  a.T = T;
  a.total = cu_seqlens ? total_tokens : B * T;
  a.D = D;
  a.init = init;
  a.y = y;
  return device_err(launch_conv(a, in_dtype == GLA_BF16, out_dtype == GLA_BF16, (hipStream_t)stream), name);
}

}  // namespace

gla_status gla_conv1d_silu(int64_t B, int64_t T, int32_t D, int32_t in_dtype, int32_t out_dtype,
                           const int32_t* cu_seqlens, int64_t total_tokens, const void* x, const float* w,
                           const float* bias, float* conv_state, const int32_t* slot_idx, int32_t init_from_state,
                           void* y, void* stream) {
  if (init_from_state && !conv_state)
    return fail(GLA_ERR_INVALID_ARGUMENT, "init_from_state needs conv_state");
  TRY(check_ptr(conv_state, "conv_state", true));
  // the window tensor is the caller's: its slot count is unknown here, so
  // only negative and repeated indices are caught under GLA_DEBUG
  return conv_call(B, T, D, in_dtype, out_dtype, cu_seqlens, total_tokens, x, w, bias, conv_state, INT64_MAX,
                   slot_idx, init_from_state, y, stream, "gla_conv1d_silu");
}

gla_status gla_conv1d_silu_pool(int64_t B, int64_t T, int32_t in_dtype, int32_t out_dtype, const int32_t* cu_seqlens,
                                int64_t total_tokens, const void* x, const float* w, const float* bias,
                                gla_state* pool, const int32_t* slot_idx, int32_t init_from_pool, void* y,
                                void* stream) {
  if (!pool) return fail(GLA_ERR_INVALID_ARGUMENT, "pool must not be NULL");
  if (!pool->conv) return fail(GLA_ERR_INVALID_ARGUMENT, "the pool has no convolution window (gla_state_alloc_conv)");
  if (!slot_idx && B > pool->n_slots)
    return fail(GLA_ERR_INVALID_ARGUMENT, "B=%lld sequences exceed the pool's %lld slots", (long long)B,
                (long long)pool->n_slots);
  return conv_call(B, T, pool->conv_D, in_dtype, out_dtype, cu_seqlens, total_tokens, x, w, bias, pool->conv,
                   pool->n_slots, slot_idx, init_from_pool, y, stream, "gla_conv1d_silu_pool");
}

}  // extern "C"

namespace {
// The log-decay gradient of the bf16 backward from the dot products q.dq and
// k.dk the second-half walks left per token: in-chunk suffix sums, then the
// later chunks' totals and <dS_T, S_T>; dS0 through the first decay.
gla_status bwd_tail(const gla_dims* dims, const BwdPlan& p, const float* rq, const float* rk, float* dg,
                    const float* dS_T, const float* S_T, float* dS0, const float* g, char* w, hipStream_t st) {
  BwdFinishArgs fa{};
  fa.rq = rq;
  fa.rk = rk;
  fa.dg = dg;
  fa.chunk_r = (float*)(w + p.off_r);
  fa.B = dims->B;
  fa.T = dims->T;
  fa.H = dims->H;
  fa.n_chunks = p.sp.n_chunks;
  hipError_t e = launch_bwd_finish(fa, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd finish");
  e = launch_dg_finish(dg, fa.chunk_r, dS_T, S_T, dS0, g, dims->B, dims->T, dims->H, p.sp.n_chunks, st);
  return device_err(e, "gla_chunk_bwd dg finish");
}
}  // namespace

extern "C" {

gla_status gla_chunk_bwd(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g,
                         const float* S0, const void* dO, const float* dS_T, void* dq, void* dk, void* dv, float* dg,
                         float* dS0, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(dims));
  TRY(check_ptr(q, "q", false));
  TRY(check_ptr(k, "k", false));
  TRY(check_ptr(v, "v", false));
  TRY(check_ptr(g, "g", false));
  TRY(check_ptr(S0, "S0", true));
  TRY(check_ptr(dO, "dO", false));
  TRY(check_ptr(dS_T, "dS_T", true));
  TRY(check_ptr(dq, "dq", false));
  TRY(check_ptr(dk, "dk", false));
  TRY(check_ptr(dv, "dv", false));
  TRY(check_ptr(dg, "dg", false));
  TRY(check_ptr(dS0, "dS0", true));
  if (dims->in_dtype == GLA_F32) return bwd_f32(dims, q, k, v, g, S0, dO, dS_T, dq, dk, dv, dg, dS0, ws, ws_bytes, stream);
  const BwdPlan p = plan_bwd(dims);
  if (ws_bytes < p.ws_total) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, p.ws_total);
  TRY(check_ptr(ws, "ws", false));
  if (p.sp.n_chunks > 1024) return fail(GLA_ERR_UNSUPPORTED, "the backward supports at most 1024 chunks (T <= 131072)");
  char* w = (char*)ws;
  const int64_t BH = dims->B * dims->H;
  const SegPlan& sp = p.sp;
  const int hw = 96;                              // dv-half width
  const size_t osz = dims->out_dtype == GLA_BF16 ? 2 : 4;
  const int out_variant = dims->out_dtype == GLA_BF16 ? WV_FWD_OUT_BF16_BF16 : WV_FWD_OUT_BF16_F32;
  hipStream_t st = (hipStream_t)stream;
  TRY(debug_checks(st, "gla_chunk_bwd", [&](int* f) {
    return debug_decay(g, dims->B, dims->T, dims->H, dims->T * dims->H, dims->H, 1, f, st);
  }));
  float* dq_part = (float*)(w + p.off_dq);
  float* dk_part = (float*)(w + p.off_dk);
  float* rq = (float*)(w + p.off_rq);
  float* rk = (float*)(w + p.off_rk);
  float* S_T = (float*)(w + p.off_st);
  float* seg_f = sp.nseg > 1 ? (float*)(w + p.off_segf) : nullptr;
  float* seg_r = sp.nseg > 1 ? (float*)(w + p.off_segr) : nullptr;

  // 1. dq.  Forward recurrence with keys = a dv-half of v, values = k (its
  //    state is the half of S^T), queries = the same half of dO; the two
  //    halves are sums over the two halves of the value width.  Also S_T when
  //    dS_T is given.
  WalkArgs f{};
  f.X = tok_view(v, 2, dims, DV, hw, false);
  f.Y = tok_view(k, 2, dims, DK, 0, false);
  f.Q = tok_view(dO, 2, dims, DV, hw, false);
  f.O = tok_view(dq_part, 4, dims, DK, 0, false);
  f.g = g;
  f.gsb = dims->T * dims->H;
  f.gsh = 1;
  f.gst = dims->H;
  f.B = dims->B;
  f.T = dims->T;
  f.H = dims->H;
  const StateView f0 = state_transposed(const_cast<float*>(S0), hw);
  const StateView ffin = state_transposed(dS_T ? S_T : nullptr, hw);

  // 2. The state gradient, backwards in time: U_t = e^{g_{t+1}} U_{t+1} +
  //    q_t^T dO_t from U = dS_T, i.e. the forward recurrence over the
  //    reversed tokens with keys q, values a dv-half of dO and the log-decay
  //    shifted by one token.
  WalkArgs r{};
  r.X = tok_view(q, 2, dims, DK, 0, true);
  r.Y = tok_view(dO, 2, dims, DV, hw, true);
  r.g = g + (dims->T - 1) * dims->H;
  r.gsb = dims->T * dims->H;
  r.gsh = 1;
  r.gst = -(int64_t)dims->H;
  r.gshift = 1;
  r.B = dims->B;
  r.T = dims->T;
  r.H = dims->H;
  const StateView r0 = state_plain(const_cast<float*>(dS_T), hw);

  // 2a. dv: queries k, outputs dv (a dv-half per slice); the final state is
  //     the gradient leaving the first token (dS0 after its decay, below).
  WalkArgs rv = r;
  rv.Q = tok_view(k, 2, dims, DK, 0, true);
  rv.O = tok_view(dv, osz, dims, DV, hw, true);
  // 2b. dk: keys a dv-half of dO, values q (the state is the transpose),
  //     queries the same half of v.
  WalkArgs rk_ = r;
  rk_.X = tok_view(dO, 2, dims, DV, hw, true);
  rk_.Y = tok_view(q, 2, dims, DK, 0, true);
  rk_.Q = tok_view(v, 2, dims, DV, hw, true);
  rk_.O = tok_view(dk_part, 4, dims, DK, 0, true);

  // dq and dk run as one walk per dv-half.  The first half writes fp32 sums;
  // the second adds them to its own (a fixed order), writes the gradient and
  // its dot product with q (k) for the log-decay gradient.
  SegPlan sp1 = sp;
  sp1.ns = 1;
  auto half = [&](WalkArgs a, int hh) {
    a.X = shifted(a.X, (int64_t)hh * hw, 2);
    a.Q = shifted(a.Q, (int64_t)hh * hw, 2);
    return a;
  };
  auto second_half = [&](WalkArgs a, const TokView& part, void* out, const void* dotted, float* rdot, bool backwards) {
    a.acc = part;
    a.O = tok_view(out, osz, dims, DK, 0, backwards);
    a.D = tok_view(dotted, 2, dims, DK, 0, backwards);
    a.rdot = token_floats(rdot, dims, backwards);
    return a;
  };
  StateView rk0 = r0;                                  // dk's state is the transpose of dv's
  rk0.sx = r0.sy;
  rk0.sy = r0.sx;
  hipError_t e = hipSuccess;

  if (sp.nseg == 2) {
    // Two segments, staggered over three launches instead of a state pass
    // and a scan: each walk's second segment starts from the state that its
    // first segment (the same walk, or the dv walk of the same recurrence)
    // left in the workspace one launch earlier, and the second dv-half of dq
    // and dk follows its first half by one launch.
    //   launch 0: dq, dk first half, segment 0; dv, segment 0
    //   launch 1: dq, dk second half, segment 0; dq, dk first half, segment 1
    //   launch 2: dq, dk second half, segment 1; dv, segment 1
    // Every launch holds 4 B H walks of the same length.
    // Segment 0 is the shorter: the second-half walks of launch 2 (the
    // slowest walks) then cover fewer chunks, the first-half walks running
    // beside them more, which balances the launches (13 of 32 chunks at the
    // training shape).
    const int c0 = std::max(1, std::min(sp.n_chunks - 1, (sp.n_chunks * 13 + 16) / 32));
    SegPlan s0 = sp, s1 = sp;
    s0.cps = c0;
    s1.cps = sp.n_chunks - c0;
    SegPlan s0h = s0, s1h = s1;
    s0h.ns = s1h.ns = 1;
    StateView fmid = state_transposed((float*)(w + p.off_segf), hw);   // S entering segment 1
    StateView rmid = state_plain((float*)(w + p.off_segr), hw);        // U entering segment 1 (reversed time)
    StateView rkmid = rmid;
    rkmid.sx = rmid.sy;
    rkmid.sy = rmid.sx;
    auto seg_walk = [&](WalkArgs a, const SegPlan& plan, int seg, StateView zinit, StateView zfin) {
      a = segments_args(a, plan, zinit, zfin);
      a.zfin_only_seg = -1;
      a.nseg_launch = 1;
      a.seg_offset = 0;
      a.chunk0 = seg ? c0 : 0;
      return a;
    };
    const TokView dq_acc = tok_view(dq_part, 4, dims, DK, 0, false);
    const TokView dk_acc = tok_view(dk_part, 4, dims, DK, 0, true);
    const int n1 = (int)BH, n2 = (int)(BH * sp.ns);
    const bool bf = dims->out_dtype == GLA_BF16;
    WalkArgs l0[4] = {seg_walk(half(f, 0), s0h, 0, f0, fmid), seg_walk(half(rk_, 0), s0h, 0, rk0, StateView{}),
                      seg_walk(rv, s0, 0, r0, rmid), WalkArgs{}};
    const int nw0[4] = {n1, n1, n2, 0};
    e = launch_out_walk_quad(l0, nw0, bf ? QUAD_F32_BF16 : QUAD_F32_F32, st);
    if (e != hipSuccess) return device_err(e, "gla_chunk_bwd walks, launch 0");
    WalkArgs l1[4] = {seg_walk(second_half(half(f, 1), dq_acc, dq, q, rq, false), s0h, 0, shifted(f0, hw),
                               shifted(fmid, hw)),
                      seg_walk(second_half(half(rk_, 1), dk_acc, dk, k, rk, true), s0h, 0, shifted(rk0, hw),
                               StateView{}),
                      seg_walk(half(f, 0), s1h, 1, fmid, ffin), seg_walk(half(rk_, 0), s1h, 1, rkmid, StateView{})};
    const int nw1[4] = {n1, n1, n1, n1};
    e = launch_out_walk_quad(l1, nw1, bf ? QUAD_ACC_BF16_F32 : QUAD_ACC_F32_F32, st);
    if (e != hipSuccess) return device_err(e, "gla_chunk_bwd walks, launch 1");
    WalkArgs l2[4] = {seg_walk(second_half(half(f, 1), dq_acc, dq, q, rq, false), s1h, 1, shifted(fmid, hw),
                               shifted(ffin, hw)),
                      seg_walk(second_half(half(rk_, 1), dk_acc, dk, k, rk, true), s1h, 1, shifted(rkmid, hw),
                               StateView{}),
                      seg_walk(rv, s1, 1, rmid, state_plain(dS0, hw)), WalkArgs{}};
    const int nw2[4] = {n1, n1, n2, 0};
    e = launch_out_walk_quad(l2, nw2, bf ? QUAD_ACC_BF16_BF16 : QUAD_ACC_F32_F32, st);
    if (e != hipSuccess) return device_err(e, "gla_chunk_bwd walks, launch 2");
    return bwd_tail(dims, p, rq, rk, dg, dS_T, S_T, dS0, g, w, st);
  }

  // Segment states of both recurrences: their pass-1 walks share one launch.
  StateView fseg = f0, rseg = r0;
  if (sp.nseg > 1) {
    fseg = seg_view(seg_f, f0, sp.entries());
    rseg = seg_view(seg_r, r0, sp.entries());
    float* dec_f = (float*)(w + p.off_decf);
    float* dec_r = (float*)(w + p.off_decr);
    const int n1 = pass1_workgroups(sp, BH);
    e = launch_state_walk_pair(pass1_args(f, sp, fseg, dec_f), n1, pass1_args(r, sp, rseg, dec_r), n1, st);
    if (e == hipSuccess) e = launch_seg_scan(fseg.p, dec_f, S0, nullptr, dims->H, BH, sp.entries(), 0, st);
    if (e == hipSuccess) e = launch_seg_scan(rseg.p, dec_r, dS_T, nullptr, dims->H, BH, sp.entries(), 0, st);
    if (e != hipSuccess) return device_err(e, "gla_chunk_bwd segment states");
    fseg = coarse(fseg, sp);
    rseg = coarse(rseg, sp);
  }
  StateView rkseg = rseg;
  rkseg.sx = rseg.sy;
  rkseg.sy = rseg.sx;
  WalkArgs q0 = segments_args(half(f, 0), sp1, fseg, ffin);
  WalkArgs k0 = segments_args(half(rk_, 0), sp1, rkseg, StateView{});
  WalkArgs q1 = segments_args(second_half(half(f, 1), q0.O, dq, q, rq, false), sp1, shifted(fseg, hw),
                              shifted(ffin, hw));
  WalkArgs k1 = segments_args(second_half(half(rk_, 1), k0.O, dk, k, rk, true), sp1, shifted(rkseg, hw), StateView{});
  const int nw = (int)(BH * sp1.nseg);
  e = launch_out_walk_pair(q0, nw, k0, nw, 0, st);
  if (e == hipSuccess) e = launch_out_walk_pair(q1, nw, k1, nw, dims->out_dtype == GLA_BF16, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd dq/dk walks");
  e = walk_segments(rv, out_variant, sp, rseg, state_plain(dS0, hw), BH, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd dv walk");
  return bwd_tail(dims, p, rq, rk, dg, dS_T, S_T, dS0, g, w, st);
}

}  // extern "C"
