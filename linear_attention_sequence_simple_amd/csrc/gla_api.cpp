// Host side of libgla: the C ABI declared in include/gla.h.
//
// Every call validates its arguments before touching the HIP runtime, picks a
// launch plan, carves the caller's workspace, and enqueues kernels on the
// caller's stream without synchronising.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "gla.h"
#include "gla_kernels.h"

using namespace gla;

struct gla_state {
  float* data;
  int64_t n_slots;
  int32_t H, dk, dv;
  int device;
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
  if ((d->T + CH - 1) / CH > (1 << 20)) return fail(GLA_ERR_UNSUPPORTED, "T too large");
  return GLA_OK;
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

constexpr int64_t kStateElems = (int64_t)DK * DV;
constexpr int kTargetWorkgroups = 256;   // one per compute unit

// Segments per (batch, head, slice) walk: enough workgroups to cover the
// chip, at least two chunks per segment.
int plan_segments(int64_t walkers, int n_chunks, const char* env) {
  int nseg = (int)std::max<int64_t>(1, (kTargetWorkgroups + walkers - 1) / walkers);
  nseg = std::min(nseg, std::max(1, n_chunks / 2));
  const int forced = env_int(env, 0);
  if (forced > 0) nseg = std::min(forced, n_chunks);
  return std::max(1, nseg);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct FwdPlan {
  int variant, ns, nseg, cps, n_chunks;
  size_t ws_seg_states, ws_seg_decay, ws_total;
};

FwdPlan plan_fwd(const gla_dims* d) {
  FwdPlan p{};
  const bool in_bf16 = d->in_dtype == GLA_BF16, out_bf16 = d->out_dtype == GLA_BF16;
  p.variant = in_bf16 ? (out_bf16 ? WV_FWD_OUT_BF16_BF16 : WV_FWD_OUT_BF16_F32)
                      : (out_bf16 ? WV_FWD_OUT_F32_BF16 : WV_FWD_OUT_F32_F32);
  p.ns = walk_slices(p.variant);
  p.n_chunks = (int)((d->T + CH - 1) / CH);
  p.nseg = plan_segments(d->B * d->H * p.ns, p.n_chunks, "GLA_FWD_SEGMENTS");
  p.cps = (p.n_chunks + p.nseg - 1) / p.nseg;
  p.nseg = (p.n_chunks + p.cps - 1) / p.cps;
  const int64_t BH = d->B * d->H;
  if (p.nseg > 1) {
    p.ws_seg_states = align256((size_t)BH * p.nseg * kStateElems * sizeof(float));
    p.ws_seg_decay = align256((size_t)BH * p.nseg * sizeof(float));
  }
  p.ws_total = p.ws_seg_states + p.ws_seg_decay;
  return p;
}

// Runs the state walk of one direction over all chunks, with segment-parallel
// passes when nseg > 1: pass 1 (state change of each segment from zero, all
// but the segment that ends the walk), a scan over segments, then the full
// walk of every segment from its entering state.
hipError_t run_walk(WalkArgs base, int variant, int ns, int nseg, int cps, int n_chunks, bool rev,
                    const float* Z0, float* Zfin, float* seg_states, float* seg_decay, int64_t BH,
                    hipStream_t st) {
  base.ns = ns;
  base.n_chunks = n_chunks;
  base.cps = cps;
  if (nseg == 1) {
    base.zinit = Z0;
    base.zinit_bh_stride = kStateElems;
    base.zinit_seg_stride = 0;
    base.zfin = Zfin;
    base.zfin_bh_stride = kStateElems;
    base.zfin_seg_stride = 0;
    base.zfin_only_seg = -1;
    base.seg_decay = nullptr;
    base.nseg_launch = 1;
    base.seg_offset = 0;
    return launch_walk(base, variant, (int)(BH * ns), st);
  }
  // pass 1: state change per segment, without outputs or per-chunk exports
  WalkArgs p1 = base;
  const int state_variant = (variant == WV_REV_BF16) ? WV_REV_BF16
                            : (variant == WV_FWD_OUT_F32_F32 || variant == WV_FWD_OUT_F32_BF16 ||
                               variant == WV_FWD_STATE_F32)
                                ? WV_FWD_STATE_F32
                                : WV_FWD_STATE_BF16;
  p1.Q = nullptr;
  p1.O = nullptr;
  p1.st_dc = p1.st_cd = nullptr;
  p1.zinit = nullptr;
  p1.zfin = seg_states;
  p1.zfin_bh_stride = (int64_t)nseg * kStateElems;
  p1.zfin_seg_stride = kStateElems;
  p1.zfin_only_seg = -1;
  p1.seg_decay = seg_decay;
  p1.seg_decay_bh_stride = nseg;
  p1.nseg_launch = nseg - 1;
  p1.seg_offset = rev ? 1 : 0;
  hipError_t e = launch_walk(p1, state_variant, (int)(BH * ns * (nseg - 1)), st);
  if (e != hipSuccess) return e;
  e = launch_seg_scan(seg_states, seg_decay, Z0, BH, nseg, rev ? 1 : 0, st);
  if (e != hipSuccess) return e;
  WalkArgs p2 = base;
  p2.zinit = seg_states;
  p2.zinit_bh_stride = (int64_t)nseg * kStateElems;
  p2.zinit_seg_stride = kStateElems;
  p2.zfin = Zfin;
  p2.zfin_bh_stride = kStateElems;
  p2.zfin_seg_stride = 0;
  p2.zfin_only_seg = rev ? 0 : nseg - 1;
  p2.seg_decay = nullptr;
  p2.nseg_launch = nseg;
  p2.seg_offset = 0;
  return launch_walk(p2, variant, (int)(BH * ns * nseg), st);
}

struct BwdPlan {
  int n_chunks, nseg_f, cps_f, nseg_r, cps_r, ns;
  size_t off_s, off_dsdc, off_dscd, off_st, off_r, off_seg, off_dec, ws_total;
};

BwdPlan plan_bwd(const gla_dims* d) {
  BwdPlan p{};
  p.n_chunks = (int)((d->T + CH - 1) / CH);
  p.ns = walk_slices(WV_REV_BF16);
  const int64_t BH = d->B * d->H;
  const int64_t walkers = BH * p.ns;
  p.nseg_f = plan_segments(walkers, p.n_chunks, "GLA_BWD_SEGMENTS");
  p.cps_f = (p.n_chunks + p.nseg_f - 1) / p.nseg_f;
  p.nseg_f = (p.n_chunks + p.cps_f - 1) / p.cps_f;
  p.nseg_r = p.nseg_f;
  p.cps_r = p.cps_f;
  const size_t frag = (size_t)BH * p.n_chunks * kStateElems * 2 * 2;   // bf16 hi + lo fragments
  size_t off = 0;
  p.off_s = off; off += align256(frag);
  p.off_dsdc = off; off += align256(frag);
  p.off_dscd = off; off += align256(frag);
  p.off_st = off; off += align256((size_t)BH * kStateElems * sizeof(float));
  p.off_r = off; off += align256((size_t)BH * p.n_chunks * sizeof(float));
  p.off_seg = off;
  if (p.nseg_f > 1) off += align256((size_t)BH * p.nseg_f * kStateElems * sizeof(float));
  p.off_dec = off;
  if (p.nseg_f > 1) off += align256((size_t)BH * p.nseg_f * sizeof(float));
  p.ws_total = off;
  return p;
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
  if (!out) return fail(GLA_ERR_INVALID_ARGUMENT, "out must not be NULL");
  *out = nullptr;
  if (n_slots < 1) return fail(GLA_ERR_INVALID_ARGUMENT, "n_slots must be >= 1 (got %lld)", (long long)n_slots);
  TRY(check_heads(H, dk, dv));
  const size_t slot = gla_state_slot_bytes(H, dk, dv);
  if ((size_t)n_slots > ((size_t)1 << 46) / slot)
    return fail(GLA_ERR_OUT_OF_MEMORY, "pool of %lld slots is too large", (long long)n_slots);
  const size_t bytes = (size_t)n_slots * slot;
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
  gla_state* s = new gla_state{(float*)p, n_slots, H, dk, dv, dev};
  *out = s;
  return ok();
}

gla_status gla_state_free(gla_state* pool) {
  if (!pool) return GLA_OK;
  int cur = 0;
  (void)hipGetDevice(&cur);
  (void)hipSetDevice(pool->device);
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipFree(pool->data);
  (void)hipSetDevice(cur);
  delete pool;
  return device_err(e, "gla_state_free");
}

float* gla_state_ptr(const gla_state* pool, int64_t slot) {
  if (!pool || slot < 0 || slot >= pool->n_slots) return nullptr;
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
    if (dims->in_dtype != GLA_BF16)
      return fail(GLA_ERR_UNSUPPORTED, "the backward is implemented for bf16 inputs only");
    *bytes = plan_bwd(dims).ws_total;
    return ok();
  }
  return fail(GLA_ERR_INVALID_ARGUMENT, "op must be GLA_OP_FWD or GLA_OP_BWD (got %d)", op);
}

gla_status gla_chunk_fwd(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g,
                         const float* S0, void* o, float* S_T, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(dims));
  TRY(check_ptr(q, "q", false));
  TRY(check_ptr(k, "k", false));
  TRY(check_ptr(v, "v", false));
  TRY(check_ptr(g, "g", false));
  TRY(check_ptr(S0, "S0", true));
  TRY(check_ptr(o, "o", false));
  TRY(check_ptr(S_T, "S_T", true));
  const FwdPlan p = plan_fwd(dims);
  if (ws_bytes < p.ws_total) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, p.ws_total);
  if (p.ws_total > 0) TRY(check_ptr(ws, "ws", false));
  WalkArgs a{};
  a.X = k;
  a.Y = v;
  a.Q = q;
  a.g = g;
  a.O = o;
  a.B = dims->B;
  a.T = dims->T;
  a.H = dims->H;
  char* w = (char*)ws;
  float* seg_states = p.nseg > 1 ? (float*)w : nullptr;
  float* seg_decay = p.nseg > 1 ? (float*)(w + p.ws_seg_states) : nullptr;
  hipError_t e = run_walk(a, p.variant, p.ns, p.nseg, p.cps, p.n_chunks, false, S0, S_T, seg_states, seg_decay,
                          dims->B * dims->H, (hipStream_t)stream);
  return device_err(e, "gla_chunk_fwd launch");
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
  StepArgs a{q, k, v, g, pool->data, slot_idx, o, B, H};
  return device_err(launch_step(a, in_dtype == GLA_BF16, out_dtype == GLA_BF16, (hipStream_t)stream),
                    "gla_recurrent_step launch");
}

gla_status gla_chunk_bwd(const gla_dims* dims, const void* q, const void* k, const void* v, const float* g,
                         const float* S0, const void* dO, const float* dS_T, void* dq, void* dk, void* dv, float* dg,
                         float* dS0, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims(dims));
  if (dims->in_dtype != GLA_BF16) return fail(GLA_ERR_UNSUPPORTED, "the backward is implemented for bf16 inputs only");
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
  const BwdPlan p = plan_bwd(dims);
  if (ws_bytes < p.ws_total) return fail(GLA_ERR_INVALID_ARGUMENT, "workspace too small: %zu < %zu", ws_bytes, p.ws_total);
  TRY(check_ptr(ws, "ws", false));
  if (p.n_chunks > 1024) return fail(GLA_ERR_UNSUPPORTED, "the backward supports at most 1024 chunks (T <= 131072)");
  char* w = (char*)ws;
  const int64_t BH = dims->B * dims->H;
  hipStream_t st = (hipStream_t)stream;
  float* seg_states = p.nseg_f > 1 ? (float*)(w + p.off_seg) : nullptr;
  float* seg_decay = p.nseg_f > 1 ? (float*)(w + p.off_dec) : nullptr;
  float* S_T = (float*)(w + p.off_st);

  // 1. forward states entering every chunk (and S_T when dS_T is given)
  WalkArgs f{};
  f.X = k;
  f.Y = v;
  f.g = g;
  f.B = dims->B;
  f.T = dims->T;
  f.H = dims->H;
  f.st_dc = w + p.off_s;
  hipError_t e = run_walk(f, WV_FWD_STATE_BF16, p.ns, p.nseg_f, p.cps_f, p.n_chunks, false, S0,
                          dS_T ? S_T : nullptr, seg_states, seg_decay, BH, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd forward-state walk");
  // 2. state gradients leaving every chunk (and dS0)
  WalkArgs r{};
  r.X = q;
  r.Y = dO;
  r.g = g;
  r.B = dims->B;
  r.T = dims->T;
  r.H = dims->H;
  r.st_dc = w + p.off_dsdc;
  r.st_cd = w + p.off_dscd;
  e = run_walk(r, WV_REV_BF16, p.ns, p.nseg_r, p.cps_r, p.n_chunks, true, dS_T, dS0, seg_states, seg_decay, BH, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd state-gradient walk");
  // 3. per-chunk gradients
  BwdArgs b{};
  b.q = q; b.k = k; b.v = v; b.dO = dO; b.g = g;
  b.s_dc = w + p.off_s;
  b.ds_dc = w + p.off_dsdc;
  b.ds_cd = w + p.off_dscd;
  b.dq = dq; b.dk = dk; b.dv = dv; b.dg = dg;
  b.chunk_r = (float*)(w + p.off_r);
  b.B = dims->B; b.T = dims->T; b.H = dims->H; b.n_chunks = p.n_chunks;
  e = launch_bwd_chunks(b, dims->out_dtype == GLA_BF16, st);
  if (e != hipSuccess) return device_err(e, "gla_chunk_bwd chunk kernel");
  // 4. d-log-decay: add later chunks and <dS_T, S_T>
  e = launch_dg_finish(dg, b.chunk_r, dS_T, S_T, dims->B, dims->T, dims->H, p.n_chunks, st);
  return device_err(e, "gla_chunk_bwd dg finish");
}

}  // extern "C"
