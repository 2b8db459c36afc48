// Launch interface between the host library and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr int CH = 128;   // chunk length (tokens)
constexpr int DK = 96;    // key/query width per head
constexpr int DV = 192;   // value width per head

enum WalkMode { WALK_FWD_OUT = 0, WALK_FWD_STATE = 1, WALK_REV = 2 };

enum WalkVariant {
  WV_FWD_OUT_BF16_BF16 = 0,
  WV_FWD_OUT_BF16_F32 = 1,
  WV_FWD_OUT_F32_F32 = 2,
  WV_FWD_OUT_F32_BF16 = 3,
  WV_FWD_STATE_BF16 = 4,
  WV_FWD_STATE_F32 = 5,
  WV_REV_BF16 = 6,
};

// Arguments of one walk launch.  Tensors are [B,T,H,D] row-major; states are
// [DK][DV] float32 blocks addressed as base + bh*bh_stride + seg*seg_stride.
struct WalkArgs {
  const void* X;        // forward: keys; reverse: queries      [B,T,H,DK]
  const void* Y;        // forward: values; reverse: dO         [B,T,H,DV]
  const void* Q;        // forward with output: queries         [B,T,H,DK]
  const float* g;       // log-decay                            [B,T,H]
  const float* zinit;   // initial state or null (zero)
  int64_t zinit_bh_stride, zinit_seg_stride;
  float* zfin;          // final state or null
  int64_t zfin_bh_stride, zfin_seg_stride;
  int zfin_only_seg;    // -1: every segment writes; else only that segment
  float* seg_decay;     // per-segment total log2-decay or null
  int64_t seg_decay_bh_stride;
  void* O;              // output [B,T,H,DV] (forward with output)
  void* st_dc;          // per-chunk entering state, bf16 fragments (m=d, k=c), or null
  void* st_cd;          // per-chunk entering state, bf16 fragments (m=c, k=d), or null
  int64_t B, T;
  int H, n_chunks, cps, ns, nseg_launch, seg_offset;
};

hipError_t launch_walk(const WalkArgs& a, int variant, int nwg, hipStream_t st);
int walk_slices(int variant);
hipError_t launch_seg_scan(float* buf, const float* decay, const float* Z0, int64_t BH, int nseg, int rev,
                           hipStream_t st);

// Decode step: see gla_step.hip.
struct StepArgs {
  const void* q; const void* k; const void* v; const float* g;
  float* pool; const int32_t* slot_idx; void* o;
  int64_t B; int H;
};
hipError_t launch_step(const StepArgs& a, int in_bf16, int out_bf16, hipStream_t st);

// Chunk-parallel backward and the d-log-decay finish: see gla_bwd.hip.
struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dO; const float* g;
  const void* s_dc;     // forward entering states, fragments (m=d, k=c)   [BH][N]
  const void* ds_dc;    // state gradient leaving each chunk (m=d, k=c)    [BH][N]
  const void* ds_cd;    // same, (m=c, k=d)                                 [BH][N]
  void* dq; void* dk; void* dv; float* dg;
  float* chunk_r;       // per-chunk sum of q.dq - k.dk                     [BH][N]
  int64_t B, T; int H, n_chunks;
};
hipError_t launch_bwd_chunks(const BwdArgs& a, int out_bf16, hipStream_t st);
hipError_t launch_dg_finish(float* dg, const float* chunk_r, const float* dS_T, const float* S_T,
                            int64_t B, int64_t T, int H, int n_chunks, hipStream_t st);

}  // namespace gla
