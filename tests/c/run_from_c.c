/* The library driven from plain C on the GPU, with device memory from the
 * HIP runtime and no torch: one prefill (gla_chunk_fwd) and one decode step
 * on a library-owned pool (gla_state_alloc, gla_recurrent_step).
 *
 *   run_from_c DIR B T H
 *
 * reads DIR/{q,k,v}.bf16 (raw bf16, [B,T,H,96|192]), DIR/g.f32 ([B,T,H]),
 * DIR/step_{q,k,v}.bf16 and DIR/step_g.f32 (one token for each of B
 * sequences) and DIR/pool.f32 (B states [H,96,192]); writes DIR/o.f32,
 * DIR/S_T.f32, DIR/step_o.f32 and DIR/pool_after.f32.  Exit status 0 on
 * success; every failure prints what failed. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "gla.h"

static const char* dir;

static void* load(const char* name, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  void* p = malloc(bytes ? bytes : 1);
  if (!f || !p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", bytes, path);
    exit(2);
  }
  fclose(f);
  return p;
}

static void save(const char* name, const void* p, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

static void* to_device(const char* name, size_t bytes) {
  void* h = load(name, bytes);
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device copy of %s failed\n", name);
    exit(3);
  }
  free(h);
  return d;
}

static void* device_buffer(size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess) {
    fprintf(stderr, "hipMalloc(%zu) failed\n", bytes);
    exit(3);
  }
  return d;
}

static void from_device(const char* name, const void* d, size_t bytes) {
  void* h = malloc(bytes);
  if (!h || hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "copy back of %s failed\n", name);
    exit(3);
  }
  save(name, h, bytes);
  free(h);
}

static void check(gla_status st, const char* what) {
  if (st != GLA_OK) {
    fprintf(stderr, "%s: %s (%s)\n", what, gla_status_str(st), gla_last_error());
    exit(4);
  }
}

int main(int argc, char** argv) {
  if (argc != 5) {
    fprintf(stderr, "usage: run_from_c DIR B T H\n");
    return 1;
  }
  dir = argv[1];
  const int64_t B = atoll(argv[2]), T = atoll(argv[3]);
  const int32_t H = atoi(argv[4]);
  const size_t tok = (size_t)B * T * H;

  /* prefill: bf16 in, fp32 out, S0 = 0 */
  gla_dims d;
  d.B = B; d.T = T; d.H = H; d.dk = 96; d.dv = 192; d.chunk = 128;
  d.in_dtype = GLA_BF16; d.out_dtype = GLA_F32; d.segments = 0;
  void* q = to_device("q.bf16", tok * 96 * 2);
  void* k = to_device("k.bf16", tok * 96 * 2);
  void* v = to_device("v.bf16", tok * 192 * 2);
  float* g = (float*)to_device("g.f32", tok * 4);
  float* o = (float*)device_buffer(tok * 192 * 4);
  float* S_T = (float*)device_buffer((size_t)B * H * 96 * 192 * 4);
  size_t ws_bytes = 0;
  check(gla_workspace_size(GLA_OP_FWD, &d, &ws_bytes), "gla_workspace_size");
  void* ws = ws_bytes ? device_buffer(ws_bytes) : NULL;
  check(gla_chunk_fwd(&d, q, k, v, g, NULL, o, S_T, ws, ws_bytes, NULL), "gla_chunk_fwd");
  if (hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "prefill failed on the device\n");
    return 3;
  }
  from_device("o.f32", o, tok * 192 * 4);
  from_device("S_T.f32", S_T, (size_t)B * H * 96 * 192 * 4);

  /* one decode step for B sequences on slots 0..B-1 of a library pool */
  gla_state* pool = NULL;
  check(gla_state_alloc(B, H, 96, 192, NULL, &pool), "gla_state_alloc");
  const size_t state = (size_t)B * H * 96 * 192 * 4;
  float* init = (float*)load("pool.f32", state);
  if (hipMemcpy(gla_state_ptr(pool, 0), init, state, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "pool upload failed\n");
    return 3;
  }
  free(init);
  const size_t seq = (size_t)B * H;
  void* sq = to_device("step_q.bf16", seq * 96 * 2);
  void* sk = to_device("step_k.bf16", seq * 96 * 2);
  void* sv = to_device("step_v.bf16", seq * 192 * 2);
  float* sg = (float*)to_device("step_g.f32", seq * 4);
  float* so = (float*)device_buffer(seq * 192 * 4);
  check(gla_recurrent_step(B, H, 96, 192, GLA_BF16, GLA_F32, sq, sk, sv, sg, pool, NULL, so, NULL),
        "gla_recurrent_step");
  if (hipDeviceSynchronize() != hipSuccess) {
    fprintf(stderr, "decode step failed on the device\n");
    return 3;
  }
  from_device("step_o.f32", so, seq * 192 * 4);
  from_device("pool_after.f32", gla_state_ptr(pool, 0), state);
  check(gla_state_free(pool), "gla_state_free");
  hipFree(q); hipFree(k); hipFree(v); hipFree(g); hipFree(o); hipFree(S_T);
  if (ws) hipFree(ws);
  hipFree(sq); hipFree(sk); hipFree(sv); hipFree(sg); hipFree(so);
  printf("ok\n");
  return 0;
}
