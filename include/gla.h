/*
 * gla.h -- C ABI of the MI355X (gfx950) Simple GLA mixer library (libgla.so).
 *
 * The mixer: every layer keeps a fixed-size matrix state per sequence and
 * head, decays it once per token with a scalar gate and adds the token's
 * key/value outer product; the query reads the updated state by content
 * ("Cómo i14 llevó Laplace 3B a AWS Trainium2", sections "Por qué atención
 * lineal importa" and "Diseño esencial de Laplace 3B"; "AWS serve Laplace 3B
 * di i14 con uno stato fisso di 29,5 MB", section "GLA sostituisce i token
 * conservati con uno stato ricorrente"):
 *
 *     S_t = exp(g_t) * S_{t-1} + k_t^T v_t ,   o_t = q_t S_t
 *
 * per (batch b, head h), S is dk x dv, S_{-1} = S0.  There is no scale on q
 * (callers pre-scale).  Heads: H >= 1; dk = 96, dv = 192 and chunk = 128 are
 * the sizes of the pages ("Diseño esencial de Laplace 3B"; "Adaptaciones para
 * AWS Trainium2", item 1) and the only ones this library accepts.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers, dense row-major, in the layouts
 *    given per argument; pointers must be 16-byte aligned.  The caller owns
 *    every tensor and the workspace; the library never frees or keeps them.
 *  - in_dtype (q, k, v, dO) and out_dtype (o, dq, dk, dv) are gla_dtype
 *    values.  The log-decay g, states (S0, S_T, dS_T, dS0, pool) and dg are
 *    always float32.  Accumulation and the carried state are float32.
 *  - g <= 0 (or -inf for a state that forgets everything) is a caller
 *    contract; g is clamped to GLA_G_MIN inside the kernels.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  They never synchronise and never allocate (except
 *    gla_state_alloc).  Faults of running kernels surface at the caller's
 *    next synchronisation.
 *  - Arguments are validated before any HIP call.  A failing call returns a
 *    non-zero gla_status, launches nothing, and leaves a message for
 *    gla_last_error() in thread-local storage.  No exception crosses the ABI.
 *  - Outputs must not alias inputs.  Calls on different streams that share
 *    an output race.
 *  - Contracts only the device can check (slot indices in range and
 *    distinct, g <= 0 and not NaN, packed offsets in order, within the token
 *    count and within max_seqlen) are checked when the environment sets
 *    GLA_DEBUG to a non-empty value other than 0: the call then runs small
 *    check kernels on `stream`, synchronises it, and returns
 *    GLA_ERR_INVALID_ARGUMENT (naming the violation) before launching its own
 *    kernels.  Such a call synchronises and allocates one word per device on
 *    first use, so it cannot be captured in a graph.  The checks of calls
 *    from several host threads run one at a time (the flag word is shared);
 *    without GLA_DEBUG nothing is checked on the device.  The convolution's window tensor
 *    (gla_conv1d_silu) is the caller's, so only its negative and repeated
 *    slot indices are caught.
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, workspace too small */
  GLA_ERR_UNSUPPORTED = 2,      /* a size or dtype this library does not implement */
  GLA_ERR_OUT_OF_MEMORY = 3,    /* device allocation failed (gla_state_alloc only) */
  GLA_ERR_DEVICE = 4            /* the HIP runtime reported an error at launch */
} gla_status;

typedef enum { GLA_F32 = 0, GLA_BF16 = 1 } gla_dtype;

typedef enum { GLA_OP_FWD = 0, GLA_OP_BWD = 1, GLA_OP_FWD_VARLEN_Q16 = 2 } gla_op;

/* Lower clamp of the log-decay inside the kernels; exp(-60) ~ 8.8e-27. */
#define GLA_G_MIN (-60.0f)

/* Problem sizes of a prefill or backward call.  B, T, H >= 1; T need not be
 * a multiple of `chunk` (the tail chunk is masked).  dk = 96, dv = 192,
 * chunk = 128.  in_dtype/out_dtype are gla_dtype values.
 *
 * segments is the one plan choice a caller may make: 0 lets the library
 * pick its launch plan (the default; a zero-initialised struct gets it);
 * n > 0 splits every (batch, head) walk over the chunks into n segments of
 * whole chunks (at most one per chunk), whose entering states come from a
 * state-only pass and a scan over the segments (the bf16 backward with two
 * segments instead starts each second segment from the state its first one
 * left, one launch later).  Any plan computes the same
 * recurrence; results differ only by rounding.  The workspace size depends
 * on it, so pass the same dims to gla_workspace_size.  Negative values are
 * INVALID_ARGUMENT. */
typedef struct {
  int64_t B, T;
  int32_t H, dk, dv, chunk;
  int32_t in_dtype, out_dtype;
  int32_t segments;
} gla_dims;

/* Opaque pool of per-sequence recurrent states. */
typedef struct gla_state gla_state;

/* ---------------------------------------------------------------------------
 * State pool.  The pages keep one fixed-size recurrent state per sequence in
 * the serving engine's memory pool ("AWS serve Laplace 3B di i14 con uno stato
 * fisso di 29,5 MB", section "Lo stato di Laplace 3B resta fisso durante
 * l'inferenza"); its size does not depend on the context length, so the pool
 * takes no T.
 *
 * gla_state_alloc: library-owned float32 pool [n_slots, H, dk, dv] on the
 * current HIP device, 256-byte aligned, zero-filled in stream order on
 * `stream` (a slot is H*dk*dv*4 bytes: 1,179,648 B at H=16).  n_slots >= 1.
 * On success *out receives the handle; free it with gla_state_free.
 * Errors: INVALID_ARGUMENT (null out, n_slots < 1, H < 1), UNSUPPORTED
 * (dk != 96 or dv != 192), OUT_OF_MEMORY, DEVICE.
 */
gla_status gla_state_alloc(int64_t n_slots, int32_t H, int32_t dk, int32_t dv,
                           void* stream, gla_state** out);

/* Frees the pool (synchronises the device first so no kernel still uses it).
 * NULL is accepted and ignored. */
gla_status gla_state_free(gla_state* pool);

/* Device pointer to slot `slot` ([H, dk, dv] float32), or NULL when the pool
 * is NULL or the slot is out of range.  Prefill may read S0 from it and write
 * S_T into it; a plain device copy saves or restores a slot. */
float* gla_state_ptr(const gla_state* pool, int64_t slot);

/* Number of slots of the pool (0 for NULL). */
int64_t gla_state_slots(const gla_state* pool);

/* Bytes of one slot: H*dk*dv*4. */
size_t gla_state_slot_bytes(int32_t H, int32_t dk, int32_t dv);

/* ---------------------------------------------------------------------------
 * 16-bit state pools.  The HEAL summary ("Resumo Técnico: Desmistificando a
 * Instabilidade Numérica na Inferência de LLMs com HEAL", section "A.
 * Mitigando o Truncamento de Atenção via Quantização INT16") stores tensors
 * as 16-bit integers to keep 16 bits per element with less truncation than a
 * 16-bit float.  A GLA_STATE_Q16 pool stores each state that way: column d
 * (a value channel) of a [dk, dv] state holds int16 mantissas m[c][d] and one
 * int32 exponent e[d]; the value is m * 2^e.  e is chosen from the column's
 * largest magnitude M after every update: with M = f 2^x, f in [1/2, 1),
 * e = x - 15, one more when M / 2^e >= 32767.5, so M sits at [2^14, 2^15)
 * quanta and mantissas, rounded half to even, stay within +-32767.  The
 * rounding error is at most half a quantum, 2^-15 M per column.  A column
 * holding a non-finite value is stored as mantissa -32768 (reads as NaN).
 * A slot takes H*(dk*dv*2 + dv*4) bytes: 602,112 B at H=16 against
 * 1,179,648 B in float32, and the decode step moves half the bytes.
 */
typedef enum { GLA_STATE_F32 = 0, GLA_STATE_Q16 = 1 } gla_state_fmt;

/* Allocates a zero-filled 16-bit pool: mantissas [n_slots, H, dk, dv] int16,
 * then (256-byte aligned) exponents [n_slots, H, dv] int32, in one device
 * allocation owned by the library; free it with gla_state_free.  Errors as
 * gla_state_alloc. */
gla_status gla_state_alloc_q16(int64_t n_slots, int32_t H, int32_t dk, int32_t dv,
                               void* stream, gla_state** out);

/* GLA_STATE_F32 or GLA_STATE_Q16; -1 for NULL. */
int32_t gla_state_format(const gla_state* pool);

/* Device pointers to slot `slot` of a 16-bit pool: mantissas [H, dk, dv] and
 * exponents [H, dv] (gla_state_ptr returns NULL for such pools).
 * Errors: INVALID_ARGUMENT (NULL arguments, a float32 pool, slot out of range). */
gla_status gla_state_q16_ptrs(const gla_state* pool, int64_t slot, int16_t** mant,
                              int32_t** expo);

/* Moves n float32 states S [n, H, dk, dv] (device) into pool slots
 * slot_idx[i] (device int32 [n]; NULL: slots 0..n-1): a copy for a float32
 * pool, encoded as above for a 16-bit pool.  gla_state_read is the inverse
 * (exact for a 16-bit pool: every stored value is a float32).  Asynchronous
 * on `stream`; slot indices in range and distinct (caller contract).
 * This is how the float32 final states of a prefill enter a 16-bit pool (the
 * packed prefill, gla_chunk_fwd_varlen, does it by itself).
 * Errors: INVALID_ARGUMENT (NULL pool or S, n < 0, n > slots with slot_idx
 * NULL, misaligned slot_idx), UNSUPPORTED, DEVICE. */
gla_status gla_state_write(gla_state* pool, int64_t n, const int32_t* slot_idx,
                           const float* S, void* stream);
gla_status gla_state_read(const gla_state* pool, int64_t n, const int32_t* slot_idx,
                          float* S, void* stream);

/* ---------------------------------------------------------------------------
 * A layer's whole per-sequence state in one slot.  The pages put 29.5 MB of
 * fixed state per sequence ("Cómo i14 llevó Laplace 3B a AWS Trainium2",
 * "Introducción"; "AWS serve Laplace 3B di i14 con uno stato fisso di 29,5
 * MB", "Lo stato di Laplace 3B resta fisso durante l'inferenza") across 24
 * layers.  Each layer carries the mixer's state and the window of the causal
 * convolution ahead of it ("Diseño esencial de Laplace 3B": width 4 over
 * D = 3,072 channels); with a float32 mixer state (16 x 96 x 192) and a
 * float32 window of 4 x 3,072 a layer-slot is 1,228,800 B and 24 of them are
 * 29,491,200 B, the printed 29.5 MB.
 *
 * gla_state_alloc_conv: a pool as gla_state_alloc (format GLA_STATE_F32) or
 * gla_state_alloc_q16 (GLA_STATE_Q16) whose slots also hold a zero-filled
 * float32 window [4, conv_D] (one allocation; conv_D a multiple of 8 in
 * [8, 65536]).  gla_conv1d_silu_pool reads and writes it; the mixer calls
 * use the pool as any other.  Errors: as gla_state_alloc, plus UNSUPPORTED
 * for conv_D and INVALID_ARGUMENT for an unknown format.
 * gla_state_conv_channels: the pool's conv_D (0 without a window or NULL).
 * gla_state_conv_ptr: device pointer to slot `slot`'s window ([4, conv_D]
 *   float32, rows as in gla_conv1d_silu), NULL without a window or out of range.
 * gla_state_seq_bytes: bytes of one slot of such a pool, mixer state plus
 *   window (conv_D = 0: the mixer state alone); 0 for invalid sizes.
 */
gla_status gla_state_alloc_conv(int64_t n_slots, int32_t H, int32_t dk, int32_t dv,
                                int32_t format, int32_t conv_D, void* stream,
                                gla_state** out);
int32_t gla_state_conv_channels(const gla_state* pool);
float* gla_state_conv_ptr(const gla_state* pool, int64_t slot);
size_t gla_state_seq_bytes(int32_t H, int32_t dk, int32_t dv, int32_t format,
                           int32_t conv_D);

/* Workspace bytes that gla_chunk_fwd (op = GLA_OP_FWD) or gla_chunk_bwd
 * (op = GLA_OP_BWD) needs for `dims`, or gla_chunk_fwd_varlen into a 16-bit
 * pool (op = GLA_OP_FWD_VARLEN_Q16: the forward's bytes plus a float32 state
 * per sequence and head, B x H x 73,728 bytes, where the final states are
 * staged before encoding).  Same validation as those calls. */
gla_status gla_workspace_size(int32_t op, const gla_dims* dims, size_t* bytes);

/* ---------------------------------------------------------------------------
 * Chunked prefill.  Computes o and the final state of the recurrence for T
 * tokens, chunk by chunk: inside a chunk the decay-masked products of queries
 * and keys weight the values, and the state carried between chunks adds the
 * earlier context ("Adaptaciones para AWS Trainium2", item 1: 16 chunks of 128
 * tokens; "Trainium2 ha richiesto modifiche ai kernel e alla comunicazione").
 *
 *   q, k : [B, T, H, dk]  in_dtype        v : [B, T, H, dv] in_dtype
 *   g    : [B, T, H] float32 log-decay     S0: [B, H, dk, dv] float32 or NULL (zero)
 *   o    : [B, T, H, dv] out_dtype        S_T: [B, H, dk, dv] float32 or NULL (not written)
 *   ws   : device workspace of at least gla_workspace_size(GLA_OP_FWD) bytes
 *          (may be NULL when that size is 0).
 * S0 and S_T may point to the same memory (the initial state is read before
 * the final state is written for each sequence).
 */
gla_status gla_chunk_fwd(const gla_dims* dims, const void* q, const void* k,
                         const void* v, const float* g, const float* S0, void* o,
                         float* S_T, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * gla_chunk_fwd for callers that cannot allocate device memory or hand over
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments and results as gla_chunk_fwd
 * (bitwise: the same kernels and plan), without ws/ws_bytes.  The workspace
 * of a segmented plan lives in a static device array of
 * GLA_NOALLOC_SCRATCH_BYTES that the library owns; each device the library
 * runs on holds its own copy until the process ends.  The call allocates
 * nothing and calls no allocating routine; its first call on a device looks
 * the array's address up (no allocation, no launch).  Every call on a device
 * shares that device's array, so calls that overlap in time on one device
 * (different streams, or several host threads) race and give undefined
 * results: serialise them.  GLA_DEBUG's device checks are not run here (they
 * synchronise and allocate).  Every plan the library picks by itself
 * (dims->segments = 0) fits the array; a plan that needs more than
 * GLA_NOALLOC_SCRATCH_BYTES (a large forced segment count) returns
 * GLA_ERR_UNSUPPORTED naming both sizes, before any launch.
 * Errors: as gla_chunk_fwd, plus UNSUPPORTED for that case and DEVICE when
 * the array's address cannot be resolved. */
#define GLA_NOALLOC_SCRATCH_BYTES (32u << 20)
gla_status gla_chunk_fwd_noalloc(const gla_dims* dims, const void* q, const void* k,
                                 const void* v, const float* g, const float* S0,
                                 void* o, float* S_T, void* stream);

/* ---------------------------------------------------------------------------
 * Element strides of a token tensor: element i of the row of (batch b, token
 * t, head h) is at p[b*batch + t*token + h*head + i] (each row contiguous).
 * For g, which has one float per (b, t, h), the same with i = 0. */
typedef struct {
  int64_t batch, token, head;
} gla_strides;

/* gla_chunk_fwd over strided views, so that q, k, v (and g) can be read in
 * place from the output of the fused projection that produces them (a
 * 9,216-wide row per token holding every head's query, key, value and gate:
 * "Diseño esencial de Laplace 3B"), and o written into a wider buffer.
 *   sq, sk, sv, so : strides of q, k, v, o (NULL: the dense [B,T,H,d] layout)
 *   sg   : strides of g (NULL: dense [B,T,H])
 *   gate : NULL, or the gate of that projection, [B,T,H,dv] in in_dtype
 *          (sgate: its strides, NULL for the dense layout).  When given, the
 *          output is gated in the walk's epilogue before it is stored:
 *              o_t[h][c] = (q_t S_t)[h][c] * SiLU(gate_t[h][c]),
 *              SiLU(a) = a / (1 + exp(-a)).
 *          The pages split the projection into q, k, v and this gate (dv
 *          wide per head) without printing how it meets the mixer's output;
 *          the elementwise SiLU gate is this library's reading of it, with
 *          the activation the same section names.  Computed in float32
 *          from the float32 output; S_T is not gated.
 * Strides are positive; for q, k, v, gate and o they are multiples of 16
 * bytes, and token and head strides times 32 rows stay under 2^31 bytes
 * (INVALID_ARGUMENT otherwise).  q, k, v, gate and o are 16-byte aligned, g
 * 4-byte aligned.  Views must not overlap o or S_T (caller contract).
 * Everything else is as gla_chunk_fwd, whose workspace size applies. */
gla_status gla_chunk_fwd_strided(const gla_dims* dims, const void* q,
                                 const gla_strides* sq, const void* k,
                                 const gla_strides* sk, const void* v,
                                 const gla_strides* sv, const float* g,
                                 const gla_strides* sg, const void* gate,
                                 const gla_strides* sgate, const float* S0, void* o,
                                 const gla_strides* so, float* S_T, void* ws,
                                 size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill of a batch of sequences of different lengths, packed along one
 * token axis, with the states kept in a pool slot per sequence: the serving
 * layout in which a wrapper ties each sequence's recurrent state to the
 * engine's memory pool and prompts of different lengths share a batch ("AWS
 * serve Laplace 3B di i14 con uno stato fisso di 29,5 MB", sections "Lo stato
 * di Laplace 3B resta fisso durante l'inferenza" and "I risultati dichiarati
 * hanno limiti precisi").  Each sequence is an independent gla_chunk_fwd.
 *
 *   dims        : B = number of sequences, T = an upper bound of every
 *                 sequence's length (it sizes the launch plan and the
 *                 workspace), H, dk, dv, chunk and dtypes as for gla_chunk_fwd
 *   total_tokens: rows of the packed tensors, < 2^31 (0: every sequence is
 *                 empty, and q, k, v, g and o may be NULL)
 *   cu_seqlens  : device int32 [B + 1]; sequence b is rows
 *                 [cu_seqlens[b], cu_seqlens[b+1]).  Non-decreasing, within
 *                 [0, total_tokens], lengths <= T (caller contract: the
 *                 kernels clamp offsets into [0, total_tokens] and lengths to
 *                 [0, T], so no access leaves the tensors).  Empty sequences
 *                 are allowed: their slot keeps (or is set to) the initial
 *                 state.
 *   q, k : [total_tokens, H, dk] in_dtype   v : [total_tokens, H, dv] in_dtype
 *   g    : [total_tokens, H] float32        o : [total_tokens, H, dv] out_dtype
 *   pool, slot_idx : sequence b uses slot slot_idx[b] (device int32 [B]) or
 *                 slot b when slot_idx is NULL; indices in range and
 *                 distinct (caller contract, checked on the device only under GLA_DEBUG).
 *   init_from_pool : 1 = start from the slot's state (a prompt continued),
 *                 0 = start from zero (a new prompt).
 *   The final state of every sequence is written to its slot.  A 16-bit
 *   pool (gla_state_alloc_q16) is read and written in its own format: the
 *   slots' states are decoded into the workspace first (init_from_pool), the
 *   walks run on float32 states there, and the final states are encoded into
 *   the slots as gla_state_write does, so the slots hold exactly what
 *   gla_state_write of the float32 result would give.
 *   ws   : at least gla_workspace_size(GLA_OP_FWD, dims) bytes for a float32
 *          pool, gla_workspace_size(GLA_OP_FWD_VARLEN_Q16, dims) for a
 *          16-bit pool.
 * Errors: as gla_chunk_fwd, plus INVALID_ARGUMENT for a NULL or misaligned
 * cu_seqlens, a pool whose H/dk/dv differ, B > slots with slot_idx NULL.
 */
gla_status gla_chunk_fwd_varlen(const gla_dims* dims, int64_t total_tokens,
                                const int32_t* cu_seqlens, const void* q,
                                const void* k, const void* v, const float* g,
                                gla_state* pool, const int32_t* slot_idx,
                                int32_t init_from_pool, void* o, void* ws,
                                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Batched single-token decode step, in place on a state pool.  For each of B
 * sequences and each head: S <- exp(g) S + k^T v, then o = q S.  The state
 * has a fixed size, so the cost per token does not depend on the context length
 * ("I risultati dichiarati hanno limiti precisi": a longer prompt barely
 * changes the cost per output token; "Resultados de entrenamiento e
 * inferencia": 1,280 concurrent sequences).
 *
 *   q, k : [B, H, dk] in_dtype    v : [B, H, dv] in_dtype    g : [B, H] float32
 *   pool : states; sequence b uses slot slot_idx[b] (device int32 [B]) or
 *          slot b when slot_idx is NULL.  Indices must be in range and
 *          distinct (caller contract, checked on the device only under GLA_DEBUG).
 *   o    : [B, H, dv] out_dtype.
 * A float32 pool is updated in float32.  A 16-bit pool (gla_state_alloc_q16)
 * is decoded, updated in float32 the same way, o is read from the updated
 * float32 values, and the result is encoded again (its rounding affects the
 * next step, not this o).
 * Errors: INVALID_ARGUMENT (null pointers, B < 1, H or dk/dv differing from
 * the pool's, B > slots when slot_idx is NULL), UNSUPPORTED, DEVICE.
 */
gla_status gla_recurrent_step(int64_t B, int32_t H, int32_t dk, int32_t dv,
                              int32_t in_dtype, int32_t out_dtype, const void* q,
                              const void* k, const void* v, const float* g,
                              gla_state* pool, const int32_t* slot_idx, void* o,
                              void* stream);

/* ---------------------------------------------------------------------------
 * Chunked backward.  Gradients of L = <dO, o> + <dS_T, S_T> with respect to
 * q, k, v, the log-decay g and S0, computed chunk by chunk; the chunk steps
 * are sequential in the reverse direction ("Adaptaciones para AWS Trainium2",
 * item 3).  The forward states are recomputed; nothing from the forward call
 * is needed.
 *
 *   q, k, v, g, S0 : as in gla_chunk_fwd (S0 NULL = zero)
 *   dO   : [B, T, H, dv] in_dtype         dS_T : [B, H, dk, dv] float32 or NULL (zero)
 *   dq, dk : [B, T, H, dk] out_dtype      dv : [B, T, H, dv] out_dtype
 *   dg   : [B, T, H] float32              dS0 : [B, H, dk, dv] float32 or NULL (not written)
 *   ws   : at least gla_workspace_size(GLA_OP_BWD) bytes.
 * in_dtype is GLA_BF16 or GLA_F32 (q, k, v and dO alike); T <= 131,072
 * (1,024 chunks; UNSUPPORTED otherwise).
 */
gla_status gla_chunk_bwd(const gla_dims* dims, const void* q, const void* k,
                         const void* v, const float* g, const float* S0,
                         const void* dO, const float* dS_T, void* dq, void* dk,
                         void* dv, float* dg, float* dS0, void* ws,
                         size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Causal depth-wise convolution of width 4 followed by SiLU: the step that
 * gives every residual vector a summary of its last four tokens before the
 * fused projection that produces q, k, v and the gate ("Cómo i14 llevó
 * Laplace 3B a AWS Trainium2", section "Diseño esencial de Laplace 3B").  For
 * channel c of token t of a sequence:
 *     a_t[c] = bias[c] + sum_{j=0..3} w[c][j] * x_{t-3+j}[c]
 *     y_t[c] = a_t[c] / (1 + exp(-a_t[c]))
 * so w[c][3] weights the current token.  Tokens before a sequence's first
 * come from its window in conv_state (init_from_state = 1) or are zero.
 *
 *   B, T, D : B sequences of at most T tokens, D channels (a multiple of 8 in
 *             [8, 65536]; 3,072 in the pages' model)
 *   cu_seqlens : NULL: x and y are [B, T, D], every sequence T tokens long.
 *             Else device int32 [B + 1]: x and y are [total_tokens, D] and
 *             sequence b is rows [cu_seqlens[b], cu_seqlens[b+1]), with the
 *             clamping and caller contract of gla_chunk_fwd_varlen.
 *   x    : in_dtype            y : out_dtype (same layout as x)
 *   w    : [D, 4] float32      bias : [D] float32 or NULL (zero)
 *   conv_state : [n_slots, 4, D] float32 or NULL: each slot is the window of
 *             the filter's width, row m holding the input four-minus-m tokens
 *             back (row 3 the newest; row 0 is kept for the window's full
 *             width but not read).  When given, each sequence's slot
 *             (slot_idx[b], device int32 [B], or b when NULL; in range and
 *             distinct, a caller contract) receives the last four rows of its
 *             window (zeros without init_from_state) followed by its tokens;
 *             an empty sequence with init_from_state keeps its window.  One
 *             decode step is T = 1.
 * Errors: INVALID_ARGUMENT (NULL or misaligned pointers, B or T < 1,
 * init_from_state without conv_state), UNSUPPORTED (D), DEVICE.
 */
gla_status gla_conv1d_silu(int64_t B, int64_t T, int32_t D, int32_t in_dtype,
                           int32_t out_dtype, const int32_t* cu_seqlens,
                           int64_t total_tokens, const void* x, const float* w,
                           const float* bias, float* conv_state,
                           const int32_t* slot_idx, int32_t init_from_state,
                           void* y, void* stream);

/* gla_conv1d_silu with the windows kept in a pool's slots (a pool made by
 * gla_state_alloc_conv), so that one slot holds a sequence's whole state for
 * the layer: the convolution's window and the mixer's state, addressed by the
 * same slot indices as gla_chunk_fwd_varlen and gla_recurrent_step.  D is the
 * pool's conv_D.  Arguments otherwise as gla_conv1d_silu (init_from_pool
 * plays init_from_state).  Under GLA_DEBUG slot indices are checked against
 * the pool's slot count.
 * Errors: as gla_conv1d_silu, plus INVALID_ARGUMENT for a NULL pool, a pool
 * without a window, B > slots when slot_idx is NULL. */
gla_status gla_conv1d_silu_pool(int64_t B, int64_t T, int32_t in_dtype,
                                int32_t out_dtype, const int32_t* cu_seqlens,
                                int64_t total_tokens, const void* x, const float* w,
                                const float* bias, gla_state* pool,
                                const int32_t* slot_idx, int32_t init_from_pool,
                                void* y, void* stream);

/* ---------------------------------------------------------------------------
 * Errors. */
const char* gla_status_str(gla_status status);
/* Message of the last failing call on this thread ("" if none). */
const char* gla_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GLA_H */
