// Device-side checks of the caller contracts under GLA_DEBUG (gla_debug.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gla {

// Bits of the flag word.
enum : int { DBG_SLOT_RANGE = 1, DBG_SLOT_DUP = 2, DBG_DECAY = 4, DBG_OFFSETS = 8 };

hipError_t debug_zero(int* flag, hipStream_t st);
// n slot indices (device) against a pool of n_slots; a null idx is skipped.
hipError_t debug_slots(const int32_t* idx, int64_t n, int64_t n_slots, int* flag, hipStream_t st);
// A [B, T, H] float view with element strides sb, st_, sh.
hipError_t debug_decay(const float* g, int64_t B, int64_t T, int64_t H, int64_t sb, int64_t st_, int64_t sh,
                       int* flag, hipStream_t st);
// n + 1 int32 offsets (device) of a packed batch of `total` rows.
hipError_t debug_offsets(const int32_t* cu, int64_t n, int64_t total, int64_t max_len, int* flag, hipStream_t st);

}  // namespace gla
