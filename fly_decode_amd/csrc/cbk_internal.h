// Internal interface between the host API (cbk_api.cpp) and the HIP launchers (cbk_kernels.hip).
// Arguments reaching these launchers are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cbk.h"

namespace cbk {

// Largest number of codebook entries staged into LDS by the fast kernels, per index width.
inline constexpr uint32_t lds_entries(uint32_t b) { return 1u << b; }

// Fields per lane unit for width b: 128 / 2^v2(b) (b >= 1).  A unit is odd_part(b) 16-byte
// chunks, so units start on 16-byte boundaries and hold whole fields.
inline constexpr uint32_t unit_fields(uint32_t b) { return 128u >> __builtin_ctz(b); }
inline constexpr uint32_t unit_chunks(uint32_t b) { return b >> __builtin_ctz(b); }

cbk_status launch_decode(const cbk_tensor &t, uint16_t *out, hipStream_t s);
cbk_status launch_gemv(const cbk_tensor &t, const uint16_t *x, float *y, hipStream_t s);
cbk_status launch_gemv_group(const cbk_tensor *ts, uint32_t count, const uint16_t *x,
                             float *const *ys, hipStream_t s);
cbk_status launch_gemm(const cbk_tensor &t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                       float *Y, uint64_t ldy, hipStream_t s);

}  // namespace cbk
