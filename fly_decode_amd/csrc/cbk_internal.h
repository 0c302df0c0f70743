// Internal interface between the host API (cbk_api.cpp, cbk_ec_host.cpp) and the HIP launchers
// (cbk_kernels.hip, cbk_encode.hip, cbk_ec.hip).
// Arguments reaching these launchers are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cbk.h"
#include "../../include/cbk_ec.h"

namespace cbk {

cbk_status launch_decode(const cbk_tensor &t, uint16_t *out, hipStream_t s);
cbk_status launch_gemv(const cbk_tensor &t, const uint16_t *x, float *y, hipStream_t s);
cbk_status launch_gemv_group(const cbk_tensor *ts, uint32_t count, const uint16_t *x,
                             float *const *ys, hipStream_t s);
cbk_status launch_gemm(const cbk_tensor &t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                       float *Y, uint64_t ldy, hipStream_t s);
cbk_status launch_gemm_group(const cbk_tensor *ts, uint32_t count, const uint16_t *X, uint64_t ldx,
                             uint32_t batch, float *const *Ys, const uint64_t *ldys, hipStream_t s);

// GPU encoder (cbk_encode.hip).
size_t encode_gpu_workspace_bytes();
cbk_status launch_encode_gpu(const uint16_t *w, uint64_t n, void *workspace, uint16_t *codebook,
                             uint32_t *words, uint32_t *meta, hipStream_t s);

// Exponent entropy-coded format (cbk_ec.hip).
cbk_status launch_ec_decode(const cbk_ec_tensor *t, uint16_t *out, hipStream_t s);
cbk_status launch_ec_gemv(const cbk_ec_tensor *t, uint64_t rows, uint64_t cols, const uint16_t *x, float *y,
                          hipStream_t s);

}  // namespace cbk
