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
cbk_status launch_decode_group(const cbk_tensor *ts, uint32_t count, uint16_t *const *outs, hipStream_t s);
cbk_status launch_gemv(const cbk_tensor &t, const uint16_t *x, float *y, hipStream_t s);
cbk_status launch_gemv_group(const cbk_tensor *ts, uint32_t count, const uint16_t *x,
                             float *const *ys, hipStream_t s);
// Chained GEMV phases (validated by cbk_gemv_chain_init).
size_t gemv_chain_bytes(uint32_t phases);
cbk_status build_gemv_chain(const cbk_gemv_phase *phases, uint32_t count, void *buffer, cbk_gemv_chain *chain);
cbk_status launch_gemv_chain(const cbk_gemv_chain &chain, uint32_t timeout_us, hipStream_t s);
cbk_status gemv_chain_check(const cbk_gemv_chain &chain);
cbk_status launch_gemm(const cbk_tensor &t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                       float *Y, uint64_t ldy, hipStream_t s);
cbk_status launch_gemm_group(const cbk_tensor *ts, uint32_t count, const uint16_t *X, uint64_t ldx,
                             uint32_t batch, float *const *Ys, const uint64_t *ldys, hipStream_t s);

// GPU encoder (cbk_encode.hip).
size_t encode_gpu_workspace_bytes();
// count jobs, in runs of up to 8 (each run uses the first min(count, 8) workspaces of
// encode_gpu_workspace_bytes() bytes).
cbk_status launch_encode_gpu(const cbk_encode_job *jobs, uint32_t count, void *workspace, hipStream_t s);
// Device address of the library's static encoder scratch on the current device (a workspace of
// encode_gpu_workspace_bytes() bytes); looked up on the device's first call.
cbk_status encode_gpu_scratch(void **ws);

// Exponent entropy-coded format (cbk_ec.hip), count tensors in launches of up to 8.
// indexes: each tensor's span index (cbk_ec_build_index), or null for the two-walk decode.
cbk_status launch_ec_decode(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                            uint16_t *const *outs, hipStream_t s);
// rows[i] * cols = ts[i].n; every y is zero-filled first (rows[i] > 0), x is read when cols > 0.
cbk_status launch_ec_gemv(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                          const uint64_t *rows, uint64_t cols, const uint16_t *x, float *const *ys, hipStream_t s);
cbk_status launch_ec_index(const cbk_ec_tensor *t, uint8_t *index, hipStream_t s);

}  // namespace cbk
