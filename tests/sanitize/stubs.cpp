// The GPU launchers, replaced for the host-only sanitizer build.  Argument validation must return
// before any of them is reached in the cases the harness runs, so each one aborts if called.
#include <stdio.h>
#include <stdlib.h>

#include "cbk_internal.h"

namespace cbk {
namespace {
[[noreturn]] void reached(const char *what) {
    fprintf(stderr, "launcher %s reached in the host-only build\n", what);
    abort();
}
}  // namespace
cbk_status launch_decode(const cbk_tensor &, uint16_t *, hipStream_t) { reached("decode"); }
cbk_status launch_decode_group(const cbk_tensor *, uint32_t, uint16_t *const *, hipStream_t) { reached("decode_group"); }
cbk_status launch_gemv(const cbk_tensor &, const uint16_t *, float *, hipStream_t) { reached("gemv"); }
cbk_status launch_gemv_group(const cbk_tensor *, uint32_t, const uint16_t *, float *const *, hipStream_t) {
    reached("gemv_group");
}
cbk_status launch_gemm(const cbk_tensor &, const uint16_t *, uint64_t, uint32_t, float *, uint64_t, hipStream_t) {
    reached("gemm");
}
cbk_status launch_gemm_group(const cbk_tensor *, uint32_t, const uint16_t *, uint64_t, uint32_t, float *const *,
                             const uint64_t *, hipStream_t) {
    reached("gemm_group");
}
size_t gemv_chain_bytes(uint32_t phases) { return 256 + size_t(phases) * 320; }
cbk_status build_gemv_chain(const cbk_gemv_phase *, uint32_t, void *, cbk_gemv_chain *) { reached("gemv_chain"); }
cbk_status launch_gemv_chain(const cbk_gemv_chain &, uint32_t, hipStream_t) { reached("gemv_chain_run"); }
cbk_status gemv_chain_check(const cbk_gemv_chain &) { reached("gemv_chain_check"); }
size_t encode_gpu_workspace_bytes() { return 65536; }
cbk_status launch_encode_gpu(const cbk_encode_job *, uint32_t, void *, hipStream_t) {
    reached("encode_gpu");
}
cbk_status encode_gpu_scratch(void **) { reached("encode_gpu_scratch"); }
cbk_status launch_ec_decode(const cbk_ec_tensor *, const uint8_t *const *, uint32_t, uint16_t *const *, hipStream_t) {
    reached("ec_decode");
}
cbk_status launch_ec_gemv(const cbk_ec_tensor *, const uint8_t *const *, uint32_t, const uint64_t *, uint64_t,
                          const uint16_t *, float *const *, hipStream_t) {
    reached("ec_gemv");
}
cbk_status launch_ec_index(const cbk_ec_tensor *, uint8_t *, hipStream_t) { reached("ec_index"); }
}  // namespace cbk
