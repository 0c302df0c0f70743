// GPU decode of the exponent entropy-coded BF16 format for gfx950.
//
// The decoder follows the DFloat11 article (gadzety360.pl, "Jak to działa w praktyce?"): a compact
// lookup table held in on-chip memory, and a two-phase pass in which each thread first finds how
// many values it will decode and, after a synchronisation, decodes them into their places.  Here
// one workgroup of 256 threads takes one block of 256 spans (64 stream bits each):
//   1. the 4,096-entry table (exponent | length << 8 for every 12-bit window) is staged in LDS
//      once per workgroup;
//   2. each thread loads its span's three stream words (the span and the 32 bits after it, which
//      cover the longest code that starts in it) and its 4-bit gap, and walks the codes that start
//      in the span, counting them;
//   3. a workgroup prefix sum of the counts gives every thread the offset of its first value
//      within the block; the thread walks its span again and writes the exponents to an LDS
//      array at those offsets;
//   4. the block's values, bases[k] .. bases[k] + total, are joined with their sign-mantissa bytes
//      (coalesced 8-byte loads) and written as 16-byte non-temporal stores (element stores at the
//      two ragged ends of the block's range).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "cbk_internal.h"

namespace cbk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSpansPerBlock = CBK_EC_BLOCK_SPANS;  // = threads per workgroup
constexpr int kMaxPerSpan = CBK_EC_SPAN_BITS;       // codes are at least one bit long
constexpr int kLutEntries = CBK_EC_LUT_ENTRIES;
constexpr int kStreamOnce = 2;                      // non-temporal: data touched once

static_assert(kSpansPerBlock == 256, "one thread per span, 256 spans per block");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
}

// The 12 stream bits starting at bit pos (< 64) of the 96-bit window w0 | w1 << 32 | w2 << 64.
__device__ __forceinline__ uint32_t window12(uint64_t lo, uint64_t hi, uint32_t pos) {
    const uint64_t v = pos < 32 ? (lo >> pos) : (hi >> (pos - 32));
    return static_cast<uint32_t>(v) & (kLutEntries - 1);
}

__global__ __launch_bounds__(kSpansPerBlock) void k_ec_decode(const uint8_t *__restrict__ sm,
                                                              const uint32_t *__restrict__ stream,
                                                              const uint32_t *__restrict__ gaps,
                                                              const uint32_t *__restrict__ bases,
                                                              const uint16_t *__restrict__ lut,
                                                              uint16_t *__restrict__ out, uint64_t n,
                                                              uint64_t total_bits, uint32_t spans, uint32_t blocks) {
    __shared__ u32x4 table4[kLutEntries / 8];
    // exponents of one block, placed so that index i holds the value of weight (base & ~7) + i;
    // 16 spare bytes cover the 8-byte reads at the end of the range
    __shared__ uint64_t exps8[(kSpansPerBlock * kMaxPerSpan + 16) / 8];
    __shared__ uint32_t wave_sum[kSpansPerBlock / 64];
    const uint16_t *table = reinterpret_cast<const uint16_t *>(table4);
    uint8_t *exps = reinterpret_cast<uint8_t *>(exps8);
    const uint32_t t = threadIdx.x, lane = t & 63, wave = t >> 6;

    for (uint32_t i = t; i < kLutEntries / 8; i += kSpansPerBlock)
        table4[i] = reinterpret_cast<const u32x4 *>(lut)[i];
    __syncthreads();

    const uint64_t stream_bytes = 8 * static_cast<uint64_t>(spans);
    const uint64_t gap_bytes = 4 * ((static_cast<uint64_t>(spans) + 7) / 8);
    for (uint32_t k = blockIdx.x; k < blocks; k += gridDim.x) {
        const uint64_t j = static_cast<uint64_t>(k) * kSpansPerBlock + t;
        // this block's stream words and gaps through resources clipped to the arrays: reads past
        // their ends give zero without touching memory
        const uint64_t sw0 = static_cast<uint64_t>(k) * kSpansPerBlock * 8;  // byte offset
        const __amdgpu_buffer_rsrc_t rs = rsrc(reinterpret_cast<const uint8_t *>(stream) + sw0,
                                               std::min<uint64_t>(stream_bytes - sw0, kSpansPerBlock * 8 + 4));
        const u32x2 ab = __builtin_amdgcn_raw_buffer_load_b64(rs, static_cast<int>(t * 8), 0, kStreamOnce);
        const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(t * 8 + 8), 0, kStreamOnce);
        const uint64_t gw0 = static_cast<uint64_t>(k) * (kSpansPerBlock / 8) * 4;
        const __amdgpu_buffer_rsrc_t rg = rsrc(reinterpret_cast<const uint8_t *>(gaps) + gw0,
                                               std::min<uint64_t>(gap_bytes - gw0, kSpansPerBlock / 2));
        const uint32_t gword = __builtin_amdgcn_raw_buffer_load_b32(rg, static_cast<int>((t / 8) * 4), 0, 0);
        const uint64_t base = bases[k];  // first weight of the block (wave-uniform)
        const uint32_t gap = (gword >> (4 * (t % 8))) & 15u;
        uint32_t end = 0;
        if (j < spans) {
            const uint64_t rem = total_bits - j * CBK_EC_SPAN_BITS;
            end = rem < CBK_EC_SPAN_BITS ? static_cast<uint32_t>(rem) : CBK_EC_SPAN_BITS;
        }
        const uint64_t lo = static_cast<uint64_t>(ab.y) << 32 | ab.x;
        const uint64_t hi = static_cast<uint64_t>(c) << 32 | ab.y;

        // phase 1: how many codes start in this span
        uint32_t cnt = 0;
        for (uint32_t pos = gap; pos < end && cnt < kMaxPerSpan; ++cnt)
            pos += table[window12(lo, hi, pos)] >> 8;

        // prefix sum of the counts over the workgroup
        uint32_t incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o);
            if (lane >= static_cast<uint32_t>(o)) incl += y;
        }
        if (lane == 63) wave_sum[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < kSpansPerBlock / 64; ++i) {
            before += static_cast<uint32_t>(i) < wave ? wave_sum[i] : 0u;
            total += wave_sum[i];
        }
        const uint32_t shift = static_cast<uint32_t>(base & 7);
        uint32_t at = shift + before + incl - cnt;

        // phase 2: decode again, exponents to their places
        uint32_t pos = gap;
        for (uint32_t q = 0; q < cnt; ++q) {
            const uint32_t e = table[window12(lo, hi, pos)];
            exps[at++] = static_cast<uint8_t>(e);
            pos += e >> 8;
        }
        __syncthreads();

        // join with the sign-mantissa bytes: weights [base, base + total), clipped to n
        const uint64_t stop = std::min<uint64_t>(base + total, n);
        if (base < stop) {
            const uint64_t s0 = base / 8, s1 = (stop + 7) / 8;  // 8-weight segments
            // the sm allocation is readable up to n rounded up to 16 bytes, so whole dwords are in range
            const uint64_t sm_bytes = (n + 15) & ~uint64_t(15);
            const __amdgpu_buffer_rsrc_t rm = rsrc(sm + s0 * 8, std::min<uint64_t>(sm_bytes - s0 * 8, (s1 - s0) * 8));
            for (uint64_t s = s0 + t; s < s1; s += kSpansPerBlock) {
                const uint64_t g0 = s * 8;
                const u32x2 smv = __builtin_amdgcn_raw_buffer_load_b64(rm, static_cast<int>((s - s0) * 8), 0, kStreamOnce);
                const uint64_t ev = exps8[s - s0];
                uint32_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t b = ((e < 4 ? smv.x : smv.y) >> (8 * (e & 3))) & 0xFFu;
                    const uint32_t x = static_cast<uint32_t>(ev >> (8 * e)) & 0xFFu;
                    v[e] = ((b & 0x80u) << 8) | (x << 7) | (b & 0x7Fu);
                }
                if (g0 >= base && g0 + 8 <= stop) {
                    u32x4 o;
                    o.x = v[0] | (v[1] << 16);
                    o.y = v[2] | (v[3] << 16);
                    o.z = v[4] | (v[5] << 16);
                    o.w = v[6] | (v[7] << 16);
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + g0));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (g0 + e >= base && g0 + e < stop) out[g0 + e] = static_cast<uint16_t>(v[e]);
                }
            }
        }
        __syncthreads();  // the next block reuses wave_sum and exps
    }
}

}  // namespace

cbk_status launch_ec_decode(const cbk_ec_tensor *t, uint16_t *out, hipStream_t s) {
    const uint64_t spans = (t->total_bits + CBK_EC_SPAN_BITS - 1) / CBK_EC_SPAN_BITS;
    const uint64_t blocks = (spans + kSpansPerBlock - 1) / kSpansPerBlock;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return CBK_E_HIP;
    // blocks loop inside each workgroup so the table is staged once per workgroup
    const uint32_t grid = static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(blocks, 8ull * cus)));
    hipLaunchKernelGGL(k_ec_decode, dim3(grid), dim3(kSpansPerBlock), 0, s, t->sm, t->stream, t->gaps, t->bases,
                       t->lut, out, t->n, t->total_bits, static_cast<uint32_t>(spans),
                       static_cast<uint32_t>(blocks));
    return hipGetLastError() == hipSuccess ? CBK_OK : CBK_E_HIP;
}

}  // namespace cbk
