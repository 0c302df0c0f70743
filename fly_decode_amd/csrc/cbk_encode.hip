// GPU encoder for gfx950: builds the same compressed form as the host cbk_encode (sorted codebook
// of the distinct 16-bit patterns, b = ceil(log2 U), indices packed LSB first into little-endian
// uint32 words) on the device, for the load-time path.  The codebook method itself (codebook
// lossless compression overview, "How it works"; Codebook-Quantization digest, "Key points")
// fixes the result; the three passes below are this library's way of computing it:
//
//  1. presence: each workgroup marks the patterns it sees in a 65,536-bit LDS bitmap (testing
//     before setting, so repeated values cost a read), then ORs its nonzero words into the
//     global bitmap;
//  2. rank: one workgroup turns the bitmap into the ascending codebook, the pattern -> index
//     table, U and b (prefix sums of the words' popcounts);
//  3. pack: a lane packs 32 consecutive fields into exactly b words in registers; a wave's 64 x b
//     words go through LDS and leave as coalesced stores.  b is read from device memory, so the
//     three launches need no host round trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "cbk_internal.h"

namespace cbk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kPatterns = 65536;
constexpr uint32_t kMapWords = kPatterns / 32;  // 2048
constexpr int kEncThreads = 512;
constexpr int kPackWaves = 8;
constexpr uint32_t kPackFields = 64 * 32;       // fields per wave block

// Workspace layout: the global bitmap, then the pattern -> index table.
constexpr size_t kWsMapBytes = kMapWords * 4;
constexpr size_t kWsIndexBytes = kPatterns * 2;

__global__ __launch_bounds__(256) void k_enc_clear(uint32_t *__restrict__ map) {
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < kMapWords; i += gridDim.x * 256) map[i] = 0;
}

__device__ __forceinline__ void mark(uint32_t *bm, uint32_t v) {
    const uint32_t bit = 1u << (v & 31);
    if (!(bm[v >> 5] & bit)) atomicOr(&bm[v >> 5], bit);
}

// Grid-stride over 16-byte chunks of w (16-byte aligned), then the n % 8 tail.
__global__ __launch_bounds__(kEncThreads) void k_enc_presence(const uint16_t *__restrict__ w, uint64_t n,
                                                              uint32_t *__restrict__ map) {
    __shared__ uint32_t bm[kMapWords];
    for (uint32_t i = threadIdx.x; i < kMapWords; i += kEncThreads) bm[i] = 0;
    __syncthreads();
    const u32x4 *w4 = reinterpret_cast<const u32x4 *>(w);
    const uint64_t chunks = n / 8;
    for (uint64_t c = static_cast<uint64_t>(blockIdx.x) * kEncThreads + threadIdx.x; c < chunks;
         c += static_cast<uint64_t>(gridDim.x) * kEncThreads) {
        const u32x4 v = __builtin_nontemporal_load(w4 + c);
        mark(bm, v.x & 0xFFFFu); mark(bm, v.x >> 16);
        mark(bm, v.y & 0xFFFFu); mark(bm, v.y >> 16);
        mark(bm, v.z & 0xFFFFu); mark(bm, v.z >> 16);
        mark(bm, v.w & 0xFFFFu); mark(bm, v.w >> 16);
    }
    if (blockIdx.x == 0 && threadIdx.x < n % 8) mark(bm, w[chunks * 8 + threadIdx.x]);
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < kMapWords; i += kEncThreads)
        if (bm[i]) atomicOr(&map[i], bm[i]);
}

// One workgroup of 1024 threads, two bitmap words each.
__global__ __launch_bounds__(1024) void k_enc_rank(const uint32_t *__restrict__ map, uint16_t *__restrict__ codebook,
                                                   uint16_t *__restrict__ index_of, uint32_t *__restrict__ meta) {
    __shared__ uint32_t part[1024];
    const uint32_t t = threadIdx.x;
    const uint32_t m0 = map[2 * t], m1 = map[2 * t + 1];
    const uint32_t c = __popc(m0) + __popc(m1);
    part[t] = c;
    __syncthreads();
    // inclusive scan (Hillis-Steele) of the per-thread counts
    for (uint32_t off = 1; off < 1024; off <<= 1) {
        const uint32_t v = t >= off ? part[t - off] : 0u;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t rank = part[t] - c;  // entries before this thread's 64 patterns
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t m = h ? m1 : m0;
        while (m) {
            const uint32_t bit = __ffs(m) - 1;
            const uint32_t v = (2 * t + h) * 32 + bit;
            codebook[rank] = static_cast<uint16_t>(v);
            index_of[v] = static_cast<uint16_t>(rank);
            ++rank;
            m &= m - 1;
        }
    }
    if (t == 1023) {
        const uint32_t U = part[1023];
        uint32_t b = 0;
        while ((1u << b) < U) ++b;
        meta[0] = U;
        meta[1] = b;
    }
}

// Each lane packs fields [32 q, 32 q + 32) of its wave block into b words; fields >= n pack as 0.
__global__ __launch_bounds__(64 * kPackWaves) void k_enc_pack(const uint16_t *__restrict__ w, uint64_t n,
                                                              const uint16_t *__restrict__ index_of,
                                                              const uint32_t *__restrict__ meta,
                                                              uint32_t *__restrict__ words) {
    __shared__ uint32_t stage[kPackWaves][64 * 16];
    const uint32_t b = meta[1];
    if (b == 0) return;
    const uint64_t words_total = ((n * b + 31) / 32 + 3) / 4 * 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t *st = stage[wave];
    const uint64_t blocks = (n + kPackFields - 1) / kPackFields;
    for (uint64_t blk = static_cast<uint64_t>(blockIdx.x) * kPackWaves + wave; blk < blocks;
         blk += static_cast<uint64_t>(gridDim.x) * kPackWaves) {
        const uint64_t f0 = blk * kPackFields + static_cast<uint64_t>(lane) * 32;
        uint32_t idx[32];
        if (f0 + 32 <= n) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(w + f0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 v = __builtin_nontemporal_load(p + q);
                const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    idx[8 * q + 2 * e] = index_of[h[e] & 0xFFFFu];
                    idx[8 * q + 2 * e + 1] = index_of[h[e] >> 16];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) idx[i] = f0 + i < n ? index_of[w[f0 + i]] : 0u;
        }
        // 32 fields of b bits = exactly b words
        uint64_t acc = 0;
        uint32_t nb = 0, k = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            acc |= static_cast<uint64_t>(idx[i]) << nb;
            nb += b;
            if (nb >= 32) {
                st[lane * b + k] = static_cast<uint32_t>(acc);
                ++k;
                acc >>= 32;
                nb -= 32;
            }
        }
        // LDS executes one wave's accesses in order; the compiler barriers keep the reads below the
        // writes and the next block's writes below these reads.
        asm volatile("" ::: "memory");
        // the wave's 64 b words are contiguous in the stream: coalesced stores, clipped at the end
        const uint64_t w0 = blk * 64 * b;
        for (uint32_t j = static_cast<uint32_t>(lane); j < 64 * b; j += 64)
            if (w0 + j < words_total) words[w0 + j] = st[j];
        asm volatile("" ::: "memory");
    }
}

}  // namespace

size_t encode_gpu_workspace_bytes() { return kWsMapBytes + kWsIndexBytes; }

cbk_status launch_encode_gpu(const uint16_t *w, uint64_t n, void *workspace, uint16_t *codebook,
                             uint32_t *words, uint32_t *meta, hipStream_t s) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return CBK_E_HIP;
    uint32_t *map = static_cast<uint32_t *>(workspace);
    uint16_t *index_of = reinterpret_cast<uint16_t *>(static_cast<unsigned char *>(workspace) + kWsMapBytes);
    hipLaunchKernelGGL(k_enc_clear, dim3(kMapWords / 256), dim3(256), 0, s, map);
    const uint64_t chunk_blocks = (n / 8 + kEncThreads - 1) / kEncThreads;
    const uint32_t pgrid = static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(static_cast<uint64_t>(cus) * 2, chunk_blocks)));
    hipLaunchKernelGGL(k_enc_presence, dim3(pgrid), dim3(kEncThreads), 0, s, w, n, map);
    hipLaunchKernelGGL(k_enc_rank, dim3(1), dim3(1024), 0, s, map, codebook, index_of, meta);
    const uint64_t blocks = (n + kPackFields - 1) / kPackFields;
    const uint32_t kgrid = static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(static_cast<uint64_t>(cus) * 4, (blocks + kPackWaves - 1) / kPackWaves)));
    hipLaunchKernelGGL(k_enc_pack, dim3(kgrid), dim3(64 * kPackWaves), 0, s, w, n, index_of, meta, words);
    return hipGetLastError() == hipSuccess ? CBK_OK : CBK_E_HIP;
}

}  // namespace cbk
