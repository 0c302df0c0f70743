// GPU encoder for gfx950: builds the same compressed form as the host cbk_encode (sorted codebook
// of the distinct 16-bit patterns, b = ceil(log2 U), indices packed LSB first into little-endian
// uint32 words) on the device, for the load-time path.  The codebook method itself (codebook
// lossless compression overview, "How it works"; Codebook-Quantization digest, "Key points")
// fixes the result; the passes below are this library's way of computing it:
//
//  1. clear: zero the global presence bitmaps;
//  2. presence: each workgroup marks the patterns it sees in a 65,536-bit LDS bitmap (testing
//     before setting, so repeated values cost a read) and ORs its nonzero words into one of eight
//     global copies of the bitmap;
//  3. pack: every workgroup ORs the copies and ranks the bitmap into an LDS table (prefix sums of the words'
//     popcounts), which gives U, b, the ascending codebook and each pattern's index; a wave takes
//     2,048 consecutive fields with coalesced loads, looks their indices up and writes them to LDS
//     in field order; each lane then packs 32 consecutive indices into exactly b words (b fixed at
//     compile time per instantiation) and the wave's 64 b words leave through LDS as coalesced
//     16-byte stores.  U and b never leave the device, so the launches need no host round trip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "cbk_internal.h"

// The presence bitmaps of cbk_encode_gpu_noalloc: eight copies of a 65,536-bit map, 64 KB, the
// same layout as the caller-owned workspace of cbk_encode_gpu.  Each GPU the library runs on holds
// one copy of this array until the process ends; every no-allocation call on that GPU uses it.
// Host code never passes the array's name to a kernel (on the host it only stands in for the
// symbol): it uses the device address looked up once per device below.
static __device__ __align__(256) uint32_t scratch[8 * 2048];

namespace cbk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kPatterns = 65536;
constexpr uint32_t kMapWords = kPatterns / 32;  // 2048
constexpr int kPresThreads = 1024;
constexpr int kPresUnroll = 4;                  // 16-byte loads per thread per pass
// Copies of the global bitmap: workgroup g ORs into copy g % kCopies, which spreads the atomics on
// each hot word over kCopies addresses (and keeps them on one XCD when workgroups are dealt to the
// eight XCDs round-robin); the pack kernel ORs the copies back together.
constexpr int kCopies = 8;
constexpr int kPackWaves = 8;
constexpr int kRankWords = kMapWords / (64 * kPackWaves);  // bitmap words per thread in the ranking
constexpr uint32_t kPackFields = 64 * 32;       // fields per wave block

// Cache policies of the raw tensor's loads.  The presence pass reads it with the ordinary policy,
// so that the pack pass's second read (non-temporal, the last use) finds it in the caches: a
// 4096^2 tensor is 33.5 MB against the 256 MB Infinity Cache.  That took the encode of such a
// tensor from 25.8 to 24.0 us; reading it in the pack pass with the ordinary policy as well
// gained nothing more.
constexpr int kKeepCached = 0;
constexpr int kStreamOnce = 2;

// Workspace: kCopies global presence bitmaps.
constexpr size_t kWsMapBytes = kCopies * kMapWords * 4;

// A launch takes up to kMaxEncGroup tensors (a transformer block's matrices encoded together), each
// with its own kCopies bitmaps: workgroups [first_wg[i], first_wg[i + 1]) of a launch work on
// tensor i.  A single tensor is a group of one.
constexpr uint32_t kMaxEncGroup = 8;
struct EncJob {
    const uint16_t *w;
    uint64_t n;
    uint32_t *map;  // its kCopies global bitmaps
    uint16_t *codebook;
    uint32_t *meta;
    uint32_t *words;
};
struct EncGroup {
    uint32_t first_wg[kMaxEncGroup + 1];
    uint32_t count;
    EncJob j[kMaxEncGroup];
};

// The member of the group that workgroup blockIdx.x works on, with the workgroup's index among
// that member's workgroups and their number (all uniform).
struct EncMember {
    uint32_t k, wg, nwg;
};
__device__ __forceinline__ EncMember enc_member(const EncGroup &g) {
    uint32_t k = 0;
#pragma unroll
    for (uint32_t i = 1; i < kMaxEncGroup; ++i) k += (i < g.count && blockIdx.x >= g.first_wg[i]) ? 1u : 0u;
    return EncMember{k, blockIdx.x - g.first_wg[k], g.first_wg[k + 1] - g.first_wg[k]};
}

// Zero `words` words of bitmaps (the group's, contiguous in the workspace).
__global__ __launch_bounds__(256) void k_enc_clear(uint32_t *__restrict__ map, uint32_t words) {
    for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < words; i += gridDim.x * 256) map[i] = 0;
}

__device__ __forceinline__ void mark(uint32_t *bm, uint32_t v) {
    const uint32_t bit = 1u << (v & 31);
    if (!(bm[v >> 5] & bit)) atomicOr(&bm[v >> 5], bit);
}

__device__ __forceinline__ void mark8(uint32_t *bm, u32x4 v) {
    mark(bm, v.x & 0xFFFFu); mark(bm, v.x >> 16);
    mark(bm, v.y & 0xFFFFu); mark(bm, v.y >> 16);
    mark(bm, v.z & 0xFFFFu); mark(bm, v.z >> 16);
    mark(bm, v.w & 0xFFFFu); mark(bm, v.w >> 16);
}

// Passes of gridDim.x * kPresThreads * kPresUnroll 16-byte chunks (w is 16-byte aligned), two
// passes in flight: the next pass's loads are issued before this pass is marked.  The loads go
// through a wave-uniform buffer resource per pass, clipped to the tensor, so they are unconditional
// (bytes past the end read as zero with no memory access and are not marked) and the waits on them
// can count.  Then the n % 8 tail.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pass_rsrc(const u32x4 *w4, uint64_t chunks, uint64_t pass,
                                                            uint64_t span) {
    const uint64_t start = std::min<uint64_t>(pass * span, chunks);
    const uint64_t bytes = std::min<uint64_t>((chunks - start) * 16, span * 16);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(w4 + start), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

__global__ __launch_bounds__(kPresThreads) void k_enc_presence(const EncGroup grp) {
    __shared__ uint32_t bm[kMapWords];
    const EncMember me = enc_member(grp);
    const EncJob &J = grp.j[me.k];
    const uint16_t *__restrict__ w = J.w;
    const uint64_t n = J.n;
    uint32_t *__restrict__ map = J.map;
    const uint32_t t = threadIdx.x;
    for (uint32_t i = t; i < kMapWords; i += kPresThreads) bm[i] = 0;
    __syncthreads();
    const u32x4 *w4 = reinterpret_cast<const u32x4 *>(w);
    const uint64_t chunks = n / 8;
    const uint32_t stride = me.nwg * kPresThreads;         // chunks between a thread's loads
    const uint64_t span = static_cast<uint64_t>(stride) * kPresUnroll;  // chunks per pass
    const uint64_t passes = (chunks + span - 1) / span;
    const uint32_t mine = me.wg * kPresThreads + t;        // chunk of this thread's first load
    u32x4 a[kPresUnroll], b[kPresUnroll];
    auto load = [&](u32x4 (&v)[kPresUnroll], uint64_t pass) {
        const __amdgpu_buffer_rsrc_t rs = pass_rsrc(w4, chunks, pass, span);
#pragma unroll
        for (int j = 0; j < kPresUnroll; ++j)
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>((mine + j * stride) * 16u), 0,
                                                         kKeepCached);
    };
    auto mark_pass = [&](const u32x4 (&v)[kPresUnroll], uint64_t pass) {
#pragma unroll
        for (int j = 0; j < kPresUnroll; ++j)
            if (pass * span + mine + static_cast<uint64_t>(j) * stride < chunks) mark8(bm, v[j]);
    };
    load(a, 0);
    for (uint64_t p = 0; p < passes; p += 2) {
        load(b, p + 1);
        mark_pass(a, p);
        load(a, p + 2);
        mark_pass(b, p + 1);
    }
    if (me.wg == 0 && t < n % 8) mark(bm, w[chunks * 8 + t]);
    __syncthreads();
    uint32_t *copy = map + (me.wg % kCopies) * kMapWords;
    for (uint32_t i = t; i < kMapWords; i += kPresThreads)
        if (bm[i]) atomicOr(&copy[i], bm[i]);
}

// Lane packs its 32 indices (two per word of p, low half first) into B words at out[0..B).
template <int B>
__device__ __forceinline__ void pack32(const uint32_t (&p)[16], uint32_t *out) {
    uint32_t o[B];
#pragma unroll
    for (int k = 0; k < B; ++k) o[k] = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t idx = (i & 1) ? (p[i >> 1] >> 16) : (p[i >> 1] & 0xFFFFu);
        const int bit = i * B, word = bit >> 5, off = bit & 31;
        o[word] |= idx << off;
        if (off + B > 32) o[word + 1] |= idx >> (32 - off);
    }
#pragma unroll
    for (int k = 0; k < B; ++k) out[k] = o[k];
}

// The index of a present pattern v is its rank among the present patterns: the number of set
// bits before it in the bitmap, i.e. the exclusive prefix of its bitmap word plus the set bits
// below it within that word.  rt[i] = {bitmap word i, present patterns in words < i}.
__device__ __forceinline__ uint32_t index_of(const uint2 *rt, uint32_t v) {
    const uint2 e = rt[v >> 5];
    return e.y + __popc(e.x & ((1u << (v & 31)) - 1u));
}

// Workgroup wg of the nwg that pack this tensor.
template <int B>
__device__ void pack_blocks(const uint16_t *__restrict__ w, uint64_t n, const uint2 *rt,
                            uint32_t *__restrict__ words, uint16_t *sidx, uint32_t *sout,
                            const u32x4 (&pre)[4], uint32_t wg, uint32_t nwg) {
    const uint64_t words_total = ((n * B + 31) / 32 + 3) / 4 * 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t blocks = (n + kPackFields - 1) / kPackFields;
    const uint64_t first = static_cast<uint64_t>(wg) * kPackWaves + wave;
    u32x4 *words4 = reinterpret_cast<u32x4 *>(words);
    for (uint64_t blk = first; blk < blocks; blk += static_cast<uint64_t>(nwg) * kPackWaves) {
        const uint64_t f0 = blk * kPackFields;
        // coalesced: load q covers fields [q*512 + lane*8, +8) of the block
        if (f0 + kPackFields <= n) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(w + f0);
            u32x4 v[4];
            if (blk == first) {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = pre[q];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = __builtin_nontemporal_load(p + q * 64 + lane);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t h[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
                uint32_t r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = index_of(rt, h[e] & 0xFFFFu) | (index_of(rt, h[e] >> 16) << 16);
                u32x4 o;
                o.x = r[0]; o.y = r[1]; o.z = r[2]; o.w = r[3];
                *reinterpret_cast<u32x4 *>(sidx + q * 512 + lane * 8) = o;
            }
        } else {
#pragma unroll 1
            for (int q = 0; q < 4; ++q)
#pragma unroll 1
                for (int e = 0; e < 8; ++e) {
                    const uint64_t f = f0 + q * 512 + lane * 8 + e;
                    sidx[q * 512 + lane * 8 + e] = f < n ? static_cast<uint16_t>(index_of(rt, w[f])) : uint16_t(0);
                }
        }
        // sidx and sout are the same wave-private stage.  LDS runs one wave's accesses in issue
        // order, so each phase reads what the previous one wrote and the next one overwrites it
        // only afterwards; the compiler barriers keep each phase's accesses on its side.
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        uint32_t pr[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(sidx + lane * 32 + j * 8);
            pr[4 * j] = v.x; pr[4 * j + 1] = v.y; pr[4 * j + 2] = v.z; pr[4 * j + 3] = v.w;
        }
        pack32<B>(pr, sout + lane * B);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // the block's 64 B words (16 B quads) are contiguous in the stream; clip at the end
        const uint64_t q0 = blk * 16 * B;
        for (uint32_t j = static_cast<uint32_t>(lane); j < 16u * B; j += 64)
            if ((q0 + j) * 4 < words_total)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(sout + 4 * j), words4 + q0 + j);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
}

// Every workgroup ranks the bitmap itself (prefix sums of its 2,048 words' popcounts into an LDS
// table), so no separate rank launch is needed; workgroups share out the codebook writes and
// workgroup 0 writes U and b.  Each wave's first block is loaded before the ranking so that the
// stream is already in flight while the table is built.
__global__ __launch_bounds__(64 * kPackWaves) void k_enc_pack(const EncGroup grp) {
    const EncMember me = enc_member(grp);
    const EncJob &J = grp.j[me.k];
    const uint16_t *__restrict__ w = J.w;
    const uint64_t n = J.n;
    const uint32_t *__restrict__ map = J.map;
    uint16_t *__restrict__ codebook = J.codebook;
    uint32_t *__restrict__ meta = J.meta;
    uint32_t *__restrict__ words = J.words;
    // one 4 KB stage per wave: first the block's 2,048 indices, then (after every lane has read its
    // 32) the block's 64 b packed words
    __shared__ u32x4 stage[kPackWaves][256];
    __shared__ uint2 rt[kMapWords];
    __shared__ uint32_t wave_sum[kPackWaves];
    const uint32_t t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(t >> 6);

    // rank table: thread t owns bitmap words kRankWords t .. kRankWords (t + 1) - 1, the OR of
    // their copies (loaded first: the wait for them then leaves the four block loads below in
    // flight)
    static_assert(kPackWaves * 64 * kRankWords == kMapWords, "whole bitmap words per thread");
    uint32_t m[kRankWords];
#pragma unroll
    for (int i = 0; i < kRankWords; ++i) m[i] = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c)
#pragma unroll
        for (int i = 0; i < kRankWords; ++i) m[i] |= map[c * kMapWords + kRankWords * t + i];
    // unconditional buffer loads through a wave-uniform resource clipped to the tensor: bytes past
    // its end read as zero without a memory access (a partial block's values go unused)
    u32x4 pre[4];
    const uint64_t first = static_cast<uint64_t>(me.wg) * kPackWaves + wave_u;
    const uint64_t f_first = std::min<uint64_t>(first * kPackFields, n);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(w + f_first), static_cast<short>(0),
        static_cast<int>(std::min<uint64_t>((n - f_first) * 2, kPackFields * 2)), 0x00020000);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        pre[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, q * 1024 + lane * 16, 0, kStreamOnce);
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < kRankWords; ++i) cnt += __popc(m[i]);
    uint32_t incl = cnt;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    uint32_t base = 0, U = 0;
#pragma unroll
    for (int i = 0; i < kPackWaves; ++i) {
        base += i < wave ? wave_sum[i] : 0u;
        U += wave_sum[i];
    }
    const uint32_t excl = base + incl - cnt;
    uint32_t run = excl;
#pragma unroll
    for (int i = 0; i < kRankWords; ++i) {
        rt[kRankWords * t + i] = make_uint2(m[i], run);
        run += __popc(m[i]);
    }
    uint32_t b = 0;
    while ((1u << b) < U) ++b;
    b = __builtin_amdgcn_readfirstlane(b);
    if (me.wg == 0 && t == 0) {
        meta[0] = U;
        meta[1] = b;
    }
    __syncthreads();
    // the codebook: word i (handled by workgroup i % nwg) holds entries [its prefix, ...) in order
    for (uint32_t i = me.wg + t * me.nwg; i < kMapWords; i += me.nwg * (64 * kPackWaves)) {
        const uint2 e = rt[i];
        uint32_t bits = e.x, r = e.y;
        while (bits) {
            codebook[r++] = static_cast<uint16_t>(i * 32 + __ffs(bits) - 1);
            bits &= bits - 1;
        }
    }

    uint16_t *si = reinterpret_cast<uint16_t *>(stage[wave]);
    uint32_t *so = reinterpret_cast<uint32_t *>(stage[wave]);
    switch (b) {
    case 1: pack_blocks<1>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 2: pack_blocks<2>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 3: pack_blocks<3>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 4: pack_blocks<4>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 5: pack_blocks<5>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 6: pack_blocks<6>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 7: pack_blocks<7>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 8: pack_blocks<8>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 9: pack_blocks<9>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 10: pack_blocks<10>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 11: pack_blocks<11>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 12: pack_blocks<12>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 13: pack_blocks<13>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 14: pack_blocks<14>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 15: pack_blocks<15>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    case 16: pack_blocks<16>(w, n, rt, words, si, so, pre, me.wg, me.nwg); break;
    default: break;  // b == 0: no words
    }
}

static_assert(sizeof(scratch) == kWsMapBytes, "the static scratch holds exactly one workspace");

// Device address of `scratch` on each device, looked up with the device current on that device's
// first no-allocation call.
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint32_t *scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t encode_gpu_workspace_bytes() { return kWsMapBytes; }

cbk_status encode_gpu_scratch(void **ws) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return CBK_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return CBK_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CBK_E_HIP;
        scratch_ptr[dev] = static_cast<uint32_t *>(p);
    }
    *ws = scratch_ptr[dev];
    return CBK_OK;
}

// Workgroups for each of a group's tensors: `need` each (at least one), scaled down in proportion
// when they add up to more than `grid`.
static uint32_t split_enc(EncGroup &g, const uint64_t *need, uint64_t grid) {
    uint64_t total = 0;
    for (uint32_t i = 0; i < g.count; ++i) total += std::max<uint64_t>(1, need[i]);
    uint32_t at = 0;
    for (uint32_t i = 0; i < g.count; ++i) {
        g.first_wg[i] = at;
        const uint64_t want = std::max<uint64_t>(1, need[i]);
        const uint64_t share = total <= grid ? want : std::max<uint64_t>(1, (grid * want + total / 2) / total);
        at += static_cast<uint32_t>(share);
    }
    for (uint32_t i = g.count; i <= kMaxEncGroup; ++i) g.first_wg[i] = at;
    return at;
}

// One run of up to kMaxEncGroup jobs: clear their bitmaps, mark presence, rank and pack.
static cbk_status launch_encode_run(const cbk_encode_job *jobs, uint32_t count, uint32_t *maps, int cus,
                                    hipStream_t s) {
    EncGroup g{};
    g.count = count;
    for (uint32_t i = 0; i < count; ++i)
        g.j[i] = EncJob{jobs[i].w, jobs[i].n, maps + static_cast<size_t>(i) * kCopies * kMapWords, jobs[i].codebook,
                        jobs[i].meta, jobs[i].words};
    const uint32_t map_words = count * kCopies * kMapWords;
    hipLaunchKernelGGL(k_enc_clear, dim3(std::min<uint32_t>(map_words / 256, 1024)), dim3(256), 0, s, maps, map_words);
    // presence: two 1,024-thread workgroups per CU, each taking kPresUnroll 16-byte chunks per
    // thread per pass
    uint64_t need[kMaxEncGroup];
    const uint64_t per_block = static_cast<uint64_t>(kPresThreads) * kPresUnroll;
    for (uint32_t i = 0; i < count; ++i) need[i] = (jobs[i].n / 8 + per_block - 1) / per_block;
    const uint32_t pgrid = split_enc(g, need, static_cast<uint64_t>(cus) * 2);
    hipLaunchKernelGGL(k_enc_presence, dim3(pgrid), dim3(kPresThreads), 0, s, g);
    // pack: two 8-wave workgroups per CU (48 KB of LDS each: the stages and the rank table), which
    // measured 6 % faster than one of 16 waves; at least one workgroup per tensor, so that U, b
    // and the codebook are written even for n == 0
    for (uint32_t i = 0; i < count; ++i) {
        const uint64_t blocks = (jobs[i].n + kPackFields - 1) / kPackFields;
        need[i] = (blocks + kPackWaves - 1) / kPackWaves;
    }
    const uint32_t kgrid = split_enc(g, need, static_cast<uint64_t>(cus) * 2);
    hipLaunchKernelGGL(k_enc_pack, dim3(kgrid), dim3(64 * kPackWaves), 0, s, g);
    return hipGetLastError() == hipSuccess ? CBK_OK : CBK_E_HIP;
}

cbk_status launch_encode_gpu(const cbk_encode_job *jobs, uint32_t count, void *workspace, hipStream_t s) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return CBK_E_HIP;
    uint32_t *maps = static_cast<uint32_t *>(workspace);
    for (uint32_t i = 0; i < count; i += kMaxEncGroup) {
        const cbk_status st = launch_encode_run(jobs + i, std::min(kMaxEncGroup, count - i), maps, cus, s);
        if (st != CBK_OK) return st;
    }
    return CBK_OK;
}

}  // namespace cbk
