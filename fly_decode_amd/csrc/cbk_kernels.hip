// HIP kernels for gfx950 (CDNA4): decode of codebook-compressed BF16 tensors, standalone and
// fused into GEMV (batch 1) and skinny GEMM (batch 2..16).
//
// What is computed follows the codebook lossless compression overview ("How it works": the
// stored index is replaced by its dictionary value, exactly) and the Codebook-Quantization
// digest ("Key points": bit-packed indices of the unique weights).  Fields are b bits wide,
// packed LSB first into little-endian uint32 words, row-major with no row padding.
//
// Decode and GEMV (templated on b so every shift and mask is a compile-time constant):
//  * A lane "unit" is 64 consecutive fields = 2b dwords; a wave step covers 64 units.  The wave
//    loads the step's bytes with coalesced 128-bit non-temporal buffer loads (lane l takes chunk
//    j*64 + l, through a resource that covers exactly the step), writes them to a wave-private
//    LDS stage and reads back its own unit: 64-bit LDS reads at an odd qword stride (odd b) or
//    128-bit reads at an odd chunk stride (even b; b % 4 == 0 pads one chunk per unit), so the
//    transposition has no bank conflicts.  The next step's loads are issued before the current
//    step is decoded.
//  * Fields are unpacked in registers straight into table byte offsets (shift/and, or alignbit +
//    and across a word boundary) and gathered from the codebook held in static LDS, padded to 2^b
//    entries with 0x7FC0 so a corrupt index cannot leave the table.  Gathers are issued one
//    8-field group ahead of use.
//  * GEMV: rows are dealt round-robin to the waves (the grid sweeps the stream front to back);
//    a row is ceil(K / 4096) wave steps, lane l of step j taking unit 64j + l of the row.  x sits
//    in LDS, 16 bytes of padding per unit so the lanes' 128-bit reads are conflict-free; BF16
//    pairs are multiplied with v_dot2c_f32_bf16 into fp32; lanes accumulate across the row's
//    steps and one wave reduction per row produces y.  The codebook and x staging loads are all
//    issued before any weight load (vector-memory data returns in issue order).
//  * One workgroup of 8 waves per CU shares one codebook table and one copy of x.
//
// Skinny GEMM: a wave owns a 16-row tile and walks its part of K in steps of 4 units (256 fields)
// per row; lane (i = l % 16, g = l / 16) decodes unit g of row i.  Batches 9..16 feed the decoded
// tile to v_mfma_f32_16x16x32_bf16 with X transposed through LDS; batches up to 8 use v_dot2c on
// the vector ALUs with X held in registers and broadcast across each 16-lane row by DPP.  When K
// is split across the waves of a workgroup, their partial tiles are added in LDS in a fixed order.
//
// Generic kernels (any b and shape, runtime field extraction straight from global memory) cover
// b == 0, rows whose length is not a multiple of 64, misaligned operands and shapes beyond the
// LDS budget (including the b = 16 GEMV).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <cstring>
#include <vector>
#include <atomic>
#include <utility>

#include "cbk_internal.h"

namespace cbk {
namespace {

constexpr uint16_t kCorrupt = 0x7FC0;
constexpr uint32_t kLdsLimit = 160 * 1024;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
}

// One step of a wave sum: v plus v moved by the DPP control CTRL within the rows in ROWS (lanes
// whose source is out of range add zero).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// The sum of v over the 64 lanes (all active), in lane 63: prefix sums within each 16-lane row
// (row_shr 1, 2, 4, 8), then lane 15 of rows 0 and 2 carried into rows 1 and 3 (row_bcast:15) and
// lane 31 into rows 2 and 3 (row_bcast:31).  VALU only, where lane shuffles would be six LDS round
// trips.
__device__ __forceinline__ float wave_sum_last(float v) {
    v = dpp_add<0x111, 0xF>(v);
    v = dpp_add<0x112, 0xF>(v);
    v = dpp_add<0x114, 0xF>(v);
    v = dpp_add<0x118, 0xF>(v);
    v = dpp_add<0x142, 0xA>(v);
    return dpp_add<0x143, 0xC>(v);
}

__device__ __forceinline__ float bf16_value(uint16_t h) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// Geometry of the 64-field lane unit for width B (decode and GEMV).
template <int B>
struct U64 {
    static constexpr int UD = 2 * B;                            // dwords per unit
    static constexpr int G = (UD % 4 == 0) ? 4 : 2;             // LDS read width (dwords)
    static constexpr int NG = UD / G;                           // reads per unit
    static constexpr bool PAD = (G == 4) && (NG % 2 == 0);      // pad to an odd chunk stride
    static constexpr int SG = PAD ? NG + 1 : NG;                // unit stride in reads
    static constexpr int LPL = (16 * UD + 1 + 63) / 64;         // 16-byte loads per lane per step
    static constexpr int STAGE_CHUNKS = 64 * LPL + (PAD ? 64 * LPL / NG + 1 : 0);
    static constexpr uint32_t NE = 1u << B;                     // codebook entries in LDS
    static constexpr uint32_t mask = (1u << B) - 1u;
};

// Table entry for field f (bits f*B .. f*B + B - 1, LSB first) of a unit held in registers; f is a
// constant once the caller's loop is unrolled.  The field is extracted straight into its byte
// offset 2 * field (shift by one less, mask b bits one place up), two VALU operations whether or
// not the field crosses a word boundary (v_alignbit joins the two words).
template <int B>
__device__ __forceinline__ uint32_t unit_gather(const uint16_t *tbl, const uint32_t *d, int f) {
    const int bit = f * B, w = bit >> 5, s = bit & 31;
    constexpr uint32_t m2 = U64<B>::mask << 1;
    uint32_t off;
    if (s == 0) off = (d[w] << 1) & m2;
    else if (s + B <= 32) off = (d[w] >> (s - 1)) & m2;
    else off = __builtin_amdgcn_alignbit(d[w + 1], d[w], s - 1) & m2;
    return *reinterpret_cast<const uint16_t *>(reinterpret_cast<const unsigned char *>(tbl) + off);
}

// Field i of a stream, runtime width (generic kernels).
__device__ __forceinline__ uint32_t stream_field(const uint32_t *__restrict__ words, uint32_t b,
                                                 uint64_t i) {
    if (b == 0) return 0;
    const uint64_t bit = i * b;
    const uint64_t w = bit >> 5;
    const uint32_t s = static_cast<uint32_t>(bit) & 31u;
    const uint32_t lo = words[w];
    const uint32_t hi = (s + b > 32) ? words[w + 1] : 0u;
    return __builtin_amdgcn_alignbit(hi, lo, s) & ((1u << b) - 1u);
}

// Codebook table in LDS: 2^b entries (at least 8) so any b-bit index stays inside it.
template <int B>
struct Table {
    static constexpr uint32_t NCH = (U64<B>::NE + 7) / 8;  // 16-byte chunks
    static constexpr uint32_t SIZE = NCH * 8;               // entries
};

// Codebook staging for the fast kernels: the table of Table<B>::NCH 16-byte chunks (entries >= U
// read 0x7FC0) is loaded branch-free by NT threads, CPT chunks each: whole 16-byte loads clamped
// into the codebook's whole chunks (from `dummy`, any readable 16-byte-aligned address, when it
// has none) plus the eight entries of the chunk that straddles U, one per lane in lanes 0..7 of
// every wave and broadcast with readlane.  Kernels issue these loads in every wave before a
// barrier and their first weight loads after it: vector-memory data returns in issue order, so
// the staging never waits behind the grid's first burst of weight loads.  Needs a 16-byte-aligned
// codebook.
template <int B, int NT>
struct CbStage {
    static constexpr int CPT = (Table<B>::NCH + NT - 1) / NT;
    u32x4 cw[CPT];
    uint32_t te;  // lane j < 8: entry 8 * full + j (clamped into the codebook)

    __device__ __forceinline__ void issue(const uint16_t *__restrict__ cb, uint32_t U, const u32x4 *dummy, int tid) {
        const uint32_t full = U / 8;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            cw[i] = full ? reinterpret_cast<const u32x4 *>(cb)[min(static_cast<uint32_t>(i * NT + tid), full - 1)] : *dummy;
        te = cb[min(8 * full + (tid & 7), U - 1)];
    }

    __device__ __forceinline__ void store(uint16_t *cbl, uint32_t U, int tid) const {
        const uint32_t full = U / 8;
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t v = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(te), j));
            e[j] = 8 * full + j < U ? v : kCorrupt;
        }
        const uint32_t fill = static_cast<uint32_t>(kCorrupt) * 0x10001u;
        const u32x4 tail = {e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        const u32x4 pad = {fill, fill, fill, fill};
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const uint32_t c = i * NT + tid;
            if (c < Table<B>::NCH) reinterpret_cast<u32x4 *>(cbl)[c] = c < full ? cw[i] : (c == full ? tail : pad);
        }
    }
};

// Workgroup barrier on LDS only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier that waits for nothing: orders the waves' instruction streams (used to put every wave's
// staging loads ahead of any weight load in the CU's memory pipeline).
__device__ __forceinline__ void issue_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Raw buffer resource over `bytes` bytes from `base`, which must be the same in every lane of the
// wave.  Loads at offsets at or past `bytes` return zeros without a memory access, so weight loads
// need neither clamped addresses nor branches, and the base and its arithmetic stay in scalar
// registers.  Word 3 sets the 32-bit data format, which this chip's untyped buffer loads need.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// Cache policy of the buffer operations on data that is touched exactly once (the packed index
// stream, the decoded output): the non-temporal bit (NT, bit 1 of the aux operand on this chip), so
// the stream does not displace the codebook, x and X from the caches.  It took the standalone
// decode of a 4096^2 tensor from 16.7 to 11.4 us and the GEMV launches 1-3 % faster.
constexpr int kStreamOnce = 2;

__device__ __forceinline__ u32x4 rsrc_load(__amdgpu_buffer_rsrc_t rs, uint32_t byte_offset) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(byte_offset), 0, kStreamOnce);
}

// Step loads: the chunks covering units [us, us + nl) start at chunk (us * UD) / 4; an odd-b step
// may start half-way into a chunk (the stage read then skips one qword).  Lane l loads chunks
// 64 j + l of the step; chunks past the step (or past the stream's nchunks) read as zero, and a
// wave with no step (valid false) touches no memory.  `us` must be wave-uniform.
template <int B>
__device__ __forceinline__ void load_step(u32x4 (&v)[U64<B>::LPL], const u32x4 *__restrict__ w4,
                                          uint32_t us, uint32_t nl, uint64_t nchunks, bool valid, int lane) {
    const uint64_t c0 = (static_cast<uint64_t>(us) * U64<B>::UD) >> 2;
    const uint64_t c1 = min((static_cast<uint64_t>(us + nl) * U64<B>::UD + 3) >> 2, nchunks);
    const auto rs = wave_rsrc(w4 + c0, valid && c1 > c0 ? static_cast<uint32_t>(c1 - c0) * 16u : 0u);
#pragma unroll
    for (int j = 0; j < U64<B>::LPL; ++j) v[j] = rsrc_load(rs, static_cast<uint32_t>(j * 64 + lane) * 16u);
}

// Write a step to the wave's stage and read back this lane's unit (UD dwords).
template <int B>
__device__ __forceinline__ void transpose_step(uint32_t (&d)[U64<B>::UD], const u32x4 (&v)[U64<B>::LPL],
                                               u32x4 *stage, uint32_t us, int lane) {
    using G = U64<B>;
    // The stage is written as 16-byte vectors and, for odd b, read as 8-byte vectors; the
    // compiler barriers keep type-based alias analysis from moving the reads above the writes
    // (or the next step's writes above these reads).  LDS executes one wave's accesses in order.
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < G::LPL; ++j) {
        const uint32_t q = j * 64 + lane;
        stage[G::PAD ? q + q / G::NG : q] = v[j];
    }
    asm volatile("" ::: "memory");
    if constexpr (G::G == 4) {
#pragma unroll
        for (int j = 0; j < G::NG; ++j) {
            const u32x4 t = stage[lane * G::SG + j];
            d[4 * j] = t.x; d[4 * j + 1] = t.y; d[4 * j + 2] = t.z; d[4 * j + 3] = t.w;
        }
    } else {
        // odd b: the step starts (us * UD) % 4 dwords into its first chunk (0 or 2)
        const u32x2 *st2 = reinterpret_cast<const u32x2 *>(stage) + ((us * G::UD) & 2u) / 2;
#pragma unroll
        for (int j = 0; j < G::NG; ++j) {
            const u32x2 t = st2[lane * G::SG + j];
            d[2 * j] = t.x; d[2 * j + 1] = t.y;
        }
    }
    asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------------------ fast decode
// Unit u decodes weights [64u, 64u + 64).  Wave steps (64 units) are dealt round-robin to the
// waves, so the grid reads the stream front to back.  A step's decoded 8 KB go back through the
// wave's stage (the weights have been read out of it by then) and leave as coalesced 16-byte
// non-temporal buffer stores.  Staging as in the GEMV: codebook loads before a barrier, the first
// weight step after it.
constexpr int kDecodeWaves = 4;  // two workgroups per CU (each stages its own table): 70.7 % of
                                 // peak on a 4096^2 decode against 67.6 % for one of 8 waves
constexpr uint32_t kOutUnit = 2 * 64 + 16;  // LDS bytes per decoded unit (16 bytes of padding)

template <int B>
constexpr uint32_t decode_stage_bytes() {
    return U64<B>::STAGE_CHUNKS * 16 > 64 * kOutUnit ? U64<B>::STAGE_CHUNKS * 16 : 64 * kOutUnit;
}

// A launch decodes up to kMaxGroup tensors of one width (a transformer block's matrices together):
// workgroups [first_wg[i], first_wg[i + 1]) take tensor i.  A single tensor is a group of one.
struct DecodeTensor {
    const u32x4 *w4;
    const uint16_t *cb;
    uint16_t *out;
    uint64_t n;
    uint32_t nchunks, U, T;
};
constexpr int kMaxDecodeGroup = 8;
struct DecodeGroup {
    uint32_t first_wg[kMaxDecodeGroup + 1];
    uint32_t count;
    DecodeTensor t[kMaxDecodeGroup];
};

template <int B>
__global__ __launch_bounds__(64 * kDecodeWaves) void k_decode_fast(const DecodeGroup grp) {
    using G = U64<B>;
    constexpr int NT = 64 * kDecodeWaves;
    __shared__ __attribute__((aligned(16))) uint16_t cbl[Table<B>::SIZE];
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint32_t k = 0;
#pragma unroll
    for (int i = 1; i < kMaxDecodeGroup; ++i) k += (i < static_cast<int>(grp.count) && blockIdx.x >= grp.first_wg[i]) ? 1u : 0u;
    const DecodeTensor &Tn = grp.t[k];
    const u32x4 *__restrict__ w4 = Tn.w4;
    const uint16_t *__restrict__ cb = Tn.cb;
    uint16_t *__restrict__ out = Tn.out;
    const uint64_t n = Tn.n;
    const uint32_t nchunks = Tn.nchunks, U = Tn.U, T = Tn.T;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char *stb = smem + wave * decode_stage_bytes<B>();
    u32x4 *stage = reinterpret_cast<u32x4 *>(stb);
    const uint32_t NW = (grp.first_wg[k + 1] - grp.first_wg[k]) * kDecodeWaves,
                   gw = (blockIdx.x - grp.first_wg[k]) * kDecodeWaves + wave;
    const uint32_t steps = (T + 63) / 64;

    CbStage<B, NT> cs;
    cs.issue(cb, U, w4, tid);
    issue_barrier();
    u32x4 nxt[G::LPL];
    load_step<B>(nxt, w4, gw * 64, 64, nchunks, gw < steps, lane);
    cs.store(cbl, U, tid);
    lds_barrier();

    for (uint32_t st = gw; st < steps; st += NW) {
        const uint32_t us = st * 64;
        uint32_t d[G::UD];
        transpose_step<B>(d, nxt, stage, us, lane);
        if (st + NW < steps) load_step<B>(nxt, w4, (st + NW) * 64, 64, nchunks, true, lane);
        // decode this lane's unit into the stage (unit stride kOutUnit bytes)
        uint32_t wv[2][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[0][i] = unit_gather<B>(cbl, d, i);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g + 1 < 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) wv[(g + 1) & 1][i] = unit_gather<B>(cbl, d, 8 * (g + 1) + i);
            }
            const uint32_t *w = wv[g & 1];
            *reinterpret_cast<u32x4 *>(stb + lane * kOutUnit + 16 * g) =
                (u32x4){w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16)};
        }
        asm volatile("" ::: "memory");
        // Coalesced stores: chunk q = j * 64 + lane of the step (unit q / 8, 8 weights at (q % 8) * 8)
        // through a resource over the step's whole output chunks, so chunks past the tensor's end
        // are dropped by the hardware; the one partial chunk a tensor can end with (n % 8 != 0) is
        // written element by element by the lane that holds it.
        const uint64_t base = static_cast<uint64_t>(us) * 64;  // first weight of the step
        const uint64_t left = n - base;                          // > 0 for every step
        const uint32_t full = static_cast<uint32_t>(min(left / 8, static_cast<uint64_t>(512)));
        const auto rs = wave_rsrc(out + base, full * 16u);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t q = j * 64 + lane;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stb + (q >> 3) * kOutUnit + (q & 7) * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, static_cast<int>(q * 16u), 0, kStreamOnce);
            if (left < 4096 && (left & 7) != 0 && q == full) {
                const uint32_t h[4] = {v.x, v.y, v.z, v.w};
                for (uint32_t k = 0; k < static_cast<uint32_t>(left & 7); ++k)
                    out[base + 8ull * q + k] = static_cast<uint16_t>(h[k >> 1] >> (16 * (k & 1)));
            }
        }
        asm volatile("" ::: "memory");
    }
}

// -------------------------------------------------------------------------------- fast GEMV
// Rows are dealt round-robin to the waves of the tensor's workgroups (row gw, gw + NW, ...; see
// gemv_rows_loop for the dynamic variant), so at any moment the grid reads one contiguous window
// of the stream, front to back.  A row of P units is S = ceil(P / 64) wave steps; lane l of step j
// decodes unit 64j + l of the row (the last step is partial when P % 64 != 0), accumulates in
// registers across the row's steps, and one wave reduction per row produces y.
//
// Up to kMaxGroup tensors that share x (same cols and width b) run in one launch: workgroups
// [first_block[t], first_block[t + 1]) belong to tensor t, so the launch's ramp-up and tail are
// paid once for the group (the same idea as decompressing a whole transformer block at once).
constexpr int kGemvWaves = 8;   // waves per workgroup, one workgroup per CU
constexpr int kMaxGroup = 8;
constexpr int kXPerThread = 8;  // x staging: 16-byte chunks per thread (K <= 8 * 8 * 512)
struct GemvTensor {
    const u32x4 *w4;
    const uint16_t *cb;
    float *y;
    uint32_t M, U;
};
struct GemvGroup {
    uint32_t first_block[kMaxGroup + 1];  // first_block[count] = grid size
    uint32_t count, P, S, dyn;
    GemvTensor t[kMaxGroup];
};

// One lane's unit of a GEMV row: gathers one 8-field group ahead of use, BF16 pairs multiplied
// with x by v_dot2c into four fp32 partial sums.
template <int B>
__device__ __forceinline__ void gemv_unit(const uint32_t (&d)[U64<B>::UD], const uint16_t *cbl, const u32x4 (&xq)[8],
                                          float (&a)[4]) {
    uint32_t wv[2][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[0][i] = unit_gather<B>(cbl, d, i);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        if (g + 1 < 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[(g + 1) & 1][i] = unit_gather<B>(cbl, d, 8 * (g + 1) + i);
        }
        const uint32_t *w = wv[g & 1];
        a[0] = dot2(w[0] | (w[1] << 16), xq[g].x, a[0]);
        a[1] = dot2(w[2] | (w[3] << 16), xq[g].y, a[1]);
        a[2] = dot2(w[4] | (w[5] << 16), xq[g].z, a[2]);
        a[3] = dot2(w[6] | (w[7] << 16), xq[g].w, a[3]);
    }
}

// The row loops of one wave: rows of one tensor for workgroup `blk` of the tensor's `nblk`
// workgroups, from the wave's first row gw (< M), whose first step's loads are in `nxt` on entry;
// the codebook table and x are staged in LDS.  Every argument is uniform across the workgroup.
// The workgroup's rows are blk * 8 + j + NW * i (j < 8), taken in the order k = 8 i + j; wave w
// starts with k = w.  With `dyn` false wave w then takes k + 8, k + 16, ...; with `dyn` true a wave
// that finishes a row claims the next k from the counter at next_row (LDS), so the waves of a
// workgroup end within about one row of each other (the host sets it when there are enough rows
// per wave for the tail to matter).  tail() is called exactly once, where the wave would issue
// its next weight loads but has no row left: the chained launch issues the next phase's first
// step there.  WT: y is stored at device scope (written through to memory, visible to every
// XCD once the store has completed), as the chained launch's barrier needs.
template <int B, bool WT, class Tail>
__device__ __forceinline__ void gemv_rows_loop(u32x4 (&nxt)[U64<B>::LPL], u32x4 *stage, const unsigned char *xl,
                                               const uint16_t *cbl, uint32_t *next_row,
                                               const u32x4 *__restrict__ w4, float *__restrict__ yt, uint32_t M,
                                               uint32_t P, uint32_t S, uint32_t blk, uint32_t nblk, bool dyn,
                                               uint32_t gw, int lane, Tail &&tail) {
    using G = U64<B>;
    constexpr uint32_t XU = 2 * 64 + 16;  // LDS bytes per unit of x (16 bytes of padding)
    const uint32_t NW = nblk * kGemvWaves;
    // The row after r: the static order, or the next k claimed from the workgroup's counter.
    auto next = [&](uint32_t r) -> uint32_t {
        if (!dyn) return r + NW;
        uint32_t kk = 0;
        if (lane == 0) kk = atomicAdd(next_row, 1u);
        kk = __builtin_amdgcn_readfirstlane(kk);
        return blk * kGemvWaves + (kk & (kGemvWaves - 1)) + NW * (kk / kGemvWaves);
    };
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    auto reduce_row = [&](uint32_t r) {
        const float acc = wave_sum_last((a[0] + a[1]) + (a[2] + a[3]));
        if (lane == 63) {
            if constexpr (WT)
                __hip_atomic_store(yt + r, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                yt[r] = acc;
        }
        a[0] = a[1] = a[2] = a[3] = 0.f;
    };

    if (S == 1) {
        // Rows of one step (K <= 4096): lane l multiplies unit l of x in every row, so its 64 x
        // values are read from LDS into registers once instead of in every step.
        const bool active = static_cast<uint32_t>(lane) < P;
        u32x4 xr[8];
#pragma unroll
        for (int g = 0; g < 8; ++g)
            xr[g] = active ? *reinterpret_cast<const u32x4 *>(xl + lane * XU + 16 * g) : (u32x4){0u, 0u, 0u, 0u};
        // rn, the row after r, is claimed one row ahead, so the claim's LDS round trip is not
        // between a row's read-back and the next row's loads
        uint32_t r = gw, rn = next(gw);
        while (true) {
            uint32_t d[G::UD];
            transpose_step<B>(d, nxt, stage, r * P, lane);
            if (rn < M) load_step<B>(nxt, w4, rn * P, P, ~uint64_t(0), true, lane);
            else tail();
            const uint32_t rnn = rn < M ? next(rn) : M;
            if (active) gemv_unit<B>(d, cbl, xr, a);
            reduce_row(r);
            if (rn >= M) break;
            r = rn;
            rn = rnn;
        }
        return;
    }

    if (S == 2) {
        // Rows of two steps (4096 < K <= 8192): lane l multiplies units l and 64 + l of x, both held
        // in registers; a row's two steps are written out in turn.
        const bool active1 = static_cast<uint32_t>(64 + lane) < P;
        u32x4 xr0[8], xr1[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            xr0[g] = *reinterpret_cast<const u32x4 *>(xl + lane * XU + 16 * g);
            xr1[g] = active1 ? *reinterpret_cast<const u32x4 *>(xl + (64 + lane) * XU + 16 * g) : (u32x4){0u, 0u, 0u, 0u};
        }
        uint32_t r = gw;
        while (true) {
            {
                uint32_t d[G::UD];
                transpose_step<B>(d, nxt, stage, r * P, lane);
                load_step<B>(nxt, w4, r * P + 64, P - 64, ~uint64_t(0), true, lane);
                gemv_unit<B>(d, cbl, xr0, a);
            }
            const uint32_t rn = next(r);
            {
                uint32_t d[G::UD];
                transpose_step<B>(d, nxt, stage, r * P + 64, lane);
                if (rn < M) load_step<B>(nxt, w4, rn * P, 64, ~uint64_t(0), true, lane);
                else tail();
                if (active1) gemv_unit<B>(d, cbl, xr1, a);
            }
            reduce_row(r);
            if (rn >= M) break;
            r = rn;
        }
        return;
    }

    if (!dyn) {
        // Rows of three or more steps, dealt statically (gw, gw + NW, ...): taken step-major in
        // groups of up to four rows, so each step's x unit is read from LDS once per group rather
        // than once per row.  On the 70B down projection (K = 28672, four rows per wave) this took
        // the launch from 64.1 to 61.6 us.
        constexpr uint32_t RG = 4;
        for (uint32_t r0 = gw; r0 < M;) {
            const uint32_t nr = min(RG, (M - r0 + NW - 1) / NW);  // rows in this group (uniform)
            float acc[RG][4];
#pragma unroll
            for (uint32_t k = 0; k < RG; ++k) acc[k][0] = acc[k][1] = acc[k][2] = acc[k][3] = 0.f;
            for (uint32_t j = 0; j < S; ++j) {
                const uint32_t cu = 64 * j + lane;  // this lane's unit within the row
                u32x4 xq[8];
                if (cu < P) {
                    const u32x4 *xb = reinterpret_cast<const u32x4 *>(xl + cu * XU);
#pragma unroll
                    for (int g = 0; g < 8; ++g) xq[g] = xb[g];
                }
#pragma unroll
                for (uint32_t k = 0; k < RG; ++k) {
                    if (k < nr) {
                        const uint32_t r = r0 + k * NW;
                        uint32_t d[G::UD];
                        transpose_step<B>(d, nxt, stage, r * P + 64 * j, lane);
                        // next step of this wave: the group's next row at this step, then its
                        // first row at the next step, then the next group's first row
                        uint32_t rn, jn;
                        if (k + 1 < nr) {
                            rn = r + NW;
                            jn = j;
                        } else if (j + 1 < S) {
                            rn = r0;
                            jn = j + 1;
                        } else {
                            rn = r0 + nr * NW;
                            jn = 0;
                        }
                        if (rn < M) load_step<B>(nxt, w4, rn * P + 64 * jn, min(64u, P - 64 * jn), ~uint64_t(0), true, lane);
                        else tail();
                        if (cu < P) gemv_unit<B>(d, cbl, xq, acc[k]);
                    }
                }
            }
#pragma unroll
            for (uint32_t k = 0; k < RG; ++k) {
                if (k < nr) {
                    a[0] = acc[k][0];
                    a[1] = acc[k][1];
                    a[2] = acc[k][2];
                    a[3] = acc[k][3];
                    reduce_row(r0 + k * NW);
                }
            }
            r0 += nr * NW;
        }
        return;
    }

    // rows claimed dynamically: one row at a time
    uint32_t r = gw, j = 0;
    while (true) {
        const uint32_t us = r * P + 64 * j;
        uint32_t d[G::UD];
        transpose_step<B>(d, nxt, stage, us, lane);
        // next step of this wave: the rest of the row, then the next row
        const bool row_end = j + 1 == S;
        const uint32_t rn = row_end ? next(r) : r;
        const uint32_t jn = row_end ? 0 : j + 1;
        if (rn < M) load_step<B>(nxt, w4, rn * P + 64 * jn, min(64u, P - 64 * jn), ~uint64_t(0), true, lane);
        else tail();

        const uint32_t cu = 64 * j + lane;  // this lane's unit within the row
        if (cu < P) {
            const u32x4 *xb = reinterpret_cast<const u32x4 *>(xl + cu * XU);
            u32x4 xq[8];
#pragma unroll
            for (int g = 0; g < 8; ++g) xq[g] = xb[g];
            gemv_unit<B>(d, cbl, xq, a);
        }
        if (row_end) reduce_row(r);
        if (rn >= M) break;
        r = rn;
        j = jn;
    }
}

// Rows of one tensor for workgroup `blk` of the tensor's `nblk` workgroups (one launch): stages the
// codebook and x, loads the wave's first step and runs the row loops.
template <int B>
__device__ __forceinline__ void gemv_rows(const u32x4 *__restrict__ w4, const uint16_t *__restrict__ cb,
                                          float *__restrict__ yt, const uint16_t *__restrict__ x, uint32_t M,
                                          uint32_t U, uint32_t P, uint32_t S, uint32_t blk, uint32_t nblk,
                                          bool dyn) {
    using G = U64<B>;
    constexpr uint32_t XU = 2 * 64 + 16;  // LDS bytes per unit of x (16 bytes of padding)
    constexpr int NT = 64 * kGemvWaves;
    __shared__ __attribute__((aligned(16))) uint16_t cbl[Table<B>::SIZE];
    __shared__ uint32_t next_row;  // next k to claim (dyn)
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *xl = smem;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    u32x4 *stage = reinterpret_cast<u32x4 *>(xl + P * XU) + wave * G::STAGE_CHUNKS;
    const uint32_t gw = blk * kGemvWaves + wave;

    // Staging loads (codebook and this thread's x chunks), issued in every wave before the first
    // weight load.
    const u32x4 *x4 = reinterpret_cast<const u32x4 *>(x);
    const uint32_t xch = P * 8;
    CbStage<B, NT> cs;
    cs.issue(cb, U, x4, tid);
    u32x4 xv[kXPerThread];
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i)
        if (static_cast<uint32_t>(i * NT + tid) < xch) xv[i] = x4[i * NT + tid];
    issue_barrier();

    // First weight step (no memory access for a wave without rows).
    u32x4 nxt[G::LPL];
    load_step<B>(nxt, w4, min(gw, M - 1) * P, min(64u, P), ~uint64_t(0), gw < M, lane);

    cs.store(cbl, U, tid);
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i) {
        const uint32_t q = i * NT + tid;
        if (q < xch) *reinterpret_cast<u32x4 *>(xl + (q >> 3) * XU + (q & 7) * 16) = xv[i];
    }
    if (tid == 0) next_row = kGemvWaves;
    lds_barrier();
    if (gw >= M) return;
    gemv_rows_loop<B, false>(nxt, stage, xl, cbl, &next_row, w4, yt, M, P, S, blk, nblk, dyn, gw, lane, [] {});
}

// One tensor per launch.  The arguments are plain scalars so that the code object can have them
// preloaded into scalar registers: the first address computations then wait for no load.
template <int B>
__global__ __launch_bounds__(64 * kGemvWaves) void k_gemv_rows(const u32x4 *__restrict__ w4,
                                                               const uint16_t *__restrict__ cb,
                                                               float *__restrict__ y,
                                                               const uint16_t *__restrict__ x, uint32_t M,
                                                               uint32_t U, uint32_t P, uint32_t S, uint32_t dyn) {
    gemv_rows<B>(w4, cb, y, x, M, U, P, S, blockIdx.x, gridDim.x, dyn != 0);
}

// Up to kMaxGroup tensors that share x: this workgroup's tensor is found by counting the group
// boundaries at or below blockIdx.x (uniform).
template <int B>
__global__ __launch_bounds__(64 * kGemvWaves) void k_gemv_rows_group(const GemvGroup grp,
                                                                     const uint16_t *__restrict__ x) {
    uint32_t k = 0;
#pragma unroll
    for (int j = 1; j < kMaxGroup; ++j) k += (j < static_cast<int>(grp.count) && blockIdx.x >= grp.first_block[j]) ? 1u : 0u;
    const GemvTensor &T = grp.t[k];
    const uint32_t b0 = grp.first_block[k], b1 = grp.first_block[k + 1];
    gemv_rows<B>(T.w4, T.cb, T.y, x, T.M, T.U, grp.P, grp.S, blockIdx.x - b0, b1 - b0, grp.dyn != 0);
}

// ------------------------------------------------------------ chained GEMV phases, one launch
// A chain of dependent GEMV phases, such as a decode step's [q, k, v] -> [o] -> [gate, up] ->
// [down] over its layers: phase p + 1 reads its x only after every workgroup has finished phase p,
// as if x were computed from phase p's outputs.  One persistent workgroup per CU runs all phases,
// and the grid meets at a barrier between two of them.  A launch per phase pays at every boundary
// for the dispatch, the codebook and x staging, the first loads' latency on an idle machine and
// the tail in which the last waves run alone.  Here a wave that has issued its last weight load of
// phase p issues its first step of phase p + 1 (the weights do not depend on x), and the
// workgroup's next codebook loads go out before the barrier, so the memory system keeps working
// while the grid drains and meets.  This carries the DFloat11 page's block-level decompression
// ("How it works in practice": a transformer block's matrices decompressed together to hide
// latency) across the dependent phases of a block.
//
// The barrier is an arrival counter in device memory, used by one thread per workgroup.  The
// launch is cooperative, so the runtime guarantees that the whole grid is resident before any
// workgroup waits; every wait is also bounded by a wall-clock limit, and a workgroup that reaches
// it (or sees that another one has) records the failure and leaves, so the kernel always ends.  Rows are computed exactly as by k_gemv_rows (same loops), so every y equals the
// single-launch result bit for bit.
struct ChainPhase {
    GemvGroup g;  // tensors, workgroup split over the chain's grid, P, S, dyn
    const uint16_t *x;
};
struct ChainSync {
    uint32_t arrived;  // arrivals so far in this run: barrier i is passed at (i + 1) * grid
    uint32_t failed;   // nonzero: a wait gave up, the outputs are incomplete
    uint32_t pad[62];  // the block fills 256 bytes
};
static_assert(sizeof(ChainSync) == 256, "sync block size");

// Member of a group that workgroup blockIdx.x works on (uniform).
__device__ __forceinline__ uint32_t group_member(const GemvGroup &g) {
    uint32_t k = 0;
#pragma unroll
    for (int j = 1; j < kMaxGroup; ++j) k += (j < static_cast<int>(g.count) && blockIdx.x >= g.first_block[j]) ? 1u : 0u;
    return k;
}

// Grid barrier number i of a run, called by one thread per workgroup after the workgroup's
// outputs of the phase have completed: true once all workgroups have arrived, false if the wait
// gave up (after `limit` wall-clock ticks, or because another workgroup did).  The counter only
// grows during a run (cleared before each run), so no reset races the next barrier's arrivals.
// Every access is a relaxed device-scope atomic, which this chip performs coherently for all its
// XCDs without touching the caches' other lines.  (An acquire load would invalidate the whole L2
// of the poller's XCD; polled in a loop by every workgroup, that made each barrier cost about
// 30 us.)  The ordering the phases need comes from the data accesses themselves: outputs are
// written through at device scope and waited for before arriving, and the next phase's x is read
// with device-coherent loads after the wait.
__device__ bool chain_barrier(ChainSync *s, uint32_t i, uint32_t nblocks, uint64_t limit) {
    const uint32_t target = (i + 1) * nblocks;
    if (__hip_atomic_fetch_add(&s->arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == target) return true;
    // a poll (a round trip past the L2) takes well over 8 ticks of the 100 MHz wall clock, so the
    // poll count bounds the wait too, should the clock not advance
    const uint64_t t0 = wall_clock64(), max_polls = (limit >> 3) + 1024;
    uint64_t polls = 0;
    while (__hip_atomic_load(&s->arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (__hip_atomic_load(&s->failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
        if (wall_clock64() - t0 > limit || ++polls > max_polls) {
            __hip_atomic_store(&s->failed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

// Cache policy of x loads after a barrier: device-coherent (SC0 | SC1), so they read what another
// XCD wrote before the barrier rather than a line left in this XCD's caches.
constexpr int kCoherent = 1 | 16;

template <int NT, int AUX>
__device__ __forceinline__ void x_stage_load(u32x4 (&xv)[kXPerThread], const uint16_t *x, uint32_t P, int tid) {
    const auto rs = wave_rsrc(x, P * 128u);  // chunks past the P units read as zero
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i)
        if (static_cast<uint32_t>(i * NT + tid) < P * 8)
            xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>((i * NT + tid) * 16u), 0, AUX);
}
template <int NT>
__device__ __forceinline__ void x_stage_store(unsigned char *xl, const u32x4 (&xv)[kXPerThread], uint32_t P, int tid) {
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i) {
        const uint32_t c = i * NT + tid;
        if (c < P * 8) *reinterpret_cast<u32x4 *>(xl + (c >> 3) * (2 * 64 + 16) + (c & 7) * 16) = xv[i];
    }
}

template <int B>
__global__ __launch_bounds__(64 * kGemvWaves) void k_gemv_chain(const ChainPhase *__restrict__ ph, uint32_t nph,
                                                                uint32_t xbytes, ChainSync *sync, uint64_t limit) {
    using G = U64<B>;
    constexpr int NT = 64 * kGemvWaves;
    __shared__ __attribute__((aligned(16))) uint16_t cbl[Table<B>::SIZE];
    __shared__ uint32_t next_row;  // next k to claim (dyn)
    __shared__ uint32_t go_on;     // the grid barrier's outcome
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *xl = smem;      // x of the current phase (xbytes: the largest phase's)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    u32x4 *stage = reinterpret_cast<u32x4 *>(smem + xbytes) + wave * G::STAGE_CHUNKS;

    // This workgroup's part of a phase (uniform): its tensor, its block among the tensor's, and
    // this wave's first row.
    struct Part {
        const u32x4 *w4;
        const uint16_t *cb, *x;
        float *y;
        uint32_t M, U, P, S, blk, nblk, gw;
        bool dyn;
    };
    auto part = [&](uint32_t p) {
        const ChainPhase &c = ph[p];
        const uint32_t k = group_member(c.g);
        const GemvTensor &T = c.g.t[k];
        Part q;
        q.w4 = T.w4;
        q.cb = T.cb;
        q.x = c.x;
        q.y = T.y;
        q.M = T.M;
        q.U = T.U;
        q.P = c.g.P;
        q.S = c.g.S;
        q.blk = blockIdx.x - c.g.first_block[k];
        q.nblk = c.g.first_block[k + 1] - c.g.first_block[k];
        q.gw = q.blk * kGemvWaves + wave;
        q.dyn = c.g.dyn != 0;
        return q;
    };
    // the wave's first step of a phase (no memory access for a wave without rows)
    auto first_step = [&](u32x4 (&v)[G::LPL], const Part &q) {
        load_step<B>(v, q.w4, min(q.gw, q.M - 1) * q.P, min(64u, q.P), ~uint64_t(0), q.gw < q.M, lane);
    };
    // Phase 0 is staged as in a single launch: codebook and x loads first, then the first step.
    Part cur = part(0);
    u32x4 nxt[G::LPL];
    {
        CbStage<B, NT> cs;
        cs.issue(cur.cb, cur.U, reinterpret_cast<const u32x4 *>(cur.x), tid);
        u32x4 xv[kXPerThread];
        x_stage_load<NT, 0>(xv, cur.x, cur.P, tid);
        issue_barrier();
        first_step(nxt, cur);
        cs.store(cbl, cur.U, tid);
        x_stage_store<NT>(xl, xv, cur.P, tid);
        if (tid == 0) next_row = kGemvWaves;
        lds_barrier();
    }
    for (uint32_t p = 0;; ++p) {
        const bool more = p + 1 < nph;
        Part nx{};
        if (more) nx = part(p + 1);
        auto tail = [&] {
            if (more) first_step(nxt, nx);
        };
        if (cur.gw < cur.M)
            gemv_rows_loop<B, true>(nxt, stage, xl, cbl, &next_row, cur.w4, cur.y, cur.M, cur.P, cur.S, cur.blk,
                                    cur.nblk, cur.dyn, cur.gw, lane, tail);
        else
            tail();
        if (!more) return;
        // End of phase p: each wave's y stores have completed (waitcnt), and after the workgroup
        // barrier no wave uses the table, x or the row counter any more.  The next codebook's
        // loads go out before the grid barrier (they do not depend on x), x's after it.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        CbStage<B, NT> cs;
        cs.issue(nx.cb, nx.U, reinterpret_cast<const u32x4 *>(nx.x), tid);
        if (tid == 0) go_on = chain_barrier(sync, p, gridDim.x, limit) ? 1u : 0u;
        __syncthreads();
        if (!go_on) return;
        u32x4 xv[kXPerThread];
        x_stage_load<NT, kCoherent>(xv, nx.x, nx.P, tid);
        cs.store(cbl, nx.U, tid);
        x_stage_store<NT>(xl, xv, nx.P, tid);
        if (tid == 0) next_row = kGemvWaves;
        lds_barrier();
        cur = nx;
    }
}

// Clears a chain's sync block before each run (a kernel, not a memset, so that graph capture
// records an ordinary node).
__global__ __launch_bounds__(64) void k_chain_reset(ChainSync *s) {
    reinterpret_cast<uint32_t *>(s)[threadIdx.x] = 0u;
}

// ------------------------------------------------------------------------- fast skinny GEMM
// Y[n][M] = X[n][K] . W^T for n = batch <= 16.  A wave owns a 16-row tile and a range of K; a wave
// step covers 256 columns (4 units of 64 fields) of the tile's 16 rows, and lane (i = l % 16,
// g = l / 16) decodes unit g of row i from the wave's private LDS stage.  Batch 9..16
// (k_gemm_mfma): the step's columns of X (all batch rows) are written over the weights once those
// have been read back, and the decoded 8-field groups are the A operand of
// v_mfma_f32_16x16x32_bf16 with X as B.  Batch 1..8 (k_gemm_valu, below) keeps X in registers.
// When the tiles alone cannot fill the CUs, the 8 waves of a workgroup take 8/TW parts of K for
// TW tiles and add their partial sums in LDS, so every Y element is written once (no atomics;
// results do not depend on timing).
constexpr int kGemmWaves = 4;  // two or more workgroups per CU (see the planner in gemm_launch)

template <int B>
struct GemmGeo {
    static constexpr int UD = 2 * B;                         // dwords per 64-field unit
    static constexpr int RCH = 2 * B + 1;                    // chunks of one row's 4-unit segment (+1: half-chunk start)
    static constexpr int SRC = RCH + ((1 - RCH) % 16 + 16) % 16;  // stage row stride, = 1 mod 16 chunks
    static constexpr int STEP_CH = 16 * RCH;                 // chunk slots loaded per step
    static constexpr int LPL = (STEP_CH + 63) / 64;          // 16-byte loads per lane per step
    static constexpr int WSTAGE = 16 * SRC * 16;             // bytes of the weight stage
};
static_assert(GemmGeo<13>::SRC == 33 && GemmGeo<16>::SRC == 33 && GemmGeo<1>::SRC == 17, "stage stride");
static_assert(GemmGeo<1>::WSTAGE >= 16 * 16 * 4, "a wave's stage holds its 16 x 16 partial tile");

constexpr uint32_t kXUnit = 2 * 64 + 16;   // LDS bytes per 64-column unit of one X row (16 B padding)
constexpr uint32_t kXRow = 4 * kXUnit + 16;  // LDS bytes per X row of one step

template <int NB>
struct GemmX {
    static constexpr int CH = NB * 32;                       // X chunks per step (NB rows x 4 units x 8)
    static constexpr int XL = (CH + 63) / 64;                // X loads per lane per step
    static constexpr int BYTES = NB * kXRow;
};

template <int B, int NB>
constexpr uint32_t gemm_stage_bytes() {
    return static_cast<uint32_t>(GemmGeo<B>::WSTAGE > GemmX<NB>::BYTES ? GemmGeo<B>::WSTAGE : GemmX<NB>::BYTES);
}

struct GemmShape {
    uint32_t M, P;          // rows, units per row (K / 64)
    uint32_t tiles;         // ceil(M / 16)
    uint32_t TW, KW;        // tiles per workgroup, parts of K per tile (TW * KW = 8)
    uint32_t part_units;    // units per part of K (multiple of 4)
    uint32_t batch, ldx, ldy;
};

// Up to kMaxGroup tensors that share X (same cols and width b) in one launch: workgroups
// [first_block[t], first_block[t + 1]) belong to tensor t.
struct GemmTensor {
    const u32x4 *w4;
    const uint16_t *cb;
    float *Y;
    uint64_t nch;  // 16-byte chunks of the index stream
    uint32_t M, U, ldy, pad;
};
struct GemmGroup {
    uint32_t first_block[kMaxGroup + 1];
    uint32_t count, P, TW, KW, part_units, batch, ldx;
    GemmTensor t[kMaxGroup];
};

// Cache policy of the skinny GEMMs' weight loads.  A wave step reads 416 bytes of each of 16 rows
// (b = 13), which is not a whole number of 128-byte lines, so the same wave's next step starts in
// the line where this one ended.  Non-temporal loads do not keep that line, and the counters then
// show 1.24x (MFMA) and 1.17x (VALU) the algorithmic bytes read; with the ordinary policy 1.05x and
// 1.04x.  The MFMA GEMM runs 2.6 % faster with the ordinary policy (70B step at batch 16, 47.7 ->
// 49.0 % of peak); the VALU GEMM 2 % slower (t4 MLP at batch 8), so it keeps the non-temporal bit.
constexpr int kGemmMfmaW = 0;
constexpr int kGemmValuW = kStreamOnce;

// Weight loads of one step: slot q = i * RCH + c holds chunk c of row i's segment, which starts at
// the chunk holding unit u0 of row row0 + i.  One buffer resource per tile (base: the chunk of
// unit u0 of row row0, wave-uniform; extent: to the stream's end), so slots past a segment read the
// stream's next chunks and rows past M read zeros; the lanes that decode them are inactive.  The
// host keeps 16 * P * UD dwords below 2^29 so the 32-bit byte offsets cannot wrap.
template <int B, int AUX>
__device__ __forceinline__ void gemm_load_w(u32x4 (&v)[GemmGeo<B>::LPL], const u32x4 *__restrict__ w4,
                                            uint64_t nch, uint32_t row0, uint32_t u0, const GemmShape &s,
                                            int lane) {
    using G = GemmGeo<B>;
    const uint64_t d0 = (static_cast<uint64_t>(row0) * s.P + u0) * G::UD;  // dwords, wave-uniform
    const uint64_t b0 = d0 >> 2;
    const uint32_t ph = static_cast<uint32_t>(d0 & 3u);
    const uint64_t left = nch > b0 ? (nch - b0) * 16 : 0;
    const auto rs = wave_rsrc(w4 + b0, static_cast<uint32_t>(min(left, static_cast<uint64_t>(0x7FFFFFF0u))));
    const uint32_t row_dw = s.P * static_cast<uint32_t>(G::UD);
#pragma unroll
    for (int j = 0; j < G::LPL; ++j) {
        const uint32_t q = min(static_cast<uint32_t>(j * 64 + lane), static_cast<uint32_t>(G::STEP_CH - 1));
        const uint32_t i = q / G::RCH, c = q - i * G::RCH;
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>((((ph + i * row_dw) >> 2) + c) * 16u), 0, AUX);
    }
}

// X loads of one step: chunk q = (n * 4 + u) * 8 + c.  Rows >= batch and units past the wave's range
// read as zero, so the zero weights of inactive lanes never meet a non-finite X value.
template <int NB>
__device__ __forceinline__ void gemm_load_x(u32x4 (&v)[GemmX<NB>::XL], const u32x4 *__restrict__ X4,
                                            uint32_t u0, uint32_t nu, const GemmShape &s, int lane) {
#pragma unroll
    for (int j = 0; j < GemmX<NB>::XL; ++j) {
        const uint32_t q = j * 64 + lane;
        const uint32_t n = q >> 5, u = (q >> 3) & 3, c = q & 7;
        v[j] = (u32x4){0u, 0u, 0u, 0u};
        if (q < static_cast<uint32_t>(GemmX<NB>::CH) && n < s.batch && u < nu)
            v[j] = X4[(static_cast<uint64_t>(n) * s.ldx) / 8 + (u0 + u) * 8 + c];
    }
}

template <int B>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm_mfma(const GemmGroup grp,
                                                               const uint16_t *__restrict__ X) {
    constexpr int NB = 16;
    using G = GemmGeo<B>;
    using XG = GemmX<NB>;
    constexpr int NT = 64 * kGemmWaves;
    constexpr uint32_t SB = gemm_stage_bytes<B, NB>();
    __shared__ __attribute__((aligned(16))) uint16_t cbl[Table<B>::SIZE];
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char *stb = smem + wave * SB;                    // this wave's stage (weights, then X)
    u32x4 *stage = reinterpret_cast<u32x4 *>(stb);
    // Wave w's partial tile (16 x 16 floats) goes to the start of its own stage, which it no longer
    // needs once its last step is read back; the other waves read it only after the barrier.
    auto part_of = [&](uint32_t w) { return reinterpret_cast<float *>(smem + w * SB); };

    // This workgroup's tensor (uniform): count the group boundaries at or below blockIdx.x.
    uint32_t k = 0;
#pragma unroll
    for (int j = 1; j < kMaxGroup; ++j) k += (j < static_cast<int>(grp.count) && blockIdx.x >= grp.first_block[j]) ? 1u : 0u;
    const GemmTensor &T = grp.t[k];
    const u32x4 *w4 = T.w4;
    const uint16_t *cb = T.cb;
    float *Y = T.Y;
    const uint32_t U = T.U;
    GemmShape s;
    s.M = T.M;
    s.P = grp.P;
    s.tiles = (T.M + 15) / 16;
    s.TW = grp.TW;
    s.KW = grp.KW;
    s.part_units = grp.part_units;
    s.batch = grp.batch;
    s.ldx = grp.ldx;
    s.ldy = T.ldy;

    const uint32_t tw = wave % s.TW, kr = wave / s.TW;
    const uint32_t tile = (blockIdx.x - grp.first_block[k]) * s.TW + tw;
    const bool has_tile = tile < s.tiles;
    const uint32_t row0 = min(tile, s.tiles - 1) * 16;
    const uint32_t ku0 = min(kr * s.part_units, s.P), ku1 = min(ku0 + s.part_units, s.P);
    const uint32_t nsteps = has_tile ? (ku1 - ku0 + 3) / 4 : 0;
    const u32x4 *X4 = reinterpret_cast<const u32x4 *>(X);

    // Codebook staging loads before the barrier, the first step's weight and X loads after it.
    CbStage<B, NT> cs;
    cs.issue(cb, U, X4, tid);
    issue_barrier();
    u32x4 nw[G::LPL], nx[XG::XL];
    // A wave whose part of K is empty (ku0 == P) still issues the first weight loads, branch-free;
    // they read the next row (or zeros past the stream) and their data is unused.
    gemm_load_w<B, kGemmMfmaW>(nw, w4, T.nch, row0, ku0, s, lane);
    gemm_load_x<NB>(nx, X4, ku0, min(4u, ku1 - ku0), s, lane);
    cs.store(cbl, U, tid);
    lds_barrier();

    const int li = lane & 15, lg = lane >> 4;
    const bool row_ok = row0 + li < s.M;
    f32x4_t cm = {0.f, 0.f, 0.f, 0.f};

    for (uint32_t st = 0; st < nsteps; ++st) {
        const uint32_t u0 = ku0 + 4 * st;
        // weights: row i's chunks at i * SRC; read back unit g of row li (qword offsets)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < G::LPL; ++j) {
            const uint32_t q = j * 64 + lane;
            if (q < G::STEP_CH) {
                const uint32_t i = q / G::RCH, c = q - i * G::RCH;
                stage[i * G::SRC + c] = nw[j];
            }
        }
        asm volatile("" ::: "memory");
        const uint64_t rr = min(row0 + li, s.M - 1);
        const uint32_t off = static_cast<uint32_t>(((rr * s.P + u0) * G::UD) & 3u);  // 0 or 2 dwords
        const u32x2 *st2 = reinterpret_cast<const u32x2 *>(stage + li * G::SRC) + off / 2 + lg * B;
        uint32_t d[G::UD];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const u32x2 t = st2[j];
            d[2 * j] = t.x; d[2 * j + 1] = t.y;
        }
        asm volatile("" ::: "memory");
        // X over the same stage: row n at n * kXRow, unit u at u * kXUnit, chunk c at 16 c
#pragma unroll
        for (int j = 0; j < XG::XL; ++j) {
            const uint32_t q = j * 64 + lane;
            if (q < static_cast<uint32_t>(XG::CH))
                *reinterpret_cast<u32x4 *>(stb + (q >> 5) * kXRow + ((q >> 3) & 3) * kXUnit + (q & 7) * 16) = nx[j];
        }
        asm volatile("" ::: "memory");
        if (st + 1 < nsteps) {
            const uint32_t nu = min(4u, ku1 - u0 - 4);
            gemm_load_w<B, kGemmMfmaW>(nw, w4, T.nch, row0, u0 + 4, s, lane);
            gemm_load_x<NB>(nx, X4, u0 + 4, nu, s, lane);
        }

        const bool valid = row_ok && u0 + lg < ku1;
        const unsigned char *xb = stb + lg * kXUnit + li * kXRow;  // X row li, unit g: + 16 * f
        uint32_t wv[2][8];
        u32x4 xq[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) wv[0][i] = unit_gather<B>(cbl, d, i);
        xq[0] = *reinterpret_cast<const u32x4 *>(xb);
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            if (f + 1 < 8) {
#pragma unroll
                for (int i = 0; i < 8; ++i) wv[(f + 1) & 1][i] = unit_gather<B>(cbl, d, 8 * (f + 1) + i);
                xq[(f + 1) & 1] = *reinterpret_cast<const u32x4 *>(xb + 16 * (f + 1));
            }
            const uint32_t *w = wv[f & 1];
            u32x4 wp = {w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16)};
            if (!valid) wp = (u32x4){0u, 0u, 0u, 0u};
            // Group f's operand passes through an empty asm that is ordered after group f + 1's
            // LDS reads, so the multiply stays behind them: otherwise the compiler moves some
            // multiplies ahead of the next group's reads and waits for every read before them.
            asm volatile("" : "+v"(wp) :: "memory");
            // B operand: lane (n = l % 16, g) holds X[n][unit g, fields 8f .. 8f + 7]
            cm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wp),
                                                         __builtin_bit_cast(bf16x8_t, xq[f & 1]), cm, 0, 0, 0);
        }
    }

    // This wave's partial tile: MFMA lane l holds rows 4 (l / 16) + r of column l % 16.
    if (s.KW == 1) {
        if (!has_tile) return;
        if (static_cast<uint32_t>(li) < s.batch) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t row = row0 + 4 * lg + r;
                if (row < s.M) Y[static_cast<uint64_t>(li) * s.ldy + row] = cm[r];
            }
        }
        return;
    }
    float *mine = part_of(wave);
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[(4 * lg + r) * 16 + li] = cm[r];
    lds_barrier();
    if (kr != 0 || !has_tile) return;
    // waves of part 0 sum the KW parts of their tile in a fixed order: lane l takes entries 4l .. 4l + 3
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t e = 4 * lane + k, row = e >> 4, n = e & 15;
        float v = 0.f;
        for (uint32_t p = 0; p < s.KW; ++p) v += part_of(p * s.TW + tw)[e];
        if (n < s.batch && n < static_cast<uint32_t>(NB) && row0 + row < s.M) Y[static_cast<uint64_t>(n) * s.ldy + row0 + row] = v;
    }
}

// ---------------------------------------------- skinny GEMM, batch 1..8 (VALU, X in registers)
// Same tiles, stage and split of K as k_gemm_mfma, but X never goes through LDS.  The 16 lanes of
// a DPP row (lanes 16g .. 16g + 15) decode unit g of the step for the tile's 16 rows, so they all
// need the same X values: lane i of the row keeps dwords [2 NB i, 2 NB (i + 1)) of that unit's X
// block, where dword e = (f NB + n) 4 + c is dword c of batch row n's fields 8f .. 8f + 7, and
// every v_dot2c reads its X operand from the owning lane with a row_newbcast DPP broadcast.  For
// group f the owners are lanes 2f and 2f + 1.  The broadcasts are written as inline asm because
// the compiler does not fold a DPP move into v_dot2c; each block starts with s_nop 1, the wait a
// DPP read of a VGPR needs after a VALU write to it, and ends with s_nop 2: on this chip another
// VALU instruction that reads a register a dot instruction has just written needs three wait
// states, and the compiler, which does not see inside the asm, would not insert them.
template <int NB>
struct DppDot;

template <>
struct DppDot<1> {
    template <int F>
    static __device__ __forceinline__ void group(float (&a)[1], const uint32_t (&xr)[2], const uint32_t (&w)[4]) {
        asm volatile(
            "s_nop 1\n"
            "v_dot2c_f32_bf16_dpp %0, %1, %3 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %2, %4 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %1, %5 row_newbcast:%c8 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %2, %6 row_newbcast:%c8 row_mask:0xf bank_mask:0xf\n"
            "s_nop 2\n"
            : "+v"(a[0])
            : "v"(xr[0]), "v"(xr[1]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "i"(2 * F), "i"(2 * F + 1));
    }
};

template <>
struct DppDot<2> {
    template <int F>
    static __device__ __forceinline__ void group(float (&a)[2], const uint32_t (&xr)[4], const uint32_t (&w)[4]) {
        asm volatile(
            "s_nop 1\n"
            "v_dot2c_f32_bf16_dpp %0, %2, %6 row_newbcast:%c10 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %3, %7 row_newbcast:%c10 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %4, %8 row_newbcast:%c10 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %5, %9 row_newbcast:%c10 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %2, %6 row_newbcast:%c11 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %3, %7 row_newbcast:%c11 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %4, %8 row_newbcast:%c11 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %5, %9 row_newbcast:%c11 row_mask:0xf bank_mask:0xf\n"
            "s_nop 2\n"
            : "+v"(a[0]), "+v"(a[1])
            : "v"(xr[0]), "v"(xr[1]), "v"(xr[2]), "v"(xr[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "i"(2 * F), "i"(2 * F + 1));
    }
};

template <>
struct DppDot<4> {
    template <int F>
    static __device__ __forceinline__ void group(float (&a)[4], const uint32_t (&xr)[8], const uint32_t (&w)[4]) {
        asm volatile(
            "s_nop 1\n"
            "v_dot2c_f32_bf16_dpp %0, %4, %12 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %5, %13 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %6, %14 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %7, %15 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %8, %12 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %9, %13 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %10, %14 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %11, %15 row_newbcast:%c16 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %4, %12 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %5, %13 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %6, %14 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %7, %15 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %8, %12 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %9, %13 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %10, %14 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %11, %15 row_newbcast:%c17 row_mask:0xf bank_mask:0xf\n"
            "s_nop 2\n"
            : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
            : "v"(xr[0]), "v"(xr[1]), "v"(xr[2]), "v"(xr[3]), "v"(xr[4]), "v"(xr[5]), "v"(xr[6]), "v"(xr[7]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "i"(2 * F), "i"(2 * F + 1));
    }
};

template <>
struct DppDot<8> {
    template <int F>
    static __device__ __forceinline__ void group(float (&a)[8], const uint32_t (&xr)[16], const uint32_t (&w)[4]) {
        asm volatile(
            "s_nop 1\n"
            "v_dot2c_f32_bf16_dpp %0, %8, %24 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %9, %25 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %10, %26 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %0, %11, %27 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %12, %24 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %13, %25 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %14, %26 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %1, %15, %27 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %16, %24 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %17, %25 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %18, %26 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %2, %19, %27 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %20, %24 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %21, %25 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %22, %26 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %3, %23, %27 row_newbcast:%c28 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %4, %8, %24 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %4, %9, %25 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %4, %10, %26 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %4, %11, %27 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %5, %12, %24 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %5, %13, %25 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %5, %14, %26 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %5, %15, %27 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %6, %16, %24 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %6, %17, %25 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %6, %18, %26 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %6, %19, %27 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %7, %20, %24 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %7, %21, %25 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %7, %22, %26 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "v_dot2c_f32_bf16_dpp %7, %23, %27 row_newbcast:%c29 row_mask:0xf bank_mask:0xf\n"
            "s_nop 2\n"
            : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
            : "v"(xr[0]), "v"(xr[1]), "v"(xr[2]), "v"(xr[3]), "v"(xr[4]), "v"(xr[5]), "v"(xr[6]), "v"(xr[7]), "v"(xr[8]), "v"(xr[9]), "v"(xr[10]), "v"(xr[11]), "v"(xr[12]), "v"(xr[13]), "v"(xr[14]), "v"(xr[15]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "i"(2 * F), "i"(2 * F + 1));
    }
};

// X registers of one step for lane (i, g): chunk q = f NB + n (16 bytes: fields 8f .. 8f + 7 of
// batch row n, unit u) for q in [i NB / 2, (i + 1) NB / 2); for NB = 1, half of chunk i / 2.  The
// loads go through a buffer resource over X's batch rows (`xs`, batch * ldx elements; the host
// keeps that under 2^30 bytes).  Rows >= batch and units past the wave's range get an offset past
// the resource and read zeros with no memory access, so there is neither a branch nor a zero fill.
constexpr uint32_t kPastResource = 0x80000000u;

template <int NB>
__device__ __forceinline__ void gemm_load_xr(uint32_t (&v)[2 * NB], __amdgpu_buffer_rsrc_t xs, uint32_t u,
                                             bool unit_ok, const GemmShape &s, int li) {
    if constexpr (NB == 1) {
        const uint32_t f = static_cast<uint32_t>(li) >> 1, c = (static_cast<uint32_t>(li) & 1u) * 2u;
        const uint32_t off = unit_ok ? (u * 64u + 8u * f + 2u * c) * 2u : kPastResource;
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(xs, static_cast<int>(off), 0, 0);
        v[0] = t.x;
        v[1] = t.y;
    } else {
#pragma unroll
        for (int h = 0; h < NB / 2; ++h) {
            const uint32_t q = static_cast<uint32_t>(li) * (NB / 2) + h;
            const uint32_t f = q / NB, n = q % NB;
            const uint32_t off = (unit_ok && n < s.batch) ? (n * s.ldx + u * 64u + 8u * f) * 2u : kPastResource;
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(xs, static_cast<int>(off), 0, 0);
            v[4 * h] = t.x; v[4 * h + 1] = t.y; v[4 * h + 2] = t.z; v[4 * h + 3] = t.w;
        }
    }
}

// Decode the lane's unit (d, UD dwords read back from the stage) and accumulate its dot products
// with the step's X registers.  The gathers of 8-field group f + 1 are issued before the dot
// products of group f (the empty asm keeps the compiler from hoisting every gather of the step
// ahead of the first multiply), so each wave's LDS latency overlaps its own VALU work.
template <int B, int NB, int F>
__device__ __forceinline__ void valu_group(float (&acc)[NB], const uint32_t (&d)[GemmGeo<B>::UD],
                                           const uint16_t *cbl, const uint32_t (&xr)[2 * NB],
                                           uint32_t (&w)[2][8]) {
    if constexpr (F + 1 < 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[(F + 1) & 1][i] = unit_gather<B>(cbl, d, 8 * (F + 1) + i);
    }
    asm volatile("" ::: "memory");
    uint32_t wp[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) wp[c] = w[F & 1][2 * c] | (w[F & 1][2 * c + 1] << 16);
    DppDot<NB>::template group<F>(acc, xr, wp);
}

template <int B, int NB, int... F>
__device__ __forceinline__ void valu_unit_groups(float (&acc)[NB], const uint32_t (&d)[GemmGeo<B>::UD],
                                                 const uint16_t *cbl, const uint32_t (&xr)[2 * NB],
                                                 std::integer_sequence<int, F...>) {
    uint32_t w[2][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[0][i] = unit_gather<B>(cbl, d, i);
    (valu_group<B, NB, F>(acc, d, cbl, xr, w), ...);
}

template <int B, int NB>
__device__ __forceinline__ void valu_unit(float (&acc)[NB], const uint32_t (&d)[GemmGeo<B>::UD],
                                          const uint16_t *cbl, const uint32_t (&xr)[2 * NB]) {
    valu_unit_groups<B, NB>(acc, d, cbl, xr, std::make_integer_sequence<int, 8>{});
}

// One wave step of k_gemm_valu: stage the step's weights (nw) and read back the lane's unit, issue
// the next step's loads (weights into nw, X into xn), then decode and multiply with this step's X
// (xc).  The caller alternates two X register sets, so no X register is copied.
template <int B, int NB, bool LAST>
__device__ __forceinline__ void valu_step(float (&acc)[NB], u32x4 (&nw)[GemmGeo<B>::LPL],
                                          const uint32_t (&xc)[2 * NB], uint32_t (&xn)[2 * NB], u32x4 *stage,
                                          const uint16_t *cbl, const u32x4 *__restrict__ w4, uint64_t nch,
                                          __amdgpu_buffer_rsrc_t xs, const GemmShape &s, uint32_t row0,
                                          uint32_t ku1, uint32_t u0, int lane) {
    using G = GemmGeo<B>;
    const int li = lane & 15, lg = lane >> 4;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < G::LPL; ++j) {
        const uint32_t q = j * 64 + lane;
        if (q < G::STEP_CH) {
            const uint32_t i = q / G::RCH, c = q - i * G::RCH;
            stage[i * G::SRC + c] = nw[j];
        }
    }
    asm volatile("" ::: "memory");
    const uint64_t rr = min(row0 + li, s.M - 1);
    const uint32_t off = static_cast<uint32_t>(((rr * s.P + u0) * G::UD) & 3u);  // 0 or 2 dwords
    const u32x2 *st2 = reinterpret_cast<const u32x2 *>(stage + li * G::SRC) + off / 2 + lg * B;
    uint32_t d[G::UD];
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const u32x2 t = st2[j];
        d[2 * j] = t.x; d[2 * j + 1] = t.y;
    }
    asm volatile("" ::: "memory");
    // The next step's loads (every step but the wave's last), ahead of the multiply, which hides
    // their latency; the wait before the multiply then covers this step's X only.
    if constexpr (!LAST) {
        gemm_load_w<B, kGemmValuW>(nw, w4, nch, row0, u0 + 4, s, lane);
        gemm_load_xr<NB>(xn, xs, u0 + 4 + lg, u0 + 4 + lg < ku1, s, li);
        asm volatile("" ::: "memory");
    }
    // A step that runs past the wave's part of K (only the last one, LAST, when K / 64 is not a
    // multiple of 4): the lanes of units past it keep their sums from before the step.  Their X is
    // zero, but the stage there holds other data, whose table entries may be NaN (the padding).
    // Lanes of rows past M need nothing: their sums stay in their own lanes and are never written.
    const bool partial = LAST && u0 + 4 > ku1;  // wave-uniform
    float kept[NB];
    if (partial) {
#pragma unroll
        for (int n = 0; n < NB; ++n) kept[n] = acc[n];
    }
    valu_unit<B, NB>(acc, d, cbl, xc);
    if (partial && u0 + lg >= ku1) {
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] = kept[n];
    }
}

template <int B, int NB>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm_valu(const GemmGroup grp,
                                                               const uint16_t *__restrict__ X) {
    using G = GemmGeo<B>;
    constexpr int NT = 64 * kGemmWaves;
    constexpr uint32_t SB = G::WSTAGE;
    __shared__ __attribute__((aligned(16))) uint16_t cbl[Table<B>::SIZE];
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    u32x4 *stage = reinterpret_cast<u32x4 *>(smem + wave * SB);  // this wave's weight stage
    // Wave w's partial tile (16 x 16 floats) goes to the start of its own stage, which it no longer
    // needs once its last step is read back; the other waves read it only after the barrier.
    auto part_of = [&](uint32_t w) { return reinterpret_cast<float *>(smem + w * SB); };

    uint32_t k = 0;
#pragma unroll
    for (int j = 1; j < kMaxGroup; ++j) k += (j < static_cast<int>(grp.count) && blockIdx.x >= grp.first_block[j]) ? 1u : 0u;
    const GemmTensor &T = grp.t[k];
    const u32x4 *w4 = T.w4;
    const uint16_t *cb = T.cb;
    float *Y = T.Y;
    const uint32_t U = T.U;
    GemmShape s;
    s.M = T.M;
    s.P = grp.P;
    s.tiles = (T.M + 15) / 16;
    s.TW = grp.TW;
    s.KW = grp.KW;
    s.part_units = grp.part_units;
    s.batch = grp.batch;
    s.ldx = grp.ldx;
    s.ldy = T.ldy;

    const uint32_t tw = wave % s.TW, kr = wave / s.TW;
    const uint32_t tile = (blockIdx.x - grp.first_block[k]) * s.TW + tw;
    const bool has_tile = tile < s.tiles;
    const uint32_t row0 = min(tile, s.tiles - 1) * 16;
    const uint32_t ku0 = min(kr * s.part_units, s.P), ku1 = min(ku0 + s.part_units, s.P);
    const uint32_t nsteps = has_tile ? (ku1 - ku0 + 3) / 4 : 0;
    const int li = lane & 15, lg = lane >> 4;

    CbStage<B, NT> cs;
    cs.issue(cb, U, reinterpret_cast<const u32x4 *>(X), tid);
    issue_barrier();
    u32x4 nw[G::LPL];
    uint32_t xa[2 * NB], xb[2 * NB];
    gemm_load_w<B, kGemmValuW>(nw, w4, T.nch, row0, ku0, s, lane);
    // X's batch rows as one buffer (the host keeps batch * ldx * 2 bytes under 2^30)
    const auto xs = wave_rsrc(X, s.batch * s.ldx * 2u);
    gemm_load_xr<NB>(xa, xs, ku0 + lg, ku0 + lg < ku1, s, li);
    cs.store(cbl, U, tid);
    lds_barrier();

    const bool row_ok = row0 + li < s.M;
    float acc[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = 0.f;

    // Two steps per trip: the first multiplies X set a and loads set b, the second the reverse.
    // The trips leave the last one or two steps to the code after the loop, so every load inside
    // the loop feeds a later step (the compiler then keeps it ahead of the multiply).
    uint32_t st = 0;
    for (; st + 2 < nsteps; st += 2) {
        valu_step<B, NB, false>(acc, nw, xa, xb, stage, cbl, w4, T.nch, xs, s, row0, ku1, ku0 + 4 * st, lane);
        valu_step<B, NB, false>(acc, nw, xb, xa, stage, cbl, w4, T.nch, xs, s, row0, ku1, ku0 + 4 * (st + 1), lane);
    }
    if (st + 1 < nsteps) {
        valu_step<B, NB, false>(acc, nw, xa, xb, stage, cbl, w4, T.nch, xs, s, row0, ku1, ku0 + 4 * st, lane);
        valu_step<B, NB, true>(acc, nw, xb, xa, stage, cbl, w4, T.nch, xs, s, row0, ku1, ku0 + 4 * (st + 1), lane);
    } else if (st < nsteps) {
        valu_step<B, NB, true>(acc, nw, xa, xb, stage, cbl, w4, T.nch, xs, s, row0, ku1, ku0 + 4 * st, lane);
    }

    // lanes with g = 0 hold row l % 16 of every column after summing the four k-groups
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        float v = acc[n];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[n] = v;
    }
    if (s.KW == 1) {
        if (!has_tile) return;
        if (lg == 0 && row_ok) {
#pragma unroll
            for (int n = 0; n < NB; ++n)
                if (static_cast<uint32_t>(n) < s.batch) Y[static_cast<uint64_t>(n) * s.ldy + row0 + li] = acc[n];
        }
        return;
    }
    float *mine = part_of(wave);
    if (lg == 0) {
#pragma unroll
        for (int n = 0; n < NB; ++n) mine[li * 16 + n] = acc[n];
    }
    lds_barrier();
    if (kr != 0 || !has_tile) return;
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
        const uint32_t e = 4 * lane + k2, row = e >> 4, n = e & 15;
        float v = 0.f;
        for (uint32_t p = 0; p < s.KW; ++p) v += part_of(p * s.TW + tw)[e];
        if (n < s.batch && n < static_cast<uint32_t>(NB) && row0 + row < s.M) Y[static_cast<uint64_t>(n) * s.ldy + row0 + row] = v;
    }
}

// ------------------------------------------------------------------------ generic kernels
__global__ __launch_bounds__(256) void k_decode_generic(const uint32_t *__restrict__ words,
                                                        uint32_t b, const uint16_t *__restrict__ cb,
                                                        uint32_t U, uint16_t *__restrict__ out,
                                                        uint64_t n) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t idx = stream_field(words, b, i);
        out[i] = idx < U ? cb[idx] : kCorrupt;
    }
}

// One wave per row, grid-stride over rows; NB batch columns (NB <= 16).
template <int NB>
__global__ __launch_bounds__(256) void k_gemm_generic(const uint32_t *__restrict__ words, uint32_t b,
                                                      const uint16_t *__restrict__ cb, uint32_t U,
                                                      const uint16_t *__restrict__ X, uint64_t ldx,
                                                      uint32_t batch, float *__restrict__ Y,
                                                      uint64_t ldy, uint32_t M, uint32_t K) {
    const int lane = threadIdx.x & 63;
    const uint32_t wpb = blockDim.x >> 6;
    for (uint32_t row = blockIdx.x * wpb + (threadIdx.x >> 6); row < M; row += gridDim.x * wpb) {
        float acc[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[n] = 0.f;
        for (uint32_t k = lane; k < K; k += 64) {
            const uint32_t idx = stream_field(words, b, static_cast<uint64_t>(row) * K + k);
            const float w = bf16_value(idx < U ? cb[idx] : kCorrupt);
#pragma unroll
            for (int n = 0; n < NB; ++n)
                if (n < static_cast<int>(batch)) acc[n] = fmaf(w, bf16_value(X[n * ldx + k]), acc[n]);
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            float v = acc[n];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0 && n < static_cast<int>(batch)) Y[n * ldy + row] = v;
        }
    }
}

// ------------------------------------------------------------------------------ host side
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

cbk_status launched() { return hipGetLastError() == hipSuccess ? CBK_OK : CBK_E_HIP; }

// Kernels above 64 KiB of dynamic LDS must raise their limit first.
template <typename K>
bool allow_lds(K kernel, uint32_t lds) {
    if (lds <= 65536) return true;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               static_cast<int>(lds)) == hipSuccess;
}

// Runs Fn<b>::run(args) for the b in Bs that matches; false when none does or run declines.
template <template <int> class Fn, typename Args, int... Bs>
bool dispatch_b(int b, Args &args, std::integer_sequence<int, Bs...>) {
    bool ok = false;
    (void)((b == Bs ? (ok = Fn<Bs>::run(args), true) : false) || ...);
    return ok;
}
using AllB = std::integer_sequence<int, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>;

// A run of up to kMaxDecodeGroup tensors of width B with n > 0 and 16-byte aligned outputs.
struct DecodeArgs {
    const cbk_tensor *ts; uint32_t count; uint16_t *const *outs; hipStream_t s; cbk_status st;
};

template <int B>
struct DecodeRun {
    static bool run(DecodeArgs &a) {
        const uint32_t lds = kDecodeWaves * decode_stage_bytes<B>();
        if (uint64_t(lds) + uint64_t(Table<B>::SIZE) * 2 > kLdsLimit) return false;
        if (!allow_lds(k_decode_fast<B>, lds)) return false;
        DecodeGroup grp{};
        grp.count = a.count;
        uint64_t need[kMaxDecodeGroup], total = 0;
        for (uint32_t i = 0; i < a.count; ++i) {
            const cbk_tensor &t = a.ts[i];
            const uint64_t n = t.rows * t.cols;
            const uint64_t T64 = (n + 63) / 64;
            const uint64_t nchunks = cbk_words_for(n, B) / 4;
            if (T64 * U64<B>::UD / 4 + 64 * U64<B>::LPL >= (uint64_t(1) << 32) || nchunks >= (uint64_t(1) << 32))
                return false;
            if (reinterpret_cast<uintptr_t>(t.codebook) & 15) return false;
            grp.t[i] = DecodeTensor{reinterpret_cast<const u32x4 *>(t.words), t.codebook, a.outs[i], n,
                                    static_cast<uint32_t>(nchunks), t.U, static_cast<uint32_t>(T64)};
            need[i] = std::max<uint64_t>(1, ((T64 + 63) / 64 + kDecodeWaves - 1) / kDecodeWaves);
            total += need[i];
        }
        // two workgroups per CU in all, divided in proportion to the tensors' wave steps, at
        // least one each
        const uint64_t grid = std::max<uint64_t>(a.count, std::min<uint64_t>(2 * cu_count(), total));
        uint32_t at = 0;
        for (uint32_t i = 0; i < a.count; ++i) {
            grp.first_wg[i] = at;
            at += static_cast<uint32_t>(
                std::max<uint64_t>(1, std::min<uint64_t>(need[i], (grid * need[i] + total / 2) / total)));
        }
        for (uint32_t i = a.count; i <= static_cast<uint32_t>(kMaxDecodeGroup); ++i) grp.first_wg[i] = at;
        hipLaunchKernelGGL(k_decode_fast<B>, dim3(at), dim3(64 * kDecodeWaves), lds, a.s, grp);
        a.st = launched();
        return true;
    }
};

// A group of tensors that share x over a grid of `grid` workgroups (grid >= count): workgroups
// per tensor in proportion to its rows, at least one each, and the row claims (dyn).
void split_group(const cbk_tensor *ts, float *const *ys, uint32_t count, uint32_t grid, GemvGroup &grp) {
    const uint64_t P = ts[0].cols / 64;
    uint64_t rows = 0;
    for (uint32_t i = 0; i < count; ++i) rows += ts[i].rows;
    grp.count = count;
    grp.P = static_cast<uint32_t>(P);
    grp.S = static_cast<uint32_t>((P + 63) / 64);
    // Rows claimed dynamically inside each workgroup from 8 rows per wave on: measured 4-7 %
    // faster on 28672 x 8192 (14 rows per wave), even at 4 rows per wave and 3 % slower at 2.
    grp.dyn = rows >= uint64_t(8) * grid * kGemvWaves ? 1u : 0u;
    uint32_t first = 0;
    uint64_t rows_before = 0;
    for (uint32_t i = 0; i < count; ++i) {
        const cbk_tensor &t = ts[i];
        const uint32_t end = (i + 1 == count)
            ? grid
            : std::max<uint32_t>(first + 1, static_cast<uint32_t>(((rows_before + t.rows) * grid + rows / 2) / rows));
        grp.t[i] = GemvTensor{reinterpret_cast<const u32x4 *>(t.words), t.codebook, ys[i], static_cast<uint32_t>(t.rows),
                              t.U};
        grp.first_block[i] = first;
        rows_before += t.rows;
        first = std::min(end, grid - (count - 1 - i));
    }
    grp.first_block[count] = grid;
}

struct GemvArgs {
    const cbk_tensor *ts; uint32_t count; const uint16_t *x; float *const *ys; hipStream_t s; cbk_status st;
};

// One launch for up to kMaxGroup tensors of width B that share x (all have the same cols).
template <int B>
struct GemvRun {
    static bool run(GemvArgs &a) {
        using G = U64<B>;
        const uint64_t K = a.ts[0].cols;
        if (K == 0 || K % 64 != 0 || a.count == 0 || a.count > kMaxGroup) return false;
        const uint64_t P = K / 64;
        if (P * 8 > static_cast<uint64_t>(kXPerThread) * 64 * kGemvWaves) return false;
        uint64_t rows = 0;
        for (uint32_t i = 0; i < a.count; ++i) {
            const cbk_tensor &t = a.ts[i];
            if (t.b != B || t.cols != K || t.rows == 0) return false;
            if (reinterpret_cast<uintptr_t>(t.codebook) & 15) return false;
            if (t.rows * P >= (uint64_t(1) << 32)) return false;
            rows += t.rows;
        }
        const uint64_t lds = P * (2 * 64 + 16) + uint64_t(kGemvWaves) * G::STAGE_CHUNKS * 16;
        if (lds + uint64_t(Table<B>::SIZE) * 2 > kLdsLimit) return false;
        const bool group = a.count > 1;
        if (!(group ? allow_lds(k_gemv_rows_group<B>, static_cast<uint32_t>(lds))
                    : allow_lds(k_gemv_rows<B>, static_cast<uint32_t>(lds))))
            return false;
        // One workgroup per CU (fewer when there are not enough rows for every wave), at least one
        // per tensor.
        const uint32_t grid = static_cast<uint32_t>(std::max<uint64_t>(
            a.count, std::min<uint64_t>(cu_count(), (rows + kGemvWaves - 1) / kGemvWaves)));

        GemvGroup grp{};
        split_group(a.ts, a.ys, a.count, grid, grp);
        if (group) {
            hipLaunchKernelGGL(k_gemv_rows_group<B>, dim3(grid), dim3(64 * kGemvWaves), static_cast<uint32_t>(lds),
                               a.s, grp, a.x);
        } else {
            const GemvTensor &t = grp.t[0];
            hipLaunchKernelGGL(k_gemv_rows<B>, dim3(grid), dim3(64 * kGemvWaves), static_cast<uint32_t>(lds), a.s,
                               t.w4, t.cb, t.y, a.x, t.M, t.U, grp.P, grp.S, grp.dyn);
        }
        a.st = launched();
        return true;
    }
};

struct GemmArgs {
    const cbk_tensor *ts; uint32_t count; const uint16_t *X; uint64_t ldx; uint32_t batch;
    float *const *Ys; const uint64_t *ldys; hipStream_t s; cbk_status st;
};

// One launch for up to kMaxGroup tensors of width B that share X (all have the same cols).
template <int B, int NB, bool MFMA>
bool gemm_launch(GemmArgs &a) {
    const uint64_t P = a.ts[0].cols / 64;
    GemmGroup grp{};
    grp.count = a.count;
    grp.P = static_cast<uint32_t>(P);
    grp.batch = a.batch;
    grp.ldx = static_cast<uint32_t>(a.ldx);
    // LDS: the waves' stages (weights only for the VALU kernel, whose X stays in registers; each
    // wave's partial tile of the split K goes into its own stage after its last step), plus the
    // codebook table.
    const uint32_t stage = MFMA ? gemm_stage_bytes<B, NB>() : static_cast<uint32_t>(GemmGeo<B>::WSTAGE);
    const uint32_t lds = kGemmWaves * stage;  // the partial tiles reuse the stages
    if (uint64_t(lds) + uint64_t(Table<B>::SIZE) * 2 > kLdsLimit) return false;
    // the VALU kernel reads X through one buffer resource with 32-bit offsets
    if (!MFMA && uint64_t(a.batch) * a.ldx * 2 >= (uint64_t(1) << 30)) return false;
    // Tiles per workgroup TW (the other kGemmWaves / TW waves split K).  The LDS decides how many
    // workgroups run on a CU at once (two at b = 13), and the grid drains in ceil(blocks / slots)
    // rounds of workgroups that each take TW tiles by the whole of K: pick the TW with the fewest
    // rounds x TW (refined by how full the rounds are), and of equal ones the largest (fewer
    // workgroups and partial-sum reductions).
    // Four-wave workgroups, two per CU, measured 5.6 % (batch 8) and 3.6 % (batch 16) faster than
    // one eight-wave workgroup per CU.
    const uint64_t per_cu = std::max<uint64_t>(1, kLdsLimit / (uint64_t(lds) + uint64_t(Table<B>::SIZE) * 2));
    const uint64_t cus = static_cast<uint64_t>(cu_count()) * per_cu;
    uint64_t best = ~uint64_t(0);
    for (uint32_t tw = 1; tw <= static_cast<uint32_t>(kGemmWaves); tw *= 2) {
        uint64_t blocks = 0;
        for (uint32_t i = 0; i < a.count; ++i) blocks += ((a.ts[i].rows + 15) / 16 + tw - 1) / tw;
        // whole rounds first, then how full they are in quarters of a round (ties between whole
        // rounds go to the TW whose work fills them better)
        const uint64_t cost = (4 * ((blocks + cus - 1) / cus) + (4 * blocks + cus - 1) / cus) * tw;
        if (cost <= best) {
            best = cost;
            grp.TW = tw;
        }
    }
    grp.KW = kGemmWaves / grp.TW;
    grp.part_units = static_cast<uint32_t>(((P + grp.KW - 1) / grp.KW + 3) / 4 * 4);
    if constexpr (MFMA) {
        if (!allow_lds(k_gemm_mfma<B>, lds)) return false;
    } else {
        if (!allow_lds(k_gemm_valu<B, NB>, lds)) return false;
    }
    uint64_t first = 0;
    for (uint32_t i = 0; i < a.count; ++i) {
        const cbk_tensor &t = a.ts[i];
        grp.t[i] = GemmTensor{reinterpret_cast<const u32x4 *>(t.words), t.codebook, a.Ys[i],
                              cbk_words_for(t.rows * t.cols, B) / 4, static_cast<uint32_t>(t.rows), t.U,
                              static_cast<uint32_t>(a.ldys[i]), 0};
        grp.first_block[i] = static_cast<uint32_t>(first);
        first += ((t.rows + 15) / 16 + grp.TW - 1) / grp.TW;
    }
    grp.first_block[a.count] = static_cast<uint32_t>(first);
    if (first >= (uint64_t(1) << 31)) return false;
    if constexpr (MFMA)
        hipLaunchKernelGGL((k_gemm_mfma<B>), dim3(static_cast<uint32_t>(first)), dim3(64 * kGemmWaves), lds,
                           a.s, grp, a.X);
    else
        hipLaunchKernelGGL((k_gemm_valu<B, NB>), dim3(static_cast<uint32_t>(first)), dim3(64 * kGemmWaves), lds,
                           a.s, grp, a.X);
    return true;
}

template <int B>
struct GemmRun {
    static bool run(GemmArgs &a) {
        const uint64_t K = a.ts[0].cols;
        if (K == 0 || K % 64 != 0 || a.count == 0 || a.count > kMaxGroup) return false;
        if (a.ldx >= (uint64_t(1) << 32)) return false;
        for (uint32_t i = 0; i < a.count; ++i) {
            const cbk_tensor &t = a.ts[i];
            if (t.b != B || t.cols != K || t.rows == 0) return false;
            if (reinterpret_cast<uintptr_t>(t.codebook) & 15) return false;
            if (t.rows * (K / 64) >= (uint64_t(1) << 32)) return false;
            if ((K / 64) * GemmGeo<B>::UD * 16 >= (uint64_t(1) << 29)) return false;  // tile offsets fit 31 bits
            if (a.ldys[i] >= (uint64_t(1) << 32)) return false;
        }
        bool ok;
        switch (a.batch) {
            case 1: ok = gemm_launch<B, 1, false>(a); break;
            case 2: ok = gemm_launch<B, 2, false>(a); break;
            case 3: case 4: ok = gemm_launch<B, 4, false>(a); break;
            case 5: case 6: case 7: case 8: ok = gemm_launch<B, 8, false>(a); break;
            default: ok = gemm_launch<B, 16, true>(a); break;
        }
        if (ok) a.st = launched();
        return ok;
    }
};

}  // namespace

static cbk_status launch_decode_generic(const cbk_tensor &t, uint16_t *out, hipStream_t s) {
    const uint64_t n = t.rows * t.cols;
    const uint32_t grid = static_cast<uint32_t>(std::min<uint64_t>((n + 255) / 256, 65536));
    hipLaunchKernelGGL(k_decode_generic, dim3(grid), dim3(256), 0, s, t.words, t.b, t.codebook, t.U,
                       out, n);
    return launched();
}

cbk_status launch_decode_group(const cbk_tensor *ts, uint32_t count, uint16_t *const *outs, hipStream_t s) {
    // Runs of up to kMaxDecodeGroup consecutive nonempty tensors of one width b > 0 with 16-byte
    // aligned outputs take one fast launch each; the rest, and any run the fast kernel declines,
    // take the generic kernel one tensor at a time.
    auto fast = [&](uint32_t k) {
        return ts[k].b > 0 && ts[k].rows * ts[k].cols > 0 && (reinterpret_cast<uintptr_t>(outs[k]) & 15) == 0;
    };
    uint32_t i = 0;
    while (i < count) {
        if (ts[i].rows * ts[i].cols == 0) {
            ++i;
            continue;
        }
        uint32_t j = i + 1;
        if (fast(i))
            while (j < count && j - i < static_cast<uint32_t>(kMaxDecodeGroup) && fast(j) && ts[j].b == ts[i].b) ++j;
        bool done = false;
        if (fast(i)) {
            DecodeArgs a{ts + i, j - i, outs + i, s, CBK_OK};
            if (dispatch_b<DecodeRun>(static_cast<int>(ts[i].b), a, AllB{})) {
                if (a.st != CBK_OK) return a.st;
                done = true;
            }
        }
        if (!done) {
            for (uint32_t k = i; k < j; ++k) {
                const cbk_status st = launch_decode_generic(ts[k], outs[k], s);
                if (st != CBK_OK) return st;
            }
        }
        i = j;
    }
    return CBK_OK;
}

cbk_status launch_decode(const cbk_tensor &t, uint16_t *out, hipStream_t s) {
    uint16_t *outs[1] = {out};
    return launch_decode_group(&t, 1, outs, s);
}

cbk_status launch_gemm_generic(const cbk_tensor &t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                               float *Y, uint64_t ldy, hipStream_t s) {
    const uint32_t M = static_cast<uint32_t>(t.rows), K = static_cast<uint32_t>(t.cols);
    const uint32_t grid = std::max(1u, std::min<uint32_t>((M + 3) / 4, 4096));
    if (batch <= 8)
        hipLaunchKernelGGL(k_gemm_generic<8>, dim3(grid), dim3(256), 0, s, t.words, t.b, t.codebook,
                           t.U, X, ldx, batch, Y, ldy, M, K);
    else
        hipLaunchKernelGGL(k_gemm_generic<16>, dim3(grid), dim3(256), 0, s, t.words, t.b, t.codebook,
                           t.U, X, ldx, batch, Y, ldy, M, K);
    return launched();
}

cbk_status launch_gemm_group(const cbk_tensor *ts, uint32_t count, const uint16_t *X, uint64_t ldx,
                             uint32_t batch, float *const *Ys, const uint64_t *ldys, hipStream_t s) {
    // Consecutive runs of tensors with the same width take one fast launch each (at most
    // kMaxGroup tensors); anything the fast kernel declines runs the generic kernel.
    const bool x_ok = (reinterpret_cast<uintptr_t>(X) & 15) == 0 && ldx % 8 == 0;
    uint32_t i = 0;
    while (i < count) {
        uint32_t j = i + 1;
        while (j < count && j - i < static_cast<uint32_t>(kMaxGroup) && ts[j].b == ts[i].b) ++j;
        bool done = false;
        if (ts[i].b > 0 && ts[i].cols > 0 && x_ok) {
            GemmArgs a{ts + i, j - i, X, ldx, batch, Ys + i, ldys + i, s, CBK_OK};
            if (dispatch_b<GemmRun>(static_cast<int>(ts[i].b), a, AllB{})) {
                if (a.st != CBK_OK) return a.st;
                done = true;
            }
        }
        if (!done) {
            for (uint32_t k = i; k < j; ++k) {
                if (ts[k].rows == 0) continue;
                cbk_status st = launch_gemm_generic(ts[k], X, ldx, batch, Ys[k], ldys[k], s);
                if (st != CBK_OK) return st;
            }
        }
        i = j;
    }
    return CBK_OK;
}

cbk_status launch_gemm(const cbk_tensor &t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                       float *Y, uint64_t ldy, hipStream_t s) {
    float *Ys[1] = {Y};
    const uint64_t ldys[1] = {ldy};
    return launch_gemm_group(&t, 1, X, ldx, batch, Ys, ldys, s);
}

cbk_status launch_gemv_generic(const cbk_tensor &t, const uint16_t *x, float *y, hipStream_t s) {
    const uint32_t M = static_cast<uint32_t>(t.rows), K = static_cast<uint32_t>(t.cols);
    const uint32_t grid = std::max(1u, std::min<uint32_t>((M + 3) / 4, 4096));
    hipLaunchKernelGGL(k_gemm_generic<1>, dim3(grid), dim3(256), 0, s, t.words, t.b, t.codebook,
                       t.U, x, uint64_t(0), 1u, y, uint64_t(0), M, K);
    return launched();
}

cbk_status launch_gemv_group(const cbk_tensor *ts, uint32_t count, const uint16_t *x, float *const *ys,
                             hipStream_t s) {
    // Consecutive runs of tensors with the same width take one fast launch each (at most
    // kMaxGroup tensors); anything the fast kernel declines runs the generic kernel.
    const bool x_aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    uint32_t i = 0;
    while (i < count) {
        uint32_t j = i + 1;
        while (j < count && j - i < static_cast<uint32_t>(kMaxGroup) && ts[j].b == ts[i].b) ++j;
        bool done = false;
        if (ts[i].b > 0 && ts[i].cols > 0 && x_aligned) {
            GemvArgs a{ts + i, j - i, x, ys + i, s, CBK_OK};
            if (dispatch_b<GemvRun>(static_cast<int>(ts[i].b), a, AllB{})) {
                if (a.st != CBK_OK) return a.st;
                done = true;
            }
        }
        if (!done) {
            for (uint32_t k = i; k < j; ++k) {
                if (ts[k].rows == 0) continue;
                cbk_status st = launch_gemv_generic(ts[k], x, ys[k], s);
                if (st != CBK_OK) return st;
            }
        }
        i = j;
    }
    return CBK_OK;
}

cbk_status launch_gemv(const cbk_tensor &t, const uint16_t *x, float *y, hipStream_t s) {
    float *ys[1] = {y};
    return launch_gemv_group(&t, 1, x, ys, s);
}

// ------------------------------------------------------------------ chained GEMV, host side
namespace {

using ChainB = std::integer_sequence<int, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15>;

struct ChainBuildArgs {
    const cbk_gemv_phase *phases; uint32_t count; void *buffer; cbk_gemv_chain *chain; cbk_status st;
};

// Plans every phase over one workgroup per CU (the grid that a cooperative launch keeps resident)
// and uploads the plan after the zeroed sync block.
template <int B>
struct ChainBuild {
    static bool run(ChainBuildArgs &a) {
        a.st = build(a);
        return true;
    }
    static cbk_status build(const ChainBuildArgs &a) {
        using G = U64<B>;
        uint64_t pmax = 0;
        for (uint32_t p = 0; p < a.count; ++p) pmax = std::max<uint64_t>(pmax, a.phases[p].ts[0].cols / 64);
        const uint64_t xbytes = pmax * (2 * 64 + 16);
        const uint64_t lds = xbytes + uint64_t(kGemvWaves) * G::STAGE_CHUNKS * 16;
        int dev = 0, coop = 0, occ = 0;
        if (hipGetDevice(&dev) != hipSuccess) return CBK_E_HIP;
        if (lds + uint64_t(Table<B>::SIZE) * 2 + 16 > kLdsLimit || !allow_lds(k_gemv_chain<B>, static_cast<uint32_t>(lds)))
            return CBK_E_UNSUPPORTED;
        if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv_chain<B>, 64 * kGemvWaves,
                                                         static_cast<size_t>(lds)) != hipSuccess)
            return CBK_E_HIP;
        if (!coop || occ < 1) return CBK_E_UNSUPPORTED;
        const uint32_t grid = static_cast<uint32_t>(cu_count());
        std::vector<unsigned char> host(gemv_chain_bytes(a.count), 0);
        for (uint32_t p = 0; p < a.count; ++p) {
            ChainPhase c{};
            split_group(a.phases[p].ts, a.phases[p].ys, a.phases[p].count, grid, c.g);
            c.x = a.phases[p].x;
            std::memcpy(host.data() + sizeof(ChainSync) + size_t(p) * sizeof(ChainPhase), &c, sizeof(c));
        }
        if (hipMemcpy(a.buffer, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess) return CBK_E_HIP;
        *a.chain = cbk_gemv_chain{a.buffer, a.count, static_cast<uint32_t>(B), grid, static_cast<uint32_t>(lds),
                                  static_cast<uint32_t>(xbytes), static_cast<uint32_t>(dev)};
        return CBK_OK;
    }
};

struct ChainRunArgs {
    const cbk_gemv_chain *chain; uint64_t limit; hipStream_t s; cbk_status st;
};

template <int B>
struct ChainLaunch {
    static bool run(ChainRunArgs &a) {
        const cbk_gemv_chain &c = *a.chain;
        ChainSync *sync = static_cast<ChainSync *>(c.buffer);
        const ChainPhase *ph = reinterpret_cast<const ChainPhase *>(static_cast<unsigned char *>(c.buffer) + sizeof(ChainSync));
        hipLaunchKernelGGL(k_chain_reset, dim3(1), dim3(64), 0, a.s, sync);
        if (hipGetLastError() != hipSuccess) {
            a.st = CBK_E_HIP;
            return true;
        }
        uint32_t nph = c.phases, xbytes = c.x_bytes;
        uint64_t limit = a.limit;
        void *args[] = {&ph, &nph, &xbytes, &sync, &limit};
        const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(k_gemv_chain<B>), dim3(c.grid),
                                                        dim3(64 * kGemvWaves), args, c.lds_bytes, a.s);
        a.st = e == hipSuccess ? CBK_OK : (e == hipErrorCooperativeLaunchTooLarge ? CBK_E_UNSUPPORTED : CBK_E_HIP);
        return true;
    }
};

}  // namespace

size_t gemv_chain_bytes(uint32_t phases) { return sizeof(ChainSync) + size_t(phases) * sizeof(ChainPhase); }

cbk_status build_gemv_chain(const cbk_gemv_phase *phases, uint32_t count, void *buffer, cbk_gemv_chain *chain) {
    ChainBuildArgs a{phases, count, buffer, chain, CBK_OK};
    if (!dispatch_b<ChainBuild>(static_cast<int>(phases[0].ts[0].b), a, ChainB{})) return CBK_E_UNSUPPORTED;
    return a.st;
}

cbk_status launch_gemv_chain(const cbk_gemv_chain &chain, uint32_t timeout_us, hipStream_t s) {
    int dev = -1, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CBK_E_HIP;
    if (static_cast<uint32_t>(dev) != chain.device) return CBK_E_INVALID;
    // wall-clock ticks of the barrier waits' limit (the counter runs at hipDeviceAttributeWallClockRate kHz)
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return CBK_E_HIP;
    ChainRunArgs a{&chain, uint64_t(timeout_us) * uint64_t(khz) / 1000u, s, CBK_OK};
    if (!dispatch_b<ChainLaunch>(static_cast<int>(chain.b), a, ChainB{})) return CBK_E_INVALID;
    return a.st;
}

cbk_status gemv_chain_check(const cbk_gemv_chain &chain) {
    uint32_t failed = 0;
    if (hipMemcpy(&failed, static_cast<unsigned char *>(chain.buffer) + offsetof(ChainSync, failed), sizeof(failed),
                  hipMemcpyDeviceToHost) != hipSuccess)
        return CBK_E_HIP;
    return failed ? CBK_E_TIMEOUT : CBK_OK;
}

}  // namespace cbk
