// GPU decode of the exponent entropy-coded BF16 format for gfx950.
//
// The decoder follows the DFloat11 article (gadzety360.pl, "Jak to działa w praktyce?"): a compact
// lookup table held in on-chip memory, and a two-phase pass in which each thread first finds how
// many values it will decode and, after a synchronisation, decodes them into their places.  Here
// one workgroup of 256 threads takes one block of 256 spans (64 stream bits each):
//   1. the format's 4,096-entry table (exponent | length << 8 for every 12-bit window) is turned,
//      once per workgroup, into an LDS table that also gives the second code of the window when
//      both fit in its 12 bits, which halves the lookups of the serial walks below;
//   2. each thread loads its span's three stream words (the span and the 32 bits after it, which
//      cover the longest code that starts in it) and its 4-bit gap (the next block's are loaded
//      while the current one is written out), and walks the codes that start in the span,
//      counting them;
//   3. a workgroup prefix sum of the counts gives every thread the offset of its first value
//      within the block; the thread walks its span again and writes the exponents to an LDS
//      array at those offsets;
//   4. the block's values, bases[k] .. bases[k] + total, are joined with their sign-mantissa bytes
//      (coalesced 8-byte loads, issued with the block's stream loads) and written as 16-byte
//      non-temporal stores (element stores at the two ragged ends of the block's range).
// With a span index (one byte per span: the codes that start in it, written once by k_ec_index
// with the same walk), the `_ix` kernels read each span's count with its stream words and skip
// the counting walk of step 2.  A launch takes up to eight tensors, its workgroups divided among
// them (a transformer block's matrices decoded together).  The `_fit` decode kernels keep half a
// block's worst case of exponents in LDS, for tensors whose blocks all hold at most kFitCodes
// codes, and so run six workgroups per CU instead of four.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "cbk_internal.h"

namespace cbk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kSpansPerBlock = CBK_EC_BLOCK_SPANS;  // = threads per workgroup
constexpr int kMaxPerSpan = CBK_EC_SPAN_BITS;       // codes are at least one bit long
constexpr int kLutEntries = CBK_EC_LUT_ENTRIES;
constexpr int kStreamOnce = 2;                      // non-temporal: data touched once
constexpr int kJoinAhead = 4;                       // join segments per thread loaded in advance
// The fitted decode holds the exponents of blocks of at most kFitCodes codes (a block's first
// weight can sit up to 7 places into the array's first 8-byte word): half the worst case, so that
// six workgroups fit a CU instead of four.
constexpr uint32_t kFitCodes = kSpansPerBlock * kMaxPerSpan / 2 - 7;

static_assert(kSpansPerBlock == 256, "one thread per span, 256 spans per block");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(static_cast<uint32_t>(bytes)), 0x00020000);
}

// The 12 stream bits starting at bit pos (< 64) of the 96-bit window w0 | w1 << 32 | w2 << 64:
// one funnel shift of the two words that hold them.
__device__ __forceinline__ uint32_t window12(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t pos) {
    const bool low = pos < 32;
    return __builtin_amdgcn_alignbit(low ? w1 : w2, low ? w0 : w1, pos & 31u) & (kLutEntries - 1);
}

// Rows a block can touch in the fused GEMV: its at most 16,384 weights over rows of at least
// kGemvMinCols columns, plus the two partial rows at its ends.
constexpr uint32_t kGemvMinCols = 64;
constexpr uint32_t kGemvBlockRows = kSpansPerBlock * kMaxPerSpan / kGemvMinCols + 2;

// Fused GEMV output: y (zero-filled beforehand) and x, for rows of `cols` weights.  Row indices
// come from v / cols computed by a multiply and shifts (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, section 4): with l = ceil(log2 cols),
// magic = floor(2^32 (2^l - cols) / cols) + 1, sh1 = min(l, 1), sh2 = max(l - 1, 0), exact for every
// 32-bit v.
struct EcGemvOut {
    const uint16_t *x;
    float *y;
    uint32_t cols, magic, sh1, sh2;
};

__device__ __forceinline__ uint32_t row_of(uint32_t v, const EcGemvOut &gv) {
    const uint32_t hi = __umulhi(v, gv.magic);
    return (hi + ((v - hi) >> gv.sh1)) >> gv.sh2;
}

// One step of a wave sum: v plus v moved by the DPP control CTRL within the rows in ROWS (lanes
// whose source is out of range add zero).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// The sum of v over the 64 lanes, in lane 63: prefix sums within each 16-lane row (row_shr 1, 2,
// 4, 8), then lane 15 of rows 0 and 2 carried into rows 1 and 3 (row_bcast:15) and lane 31 into
// rows 2 and 3 (row_bcast:31).  All VALU; no LDS round trips.
__device__ __forceinline__ float wave_sum_last(float v) {
    v = dpp_add<0x111, 0xF>(v);
    v = dpp_add<0x112, 0xF>(v);
    v = dpp_add<0x114, 0xF>(v);
    v = dpp_add<0x118, 0xF>(v);
    v = dpp_add<0x142, 0xA>(v);
    return dpp_add<0x143, 0xC>(v);
}

// Inclusive prefix sum of v over the wave's 64 lanes (all active), on the VALU: the same row
// shifts and row broadcasts as wave_sum_last leave every lane with the sum up to itself.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_addu(uint32_t v) {
    return v + static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, false));
}

__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
    v = dpp_addu<0x111, 0xF>(v);
    v = dpp_addu<0x112, 0xF>(v);
    v = dpp_addu<0x114, 0xF>(v);
    v = dpp_addu<0x118, 0xF>(v);
    v = dpp_addu<0x142, 0xA>(v);
    return dpp_addu<0x143, 0xC>(v);
}

// a.lo * b.lo + a.hi * b.hi + acc for two BF16 pairs, products and sum in fp32
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                           false);
}

// The two-code table, built in LDS by every workgroup from the format's 4,096-entry one-code table
// (exponent | length << 8 per 12-bit window): entry = first exponent | second exponent << 8 |
// first length << 16 | both lengths << 20 | count << 24, count 2 when the second code also lies in
// the 12 bits.  `stage` is 8 KB of LDS for the one-code table, free again on return.  Lengths are
// clamped to 1..12, so every walk advances (a corrupt table cannot stall it).  All threads of the
// workgroup call it (two barriers).
__device__ __forceinline__ void build_multi(const uint16_t *__restrict__ lut, uint32_t *multi, u32x4 *stage,
                                            uint32_t t) {
    const uint16_t *single = reinterpret_cast<const uint16_t *>(stage);
    for (uint32_t i = t; i < kLutEntries / 8; i += kSpansPerBlock) stage[i] = reinterpret_cast<const u32x4 *>(lut)[i];
    __syncthreads();
    for (uint32_t v = t; v < kLutEntries; v += kSpansPerBlock) {
        const uint32_t e1 = single[v], l1 = std::min(std::max(e1 >> 8, 1u), 12u);
        const uint32_t e2 = single[v >> l1], l2 = std::min(std::max(e2 >> 8, 1u), 12u);
        const bool two = l1 + l2 <= CBK_EC_MAX_LEN;
        multi[v] = (e1 & 0xFFu) | (two ? (e2 & 0xFFu) << 8 : 0u) | (l1 << 16) | ((two ? l1 + l2 : l1) << 20) |
                   ((two ? 2u : 1u) << 24);
    }
    __syncthreads();
}

// The number of codes that start in a span: the walk from its gap to its end (end <= 64 bits).
// While the whole 12-bit window lies before the span's end, both codes of a lookup start inside
// the span; the last few bits go one code at a time.  Every step advances at least one bit per
// code, so no span yields more than 64 codes.
__device__ __forceinline__ uint32_t count_span(const uint32_t *multi, uint32_t w0, uint32_t w1, uint32_t w2,
                                               uint32_t gap, uint32_t end) {
    uint32_t cnt = 0, pos = gap;
    for (; pos + CBK_EC_MAX_LEN <= end;) {
        const uint32_t m = multi[window12(w0, w1, w2, pos)];
        cnt += m >> 24;
        pos += (m >> 20) & 15u;
    }
    for (; pos < end; ++cnt) pos += (multi[window12(w0, w1, w2, pos)] >> 16) & 15u;
    return cnt;
}

// GEMV == false: decode to BF16 in out.  GEMV == true: y[r] += sum of W[r][k] x[k] over the
// block's weights, per row in LDS first, then one global atomic add per row the block touches.
// FIT: the exponent array holds kFitCodes values; a block with more (possible only when the
// caller's bound on the codes per block was wrong) is skipped, its outputs left as they were.
// The workgroup takes blocks k_first, k_first + stride, ... of its tensor.
template <bool GEMV, bool IX, bool FIT>
__device__ __forceinline__ void ec_blocks(const uint8_t *__restrict__ sm, const uint32_t *__restrict__ stream,
                                          const uint32_t *__restrict__ gaps, const uint32_t *__restrict__ bases,
                                          const uint16_t *__restrict__ lut, const uint8_t *__restrict__ index,
                                          uint16_t *__restrict__ out, EcGemvOut gv, uint64_t n, uint64_t total_bits,
                                          uint32_t spans, uint32_t blocks, uint32_t k_first, uint32_t stride) {
    // two codes per lookup: entry = first exponent | second exponent << 8 | first length << 16 |
    // both lengths << 20 | count << 24, count 2 when the second code also lies in the 12 bits
    __shared__ uint32_t multi[kLutEntries];
    // exponents of one block, placed so that index i holds the value of weight (base & ~7) + i;
    // 16 spare bytes cover the 8-byte reads at the end of the range (FIT: and 64 the codes a
    // thread can write past its count when an index is wrong)
    __shared__ uint64_t exps8[FIT ? (kFitCodes + 7 + 16 + kMaxPerSpan) / 8 : (kSpansPerBlock * kMaxPerSpan + 16) / 8];
    __shared__ uint32_t wave_sum[kSpansPerBlock / 64];
    __shared__ float row_sum[GEMV ? kGemvBlockRows : 1];
    uint8_t *exps = reinterpret_cast<uint8_t *>(exps8);
    const uint32_t t = threadIdx.x, lane = t & 63, wave = t >> 6;

    // the format's one-code table goes through the (still unused) exponent array
    static_assert(sizeof(exps8) >= kLutEntries * 2, "table staging fits the exponent array");
    if constexpr (GEMV)
        for (uint32_t i = t; i < kGemvBlockRows; i += kSpansPerBlock) row_sum[i] = 0.f;
    build_multi(lut, multi, reinterpret_cast<u32x4 *>(exps8), t);

    const uint64_t stream_bytes = 8 * static_cast<uint64_t>(spans);
    const uint64_t gap_bytes = 4 * ((static_cast<uint64_t>(spans) + 7) / 8);
    // one block's inputs: its stream words and gaps go through resources clipped to the arrays
    // (reads past their ends give zero without touching memory; a block past the last reads
    // nothing)
    // the sm allocation is readable up to n rounded up to 16 bytes, so whole dwords are in range
    const uint64_t sm_bytes = (n + 15) & ~uint64_t(15);
    struct BlockIn {
        u32x2 ab;
        uint32_t c, gword;
        uint32_t cnt;  // IX: the span's code count from the index
        uint64_t base;
        u32x2 smp[kJoinAhead];  // sm bytes of the block's first kJoinAhead segments per thread
        // GEMV: x under those segments and their rows
        u32x4 xq[GEMV ? kJoinAhead : 1];
        uint32_t row[GEMV ? kJoinAhead : 1];
    };
    // base, limit: bases[k] and bases[k + 1] (n for the last block), read one block earlier so that
    // the sm loads need not wait for them; the loads stay within the block's own bytes
    auto fetch = [&](uint32_t k, uint64_t base, uint64_t limit) {
        BlockIn in;
        const bool live = k < blocks;
        const uint64_t sw0 = static_cast<uint64_t>(k) * kSpansPerBlock * 8;  // byte offset
        const __amdgpu_buffer_rsrc_t rs = rsrc(reinterpret_cast<const uint8_t *>(stream) + (live ? sw0 : 0),
                                               live ? std::min<uint64_t>(stream_bytes - sw0, kSpansPerBlock * 8 + 4) : 0);
        in.ab = __builtin_amdgcn_raw_buffer_load_b64(rs, static_cast<int>(t * 8), 0, kStreamOnce);
        in.c = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(t * 8 + 8), 0, kStreamOnce);
        const uint64_t gw0 = static_cast<uint64_t>(k) * (kSpansPerBlock / 8) * 4;
        const __amdgpu_buffer_rsrc_t rg = rsrc(reinterpret_cast<const uint8_t *>(gaps) + (live ? gw0 : 0),
                                               live ? std::min<uint64_t>(gap_bytes - gw0, kSpansPerBlock / 2) : 0);
        in.gword = __builtin_amdgcn_raw_buffer_load_b32(rg, static_cast<int>((t / 8) * 4), 0, 0);
        in.cnt = 0;
        if constexpr (IX) {
            const uint64_t i0 = static_cast<uint64_t>(k) * kSpansPerBlock;
            const __amdgpu_buffer_rsrc_t ri = rsrc(index + (live ? i0 : 0),
                                                   live ? std::min<uint64_t>(spans - i0, kSpansPerBlock) : 0);
            in.cnt = __builtin_amdgcn_raw_buffer_load_b8(ri, static_cast<int>(t), 0, kStreamOnce);
        }
        in.base = base;
        const uint64_t m0 = (base / 8) * 8;
        const uint64_t m1 = std::min<uint64_t>((std::min(limit, n) + 7) / 8 * 8, sm_bytes);
        const bool sm_live = live && m0 < m1;
        const __amdgpu_buffer_rsrc_t rm = rsrc(sm + (sm_live ? m0 : 0),
                                               sm_live ? std::min<uint64_t>(m1 - m0, kJoinAhead * kSpansPerBlock * 8) : 0);
#pragma unroll
        for (int i = 0; i < kJoinAhead; ++i)
            in.smp[i] = __builtin_amdgcn_raw_buffer_load_b64(rm, static_cast<int>((t + i * kSpansPerBlock) * 8), 0, kStreamOnce);
        if constexpr (GEMV) {
            // Loaded here, one block ahead, with the block's other inputs: the memory counter is
            // in order, so an x load issued in the join would also wait for the next block's
            // prefetch.  Weight index g (wrapped to 32 bits past the end) lies in row g / cols
            // at column g - row * cols < cols, so every load is inside x.
#pragma unroll
            for (int i = 0; i < kJoinAhead; ++i) {
                const uint32_t g32 = static_cast<uint32_t>((base / 8 + t + i * kSpansPerBlock) * 8);
                const uint32_t r = row_of(g32, gv);
                in.row[i] = r;
                in.xq[i] = *reinterpret_cast<const u32x4 *>(gv.x + (g32 - r * gv.cols));
            }
        }
        return in;
    };

    auto base_of = [&](uint32_t k) { return k < blocks ? static_cast<uint64_t>(bases[k]) : n; };
    BlockIn cur = fetch(k_first, base_of(k_first), base_of(k_first + 1));
    for (uint32_t k = k_first; k < blocks; k += stride) {
        const uint64_t j = static_cast<uint64_t>(k) * kSpansPerBlock + t;
        const uint64_t base = cur.base;
        const uint64_t base_after = base_of(k + stride), limit_after = base_of(k + stride + 1);
        const uint32_t gap = (cur.gword >> (4 * (t % 8))) & 15u;
        uint32_t end = 0;
        if (j < spans) {
            const uint64_t rem = total_bits - j * CBK_EC_SPAN_BITS;
            end = rem < CBK_EC_SPAN_BITS ? static_cast<uint32_t>(rem) : CBK_EC_SPAN_BITS;
        }
        const uint32_t w0 = cur.ab.x, w1 = cur.ab.y, w2 = cur.c;

        // phase 1: how many codes start in this span, walked, or read from the index (a count
        // above 64 can only come from a wrong index; clamped, every write below stays in the
        // exponent array and the block's range)
        uint32_t cnt;
        if constexpr (IX)
            cnt = j < spans ? std::min(cur.cnt, static_cast<uint32_t>(kMaxPerSpan)) : 0u;
        else
            cnt = count_span(multi, w0, w1, w2, gap, end);

        // prefix sum of the counts over the workgroup
        const uint32_t incl = wave_scan(cnt);
        if (lane == 63) wave_sum[wave] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int i = 0; i < kSpansPerBlock / 64; ++i) {
            before += static_cast<uint32_t>(i) < wave ? wave_sum[i] : 0u;
            total += wave_sum[i];
        }
        uint32_t at = static_cast<uint32_t>(base & 7) + before + incl - cnt;
        // FIT: the block's exponents fit the array (the same in every lane)
        const bool fits = !FIT || __builtin_amdgcn_readfirstlane(total) <= kFitCodes;

        // phase 2: the walk again (the only one with the index), exponents to their places
        uint32_t pos = fits ? gap : end;
        for (; pos + CBK_EC_MAX_LEN <= end;) {
            const uint32_t m = multi[window12(w0, w1, w2, pos)];
            exps[at] = static_cast<uint8_t>(m);
            if ((m >> 24) == 2u) exps[at + 1] = static_cast<uint8_t>(m >> 8);
            at += m >> 24;
            pos += (m >> 20) & 15u;
        }
        for (; pos < end; ++at) {
            const uint32_t m = multi[window12(w0, w1, w2, pos)];
            exps[at] = static_cast<uint8_t>(m);
            pos += (m >> 16) & 15u;
        }
        __syncthreads();
        const BlockIn nxt = fetch(k + stride, base_after, limit_after);  // in flight during the join

        // join with the sign-mantissa bytes: weights [base, base + total), clipped to n, in
        // 8-weight segments s0 .. s1 (segment s0 + t + i * 256 for the thread's i-th)
        const uint64_t stop = std::min<uint64_t>(base + total, n);
        if (fits && base < stop) {
            const uint64_t s0 = base / 8, s1 = (stop + 7) / 8;
            // GEMV: one wave-wide call (every lane, `valid` false past s1) can reduce the wave's
            // partial sums in registers when they all belong to one row, the common case
            const uint32_t r0 = GEMV ? row_of(static_cast<uint32_t>(base), gv) : 0u;
            // (xq, r: x under segment sg and its row, GEMV only)
            auto join = [&](uint64_t sg, u32x2 smv, u32x4 xq, uint32_t r, bool valid, bool whole_wave) {
                const uint64_t g0 = sg * 8;
                const uint64_t ev = valid ? exps8[sg - s0] : 0;
                // four weights per word: high byte = sign | exponent >> 1, low byte = exponent
                // bit 0 << 7 | mantissa; v_perm interleaves the low and high bytes
                u32x4 o;
                uint32_t *op = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t b4 = h ? smv.y : smv.x;
                    const uint32_t e4 = static_cast<uint32_t>(ev >> (32 * h));
                    const uint32_t hi4 = (b4 & 0x80808080u) | ((e4 >> 1) & 0x7F7F7F7Fu);
                    const uint32_t lo4 = ((e4 & 0x01010101u) << 7) | (b4 & 0x7F7F7F7Fu);
                    op[2 * h] = __builtin_amdgcn_perm(hi4, lo4, 0x05010400u);
                    op[2 * h + 1] = __builtin_amdgcn_perm(hi4, lo4, 0x07030602u);
                }
                if constexpr (GEMV) {
                    // 8 weights of one row (cols % 8 == 0): BF16 pair products summed in fp32,
                    // added to the row's LDS partial
                    uint32_t rl = ~0u;
                    float acc = 0.f;
                    if (valid) {
                        uint32_t *xw = reinterpret_cast<uint32_t *>(&xq);
                        if (g0 < base || g0 + 8 > stop) {
                            // a segment at an end of the block: the weights outside [base, stop)
                            // belong to the neighbouring block, so both operands of theirs are
                            // zeroed (0 x 0, whatever x holds)
#pragma unroll
                            for (int h = 0; h < 4; ++h) {
                                const uint64_t e = g0 + 2 * h;
                                const uint32_t keep = (e >= base && e < stop ? 0x0000FFFFu : 0u) |
                                                      (e + 1 >= base && e + 1 < stop ? 0xFFFF0000u : 0u);
                                op[h] &= keep;
                                xw[h] &= keep;
                            }
                        }
                        acc = dot2(op[3], xw[3], dot2(op[2], xw[2], dot2(op[1], xw[1], dot2(op[0], xw[0], 0.f))));
                        rl = r - r0;
                    }
                    if (whole_wave) {
                        const uint32_t first = __builtin_amdgcn_readfirstlane(rl);
                        if (__all(!valid || rl == first)) {
                            acc = wave_sum_last(acc);
                            if (lane == 63 && first != ~0u) atomicAdd(&row_sum[first], acc);
                            return;
                        }
                    }
                    if (valid) atomicAdd(&row_sum[rl], acc);
                } else if (!valid) {
                    return;
                } else if (g0 >= base && g0 + 8 <= stop) {
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + g0));
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (g0 + e >= base && g0 + e < stop)
                            out[g0 + e] = static_cast<uint16_t>(op[e >> 1] >> (16 * (e & 1)));
                }
            };
#pragma unroll
            for (int i = 0; i < kJoinAhead; ++i) {
                const uint64_t sg = s0 + t + i * kSpansPerBlock;
                if (GEMV)
                    join(sg, cur.smp[i], cur.xq[i], cur.row[i], sg < s1, true);
                else if (sg < s1)
                    join(sg, cur.smp[i], u32x4{}, 0, true, false);
            }
            // blocks with more than kJoinAhead * 2048 values (codes under 2 bits on average)
            if (s0 + kJoinAhead * kSpansPerBlock < s1) {
                const __amdgpu_buffer_rsrc_t rm = rsrc(sm + s0 * 8, std::min<uint64_t>(sm_bytes - s0 * 8, (s1 - s0) * 8));
                for (uint64_t sg = s0 + t + kJoinAhead * kSpansPerBlock; sg < s1; sg += kSpansPerBlock) {
                    const u32x2 smv = __builtin_amdgcn_raw_buffer_load_b64(rm, static_cast<int>((sg - s0) * 8), 0, kStreamOnce);
                    if constexpr (GEMV) {
                        const uint32_t g32 = static_cast<uint32_t>(sg * 8), r = row_of(g32, gv);
                        join(sg, smv, *reinterpret_cast<const u32x4 *>(gv.x + (g32 - r * gv.cols)), r, true, false);
                    } else {
                        join(sg, smv, u32x4{}, 0, true, false);
                    }
                }
            }
        }
        if constexpr (GEMV) {
            // the block's rows: one global add each (rows at the block's ends are shared with the
            // neighbouring blocks), then the partials are cleared for the next block
            __syncthreads();
            if (base < stop) {
                const uint32_t r0 = row_of(static_cast<uint32_t>(base), gv);
                const uint32_t nr = row_of(static_cast<uint32_t>(stop - 1), gv) - r0 + 1;
                for (uint32_t i = t; i < nr; i += kSpansPerBlock) {
                    atomicAdd(&gv.y[r0 + i], row_sum[i]);
                    row_sum[i] = 0.f;
                }
            }
        }
        __syncthreads();  // the next block reuses wave_sum and exps
        cur = nxt;
    }
}

// One launch decodes up to kMaxEcGroup tensors (a transformer block's matrices together, as in the
// DFloat11 page's block-level decompression): workgroups [first_wg[i], first_wg[i + 1]) take the
// blocks of tensor i, and a single tensor is a group of one.
constexpr uint32_t kMaxEcGroup = 8;
struct EcArgs {
    const uint8_t *sm;
    const uint32_t *stream, *gaps, *bases;
    const uint16_t *lut;
    const uint8_t *index;  // span index (the `_ix` kernels only)
    void *out;             // decode: BF16 patterns; fused GEMV: y (fp32)
    uint64_t n, total_bits;
    uint32_t spans, blocks;
};
struct EcGroup {
    uint32_t first_wg[kMaxEcGroup + 1];  // first_wg[count] = grid size
    uint32_t count;
    uint32_t cols, magic, sh1, sh2;  // fused GEMV: the shared row length and row_of's constants
    const uint16_t *x;
    EcArgs t[kMaxEcGroup];
};

#define CBK_EC_KERNEL(NAME, GEMV, IX, FIT)                                                                     \
    __global__ __launch_bounds__(kSpansPerBlock) void NAME(const EcGroup grp) {                                \
        uint32_t k = 0;                                                                                        \
        _Pragma("unroll") for (uint32_t j = 1; j < kMaxEcGroup; ++j) k +=                                      \
            (j < grp.count && blockIdx.x >= grp.first_wg[j]) ? 1u : 0u;                                        \
        const EcArgs &T = grp.t[k];                                                                            \
        const uint32_t w0 = grp.first_wg[k];                                                                   \
        const EcGemvOut gv{grp.x, static_cast<float *>(T.out), grp.cols, grp.magic, grp.sh1, grp.sh2};         \
        ec_blocks<GEMV, IX, FIT>(T.sm, T.stream, T.gaps, T.bases, T.lut, T.index, static_cast<uint16_t *>(T.out),  \
                                 gv,                                                                              \
                            T.n, T.total_bits, T.spans, T.blocks, blockIdx.x - w0, grp.first_wg[k + 1] - w0);   \
    }
// decode to BF16 and the fused GEMV, each with two walks per span or one walk and the span index;
// the decode also for blocks of at most kFitCodes codes (the fused GEMV keeps four workgroups per
// CU, its registers allowing no more than five, which measured slower)
CBK_EC_KERNEL(k_ec_decode, false, false, false)
CBK_EC_KERNEL(k_ec_gemv, true, false, false)
CBK_EC_KERNEL(k_ec_decode_ix, false, true, false)
CBK_EC_KERNEL(k_ec_gemv_ix, true, true, false)
CBK_EC_KERNEL(k_ec_decode_fit, false, false, true)
CBK_EC_KERNEL(k_ec_decode_ix_fit, false, true, true)
#undef CBK_EC_KERNEL

// The span index: the table walk of phase 1 over every span, its count stored as a byte.
__global__ __launch_bounds__(kSpansPerBlock) void k_ec_index(const uint32_t *__restrict__ stream,
                                                             const uint32_t *__restrict__ gaps,
                                                             const uint16_t *__restrict__ lut, uint8_t *__restrict__ index,
                                                             uint64_t total_bits, uint32_t spans, uint32_t blocks) {
    __shared__ uint32_t multi[kLutEntries];
    __shared__ u32x4 stage[kLutEntries / 8];
    const uint32_t t = threadIdx.x;
    build_multi(lut, multi, stage, t);
    const uint64_t stream_bytes = 8 * static_cast<uint64_t>(spans);
    for (uint32_t k = blockIdx.x; k < blocks; k += gridDim.x) {
        const uint64_t j = static_cast<uint64_t>(k) * kSpansPerBlock + t;
        const uint64_t sw0 = static_cast<uint64_t>(k) * kSpansPerBlock * 8;
        const __amdgpu_buffer_rsrc_t rs = rsrc(reinterpret_cast<const uint8_t *>(stream) + sw0,
                                               std::min<uint64_t>(stream_bytes - sw0, kSpansPerBlock * 8 + 4));
        const u32x2 ab = __builtin_amdgcn_raw_buffer_load_b64(rs, static_cast<int>(t * 8), 0, kStreamOnce);
        const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(t * 8 + 8), 0, kStreamOnce);
        if (j < spans) {
            const uint32_t gap = (gaps[j / 8] >> (4 * (j % 8))) & 15u;
            const uint64_t rem = total_bits - j * CBK_EC_SPAN_BITS;
            const uint32_t end = rem < CBK_EC_SPAN_BITS ? static_cast<uint32_t>(rem) : CBK_EC_SPAN_BITS;
            index[j] = static_cast<uint8_t>(count_span(multi, ab.x, ab.y, c, gap, end));
        }
    }
}

// Zero-fill of the fused GEMV's outputs (a group's in one launch).
struct EcZero {
    float *y[kMaxEcGroup];
    uint64_t rows[kMaxEcGroup];
    uint32_t count;
};
__global__ __launch_bounds__(256) void k_ec_zero(const EcZero z) {
    for (uint32_t g = 0; g < z.count; ++g)
        for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; i < z.rows[g];
             i += static_cast<uint64_t>(gridDim.x) * 256)
            z.y[g][i] = 0.f;
}

// As many workgroups as fit the CUs at once (LDS bound); they loop over the blocks, so the tables
// are built once per workgroup and the next block's loads overlap the current block's output.
template <typename K>
cbk_status resident_grid(K kernel, uint64_t blocks, std::atomic<int> (&per_cu)[64], uint32_t &grid) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return CBK_E_HIP;
    // (the per-device count is queried once; concurrent first calls store the same value)
    if (dev < 0 || dev >= 64) return CBK_E_HIP;
    int occ = per_cu[dev].load(std::memory_order_relaxed);
    if (occ <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kSpansPerBlock, 0) != hipSuccess || occ <= 0)
            return CBK_E_HIP;
        per_cu[dev].store(occ, std::memory_order_relaxed);
    }
    grid = static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(blocks, static_cast<uint64_t>(occ) * cus)));
    return CBK_OK;
}

// One launch for up to kMaxEcGroup tensors with n > 0: the resident grid split over them in
// proportion to their blocks, at least one workgroup each.
template <bool GEMV, bool IX, bool FIT>
cbk_status launch_ec_run(EcGroup &g, hipStream_t s) {
    auto kernel = GEMV ? (IX ? k_ec_gemv_ix : k_ec_gemv)
                       : FIT ? (IX ? k_ec_decode_ix_fit : k_ec_decode_fit) : (IX ? k_ec_decode_ix : k_ec_decode);
    static std::atomic<int> per_cu[64];
    uint64_t total = 0;
    for (uint32_t i = 0; i < g.count; ++i) total += g.t[i].blocks;
    uint32_t grid = 0;
    const cbk_status st = resident_grid(kernel, total, per_cu, grid);
    if (st != CBK_OK) return st;
    uint32_t at = 0;
    for (uint32_t i = 0; i < g.count; ++i) {
        g.first_wg[i] = at;
        const uint64_t share = (static_cast<uint64_t>(grid) * g.t[i].blocks + total / 2) / total;
        at += static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>(share, g.t[i].blocks)));
    }
    for (uint32_t i = g.count; i <= kMaxEcGroup; ++i) g.first_wg[i] = at;
    hipLaunchKernelGGL(kernel, dim3(at), dim3(kSpansPerBlock), 0, s, g);
    return hipGetLastError() == hipSuccess ? CBK_OK : CBK_E_HIP;
}

// The tensors with n > 0, in runs of up to kMaxEcGroup per launch.  outs[i]: BF16 output or y.
template <bool GEMV>
cbk_status launch_ec_all(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count, void *const *outs,
                         EcGroup g, hipStream_t s) {
    g.count = 0;
    bool fit = true;  // every tensor of the run has a known bound of at most kFitCodes per block
    auto flush = [&]() -> cbk_status {
        if (g.count == 0) return CBK_OK;
        cbk_status st;
        if (!GEMV && fit)
            st = indexes ? launch_ec_run<GEMV, true, true>(g, s) : launch_ec_run<GEMV, false, true>(g, s);
        else
            st = indexes ? launch_ec_run<GEMV, true, false>(g, s) : launch_ec_run<GEMV, false, false>(g, s);
        g.count = 0;
        fit = true;
        return st;
    };
    for (uint32_t i = 0; i < count; ++i) {
        const cbk_ec_tensor &t = ts[i];
        if (t.n == 0) continue;
        const uint64_t spans = (t.total_bits + CBK_EC_SPAN_BITS - 1) / CBK_EC_SPAN_BITS;
        fit = fit && t.max_block_codes > 0 && t.max_block_codes <= kFitCodes;
        EcArgs &a = g.t[g.count++];
        a = EcArgs{t.sm, t.stream, t.gaps, t.bases, t.lut, indexes ? indexes[i] : nullptr, outs[i], t.n, t.total_bits,
                   static_cast<uint32_t>(spans), static_cast<uint32_t>((spans + kSpansPerBlock - 1) / kSpansPerBlock)};
        if (g.count == kMaxEcGroup) {
            const cbk_status st = flush();
            if (st != CBK_OK) return st;
        }
    }
    return flush();
}

}  // namespace

cbk_status launch_ec_decode(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                            uint16_t *const *outs, hipStream_t s) {
    EcGroup g{};
    g.cols = g.magic = 1;
    return launch_ec_all<false>(ts, indexes, count, reinterpret_cast<void *const *>(outs), g, s);
}

cbk_status launch_ec_index(const cbk_ec_tensor *t, uint8_t *index, hipStream_t s) {
    const uint64_t spans = (t->total_bits + CBK_EC_SPAN_BITS - 1) / CBK_EC_SPAN_BITS;
    const uint64_t blocks = (spans + kSpansPerBlock - 1) / kSpansPerBlock;
    static std::atomic<int> per_cu[64];
    uint32_t grid = 0;
    const cbk_status st = resident_grid(k_ec_index, blocks, per_cu, grid);
    if (st != CBK_OK) return st;
    hipLaunchKernelGGL(k_ec_index, dim3(grid), dim3(kSpansPerBlock), 0, s, t->stream, t->gaps, t->lut, index,
                       t->total_bits, static_cast<uint32_t>(spans), static_cast<uint32_t>(blocks));
    return hipGetLastError() == hipSuccess ? CBK_OK : CBK_E_HIP;
}

cbk_status launch_ec_gemv(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                          const uint64_t *rows, uint64_t cols, const uint16_t *x, float *const *ys, hipStream_t s) {
    // y is accumulated with atomics, so it starts from zeros: one fill kernel per run of up to
    // kMaxEcGroup outputs (graph capture records it as an ordinary node)
    for (uint32_t i0 = 0; i0 < count; i0 += kMaxEcGroup) {
        EcZero z{};
        uint64_t most = 0;
        for (uint32_t i = i0; i < count && i < i0 + kMaxEcGroup; ++i) {
            if (rows[i] == 0) continue;
            z.y[z.count] = ys[i];
            z.rows[z.count++] = rows[i];
            most = std::max(most, rows[i]);
        }
        if (z.count == 0) continue;
        const uint32_t zgrid = static_cast<uint32_t>(std::max<uint64_t>(1, std::min<uint64_t>((most + 255) / 256, 1024)));
        hipLaunchKernelGGL(k_ec_zero, dim3(zgrid), dim3(256), 0, s, z);
        if (hipGetLastError() != hipSuccess) return CBK_E_HIP;
    }
    if (cols == 0) return CBK_OK;
    // the divisor constants of row_of (cols < 2^32 here, so the product fits 64 bits)
    uint32_t l = 0;
    while ((uint64_t(1) << l) < cols) ++l;
    EcGroup g{};
    g.cols = static_cast<uint32_t>(cols);
    g.magic = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << l) - cols)) / cols + 1);
    g.sh1 = std::min<uint32_t>(l, 1);
    g.sh2 = l > 0 ? l - 1 : 0;
    g.x = x;
    return launch_ec_all<true>(ts, indexes, count, reinterpret_cast<void *const *>(ys), g, s);
}

}  // namespace cbk
