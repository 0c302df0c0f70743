// Host side of the exponent entropy-coded format (DFloat11 article on gadzety360.pl, sections
// "Przełom: DFloat11" and "Jak to działa w praktyce?": Huffman-code the BF16 exponent only, keep
// sign and mantissa raw).  Encoder passes, size helpers and the validation of the GPU decode.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "cbk.h"
#include "cbk_ec.h"
#include "cbk_internal.h"

namespace {

constexpr int kMaxLen = CBK_EC_MAX_LEN;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint64_t spans_for(uint64_t bits) { return (bits + CBK_EC_SPAN_BITS - 1) / CBK_EC_SPAN_BITS; }

// Optimal code lengths under a cap (package-merge): the cheapest 2m - 2 items of the list built by
// kMaxLen - 1 rounds of "pair adjacent items of the sorted list, merge the pairs with the
// leaves" give every symbol's length as its number of appearances.
void capped_lengths(const uint64_t freq[256], uint8_t len[256]) {
    memset(len, 0, 256);
    std::vector<int> syms;
    for (int s = 0; s < 256; ++s)
        if (freq[s]) syms.push_back(s);
    const size_t m = syms.size();
    if (m == 0) return;
    if (m == 1) {
        len[syms[0]] = 1;
        return;
    }
    struct Item {
        uint64_t weight;
        std::vector<uint16_t> count;  // appearances of each present symbol
    };
    std::vector<Item> leaves;
    std::vector<size_t> order(m);
    for (size_t i = 0; i < m; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return freq[syms[a]] < freq[syms[b]]; });
    for (size_t i : order) {
        Item it{freq[syms[i]], std::vector<uint16_t>(m, 0)};
        it.count[i] = 1;
        leaves.push_back(std::move(it));
    }
    std::vector<Item> list = leaves;
    for (int round = 1; round < kMaxLen; ++round) {
        std::vector<Item> packages;
        for (size_t a = 0; a + 1 < list.size(); a += 2) {
            Item p{list[a].weight + list[a + 1].weight, list[a].count};
            for (size_t i = 0; i < m; ++i) p.count[i] += list[a + 1].count[i];
            packages.push_back(std::move(p));
        }
        std::vector<Item> merged;
        merged.reserve(leaves.size() + packages.size());
        size_t i = 0, j = 0;
        while (i < leaves.size() || j < packages.size()) {
            if (j == packages.size() || (i < leaves.size() && leaves[i].weight <= packages[j].weight))
                merged.push_back(leaves[i++]);
            else
                merged.push_back(std::move(packages[j++]));
        }
        list = std::move(merged);
    }
    std::vector<uint32_t> total(m, 0);
    for (size_t k = 0; k < 2 * m - 2; ++k)
        for (size_t i = 0; i < m; ++i) total[i] += list[k].count[i];
    for (size_t i = 0; i < m; ++i) len[syms[i]] = static_cast<uint8_t>(total[i]);
}

// Canonical codes, stored bit-reversed (the code's first bit at bit 0) as the stream holds them.
bool reversed_codes(const uint8_t len[256], uint32_t rev[256]) {
    uint32_t kraft = 0;  // in units of 2^-12
    for (int s = 0; s < 256; ++s) {
        rev[s] = 0;
        if (len[s] > kMaxLen) return false;
        if (len[s]) kraft += 1u << (kMaxLen - len[s]);
    }
    if (kraft > (1u << kMaxLen)) return false;
    uint32_t code = 0;
    int prev = 0;
    bool first = true;
    for (int l = 1; l <= kMaxLen; ++l) {
        for (int s = 0; s < 256; ++s) {
            if (len[s] != l) continue;
            if (first) {
                code = 0;
                first = false;
            } else {
                code = (code + 1) << (l - prev);
            }
            prev = l;
            uint32_t r = 0;
            for (int k = 0; k < l; ++k) r |= ((code >> (l - 1 - k)) & 1u) << k;
            rev[s] = r;
        }
    }
    return true;
}

}  // namespace

extern "C" {

uint64_t cbk_ec_spans(const cbk_ec_header *h) { return h ? spans_for(h->total_bits) : 0; }
uint64_t cbk_ec_stream_words(const cbk_ec_header *h) { return 2 * cbk_ec_spans(h); }
uint64_t cbk_ec_gap_words(const cbk_ec_header *h) { return (cbk_ec_spans(h) + 7) / 8; }
uint64_t cbk_ec_blocks(const cbk_ec_header *h) {
    return (cbk_ec_spans(h) + CBK_EC_BLOCK_SPANS - 1) / CBK_EC_BLOCK_SPANS;
}
uint32_t cbk_ec_max_block_codes(const cbk_ec_header *h, const uint32_t *bases) {
    if (!h || !bases || h->n == 0) return 0;
    const uint64_t blocks = cbk_ec_blocks(h);
    uint64_t most = 0;
    for (uint64_t k = 0; k < blocks; ++k) {
        const uint64_t next = k + 1 < blocks ? bases[k + 1] : h->n;
        if (next > bases[k]) most = std::max<uint64_t>(most, next - bases[k]);
    }
    return static_cast<uint32_t>(std::min<uint64_t>(most, uint64_t(CBK_EC_BLOCK_SPANS) * CBK_EC_SPAN_BITS));
}

uint64_t cbk_ec_stored_bytes(const cbk_ec_header *h) {
    if (!h) return 0;
    return h->n + 4 * (cbk_ec_stream_words(h) + cbk_ec_gap_words(h) + cbk_ec_blocks(h)) + 2 * CBK_EC_LUT_ENTRIES + 256;
}

cbk_status cbk_ec_plan(const uint16_t *w, uint64_t n, cbk_ec_header *h) {
    if (!h || (n > 0 && !w)) return CBK_E_INVALID;
    if (n >= (uint64_t(1) << 32)) return CBK_E_UNSUPPORTED;
    uint64_t freq[256] = {0};
    for (uint64_t i = 0; i < n; ++i) ++freq[(w[i] >> 7) & 0xFF];
    h->n = n;
    capped_lengths(freq, h->lengths);
    uint64_t bits = 0;
    for (int s = 0; s < 256; ++s) bits += freq[s] * h->lengths[s];
    h->total_bits = bits;
    return CBK_OK;
}

cbk_status cbk_ec_encode(const uint16_t *w, const cbk_ec_header *h, uint8_t *sm, uint32_t *stream,
                         uint32_t *gaps, uint32_t *bases, uint16_t *lut) {
    if (!h || !lut) return CBK_E_INVALID;
    const uint64_t n = h->n, spans = cbk_ec_spans(h), blocks = cbk_ec_blocks(h);
    if (n >= (uint64_t(1) << 32)) return CBK_E_UNSUPPORTED;
    if (n > 0 && (!w || !sm || !stream || !gaps || !bases)) return CBK_E_INVALID;
    uint32_t rev[256];
    if (!reversed_codes(h->lengths, rev)) return CBK_E_INVALID;
    uint64_t bits = 0;
    for (uint64_t i = 0; i < n; ++i) {
        const uint32_t l = h->lengths[(w[i] >> 7) & 0xFF];
        if (!l) return CBK_E_INVALID;
        bits += l;
    }
    if (bits != h->total_bits) return CBK_E_INVALID;

    // decode table: every 12-bit window that begins with a code maps to that code
    for (int v = 0; v < CBK_EC_LUT_ENTRIES; ++v) lut[v] = static_cast<uint16_t>(kMaxLen << 8);
    for (int s = 0; s < 256; ++s) {
        const int l = h->lengths[s];
        if (!l) continue;
        for (int hi = 0; hi < (1 << (kMaxLen - l)); ++hi)
            lut[rev[s] | (static_cast<uint32_t>(hi) << l)] = static_cast<uint16_t>(s | (l << 8));
    }
    if (n == 0) return CBK_OK;

    memset(stream, 0, cbk_ec_stream_words(h) * 4);
    memset(gaps, 0, cbk_ec_gap_words(h) * 4);
    uint64_t acc = 0, pos = 0, wi = 0, next_span = 0, next_block = 0;
    uint32_t nacc = 0;
    for (uint64_t i = 0; i < n; ++i) {
        const uint32_t e = (w[i] >> 7) & 0xFF;
        sm[i] = static_cast<uint8_t>(((w[i] >> 8) & 0x80) | (w[i] & 0x7F));
        // spans and blocks whose first code is this one
        while (next_span < spans && next_span * CBK_EC_SPAN_BITS <= pos) {
            const uint64_t gap = pos - next_span * CBK_EC_SPAN_BITS;
            gaps[next_span / 8] |= static_cast<uint32_t>(gap) << (4 * (next_span % 8));
            ++next_span;
        }
        while (next_block < blocks && next_block * CBK_EC_SPAN_BITS * CBK_EC_BLOCK_SPANS <= pos)
            bases[next_block++] = static_cast<uint32_t>(i);
        const uint32_t l = h->lengths[e];
        acc |= static_cast<uint64_t>(rev[e]) << nacc;
        nacc += l;
        pos += l;
        if (nacc >= 32) {
            stream[wi++] = static_cast<uint32_t>(acc);
            acc >>= 32;
            nacc -= 32;
        }
    }
    if (nacc) stream[wi] = static_cast<uint32_t>(acc);
    // a last span in which no code starts: its gap points at the stream end
    for (; next_span < spans; ++next_span)
        gaps[next_span / 8] |= static_cast<uint32_t>(pos - next_span * CBK_EC_SPAN_BITS) << (4 * (next_span % 8));
    for (; next_block < blocks; ++next_block) bases[next_block] = static_cast<uint32_t>(n);
    return CBK_OK;
}

// Validation shared by the GPU calls of a tensor with n > 0 weights (stream, gaps, bases, table and
// sign-mantissa bytes present, aligned and consistent with n).
static cbk_status check_ec_arrays(const cbk_ec_tensor *t) {
    const uint64_t n = t->n;
    if (!t->sm || !t->stream || !t->gaps || !t->bases || !t->lut) return CBK_E_INVALID;
    if (t->max_block_codes > uint32_t(CBK_EC_BLOCK_SPANS) * CBK_EC_SPAN_BITS) return CBK_E_INVALID;
    if (t->total_bits < n || t->total_bits > uint64_t(CBK_EC_MAX_LEN) * n) return CBK_E_INVALID;
    if (!aligned16(t->sm) || !aligned16(t->stream) || !aligned16(t->gaps) || !aligned16(t->bases) ||
        !aligned16(t->lut))
        return CBK_E_ALIGN;
    return CBK_OK;
}

// The single call's checks for one tensor of a decode; ok: launch it (n > 0).
static cbk_status check_decode(const cbk_ec_tensor *t, const uint8_t *index, bool indexed, const uint16_t *out) {
    if (!t) return CBK_E_INVALID;
    const uint64_t n = t->n;
    if (n >= (uint64_t(1) << 32)) return CBK_E_UNSUPPORTED;
    if (n == 0) return CBK_OK;
    if (!out || (indexed && !index)) return CBK_E_INVALID;
    const cbk_status st = check_ec_arrays(t);
    if (st != CBK_OK) return st;
    if (!aligned16(out) || (indexed && !aligned16(index))) return CBK_E_ALIGN;
    return CBK_OK;
}

// The single call's checks for one tensor of a fused GEMV.
static cbk_status check_gemv(const cbk_ec_tensor *t, const uint8_t *index, bool indexed, uint64_t rows, uint64_t cols,
                             const uint16_t *x, const float *y) {
    if (!t) return CBK_E_INVALID;
    const uint64_t n = t->n;
    if (n >= (uint64_t(1) << 32)) return CBK_E_UNSUPPORTED;
    if (cols != 0 && rows > (uint64_t(1) << 32) / cols) return CBK_E_INVALID;
    if (rows * cols != n) return CBK_E_INVALID;
    if (rows == 0) return CBK_OK;
    if (!y || (cols > 0 && !x)) return CBK_E_INVALID;  // cols == 0: y is zero-filled, x unread
    if ((reinterpret_cast<uintptr_t>(y) & 3u) != 0) return CBK_E_ALIGN;
    if (n > 0) {
        if (cols % 8 != 0 || cols < 64) return CBK_E_UNSUPPORTED;
        if (indexed && !index) return CBK_E_INVALID;
        const cbk_status st = check_ec_arrays(t);
        if (st != CBK_OK) return st;
        if (!aligned16(x) || (indexed && !aligned16(index))) return CBK_E_ALIGN;
    }
    return CBK_OK;
}

static cbk_status ec_decode(const cbk_ec_tensor *t, const uint8_t *index, bool indexed, uint16_t *out,
                            void *stream) {
    const cbk_status st = check_decode(t, index, indexed, out);
    if (st != CBK_OK || t->n == 0) return st;
    return cbk::launch_ec_decode(t, indexed ? &index : nullptr, 1, &out, static_cast<hipStream_t>(stream));
}

static cbk_status ec_gemv(const cbk_ec_tensor *t, const uint8_t *index, bool indexed, uint64_t rows, uint64_t cols,
                          const uint16_t *x, float *y, void *stream) {
    const cbk_status st = check_gemv(t, index, indexed, rows, cols, x, y);
    if (st != CBK_OK || rows == 0) return st;
    return cbk::launch_ec_gemv(t, indexed ? &index : nullptr, 1, &rows, cols, x, &y, static_cast<hipStream_t>(stream));
}

cbk_status cbk_ec_decode_bf16(const cbk_ec_tensor *t, uint16_t *out, void *stream) {
    return ec_decode(t, nullptr, false, out, stream);
}

cbk_status cbk_ec_decode_bf16_indexed(const cbk_ec_tensor *t, const uint8_t *index, uint16_t *out, void *stream) {
    return ec_decode(t, index, true, out, stream);
}

cbk_status cbk_ec_gemv(const cbk_ec_tensor *t, uint64_t rows, uint64_t cols, const uint16_t *x, float *y,
                       void *stream) {
    return ec_gemv(t, nullptr, false, rows, cols, x, y, stream);
}

cbk_status cbk_ec_gemv_indexed(const cbk_ec_tensor *t, const uint8_t *index, uint64_t rows, uint64_t cols,
                               const uint16_t *x, float *y, void *stream) {
    return ec_gemv(t, index, true, rows, cols, x, y, stream);
}

cbk_status cbk_ec_decode_group(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                               uint16_t *const *outs, void *stream) {
    if (count == 0) return CBK_OK;
    if (!ts || !outs) return CBK_E_INVALID;
    for (uint32_t i = 0; i < count; ++i) {
        const cbk_status st = check_decode(&ts[i], indexes ? indexes[i] : nullptr, indexes != nullptr, outs[i]);
        if (st != CBK_OK) return st;
    }
    return cbk::launch_ec_decode(ts, indexes, count, outs, static_cast<hipStream_t>(stream));
}

cbk_status cbk_ec_gemv_group(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                             const uint64_t *rows, uint64_t cols, const uint16_t *x, float *const *ys, void *stream) {
    if (count == 0) return CBK_OK;
    if (!ts || !rows || !ys) return CBK_E_INVALID;
    for (uint32_t i = 0; i < count; ++i) {
        const cbk_status st =
            check_gemv(&ts[i], indexes ? indexes[i] : nullptr, indexes != nullptr, rows[i], cols, x, ys[i]);
        if (st != CBK_OK) return st;
    }
    return cbk::launch_ec_gemv(ts, indexes, count, rows, cols, x, ys, static_cast<hipStream_t>(stream));
}

uint64_t cbk_ec_index_bytes(uint64_t total_bits) {
    const uint64_t spans = (total_bits + CBK_EC_SPAN_BITS - 1) / CBK_EC_SPAN_BITS;
    return (spans + 15) / 16 * 16;
}

cbk_status cbk_ec_build_index(const cbk_ec_tensor *t, uint8_t *index, void *stream) {
    if (!t) return CBK_E_INVALID;
    const uint64_t n = t->n;
    if (n >= (uint64_t(1) << 32)) return CBK_E_UNSUPPORTED;
    if (n == 0) return CBK_OK;
    if (!index) return CBK_E_INVALID;
    const cbk_status st = check_ec_arrays(t);
    if (st != CBK_OK) return st;
    if (!aligned16(index)) return CBK_E_ALIGN;
    return cbk::launch_ec_index(t, index, static_cast<hipStream_t>(stream));
}

}  // extern "C"
