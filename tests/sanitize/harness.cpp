// Host-only driver for the sanitizer runs of tests/test_sanitize.py.  Reads tensors written by the
// test (seeded synthetic inputs from synth/) and, for each, runs the library's host code next to the
// C oracle: cbk_encode (size query, then the encode) against oracle_encode byte for byte, the
// oracle's decode back to the input, cbk_cap_patterns, the entropy-coded plan and encode into
// buffers of exactly the announced sizes, and the GPU entry points' argument checks, which must
// return before any launch.  Exits non-zero on the first mismatch; the sanitizers abort on any
// memory or undefined-behaviour error.
//
// Input file: records of {uint64 n, uint32 K, uint32 pad, n x uint16 patterns}.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "cbk.h"
#include "cbk_ec.h"

extern "C" {
uint64_t oracle_stream_words(uint64_t n, uint32_t b);
int oracle_encode(const uint16_t *w, uint64_t n, uint16_t *codebook, uint32_t *U_out, uint32_t *b_out,
                  uint32_t *words, uint64_t words_cap);
void oracle_decode_range(const uint16_t *codebook, uint32_t U, uint32_t b, const uint32_t *words, uint64_t i0,
                         uint64_t i1, uint16_t *out);
}

static int fail(const char *what, uint64_t rec) {
    fprintf(stderr, "record %llu: %s\n", (unsigned long long)rec, what);
    return 1;
}

static int check_record(const std::vector<uint16_t> &w, uint32_t K, uint64_t rec) {
    const uint64_t n = w.size();
    const uint16_t *wp = n ? w.data() : nullptr;
    // library encoder: size query, then the encode into a buffer of exactly that size
    std::vector<uint16_t> cb(65536), ocb(65536);
    uint32_t U = 0, b = 0, oU = 0, ob = 0;
    uint64_t need = 0;
    if (cbk_encode(wp, n, cb.data(), &U, &b, nullptr, 0, &need) != (need ? CBK_E_CAPACITY : CBK_OK))
        return fail("size query", rec);
    std::vector<uint32_t> words(need);
    if (cbk_encode(wp, n, cb.data(), &U, &b, need ? words.data() : nullptr, need, &need) != CBK_OK)
        return fail("encode", rec);
    // oracle
    const uint64_t cap = n ? (n * 16 + 31) / 32 : 1;
    std::vector<uint32_t> owords(cap);
    if (oracle_encode(wp, n, ocb.data(), &oU, &ob, owords.data(), cap) != 0) return fail("oracle encode", rec);
    if (U != oU || b != ob) return fail("U or b differ", rec);
    if (memcmp(cb.data(), ocb.data(), U * sizeof(uint16_t))) return fail("codebook differs", rec);
    const uint64_t nw = oracle_stream_words(n, b);
    if (nw > need || (nw && memcmp(words.data(), owords.data(), nw * 4))) return fail("words differ", rec);
    for (uint64_t i = nw; i < need; ++i)
        if (words[i]) return fail("padding not zero", rec);
    std::vector<uint16_t> back(n ? n : 1);
    oracle_decode_range(cb.data(), U, b, need ? words.data() : owords.data(), 0, n, back.data());
    if (n && memcmp(back.data(), w.data(), n * 2)) return fail("round trip", rec);
    if (cbk_compressed_bytes(n, U) != 2ull * U + (n * b + 7) / 8) return fail("compressed_bytes", rec);

    // capped codebook into a separate buffer, then in place
    std::vector<uint16_t> capped(n ? n : 1), inplace(w);
    uint32_t Uc = 0, Ui = 0;
    if (K && n) {
        const int st = cbk_cap_patterns(wp, n, K, capped.data(), &Uc);
        if (st != CBK_OK && st != CBK_E_UNSUPPORTED) return fail("cap_patterns", rec);
        if (st == CBK_OK) {
            if (cbk_cap_patterns(inplace.data(), n, K, inplace.data(), &Ui) != CBK_OK) return fail("cap in place", rec);
            if (Ui != Uc || memcmp(inplace.data(), capped.data(), n * 2)) return fail("cap in place differs", rec);
            std::vector<uint8_t> seen(65536, 0);
            uint32_t distinct = 0;
            for (uint64_t i = 0; i < n; ++i)
                if (!seen[capped[i]]) {
                    seen[capped[i]] = 1;
                    ++distinct;
                }
            if (distinct != Uc || Uc > K) return fail("capped distinct count", rec);
        }
    }

    // entropy-coded format: plan, then encode into buffers of exactly the announced sizes
    if (n < (uint64_t(1) << 32)) {
        cbk_ec_header h;
        if (cbk_ec_plan(wp, n, &h) != CBK_OK) return fail("ec_plan", rec);
        std::vector<uint8_t> sm(n ? n : 1);
        std::vector<uint32_t> stream(cbk_ec_stream_words(&h) ? cbk_ec_stream_words(&h) : 1);
        std::vector<uint32_t> gaps(cbk_ec_gap_words(&h) ? cbk_ec_gap_words(&h) : 1);
        std::vector<uint32_t> bases(cbk_ec_blocks(&h) ? cbk_ec_blocks(&h) : 1);
        std::vector<uint16_t> lut(4096);
        if (cbk_ec_encode(wp, &h, sm.data(), stream.data(), gaps.data(), bases.data(), lut.data()) != CBK_OK)
            return fail("ec_encode", rec);
        if (n && cbk_ec_stored_bytes(&h) < n) return fail("ec stored bytes", rec);
        // the largest per-block code count, from bases
        uint64_t most = 0;
        for (uint64_t k = 0; n && k < cbk_ec_blocks(&h); ++k)
            most = std::max<uint64_t>(most, (k + 1 < cbk_ec_blocks(&h) ? bases[k + 1] : n) - bases[k]);
        if (cbk_ec_max_block_codes(&h, bases.data()) != most) return fail("ec max block codes", rec);
        // grouped calls with bad arguments (device addresses stand in; nothing is dereferenced)
        if (n) {
            const cbk_ec_tensor et = {n, h.total_bits, reinterpret_cast<const uint8_t *>(0x10000),
                                      reinterpret_cast<const uint32_t *>(0x20000),
                                      reinterpret_cast<const uint32_t *>(0x30000),
                                      reinterpret_cast<const uint32_t *>(0x40000),
                                      reinterpret_cast<const uint16_t *>(0x50000)};
            cbk_ec_tensor two[2] = {et, et};
            uint16_t *outs[2] = {reinterpret_cast<uint16_t *>(0x60000), nullptr};
            if (cbk_ec_decode_group(two, nullptr, 2, outs, nullptr) != CBK_E_INVALID)
                return fail("ec group decode without its second output", rec);
            outs[1] = reinterpret_cast<uint16_t *>(0x70008);
            if (cbk_ec_decode_group(two, nullptr, 2, outs, nullptr) != CBK_E_ALIGN)
                return fail("ec group decode with a misaligned output", rec);
            const uint8_t *ix[2] = {reinterpret_cast<const uint8_t *>(0x80000), nullptr};
            outs[1] = reinterpret_cast<uint16_t *>(0x70000);
            if (cbk_ec_decode_group(two, ix, 2, outs, nullptr) != CBK_E_INVALID)
                return fail("ec group decode with a missing index", rec);
            if (cbk_ec_decode_group(nullptr, nullptr, 0, nullptr, nullptr) != CBK_OK)
                return fail("ec group decode of no tensors", rec);
            // an empty first tensor, then one whose rows do not match its n
            two[0].n = 0;
            two[0].total_bits = 0;
            const uint64_t rows[2] = {0, n + 1};
            float *ys[2] = {reinterpret_cast<float *>(0x90000), reinterpret_cast<float *>(0xA0000)};
            if (cbk_ec_gemv_group(two, nullptr, 2, rows, 1, reinterpret_cast<const uint16_t *>(0xB0000), ys,
                                  nullptr) != CBK_E_INVALID)
                return fail("ec group gemv with rows * cols != n", rec);
        }
    }

    // GPU entry points with bad arguments: validation returns before any launch (the launchers of
    // this build abort if reached)
    cbk_tensor t = {n ? uint64_t(1) : uint64_t(0), n, U, b, reinterpret_cast<const uint16_t *>(0x1000),
                    reinterpret_cast<const uint32_t *>(0x2000)};
    if (n && cbk_gemv(&t, reinterpret_cast<const uint16_t *>(0x3000), nullptr, nullptr) != CBK_E_INVALID)
        return fail("gemv without y", rec);
    if (n && cbk_decode_bf16(&t, nullptr, nullptr) != CBK_E_INVALID) return fail("decode without out", rec);
    if (n && cbk_gemm_small(&t, reinterpret_cast<const uint16_t *>(0x3000), n, 17, reinterpret_cast<float *>(0x4000),
                            1, nullptr) != CBK_E_INVALID)
        return fail("gemm batch 17", rec);
    t.b = b + 1;
    if (n && cbk_gemv(&t, reinterpret_cast<const uint16_t *>(0x3000), reinterpret_cast<float *>(0x4000), nullptr) !=
                 CBK_E_INVALID)
        return fail("gemv with a wrong b", rec);
    if (cbk_encode_gpu_noalloc(nullptr, n + 1, nullptr, nullptr, 0, nullptr, nullptr) != CBK_E_INVALID)
        return fail("noalloc encode without pointers", rec);
    // a GEMV chain of two phases of this tensor (a 64-column row shape when it has any): a buffer
    // one byte short, a misaligned x, then a phase with a second tensor of other cols
    if (n && b >= 1 && b <= 15) {
        t.b = b;
        cbk_tensor two[2] = {t, t};
        two[0].rows = 1;
        two[0].cols = 64;
        two[1] = two[0];
        float *ys[2] = {reinterpret_cast<float *>(0x4000), reinterpret_cast<float *>(0x5000)};
        cbk_gemv_phase ph[2] = {{two, 1, reinterpret_cast<const uint16_t *>(0x3000), ys},
                                {two, 2, reinterpret_cast<const uint16_t *>(0x3000), ys}};
        cbk_gemv_chain chain;
        void *buf = reinterpret_cast<void *>(0x100000);
        const size_t need = cbk_gemv_chain_bytes(2);
        if (U > 0 && cbk_gemv_chain_init(ph, 2, buf, need - 1, &chain) != CBK_E_CAPACITY)
            return fail("chain buffer one byte short", rec);
        ph[1].x = reinterpret_cast<const uint16_t *>(0x3008);
        if (U > 0 && cbk_gemv_chain_init(ph, 2, buf, need, &chain) != CBK_E_ALIGN) return fail("chain x misaligned", rec);
        two[1].cols = 128;
        ph[1].x = reinterpret_cast<const uint16_t *>(0x3000);
        if (U > 0 && cbk_gemv_chain_init(ph, 2, buf, need, &chain) != CBK_E_INVALID)
            return fail("chain phase with differing cols", rec);
    }
    return 0;
}

int main(int argc, char **argv) {
    if (argc != 2) return 2;
    FILE *f = fopen(argv[1], "rb");
    if (!f) return 2;
    uint64_t rec = 0;
    for (;;) {
        uint64_t n;
        uint32_t kk[2];
        if (fread(&n, 8, 1, f) != 1) break;
        if (fread(kk, 4, 2, f) != 2) return 2;
        std::vector<uint16_t> w(n);
        if (n && fread(w.data(), 2, n, f) != n) return 2;
        if (check_record(w, kk[0], rec)) return 1;
        ++rec;
    }
    fclose(f);
    printf("%llu records ok\n", (unsigned long long)rec);
    return 0;
}
