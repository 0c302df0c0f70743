// Host half of libcbk: size helpers, the encoder, and argument validation in front of the HIP
// launchers.  Nothing here touches the GPU until every argument has been checked.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <thread>
#include <vector>

#include "cbk_internal.h"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Presence of every 16-bit pattern in w[begin, end).
void mark_present(const uint16_t *w, uint64_t begin, uint64_t end, uint8_t *seen) {
    for (uint64_t i = begin; i < end; ++i) seen[w[i]] = 1;
}

// Pack fields [f0, f1) (f0 a multiple of 32, so it starts on word f0*b/32) into words.
void pack_range(const uint16_t *w, uint64_t f0, uint64_t f1, const uint16_t *index_of, uint32_t b,
                uint32_t *words) {
    uint64_t acc = 0;
    uint32_t nbits = 0;
    uint32_t *dst = words + (f0 * b) / 32;
    for (uint64_t i = f0; i < f1; ++i) {
        acc |= static_cast<uint64_t>(index_of[w[i]]) << nbits;
        nbits += b;
        if (nbits >= 32) {
            *dst++ = static_cast<uint32_t>(acc);
            acc >>= 32;
            nbits -= 32;
        }
    }
    if (nbits) *dst = static_cast<uint32_t>(acc);
}

unsigned worker_count(uint64_t n) {
    if (n < (uint64_t(1) << 22)) return 1;
    unsigned hw = std::thread::hardware_concurrency();
    return std::max(1u, std::min(hw ? hw : 1u, 16u));
}

cbk_status check_tensor(const cbk_tensor *t) {
    if (!t) return CBK_E_INVALID;
    if (t->rows && t->cols > UINT64_MAX / t->rows) return CBK_E_INVALID;
    const uint64_t n = t->rows * t->cols;
    if (t->U > 65536u) return CBK_E_INVALID;
    if (t->b != cbk_bits_for(t->U)) return CBK_E_INVALID;
    if (n > 0 && t->U == 0) return CBK_E_INVALID;
    if (t->U > 0 && !t->codebook) return CBK_E_INVALID;
    if (n > 0 && t->b > 0 && !t->words) return CBK_E_INVALID;
    if (t->words && !aligned(t->words, 16)) return CBK_E_ALIGN;
    if (t->codebook && !aligned(t->codebook, 2)) return CBK_E_ALIGN;
    // Field offsets are computed in 64-bit; the kernels index 16-byte chunks in 32-bit.
    if (n > (uint64_t(1) << 36)) return CBK_E_UNSUPPORTED;
    if (t->rows > 0xFFFFFFFFull || t->cols > 0xFFFFFFFFull) return CBK_E_UNSUPPORTED;
    return CBK_OK;
}

}  // namespace

extern "C" {

uint32_t cbk_bits_for(uint32_t U) {
    uint32_t b = 0;
    while ((uint64_t(1) << b) < U) ++b;
    return b;
}

uint64_t cbk_words_for(uint64_t n, uint32_t b) {
    const uint64_t words = (n * b + 31) / 32;
    return (words + 3) & ~uint64_t(3);
}

uint64_t cbk_compressed_bytes(uint64_t n, uint32_t U) {
    return 2ull * U + (n * cbk_bits_for(U) + 7) / 8;
}

const char *cbk_status_str(int status) {
    switch (status) {
        case CBK_OK: return "ok";
        case CBK_E_INVALID: return "invalid argument";
        case CBK_E_CAPACITY: return "output buffer too small";
        case CBK_E_ALIGN: return "misaligned pointer or leading dimension";
        case CBK_E_UNSUPPORTED: return "unsupported shape";
        case CBK_E_HIP: return "HIP runtime error";
        case CBK_E_TIMEOUT: return "a chained launch gave up waiting";
        default: return "unknown status";
    }
}

cbk_status cbk_encode(const uint16_t *w, uint64_t n, uint16_t *codebook, uint32_t *U_out,
                      uint32_t *b_out, uint32_t *words, uint64_t words_cap, uint64_t *words_needed) {
    if ((n > 0 && !w) || !codebook || !U_out || !b_out) return CBK_E_INVALID;
    if (n > (uint64_t(1) << 40)) return CBK_E_UNSUPPORTED;

    // 1. which of the 65,536 patterns occur (threads mark private tables, then merge)
    const unsigned nt = worker_count(n);
    std::vector<std::vector<uint8_t>> seen(nt, std::vector<uint8_t>(65536, 0));
    if (nt == 1) {
        mark_present(w, 0, n, seen[0].data());
    } else {
        std::vector<std::thread> pool;
        for (unsigned k = 0; k < nt; ++k)
            pool.emplace_back(mark_present, w, n * k / nt, n * (k + 1) / nt, seen[k].data());
        for (auto &th : pool) th.join();
        for (unsigned k = 1; k < nt; ++k)
            for (uint32_t v = 0; v < 65536; ++v) seen[0][v] |= seen[k][v];
    }
    // 2. ascending scan gives the sorted codebook and every pattern's index
    std::vector<uint16_t> index_of(65536, 0);
    uint32_t U = 0;
    for (uint32_t v = 0; v < 65536; ++v) {
        if (seen[0][v]) {
            index_of[v] = static_cast<uint16_t>(U);
            codebook[U++] = static_cast<uint16_t>(v);
        }
    }
    const uint32_t b = cbk_bits_for(U);
    const uint64_t need = cbk_words_for(n, b);
    *U_out = U;
    *b_out = b;
    if (words_needed) *words_needed = need;
    if (need > words_cap || (need > 0 && !words)) return CBK_E_CAPACITY;
    if (need == 0) return CBK_OK;
    memset(words, 0, need * sizeof(uint32_t));
    if (b == 0) return CBK_OK;

    // 3. pack, LSB first; chunks start on multiples of 32 fields so they own whole words
    if (nt == 1) {
        pack_range(w, 0, n, index_of.data(), b, words);
    } else {
        const uint64_t groups = (n + 31) / 32;
        std::vector<std::thread> pool;
        for (unsigned k = 0; k < nt; ++k) {
            const uint64_t f0 = std::min(n, 32 * (groups * k / nt));
            const uint64_t f1 = std::min(n, 32 * (groups * (k + 1) / nt));
            if (f1 > f0) pool.emplace_back(pack_range, w, f0, f1, index_of.data(), b, words);
        }
        for (auto &th : pool) th.join();
    }
    return CBK_OK;
}

cbk_status cbk_cap_patterns(const uint16_t *w, uint64_t n, uint32_t K, uint16_t *w_out, uint32_t *U_out) {
    if ((n > 0 && (!w || !w_out)) || !U_out || K == 0) return CBK_E_INVALID;
    if (n > (uint64_t(1) << 40)) return CBK_E_UNSUPPORTED;
    std::vector<uint64_t> count(65536, 0);
    for (uint64_t i = 0; i < n; ++i) ++count[w[i]];
    uint32_t U = 0, specials = 0;
    for (uint32_t v = 0; v < 65536; ++v) {
        if (!count[v]) continue;
        ++U;
        if (((v >> 7) & 0xFF) == 0xFF) ++specials;
    }
    if (U <= K) {
        if (w_out != w && n > 0) memcpy(w_out, w, n * sizeof(uint16_t));
        *U_out = U;
        return CBK_OK;
    }
    if (specials > K || (specials == K && U > specials)) return CBK_E_UNSUPPORTED;
    // keep every Inf/NaN pattern, then the most frequent finite ones (ties: smaller pattern)
    std::vector<uint8_t> kept(65536, 0);
    std::vector<uint32_t> finite;
    for (uint32_t v = 0; v < 65536; ++v) {
        if (!count[v]) continue;
        if (((v >> 7) & 0xFF) == 0xFF)
            kept[v] = 1;
        else
            finite.push_back(v);
    }
    const size_t room = K - specials;
    std::partial_sort(finite.begin(), finite.begin() + room, finite.end(), [&](uint32_t a, uint32_t b) {
        return count[a] != count[b] ? count[a] > count[b] : a < b;
    });
    auto value = [](uint32_t p) {
        uint32_t bits = p << 16;
        float f;
        memcpy(&f, &bits, 4);
        return static_cast<double>(f);
    };
    std::vector<uint32_t> near(finite.begin(), finite.begin() + room);
    for (uint32_t v : near) kept[v] = 1;
    std::sort(near.begin(), near.end(), [&](uint32_t a, uint32_t b) {
        return value(a) != value(b) ? value(a) < value(b) : a < b;
    });
    // every other pattern goes to the nearest kept finite value (ties: closer to zero, then the
    // smaller pattern); the candidates are the neighbours of its place in value order
    std::vector<uint16_t> map(65536, 0);
    for (uint32_t v = 0; v < 65536; ++v) {
        if (!count[v]) continue;
        if (kept[v]) {
            map[v] = static_cast<uint16_t>(v);
            continue;
        }
        const double f = value(v);
        const size_t i = std::lower_bound(near.begin(), near.end(), f,
                                          [&](uint32_t r, double x) { return value(r) < x; }) - near.begin();
        uint32_t best = 0;
        bool have = false;
        for (size_t j = (i >= 2 ? i - 2 : 0); j < std::min(near.size(), i + 2); ++j) {
            const uint32_t r = near[j];
            if (!have) {
                best = r;
                have = true;
                continue;
            }
            const double dr = std::fabs(f - value(r)), db = std::fabs(f - value(best));
            const double ar = std::fabs(value(r)), ab = std::fabs(value(best));
            if (dr < db || (dr == db && (ar < ab || (ar == ab && r < best)))) best = r;
        }
        map[v] = static_cast<uint16_t>(best);
    }
    for (uint64_t i = 0; i < n; ++i) w_out[i] = map[w[i]];
    *U_out = K;
    return CBK_OK;
}

size_t cbk_encode_gpu_workspace_bytes(void) { return cbk::encode_gpu_workspace_bytes(); }

// The checks of one GPU encode job (the workspace is checked by the caller).
static cbk_status check_encode_job(const cbk_encode_job &j) {
    if (!j.codebook || !j.meta || (j.n > 0 && (!j.w || !j.words))) return CBK_E_INVALID;
    if (j.n >= (uint64_t(1) << 40)) return CBK_E_UNSUPPORTED;
    if (!aligned(j.codebook, 2) || !aligned(j.meta, 4) || (j.n > 0 && (!aligned(j.w, 16) || !aligned(j.words, 16))))
        return CBK_E_ALIGN;
    if (j.words_cap < cbk_words_for(j.n, 16)) return CBK_E_CAPACITY;
    return CBK_OK;
}

cbk_status cbk_encode_gpu(const uint16_t *w, uint64_t n, void *workspace, uint16_t *codebook, uint32_t *words,
                          uint64_t words_cap, uint32_t *meta, void *stream) {
    if (!workspace) return CBK_E_INVALID;
    const cbk_encode_job job{w, n, codebook, words, words_cap, meta};
    cbk_status st = check_encode_job(job);
    if (st != CBK_OK) return st;
    if (!aligned(workspace, 16)) return CBK_E_ALIGN;
    return cbk::launch_encode_gpu(&job, 1, workspace, static_cast<hipStream_t>(stream));
}

cbk_status cbk_encode_gpu_group(const cbk_encode_job *jobs, uint32_t count, void *workspace, void *stream) {
    if (count == 0) return CBK_OK;
    if (!jobs || !workspace) return CBK_E_INVALID;
    for (uint32_t i = 0; i < count; ++i) {
        const cbk_status st = check_encode_job(jobs[i]);
        if (st != CBK_OK) return st;
    }
    if (!aligned(workspace, 16)) return CBK_E_ALIGN;
    return cbk::launch_encode_gpu(jobs, count, workspace, static_cast<hipStream_t>(stream));
}

cbk_status cbk_encode_gpu_noalloc(const uint16_t *w, uint64_t n, uint16_t *codebook, uint32_t *words,
                                  uint64_t words_cap, uint32_t *meta, void *stream) {
    const cbk_encode_job job{w, n, codebook, words, words_cap, meta};
    cbk_status st = check_encode_job(job);
    if (st != CBK_OK) return st;
    void *ws = nullptr;
    st = cbk::encode_gpu_scratch(&ws);
    if (st != CBK_OK) return st;
    return cbk::launch_encode_gpu(&job, 1, ws, static_cast<hipStream_t>(stream));
}

// The checks of one decode (n == 0 passes: nothing to do).
static cbk_status check_decode(const cbk_tensor *t, const uint16_t *out) {
    cbk_status st = check_tensor(t);
    if (st != CBK_OK) return st;
    if (t->rows * t->cols == 0) return CBK_OK;
    if (!out) return CBK_E_INVALID;
    if (!aligned(out, 2)) return CBK_E_ALIGN;
    return CBK_OK;
}

cbk_status cbk_decode_bf16(const cbk_tensor *t, uint16_t *out, void *stream) {
    const cbk_status st = check_decode(t, out);
    if (st != CBK_OK || t->rows * t->cols == 0) return st;
    return cbk::launch_decode(*t, out, static_cast<hipStream_t>(stream));
}

cbk_status cbk_decode_group(const cbk_tensor *ts, uint32_t count, uint16_t *const *outs, void *stream) {
    if (count == 0) return CBK_OK;
    if (!ts || !outs) return CBK_E_INVALID;
    for (uint32_t i = 0; i < count; ++i) {
        const cbk_status st = check_decode(&ts[i], outs[i]);
        if (st != CBK_OK) return st;
    }
    return cbk::launch_decode_group(ts, count, outs, static_cast<hipStream_t>(stream));
}

cbk_status cbk_gemv(const cbk_tensor *t, const uint16_t *x, float *y, void *stream) {
    cbk_status st = check_tensor(t);
    if (st != CBK_OK) return st;
    if (t->rows == 0) return CBK_OK;
    if (!y || (t->cols > 0 && !x)) return CBK_E_INVALID;
    if (!aligned(y, 4) || (x && !aligned(x, 2))) return CBK_E_ALIGN;
    return cbk::launch_gemv(*t, x, y, static_cast<hipStream_t>(stream));
}

cbk_status cbk_gemv_group(const cbk_tensor *ts, uint32_t count, const uint16_t *x, float *const *ys,
                          void *stream) {
    if (count == 0) return CBK_OK;
    if (!ts || !ys || count > 4096) return CBK_E_INVALID;
    const uint64_t K = ts[0].cols;
    for (uint32_t i = 0; i < count; ++i) {
        cbk_status st = check_tensor(&ts[i]);
        if (st != CBK_OK) return st;
        if (ts[i].cols != K) return CBK_E_INVALID;
        if (ts[i].rows > 0 && !ys[i]) return CBK_E_INVALID;
        if (ys[i] && !aligned(ys[i], 4)) return CBK_E_ALIGN;
    }
    if (K > 0 && !x) return CBK_E_INVALID;
    if (x && !aligned(x, 2)) return CBK_E_ALIGN;
    return cbk::launch_gemv_group(ts, count, x, ys, static_cast<hipStream_t>(stream));
}

size_t cbk_gemv_chain_bytes(uint32_t phases) { return cbk::gemv_chain_bytes(phases); }

cbk_status cbk_gemv_chain_init(const cbk_gemv_phase *phases, uint32_t count, void *buffer, size_t bytes,
                               cbk_gemv_chain *chain) {
    if (!phases || !buffer || !chain || count == 0 || count > 65536) return CBK_E_INVALID;
    uint32_t b = 0;
    for (uint32_t p = 0; p < count; ++p) {
        const cbk_gemv_phase &ph = phases[p];
        if (!ph.ts || !ph.ys || !ph.x || ph.count == 0 || ph.count > 8) return CBK_E_INVALID;
        const uint64_t K = ph.ts[0].cols;
        for (uint32_t i = 0; i < ph.count; ++i) {
            const cbk_status st = check_tensor(&ph.ts[i]);
            if (st != CBK_OK) return st;
            if (ph.ts[i].cols != K || ph.ts[i].rows == 0 || !ph.ys[i]) return CBK_E_INVALID;
            if (!aligned(ph.ys[i], 4)) return CBK_E_ALIGN;
        }
        if (p == 0) b = ph.ts[0].b;
        for (uint32_t i = 0; i < ph.count; ++i) {
            if (ph.ts[i].b != b || b < 1 || b > 15) return CBK_E_UNSUPPORTED;
            if (!aligned(ph.ts[i].codebook, 16)) return CBK_E_ALIGN;
            if (ph.ts[i].rows * (K / 64) >= (uint64_t(1) << 32)) return CBK_E_UNSUPPORTED;
        }
        if (K == 0 || K % 64 != 0 || K > 32768) return CBK_E_UNSUPPORTED;
        if (!aligned(ph.x, 16)) return CBK_E_ALIGN;
    }
    if (!aligned(buffer, 256)) return CBK_E_ALIGN;
    if (bytes < cbk::gemv_chain_bytes(count)) return CBK_E_CAPACITY;
    return cbk::build_gemv_chain(phases, count, buffer, chain);
}

cbk_status cbk_gemv_chain_run(const cbk_gemv_chain *chain, uint32_t timeout_us, void *stream) {
    if (!chain || !chain->buffer || chain->phases == 0) return CBK_E_INVALID;
    return cbk::launch_gemv_chain(*chain, timeout_us, static_cast<hipStream_t>(stream));
}

cbk_status cbk_gemv_chain_check(const cbk_gemv_chain *chain) {
    if (!chain || !chain->buffer) return CBK_E_INVALID;
    return cbk::gemv_chain_check(*chain);
}

cbk_status cbk_gemm_small(const cbk_tensor *t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                          float *Y, uint64_t ldy, void *stream) {
    cbk_status st = check_tensor(t);
    if (st != CBK_OK) return st;
    if (batch < 1 || batch > 16) return CBK_E_INVALID;
    if (t->rows == 0) return CBK_OK;
    if (!Y || (t->cols > 0 && !X)) return CBK_E_INVALID;
    if (ldx < t->cols || ldy < t->rows) return CBK_E_INVALID;
    if (!aligned(Y, 4) || (X && !aligned(X, 2))) return CBK_E_ALIGN;
    if (ldx > 0xFFFFFFFFull || ldy > 0xFFFFFFFFull) return CBK_E_UNSUPPORTED;
    return cbk::launch_gemm(*t, X, ldx, batch, Y, ldy, static_cast<hipStream_t>(stream));
}

cbk_status cbk_gemm_group(const cbk_tensor *ts, uint32_t count, const uint16_t *X, uint64_t ldx,
                          uint32_t batch, float *const *Ys, const uint64_t *ldys, void *stream) {
    if (count == 0) return CBK_OK;
    if (!ts || !Ys || !ldys || count > 4096) return CBK_E_INVALID;
    if (batch < 1 || batch > 16) return CBK_E_INVALID;
    const uint64_t K = ts[0].cols;
    for (uint32_t i = 0; i < count; ++i) {
        cbk_status st = check_tensor(&ts[i]);
        if (st != CBK_OK) return st;
        if (ts[i].cols != K) return CBK_E_INVALID;
        if (ts[i].rows > 0 && (!Ys[i] || ldys[i] < ts[i].rows)) return CBK_E_INVALID;
        if (Ys[i] && !aligned(Ys[i], 4)) return CBK_E_ALIGN;
        if (ldys[i] > 0xFFFFFFFFull) return CBK_E_UNSUPPORTED;
    }
    if (K > 0 && !X) return CBK_E_INVALID;
    if (ldx < K) return CBK_E_INVALID;
    if (X && !aligned(X, 2)) return CBK_E_ALIGN;
    if (ldx > 0xFFFFFFFFull) return CBK_E_UNSUPPORTED;
    return cbk::launch_gemm_group(ts, count, X, ldx, batch, Ys, ldys, static_cast<hipStream_t>(stream));
}

}  // extern "C"
