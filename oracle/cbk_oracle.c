/*
 * cbk_oracle.c -- plain, slow, obviously correct CPU reference for lossless codebook
 * compression of BF16 weights and the GEMV / skinny GEMM that consumes them.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no code, header or table with the HIP library
 * and the HIP library never calls it.
 *
 * What it follows (page = the scraped web pages on codebook lossless compression):
 *  - "Codebook Lossless Compression" overview (ai-manual.ru), section "How it works": each
 *    weight is replaced by its index in a dictionary of values, and at inference the original
 *    value is substituted back exactly ("pure pointer replacement, no approximation").
 *  - setupai.cc digest of the Codebook-Quantization proof of concept, "Key points" and the
 *    competitor table: the indices of the unique weights are bit-packed, about 12-13 bits each.
 *  - The fixed format this library implements: the codebook is the set of distinct 16-bit
 *    patterns sorted ascending as unsigned integers, b is the smallest width with 2^b >= U
 *    (b = 0 when U <= 1), and index i occupies bits [i*b, i*b + b) of a little-endian uint32
 *    stream, least significant bit first.
 *
 * Every step is written the plainest way: qsort + de-duplication for the codebook, binary
 * search for each index, one bit at a time for packing and unpacking, and float64 sums for
 * the products.  Nothing is blocked, fused or reordered.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - "distinct" means distinct bit patterns (+0 and -0 differ, every NaN payload is its own entry);
 *  - the sort order is unsigned 16-bit order;
 *  - U = 1 gives b = 0 and no stream words; n = 0 gives U = 0, b = 0;
 *  - an index >= U (a corrupt stream; the encoder never writes one) decodes to 0x7FC0.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_CORRUPT_VALUE 0x7FC0u

/* Smallest b with 2^b >= U; 0 for U <= 1. */
uint32_t oracle_bits_for(uint32_t U)
{
    uint32_t b = 0;
    while (((uint64_t)1 << b) < (uint64_t)U)
        b++;
    return b;
}

/* Number of uint32 words that hold n fields of b bits: ceil(n*b/32). */
uint64_t oracle_stream_words(uint64_t n, uint32_t b)
{
    return (n * (uint64_t)b + 31u) / 32u;
}

static int cmp_u16(const void *pa, const void *pb)
{
    uint16_t a = *(const uint16_t *)pa, b = *(const uint16_t *)pb;
    return (a > b) - (a < b);
}

/* Codebook: the distinct patterns of w, ascending as unsigned 16-bit integers.
 * codebook must hold 65536 entries.  Returns U, or -1 on allocation failure. */
int64_t oracle_codebook(const uint16_t *w, uint64_t n, uint16_t *codebook)
{
    if (n == 0)
        return 0;
    uint16_t *sorted = (uint16_t *)malloc(n * sizeof(uint16_t));
    if (!sorted)
        return -1;
    memcpy(sorted, w, n * sizeof(uint16_t));
    qsort(sorted, n, sizeof(uint16_t), cmp_u16);
    int64_t U = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (i == 0 || sorted[i] != sorted[i - 1])
            codebook[U++] = sorted[i];
    }
    free(sorted);
    return U;
}

/* Position of value v in the sorted codebook (binary search); -1 if absent. */
int64_t oracle_index_of(const uint16_t *codebook, uint32_t U, uint16_t v)
{
    int64_t lo = 0, hi = (int64_t)U - 1;
    while (lo <= hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (codebook[mid] == v)
            return mid;
        if (codebook[mid] < v)
            lo = mid + 1;
        else
            hi = mid - 1;
    }
    return -1;
}

/* Encode: codebook, U, b and the packed words.  words must hold oracle_stream_words(n, b)
 * entries (at most ceil(n*16/32)); every bit at position >= n*b is zero.
 * Returns 0 on success, -1 on failure. */
int oracle_encode(const uint16_t *w, uint64_t n, uint16_t *codebook, uint32_t *U_out,
                  uint32_t *b_out, uint32_t *words, uint64_t words_cap)
{
    int64_t U = oracle_codebook(w, n, codebook);
    if (U < 0)
        return -1;
    uint32_t b = oracle_bits_for((uint32_t)U);
    uint64_t nwords = oracle_stream_words(n, b);
    if (nwords > words_cap)
        return -1;
    for (uint64_t k = 0; k < nwords; k++)
        words[k] = 0;
    for (uint64_t i = 0; i < n; i++) {
        int64_t idx = oracle_index_of(codebook, (uint32_t)U, w[i]);
        if (idx < 0)
            return -1;
        for (uint32_t j = 0; j < b; j++) {
            if (((uint64_t)idx >> j) & 1u) {
                uint64_t p = (uint64_t)i * b + j;
                words[p >> 5] |= (uint32_t)1u << (p & 31u);
            }
        }
    }
    *U_out = (uint32_t)U;
    *b_out = b;
    return 0;
}

/* Field i of the stream, read one bit at a time, least significant bit first. */
uint32_t oracle_field(const uint32_t *words, uint32_t b, uint64_t i)
{
    uint32_t idx = 0;
    for (uint32_t j = 0; j < b; j++) {
        uint64_t p = i * b + j;
        uint32_t bit = (words[p >> 5] >> (p & 31u)) & 1u;
        idx |= bit << j;
    }
    return idx;
}

/* The 16-bit pattern of weight i: codebook[field i] (0x7FC0 for an index >= U). */
uint16_t oracle_weight(const uint16_t *codebook, uint32_t U, uint32_t b, const uint32_t *words,
                       uint64_t i)
{
    uint32_t idx = oracle_field(words, b, i);
    return idx < U ? codebook[idx] : (uint16_t)ORACLE_CORRUPT_VALUE;
}

/* Decode weights [i0, i1) into out[0 .. i1-i0). */
void oracle_decode_range(const uint16_t *codebook, uint32_t U, uint32_t b, const uint32_t *words,
                         uint64_t i0, uint64_t i1, uint16_t *out)
{
    for (uint64_t i = i0; i < i1; i++)
        out[i - i0] = oracle_weight(codebook, U, b, words, i);
}

/* The real value of a BF16 pattern: BF16 is the upper half of an IEEE binary32. */
double oracle_bf16_value(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* GEMV rows [r0, r1): y[r] = sum_k W[r][k] * x[k] and absb[r] = sum_k |W[r][k] * x[k]|, both in
 * float64, with W[r][k] decoded from the stream (row-major, cols fields per row). */
void oracle_gemv_rows(const uint16_t *codebook, uint32_t U, uint32_t b, const uint32_t *words,
                      uint64_t cols, const uint16_t *x, uint64_t r0, uint64_t r1, double *y,
                      double *absb)
{
    for (uint64_t r = r0; r < r1; r++) {
        double s = 0.0, a = 0.0;
        for (uint64_t k = 0; k < cols; k++) {
            double wv = oracle_bf16_value(oracle_weight(codebook, U, b, words, r * cols + k));
            double p = wv * oracle_bf16_value(x[k]);
            s += p;
            a += p < 0 ? -p : p;
        }
        y[r] = s;
        if (absb)
            absb[r] = a;
    }
}

/* Skinny GEMM rows [r0, r1): Y[j][r] = sum_k W[r][k] * X[j][k] for j < batch, float64.
 * X is [batch][ldx], Y and absb are [batch][ldy]. */
void oracle_gemm_rows(const uint16_t *codebook, uint32_t U, uint32_t b, const uint32_t *words,
                      uint64_t cols, const uint16_t *X, uint64_t ldx, uint32_t batch, uint64_t r0,
                      uint64_t r1, double *Y, double *absb, uint64_t ldy)
{
    for (uint32_t j = 0; j < batch; j++)
        oracle_gemv_rows(codebook, U, b, words, cols, X + (uint64_t)j * ldx, r0, r1,
                         Y + (uint64_t)j * ldy, absb ? absb + (uint64_t)j * ldy : NULL);
}
