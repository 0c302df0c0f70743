/*
 * cbk_ec.h -- C ABI of libcbk's exponent entropy-coded BF16 format: the sign and the 7 mantissa
 * bits of every weight stay as they are (one byte), and only the 8 exponent bits are replaced by
 * a prefix (Huffman) code, decoded on an MI355X (gfx950) GPU back to the exact BF16 patterns.
 *
 * The method (DFloat11 article on gadzety360.pl, sections "Przełom: DFloat11" and "Jak to działa
 * w praktyce?"): of the 16 bits of a BF16 weight, the sign and mantissa carry nearly their full
 * information but the exponent only about 2.6 bits, so an entropy code on the exponent alone
 * gives a lossless format of about 11 bits per weight; the GPU decoder keeps small lookup tables
 * in on-chip memory, and its threads first find how many values they will decode, synchronise,
 * then write the values to their places.  The format fixed here:
 *
 *   sm        n bytes, sm[i] = sign << 7 | mantissa of weight i;
 *   code      for every exponent value present, a length in 1..12: an optimal prefix code
 *             among those with lengths <= 12 (a tensor with one exponent value gets length 1);
 *             codes are canonical: ordered by (length, exponent value), each the previous plus
 *             one, shifted left where the length grows;
 *   stream    the exponents' codes in weight order, first code bit first, packed into a
 *             little-endian uint32 stream read least significant bit first; total_bits long,
 *             padded with zero bits to whole 64-bit spans (2 words per span);
 *   gaps      per span j, 4 bits (eight per uint32, span j at bits 4*(j%8) of word j/8): the
 *             offset within the span of the first code that starts in it (the stream end if none
 *             does), so every span decodes on its own;
 *   bases     per block of 256 spans, the index of the first weight whose code starts in it;
 *   lut       4096 uint16: entry v = exponent | length << 8 of the code that the 12 stream bits
 *             v (first bit = bit 0) begin with; entries no code reaches hold 12 << 8.
 *
 * Conventions as in cbk.h: status codes, host-side validation before any HIP call, device
 * pointers in a host struct, caller-owned buffers, no allocation, asynchronous on `stream`.
 */
#ifndef CBK_EC_H
#define CBK_EC_H

#include <stddef.h>
#include <stdint.h>

#include "cbk.h"

#ifdef __cplusplus
extern "C" {
#endif

#define CBK_EC_MAX_LEN 12
#define CBK_EC_SPAN_BITS 64
#define CBK_EC_BLOCK_SPANS 256
#define CBK_EC_LUT_ENTRIES 4096

/* What the host encoder's first pass decides; fixes every array size. */
typedef struct {
    uint64_t n;            /* weights, < 2^32                                          */
    uint64_t total_bits;   /* length of the exponent code stream in bits              */
    uint8_t lengths[256];  /* code length of each exponent value; 0 = value absent    */
} cbk_ec_header;

/* Sizes that follow from a header: spans = ceil(total_bits / 64); stream words = 2 * spans;
 * gap words = ceil(spans / 8); blocks = ceil(spans / 256).  Stored bytes (the accounting size):
 * n + 4 * (stream words + gap words + blocks) + 2 * 4096 + 256. */
uint64_t cbk_ec_spans(const cbk_ec_header *h);
uint64_t cbk_ec_stream_words(const cbk_ec_header *h);
uint64_t cbk_ec_gap_words(const cbk_ec_header *h);
uint64_t cbk_ec_blocks(const cbk_ec_header *h);
uint64_t cbk_ec_stored_bytes(const cbk_ec_header *h);

/*
 * cbk_ec_plan -- host, synchronous.  First pass over n patterns w: exponent counts, the capped
 * optimal code lengths and the stream length, into *h.
 * Errors: CBK_E_INVALID (NULL h, or NULL w with n > 0), CBK_E_UNSUPPORTED (n >= 2^32).
 */
cbk_status cbk_ec_plan(const uint16_t *w, uint64_t n, cbk_ec_header *h);

/*
 * cbk_ec_encode -- host, synchronous.  Second pass: writes the arrays for the header that
 * cbk_ec_plan produced on the same w (sizes as above; lut has 4096 entries).  Arrays of size 0
 * may be NULL.  Errors: CBK_E_INVALID (NULL pointer where a size is nonzero, or a header that
 * does not describe w: an exponent without a code, a length above 12 or a wrong total_bits).
 */
cbk_status cbk_ec_encode(const uint16_t *w, const cbk_ec_header *h, uint8_t *sm, uint32_t *stream,
                         uint32_t *gaps, uint32_t *bases, uint16_t *lut);

/* An encoded tensor as the GPU sees it.  Host struct, device pointers, each 16-byte aligned. */
typedef struct {
    uint64_t n;
    uint64_t total_bits;
    const uint8_t *sm;       /* n bytes, in an allocation readable up to n rounded up
                                to a multiple of 16 bytes     */
    const uint32_t *stream;  /* cbk_ec_stream_words words     */
    const uint32_t *gaps;    /* cbk_ec_gap_words words        */
    const uint32_t *bases;   /* cbk_ec_blocks words           */
    const uint16_t *lut;     /* 4096 entries                  */
    uint32_t max_block_codes;  /* cbk_ec_max_block_codes of the host arrays, or 0 if unknown */
} cbk_ec_tensor;

/*
 * cbk_ec_max_block_codes -- host.  The most codes that start in one block of 256 spans
 * (bases[k + 1] - bases[k], n - bases[last] for the last block), 0 for n == 0; h and bases as
 * cbk_ec_encode wrote them (NULL bases or h: 0).  Carried in cbk_ec_tensor.max_block_codes: at
 * most 8185 (every block of codes averaging about two bits or more, as weights' exponents do)
 * lets the GPU decode hold half a block's worst case of exponents in LDS and run more workgroups
 * per CU.  A nonzero value below a block's true count gives unspecified values for that block's
 * weights (never an access outside the arrays); values above 16384 are rejected (CBK_E_INVALID).
 */
uint32_t cbk_ec_max_block_codes(const cbk_ec_header *h, const uint32_t *bases);

/*
 * cbk_ec_decode_bf16 -- GPU.  out[i] = the original pattern of weight i, for i < n.  One
 * workgroup per block of 256 spans: each thread decodes its span from its gap with the table
 * (held in LDS) into LDS, a prefix sum of the per-thread counts places the values, and the
 * block's outputs are joined with their sign-mantissa bytes and written with coalesced stores.
 *   out   device, n uint16, 16-byte aligned.
 * A corrupt stream cannot make the kernel read or write outside the arrays given (a span emits
 * at most 64 values and the block writes at most its own range); the values are then undefined.
 * Errors: CBK_E_INVALID (NULL pointer with n > 0, total_bits > 12 n or < n), CBK_E_ALIGN,
 * CBK_E_UNSUPPORTED (n >= 2^32), CBK_E_HIP.
 */
cbk_status cbk_ec_decode_bf16(const cbk_ec_tensor *t, uint16_t *out, void *stream);

/*
 * cbk_ec_gemv -- GPU.  Decode fused into the batch-1 GEMV for a tensor of rows x cols weights
 * (row-major, rows * cols == t->n): y[r] = sum_k W[r][k] * x[k], fp32 products and sums.  The same
 * two-phase block decode as cbk_ec_decode_bf16, with each block's weights multiplied by x as they
 * are joined, summed per row in LDS and added to y with one atomic per row the block touches (a
 * row can span blocks), so the summation order varies between calls; y is zero-filled first by a
 * kernel on the same stream.  The BF16 weights never reach HBM.
 *   x     device, cols BF16 patterns, 16-byte aligned.
 *   y     device, rows fp32, 4-byte aligned; fully overwritten.
 * Errors: as cbk_ec_decode_bf16; CBK_E_INVALID for rows * cols != n, a NULL y with rows > 0 or a
 * NULL x with cols > 0 (with cols == 0 and rows > 0, y is set to zeros and x is not read);
 * CBK_E_UNSUPPORTED for cols % 8 != 0 or cols < 64 (when n > 0); CBK_E_ALIGN for x or y.
 */
cbk_status cbk_ec_gemv(const cbk_ec_tensor *t, uint64_t rows, uint64_t cols, const uint16_t *x, float *y,
                       void *stream);

/*
 * Span index -- a derived structure built once at load time, not part of the stored format.
 * Byte j is the number of codes that start in span j (0..64): what the decoder's first walk over
 * the span counts.  The per-block output positions (bases) come from the same kind of count; the
 * index carries it down to each span, so the decode and the fused GEMV below walk each span once
 * instead of twice, for one more byte per 64 stream bits read.
 *
 * cbk_ec_index_bytes(total_bits) -- bytes of a tensor's index: its spans, rounded up to 16.
 * cbk_ec_build_index -- GPU.  Writes the index of t (one walk over every span with the table).
 *   index   out, device, cbk_ec_index_bytes(t->total_bits) bytes, 16-byte aligned, caller-owned.
 *   Errors: as cbk_ec_decode_bf16 (NULL index with n > 0 gives CBK_E_INVALID).
 * cbk_ec_decode_bf16_indexed, cbk_ec_gemv_indexed -- GPU.  As cbk_ec_decode_bf16 (bit for bit) and
 *   cbk_ec_gemv (the same products, summed in an order that varies between calls), with the index
 *   that cbk_ec_build_index wrote for t (device, 16-byte aligned).  An index that does not match
 *   the stream gives wrong values but no access outside the arrays: counts above 64 are read as
 *   64, and each block writes only weights below n.
 */
uint64_t cbk_ec_index_bytes(uint64_t total_bits);
cbk_status cbk_ec_build_index(const cbk_ec_tensor *t, uint8_t *index, void *stream);
cbk_status cbk_ec_decode_bf16_indexed(const cbk_ec_tensor *t, const uint8_t *index, uint16_t *out, void *stream);
cbk_status cbk_ec_gemv_indexed(const cbk_ec_tensor *t, const uint8_t *index, uint64_t rows, uint64_t cols,
                               const uint16_t *x, float *y, void *stream);

/*
 * Grouped calls -- the matrices of a transformer block decoded together, following the DFloat11
 * page's block-level decompression ("How it works in practice"): one launch takes up to 8 tensors
 * (more are split into runs of 8), its workgroups divided among them in proportion to their
 * blocks, so the launch's start-up and tail are paid once per run instead of once per tensor.
 *
 * cbk_ec_decode_group -- GPU.  outs[i] = the patterns of ts[i], bit for bit as cbk_ec_decode_bf16.
 *   ts       host array of count tensors (device arrays inside, as for cbk_ec_decode_bf16).
 *   indexes  NULL (two walks per span), or a host array of count device pointers, indexes[i] the
 *            span index of ts[i] (every one non-NULL where ts[i].n > 0, 16-byte aligned).
 *   outs     host array of count device pointers, outs[i] holds ts[i].n BF16 patterns, 16-byte
 *            aligned; outputs must not overlap.
 * cbk_ec_gemv_group -- GPU.  ys[i] = W_i x for tensors of rows[i] x cols weights that share x, as
 *   cbk_ec_gemv (within the same bound; summation order varies); every ys[i] with rows[i] > 0 is
 *   zero-filled first, by one kernel per run.
 *   rows     host array of count row counts, rows[i] * cols == ts[i].n.
 *   x        device, cols BF16 patterns, 16-byte aligned (read when cols > 0).
 *   ys       host array of count device pointers, ys[i] holds rows[i] fp32, 4-byte aligned.
 * count == 0 is a no-op.  Errors: a NULL ts, outs, rows or ys array: CBK_E_INVALID.  Every tensor is checked
 * as by the single call before anything is launched, and the first failure's status is returned
 * with nothing enqueued.
 */
cbk_status cbk_ec_decode_group(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                               uint16_t *const *outs, void *stream);
cbk_status cbk_ec_gemv_group(const cbk_ec_tensor *ts, const uint8_t *const *indexes, uint32_t count,
                             const uint64_t *rows, uint64_t cols, const uint16_t *x, float *const *ys, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CBK_EC_H */
