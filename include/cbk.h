/*
 * cbk.h -- C ABI of libcbk: lossless codebook compression of BF16 weight tensors, decoded on
 * an MI355X (gfx950) GPU standalone or fused into the decode-step GEMV / skinny GEMM.
 *
 * The operation (codebook lossless compression overview, section "How it works"; and the
 * Codebook-Quantization digest, "Key points" and competitor table): a weight tensor is stored
 * as a dictionary of its distinct values plus, for every weight, the index of its value in that
 * dictionary, the indices bit-packed at a fixed width of about 12-13 bits; at inference the
 * original values are substituted back exactly.  The format fixed here:
 *
 *   codebook  U distinct 16-bit patterns of the tensor, strictly ascending as unsigned
 *             integers (+0 and -0 differ; every NaN payload is its own entry), 0 <= U <= 65536;
 *   b         the smallest width with 2^b >= U (0 when U <= 1);
 *   words     index i occupies bits [i*b, i*b + b) of a little-endian uint32 stream, least
 *             significant bit first; bits at positions >= n*b are zero.  Buffers handed to the
 *             GPU calls hold cbk_words_for(n, b) words (the stream rounded up to 16 bytes).
 *
 * Tensors are row-major [rows][cols] (rows = output features, cols = input features) and the
 * stream runs through them in that order with no per-row padding.
 *
 * Conventions for every call:
 *  - Every call returns a cbk_status; nothing throws across the ABI.
 *  - Arguments are validated on the host before any HIP call; on error nothing is enqueued.
 *  - GPU calls take device pointers (in the arguments and inside cbk_tensor, which itself lives
 *    in host memory), enqueue work on `stream` (a hipStream_t; NULL = the null stream) and
 *    return without waiting.  Buffers must stay alive until that work completes.
 *  - The caller owns every buffer.  The library allocates no memory and keeps no per-call state,
 *    so calls are safe from several host threads and streams at once.  The exceptions are
 *    cbk_encode_gpu_noalloc, which uses a static device array of the library, and a GEMV chain,
 *    whose caller-owned buffer holds the state of its runs (see each).
 *  - Outputs must not alias inputs.
 *  - An index >= U in a (corrupt) stream never causes an out-of-bounds access; the weight it
 *    names reads as 0x7FC0 (a quiet NaN).
 */
#ifndef CBK_H
#define CBK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CBK_OK = 0,
    CBK_E_INVALID = 1,      /* null pointer, bad size, U/b mismatch, batch out of range      */
    CBK_E_CAPACITY = 2,     /* cbk_encode: output word buffer too small (see words_needed)  */
    CBK_E_ALIGN = 3,        /* a device pointer or leading dimension breaks an alignment rule */
    CBK_E_UNSUPPORTED = 4,  /* shape beyond what the kernels accept (see each call)          */
    CBK_E_HIP = 5,          /* the HIP runtime reported an error at launch                   */
    CBK_E_TIMEOUT = 6       /* a chained launch gave up waiting (cbk_gemv_chain_check)        */
} cbk_status;

/* A compressed tensor as the GPU calls see it.  Host struct, device pointers. */
typedef struct {
    uint64_t rows;             /* output features; rows * cols must not overflow              */
    uint64_t cols;             /* input features                                              */
    uint32_t U;                /* codebook entries, 0..65536 (0 only when rows * cols == 0)   */
    uint32_t b;                /* index width; must equal cbk_bits_for(U)                     */
    const uint16_t *codebook;  /* device, U entries (may be NULL when U == 0)                 */
    const uint32_t *words;     /* device, cbk_words_for(rows*cols, b) words, 16-byte aligned
                                  (may be NULL when b == 0)                                   */
} cbk_tensor;

/* Smallest b with 2^b >= U; 0 for U <= 1. */
uint32_t cbk_bits_for(uint32_t U);

/* Words a GPU call reads for n fields of b bits: ceil(n*b/32) rounded up to a multiple of 4. */
uint64_t cbk_words_for(uint64_t n, uint32_t b);

/* Accounting size of a compressed tensor in bytes: 2*U + ceil(n*b/8) (the padding of the word
 * buffer is not counted).  This is the size the compression ratio and GB/s figures use. */
uint64_t cbk_compressed_bytes(uint64_t n, uint32_t U);

/* Static, NUL-terminated description of a status code. */
const char *cbk_status_str(int status);

/*
 * cbk_encode -- host, synchronous, re-entrant.  Compresses n 16-bit patterns w[0..n).
 *   codebook   out, capacity 65536 entries (host); receives the U sorted distinct patterns.
 *   U, b       out (host).
 *   words      out (host), capacity words_cap words; receives cbk_words_for(n, b) words, the
 *              padding words zero.  May be NULL with words_cap == 0 to query the size.
 *   words_needed  out (host, may be NULL): cbk_words_for(n, b).
 * Returns CBK_E_CAPACITY (after filling codebook, U, b and words_needed) when words_cap is too
 * small, CBK_E_INVALID for a NULL w with n > 0 or a NULL codebook/U/b.
 */
cbk_status cbk_encode(const uint16_t *w, uint64_t n, uint16_t *codebook, uint32_t *U, uint32_t *b,
                      uint32_t *words, uint64_t words_cap, uint64_t *words_needed);

/*
 * cbk_cap_patterns -- host, synchronous.  The lossy "capped codebook" step that comes before
 * cbk_encode when the stored codebook may hold at most K entries (the codebook overview's how-to
 * section sets codebook_size=8192; the Codebook-Quantization digest mentions lossy, balanced
 * variants).  w_out[i] receives w[i] mapped as follows:
 *   - a tensor with at most K distinct patterns is copied unchanged (the lossless case);
 *   - otherwise exactly K patterns are kept: every Inf/NaN pattern present (exponent field 255),
 *     then the most frequent finite ones, ties to the smaller pattern;
 *   - every other pattern becomes the kept finite value nearest to it as a real number, ties
 *     going to the value closer to zero, then to the smaller pattern.
 *   U_out  out: distinct patterns in w_out (min(U, K)).
 * w_out may equal w.  Errors: CBK_E_INVALID (NULL pointer, K == 0), CBK_E_UNSUPPORTED (the
 * Inf/NaN patterns alone leave no room for a finite value, or n > 2^40).
 */
cbk_status cbk_cap_patterns(const uint16_t *w, uint64_t n, uint32_t K, uint16_t *w_out, uint32_t *U_out);

/*
 * Kernel choice (all calls): a width b >= 1 whose rows hold a whole number of lane units
 * (cols % (128 >> ctz(b)) == 0) takes the fast kernels, which stage the codebook (and x) in LDS;
 * b == 0, ragged rows, misaligned operands and shapes beyond the LDS budget take generic kernels
 * that give the same results.
 */

/*
 * cbk_encode_gpu -- the same encoding as cbk_encode, computed on the GPU for the load-time path
 * (the codebook overview's "Pitfalls": loading a compressed model is slower; this moves the
 * compression step onto the device).  Enqueued on `stream`; nothing is copied to the host.
 *   w          in, device, n 16-bit patterns, 16-byte aligned (when n > 0).
 *   workspace  device scratch of cbk_encode_gpu_workspace_bytes() bytes, 16-byte aligned, owned by
 *              the caller; its contents on entry do not matter and are left undefined.
 *   codebook   out, device, capacity 65536 entries; receives the U sorted distinct patterns.
 *   words      out, device, 16-byte aligned, capacity words_cap >= cbk_words_for(n, 16) words (b is
 *              known only on the device); receives cbk_words_for(n, b) words, the last ones
 *              zero-padded exactly as cbk_encode writes them.  Words past that are not written.
 *   meta       out, device, two uint32: meta[0] = U, meta[1] = b.
 * The result is bit-identical to cbk_encode on the same input.  Several calls may run at once
 * only with separate workspaces.
 * Errors: CBK_E_INVALID (null pointer), CBK_E_ALIGN, CBK_E_CAPACITY (words_cap too small),
 * CBK_E_UNSUPPORTED (n >= 2^40), CBK_E_HIP (launch failure).
 */
size_t cbk_encode_gpu_workspace_bytes(void);
cbk_status cbk_encode_gpu(const uint16_t *w, uint64_t n, void *workspace, uint16_t *codebook, uint32_t *words,
                          uint64_t words_cap, uint32_t *meta, void *stream);

/*
 * cbk_encode_gpu_group -- GPU.  cbk_encode_gpu for several tensors, such as a transformer block's
 * matrices, with one clear, one presence and one pack launch per run of up to 8 tensors (more are
 * split into runs of 8) instead of three launches each: the launches' start-up and tail are paid
 * once per run, as the DFloat11 page does for a block's matrices ("How it works in practice",
 * block-level decompression).  Each job's result is bit-identical to cbk_encode_gpu on it.
 *   jobs       host array of count jobs; each job's fields mean what the same-named arguments of
 *              cbk_encode_gpu mean, with the same alignment rules.
 *   workspace  device scratch of min(count, 8) * cbk_encode_gpu_workspace_bytes() bytes, 16-byte
 *              aligned, owned by the caller; its contents on entry do not matter.
 * count == 0 is a no-op.  Errors: CBK_E_INVALID (NULL jobs or workspace, or a job with a null
 * pointer); then each job's checks as in cbk_encode_gpu, in order; the first failure is returned
 * and nothing is enqueued.
 */
typedef struct {
    const uint16_t *w;   /* in, device, n patterns                                   */
    uint64_t n;
    uint16_t *codebook;  /* out, device, capacity 65536 entries                       */
    uint32_t *words;     /* out, device, capacity words_cap >= cbk_words_for(n, 16)   */
    uint64_t words_cap;
    uint32_t *meta;      /* out, device, meta[0] = U, meta[1] = b                     */
} cbk_encode_job;
cbk_status cbk_encode_gpu_group(const cbk_encode_job *jobs, uint32_t count, void *workspace, void *stream);

/*
 * cbk_encode_gpu_noalloc -- GPU.  For callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same encoding as
 * cbk_encode_gpu (arguments, result, alignment and errors as there), without the workspace
 * argument: the 65,536 bytes of presence bitmaps live in a static device array of the library,
 * one per GPU, held until the process ends.  Nothing is allocated by this call.
 *   Scratch limit: the array is a fixed 65,536 bytes, enough for every n the encoder accepts
 *   (n < 2^40; larger n gives CBK_E_UNSUPPORTED before any HIP call).
 *   Sharing: every call on one GPU uses that GPU's array, and each call clears it (with a kernel,
 *   no memset) before use.  Calls that overlap on one GPU (from several streams or threads
 *   without ordering between them) race on it and give undefined results; order them.
 *   The first call on a device looks up the array's device address (hipGetSymbolAddress, not a
 *   stream operation) with that device current; CBK_E_HIP if the lookup fails.
 */
cbk_status cbk_encode_gpu_noalloc(const uint16_t *w, uint64_t n, uint16_t *codebook, uint32_t *words,
                                  uint64_t words_cap, uint32_t *meta, void *stream);

/*
 * cbk_decode_bf16 -- GPU.  Standalone decode: out[i] = codebook[index i] for i < rows*cols,
 * the exact original bit patterns (no float conversion anywhere).
 * Passage: the codebook overview ("Codebook Lossless Compression", ai-manual.ru), section
 * "Как работает эта магия?" (how it works): at inference every dictionary index is replaced by the
 * original value it stands for, with nothing approximated; and the Codebook-Quantization digest
 * (setupai.cc), section "關鍵要點" (key points): the indices of the unique weights are bit-packed.
 * This call performs that substitution for a whole tensor and writes the BF16 weights to HBM.
 *   out   device, rows*cols uint16, 2-byte aligned.
 */
cbk_status cbk_decode_bf16(const cbk_tensor *t, uint16_t *out, void *stream);

/*
 * cbk_decode_group -- GPU.  cbk_decode_bf16 for count tensors: consecutive tensors of one width
 * (up to 8) are decoded by one launch whose workgroups are divided among them, so a transformer
 * block's matrices pay one launch's start-up and tail (the DFloat11 page, "How it works in
 * practice": a block's matrices decompressed together).  Each output is bit-identical to
 * cbk_decode_bf16 on its tensor.
 *   ts    host array of count tensors (device arrays inside).
 *   outs  host array of count device pointers, outs[i] holds rows*cols uint16 of ts[i], 2-byte
 *         aligned (16-byte aligned outputs take the fast kernel); outputs must not overlap.
 * count == 0 is a no-op.  Errors: CBK_E_INVALID for a NULL array; every tensor is checked as by
 * cbk_decode_bf16 before anything is launched, and the first failure's status is returned.
 */
cbk_status cbk_decode_group(const cbk_tensor *ts, uint32_t count, uint16_t *const *outs, void *stream);

/*
 * cbk_gemv -- GPU.  Fused decode + GEMV at batch 1: y[r] = sum_k W[r][k] * x[k], products and
 * sums in fp32 (the summation order is unspecified; each BF16 x BF16 product is exact in fp32).
 * Passage: the same two sections as cbk_decode_bf16 (the overview's "Как работает эта магия?":
 * original values substituted back at inference; the digest's "關鍵要點": bit-packed indices of
 * the unique weights).  Here the substituted weights feed the decode step's matrix-vector product
 * directly, in registers, without being written to memory.
 *   x   device, cols BF16 patterns, 2-byte aligned (16-byte aligned for the fast kernels).
 *   y   device, rows fp32, 4-byte aligned.  Fully overwritten (zeros when cols == 0).
 */
cbk_status cbk_gemv(const cbk_tensor *t, const uint16_t *x, float *y, void *stream);

/*
 * cbk_gemv_group -- GPU.  The same GEMV for `count` tensors that share one input vector x (for
 * example the query/key/value projections of a layer, or its gate and up projections):
 * ys[i][r] = sum_k W_i[r][k] * x[k].  Tensors of equal width b are decoded together in one launch
 * (up to 8 per launch), so the launch's ramp-up and tail are paid once for the group.  This
 * follows the DFloat11 page ("No more compromises! DFloat11 ...", section "How it works in
 * practice"): decompressing all matrices of a transformer block together keeps the GPU busy
 * and hides latency.
 *   ts     host array of count tensors (device pointers inside), all with the same cols.
 *   x      device, cols BF16 patterns (alignment as for cbk_gemv).
 *   ys     host array of count device pointers; ys[i] receives ts[i].rows fp32 values.
 * count == 0 is a no-op; count > 4096 or differing cols give CBK_E_INVALID.
 */
cbk_status cbk_gemv_group(const cbk_tensor *ts, uint32_t count, const uint16_t *x, float *const *ys,
                          void *stream);

/*
 * GEMV chain -- GPU.  A sequence of dependent grouped GEMVs ("phases", each as cbk_gemv_group)
 * run by one persistent launch: phase p + 1 reads its x only after every output of phase p is
 * written, as when x is computed from phase p's outputs (a decode step's [q, k, v] -> [o] ->
 * [gate, up] -> [down] over its layers).  Each phase's outputs are the cbk_gemv_group results,
 * bit for bit.
 * Passage: the DFloat11 page ("No more compromises! DFloat11 ...", section "How it works in
 * practice"): decompressing a transformer block's matrices together keeps the GPU busy and hides
 * latency.  The chain carries that across the block's dependent phases: while the last rows of a
 * phase are decoded, the first weights of the next one are already being read (the weights do not
 * depend on x), and no launch boundary separates the phases.
 *
 * One workgroup per compute unit runs every phase, and the grid meets at a barrier between two
 * phases.  The launch is cooperative (the runtime places the whole grid before it starts), and
 * every wait at a barrier is bounded: past timeout_us microseconds of waiting a workgroup records
 * the failure and stops, the others stop at their next wait, and cbk_gemv_chain_check reports
 * CBK_E_TIMEOUT (the outputs are then incomplete).  So a run always ends.
 *
 * cbk_gemv_chain_bytes(phases) -- device bytes of a chain of that many phases (256 of state plus
 *   the phase descriptors).
 * cbk_gemv_chain_init -- host, synchronous.  Validates the phases, plans each over the chain's
 *   grid and copies the plan into `buffer` (hipMemcpy to the current device).
 *   phases   host array of count phases.  Every tensor of every phase has the same b (1..15);
 *            within a phase every tensor has the same cols; cols % 64 == 0, cols <= 32768,
 *            rows >= 1; codebooks and every x 16-byte aligned; ys[i] 4-byte aligned.
 *   count    1..65536 phases.
 *   buffer   device, caller-owned, >= cbk_gemv_chain_bytes(count) bytes, 256-byte aligned; it
 *            must outlive every run, and holds the chain's barrier state: runs of one chain must
 *            not overlap (order them on one stream).
 *   chain    out (host): the handle the other calls take.  The tensors, x and ys are recorded by
 *            address: they must stay allocated, and their contents are read at each run.
 *   Errors: CBK_E_INVALID (null pointer, count or a phase's count out of range, differing cols
 *   within a phase, rows == 0), CBK_E_CAPACITY (buffer too small), CBK_E_ALIGN,
 *   CBK_E_UNSUPPORTED (differing b across phases, b outside 1..15, cols outside the limits,
 *   rows * cols / 64 >= 2^32, no cooperative launch on this device or not enough LDS), CBK_E_HIP.
 * cbk_gemv_chain_run -- GPU.  Enqueues one run of every phase on `stream` (a small kernel that
 *   clears the barrier state, then the chained kernel), on the device the chain was built on.
 *   timeout_us bounds each barrier wait (0: give up at once when a wait is needed; a
 *   million is a safe value for any shape).
 * cbk_gemv_chain_check -- host, synchronous.  After a run has completed (its stream
 *   synchronized): CBK_OK if it finished every phase, CBK_E_TIMEOUT if a wait gave up.
 */
typedef struct {
    const cbk_tensor *ts;  /* host array of count tensors (device pointers inside)          */
    uint32_t count;        /* 1..8                                                          */
    const uint16_t *x;     /* device, cols BF16 patterns                                    */
    float *const *ys;      /* host array of count device pointers, ys[i]: ts[i].rows fp32   */
} cbk_gemv_phase;

typedef struct {           /* filled by cbk_gemv_chain_init; the caller only passes it on   */
    void *buffer;          /* the caller's device buffer                                    */
    uint32_t phases, b, grid, lds_bytes, x_bytes, device;
} cbk_gemv_chain;

size_t cbk_gemv_chain_bytes(uint32_t phases);
cbk_status cbk_gemv_chain_init(const cbk_gemv_phase *phases, uint32_t count, void *buffer, size_t bytes,
                               cbk_gemv_chain *chain);
cbk_status cbk_gemv_chain_run(const cbk_gemv_chain *chain, uint32_t timeout_us, void *stream);
cbk_status cbk_gemv_chain_check(const cbk_gemv_chain *chain);

/*
 * cbk_gemm_small -- GPU.  Fused decode + skinny GEMM: Y[j][r] = sum_k W[r][k] * X[j][k] for
 * j < batch, fp32 products and sums.
 * Passage: as cbk_gemv (the overview's "Как работает эта магия?" and the digest's "關鍵要點"),
 * for a decode step that serves up to 16 sequences at once: each substituted weight meets every
 * row of X.
 *   X     device, [batch][ldx] BF16, 2-byte aligned, ldx >= cols.  The fast kernels need X
 *         16-byte aligned and ldx % 8 == 0; other layouts take the generic kernel.
 *   batch 1..16.  Batches up to 8 run on the vector ALUs; 9..16 run on the matrix cores.
 *   Y     device, [batch][ldy] fp32, 4-byte aligned; ldy >= rows.  Y[j][0..rows) overwritten.
 */
cbk_status cbk_gemm_small(const cbk_tensor *t, const uint16_t *X, uint64_t ldx, uint32_t batch,
                          float *Y, uint64_t ldy, void *stream);

/*
 * cbk_gemm_group -- GPU.  cbk_gemm_small for `count` tensors that share one input X (the
 * query/key/value projections, or gate and up, of a layer at batch > 1):
 * Ys[i][j][r] = sum_k W_i[r][k] * X[j][k] for j < batch.  Tensors of equal width b run in one
 * launch (up to 8 per launch), so a small tensor (a 1024-row key projection, say) shares the
 * machine with its neighbours instead of occupying a few CUs on its own; same source as
 * cbk_gemv_group (the DFloat11 page, "How it works in practice": decompress a block's
 * matrices together).
 *   ts       host array of count tensors (device pointers inside), all with the same cols.
 *   X, ldx, batch   as for cbk_gemm_small (shared by all tensors).
 *   Ys       host array of count device pointers; Ys[i] is [batch][ldys[i]] fp32, 4-byte aligned.
 *   ldys     host array of count leading dimensions, ldys[i] >= ts[i].rows.
 * count == 0 is a no-op.  count > 4096, differing cols, a null array, ldys[i] < rows or any
 * argument cbk_gemm_small would reject give the same status codes (checked before any launch).
 */
cbk_status cbk_gemm_group(const cbk_tensor *ts, uint32_t count, const uint16_t *X, uint64_t ldx,
                          uint32_t batch, float *const *Ys, const uint64_t *ldys, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CBK_H */
