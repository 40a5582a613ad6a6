/*
 * tq.h -- C ABI of libtq, the TurboQuant KV-cache codec for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (sources are the web pages describing it):
 *   [PyPI]     pypi.org/project/aither-kvcache, project page "aither-kvcache":
 *              "Algorithm" (steps 1-5 and their reverse), "API Reference"
 *              (TurboQuant(head_dim, bits, seed), encode, decode,
 *              compression_ratio; TQPagedAttention.forward), "Paged KV cache",
 *              "Zero-buffer fused attention".
 *   [Crucible] aitherium.github.io/aitherkvcache, "aitherkvcache -- the
 *              crucible": hero sample ([..., 128] fp16 -> [..., 64] uint8 plus
 *              [...] f32 at 4 bits; 2-4 bits; 3.8-7.1x against fp16).
 *   [QBC]      qbc.network/blog/turboquant-efficient-inference: "What
 *              TurboQuant is" (multiplier-free Walsh-Hadamard rotation,
 *              Gaussian-optimal levels); "What we shipped" item 2 (rotate the
 *              query once, fold the inverse rotation into the output).
 *
 * Encode, per vector x of head_dim = d binary16 values (d = 64, 128 or 256;
 * the crucible page's sample uses 128):
 *   n = ||x||_2 (stored as f32);  z = H * D * x / n  (D = diag(sigma), sigma
 *   the seeded +-1 sign flip, H the Sylvester Hadamard matrix, so
 *   z = sqrt(d) * R * (x/n) with R = H D / sqrt(d) orthogonal and z ~ N(0,1)
 *   per coordinate);  code_i = number of Lloyd-Max N(0,1) thresholds strictly
 *   below z_i;  codes packed LSB-first, d*bits/8 bytes per vector.
 * Decode: xhat = n * D * H * c[code] / d, rounded to binary16 (nearest-even).
 *
 * Conventions for every entry point below:
 *   - Every data pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *     tensor's storage) owned by the caller; the library never allocates,
 *     frees or retains memory and keeps no state beyond an immutable codebook
 *     table computed once per process (and, for tq_attn_decode_kv_noalloc
 *     only, one fixed workspace array per GPU that is part of the loaded
 *     code object).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  A status of TQ_OK means the work was enqueued; a kernel fault
 *     surfaces at the caller's next synchronisation.
 *   - Argument errors are reported before anything is enqueued; no exception
 *     crosses the ABI.
 *   - bits must be 2, 3 or 4 and head_dim 64, 128 or 256, for every entry
 *     point (TQ_ERR_UNSUPPORTED otherwise); at head_dim 256 the attention
 *     entry points take at most 8 query heads per kv head.
 *   - binary16 and packed arrays must be 16-byte aligned, f32/int32 arrays
 *     4-byte aligned (TQ_ERR_MISALIGNED otherwise).  Inputs and outputs must
 *     not overlap (TQ_ERR_INVALID_ARG).
 *   - Inputs holding Inf or NaN are outside the method's domain: the call
 *     completes and touches only its own outputs, but their values are
 *     unspecified.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 1

typedef enum {
    TQ_OK = 0,
    TQ_ERR_INVALID_ARG = 1,  /* NULL pointer, negative size, overlap, bad shape */
    TQ_ERR_UNSUPPORTED = 2,  /* head_dim or bits outside what is implemented      */
    TQ_ERR_MISALIGNED = 3,   /* a pointer violates the alignment rules above      */
    TQ_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required        */
    TQ_ERR_HIP = 5           /* the HIP runtime refused a launch                  */
} tq_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *tq_status_string(tq_status s);

/* Version of this ABI (TQ_ABI_VERSION of the header the library was built from). */
int tq_abi_version(void);

/*
 * Bytes of packed codes per vector: head_dim * bits / 8 (64, 48, 32 for
 * bits 4, 3, 2 at head_dim 128).  With the 4-byte norm a vector costs 68/52/36
 * bytes against 256 bytes of fp16, the 3.8-7.1x of [Crucible] hero and
 * [PyPI] intro.  Returns 0 for an unsupported (head_dim, bits).
 */
size_t tq_packed_bytes(int head_dim, int bits);

/*
 * Encode n vectors ([PyPI] "Algorithm", steps 1-5; [Crucible] hero sample).
 *   x_f16   [n, head_dim] binary16, row-major (any leading shape flattened)
 *   packed  [n, head_dim*bits/8] uint8, written
 *   norms   [n] f32, written: the L2 norm of each input vector
 *   seed    selects the sign flip (the TurboQuant(seed=42) constructor argument
 *           of [PyPI] "API Reference"); the same seed must be used to decode
 * n == 0 is a no-op returning TQ_OK.
 */
tq_status tq_encode(const void *x_f16, int64_t n, int head_dim, int bits, uint64_t seed,
                    uint8_t *packed, float *norms, void *stream);

/*
 * Decode n vectors ([PyPI] "Algorithm": decoding runs steps 4 to 1 in
 * reverse).
 *   packed  [n, head_dim*bits/8] uint8, norms [n] f32 (as written by tq_encode)
 *   out_f16 [n, head_dim] binary16, written (round-to-nearest-even)
 * n == 0 is a no-op returning TQ_OK.
 */
tq_status tq_decode(const uint8_t *packed, const float *norms, int64_t n, int head_dim,
                    int bits, uint64_t seed, void *out_f16, void *stream);

/*
 * Encode n new vectors straight into a paged cache (the write side of
 * [PyPI] "Custom inference loop" -- compress where the cache is written --
 * for the block-structured cache of [PyPI] "Paged KV cache").
 *   x_f16        [n, head_dim] binary16 (e.g. one decode step's K or V,
 *                [batch * num_kv_heads, head_dim])
 *   slots        [n] int64: destination row of each vector, counted in
 *                vectors from the start of the cache, i.e.
 *                (block * block_size + offset) * num_kv_heads + kv_head;
 *                a negative slot skips its vector (padding)
 *   cache_packed [num_slots, head_dim*bits/8] uint8, rows `slots` written
 *   cache_norms  [num_slots] f32, entries `slots` written
 * Slots must be distinct (duplicates race) and below num_slots
 * (TQ_ERR_INVALID_ARG is not detected on the device: an out-of-range slot is
 * skipped by the kernel).  The bytes written equal tq_encode's for the same
 * vectors.
 */
tq_status tq_encode_paged(const void *x_f16, const int64_t *slots, int64_t n, int head_dim,
                          int bits, uint64_t seed, uint8_t *cache_packed, float *cache_norms,
                          int64_t num_slots, void *stream);

/*
 * Hybrid modes tq35 and tq25 ([PyPI] "Hybrid modes (tq35/tq25)": split-group
 * quantization with a QJL residual; "API Reference": HybridTurboQuant, whose
 * encode returns the packed bytes only, norms embedded), head_dim 128.
 *   mode  35 (tq35) or 25 (tq25): 3.5 or 2.5 bits per coordinate of codes
 *   perm  HOST array of head_dim int32, a permutation of the channels from
 *         calibration (NULL = identity): channels perm[0..63] form group A,
 *         perm[64..127] group B
 * Encode, for y = x[perm]: each half of y is a TurboQuant vector of dimension
 * 64 (norm, sign flip, 64-point Walsh-Hadamard transform, Lloyd-Max code) at
 * 3 and 2 bits (tq35) or 2 and 1 bits (tq25); the residual r = y - (decode
 * of the halves) is kept as the sign bits of H_128 D_Q r and its norm rho
 * (a QJL sign sketch with the structured projection H_128 D_Q).  The signs of
 * the seed's SplitMix64 stream are those of group A (outputs 0-63), group B
 * (64-127) and D_Q (128-255).  Row, one per vector: codes A | codes B |
 * 16 bytes of sign bits | f32 norm A | f32 norm B | f32 rho, LSB-first
 * bitstreams; 68 bytes (tq35) or 52 bytes (tq25), 4-byte aligned.
 * Decode: yhat = (decode of the halves) + sqrt(pi/2)/128 * rho * D_Q H_128 s,
 * s_i = -1 where sign bit i is set, else +1; out[perm[k]] = binary16
 * (nearest-even) of yhat[k].
 * tq_hybrid_packed_bytes returns the row bytes, 0 for an unsupported
 * (head_dim, mode).  Errors: TQ_ERR_UNSUPPORTED (head_dim other than 128, an
 * unknown mode), TQ_ERR_INVALID_ARG (null pointers, negative n, perm not a
 * permutation, overlapping input and output), TQ_ERR_MISALIGNED (x or out not
 * 16-byte aligned, packed not 4-byte aligned).  n == 0 is a no-op.
 */
size_t tq_hybrid_packed_bytes(int head_dim, int mode);
tq_status tq_hybrid_encode(const void *x_f16, int64_t n, int head_dim, int mode, uint64_t seed,
                           const int32_t *perm, uint8_t *packed, void *stream);
tq_status tq_hybrid_decode(const uint8_t *packed, int64_t n, int head_dim, int mode,
                           uint64_t seed, const int32_t *perm, void *out_f16, void *stream);

/*
 * Workspace bytes tq_attn_decode needs for this problem shape: the partial
 * softmax state (running max, sum, head_dim rotated-domain accumulators) of
 * every (sequence, query head, context split).  Deterministic in its
 * arguments.
 */
size_t tq_attn_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq);

/*
 * Single-token decode attention straight from the packed, paged cache
 * ([PyPI] "Zero-buffer fused attention": the query is rotated once, scores and
 * the value sum are formed in the rotated domain against codebook values, and
 * one inverse rotation is applied at the end; [QBC] "What we shipped" item 2;
 * argument list of TQPagedAttention.forward in [PyPI] "API Reference").
 *   q_f16        [batch, num_q_heads, head_dim] binary16
 *   k_packed     [num_blocks, block_size, num_kv_heads, head_dim*bits/8] uint8
 *   k_norms      [num_blocks, block_size, num_kv_heads] f32
 *   v_packed, v_norms: same layout as K; K and V share bits and seed
 *   block_tables [batch, max_blocks_per_seq] int32: physical block of each
 *                16-token page of each sequence (entries past the context
 *                are not read)
 *   context_lens [batch] int32, each in [0, max_blocks_per_seq*block_size]
 *   scale        softmax scale (1/sqrt(head_dim) is the usual value)
 *   out_f16      [batch, num_q_heads, head_dim] binary16, written:
 *                softmax(scale * q.K^T) V over the first context_lens[b]
 *                tokens, with query head h reading kv head
 *                h / (num_q_heads / num_kv_heads); zeros when the context is 0
 *   workspace    device scratch of at least tq_attn_workspace_bytes(...) bytes
 *                (16-byte aligned); contents on entry are ignored
 *   num_blocks   number of physical blocks in the cache arrays; a block-table
 *                entry outside [0, num_blocks) is never dereferenced -- its
 *                tokens are left out of the softmax (the output for that
 *                sequence is then unspecified but memory stays in bounds)
 * num_q_heads must be a multiple of num_kv_heads with at most 16 query heads
 * per kv head (8 at head_dim 256); block_size must be 16; batch at most
 * 65535, batch * num_q_heads at most 2^31 - 1 and max_blocks_per_seq at most
 * (2^31 - 1) / 16 (TQ_ERR_UNSUPPORTED otherwise; tq_attn_workspace_bytes
 * returns 0 for such shapes).  A context length outside
 * [0, max_blocks_per_seq * block_size] is clamped into that range.
 * Errors: TQ_ERR_INVALID_ARG (null pointers, negative sizes, a non-finite
 * scale, an output or workspace overlapping any other array),
 * TQ_ERR_UNSUPPORTED (head_dim, bits, group size
 * or block_size outside the supported set), TQ_ERR_MISALIGNED,
 * TQ_ERR_WORKSPACE (missing or short workspace), TQ_ERR_HIP (launch failure).
 */
tq_status tq_attn_decode(const void *q_f16, const uint8_t *k_packed, const float *k_norms,
                         const uint8_t *v_packed, const float *v_norms,
                         const int32_t *block_tables, const int32_t *context_lens, int batch,
                         int num_q_heads, int num_kv_heads, int head_dim, int bits,
                         uint64_t seed, int block_size, int max_blocks_per_seq,
                         int64_t num_blocks, float scale, void *out_f16, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * tq_attn_decode with keys and values stored at different widths: k_packed
 * rows hold head_dim*k_bits/8 bytes and v_packed rows head_dim*v_bits/8
 * (for instance 4-bit keys with 2-bit values, as on the KVarN repository
 * page, "What it does").  Both use the seed's sign flip; every other argument,
 * the workspace size and the error behaviour are those of tq_attn_decode,
 * which equals this call with k_bits = v_bits = bits.
 */
tq_status tq_attn_decode_kv(const void *q_f16, const uint8_t *k_packed, const float *k_norms,
                            const uint8_t *v_packed, const float *v_norms,
                            const int32_t *block_tables, const int32_t *context_lens, int batch,
                            int num_q_heads, int num_kv_heads, int head_dim, int k_bits,
                            int v_bits, uint64_t seed, int block_size, int max_blocks_per_seq,
                            int64_t num_blocks, float scale, void *out_f16, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * tq_attn_decode_kv for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid hipMalloc):
 * the same computation, arguments, output and errors, but no workspace
 * argument.  The partial softmax state lives in a fixed array inside the
 * library, TQ_ATTN_NOALLOC_WORKSPACE_BYTES bytes on each GPU it runs on
 * (held from the first call on that device until the process ends); the
 * first call on a device looks up that array's address there.  The call
 * allocates nothing.
 *   - A shape whose tq_attn_workspace_bytes(...) exceeds
 *     TQ_ATTN_NOALLOC_WORKSPACE_BYTES returns TQ_ERR_WORKSPACE before
 *     anything is enqueued (at head_dim 128: batch * num_q_heads * splits
 *     up to 64,527 partial states of 520 bytes, e.g. batch 16 x 32 heads at
 *     a 32K context uses 8.5 MB).
 *   - Every call on a GPU uses that GPU's one array: calls that may overlap
 *     on one GPU (on different streams, or from different host threads)
 *     race and must be serialised by the caller.  Nothing in the array needs
 *     to start at zero; its contents after a call are unspecified.
 *   - TQ_ERR_HIP also reports a failed address lookup.
 */
#define TQ_ATTN_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
tq_status tq_attn_decode_kv_noalloc(const void *q_f16, const uint8_t *k_packed,
                                    const float *k_norms, const uint8_t *v_packed,
                                    const float *v_norms, const int32_t *block_tables,
                                    const int32_t *context_lens, int batch, int num_q_heads,
                                    int num_kv_heads, int head_dim, int k_bits, int v_bits,
                                    uint64_t seed, int block_size, int max_blocks_per_seq,
                                    int64_t num_blocks, float scale, void *out_f16,
                                    void *stream);

/*
 * Host-side test hooks (no device work).
 * tq_codebook: the f32 Lloyd-Max levels (2^bits, ascending) and decision
 *   thresholds (2^bits - 1, the level midpoints) the kernels use
 *   ([PyPI] "Algorithm" step 3; [QBC] "What TurboQuant is").
 * tq_signs: the sign flip as a bit mask, bit i of mask[i/32] set iff
 *   sigma_i = -1 (head_dim/32 words; sigma of a shorter head_dim is a prefix
 *   of sigma of a longer one).
 */
tq_status tq_codebook(int bits, float *levels, float *thresholds);
tq_status tq_signs(uint64_t seed, int head_dim, uint32_t *mask);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
