/*
 * tq_ceiling.h -- measurement support in libtq (not part of the codec).
 *
 * tq_ceiling_stream runs a kernel with no codec arithmetic that moves exactly
 * the bytes of tq_encode / tq_decode at head_dim 128, in their grid (one
 * 256-thread block per 64 vectors) with every wave's loads and stores
 * contiguous, so that the codec kernels can be rated against the bandwidth
 * this byte mix reaches on the same chip, beside the HBM peak.
 *   mode 0 (encode mix): reads in0 [n, 256] bytes; writes out0 [n, packed_bytes]
 *                        and out1 [n] 4-byte words
 *   mode 1 (decode mix): reads in0 [n, packed_bytes] and in1 [n] 4-byte words;
 *                        writes out0 [n, 256] bytes
 * packed_bytes is 64, 48 or 32 (4, 3 or 2 bits).  Device pointers, 16-byte
 * aligned rows (4-byte for the word arrays), no overlap; asynchronous on
 * `stream`.  The bytes written are an XOR fold of the bytes read (unspecified
 * beyond that).  Returns 0 when enqueued, 1 for a bad argument (nothing
 * enqueued), 5 when the launch failed.
 */
#ifndef TQ_CEILING_H
#define TQ_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int tq_ceiling_stream(int mode, int packed_bytes, const void *in0, const void *in1, int64_t n,
                      void *out0, void *out1, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_CEILING_H */
