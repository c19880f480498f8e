/*
 * sgqa_probe.h -- C ABI of libsgqa_probe.so, the machine-peak probes that the benchmark quotes
 * its rooflines against (measured peaks beside the vendor ones).  They are measurement tools,
 * not calls of the layer, so they live in a library of their own next to libsgqa.so.
 *
 * Pointers marked "device" are device memory of the current HIP device; every call is
 * asynchronous on `stream` (a hipStream_t, NULL for the default stream).  Each call returns
 * SGQA_OK or an sgqa_status error code; sgqa_probe_last_error() describes the calling
 * thread's most recent failure.
 */
#ifndef SGQA_PROBE_H
#define SGQA_PROBE_H

#include "sgqa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * sgqa_probe_mfma_bf16: `waves` waves (1 <= waves <= 1 << 20) each run iters (1..8192)
 * rounds of 8 independent 32x32x16 bf16 matrix products (32 768 flop each) on operands equal
 * to 1.0, and wave w writes 2048 * iters (exact) to sink[w] (device, fp32, [waves]).
 * Total work: waves * iters * 8 * 32768 flop.
 *
 * sgqa_probe_read: reads `bytes` (a positive multiple of 16) of device memory at buf
 * (16-byte aligned) once, `blocks` workgroups (1..65536) striding over it, and writes to
 * sink[b] (device, uint32, [blocks]) the sum modulo 2^32 of the 32-bit words workgroup b
 * read; the partial sums add up (mod 2^32) to the sum of all the buffer's words.
 *
 * sgqa_probe_gather: the access pattern of the sparse attention's K/V gathers without its
 * arithmetic.  table (device, 16-byte aligned) holds rows of row_bytes (a positive multiple
 * of 16, at most 65536); for i < n it reads row idx[i] (device int32, each in
 * [0, table_rows), unchecked on the device: the caller guarantees it), `blocks` workgroups
 * (1..65536) striding over the n * row_bytes / 16 words; sink[b] (device, uint32, [blocks])
 * gets the sum modulo 2^32 of the 32-bit words workgroup b read, so the partial sums add up
 * to the sum over i of the words of row idx[i].
 */
sgqa_status sgqa_probe_mfma_bf16(int32_t waves, int32_t iters, float *sink, void *stream);
sgqa_status sgqa_probe_read(const void *buf, size_t bytes, uint32_t *sink, int32_t blocks,
                            void *stream);
sgqa_status sgqa_probe_gather(const void *table, int64_t table_rows, int32_t row_bytes,
                              const int32_t *idx, int64_t n, uint32_t *sink, int32_t blocks,
                              void *stream);

/* Per-thread description of the most recent failure of a probe call ("" if none). */
const char *sgqa_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SGQA_PROBE_H */
