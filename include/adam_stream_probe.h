/*
 * adam_stream_probe.h -- a measurement kernel for AMD Instinct MI355X
 * (gfx950), shipped beside the Adam step library and not part of the step.
 *
 * The compressed-moment Adam step ("feat: add 8-bit Adam optimizer for
 * memory efficiency", AiDotNet PR #814; "perf(training): make BF16-Adam
 * fused-compatible", AiDotNet PR #1745) is a streaming map: per parameter it
 * reads the param, the grad and each moment once and writes the param and
 * each moment once, plus one scale per 2048-element block per 8-bit moment.
 * Its roofline is HBM bandwidth.  The probe moves the same bytes in the same
 * pattern with no arithmetic, so its rate is the bandwidth that pattern can
 * reach on the part: the ceiling to set the step's rate against, besides the
 * 8 TB/s peak.
 *
 * Pattern (the step's): one 256-thread workgroup per 2048-element block;
 * thread t handles elements 4t..4t+3 and 1024+4t..1024+4t+3 of its block;
 * every load and store is non-temporal and as wide as four elements allow
 * (16 bytes of fp32, 8 of bf16, 4 of 8-bit codes); every thread reads the
 * block's scales (block-uniform addresses) and thread 0 writes them.  With
 * 8-bit moments the block's loads all complete before
 * a workgroup barrier (the step's block statistic), and the stores follow
 * it.  Workgroups take blocks in the step's XCD order (runs of 16
 * consecutive blocks per XCD) and an LDS reservation caps how many share a
 * CU.
 *
 * Stored values: param' = param + grad (bf16 grads widened exactly), every
 * 32-bit word of a moment buffer XORed with 0x01010101, every scale's bit
 * pattern plus 1.
 */
#ifndef ADAM_STREAM_PROBE_H
#define ADAM_STREAM_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One probe launch over n_blocks full blocks, enqueued on `stream`
 * (hipStream_t as void*; NULL is the null stream).
 *   param   float[n_blocks * 2048], read and written
 *   grad    float or bf16 (grad_bytes 4 or 2) [n_blocks * 2048], read
 *   m       storage 1 (bf16 moments): uint16[n_blocks * 2048];
 *           storage 2 (8-bit m and v): uint8[n_blocks * 2048];
 *           storage 3 (fp32 m, 8-bit v): float[n_blocks * 2048]; read and written
 *   v       storage 1: uint16[...]; storages 2, 3: uint8[...]; read and written
 *   w       with amsgrad != 0, the running maximum of v, stored as v is;
 *           else ignored (may be NULL)
 *   scales  float[n_scales * n_blocks], moment-major (m, v, then w), with
 *           n_scales = 0 for storage 1, 2 (+1 with amsgrad) for storage 2,
 *           1 (+1 with amsgrad) for storage 3; may be NULL when n_scales = 0
 *   resident_per_cu  at most this many workgroups per CU, 2..8 (8: no cap)
 * Device buffers are the caller's and must be 16-byte aligned.  Returns 0,
 * -1 (bad argument: storage or grad_bytes out of range, n_blocks 0 or at
 * least 2^24, resident_per_cu outside 2..8, a NULL or misaligned buffer that
 * the storage needs; nothing is enqueued) or -5 (the launch failed).
 */
int adam_stream_probe(void *param, const void *grad, void *m, void *v, void *w, float *scales,
                      uint32_t n_blocks, int32_t grad_bytes, int32_t storage, int32_t amsgrad,
                      int32_t resident_per_cu, void *stream);

/* Bytes one launch moves (reads + writes), as laid out above; 0 for bad
 * arguments.  Pure host function. */
uint64_t adam_stream_probe_bytes(uint32_t n_blocks, int32_t grad_bytes, int32_t storage,
                                 int32_t amsgrad);

#ifdef __cplusplus
}
#endif

#endif /* ADAM_STREAM_PROBE_H */
