/*
 * pa_probes.h -- measurement probes (libpa_probes.so), not part of the paged
 * attention library: plain kernels that read whole pool blocks or only issue
 * matrix-core instructions, so that a benchmark can report what this GPU
 * reaches for the same bytes or the same instruction mix, and one that repeats
 * a single LDS access pattern for the bank-conflict counter.  Statuses and
 * stream convention as in include/pa.h.
 */
#ifndef PA_PROBES_H_
#define PA_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#include "../../include/pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Measured ceilings.  Each launches num_wgs workgroups of 256 threads on `stream`.
 *
 * pa_ceiling_stream_read: reads bytes (a multiple of 16) of buf once,
 *   contiguously, 16-byte non-temporal loads with 8 in flight per lane; sink
 *   as below, over the buffer's words.
 * pa_ceiling_gather_read: reads whole blocks of block_bytes (a multiple of
 *   16) from k_pool and v_pool with 16-byte non-temporal loads, block
 *   blocks[i] for i < n in list order (a block table's order is the order a
 *   paged decode reads them in; 0, 1, 2, ... is a contiguous read); entries
 *   outside [0, pool_blocks) read block 0.  Workgroup w takes an equal
 *   contiguous share of the list, and sink[4 w + v] (uint32 [num_wgs * 4])
 *   receives the XOR of the 32-bit words wave v of workgroup w read, so the
 *   XOR of all sink entries is the XOR of every word of the listed blocks of
 *   both pools.
 * pa_ceiling_mfma_bf16: each of the num_wgs * 4 waves issues iters rounds of 4
 *   independent v_mfma_f32_32x32x16_bf16 (A = B = 1); sink (float
 *   [num_wgs * 4]) receives 64 * 16 * iters per wave.  FLOPs per launch:
 *   num_wgs * 4 * iters * 4 * 32768.
 * pa_ceiling_mfma_bf16_lds: the same, with each MFMA's A operand (1 KiB per
 *   wave) read from LDS by one ds_read_b128 per lane (the prefill kernel's
 *   operand traffic for its score and PV products); LDS holds bf16 1.0, so
 *   sink receives the same values.  FLOPs per launch as above.
 */
pa_status pa_ceiling_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                                 int32_t num_wgs, void* stream);
pa_status pa_ceiling_gather_read(const void* k_pool, const void* v_pool, int64_t pool_blocks,
                                 int32_t block_bytes, const int32_t* blocks, int64_t n,
                                 uint32_t* sink, int32_t num_wgs, void* stream);
pa_status pa_ceiling_mfma_bf16(float* sink, int32_t num_wgs, int32_t iters, void* stream);
pa_status pa_ceiling_mfma_bf16_lds(float* sink, int32_t num_wgs, int32_t iters, void* stream);

/*
 * pa_probe_lds_pattern: LDS bank groups, one access pattern per launch, read
 * with the SQ_LDS_BANK_CONFLICT counter.  num_wgs workgroups of one wave;
 * each fills a 16 KiB LDS area (16-bit element k = (k * 40503) mod 2^16),
 * then repeats iters times one access per lane at byte offsets[lane]
 * (uint32 [64], device; clamped into the area and aligned down to the access
 * size): kind 0 ds_write_b128, 1 ds_read_b128, 2 ds_read_b64_tr_b16,
 * 3 ds_read_b64.  sink[w] (uint32 [num_wgs]) receives, for reads, the XOR of
 * every 16-bit element the wave read when iters is odd (0 when even), and
 * 0 for writes.
 */
pa_status pa_probe_lds_pattern(const uint32_t* offsets, int32_t kind, int32_t iters,
                               uint32_t* sink, int32_t num_wgs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBES_H_ */
