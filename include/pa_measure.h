/*
 * pa_measure.h -- measured ceilings for the attention kernels of libpa.so.
 *
 * Two kernels that do nothing but what bounds the attention kernels, so that
 * their speed can be reported against what this GPU achieves on the same
 * pattern as well as against the published peaks: the decode path is bound
 * by streaming scattered 4 KiB K/V tiles from HBM (the chapter "Inference
 * optimisation", section 8.2.1: decode reads the whole KV cache every step),
 * the chunk path by bf16 matrix products.  Neither is part of the attention
 * computation; both follow pa.h's conventions (device pointers owned by the
 * caller, work enqueued on `stream`, host-side errors before any launch).
 */
#ifndef PA_MEASURE_H_
#define PA_MEASURE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read tiles[i] of both caches for i < num_tiles: the 4 KiB tile at byte
 * offset 4096 * tiles[i] of k_cache and of v_cache, with the loads the decode
 * kernel uses (128-bit, non-temporal, one 1 KiB row group per wave
 * instruction), and fold the words into one uint32 per workgroup written to
 * sink[workgroup] (so no load can be dropped).  Workgroups of 256 threads take
 * `tiles_per_wg` consecutive entries each; grid = ceil(num_tiles /
 * tiles_per_wg), and sink must hold that many words.  Tile indices are the
 * caller's (e.g. physical block * num_kv_heads + KV head, as the decode kernel
 * addresses them) and must lie inside both caches.  Errors: PA_ERR_NULL_ARG,
 * PA_ERR_BAD_SHAPE (num_tiles < 0 or tiles_per_wg < 1), PA_ERR_LAUNCH. */
pa_status pa_measure_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                                int64_t num_tiles, int32_t tiles_per_wg, uint32_t* sink,
                                void* stream);

/* bf16 matrix-core throughput: `workgroups` workgroups of 256 threads, each
 * wave running `iters` rounds of four independent v_mfma_f32_32x32x16_bf16
 * chains (32 x 32 x 16 multiply-adds each, 32,768 FLOP per product), then
 * writing one float per wave to sink (workgroups * 4 floats).  FLOP per call:
 * workgroups * 4 waves * iters * 4 * 32768.  Errors: PA_ERR_NULL_ARG,
 * PA_ERR_BAD_SHAPE (workgroups < 1 or iters < 1), PA_ERR_LAUNCH. */
pa_status pa_measure_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif  // PA_MEASURE_H_
