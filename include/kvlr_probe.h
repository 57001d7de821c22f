/*
 * kvlr_probe.h -- measurement probes of the kvlr library (MI355X, gfx950).
 *
 * Not part of the method: plain kernels that measure what the hardware
 * delivers, so the path's kernels can be compared with measured ceilings
 * as well as against the vendor peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16
 * MFMA).  Every call enqueues one kernel on `stream` (a hipStream_t as void*)
 * and returns without waiting; the caller times it with events.  Pointers
 * are device memory owned by the caller.  Returns 0 (KVLR_OK) or 1
 * (KVLR_EINVAL) for bad arguments, 4 (KVLR_ELAUNCH) for a failed launch.
 */
#ifndef KVLR_PROBE_H
#define KVLR_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stream-read `bytes` (a multiple of 16 KiB) from src once.
 *   method 0: 16-byte loads into registers, each of the 256 threads of a
 *             block keeping `depth` (1..16) loads in flight; grid-stride over
 *             `blocks` blocks;
 *   method 1: direct global -> LDS loads (16 bytes per lane) into a ring of
 *             4 LDS stages of 32 KiB, three stages in flight, 512 threads per
 *             block (the scheme of the latent scoring kernel, with no compute);
 *             `depth` is ignored;
 *   method 2: method 1 with non-temporal loads (the cache policy of the
 *             latent scan: streamed data is not kept in the caches);
 *   method 3: the ring of method 1 over rows of 2048 bytes (a token row of
 *             D' = 1024 bf16 channels): a block owns tiles of 32768 / depth
 *             rows and reads each tile in column slabs of `depth` bytes, one
 *             slab per stage, as a product stepping over the channels reads
 *             its token rows; depth in {64, 128, 256, 512, 2048} (2048 =
 *             contiguous); `bytes` a multiple of one tile (32768 / depth
 *             rows of 2048 bytes);
 *   method 4: method 3 with non-temporal loads.
 *   sink      device, >= blocks uint32: written only if an impossible value
 *             turns up, so the loads cannot be optimised away. */
int kvlr_probe_read(const void* src, size_t bytes, int method, int blocks, int depth,
                    uint32_t* sink, void* stream);

/* Dense bf16 MFMA issue rate: `blocks` blocks of 256 threads, each wave runs
 * `iters` rounds of 8 independent MFMAs on register operands.
 *   shape 0: v_mfma_f32_16x16x32_bf16 (16 384 flops each);
 *   shape 1: v_mfma_f32_32x32x16_bf16 (32 768 flops each).
 *   sink      device, >= blocks floats, written only for an impossible value.
 * Flops per launch = blocks * 4 * iters * 8 * flops per MFMA. */
int kvlr_probe_mfma(int shape, int64_t iters, int blocks, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVLR_PROBE_H */
