/*
 * nvfp4mi_probe.h - measurement entry points of libnvfp4mi.so.
 *
 * Not part of the quantization method: these calls exist so that a benchmark
 * can report the path's kernels against what the device itself achieves (HBM
 * read, write and copy ceilings) and against the work its sweep executes
 * (evaluated codes per block, lane utilisation).  Conventions, status codes
 * and validation are those of nvfp4mi.h: device pointers owned by the
 * caller, stream as void*, host-side validation before any HIP call.
 */
#ifndef NVFP4MI_PROBE_H
#define NVFP4MI_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` bytes: workgroup w of `workgroups` (0 = 512)
 * reads the w-th contiguous share, 16 bytes per lane (1 KiB contiguous per
 * wave instruction), non-temporal loads, eight in flight per lane.  The data
 * are xor-folded; the fold is stored to sink[0] only if it equals 0x9E3779B9
 * (never for zero-filled buffers), which keeps the loads from being
 * optimised away.
 * buf: 16-byte aligned, bytes a multiple of 16.  sink: device uint32[1].
 * Errors: NULL_ARG, BAD_SHAPE (bytes % 16), BAD_INPUT (workgroups < 0 or
 *         > 65535), MISALIGNED, HIP.
 */
int nvfp4_probe_read(const void* buf, size_t bytes, void* sink, int workgroups, void* stream);

/*
 * Streaming write: every 32-bit word of buf[0..bytes) is set to `value`
 * (16-byte stores, grid-stride over `workgroups` workgroups, 0 = 512).
 * buf: 16-byte aligned, bytes a multiple of 16.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_INPUT, MISALIGNED, HIP.
 */
int nvfp4_probe_write(void* buf, size_t bytes, uint32_t value, int workgroups, void* stream);

/*
 * Streaming copy dst[0..bytes) = src[0..bytes): contiguous share per
 * workgroup (0 = 512), non-temporal 16-byte loads, plain 16-byte stores, four
 * in flight per lane.  src and dst must not overlap (BAD_INPUT).
 * Errors: NULL_ARG, BAD_SHAPE, BAD_INPUT, MISALIGNED, HIP.
 */
int nvfp4_probe_copy(const void* src, void* dst, size_t bytes, int workgroups, void* stream);

/*
 * nvfp4_scale_sweep (uncapped) that also counts the work of its search:
 * the same kernel body and the same outputs bit for bit, built with counters
 * in scalar registers.  Adds to the device uint64 stats[6]:
 *   [0] code evaluations whose cost the search used (code 0, the block's
 *       max-based code, and every window step of a block still searching),
 *       summed over blocks;
 *   [1] wave steps (each one evaluation slot for each of 64 lanes, whether
 *       the lane's block is still searching or not);
 *   [2] wave steps that evaluated the full quadratic form;
 *   [3] wave steps that evaluated the diagonal screen;
 *   [4] blocks (valid lanes);
 *   [5] waves.
 * stats must be zeroed by the caller before the first call it should count
 * (8-byte aligned).  No costs are written.
 * Other arguments and errors: as nvfp4_scale_sweep, plus NULL_ARG for stats.
 */
int nvfp4_scale_sweep_stats(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw,
                            const float* H, const float* scale2, uint8_t* packed,
                            uint8_t* codes, uint64_t* stats, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MI_PROBE_H */
