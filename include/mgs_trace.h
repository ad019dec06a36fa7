/* Tile-timeline diagnostic of the dim0-family kernels.
 *
 * These calls exist only in libmgs_trace.so, a build of the same sources as
 * libmgs.so with MGS_TILE_TRACE defined; libmgs.so does not export them. The
 * trace build runs the same kernels and additionally records, per tile item,
 * when the item started, found its tile, finished its loads and column
 * maxima, finished the reduction across the workgroup and issued its stores,
 * with the workgroup's compute-unit placement and the tile's class, rows,
 * group and strip. It is for measuring where a launch's time goes, not for
 * production use: the recording costs a few stores per tile.
 *
 * The record is one device-global array of mgs_tile_trace_capacity() items
 * of eight 64-bit words, on the current device. Each launch overwrites the
 * items it runs; items past the capacity are not recorded. Both calls below
 * synchronise the whole device and return a hipError_t code (0 = success).
 */
#ifndef MGS_TRACE_H
#define MGS_TRACE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of tile items the record holds. */
int mgs_tile_trace_capacity(void);

/* Sets every word of the record to zero (synchronous). */
int mgs_tile_trace_clear(void);

/* Waits for the device, then copies the first `bytes` bytes of the record to
 * host memory at `dst` (caller-owned, at least `bytes` long). bytes must not
 * exceed mgs_tile_trace_capacity() * 64; returns hipErrorInvalidValue
 * otherwise or when dst is NULL. */
int mgs_tile_trace_read(void* dst, int64_t bytes);

/* Enqueues on `stream` (a hipStream_t; NULL = the default stream) a
 * one-thread kernel that writes the 100 MHz device wall clock, the clock of
 * the record's stamps, to the 8-byte-aligned device address `dst`
 * (caller-owned). Stamps right before and after a launch on the same stream
 * bound when the launch started and ended. Returns hipErrorInvalidValue for
 * a NULL or misaligned dst, else the launch's error code. */
int mgs_tile_trace_stamp(void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MGS_TRACE_H */
