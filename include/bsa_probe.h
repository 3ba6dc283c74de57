/*
 * bsa_probe.h -- HBM read-rate probe of libbsa.so (measurement only; no part
 * of the decode step).
 *
 * The decode step's kernels are held against the rate at which one launch can
 * read the same byte pattern: long contiguous runs (the block scan's 9 KiB key
 * records) or 32 KiB tiles at scattered offsets of a large cache (the
 * attention's selected key and value blocks, Jet-QSparse abstract: contiguous
 * tile loads of the chosen 128-token blocks). The probe reads such a pattern
 * and folds the bytes into one word per thread; nothing is written unless that
 * word equals a fixed constant no workload here produces.
 */
#ifndef BSA_PROBE_H_
#define BSA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read n_tiles tiles of tile_bytes (a multiple of 16; of 1024 for mode 1)
 * from device memory buf (buf_bytes long). Tile t starts at byte tile_off[t]
 * (device int64 [n_tiles], 16-byte aligned, each tile inside buf: the caller
 * checks this, the library cannot read the offsets), or at t * tile_bytes when
 * tile_off is NULL (then n_tiles * tile_bytes <= buf_bytes is checked).
 * One work-group of 256 threads reads tiles_per_group consecutive tiles.
 * mode 0: 16-byte vector loads into registers, depth (1, 2, 4 or 8) loads in
 *         flight per thread;
 * mode 1: gfx950 global-to-LDS loads of 1 KiB per wave instruction, depth
 *         (4, 8, 16 or 32) of them in flight per wave;
 * mode 2: short tiles (tile_bytes divides 4096: the token-mode attention's
 *         256-byte key and value rows, JSSA Figure 6), tiles_per_group <=
 *         1024: the group's offsets are staged in LDS, then tile_bytes / 16
 *         threads per tile, one 16-byte load each, depth (1, 2, 4 or 8)
 *         tiles in flight per thread.
 * sink: device uint32 [groups * 256] (written only in the case above).
 * Asynchronous on stream; returns 0, -1 (bad argument), -2 (unsupported mode
 * or depth) or -3 (launch failed). */
int bsa_probe_read(const void* buf, int64_t buf_bytes, const int64_t* tile_off, int64_t n_tiles,
                   int64_t tile_bytes, int32_t tiles_per_group, int32_t mode, int32_t depth,
                   uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_PROBE_H_ */
