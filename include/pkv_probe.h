/*
 * pkv_probe.h -- C ABI of libpkv_probe: read-bandwidth probes that measure
 * the HBM ceiling on the part the attention kernels run on (gfx950).  They
 * are measurement aids beside libpkv, not part of the decode path.
 *
 * The decode kernels of libpkv move whole K and V tiles (block * head_dim
 * bytes, 2 KiB at block 32 and head_dim 64) from places the block table
 * chooses (page "GPT-OSS-120B giga-kernel decode", section "KV-cache layout
 * (per-buffer, HMA-preserving)").  The probes read a device buffer either as
 * one stream or as whole tiles in a scrambled order, with plain or
 * non-temporal loads, and nothing else: their rate is what a kernel with the
 * same traffic and no arithmetic reaches.
 *
 * Conventions:
 *   - `src` and `sink` are DEVICE pointers owned by the caller; `src` is
 *     16-byte aligned; `sink` holds at least `grid` uint32 words: workgroup i
 *     stores into sink[i] the XOR of every 32-bit word it read, so the XOR of
 *     sink[0 .. grid) is the XOR of everything the launch read.
 *   - `stream` is a hipStream_t passed as void*; the launch is asynchronous.
 *   - Each call returns the number of bytes its launch reads (>= 0), or a
 *     negative status; on a negative status nothing was enqueued, except
 *     PKV_PROBE_ERR_HIP (the launch itself failed).
 *   - Nothing is allocated and no state is kept.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_PROBE_ERR_ARG (-1) /* null or misaligned pointer, bad size, grid or tile size */
#define PKV_PROBE_ERR_HIP (-4) /* the kernel launch failed */

/* Reads every 16-byte word of src[0, bytes) once.  bytes > 0, a multiple of
 * 16; grid in [1, 2^20] workgroups of 256 threads; nontemporal != 0 uses
 * non-temporal loads.  Returns bytes. */
int64_t pkv_probe_stream_read(const void* src, int64_t bytes, int32_t grid, int32_t nontemporal,
                              uint32_t* sink, void* stream);

/* Bytes that pkv_probe_tile_read reads for these sizes: the largest number of
 * whole tiles, at most bytes / tile_bytes, that grid * 4 waves split evenly
 * in groups of 16 KiB per wave.  bytes and tile_bytes are powers of two,
 * 1024 <= tile_bytes <= 16384, tile_bytes <= bytes.  Host only. */
int64_t pkv_probe_tile_read_bytes(int64_t bytes, int32_t tile_bytes, int32_t grid);

/* Reads that many distinct whole tiles of src[0, bytes), each once, in an
 * order given by a bijective scramble of the tile index (consecutive tiles of
 * one wave land far apart).  Arguments as above.  Returns the bytes read. */
int64_t pkv_probe_tile_read(const void* src, int64_t bytes, int32_t tile_bytes, int32_t grid,
                            int32_t nontemporal, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
