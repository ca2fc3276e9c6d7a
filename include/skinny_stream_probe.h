/* Read-stream probe: the rate at which a plain streaming kernel reads HBM on this
 * device, a measured reference beside which the GEMV's weight stream is judged
 * (the 8 TB/s peak is a datasheet figure). It is not an upper bound: a GEMV plan
 * tuned per shape can read as fast or faster. Measurement only; not part of the
 * GEMM.
 *
 * The measured-ceiling comparison follows vLLM PR #65306 (SM90 skinny GEMM plans),
 * section Validation, which rates the kernels by weight bytes per second against
 * the memory system; the probe gives the same rate for a kernel that does nothing
 * but read.
 *
 * Library: libskinny_stream_probe.so (built next to libskinny_gemm_bf16.so).
 */
#ifndef SKINNY_STREAM_PROBE_H
#define SKINNY_STREAM_PROBE_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of sink words a call with this grid writes: grid_blocks * 256. */
size_t skinny_probe_sink_words(int grid_blocks);

/* Reads `bytes` bytes at device pointer `buf` once, with 16-byte buffer loads
 * (non-temporal hint if `nontemporal` != 0), in one kernel launch on `stream`.
 * The buffer is read in 32 KiB chunks, chunk c by block c mod `grid_blocks` (256
 * threads each), each block loading its next chunk while it consumes the current
 * one. Every thread XORs the 32-bit words it read into one word and stores it to
 * sink[b * 256 + thread], so the XOR of all skinny_probe_sink_words(grid_blocks)
 * sink words equals the XOR of all 32-bit words of the buffer (the check that
 * every byte was read).
 *
 * Arguments: `buf` 16-byte aligned, `bytes` a multiple of 16 (0 allowed: the sink
 * is written with zeros), `grid_blocks` in 1..65536, `sink` a 4-byte aligned
 * device buffer of skinny_probe_sink_words(grid_blocks) uint32 words that does not
 * overlap `buf`. The caller owns both buffers; nothing is allocated.
 * Returns 0, -1 (invalid argument: nothing enqueued) or -4 (launch failed). */
int skinny_probe_read(const void *buf, size_t bytes, int nontemporal, int grid_blocks,
                      uint32_t *sink, hipStream_t stream);

/* Sink words skinny_probe_read_tiles writes for this buffer size and shape: one
 * per wave, ceil(bytes / tile) * threads / 64 with tile = threads / 64 * loads KiB;
 * 0 for a shape it refuses. */
size_t skinny_probe_tiles_sink_words(size_t bytes, int loads, int threads);

/* Reads `bytes` bytes at `buf` once, one block of `threads` threads per tile of
 * threads / 64 * `loads` KiB, with the load schedule of the GEMV's one-block-per-
 * tile plans at M = 1: each wave issues `loads` 16-byte-per-lane loads over
 * `loads` consecutive KiB before consuming any (non-temporal hint if
 * `nontemporal` != 0). Each wave stores the XOR of the 32-bit words it read to its
 * own sink word, so the XOR of all skinny_probe_tiles_sink_words() words equals
 * the XOR of the buffer's words. A ragged last tile reads zeros past the end.
 *
 * Arguments: `loads` 2, 4, 8 or 16; `threads` a multiple of 64 in 64..1024;
 * `buf` 16-byte aligned and non-null; `bytes` a positive multiple of 16; `sink`
 * 4-byte aligned, skinny_probe_tiles_sink_words() words, not overlapping `buf`.
 * Returns 0, -1 (invalid argument: nothing enqueued) or -4 (launch failed). */
int skinny_probe_read_tiles(const void *buf, size_t bytes, int nontemporal, int loads, int threads,
                            uint32_t *sink, hipStream_t stream);

/* Launches a kernel that does nothing, `grid_blocks` (1..2^24) blocks of `threads`
 * (a multiple of 64 in 64..1024): the per-launch floor under graph replay.
 * Returns 0, -1 (invalid argument) or -4 (launch failed). */
int skinny_probe_empty(int grid_blocks, int threads, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_STREAM_PROBE_H */
