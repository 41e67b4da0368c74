/*
 * paprobe.h -- C ABI of libpaprobe.so: bandwidth ceilings of the GPU, for
 * the benchmark.  Not part of the decode library (libpagedattn.so); it
 * measures what the memory system delivers to the access patterns the
 * decode kernels use, so that a kernel's rate can be stated as a fraction
 * of that as well as of the nominal HBM peak.
 *
 * Both calls launch one kernel, asynchronously on `stream` (a hipStream_t
 * as void*, NULL = default), and return 0, -1 for bad arguments (nothing
 * launched) or -5 for a HIP launch error.  Pointers are device memory the
 * caller owns, 16-byte aligned.  `sink` receives waves * 64 uint32 words
 * (a fold of what each lane read, so that no load can be dropped).
 * `depth` (1, 2 or 4) is the number of 4 KiB chunks or blocks each wave
 * has in flight; `nontemporal` != 0 streams the loads past the caches, as
 * the decode kernels do when every block is read once.
 */
#ifndef PAPROBE_H
#define PAPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read every byte of buf[0, bytes) once (bytes a positive multiple of
 * 4096): wave w reads the 4 KiB chunks w, w + waves, w + 2 * waves, ... */
int32_t probe_stream_read(const void *buf, int64_t bytes, void *sink, int32_t waves,
                          int32_t depth, int32_t nontemporal, void *stream);

/* Read the 4 KiB blocks pool + block_ids[i] * 4096, i < num_ids (device
 * int32 list): wave w reads entries [num_ids * w / waves, num_ids * (w + 1)
 * / waves) in order.  Ids outside [0, pool_blocks) read block 0. */
int32_t probe_block_gather(const void *pool, int64_t pool_blocks, const int32_t *block_ids,
                           int64_t num_ids, void *sink, int32_t waves, int32_t depth,
                           int32_t nontemporal, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAPROBE_H */
