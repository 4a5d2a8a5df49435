/*
 * fm_probe.h - memory-system probes that the benchmark records beside the
 * attention kernels' figures (libfm_probe.so).  They compute nothing of the
 * draft step: each reads bytes and folds them into a small sink so the reads
 * cannot be dropped.  They give the rate at which this GPU delivers
 *   (1) a plain streaming read of one large buffer, and
 *   (2) exactly the K/V tiles a paged cross-attention call reads, in the same
 *       order and with the same split over resident wavefronts, with no
 *       arithmetic,
 * so that an HBM-bound kernel can be placed against what the memory system
 * delivers on the same box, next to the published 8 TB/s.  Every load is a
 * whole-line 16-byte-per-lane load with the nontemporal hint (the kind the
 * attention kernel issues). 
 *
 * Conventions: DEVICE pointers are caller-owned device memory; calls are
 * asynchronous on ``stream`` and return 0 (or a negative fm_status value of
 * fm.h on a bad argument or launch failure, nothing enqueued on a bad
 * argument).
 */
#ifndef FM_PROBE_H
#define FM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of ``buf`` (DEVICE, 16-byte aligned): n_waves wavefronts of
 * 256-thread workgroups each read an equal contiguous share, 1 KB per load
 * instruction, four 8 KB blocks in flight.  Only whole 8 KB blocks of each
 * share are read: the bytes read are n_waves * floor(bytes / n_waves / 8192) *
 * 8192, returned through *bytes_read (HOST).  sink DEVICE uint32[n_waves * 64].
 * n_waves a positive multiple of 4. */
int fm_probe_stream_read(const void* buf, size_t bytes, int32_t n_waves, uint32_t* sink, size_t* bytes_read,
                         hipStream_t stream);

/* Gather of n_tiles K/V tile pairs: tile i is tile_bytes contiguous bytes at
 * k + tile_off[i] and as many at v + tile_off[i] (tile_off DEVICE int64
 * [n_tiles], byte offsets, 16-byte aligned; tile_bytes 1024, 2048, 4096 or
 * 8192, -2 otherwise).  The tiles are cut into n_waves equal contiguous ranges,
 * one per wavefront (the attention plan's equal shares), each read in order
 * the way the attention kernel reads them: direct-to-LDS loads of 1 KB per
 * instruction, two tile pairs in flight, each read back from LDS.
 * sink DEVICE uint32[n_waves * 64].  n_waves a positive multiple of 4. */
int fm_probe_tile_gather(const void* k, const void* v, const int64_t* tile_off, int64_t n_tiles, int32_t tile_bytes,
                         int32_t n_waves, uint32_t* sink, hipStream_t stream);

/* fm_probe_tile_gather that also times every wave: wave_rec DEVICE uint64
 * [n_waves][4] receives, for wave w, its start and end on the GPU's constant
 * 100 MHz clock (s_memrealtime), the XCD it ran on (0-7) and the tiles it
 * read: the XCDs' memory rates with no arithmetic beside them (the attention
 * kernel's own, which fm_paged_cross_attention_timed of fm.h measures, spread
 * wider).  -1 if wave_rec is null. */
int fm_probe_tile_gather_timed(const void* k, const void* v, const int64_t* tile_off, int64_t n_tiles,
                               int32_t tile_bytes, int32_t n_waves, uint32_t* sink, uint64_t* wave_rec,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FM_PROBE_H */
