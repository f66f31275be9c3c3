/* zsprobe.h -- C ABI of libzsprobe: HBM bandwidth probes on gfx950.
 *
 * Measurement tools only (not part of the optimizer step): plain stream
 * kernels that read and write HBM in the read:write ratios of the step's
 * workloads, so that the step's achieved bandwidth can be set against what
 * the same mix reaches with no arithmetic at all.  The ratios follow the
 * step's bytes per element, 2P gradient bytes + 12 read + 14 written
 * ([DP-III] §(四) steps 2-4 for one shard of P ranks):
 *   P = 64: 140 read : 14 written = 10 : 1      (ZSP_MIX_10_1, 154 B/elem)
 *   P = 16:  44 read : 14 written = 22 : 7      (ZSP_MIX_22_7,  58 B/elem)
 *   P = 8:   28 read : 14 written =  2 : 1      (ZSP_MIX_2_1,   42 B/elem)
 * plus pure reads (ZSP_READ8: eight read streams) and a copy (ZSP_COPY).
 */
#ifndef ZSPROBE_H
#define ZSPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Interleaved kernels (ZSP_READ8 .. ZSP_MIX_10_1): grid-stride, each unit's
 * loads then its stores.  Phased kernels (ZSP_PHASED_*): one workgroup per
 * CU over chunks of 16 x 256 vectors per stream, all read streams of a chunk
 * first (16 loads in flight per stream), then all its writes -- the phase
 * separation of the step's whole-chunk kernels. */
enum {
  ZSP_READ8 = 0, ZSP_COPY = 1, ZSP_MIX_2_1 = 2, ZSP_MIX_22_7 = 3, ZSP_MIX_10_1 = 4,
  ZSP_PHASED_READ8 = 5, ZSP_PHASED_COPY = 6, ZSP_PHASED_2_1 = 7, ZSP_PHASED_22_7 = 8,
  ZSP_PHASED_10_1 = 9,
  /* more pure-read shapes: read streams x 16-byte loads in flight per lane
   * and stream (ZSP_READ8 is 8 x 4) */
  ZSP_READ1_U16 = 10, ZSP_READ2_U8 = 11, ZSP_READ4_U8 = 12, ZSP_READ8_U8 = 13, ZSP_READ1_U32 = 14
};

/* Read and write streams of a mix; 0 on success, 1 on a bad mix. */
int32_t zsp_streams(int32_t mix, int32_t* nread, int32_t* nwrite);

/* One launch of the mix's stream kernel on `stream` (hipStream_t):
 * stream r (r < nread) is src + r * stream_bytes, stream w (w < nwrite) is
 * dst + w * stream_bytes, each nvec 16-byte vectors (stream_bytes >= 16 *
 * nvec, so src must hold nread * stream_bytes bytes and dst nwrite *
 * stream_bytes).  grid workgroups of 256 lanes.  sink: 4 KiB of device
 * memory that a read-only probe may write to keep its loads alive.  Every
 * read stream is read once and every write stream written once.  Returns 0,
 * 1 on bad arguments (nothing launched), 2 if the launch failed. */
int32_t zsp_stream(int32_t mix, const void* src, void* dst, int64_t stream_bytes, int64_t nvec,
                   int32_t grid, void* sink, void* stream);

/* The fused step's read phase alone, in its own pattern: p <= 64 rank
 * buffers of 16-bit values (fp16), each at least `elems` elements; the
 * whole chunks of 57,344 elements (elems / 57,344 of them) go round-robin
 * over `grid` workgroups of 256 lanes; per chunk, rank by rank, a first
 * load per lane alone, then the other 27 back to back, summed in fp32 in
 * rank order ([DP-III] §(四) step 2).  Reads 2 * p * 57,344 bytes per
 * chunk and writes nothing but, never in practice, `sink` (4 KiB of device
 * memory).  Returns 0, 1 on bad arguments (nothing launched), 2 if the
 * launch failed. */
int32_t zsp_step_reads(const void* const* ranks, int32_t p, int64_t elems, int32_t grid,
                       void* sink, void* stream);

/* The same read phase paced like the library's whole-chunk kernels: the
 * chunks go in rounds of one per workgroup, and every `pace_rounds` rounds
 * (>= 1) each workgroup passes the library's soft barrier (it waits until
 * 90% of the grid has arrived, at most 200 us).  Same arguments and
 * returns as zsp_step_reads; pace_rounds < 1 returns 1. */
int32_t zsp_step_reads_paced(const void* const* ranks, int32_t p, int64_t elems, int32_t grid,
                             int32_t pace_rounds, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZSPROBE_H */
