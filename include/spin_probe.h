/*
 * A measurement helper beside the SPIN library, not a stage of the method:
 * an HBM read probe over KV pages with the access pattern of the fp8 score
 * kernel (spin_sparse_index_score).  It reads whole 8,192-byte pages (64
 * slots x 128 fp8 bytes) with the same 16-byte non-temporal loads, two pages
 * in flight per wave, each of SPIN_READ_PROBE_WAVES waves taking a contiguous
 * run of the list, and folds the bytes into a checksum so that no load is
 * dead.  Timed beside the score kernel on the same pages, it gives what a
 * plain read of those pages reaches on the part, the practical ceiling the
 * score kernel's bandwidth is compared with.
 */
#ifndef SPIN_PROBE_H_
#define SPIN_PROBE_H_

#include <stdint.h>
#include "spin.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SPIN_READ_PROBE_WAVES 2048
#define SPIN_READ_PROBE_SINK_WORDS (SPIN_READ_PROBE_WAVES * 64)

/*
 * Reads pages page_ids[0 .. n_ids) of k_pages (device, n_pages pages of
 * 8,192 bytes; an id outside [0, n_pages) reads page 0) on `stream`, and
 * writes one checksum word per lane of every wave into sink (device,
 * SPIN_READ_PROBE_SINK_WORDS uint32, caller-owned; its contents carry no
 * meaning).  n_ids = 0 launches nothing.  NULL buffers: SPIN_E_NULL;
 * n_ids < 0 or n_pages < 1: SPIN_E_SHAPE.
 */
spin_status spin_read_pages(const void* k_pages, int64_t n_pages, const int32_t* page_ids,
                            int32_t n_ids, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPIN_PROBE_H_ */
