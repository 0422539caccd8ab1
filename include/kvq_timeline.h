/* Decode timeline, a profiling variant of the library (libkvq_timeline.so, built by
 * `python kv_cache_bit_fwht_amd/build.py --timeline`; the default libkvq.so does not
 * export it).
 *
 * In that build, lane 0 of every wavefront of the MFMA decode (kvq_decode_attn on the
 * head_dim-256 MFMA path, and the codec-map kernel) records the GPU's 100 MHz
 * s_memrealtime clock at fixed points of its work: the per-step hand-out, the in-kernel
 * merge of the split-K partials ([E22L] "Can 4-bit keys and 2-bit values hit a
 * 1M-token memory budget?", What I tested: the 64K-token decode whose fixed costs this
 * shows).  Stamps are kept for blocks b = x + X*(y + Y*z) < 4096 of the grid, 8
 * wavefronts each, 16 slots per wavefront; a slot a wavefront did not reach is 0:
 *   0 entry, 1 query prologue done, 2 after the prologue barrier, 3 loop end,
 *   4 wavefront reduced, 5 after the block barrier, 6 partial stores issued,
 *   7 partial stores complete, 8 block counted, 9 last block: merge tables in,
 *   10 merge end (outputs issued); 11..15 unused.
 *
 * kvq_timeline_read copies the first `count` stamps (laid out [block][wave][slot],
 * unsigned 64-bit) to host memory dst, then clears them all.  Synchronous (it waits for
 * the device); call it after the decode to be read has finished.  Returns KVQ_ERR_ARG
 * for a null dst or count > 4096*8*16, KVQ_ERR_HIP on a runtime error. */
#ifndef KVQ_TIMELINE_H
#define KVQ_TIMELINE_H
#include <stddef.h>
#include "kvq.h"
#ifdef __cplusplus
extern "C" {
#endif
kvq_status kvq_timeline_read(unsigned long long* dst, size_t count);
#ifdef __cplusplus
}
#endif
#endif
