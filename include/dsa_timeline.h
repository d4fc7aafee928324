/*
 * dsa_timeline.h - phase stamps of the measurement build of the library.
 *
 * Exported only by libdsa_timeline.so, which is libdsa.so compiled with -DDSA_TIMELINE
 * (`python -m sparse_indexed_attention_amd.build --timeline`).  libdsa.so exports neither
 * function and its kernels record nothing.
 *
 * In the measurement build, thread 0 of every workgroup of the indexer, attention and
 * combine kernels writes the 100 MHz constant clock (s_memrealtime, 10 ns ticks) at the end
 * of each phase of its work into the registered buffer:
 *
 *   uint64 stamps[kernel][workgroup][slot],  kernel 0 = indexer, 1 = attention, 2 = combine,
 *                                            workgroup < 4096 (flattened grid index),
 *                                            slot < 32.
 *
 * Indexer slots: 0 start, 1 split scored, 2 candidates stored, 3 arrival counted, and for the
 * workgroup that merges its query: 4 headers read, 5 list staged, 6 K-th key found, 7 output
 * written; slot 14 holds (query << 16 | split) and slot 15 is 1 for the merging workgroup;
 * slot 16 the split's candidate cut chosen, 17 its candidate and header stores issued (slot 2
 * ends their drain), 18 the merge's bin of the K-th key found.  Slots 8-10 hold wave 0's
 * shader-clock cycles waiting for loads and computing in the scoring loop and its steps, 11 and
 * 12 the shader clock (s_memtime) at the start and after scoring, 13 the scoring loop's start.
 * Attention slots: 0 start, 1 pool rows resolved, 2 first tile pair and query rows landed, 3 query
 * fragments in registers, 4 last tile done, 5 outputs or partials written; slot 14 holds
 * (query << 16 | head group << 8 | slice), slots 8-10 the tile loop's wait and compute cycles
 * and steps, 11 and 12 the shader clock at the start and after the last tile, 19 (the 128-head
 * kernel) the loop's cycles issuing later tiles' loads.  Combine slots:
 * 0 start, 5 written.
 *
 * A slot a workgroup never reaches keeps whatever the caller left there: clear the buffer
 * before the call whose stamps you want.  Stamps are plain stores, visible once the stream
 * has synchronized.  Multi-query (prefill) indexer tiles record no stamps.
 */
#ifndef DSA_TIMELINE_H_
#define DSA_TIMELINE_H_

#include <stddef.h>

#include "dsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes the stamp buffer must hold: 3 kernels x 4096 workgroups x 32 slots x 8. */
size_t dsa_timeline_bytes(void);

/* Registers `buf` (device memory of at least dsa_timeline_bytes(), 16-byte aligned; owned by
 * the caller, who must keep it alive while calls run) as the stamp buffer of every later
 * call in this process; NULL stops recording.  Returns DSA_ERR_WORKSPACE if `bytes` is too
 * small, DSA_ERR_ALIGN if misaligned, else DSA_OK.  Not thread-safe against concurrent calls. */
dsa_status dsa_timeline_register(void* buf, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* DSA_TIMELINE_H_ */
