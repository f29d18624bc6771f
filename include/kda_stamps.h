/*
 * kda_stamps.h -- cycle stamps of the fused prefill, exported only by the
 * profiling build libkda_stamps.so (the same sources as libkda.so, compiled
 * with KDA_CYCLE_STAMPS; it also exports everything kda.h declares).
 *
 * Not part of the method: a measurement aid that says where the fused
 * prefill (kda_fwd_chunked, one persistent work-group per CU) spends its
 * cycles on each side of the record hand-off, the producers that form the
 * chunk records (Gram tiles, the inverse of I + A, W and U) and the state
 * pass that carries S from chunk to chunk.
 *
 * Each wave of the fused kernel adds up shader-clock cycles (s_memtime)
 * between marks at its phase boundaries and stores the sums when it leaves,
 * so after a call the buffer describes that call's last launch (a call with
 * more heads than one launch takes is described by its last batch only).
 * Layout: unsigned 64-bit [KDA_STAMP_WGS][8 waves][KDA_STAMP_SLOTS],
 * work-group = the launch's block index (XCD = index % 8).
 *   slot 29 (KDA_STAMP_ROLE): 1 producer, 2 state-pass owner wave (keeps 16
 *           value columns of S), 3 state-pass staging wave (copies records
 *           into LDS); 0 for a work-group the launch did not use.
 *   slot 30 (KDA_STAMP_COUNT): items (producer) or chunks (state pass).
 *   producer: 0 entry, 1-8 the work of the barrier-separated phases
 *     (1 staging of k/q/g/beta, 2 block scans, 3 factors and K-hat, 4 Gram
 *     tiles with the diagonal inverses and Q-bar, 5 K-bar/V transposes and
 *     the distance-1 inverse blocks, 6 distance 2, 7 distance 3, 8 Tm) and
 *     17-24 the wait at the barrier that ends each of them, 9 W and U to the
 *     record, 10 the hand-off (record visible, ready flag).
 *   owner: 0 loop top, 1 barrier, 2 abort word, 3 U accumulators, 4 U and
 *     Q-bar products issued, 5 K-hat/M/decay operands and the U range,
 *     6 state update, output and stores, 7 snapshots and the next chunk's
 *     range scale and fp16 copy of the state.
 *   staging: 0 loop top, 1 barrier, 2 abort word and progress store,
 *     3 wait for the next record, 4 loads issued, 5 loads completed and
 *     written to LDS.
 * Reading the clock also waits for the wave's outstanding LDS and scalar
 * accesses, so a stamped call runs a few percent slower than libkda.so.
 */
#ifndef KDA_STAMPS_H
#define KDA_STAMPS_H
#include <stddef.h>
#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_STAMP_WGS 256
#define KDA_STAMP_SLOTS 32
#define KDA_STAMP_ROLE 29
#define KDA_STAMP_COUNT 30

/* Copies the stamp buffer (count = KDA_STAMP_WGS * 8 * KDA_STAMP_SLOTS
 * entries) into host memory.  Synchronous with respect to the device (the
 * copy waits for the launches before it).  Returns KDA_OK, KDA_ERR_NULL
 * (host NULL), KDA_ERR_SHAPE (another count) or KDA_ERR_HIP. */
int kda_stamps_read(unsigned long long* host, size_t count);

#ifdef __cplusplus
}
#endif
#endif
