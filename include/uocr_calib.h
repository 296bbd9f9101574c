/*
 * uocr_calib.h -- measurement kernels of libuocr.so (gfx950).
 *
 * These calls are not part of the method: they give the denominators the
 * decode kernels are measured against on the machine at hand, so that the
 * figures quoted for them can be reproduced from the library alone.
 *   - uocr_calib_read: the read bandwidth a plain streaming kernel reaches
 *     over a large buffer, with ordinary or nontemporal 16-byte loads (the
 *     "attainable" HBM rate next to the published 8 TB/s peak);
 *   - uocr_calib_empty: a launch that does nothing, the floor of any kernel
 *     in a HIP graph at a given grid;
 *   - uocr_calib_pull: each of `groups` workgroups reads its own contiguous
 *     run of bytes_per_group bytes and nothing else, the time one compute
 *     unit needs to bring in a given amount of data when only some units of
 *     the chip are busy (the floor of a step whose units each read that much);
 *   - uocr_calib_start: when each workgroup of a launch starts;
 *   - uocr_calib_exchange: what merging several workgroups' partial states
 *     inside one kernel costs (instead of a second kernel);
 *   - uocr_phase_stamps: when each phase of the fused SR-SWA step ends, per
 *     workgroup (a separately built library records them).
 *
 * Conventions as in uocr.h: device pointers, the caller owns every buffer,
 * stream is a hipStream_t passed as void* (NULL = default stream), the call
 * returns once the work is enqueued, 0 on success and a negative uocr_status
 * on failure.  src must be 16-byte aligned;
 * `sink` receives at most one word per workgroup and only if the data hash to
 * a value no real buffer produces, so that the loads cannot be dropped; it
 * needs room for one uint32 per workgroup.
 */
#ifndef UOCR_CALIB_H
#define UOCR_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, > 0) from src with one grid of 4096
 * workgroups x 256 threads, each streaming its own contiguous 1/4096 of the
 * buffer; nontemporal != 0 uses nontemporal loads.  sink: 4096 uint32.     */
int uocr_calib_read(const void* src, size_t bytes, int32_t nontemporal, uint32_t* sink, void* stream);

/* An empty kernel of `groups` workgroups of `threads` threads
 * (1 <= groups <= 2^20, threads in {64, 128, 256, 512, 1024}).             */
int uocr_calib_empty(int32_t groups, int32_t threads, void* stream);

/* Workgroup g (0 <= g < groups) reads bytes [g * bytes_per_group,
 * (g + 1) * bytes_per_group) of src with `threads` threads, 16 bytes per
 * load, up to 8 loads per thread in flight.  bytes_per_group a multiple of
 * 16 in [16, 2^26]; groups and threads as for uocr_calib_empty; src must hold
 * groups * bytes_per_group bytes.  sink: `groups` uint32.                   */
int uocr_calib_pull(const void* src, size_t bytes_per_group, int32_t groups, int32_t threads,
                    int32_t nontemporal, uint32_t* sink, void* stream);

/* Thread 0 of every workgroup of a grid of `groups` x `threads` stores the
 * device's constant-rate real-time counter (100 MHz on MI355X) as the
 * workgroup starts: stamps[g] for workgroup g (`groups` uint64).  Workgroups
 * are dealt to the XCDs in turn (g mod 8), so the stamps show how the start
 * of a launch spreads over the chip.                                        */
int uocr_calib_start(int32_t groups, int32_t threads, uint64_t* stamps, void* stream);

/* The cost of merging partial states inside one kernel: `units` x `split`
 * workgroups of 256 threads; each writes a partial of 130 floats to
 * part[(unit * split + s) * 130 ...] and adds one to count[unit]; the
 * workgroup that arrives last (no workgroup ever waits) sums its unit's
 * partials into out[unit * 130 ...] and sets count[unit] back to 0.
 * mode 0: plain stores and loads around __threadfence(); mode 1: agent-scope
 * relaxed atomic stores and loads of the partials; mode 2: the count alone.
 * count must start at 0 (it is left at 0); part holds units * split * 130
 * floats, out units * 130.  1 <= units * split <= 2^20.                     */
int uocr_calib_exchange(int32_t mode, int32_t units, int32_t split, float* part, int32_t* count, float* out,
                        void* stream);

/* Phase stamps of the fused SR-SWA step (uocr_srswa_step): where the time of
 * one launch goes, workgroup by workgroup.  Only the library built with
 * UOCR_PHASE_STAMPS (libuocr_stamps.so, the same sources) records them; in
 * libuocr.so this call returns UOCR_ERR_UNSUPPORTED and the step kernels hold
 * no stamping code.  Copies the stamps of units [0, units) left by the
 * latest uocr_srswa_step launches (each launch overwrites its units' rows)
 * into host memory dst[units][64] (uint64) after the work queued on `stream`
 * is done, and returns when the copy is complete; 1 <= units <= 4096.
 * Each value is the device's 100 MHz real-time counter (common to all XCDs)
 * when the phase ended, recorded by thread 0 or by lane 0 of wave w:
 *   0 the workgroup starts            5 q_idx = P^T q formed
 *   6 the first batch of block keys scored   1 every block score in LDS
 *   2 wave 0 has routed the unit and published the selection
 *  32+w wave w (w >= 1) has the selection (all waves stamp 2 or 32+w at the
 *     same point, after seeing it published)
 *  16+w wave w (w >= 1) has attended over its share of the window
 *  48+w wave w has attended over its live blocks
 *  56+w wave w has left its share of the merge in LDS
 *   7 the workgroup merge's barrier has passed
 *   4 the output row is written
 *   9-13 inside the routing of wave 0 (one-wave path only): 9 the scores'
 *     maximum taken, 10 the threshold of the candidate set A found, 11 A
 *     compacted (and its rank keys and the entmax candidates in LDS),
 *     12 ranks counted, 13 the entmax threshold found
 *   3 (not a time) the XCD the workgroup ran on (hardware register XCC_ID)
 *   8 (not a time) hardware register HW_ID of wave 0: bits 8-11 the compute
 *     unit, 12 the shader array, 13-15 the shader engine within the XCD
 * Slots 16+w and 48+w are taken after the wave's loads have all arrived
 * (the stamping build waits for them there).  Other slots are unspecified. */
int uocr_phase_stamps(uint64_t* dst, int32_t units, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* UOCR_CALIB_H */
