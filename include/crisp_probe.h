/*
 * crisp_probe.h -- attainable-peak probe of libcrisp_probe.so (gfx950).
 *
 * The benchmark reports the sparse attention kernel against the MI355X
 * published dense bf16 MFMA peak and, beside it, against the rate this same
 * GPU sustains on nothing but MFMAs under the same clock and power limits.
 * This library holds only that probe; it takes no part in the attention path.
 */
#ifndef CRISP_PROBE_H
#define CRISP_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue one launch of a bf16 MFMA loop: `blocks` work-groups of 512 threads
 * (8 waves, two per SIMD, the occupancy of the attention kernel), each wave
 * issuing `iters` x 4 independent v_mfma_f32_32x32x16_bf16 (32768 flop each).
 * Total work = blocks * 8 * iters * 4 * 32768 flop; the caller times the
 * launch (events on `stream`, NULL = default stream).
 *   out    device buffer of blocks * 512 floats (written, so the loop is kept)
 *   blocks 1 .. 65536;  iters 1 .. 2^26
 * Returns 0, -1 for an invalid argument (nothing launched), -4 when the launch
 * fails.  Allocates nothing and never synchronises the host.
 */
int crisp_probe_mfma_bf16(float *out, int blocks, int iters, void *stream);

/*
 * The same loop, same work per iteration, but each wave's operands cycle over
 * eight pseudo-random bf16 fragment pairs instead of staying constant, so the
 * multipliers switch as they do on real tiles.  `iters` must be even
 * (2 .. 2^26); total work = blocks * 8 * iters * 4 * 32768 flop, as above.
 * Same returns, same guarantees.
 */
int crisp_probe_mfma_bf16_data(float *out, int blocks, int iters, void *stream);

#ifdef __cplusplus
}
#endif
#endif
