/*
 * retro_probe.h - measured ceilings for the roofline of retro_out_prod.
 *
 * The roofline fractions of the OUT_PROD kernels are quoted against MI355X's
 * published peaks (F32 matrix core 157.3 TFLOP/s, bf16 2.5 PFLOP/s, HBM
 * 8 TB/s). These two probes measure what this GPU reaches on the same
 * instructions with nothing else in the way, so that a kernel can also be
 * placed against a measured ceiling:
 *   - a matrix-core loop with no memory traffic, for F32-input and bf16
 *     MFMA;
 *   - the F32-input matrix-core loop beside vector FMA work on the same
 *     SIMDs, to show whether the two share issue time;
 *   - a device-to-device copy with 16-byte accesses (a STREAM-style copy).
 * They compute nothing of OUT_PROD and are not on its path. All are
 * asynchronous on `stream` (a hipStream_t, NULL = the null stream), allocate
 * nothing and return the error codes of retro_out_prod.h.
 */
#ifndef RETRO_PROBE_H
#define RETRO_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum retro_probe_kind {
    RETRO_PROBE_MFMA_F32 = 0,  /* v_mfma_f32_32x32x2_f32, 4096 FLOP each */
    RETRO_PROBE_MFMA_BF16 = 1  /* v_mfma_f32_32x32x16_bf16, 32768 FLOP each */
};

/* Floats the matrix-core probe writes to `sink` (one per thread of its grid
 * of 2048 workgroups x 256 threads, 8 per CU). */
int64_t retro_probe_sink_floats(void);

/* Matrix-core probe: every wave runs `iterations` rounds of 4 independent
 * MFMAs of `kind` on register operands, then writes the sum of its
 * accumulators to `sink` (device memory, retro_probe_sink_floats() floats,
 * 4-byte aligned; its values only keep the loop from being removed).
 * *flops (host memory, may be NULL) receives the FLOPs one launch performs.
 * Errors: RETRO_E_TYPE for an unknown kind, RETRO_E_SHAPE unless
 * 1 <= iterations <= 2^20, RETRO_E_NULL for a null sink, RETRO_E_ALIGN for
 * a misaligned one, RETRO_E_HIP for a launch error. */
int retro_probe_mfma(int kind, float *sink, int64_t iterations, double *flops, void *stream);

/* Matrix core beside vector ALU: 512 workgroups of 8 waves (two per CU,
 * two waves per SIMD). Waves 0-3 of each run `mfma_iterations` rounds of 4
 * independent v_mfma_f32_16x16x4_f32 (2048 FLOP each, the small-T kernel's
 * instruction); waves 4-7 run `valu_iterations` rounds of 16 v_fma_f32 over
 * 8 independent chains. Either count may be 0. Timed with one count at 0,
 * then the other, then both: if the two kinds of work ran side by side the
 * last time would be the larger of the first two, if they share the
 * SIMDs' issue time it is their sum. Every thread writes one float to
 * `sink` (device memory of at least retro_probe_sink_floats() floats,
 * 4-byte aligned). *flops and *valu_instructions (host memory, may be NULL)
 * receive the MFMA FLOPs and the wave-level FMA instructions of one launch.
 * Errors: RETRO_E_SHAPE unless both counts are in 0 .. 2^20, RETRO_E_NULL,
 * RETRO_E_ALIGN, RETRO_E_HIP. */
int retro_probe_mfma_valu(int64_t mfma_iterations, int64_t valu_iterations, float *sink, double *flops,
                          int64_t *valu_instructions, void *stream);

/* Copy probe: dst[0 .. bytes) = src[0 .. bytes), both device memory,
 * 16-byte aligned, not overlapping; bytes a multiple of 16 (0 is a no-op).
 * Each workgroup copies one 16 KiB tile, each thread four 16-byte units
 * with all four loads in flight. The copy moves 2 * bytes
 * over HBM. Errors: RETRO_E_SHAPE for a negative or unaligned size or one of
 * 2^40 bytes or more, RETRO_E_NULL, RETRO_E_ALIGN, RETRO_E_ALIAS for
 * overlapping ranges, RETRO_E_HIP. */
int retro_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RETRO_PROBE_H */
