/*
 * nvfp4_mainloop_probe.h - measurement kernels behind the mainloop choice of
 * the NVFP4 grouped GEMM on gfx950 (libnvfp4_mainloop_probe.so). Not part of
 * the GEMM's path: they time the inner loops of the two exact ways of applying
 * NVFP4's per-16 E4M3 scales (the block-scaled MMA of submissions 506336 /
 * 385043 / 499344, kernelindex.com "kernelbot nvfp4 group gemm") and show what
 * the scaled FP4 conversion does with a scale that is not a power of two.
 *
 * Calls are asynchronous on `stream` (a hipStream_t, NULL = default stream);
 * the caller owns every buffer. Return 0, -1 for invalid arguments (nothing is
 * launched), -3 if the launch failed (nvfp4_probe_last_hip_error() has the HIP
 * code of the calling thread's last failed launch).
 */
#ifndef NVFP4_MAINLOOP_PROBE_H
#define NVFP4_MAINLOOP_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nvfp4_probe_mainloop - run `iters` iterations of one inner loop on `grid`
 * workgroups of 256 threads (one per compute unit when grid equals the
 * compute-unit count). One iteration is 64 K of a 128x128 wave tile (128x64
 * for variant 1) on each of the four waves, i.e.
 * nvfp4_probe_flops_per_iteration(variant) flops of useful 32x32x16 MFMA work
 * per workgroup.
 *   variant 0: exact dequantisation to f16 (FP4 conversion, then one f16
 *              multiply by the E4M3 scale) feeding v_mfma_f32_32x32x16_f16;
 *   variant 1: v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 codes, one 16-block
 *              per MFMA, then each fp32 partial product times the row and
 *              column scale factors added into the accumulator on the VALU
 *              (accumulators in VGPRs, so a 128x64 wave tile);
 *   variant 2: the bare f16 MFMA loop (operands read from LDS, no VALU work);
 *   variant 3: the bare v_mfma_scale_f32_32x32x64_f8f6f4 loop on E2M1 codes
 *              with E8M0 scales, one 16-block per 32-K lane slice (two
 *              instructions per 32x32 block per 64 K), as in the
 *              power-of-two-scale path;
 *   variant 4: a bare f16 loop with v_mfma_f32_16x16x32_f16 doing the same
 *              work per iteration (8 x 4 blocks of 16x16, four 32-K steps);
 *   variant 5: variant 0 on a 128x64 wave tile (6 dequantisation VALU per
 *              MFMA), four waves per workgroup (one per SIMD);
 *   variant 6: variant 5 with eight waves per workgroup (two per SIMD);
 *   variant 7: (b) on a 256x128 workgroup tile as four 64x128 wave tiles, B
 *              dequantised once per workgroup (each wave one of the four B
 *              fragments) and shared through LDS with one barrier per
 *              iteration (3 dequantisation VALU per MFMA);
 *   variant 8: variant 7 with the exchange a step ahead (each iteration
 *              writes the next one's B while its MFMAs run);
 *   variant 9: variant 2 on operands with 6 significant bits (like the
 *              dequantised a * s) instead of a random 10-bit mantissa;
 *   variant 10: the bare bf16 MFMA loop (v_mfma_f32_32x32x16_bf16) on
 *              operands with 6 significant bits.
 *   sink: device fp32 [grid * 512], written with per-lane sums (so the work
 *         is kept).
 */
int nvfp4_probe_mainloop(int variant, int iters, int grid, float* sink, void* stream);

/* Useful flops of one iteration of one workgroup (4 waves x 64 MFMAs, or x 32
 * for variants 1, 5, 7 and 8, or 8 waves x 32 for variant 6, of 32x32x16). */
double nvfp4_probe_flops_per_iteration(int variant);

/*
 * nvfp4_probe_cvt_scale - out[i] = the f16 bits that v_cvt_scalef32_pk_f16_fp4
 * gives for FP4 code 0x2 (1.0) under the f32 scale scales[i]. scales: device
 * float [n]; out: device uint16 [n].
 */
int nvfp4_probe_cvt_scale(const float* scales, int n, uint16_t* out, void* stream);

int nvfp4_probe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MAINLOOP_PROBE_H */
