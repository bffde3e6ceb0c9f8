/*
 * bca_probe.h — measurement hooks of libbca (not part of the attention path).
 *
 * The attention kernels are priced against the matrix cores' dense rate. The
 * published MI355X figures are 2.5 PFLOP/s for bf16 and 5.0 PFLOP/s for fp8; the
 * rate the chip reaches at the clock it holds under load is measured by these
 * probe kernels, so that a kernel's fraction of peak can be read against both.
 *
 * Each probe launches `wgs` work groups of 512 threads (8 waves, two per SIMD)
 * on `stream` (a hipStream_t, 0 = the null stream); every wave issues `iters`
 * rounds of four independent 32x32 MFMAs back to back:
 *   bf16: v_mfma_f32_32x32x16_bf16      (32*32*16*2 FLOP each)
 *   fp8:  v_mfma_f32_32x32x64_f8f6f4 on e4m3 operands (32*32*64*2 FLOP each)
 * and lane 0 of each wave writes one float to out[wg * 8 + wave], so `out` is
 * caller-owned device memory of at least wgs * 8 floats. The call is
 * asynchronous; time it with events on `stream`. Returns 0, -1 for wgs < 1,
 * iters < 1 or a null out, else the HIP launch error code.
 * The *_flops functions return the FLOP count of one launch with those sizes.
 */
#ifndef BCA_PROBE_H
#define BCA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

double bca_probe_mfma_bf16_flops(int wgs, int iters);
int bca_probe_mfma_bf16(int wgs, int iters, float* out, void* stream);
double bca_probe_mfma_fp8_flops(int wgs, int iters);
int bca_probe_mfma_fp8(int wgs, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif
