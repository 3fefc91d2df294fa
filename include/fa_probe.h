/*
 * fa_probe.h -- C ABI of libfa_probe_gfx950.so, a measurement library that
 * is not part of the attention path: it holds one register-only matrix-core
 * kernel whose rate is the attainable bf16 MFMA ceiling of the GPU it runs
 * on (the clock under sustained matrix-core load sits below the 2.4 GHz of
 * the published 2.5 PFLOP/s).  bench.py reports the attention kernels'
 * rates against both.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue `workgroups` workgroups of 4 waves (256 = one wave per SIMD on
 * every CU; 256 * w gives w waves per SIMD), each wave running `iters`
 * iterations of 16 v_mfma_f32_32x32x16_bf16 on operands held in registers.
 *   operands: DEVICE pointer to 8 * 64 * 8 bf16 values (8 operand fragments
 *     of 64 lanes x 8 elements; each lane reads its 8 fragments once).
 *   sink: DEVICE pointer to workgroups * 256 floats (one per thread, the sum
 *     of its accumulators, so that the products are not optimised away).
 *   stream: hipStream_t (NULL = the null stream).
 * Returns 0, 1 for a NULL pointer, 2 for workgroups outside [1, 2^20] or
 * iters < 1, 7 for a launch error.
 */
int fa_probe_mfma_bf16(const void* operands, float* sink, int workgroups, int iters, void* stream);

/* Floating-point operations of one fa_probe_mfma_bf16 call (2 per multiply-add). */
double fa_probe_mfma_bf16_flops(int workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */
