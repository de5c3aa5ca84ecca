/*
 * flashot_probe.h -- throughput probes for the roofline of the streamed
 * log-sum-exp pass (measurement helpers; not part of the Sinkhorn path).
 *
 * A Sinkhorn half-step costs, per (i, j) pair, a d-long dot product on the
 * matrix cores and one exponential of the biased score (the online
 * log-sum-exp of §2.3 / App. D.3 of "FlashSinkhorn: IO-Aware Entropic Optimal
 * Transport on GPU"; the page's own profile, App. H.2.1, accounts for the
 * kernel by the same two units). The probes measure what each unit sustains
 * on this chip, alone, so that the pass's time can be set against them.
 */
#ifndef FLASHOT_PROBE_H
#define FLASHOT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OT_PROBE_EXP2         0  /* v_exp_f32 throughput: exponentials */
#define OT_PROBE_MFMA_F16     1  /* 32x32x16 fp16 matrix instruction throughput: flops */
#define OT_PROBE_MFMA_F16_1C2W 2 /* the same with 1 chain per wave, 2 waves per SIMD */
#define OT_PROBE_MFMA_F16_2C2W 3 /* 2 chains per wave, 2 waves per SIMD */
#define OT_PROBE_MIX_2W       4  /* 2 chains of 13 matrix instructions per wave interleaved with
                                    34 exponentials and 48 fp32 additions, 2 waves per SIMD
                                    (the d = 64 fp32 pass's per-stage mix): matrix flops */

/*
 * ot_probe_rate -- enqueue one probe kernel of `blocks` workgroups of 256
 * threads, each thread (OT_PROBE_EXP2) running 8 independent chains of
 * `iters` exponentials x <- exp2(-x), or each wave (OT_PROBE_MFMA_F16)
 * running 4 independent chains of `iters` 32x32x16 fp16 matrix
 * instructions. The *_2W kinds reserve 64 KiB of LDS per workgroup so that
 * two waves share each SIMD (the occupancy of the register-resident pass)
 * and run 1 or 2 chains per wave, or (OT_PROBE_MIX_2W) `iters` copies of
 * that pass's per-stage instruction mix on independent data. The caller
 * times the launch on `stream` (HIP events) and divides *work by the time.
 *   iters   >= 1
 *   blocks  >= 1 (several per compute unit fill the chip: 2048 is plenty)
 *   out     device fp32, blocks * 256 values (one per thread; keeps the work live)
 *   work    host: receives the launch's exponentials or flops
 * Asynchronous. Errors: OT_ERR_INVALID_ARG (null pointer, iters or
 * blocks < 1, unknown kind), OT_ERR_HIP (launch failure).
 */
int ot_probe_rate(int kind, int64_t iters, int32_t blocks, float* out, double* work, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHOT_PROBE_H */
