/*
 * moe_peak.h -- measurement kernels of the MI355X roofline that the routed
 * MoE layer (include/moe.h) is judged against.
 *
 * The layer's decode path streams each activated expert's quantised
 * weights from HBM ("antirez ds4: DeepSeek Metal inference", section
 * 技术深度解析: only the routed experts' weights are read, so decode is a
 * weight stream), and its prefill path is a grouped product on the bf16
 * matrix cores.  The published peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16,
 * 5.0 PFLOP/s dense fp8) are what the chip is sold at; these kernels measure
 * what a plain kernel reaches on the same box, so that a fraction of the
 * measured peak can sit beside the fraction of the published one.
 *
 * Each only ENQUEUES on `stream`; time them with HIP events on that stream.
 * Pointers are device pointers; the caller owns every buffer.  They return
 * MOE_OK (0), MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN or MOE_ERR_HIP
 * (the codes of include/moe.h).
 */
#ifndef QUANTIZED_ROUTED_MOE_AMD_MOE_PEAK_H
#define QUANTIZED_ROUTED_MOE_AMD_MOE_PEAK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads buf[0 .. bytes) once with 16-byte loads spread over the whole chip
   (`workgroups` workgroups of 512 threads; 0 picks 2048) and writes one
   32-bit xor of what it read per workgroup to sink[0 .. workgroups) (so the
   loads cannot be dropped).  buf 16-byte aligned, bytes a positive multiple
   of 16; sink holds `workgroups` words.  The HBM read rate is bytes / the
   kernel's duration; reading a buffer that no recent kernel touched (the
   256 MB Infinity Cache is evicted by reading other data first) measures
   cold HBM. */
int moe_peak_stream(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream);

/* Dense matrix-core loop: `workgroups` workgroups of 256 threads (4 waves,
   0 picks 4 per CU = 1024), each wave issuing `iters` rounds of 8
   independent 32x32 products with fp32 accumulation on register operands,
   then writing one float per wave to sink (so nothing is dropped).
     kind 0: v_mfma_f32_32x32x16_bf16      (32 x 32 x 16 bf16, 32768 flop each)
     kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 with fp4 A and fp8 B
             (32 x 32 x 64, 131072 flop each; the MXFP8-activation path)
     kind 2: the same instruction with fp4 A and fp4 B (the MXFP4-activation
             path)
   flop = workgroups * 4 * iters * 8 * (flop each); the rate is flop / the
   kernel's duration.  sink holds workgroups * 4 floats. */
int moe_peak_mfma(int32_t kind, int32_t iters, int32_t workgroups, float* sink, hipStream_t stream);

/* Keeps `stream` busy for `microseconds` (1 .. 1,000,000): one wave reads
   the GPU's constant 100 MHz clock until that much time has passed, then
   returns.  Timing code enqueues it ahead of a timed loop so that the host
   gets ahead of the GPU while it waits: the loop's kernels then run back to
   back from the queue, and event pairs around them time the kernels rather
   than the host's launch rate.  Returns MOE_OK, MOE_ERR_SHAPE or
   MOE_ERR_HIP. */
int moe_peak_hold(uint32_t microseconds, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QUANTIZED_ROUTED_MOE_AMD_MOE_PEAK_H */
