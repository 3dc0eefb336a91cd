/*
 * moe_calib.h -- measurement probes of libmoe.so: the two ceilings the layer's kernels are judged
 * against on this part, measured rather than taken from the datasheet.
 *
 * The roofline method (inference-optimisation chapter, roofline section: attainable rate is the
 * smaller of peak compute and bandwidth times intensity) needs the two roofs. The datasheet gives
 * 8 TB/s of HBM and 2.5 PFLOP/s of dense bf16 matrix math; these probes measure what a streaming
 * read and a register-only matrix loop reach on the running GPU, so a kernel's fraction can also
 * be stated against what the part sustains. Time them with HIP events or a kernel trace.
 *
 * Conventions as in moe.h: device pointers, asynchronous on `stream`, validation on the host
 * before anything is enqueued, no allocation.
 */
#ifndef MOE_CALIB_H_
#define MOE_CALIB_H_

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups each probe launches: the entries of its `sink`. */
#define MOE_CALIB_READ_BLOCKS 512
#define MOE_CALIB_MFMA_BLOCKS 256

/*
 * moe_calib_read_stream -- read `bytes` of `buf` once, 16 bytes per lane per load: each of
 * MOE_CALIB_READ_BLOCKS workgroups of 256 threads reads its own contiguous share of the buffer,
 * 1 KB per load instruction, its four waves taking alternate kilobytes with eight loads each in
 * flight: a few long streams per compute unit, the fastest read pattern measured on the part.
 * nontemporal != 0 gives every load the non-temporal hint, as the weight-streaming kernels use.
 * Each workgroup folds what it read into one word of sink[MOE_CALIB_READ_BLOCKS] (uint32), so no load
 * can be dropped. bytes must be a non-zero multiple of 16; buf 16-byte aligned.
 */
moe_status moe_calib_read_stream(const void* buf, size_t bytes, uint32_t* sink, int nontemporal, void* stream);

/*
 * moe_calib_mfma -- a register-only loop of bf16 matrix instructions (32x32x16, fp32
 * accumulators): MOE_CALIB_MFMA_BLOCKS workgroups of 8 waves, one workgroup per compute unit (two
 * waves per SIMD, as in the grouped GEMM), each wave issuing `iters` x 8 independent MFMAs
 * (32768 flops each) on operands it loaded once from `operands` (bf16, MOE_CALIB_MFMA_BLOCKS x
 * 512 lanes x 32 bytes: two 16-byte fragments per lane), alternating
 * two operand sets so that the multiplier inputs change from one instruction to the next. The
 * caller picks the data: random values draw more power (and a lower clock) than constant ones.
 * Total flops = MOE_CALIB_MFMA_BLOCKS * 8 * iters * 8 * 32768. sink[MOE_CALIB_MFMA_BLOCKS] (float32)
 * receives one sum of accumulators per workgroup. clocks (uint64, 4 per wave, may be NULL) holds
 * each wave's shader-clock counter and 100 MHz real-time counter at its start and end (in that
 * order), so the host can read the shader clock the loop ran at. iters >= 1.
 */
moe_status moe_calib_mfma(const void* operands, int32_t iters, float* sink, uint64_t* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CALIB_H_ */
