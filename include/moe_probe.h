/*
 * moe_probe.h -- measurement probes of the GPU the MoE layer runs on (C ABI,
 * same library and conventions as moe.h).
 *
 * The layer's kernels are graded against the chip's published peaks: dense
 * bf16 matrix throughput for the grouped expert GEMMs and HBM bandwidth for
 * the dispatch and combine.  These probes measure what the chip in hand
 * actually sustains -- a plain streaming copy and read, a dense stream of
 * bf16 MFMA instructions -- and the core clock it runs at meanwhile, so that
 * a kernel's fraction of the published peak can be read beside its fraction
 * of the measured one.  They touch no data of the layer and are never called
 * on its path.
 *
 * Device pointers, 16-byte aligned; `stream` is a hipStream_t passed as void*;
 * every call only enqueues work and returns a moe_status (validation on the
 * host first, nothing enqueued on error).
 */
#ifndef MOE_MI355X_PROBE_H
#define MOE_MI355X_PROBE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0 .. bytes) = src[0 .. bytes): 16-byte non-temporal loads and stores,
 * a grid of `blocks` workgroups of 256 threads striding over the buffer
 * (blocks in [1, 65536]; 0 picks 8 per CU).  bytes % 16 == 0.  HBM traffic:
 * 2 * bytes (read + write).  src and dst must not overlap. */
moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, int32_t blocks,
                          void* stream);

/* Reads src[0 .. bytes) with 16-byte non-temporal loads and writes one fp32
 * per thread (a sum of the words read, so no load is dead) to
 * sink[blocks * 256].  bytes % 16 == 0; blocks as for moe_probe_copy (0: 8 per
 * CU; sink must then hold 8 * CUs * 256 floats).  HBM traffic: bytes. */
moe_status moe_probe_read(const void* src, size_t bytes, float* sink, int32_t blocks,
                          void* stream);

/* A dense stream of v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 bf16 products into
 * fp32, 16384 flops each) from registers, no memory traffic: `blocks`
 * workgroups of 8 waves, each wave `iters` iterations of 8 independent
 * accumulations, so the launch does blocks * 8 * iters * 8 * 16384 flops.
 * blocks in [1, 65536], iters in [1, 2^24].
 *   sink   [blocks * 512] fp32 out  the accumulators' sums (keeps them live)
 *   stamps [blocks * 4]   u64  out  per workgroup, read by its first wave:
 *          core clock counter at start and end, then the constant-rate
 *          real-time counter (100 MHz on this chip) at start and end; the
 *          core clock in MHz is (end - start) cycles / ((rt_end - rt_start) / 100). */
moe_status moe_probe_mfma(int32_t blocks, int32_t iters, float* sink, uint64_t* stamps,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_PROBE_H */
