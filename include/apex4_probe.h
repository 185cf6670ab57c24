/*
 * apex4_probe.h -- measurement probes of libapex4.so: five kernels that
 * measure, on the GPU at hand, the ceilings the W4A4 GEMM kernels are held
 * against (the int8 and FP6 matrix-unit rates, the HBM read rate, the fp32
 * vector-ALU rate, the LDS read rate), so that a result can be quoted against
 * the chip's measured ceiling as well as its datasheet peak.  The APEX4 page (aiqbench news page,
 * Abstract) frames the method by the balance of the matrix (Tensor Core) and
 * vector (CUDA Core) throughputs of a GPU; these probes measure that balance
 * here.
 *
 * Conventions as in apex4.h: device pointers unless noted, host-side argument
 * checks before any launch, asynchronous and ordered on `stream` (a
 * hipStream_t, NULL = legacy default stream); the caller times the call (e.g.
 * with events on the same stream) and divides the work the call reports.
 * The probes allocate nothing; `sink` is written only if a result hits a
 * sentinel value (never in practice), which keeps the work from being
 * optimized away.
 */
#ifndef APEX4_PROBE_H
#define APEX4_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "apex4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Independent v_mfma_i32_32x32x32_i8 instructions: 1024 workgroups of 4 waves,
 * each wave issuing `iters` rounds of 4 MFMAs on 4 independent accumulators.
 *   iters: >= 1.   sink: device int32[1], 4-byte aligned.
 *   ops_out: HOST double, set to the integer operations issued
 *            (1024 * 4 * iters * 4 * 2 * 32*32*32).
 */
apex4_status apex4_probe_mfma_i8(int64_t iters, int32_t* sink, double* ops_out, void* stream);

/*
 * Independent v_mfma_scale_f32_32x32x64_f8f6f4 instructions on FP6 E2M3
 * operands with unit block scales (the instruction apex4_gemm_w4a4_f6 runs):
 * the same grid and rounds as apex4_probe_mfma_i8.
 *   iters: >= 1.   sink: device int32[1], 4-byte aligned.
 *   ops_out: HOST double, set to the floating-point operations issued
 *            (1024 * 4 * iters * 4 * 2 * 32*32*64).
 */
apex4_status apex4_probe_mfma_f6(int64_t iters, int32_t* sink, double* ops_out, void* stream);

/*
 * Streaming read of `bytes` bytes: every wave reads whole 4 KB rows (16 bytes
 * per lane and load, four loads per row), 1024 workgroups of 4 waves taking
 * rows round-robin -- the access pattern that reads HBM fastest here.
 *   buf: device memory, 16-byte aligned; bytes: > 0, a multiple of 4096.
 *   sink: device int32[1], 4-byte aligned.
 *   bytes_out: HOST double, set to the bytes read.
 */
apex4_status apex4_probe_hbm_read(const void* buf, int64_t bytes, int32_t* sink, double* bytes_out,
                                  void* stream);

/*
 * fp32 fused multiply-adds on the vector ALU (no packed-fp32 instructions, as
 * in every kernel of this library): 1024 workgroups of 256 threads, each
 * thread running 8 independent chains of `iters` FMAs.
 *   iters: >= 1.   sink: device float[1], 4-byte aligned.
 *   flops_out: HOST double, set to the floating-point operations
 *              (1024 * 256 * iters * 8 * 2).
 */
apex4_status apex4_probe_valu_f32(int64_t iters, float* sink, double* flops_out, void* stream);

/*
 * 16-byte LDS reads (ds_read_b128): 1024 workgroups of 4 waves, each with a
 * 16 KB LDS buffer, every wave reading `iters` rounds of 8 independent
 * 1 KB pieces (lane l at byte 16 l of a piece: no bank conflicts).  The LDS
 * bytes a compute unit can deliver per clock bound how many operand bytes a
 * GEMM can feed its matrix instructions from LDS.
 *   iters: 1 .. 2^30.   sink: device int32[1], 4-byte aligned.
 *   bytes_out: HOST double, set to the LDS bytes read
 *              (1024 * 256 * iters * 8 * 16).
 */
apex4_status apex4_probe_lds_read(int64_t iters, int32_t* sink, double* bytes_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* APEX4_PROBE_H */
