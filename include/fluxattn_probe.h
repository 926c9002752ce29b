/*
 * fluxattn_probe — a measurement aid beside the fluxattn library, not part of
 * the attention path: the practical matrix-core rate of the GPU, against
 * which the attention kernels' roofline fractions can be read.  The blog
 * post "Speed up image generation with FLUX 3 Image Klein on NVIDIA
 * Blackwell GPUs" (section "Quantized and sparse attention") places dense
 * attention's cost in its matrix products; on a power-limited MI355X the
 * dense MFMA peak (2516.6 bf16 / 5033.2 fp8 TFLOP/s at 2.4 GHz) is not what
 * the matrix cores sustain, and this probe measures what they do.
 */
#ifndef FLUXATTN_PROBE_H
#define FLUXATTN_PROBE_H

#include <stdint.h>

#include "fluxattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueues on `stream` one launch of `workgroups` workgroups of 8 waves (two
 * per SIMD, as the attention kernels run) that issue back-to-back MFMAs on
 * register operands: kind 0 bf16 32x32x16 and kind 1 OCP E4M3 32x32x64
 * (per wave `iterations` rounds of 8 MFMAs over 4 independent accumulator
 * chains; kind 1 is the fp8 attention kernel's shape), kind 2 bf16
 * 16x16x32 (rounds of 16 MFMAs over 8 chains, the same flops per round as
 * kind 0; the bf16 attention kernel's shape).  A and B operands cycle
 * through 8 pseudo-random fragments each, so the operand data changes from
 * one MFMA to the next.
 *   sink   device fp32 [workgroups * 8], receives one sum per wave (keeps
 *          the work observable; the values have no meaning).
 *   flops  host: receives the launch's matrix flops (per round and wave
 *          8 * 2*32*32*k, k = 16 for kinds 0 and 2, 64 for kind 1).
 * Nothing is allocated and nothing synchronised; time the launch with
 * events on `stream`.  Errors: NULL sink or flops, kind not 0, 1 or 2,
 * iterations outside [1, 2^40], workgroups outside [1, 2^20], a sink not
 * 4-byte aligned, no gfx950 device; checks run before anything is
 * enqueued.
 */
fluxattn_status fluxattn_probe_mfma(int32_t kind, int64_t iterations,
                                    int32_t workgroups, float *sink,
                                    double *flops, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUXATTN_PROBE_H */
