/*
 * g4probe.h - roofline probes for the attention kernels' measurements.
 *
 * Two plain kernels that measure, on the GPU at hand, the two ceilings the
 * attention path is priced against: the dense bf16 matrix-core rate (the
 * prefill is a dense contraction) and the HBM streaming-read rate (the decode
 * reads each cached row once).  They compute nothing of the attention method;
 * they exist so that a roofline fraction can be quoted against a measured
 * attainable peak as well as the vendor figure.  Built as libg4probe.so, a
 * library of its own, beside libg4attn.so.
 *
 * Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream) and returns 0 on success, -1 for an invalid argument (nothing is
 * launched), or the hipError_t of the launch.
 */
#ifndef G4PROBE_H
#define G4PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Operand data of the MFMA loop.  The sustained matrix-core rate depends on
 * it: the chip lowers its clock under the switching activity of full-width
 * random operands (as in attention), and holds it when the operands barely
 * switch. */
enum {
  G4PROBE_RANDOM = 0,       /* hashed values in [-1, 1), eight distinct operand pairs */
  G4PROBE_LOW_ACTIVITY = 1  /* every odd bf16 element zero, the others one of eight constants */
};

/* Dense bf16 MFMA loop: `workgroups` workgroups of 256 threads (4 waves);
 * every wave issues `iters` rounds of 8 independent 32x32x16 bf16 matrix
 * products, each with its own operand pair (`operands` picks their data),
 * into fp32 accumulators held in registers, with no memory traffic inside
 * the loop.  Work: workgroups * 4 * iters * 8 * 32768 flop.  Each thread
 * writes one float (a sum of its accumulators, so nothing is elided) to
 * out[workgroups * 256] (device memory, caller-owned).
 * Invalid: out NULL, workgroups < 1, iters < 1, unknown `operands`. */
int g4probe_mfma_bf16(float* out, int32_t workgroups, int64_t iters, int32_t operands, void* stream);

/* HBM streaming read: `workgroups` workgroups of 256 threads split `bytes`
 * of `src` (device memory, 16-byte aligned, bytes a multiple of 16) into
 * contiguous chunks and read them once with 16-byte non-temporal loads,
 * 8 loads in flight per thread.  Each thread writes one word (an XOR of what
 * it read) to sink[workgroups * 256] (device memory, caller-owned).  Work:
 * `bytes` read.
 * Invalid: src or sink NULL, src not 16-byte aligned, bytes < 16 or not a
 * multiple of 16, workgroups < 1. */
int g4probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* G4PROBE_H */
