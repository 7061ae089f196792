/*
 * moe_probe.h -- measurement probes of the MI355X the layer runs on.
 *
 * Not part of the MoE layer: two kernels whose rates are the measured peaks
 * the layer's kernels are compared with in the same run (the vendor peaks
 * assume the maximum engine clock, which sustained matrix work does not
 * hold).  Same conventions as moe_mi355x.h: device pointers to caller-owned
 * memory, `stream` is a hipStream_t passed as void*, arguments validated on
 * the host first (nothing enqueued on error), the call only enqueues work.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "moe_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sustained bf16 matrix rate: 256 workgroups of 8 waves, each wave issuing
 * `iterations` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
 * pseudo-random operands (bits that change between instructions, as GEMM
 * data does).  One launch performs exactly moe_probe_mfma_flops(iterations)
 * FLOPs; the caller times it.  `sink` (one float, device) receives a value
 * only if the accumulators reach an impossible pattern, so the work cannot be
 * optimised away.  iterations must be a positive multiple of 4, sink
 * non-null. */
moe_status moe_probe_mfma_bf16(int32_t iterations, float* sink, void* stream);

/* FLOPs of one moe_probe_mfma_bf16 launch: 256 * 8 * 8 * 32768 * iterations. */
double moe_probe_mfma_flops(int32_t iterations);

/* Streaming read of `bytes` bytes of `buf` (16-byte aligned, bytes a multiple
 * of 16) with 16-byte loads spread over every CU, XOR-reduced per thread;
 * `sink` (one uint32, device) is written only for an impossible reduction
 * value.  The caller times it: bytes / time is the read bandwidth. */
moe_status moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
