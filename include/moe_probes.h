/* libmoe_probes.so: measurement instruments, not part of the MoE path.
 *
 * Two kernels that bound what any kernel of the path can reach on the device at hand:
 * a streaming read of a large buffer (the attainable HBM read bandwidth) and a loop of
 * dense bf16 matrix-core instructions with no memory traffic (the attainable MFMA rate).
 * The benchmark prints both beside the published peaks.
 *
 * Pointers are device pointers owned by the caller; calls are asynchronous on `stream`
 * (a hipStream_t, NULL for the default stream) and return a hipError_t value (0 on
 * success). Nothing is allocated.
 */
#ifndef MOE_PROBES_H
#define MOE_PROBES_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of `src` (16-byte aligned, bytes a multiple of 16) once with
 * non-temporal 16-byte loads, `grid` workgroups of 256 threads each reading one
 * contiguous 1/grid of the buffer, eight loads in flight per thread. `sink` holds
 * `grid` ints; a workgroup writes its entry only when its checksum of the data equals
 * a value ordinary data does not produce, so the loads cannot be optimised away and
 * nothing is written in practice. Returns hipErrorInvalidValue on bad sizes. */
int moe_probe_stream_read(const void* src, int64_t bytes, int32_t* sink, int32_t grid,
                          void* stream);

/* Every wave of `grid` workgroups of 256 threads (four waves) runs `iters` iterations of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands: 4 * 32768 flop per
 * iteration and wave. `sink` holds `grid` floats, written under the same rule as above. */
int moe_probe_mfma_bf16(int64_t iters, float* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif
#endif
