/* libmoe_probes.so: measurement instruments, not part of the MoE path.
 *
 * Kernels that bound what any kernel of the path can reach on the device at hand: a
 * streaming read of a large buffer (the attainable HBM read bandwidth), repeated reads
 * of an L2-resident region (the rate at which the compute units take in cached data, in
 * the two load forms the GEMMs could use) and a loop of dense bf16 matrix-core
 * instructions with no memory traffic (the attainable MFMA rate). The benchmark prints
 * them beside the published peaks.
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

/* Every wave of `grid` workgroups of 512 threads (eight waves) reads the first `region`
 * bytes of `src` (a multiple of 1024, at most 1 GiB, 16-byte aligned; small enough, e.g.
 * 1 MiB, to stay in each XCD's L2) `rounds` (even) x 16 times in 1 KB pieces, 16-byte loads:
 * direct-to-LDS buffer loads when `to_lds` is nonzero, loads into registers otherwise;
 * grid x 512 x 16 x 16 x rounds bytes in all. `sink` as above. Returns
 * hipErrorInvalidValue on bad sizes. */
int moe_probe_l2_read(const void* src, int64_t region, int64_t rounds, int32_t to_lds,
                      int32_t* sink, int32_t grid, void* stream);

/* Every wave of `grid` workgroups of 256 threads (four waves) runs `iters` iterations of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands: 4 * 32768 flop per
 * iteration and wave. `sink` holds `grid` floats, written under the same rule as above. */
int moe_probe_mfma_bf16(int64_t iters, float* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif
#endif
