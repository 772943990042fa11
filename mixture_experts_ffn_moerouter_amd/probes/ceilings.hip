// Measurement instruments (include/moe_probes.h): the attainable streaming-read bandwidth,
// the rate at which the compute units read L2-resident data, and the attainable dense bf16
// matrix-core rate of the device, measured by the benchmark beside the published peaks.
// Not part of the MoE path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probes.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kThreads = 256;
constexpr int kMagic = 0x5a5a1234;  // a checksum ordinary probe data does not produce

// Workgroup b reads the contiguous run of 16-byte vectors [b per, (b + 1) per); each thread
// keeps eight non-temporal loads in flight (lines are streamed once, so they are fetched
// with the hint that they will not be reused) and folds them into a checksum.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const i32x4* __restrict__ src,
                                                               int64_t n, int64_t per,
                                                               int32_t* sink) {
  constexpr int U = 8;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  i32x4 acc = {0, 0, 0, 0};
  int64_t i = lo + threadIdx.x;
  for (; i + (U - 1) * kThreads < hi; i += U * kThreads) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < hi; i += kThreads) acc ^= src[i];
  const int v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == kMagic) sink[blockIdx.x] = v;
}

// Four independent accumulator chains per wave; operands come from the thread index so
// they are not constants.
__global__ __launch_bounds__(kThreads) void mfma_bf16_kernel(int64_t iters, float* sink) {
  const short t = (short)threadIdx.x;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (short)(0x3c00 + ((t + j) & 7));   // small positive bf16 values
    b[j] = (short)(0x3b80 + ((t * 3 + j) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int64_t k = 0; k < iters; ++k) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (s == -1.0f) sink[blockIdx.x] = s;  // the sums are positive
}

// L2-resident reads: every workgroup (eight waves, one per CU) reads a region small enough
// to stay in each XCD's L2 over and over, 1 KB per wave and instruction (lane l takes the
// 16 bytes at 16 l), in rounds of 16 loads per wave, each round issued before the previous
// one is waited for (16 to 32 loads in flight per wave). LDS form: direct-to-LDS buffer
// loads into a wave-private 8 KB ring of landing slots; register form: the same loads into
// two register sets used alternately, each folded into a checksum once the next round is
// issued. The landed LDS data is folded into the checksum at the end, so neither form's
// loads are dead.
constexpr int kL2Threads = 512;
constexpr int kL2Unroll = 16;
typedef __attribute__((address_space(3))) void lds_void;

template <bool LDS>
__global__ __launch_bounds__(kL2Threads) void l2_read_kernel(const void* __restrict__ src,
                                                              uint32_t region, int64_t rounds,
                                                              int32_t* sink) {
  __shared__ __align__(16) unsigned char land[kL2Threads / 64][8][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)region, 0x00020000);
  const uint32_t lines = region / 1024;  // 1 KB pieces in the region
  uint32_t piece = (uint32_t)(blockIdx.x * (kL2Threads / 64) + wave) * 7u;
  i32x4 acc = {0, 0, 0, 0};
  auto issue = [&](i32x4* v) {  // one round of loads
#pragma unroll
    for (int u = 0; u < kL2Unroll; ++u) {
      const uint32_t off = (piece % lines) * 1024u + 16u * (uint32_t)lane;
      piece += kL2Threads / 64;
      if constexpr (LDS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)&land[wave][u & 7][0], 16, off,
                                                 0, 0, 0);
      else
        v[u] = __builtin_bit_cast(i32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto fold = [&](const i32x4* v) {
#pragma unroll
    for (int u = 0; u < kL2Unroll; ++u) acc ^= v[u];
    __builtin_amdgcn_sched_barrier(0);
  };
  i32x4 va[LDS ? 1 : kL2Unroll], vb[LDS ? 1 : kL2Unroll];
  issue(va);
  for (int64_t k = 1; k < rounds; k += 2) {  // rounds is even
    issue(vb);
    if constexpr (LDS) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kL2Unroll) : "memory");
    else fold(va);
    if (k + 1 < rounds) {
      issue(va);
      if constexpr (LDS) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kL2Unroll) : "memory");
      else fold(vb);
    }
  }
  if constexpr (LDS) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    acc ^= *(const i32x4*)&land[wave][lane & 7][16 * (lane >> 3)];
  } else {
    fold(vb);
  }
  const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == kMagic) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" {

int moe_probe_stream_read(const void* src, int64_t bytes, int32_t* sink, int32_t grid,
                          void* stream) {
  if (!src || !sink || grid < 1 || bytes < 16 || bytes % 16 || ((uintptr_t)src & 15))
    return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16, per = (n + grid - 1) / grid;
  stream_read_kernel<<<grid, kThreads, 0, (hipStream_t)stream>>>((const i32x4*)src, n, per,
                                                                  sink);
  return (int)hipGetLastError();
}

int moe_probe_l2_read(const void* src, int64_t region, int64_t rounds, int32_t to_lds,
                      int32_t* sink, int32_t grid, void* stream) {
  if (!src || !sink || grid < 1 || rounds < 2 || rounds % 2 || region < 1024 ||
      region % 1024 ||
      region > ((int64_t)1 << 30) || ((uintptr_t)src & 15))
    return (int)hipErrorInvalidValue;
  if (to_lds)
    l2_read_kernel<true><<<grid, kL2Threads, 0, (hipStream_t)stream>>>(src, (uint32_t)region,
                                                                        rounds, sink);
  else
    l2_read_kernel<false><<<grid, kL2Threads, 0, (hipStream_t)stream>>>(src, (uint32_t)region,
                                                                         rounds, sink);
  return (int)hipGetLastError();
}

int moe_probe_mfma_bf16(int64_t iters, float* sink, int32_t grid, void* stream) {
  if (!sink || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  mfma_bf16_kernel<<<grid, kThreads, 0, (hipStream_t)stream>>>(iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
