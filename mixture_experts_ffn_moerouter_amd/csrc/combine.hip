// Weighted combine: back to token order, routing weights applied, top-k reduced, cast.
//
// [TO] TileOPs "MoE Operators", MoEPostPermuteFwdOp (token order restored, routing
//      weights applied once, top-k reduced, then cast) and FusedMoEExpertsFwdOp
//      (output[t] = scale * sum_k w[t,k] * expert output of route (t, k)).
//
// One workgroup per token; each thread owns 8 consecutive hidden elements (16-byte
// loads of bf16 rows), sums its K rows in float32 in k order and writes once.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename YT>
__device__ __forceinline__ void load8(const YT* p, float* v);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  i32x4 q = *(const i32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(((uint32_t)q[i]) << 16);
    v[2 * i + 1] = __uint_as_float(((uint32_t)q[i]) & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

template <typename YT, bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ route_pos,
                                                      int T, int K, int H, float scale,
                                                      void* out, int out_dt) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const float* wt = w + (int64_t)t * K;
  const int32_t* pt = route_pos + (int64_t)t * K;
  if (VEC) {
    for (int h = threadIdx.x * 8; h < H; h += blockDim.x * 8) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        float v[8];
        load8<YT>(y + (int64_t)pt[k] * H + h, v);
        const float wk = wt[k];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wk, v[i], acc[i]);
      }
      if (out_dt == 1) {
        i32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          q[i] = (int)((uint32_t)f32_to_bf16(scale * acc[2 * i]) |
                       ((uint32_t)f32_to_bf16(scale * acc[2 * i + 1]) << 16));
        *(i32x4*)((uint16_t*)out + (int64_t)t * H + h) = q;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) store_dt(out, out_dt, (int64_t)t * H + h + i, scale * acc[i]);
      }
    }
  } else {
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
      float acc = 0.f;
      for (int k = 0; k < K; ++k) {
        const YT* p = y + (int64_t)pt[k] * H + h;
        float v = sizeof(YT) == 4 ? *(const float*)p : bf16_to_f32(*(const uint16_t*)p);
        acc = fmaf(wt[k], v, acc);
      }
      store_dt(out, out_dt, (int64_t)t * H + h, scale * acc);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dt, const float* w, const int32_t* route_pos,
                          int T, int K, int H, float scale, void* out, int out_dt,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const bool vec = (H % 8) == 0;
  if (y_dt == 0) {
    if (vec) combine_kernel<float, true><<<T, 256, 0, s>>>((const float*)y, w, route_pos, T, K, H, scale, out, out_dt);
    else combine_kernel<float, false><<<T, 256, 0, s>>>((const float*)y, w, route_pos, T, K, H, scale, out, out_dt);
  } else {
    if (vec) combine_kernel<uint16_t, true><<<T, 256, 0, s>>>((const uint16_t*)y, w, route_pos, T, K, H, scale, out, out_dt);
    else combine_kernel<uint16_t, false><<<T, 256, 0, s>>>((const uint16_t*)y, w, route_pos, T, K, H, scale, out, out_dt);
  }
  return hipGetLastError();
}

}  // namespace moe
