// Weighted combine: back to token order, routing weights applied, top-k reduced, cast.
//
// [TO] TileOPs "MoE Operators", MoEPostPermuteFwdOp (token order restored, routing
//      weights applied once, top-k reduced, then cast) and FusedMoEExpertsFwdOp
//      (output[t] = scale * sum_k w[t,k] * expert output of route (t, k)). route_pos is
//      any layout's inverse index; a negative entry (a route a masked slab had no room
//      for) contributes nothing.
//
// One workgroup per token and chunk of kChunk hidden elements (several per token when H is
// large, so small batches still spread over the chip); each thread owns 8 consecutive
// elements (16-byte loads of 16-bit rows, non-temporal: each expert output is read once),
// sums its K rows in float32 in k order and writes once. A float32 y may come as partial
// slabs of a split contraction (the decode backend's down projection): a route's slabs are
// added in slab order before its weight is applied.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = kThreads * 8;  // hidden elements per workgroup

// Eight elements of y (dtype YDT: 0 f32, 1 bf16, 2 f16) as float32.
template <int YDT>
__device__ __forceinline__ void load8(const void* p, float* v) {
  if constexpr (YDT == 0) {
    f32x4 a = *(const f32x4*)p, b = *(const f32x4*)((const float*)p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  } else {
    i32x4 q = __builtin_nontemporal_load((const i32x4*)p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = h16_to_f32<YDT>((uint16_t)((uint32_t)q[i] & 0xffffu));
      v[2 * i + 1] = h16_to_f32<YDT>((uint16_t)((uint32_t)q[i] >> 16));
    }
  }
}

template <int YDT, bool VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ route_pos,
                                                      int T, int K, int H, float scale,
                                                      void* out, int out_dt, int nchunk,
                                                      int64_t chunk_stride) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const float* wt = w + (int64_t)t * K;
  const int32_t* pt = route_pos + (int64_t)t * K;
  const int ysz = YDT == 0 ? 4 : 2;
  const int h_end = min(H, (int)(blockIdx.y + 1) * kChunk);
  if (VEC) {
    for (int h = blockIdx.y * kChunk + threadIdx.x * 8; h < h_end; h += kChunk) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        if (pt[k] < 0) continue;  // a route without a row contributes nothing
        float v[8];
        load8<YDT>((const char*)y + ((int64_t)pt[k] * H + h) * ysz, v);
        if constexpr (YDT == 0) {  // partial slabs of a split contraction, in order
          for (int c = 1; c < nchunk; ++c) {
            float u[8];
            load8<YDT>((const float*)y + c * chunk_stride + (int64_t)pt[k] * H + h, u);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += u[i];
          }
        }
        const float wk = wt[k];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wk, v[i], acc[i]);
      }
      if (out_dt != 0) {
        i32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = scale * acc[2 * i], a1 = scale * acc[2 * i + 1];
          q[i] = out_dt == 1 ? (int)((uint32_t)f32_to_bf16(a0) | ((uint32_t)f32_to_bf16(a1) << 16))
                             : (int)((uint32_t)f32_to_f16(a0) | ((uint32_t)f32_to_f16(a1) << 16));
        }
        *(i32x4*)((uint16_t*)out + (int64_t)t * H + h) = q;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) store_dt(out, out_dt, (int64_t)t * H + h + i, scale * acc[i]);
      }
    }
  } else {
    for (int h = blockIdx.y * kChunk + threadIdx.x; h < h_end; h += kThreads) {
      float acc = 0.f;
      for (int k = 0; k < K; ++k) {
        if (pt[k] < 0) continue;
        float v = load_dt(y, YDT, (int64_t)pt[k] * H + h);
        if constexpr (YDT == 0)
          for (int c = 1; c < nchunk; ++c)
            v += ((const float*)y)[c * chunk_stride + (int64_t)pt[k] * H + h];
        acc = fmaf(wt[k], v, acc);
      }
      store_dt(out, out_dt, (int64_t)t * H + h, scale * acc);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dt, const float* w, const int32_t* route_pos,
                          int T, int K, int H, float scale, void* out, int out_dt,
                          hipStream_t s, int nchunk, int64_t chunk_stride) {
  if (nchunk > 1 && y_dt != 0) return hipErrorInvalidValue;
  if (T <= 0 || H <= 0) return hipSuccess;
  const bool vec = (H % 8) == 0;
  const dim3 grid(T, (H + kChunk - 1) / kChunk);
#define MOE_COMBINE(D)                                                                        \
  (vec ? combine_kernel<D, true><<<grid, kThreads, 0, s>>>(y, w, route_pos, T, K, H, scale, out, \
                                                           out_dt, nchunk, chunk_stride)       \
       : combine_kernel<D, false><<<grid, kThreads, 0, s>>>(y, w, route_pos, T, K, H, scale, out, \
                                                            out_dt, nchunk, chunk_stride))
  if (y_dt == 0) MOE_COMBINE(0);
  else if (y_dt == 1) MOE_COMBINE(1);
  else MOE_COMBINE(2);
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
