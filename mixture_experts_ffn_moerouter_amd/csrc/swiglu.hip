// Standalone SwiGLU operator.
//
// [MR] ONNX Runtime PR 32126, SwiGLU: out = G * sigmoid(alpha G) * (L + beta) with
//      G = min(gate, limit), L = clamp(up, -limit, limit), float arithmetic whatever the
//      storage type, limit <= 0 disabling both clamps; up is optional, and without it gate
//      holds both halves of one [.., 2F] projection, gate first, then up.
// [SPEC] ONNX Runtime PR 25619, Fusion Behavior: the fused projection may also be
//      interleaved (element 2j gate j, 2j + 1 up j).
//
// An elementwise pass bound by HBM: each thread produces eight consecutive outputs of a
// row from one 16-byte (16-bit types) or 32-byte (float32) read of each operand, so every
// load and store is a full vector; rows whose width is not a multiple of eight (or
// pointers not 16-byte aligned) fall back to one element per thread. Grid-stride over
// rows x F/8 items. Every byte is read or written once, so the vector loads and stores
// are non-temporal (3.5 % faster than the default policy on 16384 x 2 x 4096 bf16).
#include "moe_internal.h"

namespace moe {
namespace {

template <int DT>
__device__ __forceinline__ void load8f(const void* base, int64_t i, float* v) {
  if constexpr (DT == 0) {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)((const float*)base + i)),
                b = __builtin_nontemporal_load((const f32x4*)((const float*)base + i + 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[k] = a[k]; v[4 + k] = b[k]; }
  } else {
    const i32x4 q = __builtin_nontemporal_load((const i32x4*)((const uint16_t*)base + i));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = h16_to_f32<DT>((uint16_t)((uint32_t)q[k] & 0xffffu));
      v[2 * k + 1] = h16_to_f32<DT>((uint16_t)((uint32_t)q[k] >> 16));
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8f(void* base, int64_t i, const float* v) {
  if constexpr (DT == 0) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4*)((float*)base + i));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, (f32x4*)((float*)base + i + 4));
  } else {
    i32x4 q;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      q[k] = (int)((uint32_t)f32_to_h16<DT>(v[2 * k]) | ((uint32_t)f32_to_h16<DT>(v[2 * k + 1]) << 16));
    __builtin_nontemporal_store(q, (i32x4*)((uint16_t*)base + i));
  }
}

// MODE 0: gate and up separate [rows, F]; 1: fused stacked [rows, 2F]; 2: fused interleaved.
// One item is eight consecutive outputs of a row.
template <int DT, int MODE>
__global__ __launch_bounds__(256) void swiglu_vec_kernel(SwigluArgs a) {
  const int F = a.F, per_row = F / 8;
  const int64_t items = a.rows * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
    const int64_t r = it / per_row;
    const int j = (int)(it - r * per_row) * 8;
    float g[8], u[8];
    if constexpr (MODE == 0) {
      load8f<DT>(a.gate, r * F + j, g);
      load8f<DT>(a.up, r * F + j, u);
    } else if constexpr (MODE == 1) {
      load8f<DT>(a.gate, r * 2 * F + j, g);
      load8f<DT>(a.gate, r * 2 * F + F + j, u);
    } else {
      float p[16];
      load8f<DT>(a.gate, r * 2 * F + 2 * j, p);
      load8f<DT>(a.gate, r * 2 * F + 2 * j + 8, p + 8);
#pragma unroll
      for (int k = 0; k < 8; ++k) { g[k] = p[2 * k]; u[k] = p[2 * k + 1]; }
    }
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = swiglu_f(g[k], u[k], a.alpha, a.beta, a.limit);
    store8f<DT>(a.out, r * F + j, o);
  }
}

__global__ __launch_bounds__(256) void swiglu_scalar_kernel(SwigluArgs a) {
  const int F = a.F;
  const int64_t n = a.rows * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / F;
    const int j = (int)(i - r * F);
    float g, u;
    if (a.up) {
      g = load_dt(a.gate, a.dt, i);
      u = load_dt(a.up, a.dt, i);
    } else if (a.fusion == 0) {
      g = load_dt(a.gate, a.dt, r * 2 * F + j);
      u = load_dt(a.gate, a.dt, r * 2 * F + F + j);
    } else {
      g = load_dt(a.gate, a.dt, r * 2 * F + 2 * j);
      u = load_dt(a.gate, a.dt, r * 2 * F + 2 * j + 1);
    }
    store_dt(a.out, a.dt, i, swiglu_f(g, u, a.alpha, a.beta, a.limit));
  }
}

template <int DT>
void launch_vec(const SwigluArgs& a, int grid, hipStream_t s) {
  const int mode = a.up ? 0 : (a.fusion == 0 ? 1 : 2);
  if (mode == 0) swiglu_vec_kernel<DT, 0><<<grid, 256, 0, s>>>(a);
  else if (mode == 1) swiglu_vec_kernel<DT, 1><<<grid, 256, 0, s>>>(a);
  else swiglu_vec_kernel<DT, 2><<<grid, 256, 0, s>>>(a);
}

}  // namespace

hipError_t launch_swiglu(const SwigluArgs& a, hipStream_t s) {
  if (a.rows <= 0 || a.F <= 0) return hipSuccess;
  // vector path: whole 8-element groups and 16-byte aligned rows
  const uintptr_t al = (uintptr_t)a.gate | (uintptr_t)a.up | (uintptr_t)a.out;
  const bool vec = a.F % 8 == 0 && (al & 15) == 0;
  const int64_t items = vec ? a.rows * (a.F / 8) : a.rows * a.F;
  const int64_t want = (items + 255) / 256;
  const int grid = (int)(want < 256 * 8 ? want : 256 * 8);  // 8 workgroups per CU at most
  if (!vec) {
    swiglu_scalar_kernel<<<grid, 256, 0, s>>>(a);
  } else if (a.dt == 0) {
    launch_vec<0>(a, grid, s);
  } else if (a.dt == 1) {
    launch_vec<1>(a, grid, s);
  } else {
    launch_vec<2>(a, grid, s);
  }
  return hipGetLastError();
}

}  // namespace moe
