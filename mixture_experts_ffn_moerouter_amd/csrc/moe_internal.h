// Internal declarations shared by the HIP translation units of libmoe.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ device helpers
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// bfloat16 <-> float32. The narrowing rounds to nearest, ties to even (the usual
// add-0x7fff-plus-lsb method); NaNs stay NaN.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// 16-bit operand types by dtype code: 1 bfloat16, 2 float16.
template <int DT> __device__ __forceinline__ float h16_to_f32(uint16_t h) {
  return DT == 2 ? f16_to_f32(h) : bf16_to_f32(h);
}
template <int DT> __device__ __forceinline__ uint16_t f32_to_h16(float f) {
  return DT == 2 ? f32_to_f16(f) : f32_to_bf16(f);
}
// Load one element of dtype `dt` (0 f32, 1 bf16, 2 f16) as float32.
__device__ __forceinline__ float load_dt(const void* p, int dt, int64_t i) {
  if (dt == 0) return ((const float*)p)[i];
  const uint16_t h = ((const uint16_t*)p)[i];
  return dt == 1 ? bf16_to_f32(h) : f16_to_f32(h);
}

// [MR] SwiGLU / [SPEC] SwiGLU Activation Function, float32: G = min(g, limit),
// L = clamp(l, -limit, limit), G * sigmoid(alpha G) * (L + beta); limit <= 0 disables
// both clamps.
__device__ __forceinline__ float swiglu_f(float g, float l, float alpha, float beta,
                                          float limit) {
  if (limit > 0.f) {
    g = fminf(g, limit);
    l = fminf(fmaxf(l, -limit), limit);
  }
  return g * (1.0f / (1.0f + __expf(-alpha * g))) * (l + beta);
}

// Exact GELU, x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2, float32.
__device__ __forceinline__ float gelu_f(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// Store one float32 value in dtype `dt` (0 f32, 1 bf16, 2 f16) at element i of p.
__device__ __forceinline__ void store_dt(void* p, int dt, int64_t i, float v) {
  if (dt == 0) ((float*)p)[i] = v;
  else if (dt == 1) ((uint16_t*)p)[i] = f32_to_bf16(v);
  else ((uint16_t*)p)[i] = f32_to_f16(v);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ------------------------------------------------------------------ launchers
// Each returns a hipError_t; arguments are validated by the caller (api.hip).
struct RouteArgs {
  const void* logits;     // [T, E] in logits_dt
  int logits_dt;          // 0 f32, 1 bf16, 2 f16
  const float* bias;
  const int32_t* expert_ids;
  int T, E, K, scoring, renormalize, G, TG;
  float rsf;
  float* topk_w;
  int32_t* topk_ids;
  void* router_probs;
  void* weight_scale;
  int rp_dtype, local_start, local_count;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// active_list: optional [E+1] int32 out; active_list[0..n) = experts with routes, in
// ascending order, and active_list[E] = n. blk_cnt: device scratch of
// permute_workspace_bytes(R, E) bytes (per-workgroup expert counts).
int permute_chunk(int R);
size_t permute_workspace_bytes(int R, int E);
hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* offsets,
                          int32_t* sorted_route, int32_t* route_pos, int32_t* active_list,
                          int32_t* blk_cnt, hipStream_t s);
hipError_t launch_gather_rows(const void* src, const int32_t* rows, int div, int M,
                              int64_t row_bytes, void* dst, hipStream_t s);

// Padded and masked layouts (layout.hip). align_len = entries of sorted_token_ids.
__host__ __device__ inline int align_len(int R, int E, int bs) { return R + (E + 1) * (bs - 1); }
hipError_t launch_align(const int32_t* off, const int32_t* sorted_route, int R, int E, int bs,
                        int32_t* padded_off, int32_t* sorted_ids, int32_t* expert_blk,
                        int32_t* num_post_pad, int32_t* seg_ends, hipStream_t s);
// Contiguous / per-row pre-permute with the align step fused in (from the tight permute's
// offsets and order): rows, inverse indices, per-row expert ids and/or segment ends.
hipError_t launch_align_rows(const void* hidden, int64_t row_bytes, int K, const int32_t* off,
                             const int32_t* sorted_route, int E, int bs, int cap, void* out,
                             int32_t* inverse, int32_t* row_ids, int32_t* seg_ends,
                             hipStream_t s);
hipError_t launch_masked_rows(const void* hidden, int64_t row_bytes, int K, int R,
                              const int32_t* off, const int32_t* sorted_route, int E,
                              int max_m, void* out, int32_t* counts, int32_t* inverse,
                              hipStream_t s);
hipError_t launch_row_runs(const int32_t* ids, int M, int E, int32_t* pairs, hipStream_t s);

// Row segments of the experts in a grouped GEMM (see build_tile_map_segments):
//   kSegOffsets  offsets[E+1] (tight layout; null = one expert owning rows 0 .. M-1)
//   kSegEnds     segment ends[E] (contiguous layout, possibly padded)
//   kSegMasked   counts[E], expert e owns rows e*max_m .. e*max_m + clamp(count) - 1
//   kSegRuns     pairs[2E] of [start, end) (the per-row layout, after launch_row_runs)
enum { kSegOffsets = 0, kSegEnds = 1, kSegMasked = 2, kSegRuns = 3 };

struct GemmArgs {
  const void* a;
  const int32_t* a_rows;
  int a_rows_div;
  int M, Kd;          // logical rows, contraction length
  const void* b;      // [E, Nw, Kd]
  const void* bias;   // [E, Nw] or null
  const int32_t* offsets;  // segment metadata, per seg_mode
  int seg_mode;
  int max_m;          // kSegMasked
  int E, Nw;          // weight rows per expert
  int act;            // 0 none, 1 gated activation
  int act_kind;       // 0 swiglu family (alpha, beta, limit), 1 gelu_and_mul
  int layout;         // moe_gu_layout when act
  float alpha, beta, limit;
  void* out;          // [M, Nout]
  int Nout;           // Nw or Nw/2
  int dt, out_dt;
  int tag;            // 1: the shared expert's launch (a separately named kernel instance)
};
hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t s);

// y may hold nchunk partial slabs ([nchunk][rows][H], float32 only when nchunk > 1), added
// in slab order before the route weight is applied.
hipError_t launch_combine(const void* y, int y_dt, const float* w, const int32_t* route_pos,
                          int T, int K, int H, float scale, void* out, int out_dt,
                          hipStream_t s, int nchunk = 1, int64_t chunk_stride = 0);

// The indexed backend's down projection splits the contraction into chunks of 512
// elements when F allows (each chunk's partial sums form one float32 y slab).
__host__ __device__ inline int indexed_down_chunks(int F) { return F % 512 == 0 ? F / 512 : 1; }

// Indexed small-route backend (bf16 or f16, silu_and_mul, no bias).
struct IndexedArgs {
  const uint16_t* hidden;     // [T, H]
  const int32_t* sorted_route;
  const int32_t* offsets;     // [E+1]
  const int32_t* active;      // [E+1] from launch_permute
  const uint16_t* w_gate_up;  // [E, 2F, H] stacked
  const uint16_t* w_down;     // [E, H, F]
  int T, H, E, F, K;
  int dt;                     // 1 bf16, 2 f16
  uint16_t* act;              // [R, F] workspace (permuted rows)
  float* y;                   // [indexed_down_chunks(F)][R, H] workspace (permuted rows)
};
hipError_t launch_indexed_mlp(const IndexedArgs& a, hipStream_t s);

// Block-scaled FP8 grouped GEMM over a masked slab (bf16 out).
struct Fp8GemmArgs {
  const uint8_t* a;       // [E, max_m, K] e4m3fn
  const float* a_scale;   // [E, max_m, K/128]
  const uint8_t* b;       // [E, N, K] e4m3fn
  const float* b_scale;   // [E, N/128, K/128]
  const int32_t* counts;  // [E]
  int E, max_m, K, N;
  uint16_t* out;          // [E, max_m, N] bf16
};
hipError_t launch_gemm_fp8_masked(const Fp8GemmArgs& g, hipStream_t s);

// Standalone gated activation: out[r, j] = act(gate[r, j], up[r, j]) over rows x F.
struct SwigluArgs {
  const void* gate;   // [rows, F] (up given) or [rows, 2F] (fused)
  const void* up;     // [rows, F] or null
  int64_t rows;
  int F;
  int fusion;         // up null: 0 stacked (gate then up), 1 interleaved
  int dt;             // 0 f32, 1 bf16, 2 f16 (inputs and output)
  float alpha, beta, limit;
  void* out;          // [rows, F]
};
hipError_t launch_swiglu(const SwigluArgs& a, hipStream_t s);

}  // namespace moe
