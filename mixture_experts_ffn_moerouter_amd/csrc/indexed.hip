// Indexed small-route expert MLP (the decode backend).
//
// [TO] TileOPs "MoE Operators", IndexedExpertMLPFwdOp: routes that share an expert are
//      grouped so each distinct expert's weights are read once; FusedMoEExpertsFwdOp
//      picks this backend when T*K <= 2E with silu_and_mul, no bias, H % 128 == 0 and
//      F % 256 == 0 (those are the widths these kernels are tiled for).
//
// With a handful of routes per expert the work is a stream of the touched experts'
// weights, so the kernels are built around reading weight rows at full HBM rate:
//   * A wave owns 32 weight rows (gate_up: 16 gate rows and the 16 matching up rows;
//     down: 32 rows of W_d) and streams them over the contraction (down: one chunk of
//     it, below) in 256-byte blocks. Each load instruction reads 4 rows x 256 contiguous bytes (16 lanes per
//     row), whole cache lines, the pattern that streams at full rate.
//   * MFMA operands need the opposite layout (a lane holds 8 contraction elements of ONE
//     row), so each block goes through a wave-private LDS tile: the wave writes the
//     block as loaded and reads it back in v_mfma_f32_16x16x32_bf16 operand order. The
//     16-byte slots are XOR-swizzled with the row so both directions are conflict-free.
//     No workgroup barrier is involved; LDS operations of one wave complete in order.
//   * Three blocks of loads are in flight per wave (register sets rotated by an unrolled
//     loop); the expert's routes (16 per pass) are the other MFMA operand, read straight
//     from the token rows (gate_up) or the activation rows (down). Weight loads are
//     non-temporal (each line is read once): 12 % faster on the whole decode layer than
//     the default policy.
// Inside a block the contraction order is permuted identically for both operands
// (MFMA u, lane quarter q takes the 8 elements of piece 4u + q), so the sums are those
// of the plain dot products up to float32 rounding order.
//   gate_up: act[route, j] = silu(h W_g[j]) * (h W_u[j]), rounded to the operand dtype
//            (bfloat16 or float16; the MFMA follows the dtype) (workspace)
//   down:    y[route, n]   = act[route] . W_d[n], float32 (workspace); the combine
//            kernel then sums the routes of each token. When F is a multiple of 512 the
//            contraction is split into chunks of 512 elements (1 KB of every row), one
//            work item per (32 rows, chunk), each writing its partial sums to its own y
//            slab; the combine adds a route's slabs in chunk order. The four waves of a
//            workgroup take the chunks of the same rows, so together they read each row's
//            bytes in one contiguous run; a load-only probe of the DeepSeek-V3 down shape
//            streams 6.0 TB/s with whole 4 KB rows per wave and 6.8-7.0 TB/s this way.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;       // waves per workgroup, each with its own work item
constexpr int kBlk = 128;       // contraction elements per block (256 bytes of a row)
constexpr int kSets = 3;        // blocks in flight per wave
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past every buffer range used here

__device__ __forceinline__ bf16x8 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Weight loads: each weight line is read once, so they are non-temporal (cache-policy
// operand 2); the route rows, read by every wave of the expert, keep the default policy.
__device__ __forceinline__ bf16x8 ld16_once(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * (1.0f / (1.0f + __expf(-g))) * u;
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// 16 x 16 x 32 MFMA on eight 16-bit elements per lane: DT 1 bfloat16, 2 float16.
template <int DT>
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One wave: rows row_g[0] + [0,16) and row_g[1] + [0,16) of the expert's weight matrix
// w (rows of Kd elements) against the routes [c0, c0 + 16) of the expert, over the
// contraction elements [k0, k0 + kn). acc[g] receives D[i][c] (lane: route c = lane % 16,
// rows 4*(lane/16)+r).
template <bool GATE_UP, int DT>
__device__ __forceinline__ void stream_rows(const IndexedArgs& p, bf16x8 (*stage)[16],
                                            __amdgpu_buffer_rsrc_t rw, const int* row_g,
                                            int Kd, int k0, int kn, int c0, int o1,
                                            f32x4* acc) {
  const int lane = threadIdx.x & 63;
  const int lr = lane >> 4, piece = lane & 15;  // load layout: row 4u + lr, 16-byte piece
  const int fr = lane & 15, fq = lane >> 4;     // MFMA layout: row / route fr, quarter fq
  // Weight offsets of this lane's 8 loads per block (group g, load u).
  uint32_t woff[8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      woff[g * 4 + u] = ((uint32_t)(row_g[g] + 4 * u + lr) * (uint32_t)Kd + k0 + piece * 8) * 2u;
  // Route operand: the row of route slot c0 + fr (token row for gate_up, permuted
  // activation row for down); pieces 4u + fq of each block.
  const int slot = c0 + fr;
  const bool has = slot < o1;
  const int src = has ? (GATE_UP ? p.sorted_route[slot] / p.K : slot) : 0;
  const void* xbase = GATE_UP ? (const void*)p.hidden : (const void*)p.act;
  const int xrows = GATE_UP ? p.T : p.T * p.K;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xbase, (short)0, (int)((int64_t)xrows * Kd * 2), 0x00020000);
  uint32_t xoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    xoff[u] = has ? ((uint32_t)src * (uint32_t)Kd + k0 + (4 * u + fq) * 8) * 2u : kOOB;

  const int nb = kn / kBlk;
  bf16x8 w0[8], w1[8], w2[8], x0[4], x1[4], x2[4];
  auto issue = [&](int b, bf16x8* w, bf16x8* x) {
    const bool in = b < nb;
    const uint32_t kb = (uint32_t)b * (kBlk * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = ld16_once(rw, in ? woff[i] + kb : kOOB);
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = ld16(rx, in ? xoff[u] + kb : kOOB);
  };
  auto step = [&](const bf16x8* w, const bf16x8* x) {
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * u + lr;
        stage[g * 16 + r][piece ^ r] = w[g * 4 + u];
      }
    __builtin_amdgcn_wave_barrier();
    bf16x8 f[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) f[g][u] = stage[g * 16 + fr][(4 * u + fq) ^ fr];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        acc[g] = mfma16<DT>(f[g][u], x[u], acc[g]);
  };

  issue(0, w0, x0);
  issue(1, w1, x1);
  issue(2, w2, x2);
  int b = 0;
  for (; b + kSets <= nb; b += kSets) {
    step(w0, x0);
    issue(b + 3, w0, x0);
    step(w1, x1);
    issue(b + 4, w1, x1);
    step(w2, x2);
    issue(b + 5, w2, x2);
  }
  if (b < nb) step(w0, x0);
  if (b + 1 < nb) step(w1, x1);
}

// Work items per expert: gate_up F/16 (16 act columns each), down H/32 (32 hidden rows)
// times the contraction chunks (chunk index fastest); each workgroup takes kWaves
// consecutive items of one expert.
template <bool GATE_UP, int DT>
__global__ __launch_bounds__(64 * kWaves, 2) void indexed_kernel(IndexedArgs p) {
  __shared__ bf16x8 stage_all[kWaves][32][16];
  const int nch = GATE_UP ? 1 : indexed_down_chunks(p.F);
  const int items = GATE_UP ? p.F / 16 : p.H / 32 * nch;
  const int wg_per_e = items / kWaves;
  const int a = blockIdx.x / wg_per_e;
  const int n_active = p.active[p.E];
  if (a >= n_active) return;  // uniform per workgroup
  const int e = p.active[a];
  const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = (blockIdx.x % wg_per_e) * kWaves + wave;
  const int item = wi / nch, ch = wi % nch;  // row block, contraction chunk
  const int H = p.H, F = p.F;
  const int Kd = GATE_UP ? H : F;
  const uint16_t* wexp = GATE_UP ? p.w_gate_up + (int64_t)e * 2 * F * H
                                 : p.w_down + (int64_t)e * H * F;
  const int nrows = GATE_UP ? 2 * F : H;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wexp, (short)0, (int)((int64_t)nrows * Kd * 2), 0x00020000);
  int row_g[2];
  if (GATE_UP) {
    row_g[0] = item * 16;      // gate rows j0 .. j0+15
    row_g[1] = F + item * 16;  // the matching up rows
  } else {
    row_g[0] = item * 32;
    row_g[1] = item * 32 + 16;
  }
  const int c = lane & 15, q = lane >> 4;
  for (int c0 = o0; c0 < o1; c0 += 16) {
    f32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    stream_rows<GATE_UP, DT>(p, stage_all[wave], rw, row_g, Kd, ch * (Kd / nch), Kd / nch, c0,
                             o1, acc);
    const int s = c0 + c;
    if (s < o1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * q + r;
        if (GATE_UP)
          p.act[(int64_t)s * F + item * 16 + i] = f32_to_h16<DT>(silu_mul(acc[0][r], acc[1][r]));
        else {
          float* ys = p.y + (int64_t)ch * p.T * p.K * H;  // this chunk's slab
          ys[(int64_t)s * H + item * 32 + i] = acc[0][r];
          ys[(int64_t)s * H + item * 32 + 16 + i] = acc[1][r];
        }
      }
    }
  }
}

}  // namespace

template <int DT>
hipError_t launch_indexed_dt(const IndexedArgs& a, int max_active, hipStream_t s) {
  indexed_kernel<true, DT><<<dim3(max_active * (a.F / 16 / kWaves)), 64 * kWaves, 0, s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int down_items = a.H / 32 * indexed_down_chunks(a.F);
  indexed_kernel<false, DT><<<dim3(max_active * (down_items / kWaves)), 64 * kWaves, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_indexed_mlp(const IndexedArgs& a, hipStream_t s) {
  const int R = a.T * a.K;
  const int max_active = R < a.E ? R : a.E;
  if (max_active <= 0) return hipSuccess;
  return a.dt == 2 ? launch_indexed_dt<2>(a, max_active, s) : launch_indexed_dt<1>(a, max_active, s);
}

}  // namespace moe
