// Grouped GEMM over the expert-contiguous layout, with an optional fused gated
// activation, for gfx950.
//
// [TO] TileOPs "MoE Operators", MoEGroupedGemmFwdOp: out[rows of e] = a[rows of e] b[e]^T
//      with b [E, N, K] (rows contiguous in K), float32 accumulation, optional bias [E, N]
//      added to the float32 product before the activation and the cast; with a gated
//      activation b holds gate and up rows (stacked or interleaved), the activation is
//      applied in the epilogue and the [.., 2F] product is never written.
// [MR] SwiGLU / [SPEC] SwiGLU Activation Function: G = min(g, limit),
//      L = clamp(l, -limit, limit), G * sigmoid(alpha G) * (L + beta), float math,
//      limit <= 0 disables both clamps.
//
// bf16 kernel: a 128 x 128 output tile per 256-thread workgroup, K in steps of 64 staged
// through LDS (double-buffered: the next step's global loads are in flight while the
// current step runs on the matrix cores), v_mfma_f32_32x32x16_bf16 with each wave owning
// a 64 x 64 sub-tile. For the gated activation the tile's 128 weight rows are 64 gate
// rows and the 64 matching up rows, placed in LDS so that a lane's gate and up
// accumulators hold the same output element; the epilogue pairs them directly. Rows of A
// may be gathered (a_rows), so the permuted activation copy is never materialised.
//
// Tile map: the number of 128-row tiles of each expert comes from expert_offsets on the
// device (no host synchronisation). The grid is an upper bound; every workgroup rebuilds
// the map in LDS, picks its (tile, n-tile) and leaves if it has none. Consecutive logical
// tiles go to the same XCD (workgroups are dealt round-robin over the 8 XCDs), so the
// n-tiles that share one A tile run close together on one L2.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;  // LDS row stride in elements
constexpr int NT = 256;
constexpr int kMaxE = 1024;
constexpr int kXcd = 8;

__device__ __forceinline__ float swiglu_f(float g, float l, float alpha, float beta,
                                          float limit) {
  if (limit > 0.f) {
    g = fminf(g, limit);
    l = fminf(fmaxf(l, -limit), limit);
  }
  return g * (1.0f / (1.0f + __expf(-alpha * g))) * (l + beta);
}

// Builds s_pre[0..E] = exclusive prefix of per-expert tile counts (and copies the
// offsets into s_off). Called by all NT threads.
// offsets == NULL means one expert that owns rows 0 .. M-1.
__device__ void build_tile_map(const int32_t* offsets, int E, int M, int bm, int* s_off,
                               int* s_pre, int* s_tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i <= E; i += NT) s_off[i] = offsets ? offsets[i] : (i == 0 ? 0 : M);
  __syncthreads();
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int e = e0 + tid;
    const int c = e < E ? (s_off[e + 1] - s_off[e] + bm - 1) / bm : 0;
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) s_tmp[wave] = x;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_tmp[w];
    const int chunk = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    if (e < E) s_pre[e] = carry + wbase + x - c;
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) s_pre[E] = carry;
  __syncthreads();
}

// Largest e with s_pre[e] <= tile (s_pre non-decreasing, s_pre[0] = 0).
__device__ __forceinline__ int find_expert(const int* s_pre, int E, int tile) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <bool ACT, int LAYOUT, bool OUT_F32>
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ int s_tmp[8];
  extern __shared__ __align__(16) uint16_t smem[];  // [2][BM + BN][LDK]
  // The tile map lives in the tile buffers until the K loop starts.
  int* s_off = (int*)smem;
  int* s_pre = s_off + kMaxE + 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = g.E;
  build_tile_map(g.offsets, E, g.M, BM, s_off, s_pre, s_tmp);

  const int n_tiles_n = ACT ? (g.Nout + BN / 2 - 1) / (BN / 2) : (g.Nw + BN - 1) / BN;
  const int n_valid = s_pre[E] * n_tiles_n;
  const int per = (n_valid + kXcd - 1) / kXcd;
  const int slot = blockIdx.x / kXcd;
  const int L = (blockIdx.x % kXcd) * per + slot;
  if (slot >= per || L >= n_valid) return;
  const int tile = L / n_tiles_n, nt = L % n_tiles_n;
  const int e = find_expert(s_pre, E, tile);
  const int m0 = s_off[e] + (tile - s_pre[e]) * BM;
  const int m1 = min(m0 + BM, s_off[e + 1]);
  const int Kd = g.Kd;
  __syncthreads();  // every thread has read the map; the buffers become tiles

  // ---- per-thread global source rows (4 A vectors, 4 B vectors of 8 elements)
  const uint16_t* pa[4];
  const uint16_t* pb[4];
  int kv[4], lrow[4];
  const uint16_t* A = (const uint16_t*)g.a;
  const uint16_t* B = (const uint16_t*)g.b + (int64_t)e * g.Nw * Kd;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = tid + NT * i;
    lrow[i] = v >> 3;
    kv[i] = (v & 7) * 8;
    int m = min(m0 + lrow[i], m1 - 1);
    int src = g.a_rows ? g.a_rows[m] / g.a_rows_div : m;
    pa[i] = A + (int64_t)src * Kd + kv[i];
    int r = lrow[i], wr;
    if (ACT) {
      const int j = min(nt * (BN / 2) + (r & (BN / 2 - 1)), g.Nout - 1);
      const bool up = r >= BN / 2;
      wr = LAYOUT == 0 ? (up ? g.Nout + j : j) : (2 * j + (up ? 1 : 0));
    } else {
      wr = min(nt * BN + r, g.Nw - 1);
    }
    pb[i] = B + (int64_t)wr * Kd + kv[i];
  }

  bf16x8 ra[4], rb[4];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = k0 + kv[i] < Kd;
      ra[i] = in ? *(const bf16x8*)(pa[i] + k0) : bf16x8{};
      rb[i] = in ? *(const bf16x8*)(pb[i] + k0) : bf16x8{};
    }
  };
  auto store_lds = [&](int buf) {
    uint16_t* sa = smem + buf * (BM + BN) * LDK;
    uint16_t* sb = sa + BM * LDK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(bf16x8*)(sa + lrow[i] * LDK + kv[i]) = ra[i];
      *(bf16x8*)(sb + lrow[i] * LDK + kv[i]) = rb[i];
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int arow0 = wm * 64 + (lane & 31);
  int brow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    brow[j] = (ACT ? (j * (BN / 2) + wn * 32) : (wn * 64 + j * 32)) + (lane & 31);
  const int kq = (lane >> 5) * 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (Kd + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const uint16_t* sa = smem + (kt & 1) * (BM + BN) * LDK;
    const uint16_t* sb = sa + BM * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = *(const bf16x8*)(sa + (arow0 + i * 32) * LDK + ks * 16 + kq);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *(const bf16x8*)(sb + brow[j] * LDK + ks * 16 + kq);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_lds((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue. Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4
  // and column l%32 of its 32 x 32 block.
  const uint16_t* bias = (const uint16_t*)g.bias;
  if (ACT) {
    const int j = nt * (BN / 2) + wn * 32 + (lane & 31);
    if (j < g.Nout) {
      float bg = 0.f, bu = 0.f;
      if (bias) {
        const uint16_t* be = bias + (int64_t)e * g.Nw;
        bg = bf16_to_f32(be[LAYOUT == 0 ? j : 2 * j]);
        bu = bf16_to_f32(be[LAYOUT == 0 ? g.Nout + j : 2 * j + 1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < m1) {
            float v = swiglu_f(acc[i][0][r] + bg, acc[i][1][r] + bu, g.alpha, g.beta, g.limit);
            if (OUT_F32) ((float*)g.out)[(int64_t)m * g.Nout + j] = v;
            else ((uint16_t*)g.out)[(int64_t)m * g.Nout + j] = f32_to_bf16(v);
          }
        }
    }
  } else {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int n = nt * BN + wn * 64 + jb * 32 + (lane & 31);
      if (n < g.Nw) {
        const float bn = bias ? bf16_to_f32(bias[(int64_t)e * g.Nw + n]) : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (m < m1) {
              float v = acc[i][jb][r] + bn;
              if (OUT_F32) ((float*)g.out)[(int64_t)m * g.Nw + n] = v;
              else ((uint16_t*)g.out)[(int64_t)m * g.Nw + n] = f32_to_bf16(v);
            }
          }
      }
    }
  }
}

// float32 operands: one workgroup per output row; the A row is staged in LDS and each
// thread forms the dot products of its output column(s). Plain FMA arithmetic; meant
// for small float32 problems.
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  extern __shared__ float srow[];
  const int m = blockIdx.x;
  const int32_t* off = g.offsets;  // NULL: one expert owning every row
  int e = 0;
  if (off) {
    if (m < off[0] || m >= off[g.E]) return;
    int lo = 0, hi = g.E - 1;  // largest e with off[e] <= m
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= m) lo = mid; else hi = mid - 1;
    }
    e = lo;
  }
  const int src = g.a_rows ? g.a_rows[m] / g.a_rows_div : m;
  const float* a = (const float*)g.a + (int64_t)src * g.Kd;
  for (int k = threadIdx.x; k < g.Kd; k += blockDim.x) srow[k] = a[k];
  __syncthreads();
  const float* B = (const float*)g.b + (int64_t)e * g.Nw * g.Kd;
  const float* bias = (const float*)g.bias;
  const int n = blockIdx.y * blockDim.x + threadIdx.x;
  if (n >= g.Nout) return;
  if (g.act) {
    const int rg = g.layout == 0 ? n : 2 * n, ru = g.layout == 0 ? g.Nout + n : 2 * n + 1;
    float sg = 0.f, su = 0.f;
    for (int k = 0; k < g.Kd; ++k) {
      sg = fmaf(srow[k], B[(int64_t)rg * g.Kd + k], sg);
      su = fmaf(srow[k], B[(int64_t)ru * g.Kd + k], su);
    }
    if (bias) {
      sg += bias[(int64_t)e * g.Nw + rg];
      su += bias[(int64_t)e * g.Nw + ru];
    }
    ((float*)g.out)[(int64_t)m * g.Nout + n] = swiglu_f(sg, su, g.alpha, g.beta, g.limit);
  } else {
    float s = 0.f;
    for (int k = 0; k < g.Kd; ++k) s = fmaf(srow[k], B[(int64_t)n * g.Kd + k], s);
    if (bias) s += bias[(int64_t)e * g.Nw + n];
    ((float*)g.out)[(int64_t)m * g.Nout + n] = s;
  }
}

template <bool ACT, int LAYOUT, bool OUT_F32>
hipError_t launch_bf16(const GemmArgs& g, hipStream_t s) {
  const int n_tiles_n = ACT ? (g.Nout + BN / 2 - 1) / (BN / 2) : (g.Nw + BN - 1) / BN;
  const int64_t max_tiles = (g.M + BM - 1) / BM + (g.E < g.M ? g.E : g.M);
  int64_t grid = max_tiles * n_tiles_n;
  grid = (grid + kXcd - 1) / kXcd * kXcd;
  const size_t lds = (size_t)2 * (BM + BN) * LDK * sizeof(uint16_t);
  hipError_t err = hipFuncSetAttribute((const void*)gemm_bf16_kernel<ACT, LAYOUT, OUT_F32>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  gemm_bf16_kernel<ACT, LAYOUT, OUT_F32><<<dim3((unsigned)grid), dim3(NT), lds, s>>>(g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (g.dt == 0) {
    dim3 grid(g.M, (g.Nout + 255) / 256);
    gemm_f32_kernel<<<grid, 256, (size_t)g.Kd * sizeof(float), s>>>(g);
    return hipGetLastError();
  }
  if (g.act) {
    if (g.layout == 0)
      return g.out_dt == 0 ? launch_bf16<true, 0, true>(g, s) : launch_bf16<true, 0, false>(g, s);
    return g.out_dt == 0 ? launch_bf16<true, 1, true>(g, s) : launch_bf16<true, 1, false>(g, s);
  }
  return g.out_dt == 0 ? launch_bf16<false, 0, true>(g, s) : launch_bf16<false, 0, false>(g, s);
}

}  // namespace moe
