// Indexed small-route expert MLP (the decode backend).
//
// [TO] TileOPs "MoE Operators", IndexedExpertMLPFwdOp: routes that share an expert are
//      grouped so each distinct expert's weights are read once; FusedMoEExpertsFwdOp
//      picks this backend when T*K <= 2E with silu_and_mul, no bias, H % 128 == 0 and
//      F % 256 == 0 (those are the widths these kernels are tiled for).
//
// Work items are (distinct expert, 64-row slice of its weights). A wave owns 16 weight
// rows (for gate_up: 16 gate rows and the 16 matching up rows) and streams them over
// the full contraction straight from HBM into v_mfma_f32_16x16x32_bf16 operands, with
// the expert's routes (at most 16 per pass) as the other operand. The order of the
// contraction inside a 128-wide block is permuted (both operands alike, so the sum is
// unchanged) so that each lane reads 64 contiguous bytes of a row per block.
//   gate_up: act[route, j] = silu(h W_g[j]) * (h W_u[j]), rounded to bf16 (workspace)
//   down:    y[route, n]   = act[route] . W_d[n], float32 (workspace); the combine
//            kernel then sums the routes of each token.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // 64
constexpr int kKBlock = 128;
constexpr int kUnroll = 2;  // 128-wide blocks in flight per lane

// One 128-wide contraction block: lane (row l%16, quarter q = l/16) holds the 32
// consecutive elements [q*32, q*32+32) as four 8-element pieces; piece u feeds MFMA u.
struct Frag {
  bf16x8 p[4];
};

__device__ __forceinline__ Frag load_frag(const uint16_t* row_block_base, int q) {
  Frag f;
  const bf16x8* src = (const bf16x8*)(row_block_base + q * 32);
#pragma unroll
  for (int u = 0; u < 4; ++u) f.p[u] = __builtin_nontemporal_load(src + u);
  return f;
}

__device__ __forceinline__ Frag load_frag_cached(const uint16_t* row_block_base, int q) {
  Frag f;
  const bf16x8* src = (const bf16x8*)(row_block_base + q * 32);
#pragma unroll
  for (int u = 0; u < 4; ++u) f.p[u] = src[u];
  return f;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * (1.0f / (1.0f + __expf(-g))) * u;
}

// gate_up: grid.x = max distinct experts, grid.y = F / 64.
__global__ __launch_bounds__(64 * kWaves) void indexed_gate_up_kernel(IndexedArgs p) {
  const int n_active = p.active[p.E];
  if ((int)blockIdx.x >= n_active) return;
  const int e = p.active[blockIdx.x];
  const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, q = lane >> 4;
  const int j = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave + row;  // act column
  const int H = p.H, F = p.F;
  const uint16_t* wg = p.w_gate_up + ((int64_t)e * 2 * F + j) * H;
  const uint16_t* wu = p.w_gate_up + ((int64_t)e * 2 * F + F + j) * H;

  for (int c0 = o0; c0 < o1; c0 += 16) {
    const int slot = c0 + row;  // route slot this lane feeds on the B side
    const bool has = slot < o1;
    const uint16_t* xr = p.hidden + (int64_t)(has ? p.sorted_route[slot] / p.K : 0) * H;
    f32x4 ag = {0, 0, 0, 0}, au = {0, 0, 0, 0};
    for (int k0 = 0; k0 < H; k0 += kKBlock * kUnroll) {
      Frag fg[kUnroll], fu[kUnroll], fx[kUnroll];
#pragma unroll
      for (int b = 0; b < kUnroll; ++b) {
        const int kb = k0 + b * kKBlock;
        const bool in = kb < H;  // H % 128 == 0; the last pair may be half empty
        for (int u = 0; u < 4; ++u) fg[b].p[u] = fu[b].p[u] = fx[b].p[u] = bf16x8{};
        if (in) {
          fg[b] = load_frag(wg + kb, q);
          fu[b] = load_frag(wu + kb, q);
          if (has) fx[b] = load_frag_cached(xr + kb, q);
        }
      }
#pragma unroll
      for (int b = 0; b < kUnroll; ++b)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fg[b].p[u], fx[b].p[u], ag, 0, 0, 0);
          au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fu[b].p[u], fx[b].p[u], au, 0, 0, 0);
        }
    }
    // D[i][s]: lane holds route slot s = lane%16 and weight rows i = 4*(lane/16) + r.
    const int s = c0 + (lane & 15);
    if (s < o1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave + 4 * q + r;
        p.act[(int64_t)s * F + jj] = f32_to_bf16(silu_mul(ag[r], au[r]));
      }
    }
  }
}

// down: grid.x = max distinct experts, grid.y = H / 64.
__global__ __launch_bounds__(64 * kWaves) void indexed_down_kernel(IndexedArgs p) {
  const int n_active = p.active[p.E];
  if ((int)blockIdx.x >= n_active) return;
  const int e = p.active[blockIdx.x];
  const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, q = lane >> 4;
  const int n = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave + row;  // hidden index
  const int H = p.H, F = p.F;
  const uint16_t* wd = p.w_down + ((int64_t)e * H + n) * F;

  for (int c0 = o0; c0 < o1; c0 += 16) {
    const int slot = c0 + row;
    const bool has = slot < o1;
    const uint16_t* ar = p.act + (int64_t)(has ? slot : 0) * F;
    f32x4 acc = {0, 0, 0, 0};
    for (int k0 = 0; k0 < F; k0 += kKBlock * kUnroll) {
      Frag fw[kUnroll], fa[kUnroll];
#pragma unroll
      for (int b = 0; b < kUnroll; ++b) {
        const int kb = k0 + b * kKBlock;
        const bool in = kb < F;
        for (int u = 0; u < 4; ++u) fw[b].p[u] = fa[b].p[u] = bf16x8{};
        if (in) {
          fw[b] = load_frag(wd + kb, q);
          if (has) fa[b] = load_frag_cached(ar + kb, q);
        }
      }
#pragma unroll
      for (int b = 0; b < kUnroll; ++b)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[b].p[u], fa[b].p[u], acc, 0, 0, 0);
    }
    const int s = c0 + (lane & 15);
    if (s < o1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int nn = blockIdx.y * kRowsPerBlock + wave * kRowsPerWave + 4 * q + r;
        p.y[(int64_t)s * H + nn] = acc[r];
      }
    }
  }
}

}  // namespace

hipError_t launch_indexed_mlp(const IndexedArgs& a, hipStream_t s) {
  const int R = a.T * a.K;
  const int max_active = R < a.E ? R : a.E;
  if (max_active <= 0) return hipSuccess;
  indexed_gate_up_kernel<<<dim3(max_active, a.F / kRowsPerBlock), 64 * kWaves, 0, s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  indexed_down_kernel<<<dim3(max_active, a.H / kRowsPerBlock), 64 * kWaves, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
