// Permute: the expert-contiguous (tight, unpadded) order of the routes.
//
// [TO] TileOPs "MoE Operators", MoEPermuteAlignFwdOp (per-expert runs of route indices
//      in expert order, counts and their prefix) and MoEGroupedGemmFwdOp's contiguous
//      layout (one run of rows per expert, described by segment ends). Here the runs are
//      not padded, and inside a run the routes are in ascending route index.
//
// Two launches, no host synchronisation:
//  1. count: workgroup b counts the expert ids of routes [b*chunk, (b+1)*chunk) in LDS and
//     writes its row of the [nblk][E] count matrix;
//  2. scatter: workgroup b reads the matrix, forms expert_offsets (exclusive scan of the
//     column sums) and the rows that earlier workgroups take per expert, then walks its
//     chunk: wave w takes a contiguous slice, counts it per expert, and after a scan over
//     the waves goes through it 64 routes at a time, in order. Lanes that carry the same
//     expert find each other with one ballot per id bit; a lane's rank among its peers
//     plus the running base gives its row, and the lowest peer advances the base.
// Chunks, and slices inside them, are walked in route order, so the result is stable.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds_tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? lds_tmp[lane] : 0;
    int xs = w;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(xs, d, 64);
      if (lane >= d) xs += y;
    }
    if (lane < kWaves) lds_tmp[kWaves + lane] = xs - w;  // exclusive wave prefix
    if (lane == kWaves - 1) lds_tmp[2 * kWaves] = xs;
  }
  __syncthreads();
  int res = x - v + lds_tmp[kWaves + wave];
  total = lds_tmp[2 * kWaves];
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kThreads) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                                 int R, int E, int chunk,
                                                                 int32_t* __restrict__ blk_cnt) {
  extern __shared__ int lds[];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kThreads) lds[i] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * chunk, r1 = min(R, r0 + chunk);
  for (int r = r0 + tid; r < r1; r += kThreads) atomicAdd(&lds[ids[r]], 1);
  __syncthreads();
  for (int i = tid; i < E; i += kThreads) blk_cnt[(int64_t)blockIdx.x * E + i] = lds[i];
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nbits, int chunk, int nblk,
    const int32_t* __restrict__ blk_cnt, int32_t* offsets, int32_t* sorted_route,
    int32_t* route_pos, int32_t* active) {
  extern __shared__ int lds[];
  int* cnt = lds;                   // [kWaves][E]: counts, then running row bases
  int* tmp = lds + kWaves * E;      // scan scratch [2*kWaves+1]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int c0 = b * chunk, c1 = min(R, c0 + chunk);

  for (int i = tid; i < kWaves * E; i += kThreads) cnt[i] = 0;
  __syncthreads();
  const int per = (((c1 - c0 + kWaves - 1) / kWaves) + 63) / 64 * 64;
  const int r0 = min(c1, c0 + wave * per), r1 = min(c1, r0 + per);
  for (int r = r0 + lane; r < r1; r += 64) atomicAdd(&cnt[wave * E + ids[r]], 1);
  __syncthreads();

  // Per expert: column sum over all workgroups (scanned into offsets) and the rows of the
  // workgroups before this one; then this workgroup's per-wave bases.
  int carry = 0, carry_active = 0;
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + tid;
    int tot = 0, before = 0;
    if (e < E)
#pragma unroll 8
      for (int bb = 0; bb < nblk; ++bb) {  // unrolled: the count loads go out together
        const int c = blk_cnt[(int64_t)bb * E + e];
        tot += c;
        before += bb < b ? c : 0;
      }
    int chunk_total;
    int excl = block_exclusive_scan(tot, tmp, chunk_total) + carry;
    int act_total;
    int act_excl = block_exclusive_scan(tot > 0 ? 1 : 0, tmp, act_total) + carry_active;
    if (e < E) {
      if (b == 0) {
        offsets[e] = excl;
        if (active && tot > 0) active[act_excl] = e;
      }
      int base = excl + before;
      for (int w = 0; w < kWaves; ++w) {
        int c = cnt[w * E + e];
        cnt[w * E + e] = base;
        base += c;
      }
    }
    carry += chunk_total;
    carry_active += act_total;
  }
  if (b == 0 && tid == 0) {
    offsets[E] = R;
    if (active) active[E] = carry_active;
  }
  __syncthreads();

  // Stable scatter of this wave's slice.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int rb = r0; rb < r1; rb += 64) {
    const int r = rb + lane;
    const bool on = r < r1;
    const int e = on ? ids[r] : 0;
    uint64_t peers = __ballot(on);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t m = __ballot(on && set);
      peers &= set ? m : ~m;
    }
    if (on) {
      const int rank = __popcll(peers & lt_mask);
      const int pos = cnt[wave * E + e] + rank;
      sorted_route[pos] = r;
      route_pos[r] = pos;
      if (rank == 0) cnt[wave * E + e] = pos + __popcll(peers);
    }
  }
}

__global__ void gather_rows_kernel(const char* __restrict__ src, const int32_t* rows, int div,
                                   int M, int64_t row_bytes, char* __restrict__ dst) {
  const int m = blockIdx.x;
  if (m >= M) return;
  const char* s = src + (int64_t)(rows[m] / div) * row_bytes;
  char* d = dst + (int64_t)m * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (int64_t i = threadIdx.x * 16; i < row_bytes; i += blockDim.x * 16)
      *(i32x4*)(d + i) = *(const i32x4*)(s + i);
  } else {
    for (int64_t i = threadIdx.x; i < row_bytes; i += blockDim.x) d[i] = s[i];
  }
}

}  // namespace

size_t permute_workspace_bytes(int R, int E) {
  const int chunk = permute_chunk(R);
  const int nblk = R > 0 ? (R + chunk - 1) / chunk : 1;
  return (size_t)nblk * E * sizeof(int32_t);
}

int permute_chunk(int R) {
  // at least 1024 routes per workgroup, and at most 64 workgroups
  int c = (R + 63) / 64;
  c = (c + 511) / 512 * 512;
  return c < 1024 ? 1024 : c;
}

hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* offsets,
                          int32_t* sorted_route, int32_t* route_pos, int32_t* active,
                          int32_t* blk_cnt, hipStream_t s) {
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const int chunk = permute_chunk(R);
  const int nblk = R > 0 ? (R + chunk - 1) / chunk : 1;
  const size_t lds = (size_t)(kWaves * E + 2 * kWaves + 1) * sizeof(int);
  hipError_t err = hipFuncSetAttribute((const void*)permute_scatter_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  permute_count_kernel<<<nblk, kThreads, (size_t)E * sizeof(int), s>>>(ids, R, E, chunk,
                                                                       blk_cnt);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scatter_kernel<<<nblk, kThreads, lds, s>>>(ids, R, E, nbits, chunk, nblk, blk_cnt,
                                                     offsets, sorted_route, route_pos, active);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, const int32_t* rows, int div, int M,
                              int64_t row_bytes, void* dst, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  gather_rows_kernel<<<M, 256, 0, s>>>((const char*)src, rows, div, M, row_bytes, (char*)dst);
  return hipGetLastError();
}

}  // namespace moe
