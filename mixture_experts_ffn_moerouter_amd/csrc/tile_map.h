// Device-side tile map shared by the grouped GEMM kernels.
//
// Expert e with M_e rows is cut into ceil(M_e / bm) row tiles of equal height (rounded up
// to 32 rows). Every workgroup rebuilds the exclusive prefix of the per-expert tile counts
// in LDS from the expert row counts on the device (no host synchronisation) and finds its
// expert by binary search.
#pragma once
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ int tiles_of(int rows, int bm) { return (rows + bm - 1) / bm; }
__device__ __forceinline__ int rows_per_tile(int rows, int bm) {
  const int n = tiles_of(rows, bm);
  return n ? ((rows + n - 1) / n + 31) / 32 * 32 : 0;
}

// s_pre[0..E] = exclusive prefix of tiles_of(rows_of(e), bm). All NT threads; s_tmp holds
// NT / 64 ints.
template <int NT, class RowsOf>
__device__ void scan_tiles(int E, int bm, RowsOf rows_of, int* s_pre, int* s_tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int W = NT / 64;
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int e = e0 + tid;
    const int c = e < E ? tiles_of(rows_of(e), bm) : 0;
    int x = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) s_tmp[wave] = x;
    __syncthreads();
    int wbase = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      wbase += w < wave ? s_tmp[w] : 0;
      chunk += s_tmp[w];
    }
    if (e < E) s_pre[e] = carry + wbase + x - c;
    carry += chunk;
    __syncthreads();
  }
  if (tid == 0) s_pre[E] = carry;
  __syncthreads();
}

// Any layout: s_start[e] / s_len[e] = expert e's rows [start, start + len) inside [0, M),
// from the metadata per mode (kSegOffsets, kSegEnds, kSegMasked, kSegRuns; see GemmArgs),
// clamped to the rows that exist; and s_pre.
template <int NT>
__device__ void build_tile_map_segments(int mode, const int32_t* meta, int E, int M, int max_m,
                                        int bm, int* s_start, int* s_len, int* s_pre,
                                        int* s_tmp) {
  for (int e = threadIdx.x; e < E; e += NT) {
    int lo, hi;
    if (mode == kSegOffsets) {
      lo = meta ? meta[e] : (e == 0 ? 0 : M);
      hi = meta ? meta[e + 1] : M;
    } else if (mode == kSegEnds) {
      lo = e ? meta[e - 1] : 0;
      hi = meta[e];
    } else if (mode == kSegMasked) {
      lo = e * max_m;
      hi = lo + min(max(meta[e], 0), max_m);
    } else {
      lo = meta[2 * e];
      hi = meta[2 * e + 1];
    }
    lo = min(max(lo, 0), M);
    hi = min(max(hi, lo), M);
    s_start[e] = lo;
    s_len[e] = hi - lo;
  }
  __syncthreads();
  scan_tiles<NT>(E, bm, [&](int e) { return s_len[e]; }, s_pre, s_tmp);
}

// Masked layout: s_cnt[e] = counts[e] clamped to [0, max_m], and s_pre.
template <int NT>
__device__ void build_tile_map_masked(const int32_t* counts, int E, int max_m, int bm,
                                      int* s_cnt, int* s_pre, int* s_tmp) {
  for (int i = threadIdx.x; i < E; i += NT) s_cnt[i] = min(max(counts[i], 0), max_m);
  __syncthreads();
  scan_tiles<NT>(E, bm, [&](int e) { return s_cnt[e]; }, s_pre, s_tmp);
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

}  // namespace moe
