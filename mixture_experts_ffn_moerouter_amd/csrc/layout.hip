// Padded and masked expert layouts: permute-align, pre-permute, per-row segment discovery.
//
// [TO] TileOPs "MoE Operators":
//   MoEPermuteAlignFwdOp - with numel = T*K routes and count[e] of them on expert e:
//     num_tokens_post_pad = sum over e of count[e] rounded up to block_size;
//     sorted_token_ids[:num_tokens_post_pad] = one range per expert, in expert order, of
//     that rounded-up length, holding the expert's routes first and numel after; past it
//     every entry is numel; expert_ids names the owner of each block of the ranges and
//     lies outside [0, E) past them. The order inside a range is left open; here it is
//     ascending route index (the tight permute's order).
//   MoEPrePermuteFwdOp - (expert_input, layout_metadata, inverse_indices) for one layout
//     of MoEGroupedGemmFwdOp's table: contiguous rows with segment ends, contiguous rows
//     with a per-row expert id, or a masked [E, max_m, H] slab with valid counts.
//
// Everything starts from the tight permute (expert_offsets, sorted_route, route_pos), so
// all layouts share its order. Permute-align is one integer pass; the contiguous and
// per-row pre-permute fuse that pass into the row copy (16-byte pieces, several rows per
// wave in flight), bound by the hidden rows they move.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kNT = 256;        // threads per workgroup of the layout kernels
constexpr int kMaxE = 1024;     // experts the LDS prefix holds
constexpr int kRowsPerWave = 2;  // destination rows a wave of align_rows_kernel copies

// s_pad[e] = exclusive prefix over experts of round_up(count[e], bs), s_pad[E] = the used
// length, for the whole workgroup (kNT threads; thread t sums experts 4t .. 4t + 3, then a
// wave scan and a scan of the four wave totals). Ends with a barrier.
__device__ void padded_prefix(const int32_t* __restrict__ off, int E, int bs, int* s_pad,
                              int* s_w) {
  constexpr int P = kMaxE / kNT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int v[P], sum = 0;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int e = P * t + j;
    const int cnt = e < E ? off[e + 1] - off[e] : 0;
    v[j] = (cnt + bs - 1) / bs * bs;
    sum += v[j];
  }
  int x = sum;  // inclusive scan of the thread sums within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) {
    base += w < wave ? s_w[w] : 0;
    total += s_w[w];
  }
  int run = base + x - sum;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int e = P * t + j;
    if (e < E) s_pad[e] = run;
    run += v[j];
  }
  if (t == 0) s_pad[E] = total;
  __syncthreads();
}

// Largest e in [0, E) with padded_off[e] <= s (the expert whose padded range holds s when
// s < padded_off[E]; empty experts share their successor's start and lose to it).
__device__ __forceinline__ int owner_of(const int* padded_off, int E, int s) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (padded_off[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Permute-align: one thread per slot s < len of sorted_token_ids (and the block entry when
// s % bs == 0); every workgroup forms the padded prefix itself, workgroup 0 also stores it
// (padded_off, and the optional num_post_pad / seg_ends copies).
__global__ __launch_bounds__(kNT) void align_fill_kernel(
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted_route, int E, int bs,
    int numel, int len, int32_t* __restrict__ padded_off, int32_t* __restrict__ num_post_pad,
    int32_t* __restrict__ seg_ends, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_blk) {
  __shared__ int s_pad[kMaxE + 1];
  __shared__ int s_w[kNT / 64];
  padded_prefix(off, E, bs, s_pad, s_w);
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e <= E; e += kNT) {
      padded_off[e] = s_pad[e];
      if (seg_ends && e < E) seg_ends[e] = s_pad[e + 1];
    }
    if (num_post_pad && threadIdx.x == 0) num_post_pad[0] = s_pad[E];
  }
  const int s = blockIdx.x * kNT + threadIdx.x;
  if (s >= len) return;
  const int used = s_pad[E];
  int val = numel, owner = -1;
  if (s < used) {
    owner = owner_of(s_pad, E, s);
    const int i = s - s_pad[owner];
    if (i < off[owner + 1] - off[owner]) val = sorted_route[off[owner] + i];
  }
  sorted_ids[s] = val;
  if (s % bs == 0) expert_blk[s / bs] = owner;
}

// Copy of 16-byte pieces (or bytes) of one row.
__device__ __forceinline__ void copy_row(const char* __restrict__ src, char* __restrict__ dst,
                                         int64_t row_bytes) {
  if ((row_bytes & 15) == 0) {
    for (int64_t i = threadIdx.x * 16; i < row_bytes; i += blockDim.x * 16)
      *(i32x4*)(dst + i) = *(const i32x4*)(src + i);
  } else {
    for (int64_t i = threadIdx.x; i < row_bytes; i += blockDim.x) dst[i] = src[i];
  }
}

// Contiguous / per-row pre-permute, the align step fused in: destination row m < cap holds
// the i-th route of expert e when m = padded_off[e] + i and i < count[e]. Every workgroup
// forms the padded prefix itself, then each wave takes kRowsPerWave rows: their routes are
// found first (owner by binary search, route from the tight order), then every 16-byte
// piece of those rows is loaded before any is stored (eight loads in flight per lane on
// 4 KB rows). Writes the row (non-temporal: nothing here reads it back), the route's
// inverse index and, for the per-row layout, the row's expert id (-1 on padding and unused
// rows); workgroup 0 writes the segment ends of the contiguous layout.
__global__ __launch_bounds__(kNT) void align_rows_kernel(
    const char* __restrict__ hidden, int64_t row_bytes, int K, const int32_t* __restrict__ off,
    const int32_t* __restrict__ sorted_route, int E, int bs, int cap, char* __restrict__ out,
    int32_t* __restrict__ inverse, int32_t* __restrict__ row_ids,
    int32_t* __restrict__ seg_ends) {
  constexpr int U = 4;  // 1 KB pieces of a row per wave and round
  __shared__ int s_pad[kMaxE + 1];
  __shared__ int s_w[kNT / 64];
  padded_prefix(off, E, bs, s_pad, s_w);
  if (seg_ends && blockIdx.x == 0)
    for (int e = threadIdx.x; e < E; e += kNT) seg_ends[e] = s_pad[e + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int used = s_pad[E];
  const int m0 = (blockIdx.x * (kNT / 64) + wave) * kRowsPerWave;
  int src[kRowsPerWave];  // source token row, or -1 (padding, unused or past cap)
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const int m = m0 + r;
    int route = -1, owner = -1;
    if (m < cap && m < used) {
      owner = owner_of(s_pad, E, m);
      const int i = m - s_pad[owner];
      if (i < off[owner + 1] - off[owner]) route = sorted_route[off[owner] + i];
    }
    src[r] = __builtin_amdgcn_readfirstlane(route < 0 ? -1 : route / K);
    if (lane == 0 && m < cap) {
      if (route >= 0) inverse[route] = m;
      if (row_ids) row_ids[m] = route >= 0 ? owner : -1;
    }
  }
  if ((row_bytes & 15) == 0) {
    for (int64_t b0 = 16 * lane; b0 < row_bytes; b0 += 1024 * U) {
      i32x4 v[kRowsPerWave][U];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t b = b0 + 1024 * u;
          if (src[r] >= 0 && b < row_bytes)
            v[r][u] = *(const i32x4*)(hidden + (int64_t)src[r] * row_bytes + b);
        }
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t b = b0 + 1024 * u;
          if (src[r] >= 0 && b < row_bytes)
            __builtin_nontemporal_store(v[r][u],
                                        (i32x4*)(out + (int64_t)(m0 + r) * row_bytes + b));
        }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
      if (src[r] >= 0)
        for (int64_t b = lane; b < row_bytes; b += 64)
          out[(int64_t)(m0 + r) * row_bytes + b] = hidden[(int64_t)src[r] * row_bytes + b];
  }
}

// Masked pre-permute: slab row (e, j), j < min(count[e], max_m), holds route
// sorted_route[off[e] + j]; counts[e] = min(count[e], max_m) (written by row (e, 0)).
__global__ __launch_bounds__(256) void masked_rows_kernel(
    const char* __restrict__ hidden, int64_t row_bytes, int K, const int32_t* __restrict__ off,
    const int32_t* __restrict__ sorted_route, int max_m, char* __restrict__ out,
    int32_t* __restrict__ counts, int32_t* __restrict__ inverse) {
  const int e = blockIdx.y, j = blockIdx.x;
  const int cnt = min(off[e + 1] - off[e], max_m);
  if (j == 0 && threadIdx.x == 0) counts[e] = cnt;
  if (j >= cnt) return;
  const int src = sorted_route[off[e] + j];
  const int64_t row = (int64_t)e * max_m + j;
  if (threadIdx.x == 0) inverse[src] = (int32_t)row;
  copy_row(hidden + (int64_t)(src / K) * row_bytes, out + row * row_bytes, row_bytes);
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n,
                                                       int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Per-row layout: the row range [start, end) of each expert's run, from the row ids
// (expert e's rows form one run: the layout's precondition). pairs[2e], pairs[2e + 1].
__global__ __launch_bounds__(256) void row_runs_kernel(const int32_t* __restrict__ ids, int M,
                                                       int E, int32_t* __restrict__ pairs) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const int id = ids[m];
  if (id < 0 || id >= E) return;
  if (m == 0 || ids[m - 1] != id) pairs[2 * id] = m;
  if (m == M - 1 || ids[m + 1] != id) pairs[2 * id + 1] = m + 1;
}

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  fill_i32_kernel<<<(int)(want < 4096 ? want : 4096), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_align(const int32_t* off, const int32_t* sorted_route, int R, int E, int bs,
                        int32_t* padded_off, int32_t* sorted_ids, int32_t* expert_blk,
                        int32_t* num_post_pad, int32_t* seg_ends, hipStream_t s) {
  const int len = align_len(R, E, bs);
  align_fill_kernel<<<(len + kNT - 1) / kNT, kNT, 0, s>>>(off, sorted_route, E, bs, R, len,
                                                         padded_off, num_post_pad, seg_ends,
                                                         sorted_ids, expert_blk);
  return hipGetLastError();
}

hipError_t launch_align_rows(const void* hidden, int64_t row_bytes, int K, const int32_t* off,
                             const int32_t* sorted_route, int E, int bs, int cap, void* out,
                             int32_t* inverse, int32_t* row_ids, int32_t* seg_ends,
                             hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  constexpr int rows = kNT / 64 * kRowsPerWave;
  align_rows_kernel<<<(cap + rows - 1) / rows, kNT, 0, s>>>(
      (const char*)hidden, row_bytes, K, off, sorted_route, E, bs, cap, (char*)out, inverse,
      row_ids, seg_ends);
  return hipGetLastError();
}

hipError_t launch_masked_rows(const void* hidden, int64_t row_bytes, int K, int R,
                              const int32_t* off, const int32_t* sorted_route, int E,
                              int max_m, void* out, int32_t* counts, int32_t* inverse,
                              hipStream_t s) {
  hipError_t err = fill_i32(inverse, R, -1, s);  // routes without room keep -1
  if (err != hipSuccess) return err;
  masked_rows_kernel<<<dim3(max_m > 0 ? max_m : 1, E), 256, 0, s>>>(
      (const char*)hidden, row_bytes, K, off, sorted_route, max_m, (char*)out, counts, inverse);
  return hipGetLastError();
}

hipError_t launch_row_runs(const int32_t* ids, int M, int E, int32_t* pairs, hipStream_t s) {
  hipError_t err = fill_i32(pairs, 2 * (int64_t)E, 0, s);  // absent experts: empty runs
  if (err != hipSuccess || M <= 0) return err;
  row_runs_kernel<<<(M + 255) / 256, 256, 0, s>>>(ids, M, E, pairs);
  return hipGetLastError();
}

}  // namespace moe
