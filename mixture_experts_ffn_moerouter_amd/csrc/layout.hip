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
// all layouts share its order. The kernels are small integer passes plus row copies (one
// workgroup per destination row, 16-byte vectors), bound by the hidden rows they move.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;  // one thread per expert (E <= 1024)

// padded_off[e] = exclusive prefix of round_up(count[e], bs); padded_off[E] = total;
// optional copies: num_post_pad[0] = total, seg_ends[e] = padded_off[e + 1].
__global__ __launch_bounds__(kScanThreads) void align_scan_kernel(
    const int32_t* __restrict__ off, int E, int bs, int32_t* __restrict__ padded_off,
    int32_t* __restrict__ num_post_pad, int32_t* __restrict__ seg_ends) {
  __shared__ int s_w[kScanThreads / 64];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const int cnt = e < E ? off[e + 1] - off[e] : 0;
  const int v = (cnt + bs - 1) / bs * bs;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    base += w < wave ? s_w[w] : 0;
    total += s_w[w];
  }
  if (e < E) {
    padded_off[e] = base + x - v;
    if (seg_ends) seg_ends[e] = base + x;
  }
  if (e == 0) {
    padded_off[E] = total;
    if (num_post_pad) num_post_pad[0] = total;
  }
}

// Largest e in [0, E) with padded_off[e] <= s (the expert whose padded range holds s when
// s < padded_off[E]; empty experts share their successor's start and lose to it).
__device__ __forceinline__ int owner_of(const int32_t* padded_off, int E, int s) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (padded_off[mid] <= s) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One thread per slot s < len of sorted_token_ids (and the block entry when s % bs == 0).
__global__ __launch_bounds__(256) void align_fill_kernel(
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted_route,
    const int32_t* __restrict__ padded_off, int E, int bs, int numel, int len,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_blk) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= len) return;
  const int used = padded_off[E];
  int val = numel, owner = -1;
  if (s < used) {
    owner = owner_of(padded_off, E, s);
    const int i = s - padded_off[owner];
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

// Contiguous / per-row pre-permute: destination row m < cap holds route sorted_ids[m] when
// m is inside the used length and the slot is not padding. Writes the row, the route's
// inverse index and (per_row) the row's expert id (-1 on padding and unused rows).
__global__ __launch_bounds__(256) void contiguous_rows_kernel(
    const char* __restrict__ hidden, int64_t row_bytes, int K,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ expert_blk,
    const int32_t* __restrict__ padded_off, int E, int bs, int numel, int cap,
    char* __restrict__ out, int32_t* __restrict__ inverse, int32_t* __restrict__ row_ids) {
  const int m = blockIdx.x;
  if (m >= cap) return;
  const int used = padded_off[E];
  const int src = m < used ? sorted_ids[m] : numel;
  const bool live = src < numel;
  if (threadIdx.x == 0) {
    if (live) inverse[src] = m;
    if (row_ids) row_ids[m] = live ? expert_blk[m / bs] : -1;
  }
  if (live) copy_row(hidden + (int64_t)(src / K) * row_bytes, out + (int64_t)m * row_bytes,
                     row_bytes);
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
  align_scan_kernel<<<1, kScanThreads, 0, s>>>(off, E, bs, padded_off, num_post_pad, seg_ends);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int len = align_len(R, E, bs);
  align_fill_kernel<<<(len + 255) / 256, 256, 0, s>>>(off, sorted_route, padded_off, E, bs, R,
                                                      len, sorted_ids, expert_blk);
  return hipGetLastError();
}

hipError_t launch_contiguous_rows(const void* hidden, int64_t row_bytes, int K,
                                  const int32_t* sorted_ids, const int32_t* expert_blk,
                                  const int32_t* padded_off, int E, int bs, int R, int cap,
                                  void* out, int32_t* inverse, int32_t* row_ids,
                                  hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  contiguous_rows_kernel<<<cap, 256, 0, s>>>((const char*)hidden, row_bytes, K, sorted_ids,
                                             expert_blk, padded_off, E, bs, R, cap,
                                             (char*)out, inverse, row_ids);
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
