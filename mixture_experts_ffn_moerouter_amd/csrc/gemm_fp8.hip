// Block-scaled FP8 grouped GEMM over a masked slab, for gfx950.
//
// [TO] TileOPs "MoE Operators", MoEGroupedGemmFP8FwdOp: for each expert g with m_g valid
//      rows (its count clamped to [0, max_m]) out[g, :m_g] = a[g, :m_g] b[g]^T, where a
//      [E, max_m, K] and b [E, N, K] are float8_e4m3fn, a_scale holds one float32 per row
//      and 128 columns of a and b_scale one per 128 x 128 block of b. Each 128-wide K
//      block is contracted from the raw FP8 values, multiplied by its two scales and added
//      to a float32 accumulator; the result is stored in bfloat16. Rows at or past m_g
//      are not written.
//
// Tile: 128 token rows x 128 weight rows (one b_scale block), eight waves (2 x 4) of 64
// token rows x 32 weight rows, one workgroup per CU. A K step is one 128-wide scale block: 128 bytes of every row (the same bytes per
// step as the bf16 kernel's 64-element step), staged through double-buffered LDS (row
// stride 144 bytes: conflict-free 16-byte fragment reads) from registers loaded two steps
// ahead with buffer loads (pieces past the tile or the matrix get an offset past the
// buffer: zeros, no branch). The step's scales travel with it: threads 0..127 load the
// a_scale of the tile's rows and thread 128 the b_scale of its weight block, into the same
// LDS stage. A wave's 64 x 32 is 4 x 2 blocks of 16 x 16; each block
// takes one v_mfma_scale_f32_16x16x128_f8f6f4 per step (neutral e8m0 scales, e4m3 on both
// operands), which contracts the whole 128-wide scale block into a fresh accumulator; that
// is multiplied by a_scale[row] * b_scale and added to the float32 accumulator, the order
// the page gives. A lane holds 32 contiguous bytes of its row (lane quarter q: bytes
// 32q .. 32q+31) for both operands, so products pair the same way on both sides and the
// sum is the plain one.
//
// Tile map: expert g with m_g rows gets ceil(m_g / 128) row tiles of equal height (rounded
// up to 32 rows), built on the device from the counts; logical tiles are ordered expert,
// n-tile, row tile and dealt so that consecutive ones run on one XCD.
#include "moe_internal.h"
#include "tile_map.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int kNT = 512, kWM = 2, kWN = 4, kRB = 2, kCB = 1;
constexpr int kBMX = 32 * kRB * kWM;             // 128 token rows per tile
constexpr int kBNW = 32 * kCB * kWN;             // 128 weight rows per tile
constexpr int kStepBytes = 128;                  // bytes of a row per K step
constexpr int kLDK = kStepBytes + 16;            // LDS row stride (bytes)
constexpr int kCPR = kStepBytes / 16;            // 16-byte pieces per row segment
constexpr int kRSTEP = kNT / kCPR;               // rows covered by one pass of the threads
constexpr int kNLD = kBMX * kCPR / kNT;          // A pieces per thread per step
constexpr int kNLDB = kBNW * kCPR / kNT;         // B pieces per thread per step
constexpr int kScaleOff = (kBMX + kBNW) * kLDK;  // scales after the two tiles in a stage
constexpr int kStageBytes = (kScaleOff + (kBMX + 1) * 4 + 15) / 16 * 16;
constexpr int kMaxE = 1024;
constexpr int kXcd = 8;
constexpr uint32_t kOOB = 0x80000000u;
static_assert(2 * kStageBytes >= 2 * (kMaxE + 1) * (int)sizeof(int), "tile map alias");

__device__ __forceinline__ i32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ i32x8 lds32(const uint8_t* p) {
  const i32x4 lo = *(const i32x4*)p, hi = *(const i32x4*)(p + 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__global__ __launch_bounds__(kNT, 1) void gemm_fp8_masked_kernel(Fp8GemmArgs g) {
  __shared__ int s_tmp[kNT / 64];
  extern __shared__ __align__(16) uint8_t smem[];  // [2][stage], tile map aliased first
  int* s_cnt = (int*)smem;
  int* s_pre = s_cnt + kMaxE + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = g.E, K = g.K, N = g.N, nkb = g.K / 128;
  build_tile_map_masked<kNT>(g.counts, E, g.max_m, kBMX, s_cnt, s_pre, s_tmp);

  const int n_tiles_n = (N + kBNW - 1) / kBNW;
  const int n_valid = s_pre[E] * n_tiles_n;
  const int per = (n_valid + kXcd - 1) / kXcd;
  const int slot = blockIdx.x / kXcd;
  const int L = (blockIdx.x % kXcd) * per + slot;
  if (slot >= per || L >= n_valid) return;  // uniform per workgroup
  const int e = find_expert(s_pre, E, L / n_tiles_n);
  const int t_e = s_pre[e + 1] - s_pre[e];
  const int local = L - s_pre[e] * n_tiles_n;
  const int nt = local / t_e, mt = local % t_e;
  const int cnt = s_cnt[e];
  const int rpt = rows_per_tile(cnt, kBMX);
  const int m0 = mt * rpt, m1 = min(m0 + rpt, cnt);
  const int rows = m1 - m0;
  const int nb = (rows + 31) / 32;
  __syncthreads();  // every thread has read the map; the buffers become stages

  // Buffer resources over expert e's slabs (32-bit offsets within one expert).
  const int64_t M = g.max_m;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a + (int64_t)e * M * K), (short)0, (int)(M * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.b + (int64_t)e * N * K), (short)0, (int)((int64_t)N * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.a_scale + (int64_t)e * M * nkb), (short)0, (int)(M * nkb * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.b_scale + (int64_t)e * (N / 128) * nkb), (short)0, (int)((N / 128) * nkb * 4),
      0x00020000);

  // Thread tid moves 16-byte piece tid % 8 of rows tid / 8 + 64 i of both tiles.
  const int kc = (tid % kCPR) * 16;
  uint32_t aoff[kNLD], boff[kNLDB];
#pragma unroll
  for (int i = 0; i < kNLD; ++i) {
    const int r = tid / kCPR + kRSTEP * i;
    aoff[i] = r < rows ? (uint32_t)(m0 + r) * (uint32_t)K + kc : kOOB;
  }
#pragma unroll
  for (int i = 0; i < kNLDB; ++i) {
    const int wr = nt * kBNW + tid / kCPR + kRSTEP * i;
    boff[i] = wr < N ? (uint32_t)wr * (uint32_t)K + kc : kOOB;
  }
  // the tile's rows of a_scale (threads 0..127) and its b_scale block (thread 128)
  const uint32_t soa = tid < rows ? (uint32_t)(m0 + tid) * nkb * 4u : kOOB;
  const uint32_t sob = tid == kBMX ? (uint32_t)nt * nkb * 4u : kOOB;

  i32x4 xa0[kNLD], xa1[kNLD], xb0[kNLDB], xb1[kNLDB];
  float xs0, xs1;
  auto load = [&](int kb, i32x4* xa, i32x4* xb, float& xs) {
    const bool in = kb < nkb;
    const uint32_t k0 = (uint32_t)kb * kStepBytes;
#pragma unroll
    for (int i = 0; i < kNLD; ++i) xa[i] = ld16(ra, in ? aoff[i] + k0 : kOOB);
#pragma unroll
    for (int i = 0; i < kNLDB; ++i) xb[i] = ld16(rb, in ? boff[i] + k0 : kOOB);
    const float sa = ld4(rsa, in ? soa + 4u * kb : kOOB);
    const float sb = ld4(rsb, in ? sob + 4u * kb : kOOB);
    xs = sa + sb;  // at most one of the two is in range for a thread
  };
  auto store = [&](int buf, const i32x4* xa, const i32x4* xb, float xs) {
    uint8_t* la = smem + buf * kStageBytes;
    uint8_t* lb = la + kBMX * kLDK;
#pragma unroll
    for (int i = 0; i < kNLD; ++i) *(i32x4*)(la + (tid / kCPR + kRSTEP * i) * kLDK + kc) = xa[i];
#pragma unroll
    for (int i = 0; i < kNLDB; ++i) *(i32x4*)(lb + (tid / kCPR + kRSTEP * i) * kLDK + kc) = xb[i];
    if (tid <= kBMX) ((float*)(la + kScaleOff))[tid] = xs;
  };

  // Wave (wm, wn): its 32-row blocks wm and wm + 2 of the tile, as 16-row blocks
  // rowblk(i) = (wm + 2 (i / 2)) 32 + 16 (i % 2), i < 4; weight rows wn*32 + 16 j, j < 2.
  const int wm = wave % kWM, wn = wave / kWM;
  const int lr = lane & 15, lq = (lane >> 4) * 32;  // operand row, byte quarter
  auto rowblk = [&](int i) { return (wm + kWM * (i >> 1)) * 32 + 16 * (i & 1); };
  const int nbw = nb > wm ? (nb - wm + kWM - 1) / kWM : 0;  // live 32-row blocks of this wave

  constexpr int NJ = 2;
  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{};

  auto main_loop = [&](auto nbw_c) {
    constexpr int NI = 2 * decltype(nbw_c)::value;  // live 16-row blocks
    // One K step from LDS buffer buf: the weight fragments, then per row block the four
    // MFMAs into fresh accumulators and their scaled accumulation. mid() (the store of
    // the next step into the other buffer and the loads two steps ahead) follows the
    // first row block.
    auto compute = [&](int buf, auto&& mid) {
      const uint8_t* la = smem + buf * kStageBytes;
      const uint8_t* lb = la + kBMX * kLDK;
      const float* sc = (const float*)(la + kScaleOff);
      i32x8 fb[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[j] = lds32(lb + (wn * 32 + 16 * j + lr) * kLDK + lq);
      const float sbv = sc[kBMX];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rb = rowblk(i);
        const i32x8 fa = lds32(la + (rb + lr) * kLDK + lq);
        f32x4 s4 = *(const f32x4*)(sc + rb + 4 * (lane >> 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) s4[q] *= sbv;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const f32x4 blk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              fa, fb[j], f32x4{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(blk[q], s4[q], acc[i][j][q]);
        }
        if (i == 0) {
          __builtin_amdgcn_sched_barrier(0);
          mid();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    auto none = [] {};
    // Step s uses LDS buffer s % 2 and register set s % 2; after storing step k+1 the
    // loads of step k+3 go into the set just freed, so one step of loads stays in flight
    // across every wait. Steps past the end load nothing (out-of-range offsets).
    load(0, xa0, xb0, xs0);
    load(1, xa1, xb1, xs1);
    store(0, xa0, xb0, xs0);
    load(2, xa0, xb0, xs0);
    __syncthreads();
    int k = 0;
    for (; k + 1 < nkb; k += 2) {
      compute(0, [&] {
        store(1, xa1, xb1, xs1);
        load(k + 3, xa1, xb1, xs1);
      });
      __syncthreads();
      compute(1, [&] {
        store(0, xa0, xb0, xs0);
        load(k + 4, xa0, xb0, xs0);
      });
      __syncthreads();
    }
    if (k < nkb) compute(0, none);  // odd number of steps: the last one is in buffer 0
  };
  if (nbw >= 2) main_loop(std::integral_constant<int, 2>{});
  else main_loop(std::integral_constant<int, 1>{});

  // Epilogue: register q of lane l holds row 4*(l/16) + q and column l%16 of its 16 x 16
  // block.
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int n = nt * kBNW + wn * 32 + 16 * j + lr;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < 2 * nbw) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = m0 + rowblk(i) + 4 * (lane >> 4) + q;
            if (m < m1) g.out[((int64_t)e * M + m) * N + n] = f32_to_bf16(acc[i][j][q]);
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_masked(const Fp8GemmArgs& g, hipStream_t s) {
  if (g.E <= 0 || g.max_m <= 0) return hipSuccess;
  const int n_tiles_n = (g.N + kBNW - 1) / kBNW;
  const int64_t max_tiles = (int64_t)g.E * ((g.max_m + kBMX - 1) / kBMX);
  int64_t grid = max_tiles * n_tiles_n;
  grid = (grid + kXcd - 1) / kXcd * kXcd;
  const size_t lds = 2 * (size_t)kStageBytes;
  hipError_t err = hipFuncSetAttribute((const void*)gemm_fp8_masked_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  gemm_fp8_masked_kernel<<<dim3((unsigned)grid), dim3(kNT), lds, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
