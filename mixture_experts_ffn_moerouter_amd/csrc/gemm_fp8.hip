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
// Tile: 160 token rows x 256 weight rows (two b_scale blocks), eight waves (2 x 4): the two
// row waves take alternate 16-row blocks (80 rows each), the four column waves 64 weight
// rows each; one workgroup per CU. A K step is one 128-wide scale block: 128 bytes of every
// row. An expert of up to 160 rows is one row tile, so its weight lines are read once.
//
// Staging. Three LDS stages form a ring filled by direct-to-LDS buffer loads (no register
// staging, no LDS write instructions): step k + 2 is requested while step k is multiplied,
// so each transfer has two steps to land. One load instruction moves 1 KB, eight rows x
// 128 bytes (whole cache lines); lane l lands in row l / 8, 16-byte slot l % 8, and fetches
// the row's byte piece (l % 8) ^ (row % 8), so slots are XOR-swizzled by row. The 20
// token-row transfers of a step are dealt three to a wave (a wave past the 20th repeats
// it, so every wave issues the same count). The scales of the step travel the same way
// (4-byte transfers: a_scale of the tile's rows, the two b_scale blocks). A wave's eight
// transfers of the next step are spread through its MFMA stream rather than issued at
// once. The compiler's workgroup barrier would wait for every
// transfer in flight, so the step boundary is an explicit "own transfers of this step
// landed (vmcnt), own LDS reads done, barrier" sequence.
//
// Multiply. Fragments are read with lane (r, q) of a 16-row block taking pieces q and q + 4
// of row r (both operands alike, so products pair as in the plain sum); with the XOR slots
// this read pattern is free of LDS bank conflicts. Each 16 x 16 block takes one
// v_mfma_scale_f32_16x16x128_f8f6f4 per step (neutral e8m0 scales, e4m3 on both
// operands) into a fresh accumulator, weights as the first operand, so a lane's four
// results share one token row and one combined scale a_scale[row] * b_scale; that
// product is folded into the float32 accumulator two MFMAs later, keeping the matrix
// core fed while the vector unit applies the scales. This is the order the page gives:
// per-block partial sums from the FP8 values, scaled, then accumulated in float32.
//
// Tile map: expert g with m_g rows gets ceil(m_g / 160) row tiles of equal height (rounded
// up to 32 rows), built on the device from the counts; logical tiles are ordered expert,
// n-tile, row tile and dealt so that consecutive ones run on one XCD (the row tiles of an
// expert share its weight lines in that XCD's L2).
#include <type_traits>

#include "moe_internal.h"
#include "tile_map.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kNT = 512;                 // 8 waves: 2 (token rows) x 4 (weight rows)
constexpr int kBMX = 160;                // token rows per tile
constexpr int kBNW = 256;                // weight rows per tile
constexpr int kNS = 3;                   // LDS stages
constexpr int kA = 0;                    // stage layout (bytes): token rows
constexpr int kB = kA + kBMX * 128;      // weight rows
constexpr int kSA = kB + kBNW * 128;     // a_scale of the tile's rows
constexpr int kSB = kSA + 3 * 256;       // the two b_scale blocks (one 256-byte transfer)
constexpr int kSink = kSB + 256;         // landing area of the idle waves' scale transfer
constexpr int kStage = kSink + 256;
constexpr int kPA = 3;                   // token-row transfers per wave and step
constexpr int kNPA = kBMX / 8;           // distinct ones (a wave past them repeats the last)
constexpr int kPieces = kPA + 5;         // transfers per wave and step: 3 A, 4 B, 1 scale
constexpr int kNI = kBMX / 32;           // 16-row blocks per wave
constexpr int kDepth = 2;                // MFMAs between a block's MFMA and its scaling
constexpr int kMaxE = 1024;
constexpr int kXcd = 8;
constexpr uint32_t kOOB = 0x80000000u;   // byte offset past every buffer range used here
static_assert(kNS * kStage >= 2 * (kMaxE + 1) * (int)sizeof(int), "tile map alias");
static_assert(kNS * kStage + 64 <= 160 * 1024, "LDS");

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, off, 0, 0, 0);
}

__global__ __launch_bounds__(kNT, 1) void gemm_fp8_masked_kernel(Fp8GemmArgs g) {
  __shared__ int s_tmp[kNT / 64];
  extern __shared__ __align__(16) uint8_t smem[];  // [kNS][kStage], tile map aliased first
  int* s_cnt = (int*)smem;
  int* s_pre = s_cnt + kMaxE + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int nb = (rows + 15) / 16;
  __syncthreads();  // every thread has read the map; the buffer becomes the stages

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

  // Wave w moves 1 KB pieces apiece(u) = min(3 w + u, 19) of the token tile (piece q holds
  // rows 8 q .. 8 q + 7) and 4w .. 4w + 3 of the weight tile (rows 32w .. 32w + 31). Rows
  // past the tile or the matrix get an offset past the buffer; what lands for them is
  // never stored.
  auto apiece = [&](int u) { return min(kPA * wave + u, kNPA - 1); };
  const int prow = lane >> 3;
  const uint32_t pbyte = 16u * (uint32_t)((lane & 7) ^ prow);
  uint32_t aoff[kPA], boff[4];
#pragma unroll
  for (int u = 0; u < kPA; ++u) {
    const int r = 8 * apiece(u) + prow;
    aoff[u] = r < rows ? (uint32_t)(m0 + r) * (uint32_t)K + pbyte : kOOB;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int wr = nt * kBNW + 8 * (4 * wave + u) + prow;
    boff[u] = wr < N ? (uint32_t)wr * (uint32_t)K + pbyte : kOOB;
  }
  // Scales: waves 0, 1 and 3 move the a_scale of rows 64 s + lane (s = 0, 1, 2; the third
  // covers rows 128 .. 159, its other lanes land zeros in the region's unused tail), wave
  // 2 the two b_scale blocks of the tile; the other waves' transfer is empty (keeps the
  // count uniform).
  uint32_t soff = kOOB;
  __amdgpu_buffer_rsrc_t rs = rsb;
  int sdst = kSink;
  if (wave < 2 || wave == 3) {
    const int sl = wave == 3 ? 2 : wave;
    const int r = 64 * sl + lane;
    soff = r < rows ? (uint32_t)(m0 + r) * nkb * 4u : kOOB;
    rs = rsa;
    sdst = kSA + 256 * sl;
  } else if (wave == 2) {
    const int blk = nt * 2 + lane;
    soff = (lane < 2 && blk < N / 128) ? (uint32_t)blk * nkb * 4u : kOOB;
    sdst = kSB;
  }
  // transfer p of this wave's share of step kb (steps past the end move nothing)
  auto piece = [&](int kb, int p) {
    uint8_t* st = smem + (kb % kNS) * kStage;
    const bool in = kb < nkb;
    const uint32_t k0 = (uint32_t)kb * 128u;
    if (p < kPA) dma16(ra, st + kA + apiece(p) * 1024, in ? aoff[p] + k0 : kOOB);
    else if (p < kPA + 4)
      dma16(rb, st + kB + (4 * wave + p - kPA) * 1024, in ? boff[p - kPA] + k0 : kOOB);
    else dma4(rs, st + sdst, in ? soff + 4u * (uint32_t)kb : kOOB);
  };

  // Wave (wm, wn): token 16-row blocks rowblk(i) = (2 i + wm) 16 (the two row waves take
  // alternate blocks, so a partly filled tile stays balanced), weight rows wn 64 + 16 j.
  // Fragment of row r: lane (r % 16, q) takes pieces q and q + 4.
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, lq = lane >> 4;
  const uint32_t fo0 = 16u * (uint32_t)(lq ^ (lr & 7));
  const uint32_t fo1 = 16u * (uint32_t)((lq ^ 4) ^ (lr & 7));
  auto rowblk = [&](int i) { return (2 * i + wm) * 16; };
  const int nbw = nb > wm ? (nb - wm + 1) / 2 : 0;  // live 16-row blocks of this wave
  auto frag = [&](const uint8_t* rowp) {
    const i32x4 lo = *(const i32x4*)(rowp + fo0), hi = *(const i32x4*)(rowp + fo1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  f32x4 acc[kNI][4];
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  auto main_loop = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;  // live 16-row blocks
    constexpr int NB = NI * 4;                 // MFMAs per step
    constexpr int EVERY = NB >= 2 * kPieces ? 2 : 1;
    static_assert(EVERY * (kPieces - 1) < NB + kDepth, "every transfer is issued");
#pragma unroll
    for (int p = 0; p < kPieces; ++p) piece(0, p);
#pragma unroll
    for (int p = 0; p < kPieces; ++p) piece(1, p);
    for (int kb = 0; kb < nkb; ++kb) {
      // This wave's transfers of step kb have landed (those of kb + 1 may not have) and
      // its reads of step kb - 1 are done; after the barrier every wave's are, so stage
      // kb % 3 is complete and stage (kb + 2) % 3 is free.
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPieces) : "memory");
      const uint8_t* st = smem + (kb % kNS) * kStage;
      // every operand of the step, in the order the MFMAs consume them
      i32x8 fa[NI], fb[4];
      float sa[NI], s1[NI];
      const float sbv = *(const float*)(st + kSB + 4 * (wn >> 1));
#pragma unroll
      for (int i = 0; i < NI; ++i) sa[i] = *(const float*)(st + kSA + 4 * (rowblk(i) + lr));
      __builtin_amdgcn_sched_barrier(0);
      fa[0] = frag(st + kA + (rowblk(0) + lr) * 128);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        fb[j] = frag(st + kB + (wn * 64 + 16 * j + lr) * 128);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 1; i < NI; ++i) {
        fa[i] = frag(st + kA + (rowblk(i) + lr) * 128);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) s1[i] = sa[i] * sbv;
      // MFMA t, the scaling of block t - kDepth, and every EVERY-th slot one transfer of
      // step kb + 2, in this order (pinned against the scheduler)
      f32x4 blk[NB];
#pragma unroll
      for (int t = 0; t < NB + kDepth; ++t) {
        if (t < NB)
          blk[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              fb[t % 4], fa[t / 4], f32x4{}, 0, 0, 0, 127, 0, 127);
        if (t >= kDepth) {
          const int u = t - kDepth;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[u / 4][u % 4][q] = fmaf(blk[u][q], s1[u / 4], acc[u / 4][u % 4][q]);
        }
        if (t % EVERY == EVERY - 1 && t / EVERY < kPieces) piece(kb + 2, t / EVERY);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // no transfer into LDS may outlive the workgroup
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // the K loop for the wave's count of live 16-row blocks (a wave without live rows runs
  // the smallest instance: its transfers and barriers are the other waves' too)
  static_assert(kNI == 5, "instances below");
  if (nbw >= 5) main_loop(std::integral_constant<int, 5>{});
  else if (nbw == 4) main_loop(std::integral_constant<int, 4>{});
  else if (nbw == 3) main_loop(std::integral_constant<int, 3>{});
  else main_loop(std::integral_constant<int, 2>{});

  // Epilogue: lane (r, q) of block (i, j) holds token row rowblk(i) + r and weight rows
  // wn 64 + 16 j + 4 q .. + 3: one 8-byte store each.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = nt * kBNW + wn * 64 + 16 * j + 4 * lq;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        const int m = m0 + rowblk(i) + lr;
        if (i < nbw && m < m1) {
          const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][j][0]) |
                              ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][j][2]) |
                              ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
          *(uint2*)(g.out + ((int64_t)e * M + m) * N + n) = make_uint2(lo, hi);
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
  const size_t lds = (size_t)kNS * kStage;
  hipError_t err = hipFuncSetAttribute((const void*)gemm_fp8_masked_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  gemm_fp8_masked_kernel<<<dim3((unsigned)grid), dim3(kNT), lds, s>>>(g);
  return hipGetLastError();
}

}  // namespace moe
