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
//      limit <= 0 disables both clamps. [TO] gelu_and_mul: gelu(gate) * up over stacked
//      rows, read as the exact GELU x * Phi(x).
//
// 16-bit kernel (bfloat16 or float16 operands; only the MFMA and the conversions differ).
//
// Tile: BM token rows (160, or 128 where the LDS cannot hold three 160-row stages beside
// the tile map) x 256 weight rows, eight waves (2 x 4): the two row waves take alternate
// 16-row blocks (BM / 2 rows each), the four column waves 64 weight rows each; a K step is
// 64 elements, 128 bytes of every row. For the gated activation the tile's 256 weight rows
// are the gate and up rows of 128 outputs, placed so that a wave's blocks j and j + 2
// hold the gate and the up row of the same outputs; the epilogue pairs them directly.
//
// Staging. LDS holds a ring of NS stages (three; two when the contraction is a single
// step) filled by direct-to-LDS buffer loads: no register staging and no LDS write
// instructions. Step k + NS - 1 is requested while step k is multiplied. One load
// instruction moves 1 KB, eight rows x 128 bytes (whole cache lines): lane l lands in row
// l / 8, 16-byte slot l % 8, and fetches the row's piece (l % 8) ^ (row % 8), so slots
// are XOR-swizzled by row. A wave's transfers of a step (BM / 64 rounded up of token rows,
// four of weight rows) are spread through its MFMA stream. Rows of A may be gathered (a_rows),
// so the permuted activation copy is never materialised. Out-of-range pieces (rows past
// the tile, weight rows past N, the K tail, steps past the end) get an offset past the
// buffer's range, so the hardware writes zeros without a branch. The compiler's
// workgroup barrier would wait for every transfer in flight, so each step starts with an
// explicit "own transfers of this step landed (vmcnt), own LDS reads done, barrier".
//
// Multiply. Fragments are read with lane (r, q) of a 16-row block taking pieces q and
// q + 4 of row r (both operands alike, so products pair as in the plain sum); with the
// XOR slots these reads are free of bank conflicts. Each 16 x 16 block takes two
// v_mfma_f32_16x16x32 per step, weights as the first operand, so a lane's four results
// are four consecutive outputs of one token row. The K loop is compiled once per count of
// a wave's live 16-row blocks, so a partly filled tile issues no MFMA for blocks that
// hold only padding.
//
// Epilogue. 16-bit outputs whose rows are whole 16-byte pieces are gathered through the
// stage the last step read (its refill is sent only after the next tile's first barrier):
// each wave writes its results there, and after a barrier the workgroup stores whole
// tile rows (256 or 512 bytes) as non-temporal 16-byte pieces. A gated tile always fits
// the stage; a non-gated tile's rows are twice as wide, so it is gathered when its live
// rows are at most half the tile height. Other tiles store each lane's four results as
// one 8-byte store (16 in float32).
//
// Cache policy. A tile of an expert that has one row tile reads each of its weight lines
// once, so that tile's weight transfers are non-temporal; an expert with more row tiles
// keeps its weight lines in the L2 for the later ones. Token rows (read by every n-tile)
// keep the default policy.
//
// Work. The grid is one workgroup per CU, each walking a list of tiles: the stage ring
// runs across tile boundaries, so the next tile's first steps load during the current
// tile's last steps and its epilogue. An expert with M_e rows gets ceil(M_e / BM) row
// tiles of equal height (rounded up to 32 rows); the map is built on the device from the
// layout metadata (no host synchronisation) and kept in LDS. Logical tiles are ordered
// expert, n-tile, row tile and each XCD takes a contiguous range, its workgroups
// striding through it together: the row tiles that share a weight slice run side by side
// on one L2, and so do the n-tiles sharing the expert's token rows.
#include <atomic>
#include <type_traits>

#include "moe_internal.h"
#include "tile_map.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

constexpr int kNT = 512;                // 8 waves: 2 (token rows) x 4 (weight rows)
constexpr int kBNW = 256;               // weight rows per tile
// K elements per step: 128 bytes of a row (dtype 0 float32, else 16-bit)
constexpr int step_elems(int dt) { return dt == 0 ? 32 : 64; }
constexpr int kPB = kBNW / 64;          // 1 KB transfers of weight rows per wave and step
constexpr int kXcd = 8;
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past every buffer range used here
constexpr int kLds = 160 * 1024;        // LDS per workgroup
// Token rows per tile: BM = 160 (one tile holds an expert of up to 160 rows) when the
// stages and the tile map fit in LDS, else 128.
constexpr int stage_bytes(int bm) { return (bm + kBNW) * 128; }
constexpr int map_bytes(int E) { return 3 * (E + 1) * (int)sizeof(int); }
constexpr int kStaticLds = 64;          // s_tmp and alignment

template <int AUX = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, AUX);
}

// 16 x 16 x 32 MFMA on eight 16-bit elements per lane: DT 1 bfloat16, 2 float16.
template <int DT>
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The gated activation of the epilogue: kind 1 gelu_and_mul, else the swiglu family.
__device__ __forceinline__ float gated_f(int kind, float g, float l, float alpha, float beta,
                                         float limit) {
  return kind == 1 ? gelu_f(g) * l : swiglu_f(g, l, alpha, beta, limit);
}

// TAG only names the instance (1: the shared expert's launches), so a profile lists the
// shared expert's GEMMs apart from the routed ones; the code is the same.
template <int NS, int BM, bool ACT, int LAYOUT, bool OUT_F32, int DT, int TAG>
__global__ __launch_bounds__(kNT, 1) void gemm_h16_kernel(GemmArgs g) {
  constexpr int LA = NS - 1;          // steps in flight ahead of the one multiplied
  constexpr int kPA = (BM + 63) / 64;  // 1 KB transfers of token rows per wave and step
  constexpr int kNPA = BM / 8;         // distinct ones (a wave past them repeats the last)
  constexpr int kPieces = kPA + kPB;
  constexpr int kStage = stage_bytes(BM);
  constexpr int kNI = BM / 32;         // 16-row blocks per wave
  static_assert(BM % 32 == 0 && kNPA <= 8 * kPA, "tile rows");
  // Element size: 2 bytes (bfloat16, float16) or 4 (float32, DT 0). A step is always 128
  // bytes of a row, so the transfers and fragment reads are the same for every dtype.
  constexpr int ES = DT == 0 ? 4 : 2;
  constexpr int KBK = 128 / ES;        // K elements per step
  constexpr int EPP = 16 / ES;         // K elements per 16-byte piece
  constexpr int KS = DT == 0 ? 8 : 2;  // MFMAs per 16 x 16 block and step
  static_assert(DT != 0 || OUT_F32, "float32 operands give float32 outputs");
  __shared__ int s_tmp[kNT / 64];
  extern __shared__ __align__(16) uint8_t smem[];  // [NS][kStage], then the tile map
  const int E = g.E;
  int* s_start = (int*)(smem + NS * kStage);
  int* s_len = s_start + E + 1;
  int* s_pre = s_len + E + 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  build_tile_map_segments<kNT>(g.seg_mode, g.offsets, E, g.M, g.max_m, BM, s_start, s_len,
                               s_pre, s_tmp);
  const int n_tiles_n = ACT ? (g.Nout + kBNW / 2 - 1) / (kBNW / 2) : (g.Nw + kBNW - 1) / kBNW;
  const int n_valid = s_pre[E] * n_tiles_n;
  // XCD x (workgroups b with b % 8 == x) owns logical tiles [x per, (x + 1) per); its
  // workgroups take them in turn, so at any time they hold a contiguous run.
  const int per = (n_valid + kXcd - 1) / kXcd;
  const int xcd = blockIdx.x % kXcd, nslot = gridDim.x / kXcd;
  const int L0 = xcd * per + blockIdx.x / kXcd;
  const int Lend = min((xcd + 1) * per, n_valid);
  if (L0 >= Lend) return;  // uniform per workgroup
  const int ntile = (Lend - L0 + nslot - 1) / nslot;
  const int Kd = g.Kd, nk = (Kd + KBK - 1) / KBK;

  // i-th tile of this workgroup: expert, n-tile, rows [m0, m1)
  auto tile = [&](int i, int& e, int& nt, int& m0, int& m1) {
    const int L = L0 + i * nslot;
    e = __builtin_amdgcn_readfirstlane(find_expert(s_pre, E, L / n_tiles_n));
    const int t_e = s_pre[e + 1] - s_pre[e];
    const int local = L - s_pre[e] * n_tiles_n;
    nt = __builtin_amdgcn_readfirstlane(local / t_e);
    const int rpt = rows_per_tile(s_len[e], BM);
    m0 = __builtin_amdgcn_readfirstlane(s_start[e] + (local % t_e) * rpt);
    m1 = __builtin_amdgcn_readfirstlane(min(m0 + rpt, s_start[e] + s_len[e]));
  };

  // Transfers: wave w moves 1 KB pieces kPA w + u of the token rows (piece q holds rows
  // 8 q .. 8 q + 7; a wave whose pieces run past the tile's kNPA repeats the last one, so
  // every wave issues the same count) and kPB w + u of the weight rows (rows 32 w ..
  // 32 w + 31); lane l takes row l / 8 of the piece and its 16-byte part (l % 8) ^ (row % 8).
  auto apiece = [&](int u) { return min(kPA * wave + u, kNPA - 1); };
  const int prow = lane >> 3;
  const int kel = EPP * ((lane & 7) ^ prow);  // first K element of the lane's part
  const uint32_t pbyte = (uint32_t)ES * (uint32_t)kel;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, 0x7fffffff, 0x00020000);
  // per-lane byte offsets (and the expert's weight buffer) of one tile
  auto offsets = [&](int e, int nt, int m0, int m1, uint32_t* ao, uint32_t* bo,
                     __amdgpu_buffer_rsrc_t& rb) {
    const int rows = m1 - m0;
#pragma unroll
    for (int u = 0; u < kPA; ++u) {
      const int r = 8 * apiece(u) + prow;
      const bool on = r < rows;
      const int m = m0 + (on ? r : 0);
      const int src = g.a_rows ? g.a_rows[m] / g.a_rows_div : m;
      ao[u] = on ? (uint32_t)src * (uint32_t)Kd * (uint32_t)ES + pbyte : kOOB;
    }
    rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)g.b + (int64_t)e * g.Nw * Kd * ES), (short)0,
        (int)((int64_t)g.Nw * Kd * ES), 0x00020000);
#pragma unroll
    for (int u = 0; u < kPB; ++u) {
      const int b = 8 * (kPB * wave + u) + prow;  // weight row of the tile
      int wr;
      bool on;
      if (ACT) {  // wave b / 64, block (b / 16) % 4: gate rows (blocks 0, 1), up rows (2, 3)
        const int j = (b >> 4) & 3;
        const int o = nt * (kBNW / 2) + (b >> 6) * 32 + 16 * (j & 1) + (b & 15);
        const bool up = j >= 2;
        on = o < g.Nout;
        wr = LAYOUT == 0 ? (up ? g.Nout + o : o) : (2 * o + (up ? 1 : 0));
      } else {
        wr = nt * kBNW + b;
        on = wr < g.Nw;
      }
      bo[u] = on ? (uint32_t)wr * (uint32_t)Kd * (uint32_t)ES + pbyte : kOOB;
    }
  };
  int te, tnt, tm0, tm1;              // the tile being multiplied
  uint32_t aC[kPA], bC[kPB], aN[kPA], bN[kPB];  // offsets of this tile and the next
  __amdgpu_buffer_rsrc_t rbC, rbN;
  tile(0, te, tnt, tm0, tm1);
  offsets(te, tnt, tm0, tm1, aC, bC, rbC);
  // transfer p of step kk of this tile (nxt false) or the next into stage st
  auto piece = [&](int stage, int kk, bool nxt, int p, auto aux_c) {
    uint8_t* st = smem + stage * kStage;
    const int k0 = kk * KBK;
    const bool in = k0 + kel < Kd;
    const uint32_t kbyte = (uint32_t)k0 * (uint32_t)ES;
    if (p < kPA) {
      const uint32_t o = nxt ? aN[p] : aC[p];
      dma16(ra, st + apiece(p) * 1024, in ? o + kbyte : kOOB);
    } else {
      const uint32_t o = nxt ? bN[p - kPA] : bC[p - kPA];
      dma16<decltype(aux_c)::value>(nxt ? rbN : rbC,
                                    st + BM * 128 + (kPB * wave + p - kPA) * 1024,
                                    in ? o + kbyte : kOOB);
    }
  };

  // Wave (wm, wn): token 16-row blocks rowblk(i) = (2 i + wm) 16 (the two row waves take
  // alternate blocks, so a partly filled tile stays balanced), weight rows wn 64 + 16 j.
  // Fragment of row r: lane (r % 16, q) takes pieces q and q + 4.
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, lq = lane >> 4;
  const uint32_t fo0 = 16u * (uint32_t)(lq ^ (lr & 7));
  const uint32_t fo1 = 16u * (uint32_t)((lq ^ 4) ^ (lr & 7));
  auto rowblk = [&](int i) { return (2 * i + wm) * 16; };

#pragma unroll
  for (int q = 0; q < LA; ++q)
#pragma unroll
    for (int p = 0; p < kPieces; ++p) piece(q, q, false, p, std::integral_constant<int, 0>{});

  const void* bias = g.bias;
  auto bias_at = [&](int64_t idx) {
    if constexpr (DT == 0) return ((const float*)bias)[idx];
    else return h16_to_f32<DT>(((const uint16_t*)bias)[idx]);
  };
  const bool aligned = ((uintptr_t)g.out & 15) == 0;
  int gs = 0;  // steps of the earlier tiles (ring position)
  for (int ti = 0; ti < ntile; ++ti) {
    if (ti + 1 < ntile) {
      int e2, nt2, m02, m12;
      tile(ti + 1, e2, nt2, m02, m12);
      offsets(e2, nt2, m02, m12, aN, bN, rbN);
    } else {  // the ring's last transfers move nothing
#pragma unroll
      for (int u = 0; u < kPA; ++u) aN[u] = kOOB;
#pragma unroll
      for (int u = 0; u < kPB; ++u) bN[u] = kOOB;
      rbN = rbC;
    }
    const int e = te, nt = tnt, m0 = tm0, m1 = tm1;
    const int nb = (m1 - m0 + 15) / 16;               // live 16-row blocks of the tile
    const int nbw = nb > wm ? (nb - wm + 1) / 2 : 0;  // ... and of this wave
    f32x4 acc[kNI][4];
#pragma unroll
    for (int i = 0; i < kNI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

    // The K loop, compiled for each count of live 16-row blocks of the wave (1 .. kNI).
    auto main_loop = [&](auto ni_c, auto aux_c) {
      constexpr int NI = decltype(ni_c)::value;
      constexpr int NB = NI * 4 * KS;  // MFMAs per step
      constexpr int EVERY = NB / kPieces;
      static_assert(EVERY >= 1 && EVERY * kPieces <= NB, "every transfer is issued");
      for (int k = 0; k < nk; ++k) {
        // This wave's transfers of step k have landed (the newer LA - 1 steps' may not
        // have) and its reads of step k - 1 are done; after the barrier every wave's are,
        // so stage s % NS is complete and stage (s + LA) % NS is free.
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((LA - 1) * kPieces)
                     : "memory");
        const int s = gs + k;
        const uint8_t* st = smem + (s % NS) * kStage;
        const uint8_t* sb = st + BM * 128;
        const int s2 = (s + LA) % NS;
        const bool nxt = k + LA >= nk;
        const int kk = nxt ? k + LA - nk : k + LA;
        bf16x8 fa[NI][2], fb[4][2];
        auto rd = [&](bf16x8* f, const uint8_t* rowp) {
          f[0] = *(const bf16x8*)(rowp + fo0);
          f[1] = *(const bf16x8*)(rowp + fo1);
        };
        // every operand of the step, in the order the MFMAs consume them
        rd(fa[0], st + (rowblk(0) + lr) * 128);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rd(fb[j], sb + (wn * 64 + 16 * j + lr) * 128);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 1; i < NI; ++i) {
          rd(fa[i], st + (rowblk(i) + lr) * 128);
          __builtin_amdgcn_sched_barrier(0);
        }
        // MFMA t and, every EVERY-th slot, one transfer of step s + LA (pinned in order)
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const int ks = t / (NI * 4), u = t % (NI * 4), i = u / 4, j = u % 4;
          if constexpr (DT == 0) {  // piece c's four floats, one per 16x16x4 MFMA
            const int c = ks >> 2, x = ks & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                __builtin_bit_cast(f32x4, fb[j][c])[x], __builtin_bit_cast(f32x4, fa[i][c])[x],
                acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = mfma16<DT>(fb[j][ks], fa[i][ks], acc[i][j]);
          }
          if (t % EVERY == EVERY - 1 && t / EVERY < kPieces) piece(s2, kk, nxt, t / EVERY, aux_c);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // One instance per count of live blocks (dead blocks would only multiply zeros). Every
    // wave runs exactly one of them, a wave without live rows the one-block instance: its
    // transfers and barriers are the other waves' too.
    const int ni = nbw < 1 ? 1 : (nbw > kNI ? kNI : nbw);
    // an expert with one row tile reads each weight line once: non-temporal weight loads
    const bool once = __builtin_amdgcn_readfirstlane(s_pre[e + 1] - s_pre[e]) == 1;
    auto run = [&](auto aux_c) {
      static_assert(kNI == 4 || kNI == 5, "instances below");
      if (ni == kNI) main_loop(std::integral_constant<int, kNI>{}, aux_c);
      else if (ni == kNI - 1) main_loop(std::integral_constant<int, kNI - 1>{}, aux_c);
      else if (ni == kNI - 2) main_loop(std::integral_constant<int, kNI - 2>{}, aux_c);
      else if (kNI == 5 && ni == 2) main_loop(std::integral_constant<int, 2>{}, aux_c);
      else main_loop(std::integral_constant<int, 1>{}, aux_c);
    };
    if (once) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 0>{});
    gs += nk;

    // Epilogue: lane (r, q) of block (i, j) holds token row rowblk(i) + r and weight rows
    // wn 64 + 16 j + 4 q .. + 3.
    auto store4 = [&](int64_t idx, const float* v, bool vec, int n, int nmax) {
      if (vec) {
        if constexpr (OUT_F32) {
          *(f32x4*)((float*)g.out + idx) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          const uint32_t lo =
              (uint32_t)f32_to_h16<DT>(v[0]) | ((uint32_t)f32_to_h16<DT>(v[1]) << 16);
          const uint32_t hi =
              (uint32_t)f32_to_h16<DT>(v[2]) | ((uint32_t)f32_to_h16<DT>(v[3]) << 16);
          *(uint2*)((uint16_t*)g.out + idx) = make_uint2(lo, hi);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (n + c < nmax) {
            if constexpr (OUT_F32) ((float*)g.out)[idx + c] = v[c];
            else ((uint16_t*)g.out)[idx + c] = f32_to_h16<DT>(v[c]);
          }
        }
      }
    };
    // Gathered epilogue (16-bit outputs whose rows are whole 16-byte pieces): the tile's
    // outputs go through the stage the last step read, whose refill is sent only after the
    // next tile's first barrier, and leave as non-temporal runs of a whole tile row
    // (writes inside the weight stream cost up to half as much that way as the waves' own
    // 32-byte pieces). A non-gated tile's rows are twice as wide, so only the
    // first half of its rows fits the stage: such tiles of more rows store as before.
    bool gathered = false;
    if constexpr (!OUT_F32 && DT != 0)
      gathered = ((ACT ? g.Nout : g.Nw) & 7) == 0 && aligned &&
                 (ACT || m1 - m0 <= BM / 2);
    if constexpr (!OUT_F32 && DT != 0) {
      if (gathered) {
        constexpr int W = ACT ? kBNW / 2 : kBNW;  // outputs per tile row
        constexpr int PITCH = 2 * W + 16;         // LDS bytes per tile row
        constexpr int RR = ACT ? BM : BM / 2;     // tile rows that can be live
        constexpr int LPR = 2 * W / 16;           // lanes per row, 16 bytes each
        constexpr int RPI = 64 / LPR;             // rows per store instruction
        constexpr int NU = RR / (8 * RPI);        // store instructions per wave and round
        static_assert(RR % (8 * RPI) == 0 && RR % 16 == 0, "gathered rows");
        static_assert(RR * PITCH <= kStage, "a round fits the stage");
        const int NO = ACT ? g.Nout : g.Nw;
        uint8_t* lo = smem + ((gs - 1) % NS) * kStage;
        // every wave's fragment reads of that stage are done
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        {
#pragma unroll
          for (int jj = 0; jj < (ACT ? 2 : 4); ++jj) {
            const int cl = ACT ? wn * 32 + 16 * jj + 4 * lq : wn * 64 + 16 * jj + 4 * lq;
            const int c0 = nt * W + cl;  // output column
            float b0[4] = {0.f, 0.f, 0.f, 0.f}, b1[4] = {0.f, 0.f, 0.f, 0.f};
            if (bias && c0 < NO) {
              const int64_t be = (int64_t)e * g.Nw;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const int o = min(c0 + c, NO - 1);
                if (ACT) {
                  b0[c] = bias_at(be + (LAYOUT == 0 ? o : 2 * o));
                  b1[c] = bias_at(be + (LAYOUT == 0 ? g.Nout + o : 2 * o + 1));
                } else {
                  b0[c] = bias_at(be + o);
                }
              }
            }
#pragma unroll
            for (int i = 0; i < kNI; ++i) {
              const int r0 = rowblk(i);
              if (i < nbw && r0 < RR) {
                float v[4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  v[c] = ACT ? gated_f(g.act_kind, acc[i][jj][c] + b0[c],
                                       acc[i][jj + 2][c] + b1[c], g.alpha, g.beta, g.limit)
                             : acc[i][jj][c] + b0[c];
                const uint32_t w0 =
                    (uint32_t)f32_to_h16<DT>(v[0]) | ((uint32_t)f32_to_h16<DT>(v[1]) << 16);
                const uint32_t w1 =
                    (uint32_t)f32_to_h16<DT>(v[2]) | ((uint32_t)f32_to_h16<DT>(v[3]) << 16);
                *(uint2*)(lo + (r0 + lr) * PITCH + 2 * cl) = make_uint2(w0, w1);
              }
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int lrow = (wave * NU + u) * RPI + lane / LPR, chunk = lane % LPR;
            const int m = m0 + lrow, col = nt * W + 8 * chunk;
            if (m < m1 && col < NO) {
              const i32x4 v = *(const i32x4*)(lo + lrow * PITCH + 16 * chunk);
              __builtin_nontemporal_store(v, (i32x4*)((uint16_t*)g.out + (int64_t)m * NO + col));
            }
          }
        }
      }
    }
    if (gathered) {
    } else if (ACT) {
      const bool vrow = (g.Nout & 3) == 0 && aligned;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int o0 = nt * (kBNW / 2) + wn * 32 + 16 * j + 4 * lq;
        if (o0 < g.Nout) {
          float bg[4] = {0.f, 0.f, 0.f, 0.f}, bu[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const int64_t be = (int64_t)e * g.Nw;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int o = min(o0 + c, g.Nout - 1);
              bg[c] = bias_at(be + (LAYOUT == 0 ? o : 2 * o));
              bu[c] = bias_at(be + (LAYOUT == 0 ? g.Nout + o : 2 * o + 1));
            }
          }
#pragma unroll
          for (int i = 0; i < kNI; ++i) {
            const int m = m0 + rowblk(i) + lr;
            if (i < nbw && m < m1) {
              float v[4];
#pragma unroll
              for (int c = 0; c < 4; ++c)
                v[c] = gated_f(g.act_kind, acc[i][j][c] + bg[c], acc[i][j + 2][c] + bu[c],
                               g.alpha, g.beta, g.limit);
              store4((int64_t)m * g.Nout + o0, v, vrow && o0 + 3 < g.Nout, o0, g.Nout);
            }
          }
        }
      }
    } else {
      const bool vrow = (g.Nw & 3) == 0 && aligned;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n0 = nt * kBNW + wn * 64 + 16 * j + 4 * lq;
        if (n0 < g.Nw) {
          float bn[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              bn[c] = bias_at((int64_t)e * g.Nw + min(n0 + c, g.Nw - 1));
          }
#pragma unroll
          for (int i = 0; i < kNI; ++i) {
            const int m = m0 + rowblk(i) + lr;
            if (i < nbw && m < m1) {
              float v[4];
#pragma unroll
              for (int c = 0; c < 4; ++c) v[c] = acc[i][j][c] + bn[c];
              store4((int64_t)m * g.Nw + n0, v, vrow && n0 + 3 < g.Nw, n0, g.Nw);
            }
          }
        }
      }
    }
    if (ti + 1 < ntile) tile(ti + 1, te, tnt, tm0, tm1);
#pragma unroll
    for (int u = 0; u < kPA; ++u) aC[u] = aN[u];
#pragma unroll
    for (int u = 0; u < kPB; ++u) bC[u] = bN[u];
    rbC = rbN;
  }
  // no transfer into LDS may outlive the workgroup
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Expert owning row m under the segment metadata of g (see GemmArgs), or -1.
__device__ int row_owner(const GemmArgs& g, int m) {
  const int32_t* meta = g.offsets;
  if (g.seg_mode == kSegMasked) {
    const int e = m / g.max_m;
    return m % g.max_m < min(max(meta[e], 0), g.max_m) ? e : -1;
  }
  if (g.seg_mode == kSegRuns) {
    for (int e = 0; e < g.E; ++e)
      if (m >= meta[2 * e] && m < meta[2 * e + 1]) return e;
    return -1;
  }
  if (g.seg_mode == kSegEnds) {  // smallest e with ends[e] > m
    if (m >= meta[g.E - 1]) return -1;
    int lo = 0, hi = g.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (meta[mid] > m) hi = mid; else lo = mid + 1;
    }
    return lo;
  }
  if (!meta) return 0;  // one expert owning every row
  if (m < meta[0] || m >= meta[g.E]) return -1;
  int lo = 0, hi = g.E - 1;  // largest e with off[e] <= m
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (meta[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  extern __shared__ float srow[];
  const int m = blockIdx.x;
  const int e = row_owner(g, m);
  if (e < 0) return;
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
    ((float*)g.out)[(int64_t)m * g.Nout + n] = gated_f(g.act_kind, sg, su, g.alpha, g.beta, g.limit);
  } else {
    float s = 0.f;
    for (int k = 0; k < g.Kd; ++k) s = fmaf(srow[k], B[(int64_t)n * g.Kd + k], s);
    if (bias) s += bias[(int64_t)e * g.Nw + n];
    ((float*)g.out)[(int64_t)m * g.Nout + n] = s;
  }
}


// Compute units of the current device (cached per device; 256 if the query fails). The
// persistent grid is sized by it; results do not depend on it.
int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      v <= 0)
    v = 256;
  if (dev < kMaxDevices) cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int NS, int BM, bool ACT, int LAYOUT, bool OUT_F32, int DT, int TAG>
hipError_t launch_h16_ns(const GemmArgs& g, hipStream_t s) {
  const int n_tiles_n = ACT ? (g.Nout + kBNW / 2 - 1) / (kBNW / 2) : (g.Nw + kBNW - 1) / kBNW;
  const int64_t max_tiles = ((int64_t)g.M + BM - 1) / BM + (g.E < g.M ? g.E : g.M);
  int64_t grid = max_tiles * n_tiles_n;
  const int64_t cap = cu_count() / kXcd * kXcd;  // one workgroup per CU
  if (grid > cap) grid = cap;
  grid = (grid + kXcd - 1) / kXcd * kXcd;       // a multiple of the XCD count
  const size_t lds = (size_t)NS * stage_bytes(BM) + map_bytes(g.E);
  const auto kern = gemm_h16_kernel<NS, BM, ACT, LAYOUT, OUT_F32, DT, TAG>;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  kern<<<dim3((unsigned)grid), dim3(kNT), lds, s>>>(g);
  return hipGetLastError();
}

// Three stages (two steps in flight) need at least two steps per tile; a single-step
// contraction runs with two.
// 160-row tiles need three stages and the tile map of E experts in LDS (E up to 335);
// otherwise 128-row tiles (E up to 1024).
// A single expert owning every row (a dense GEMM, e.g. the shared expert) has a tile count
// the host knows: there the tile height with fewer rounds of tiles over the CUs wins, each
// round weighted by its tile's transfer bytes per step (tile rows + 256).
template <bool ACT, int LAYOUT, bool OUT_F32, int DT, int TAG = 0>
hipError_t launch_h16_act(const GemmArgs& g, hipStream_t s) {
  if (g.Kd <= step_elems(DT)) return launch_h16_ns<2, 128, ACT, LAYOUT, OUT_F32, DT, TAG>(g, s);
  bool tall = 3 * stage_bytes(160) + map_bytes(g.E) + kStaticLds <= kLds;
  if (tall && g.seg_mode == kSegOffsets && !g.offsets) {
    const int64_t nt = ACT ? (g.Nout + kBNW / 2 - 1) / (kBNW / 2) : (g.Nw + kBNW - 1) / kBNW;
    const int64_t cus = cu_count() / kXcd * kXcd;
    auto cost = [&](int bm) {
      const int64_t rows = ((int64_t)g.M + bm - 1) / bm, tpt = (g.M + rows - 1) / rows;
      const int64_t h = (tpt + 31) / 32 * 32;  // rows_per_tile
      return ((rows * nt + cus - 1) / cus) * (h + kBNW);
    };
    tall = cost(160) <= cost(128);
  }
  if (tall) return launch_h16_ns<3, 160, ACT, LAYOUT, OUT_F32, DT, TAG>(g, s);
  return launch_h16_ns<3, 128, ACT, LAYOUT, OUT_F32, DT, TAG>(g, s);
}
static_assert(3 * stage_bytes(128) + map_bytes(1024) + kStaticLds <= kLds, "LDS");

template <int DT>
hipError_t launch_h16(const GemmArgs& g, hipStream_t s) {
  if constexpr (DT == 0) {  // float32 operands: float32 outputs only
    if (g.tag == 1 && (!g.act || g.layout == 0))  // the shared expert
      return g.act ? launch_h16_act<true, 0, true, 0, 1>(g, s)
                   : launch_h16_act<false, 0, true, 0, 1>(g, s);
    if (g.act)
      return g.layout == 0 ? launch_h16_act<true, 0, true, 0>(g, s)
                           : launch_h16_act<true, 1, true, 0>(g, s);
    return launch_h16_act<false, 0, true, 0>(g, s);
  } else {
    if (g.tag == 1 && g.out_dt == g.dt && (!g.act || g.layout == 0))  // the shared expert
      return g.act ? launch_h16_act<true, 0, false, DT, 1>(g, s)
                   : launch_h16_act<false, 0, false, DT, 1>(g, s);
    if (g.act) {
      if (g.layout == 0)
        return g.out_dt == 0 ? launch_h16_act<true, 0, true, DT>(g, s)
                             : launch_h16_act<true, 0, false, DT>(g, s);
      return g.out_dt == 0 ? launch_h16_act<true, 1, true, DT>(g, s)
                           : launch_h16_act<true, 1, false, DT>(g, s);
    }
    return g.out_dt == 0 ? launch_h16_act<false, 0, true, DT>(g, s)
                         : launch_h16_act<false, 0, false, DT>(g, s);
  }
}

// The tiled MFMA kernel takes float32 operands whose rows are whole 16-byte pieces (K a
// multiple of 4) and whose byte offsets fit 32 bits, once the product has 2^24
// multiply-adds or more: below that its fixed cost (tile map, ring fill) exceeds the
// row-at-a-time kernel's whole time (the 64-token float32 layer: 25 against 35 us).
bool f32_tiles_ok(const GemmArgs& g) {
  const int64_t lim = (int64_t)1 << 31;
  return g.Kd % 4 == 0 && (int64_t)g.M * g.Kd * 4 < lim && (int64_t)g.Nw * g.Kd * 4 < lim &&
         (int64_t)g.M * g.Nw * g.Kd >= ((int64_t)1 << 24);
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (g.dt == 0 && !f32_tiles_ok(g)) {
    dim3 grid(g.M, (g.Nout + 255) / 256);
    gemm_f32_kernel<<<grid, 256, (size_t)g.Kd * sizeof(float), s>>>(g);
    return hipGetLastError();
  }
  if (g.dt == 0) return launch_h16<0>(g, s);
  return g.dt == 2 ? launch_h16<2>(g, s) : launch_h16<1>(g, s);
}

}  // namespace moe
