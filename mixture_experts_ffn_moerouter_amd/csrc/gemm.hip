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
// 16-bit kernel (bfloat16 or float16 operands, the same tiles; only the MFMA and the
// conversions differ), templated on the tile shape: RB and CB 32-row blocks of token rows and of
// weight rows per wave, waves arranged WM x WN, so a tile is 32*RB*WM token rows x
// 32*CB*WN weight rows, K in steps of 64 (v_mfma_f32_32x32x16_bf16, float32
// accumulators); 128 x 128 and 128 x 256 are in use (see launch_bf16). The loop keeps
// the loads of the next K steps in flight in registers (token rows PA steps ahead,
// weights two) while the matrix cores work on the step held in LDS; LDS is double
// buffered (row stride 72 elements: conflict-free 16-byte
// fragment reads), and each load instruction reads whole 128-byte row segments. For the
// gated activation the tile's weight rows are gate rows and the matching up rows, placed
// so that a lane's gate and up accumulators hold the same output element; the epilogue
// pairs them directly. Rows of A may be gathered (a_rows), so the permuted activation
// copy is never materialised. Loads use buffer resources (32-bit offsets from a scalar
// base); out-of-range pieces (rows past the tile, weight rows past N, the K tail, steps
// past the end) get an offset past the buffer's range so the hardware returns zeros
// without a branch, which keeps the compiler's wait counts of the pipeline exact.
//
// Tile map: an expert with M_e rows gets ceil(M_e / (64*RB)) tiles of equal height
// (rounded up to 32 rows); a wave's K loop is compiled for its count of live row blocks.
// Tile counts come from expert_offsets on the device (no host synchronisation); the grid
// is an upper bound, every workgroup rebuilds the map in LDS, picks its (tile, n-tile)
// and leaves if it has none. Consecutive logical tiles go to the same XCD (workgroups are
// dealt round-robin over the 8 XCDs) and are ordered expert, n-tile, row tile: the row
// tiles sharing a weight slice run side by side on one L2, and so do the n-tiles sharing
// the expert's token rows.
#include <type_traits>

#include "moe_internal.h"
#include "tile_map.h"

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kXcd = 8;
// Tile shape: RB 32-row blocks of token rows and CB 32-row blocks of weight rows per wave;
// waves (wm, wn) are WM x WN, so a tile holds 32*RB*WM token rows and 32*CB*WN weight rows.
// BK = K step; LDS rows are BK + 8 elements apart (16-byte fragment reads conflict-free).
template <int RB, int CB, int BK, int NT, int WM> constexpr int stage_elems() {
  return (32 * RB * WM + 32 * CB * (NT / 64 / WM)) * (BK + 8);
}
template <int RB, int CB, int BK, int NT, int WM, int NBUF>
constexpr size_t lds_bytes() { return (size_t)NBUF * stage_elems<RB, CB, BK, NT, WM>() * 2; }
constexpr uint32_t kOOB = 0x80000000u;  // byte offset past every buffer range used here


__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// 32 x 32 x 16 MFMA on eight 16-bit elements per lane: DT 1 bfloat16, 2 float16.
template <int DT>
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The gated activation of the epilogue: kind 1 gelu_and_mul, else the swiglu family.
__device__ __forceinline__ float gated_f(int kind, float g, float l, float alpha, float beta,
                                         float limit) {
  return kind == 1 ? gelu_f(g) * l : swiglu_f(g, l, alpha, beta, limit);
}

template <int RB, int CB, int PA, int BK, int NT, int WM, int OCC, int MID, int NBUF, bool ACT,
          int LAYOUT, bool OUT_F32, int DT>
__global__ __launch_bounds__(NT, OCC) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int LDK = BK + 8, CPR = BK / 8, RSTEP = NT / CPR;  // 16-byte pieces per row
  constexpr int WN = NT / 64 / WM;  // waves: WM along the token rows x WN along the weights
  constexpr int BMX = 32 * RB * WM, BNW = 32 * CB * WN;
  constexpr int NLD = (BMX * BK / 8) / NT, NLDB = (BNW * BK / 8) / NT;
  constexpr int kStageElems = stage_elems<RB, CB, BK, NT, WM>();
  static_assert(lds_bytes<RB, CB, BK, NT, WM, NBUF>() >= 3 * (kMaxE + 1) * sizeof(int),
                "tile map alias");
  static_assert(NBUF == 2 || PA == 1, "one LDS buffer goes with A one step ahead");
  static_assert(NBUF == 2 || MID >= BK / 16, "one LDS buffer: the store follows the last MFMA");
  static_assert(CB == 2 || CB == 4, "weight blocks per wave");
  __shared__ int s_tmp[NT / 64];
  extern __shared__ __align__(16) uint16_t smem[];  // [2][BMX + BNW][LDK]
  int* s_start = (int*)smem;  // the tile map lives in the stage buffers until the K loop
  int* s_len = s_start + kMaxE + 1;
  int* s_pre = s_len + kMaxE + 1;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = g.E;
  build_tile_map_segments<NT>(g.seg_mode, g.offsets, E, g.M, g.max_m, BMX, s_start, s_len,
                              s_pre, s_tmp);

  const int n_tiles_n = ACT ? (g.Nout + BNW / 2 - 1) / (BNW / 2) : (g.Nw + BNW - 1) / BNW;
  const int n_valid = s_pre[E] * n_tiles_n;
  const int per = (n_valid + kXcd - 1) / kXcd;
  const int slot = blockIdx.x / kXcd;
  const int L = (blockIdx.x % kXcd) * per + slot;
  if (slot >= per || L >= n_valid) return;  // uniform per workgroup
  // Logical order: expert, then n-tile, then row tile, so the row tiles that share one
  // weight slice are adjacent (they run side by side on one XCD and the weight lines are
  // fetched from HBM once); expert e owns [s_pre[e], s_pre[e+1]) * n_tiles_n.
  const int e = find_expert(s_pre, E, L / n_tiles_n);
  const int t_e = s_pre[e + 1] - s_pre[e];
  const int local = L - s_pre[e] * n_tiles_n;
  const int nt = local / t_e, mt = local % t_e;
  const int rpt = rows_per_tile(s_len[e], BMX);
  const int m0 = s_start[e] + mt * rpt;
  const int m1 = min(m0 + rpt, s_start[e] + s_len[e]);
  const int rows = m1 - m0;
  const int nb = (rows + 31) / 32;  // live 32-row blocks
  const int Kd = g.Kd;
  __syncthreads();  // every thread has read the map; the buffers become stages

  // ---- loads: thread tid moves 16-byte piece tid % CPR of rows tid / CPR + RSTEP i, i < NLD,
  // of both the A and the B tile (CPR consecutive lanes read one row segment).
  const int kc = (tid % CPR) * 8;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, 0x7fffffff, 0x00020000);
  const uint16_t* Bexp = (const uint16_t*)g.b + (int64_t)e * g.Nw * Kd;
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Bexp, (short)0, (int)((int64_t)g.Nw * Kd * 2), 0x00020000);
  uint32_t aoff[NLD], boff[NLDB];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = tid / CPR + RSTEP * i;
    const bool aon = r < rows;
    const int m = m0 + (aon ? r : 0);
    const int src = g.a_rows ? g.a_rows[m] / g.a_rows_div : m;
    aoff[i] = aon ? ((uint32_t)src * (uint32_t)Kd + kc) * 2u : kOOB;
  }
#pragma unroll
  for (int i = 0; i < NLDB; ++i) {
    const int r = tid / CPR + RSTEP * i;
    int wr;
    bool bon;
    if (ACT) {
      const int j = nt * (BNW / 2) + (r & (BNW / 2 - 1));
      const bool up = r >= BNW / 2;
      bon = j < g.Nout;
      wr = LAYOUT == 0 ? (up ? g.Nout + j : j) : (2 * j + (up ? 1 : 0));
    } else {
      wr = nt * BNW + r;
      bon = wr < g.Nw;
    }
    boff[i] = bon ? ((uint32_t)wr * (uint32_t)Kd + kc) * 2u : kOOB;
  }

  // A (token rows, mostly from L2) is prefetched PA K steps ahead, the weights (from HBM)
  // two: sa0/sa1 hold A of the next step(s), sb0/sb1 the weights of the next two.
  bf16x8 sa0[NLD], sa1[PA == 2 ? NLD : 1], sb0[NLDB], sb1[NLDB];
  auto load_a = [&](int k0, bf16x8* xa) {
    const bool kin = k0 + kc < Kd;
#pragma unroll
    for (int i = 0; i < NLD; ++i) xa[i] = buf_load16(ra, kin ? aoff[i] + 2u * (uint32_t)k0 : kOOB);
  };
  auto load_b = [&](int k0, bf16x8* xb) {
    const bool kin = k0 + kc < Kd;
#pragma unroll
    for (int i = 0; i < NLDB; ++i) xb[i] = buf_load16(rb, kin ? boff[i] + 2u * (uint32_t)k0 : kOOB);
  };
  auto store_stage = [&](int buf, const bf16x8* xa, const bf16x8* xb) {
    uint16_t* la = smem + buf * kStageElems;
    uint16_t* lb = la + BMX * LDK;
#pragma unroll
    for (int i = 0; i < NLD; ++i) *(bf16x8*)(la + (tid / CPR + RSTEP * i) * LDK + kc) = xa[i];
#pragma unroll
    for (int i = 0; i < NLDB; ++i) *(bf16x8*)(lb + (tid / CPR + RSTEP * i) * LDK + kc) = xb[i];
  };

  // wave (wm, wn): row blocks wm, wm+WM, ... (RB of them); weight rows: for the gated
  // activation gate rows wn*16*CB + [0,16*CB) and the matching up rows BNW/2 + the same;
  // else wn*32*CB + [0,32*CB).
  const int wm = wave % WM, wn = wave / WM;
  int brow[CB];
#pragma unroll
  for (int j = 0; j < CB; ++j)
    brow[j] = (ACT ? ((j / (CB / 2)) * (BNW / 2) + wn * 16 * CB + (j % (CB / 2)) * 32)
                   : (wn * 32 * CB + j * 32)) +
              (lane & 31);
  const int kq = (lane >> 5) * 8;
  const int nbw = nb > wm ? (nb - wm + WM - 1) / WM : 0;  // live row blocks of this wave

  f32x16 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x16{};

  // The K loop, compiled once per count of live row blocks so that every fragment read
  // of a sub-step is issued before its MFMAs.
  auto main_loop = [&](auto nbw_c) {
    constexpr int NBW = decltype(nbw_c)::value;
    // compute(buf, mid): the MFMAs of one K step from LDS buffer buf; mid() (the store of
    // the next step and the loads two steps ahead) runs after sub-step MID - 1, pinned
    // there, so those waits and LDS writes overlap the remaining MFMAs (MID = BK/16: at
    // the end).
    auto compute = [&](int buf, auto&& mid) {
      const uint16_t* sa = smem + buf * kStageElems;
      const uint16_t* sb = sa + BMX * LDK;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        if (ks == MID) {
          __builtin_amdgcn_sched_barrier(0);
          mid();
          __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 fb[CB], fa[NBW];
#pragma unroll
        for (int j = 0; j < CB; ++j) fb[j] = *(const bf16x8*)(sb + brow[j] * LDK + ks * 16 + kq);
#pragma unroll
        for (int i = 0; i < NBW; ++i)
          fa[i] = *(const bf16x8*)(sa + ((wm + WM * i) * 32 + (lane & 31)) * LDK + ks * 16 + kq);
#pragma unroll
        for (int i = 0; i < NBW; ++i)
#pragma unroll
          for (int j = 0; j < CB; ++j)
            acc[i][j] = mfma32<DT>(fa[i], fb[j], acc[i][j]);
      }
      if (MID >= BK / 16) mid();
    };
    auto none = [] {};
    // Step s uses LDS buffer s % 2 and weight set sb[s % 2] (and, with PA = 2, A set
    // sa[s % 2]). After storing step k+1 the loads of the steps two ahead (PA = 2: A and
    // weights of k+3) or A of k+2 and then the weights of k+3 (PA = 1) are issued, so the
    // wait before the next store leaves the newest loads in flight. Every half-iteration
    // issues the same loads (steps past the end load nothing: their offsets are out of
    // range), which keeps the compiler's wait counts exact.
    const int nk = (Kd + BK - 1) / BK;
    int k = 0;
    if constexpr (PA == 2) {
      load_a(0, sa0);
      load_b(0, sb0);
      load_a(BK, sa1);
      load_b(BK, sb1);
      store_stage(0, sa0, sb0);
      load_a(2 * BK, sa0);
      load_b(2 * BK, sb0);
      __syncthreads();
      for (; k + 1 < nk; k += 2) {
        compute(0, [&] {
          store_stage(1, sa1, sb1);
          load_a((k + 3) * BK, sa1);
          load_b((k + 3) * BK, sb1);
        });
        __syncthreads();
        compute(1, [&] {
          store_stage(0, sa0, sb0);
          load_a((k + 4) * BK, sa0);
          load_b((k + 4) * BK, sb0);
        });
        __syncthreads();
      }
    } else {
      // With one LDS buffer (NBUF == 1) every step ends with a barrier before the store
      // that overwrites it, and a barrier after.
      constexpr int B1 = NBUF == 2 ? 1 : 0;
      load_a(0, sa0);
      load_b(0, sb0);
      load_b(BK, sb1);
      store_stage(0, sa0, sb0);
      load_a(BK, sa0);
      load_b(2 * BK, sb0);
      __syncthreads();
      for (; k + 1 < nk; k += 2) {
        compute(0, [&] {
          if (NBUF == 1) __syncthreads();
          store_stage(B1, sa0, sb1);
          load_a((k + 2) * BK, sa0);
          load_b((k + 3) * BK, sb1);
        });
        __syncthreads();
        compute(B1, [&] {
          if (NBUF == 1) __syncthreads();
          store_stage(0, sa0, sb0);
          load_a((k + 3) * BK, sa0);
          load_b((k + 4) * BK, sb0);
        });
        __syncthreads();
      }
    }
    if (k < nk) compute(0, none);  // odd number of K steps: the last one is in buffer 0
  };
  // With 128-row tiles the loop is compiled for 2 and for 1 live row blocks of the wave;
  // with 256-row tiles one loop covers all 4 (blocks past the tile's last row read rows
  // that load as zeros, and their results are not written).
  if constexpr (RB == 2) {
    if (nbw >= 2) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 1>{});
  } else if constexpr (RB == 4 && CB == 2) {
    if (nbw >= 3) main_loop(std::integral_constant<int, 4>{});
    else main_loop(std::integral_constant<int, 2>{});
  } else {
    main_loop(std::integral_constant<int, RB>{});
  }

  // ---- epilogue. Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4
  // and column l%32 of its 32 x 32 block.
  const uint16_t* bias = (const uint16_t*)g.bias;
  if (ACT) {
#pragma unroll
    for (int h = 0; h < CB / 2; ++h) {  // 32-column groups of this wave's 16*CB outputs
      const int j = nt * (BNW / 2) + wn * 16 * CB + h * 32 + (lane & 31);
      if (j < g.Nout) {
        float bg = 0.f, bu = 0.f;
        if (bias) {
          const uint16_t* be = bias + (int64_t)e * g.Nw;
          bg = h16_to_f32<DT>(be[LAYOUT == 0 ? j : 2 * j]);
          bu = h16_to_f32<DT>(be[LAYOUT == 0 ? g.Nout + j : 2 * j + 1]);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          if (i < nbw) {
            const int rb = wm + WM * i;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = m0 + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              if (m < m1) {
                float v = gated_f(g.act_kind, acc[i][h][r] + bg, acc[i][CB / 2 + h][r] + bu,
                                  g.alpha, g.beta, g.limit);
                if (OUT_F32) ((float*)g.out)[(int64_t)m * g.Nout + j] = v;
                else ((uint16_t*)g.out)[(int64_t)m * g.Nout + j] = f32_to_h16<DT>(v);
              }
            }
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int jb = 0; jb < CB; ++jb) {
      const int n = nt * BNW + wn * 32 * CB + jb * 32 + (lane & 31);
      if (n < g.Nw) {
        const float bn = bias ? h16_to_f32<DT>(bias[(int64_t)e * g.Nw + n]) : 0.f;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          if (i < nbw) {
            const int rb = wm + WM * i;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = m0 + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              if (m < m1) {
                float v = acc[i][jb][r] + bn;
                if (OUT_F32) ((float*)g.out)[(int64_t)m * g.Nw + n] = v;
                else ((uint16_t*)g.out)[(int64_t)m * g.Nw + n] = f32_to_h16<DT>(v);
              }
            }
          }
        }
      }
    }
  }
}

// float32 operands: one workgroup per output row; the A row is staged in LDS and each
// thread forms the dot products of its output column(s). Plain FMA arithmetic; meant
// for small float32 problems.
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

template <int RB, int CB, int PA, int BK, int NT, int WM, int OCC, int MID, int NBUF, bool ACT,
          int LAYOUT, bool OUT_F32, int DT>
hipError_t launch_bf16_shape(const GemmArgs& g, hipStream_t s) {
  constexpr int BMX = 32 * RB * WM, BNW = 32 * CB * (NT / 64 / WM);
  const int n_tiles_n = ACT ? (g.Nout + BNW / 2 - 1) / (BNW / 2) : (g.Nw + BNW - 1) / BNW;
  const int64_t max_tiles = (g.M + BMX - 1) / BMX + (g.E < g.M ? g.E : g.M);
  int64_t grid = max_tiles * n_tiles_n;
  grid = (grid + kXcd - 1) / kXcd * kXcd;
  const auto kern = gemm_bf16_kernel<RB, CB, PA, BK, NT, WM, OCC, MID, NBUF, ACT, LAYOUT, OUT_F32, DT>;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes<RB, CB, BK, NT, WM, NBUF>());
  if (err != hipSuccess) return err;
  kern<<<dim3((unsigned)grid), dim3(NT), lds_bytes<RB, CB, BK, NT, WM, NBUF>(), s>>>(g);
  return hipGetLastError();
}

// Two shapes, chosen by the contraction length. Long contractions (Kd >= 2560) take 128
// token rows x 256 weight rows per workgroup, eight waves (2 x 4) of 64 x 64, one
// workgroup per CU: half as many n-tiles re-read each expert's token rows per weight
// byte. Shorter ones take 128 x 128 with four waves and two workgroups per CU, where one
// workgroup's prologue and epilogue overlap the other's K loop. Both keep the two
// operands two K steps ahead. Measured in one process, alternating the shapes: 5% and 3%
// faster layers with the wide tile at Kd 7168 and 2880, 2% slower at Kd 2048 / 768.
template <bool ACT, int LAYOUT, bool OUT_F32, int DT>
hipError_t launch_bf16(const GemmArgs& g, hipStream_t s) {
  // <RB, CB, PA, BK, NT, WM, OCC, MID, NBUF>
  if (g.Kd >= 2560)
    return launch_bf16_shape<2, 2, 2, 64, 512, 2, 1, 4, 2, ACT, LAYOUT, OUT_F32, DT>(g, s);
  return launch_bf16_shape<2, 2, 2, 64, 256, 2, 2, 4, 2, ACT, LAYOUT, OUT_F32, DT>(g, s);
}

template <int DT>
hipError_t launch_h16(const GemmArgs& g, hipStream_t s) {
  if (g.act) {
    if (g.layout == 0)
      return g.out_dt == 0 ? launch_bf16<true, 0, true, DT>(g, s)
                           : launch_bf16<true, 0, false, DT>(g, s);
    return g.out_dt == 0 ? launch_bf16<true, 1, true, DT>(g, s)
                         : launch_bf16<true, 1, false, DT>(g, s);
  }
  return g.out_dt == 0 ? launch_bf16<false, 0, true, DT>(g, s)
                       : launch_bf16<false, 0, false, DT>(g, s);
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0) return hipSuccess;
  if (g.dt == 0) {
    dim3 grid(g.M, (g.Nout + 255) / 256);
    gemm_f32_kernel<<<grid, 256, (size_t)g.Kd * sizeof(float), s>>>(g);
    return hipGetLastError();
  }
  return g.dt == 2 ? launch_h16<2>(g, s) : launch_h16<1>(g, s);
}

}  // namespace moe
