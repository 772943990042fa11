// Router kernels: scoring, (grouped) top-k selection, weights and the expert-parallel
// router row; one wave64 per token, or four tokens per wave (one per 16-lane row) for
// batches of 1024 tokens or more in the common configurations.
//
// [MR] ONNX Runtime PR 32126 "[CUDA] Add MoERouter and SwiGLU contrib operators",
//      MoERouter: scoring softmax | sigmoid | sqrt_softplus, selection topk | noaux_tc
//      (bias added before the top-k), ties to the lower expert index, expert_ids hash
//      override, router_probs / weight_scale for a local expert slice.
// [TO] TileOPs "MoE Operators", FusedTopKFwdOp / FusedMoEFwdOp: float32 scoring and
//      selection, DeepSeek-V3 group limit, renormalize, routed_scaling_factor once.
//
// Layout: lane l of the token's wave holds experts l, l+64, l+128, ... (coalesced
// loads of the logits row). A selection key is the 64-bit integer
// (order-preserving bits of the float32 key) << 32 | (0xffffffff - expert), so the
// largest key is the largest value and, among equal values, the lowest index; one
// wave-wide max per round picks the next expert.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ uint32_t order_bits(float x) {
  if (x == 0.0f) x = 0.0f;  // -0.0 and +0.0 compare equal, so give them one key
  uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float v, int idx) {
  return ((uint64_t)order_bits(v) << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}

__device__ __forceinline__ int key_index(uint64_t k) {
  return (int)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
}

// Wave reductions (every lane of the wave active). Inside each 16-lane row, four DPP
// exchanges (swap neighbours, swap pairs, mirror halves of 8, mirror the row) leave every
// lane with its row's result; the four rows are then combined from lanes 0, 16, 32, 48 in
// scalar registers, so the result is wave-uniform. No LDS-crossbar shuffles.
constexpr int kDppSwap1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __uint_as_float(lane_u32(__float_as_uint(v), l));
}
__device__ __forceinline__ int lane_i32(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  return ((uint64_t)lane_u32((uint32_t)(v >> 32), l) << 32) | lane_u32((uint32_t)v, l);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppSwap1>(v));
  v = max_u64(v, dpp_u64<kDppSwap2>(v));
  v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
  v = max_u64(v, dpp_u64<kDppMirror>(v));
  return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)),
                 max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

// Sum in a fixed tree order (deterministic for a given wave content).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppSwap1>(v);
  v += dpp_f32<kDppSwap2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// Top two of (a1, a2) and (b1, b2), each pair ordered: the largest and the second largest
// of the four values (duplicates count separately).
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  const float n2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
  a1 = fmaxf(a1, b1);
  a2 = n2;
}
template <int CTRL>
__device__ __forceinline__ void top2_step(float& a1, float& a2) {
  top2_merge(a1, a2, dpp_f32<CTRL>(a1), dpp_f32<CTRL>(a2));
}

// Top two values of a wave (a1 >= a2 in every lane on entry; uniform on exit).
__device__ __forceinline__ void wave_top2(float& a1, float& a2) {
  top2_step<kDppSwap1>(a1, a2);
  top2_step<kDppSwap2>(a1, a2);
  top2_step<kDppHalfMirror>(a1, a2);
  top2_step<kDppMirror>(a1, a2);
  float r1 = lane_f32(a1, 0), r2 = lane_f32(a2, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) top2_merge(r1, r2, lane_f32(a1, l), lane_f32(a2, l));
  a1 = r1;
  a2 = r2;
}

// The N logits of a lane (experts first + STRIDE j of row z0), widened to float32, -inf
// where not valid. The dtype is dispatched once outside the loop, so the N loads are
// issued back to back instead of each behind its own branch.
template <int N, int STRIDE>
__device__ __forceinline__ void load_logits(const RouteArgs& p, int64_t z0, int first,
                                            const bool* valid, float* s) {
  if (p.logits_dt == 0) {
    const float* x = (const float*)p.logits + z0 + first;
#pragma unroll
    for (int j = 0; j < N; ++j) s[j] = valid[j] ? x[STRIDE * j] : -INFINITY;
  } else {
    const uint16_t* x = (const uint16_t*)p.logits + z0 + first;
    uint16_t h[N];
#pragma unroll
    for (int j = 0; j < N; ++j) h[j] = valid[j] ? x[STRIDE * j] : (uint16_t)0;
    if (p.logits_dt == 1) {
#pragma unroll
      for (int j = 0; j < N; ++j) s[j] = valid[j] ? bf16_to_f32(h[j]) : -INFINITY;
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) s[j] = valid[j] ? f16_to_f32(h[j]) : -INFINITY;
    }
  }
}

// u = s + bias (noaux_tc) where a bias is given and the expert is valid, else s.
template <int N, int STRIDE>
__device__ __forceinline__ void add_bias(const RouteArgs& p, int first, const bool* valid,
                                         const float* s, float* u) {
  if (p.bias) {
    float b[N];
#pragma unroll
    for (int j = 0; j < N; ++j) b[j] = valid[j] ? p.bias[first + STRIDE * j] : 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) u[j] = valid[j] ? s[j] + b[j] : s[j];
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) u[j] = s[j];
  }
}

template <int PL>
__global__ __launch_bounds__(64 * kWavesPerBlock) void route_kernel(RouteArgs p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= p.T) return;  // uniform per wave
  const int E = p.E;
  const int64_t z0 = (int64_t)t * E;

  float s[PL], u[PL];
  bool valid[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) valid[j] = lane + 64 * j < E;
  load_logits<PL, 64>(p, z0, lane, valid, s);
  // ---- scoring, float32
  if (p.scoring == 0) {  // softmax over all E experts
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PL; ++j) m = fmaxf(m, s[j]);
    m = wave_max_f32(m);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      s[j] = valid[j] ? expf(s[j] - m) : 0.f;
      sum += s[j];
    }
    sum = wave_sum_f32(sum);
#pragma unroll
    for (int j = 0; j < PL; ++j) s[j] = s[j] / sum;
  } else if (p.scoring == 1) {  // sigmoid
#pragma unroll
    for (int j = 0; j < PL; ++j) s[j] = valid[j] ? 1.0f / (1.0f + expf(-s[j])) : 0.f;
  } else {  // sqrt(softplus(z)) = sqrt(max(z,0) + log1p(exp(-|z|)))
#pragma unroll
    for (int j = 0; j < PL; ++j)
      s[j] = valid[j] ? sqrtf(fmaxf(s[j], 0.f) + log1pf(expf(-fabsf(s[j])))) : 0.f;
  }
  add_bias<PL, 64>(p, lane, valid, s, u);

  // Lane k (< K) ends up holding the k-th chosen expert and its unbiased score.
  int my_sel = 0;
  float my_w = 0.f;
  float wsum = 0.f;  // sum of the chosen scores, k ascending (uniform)
  const int K = p.K;

  if (p.expert_ids) {
    // ---- hash routing: the given experts, bias and groups ignored
    for (int k = 0; k < K; ++k) {
      const int e = __builtin_amdgcn_readfirstlane(p.expert_ids[(int64_t)t * K + k]);
      const int slot = e >> 6;
      float v = 0.f;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (j == slot) v = s[j];
      const float w = lane_f32(v, e & 63);
      wsum += w;
      if (lane == k) { my_sel = e; my_w = w; }
    }
  } else {
    bool elig[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) elig[j] = valid[j];
    if (p.G > 1) {
      // ---- group limit: lane g computes the score of group g
      const int gsz = E / p.G;
      float my_gs = -INFINITY;
      for (int g = 0; g < p.G; ++g) {
        float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < PL; ++j) {
          int e = lane + 64 * j;
          if (valid[j] && e / gsz == g) {
            float v = u[j];
            if (v > a1) { a2 = a1; a1 = v; }
            else if (v > a2) { a2 = v; }
          }
        }
        wave_top2(a1, a2);
        float gs = (p.bias && gsz >= 2) ? a1 + a2 : a1;
        if (lane == g) my_gs = gs;
      }
      uint64_t gkey = lane < p.G ? make_key(my_gs, lane) : 0ull;
      uint64_t kept = 0ull;
      for (int i = 0; i < p.TG; ++i) {
        uint64_t m = wave_max_u64(gkey);
        int g = key_index(m);
        kept |= 1ull << g;
        if (lane == g) gkey = 0ull;
      }
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        int e = lane + 64 * j;
        if (valid[j]) elig[j] = (kept >> (e / gsz)) & 1ull;
      }
    }
    // ---- top-k: K rounds of a wave-wide max over the remaining eligible keys
    uint64_t keys[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) keys[j] = elig[j] ? make_key(u[j], lane + 64 * j) : 0ull;
    for (int k = 0; k < K; ++k) {
      uint64_t best = 0ull;
      float best_s = 0.f;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (keys[j] > best) { best = keys[j]; best_s = s[j]; }
      const uint64_t m = wave_max_u64(best);
      const int e = key_index(m);
      const float w = lane_f32(best_s, e & 63);
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (lane + 64 * j == e) keys[j] = 0ull;
      wsum += w;
      if (lane == k) { my_sel = e; my_w = w; }
    }
  }

  // ---- weights: renormalize, then routed_scaling_factor once
  float wn = p.renormalize ? my_w / wsum : my_w;
  if (lane < K) {
    p.topk_w[(int64_t)t * K + lane] = wn * p.rsf;
    p.topk_ids[(int64_t)t * K + lane] = my_sel;
  }

  // ---- expert-parallel router row and scale
  if (p.router_probs) {
    const int a0 = p.local_start, n = p.local_count;
    const float fill = p.rp_dtype == 2 ? -1.0e4f : -1.0e30f;
    float w_local = 0.f;  // k ascending, uniform
    for (int k = 0; k < K; ++k) {
      const int e = lane_i32(my_sel, k);
      const float w = lane_f32(wn, k);
      if (e >= a0 && e < a0 + n) w_local += w;
    }
    for (int c0 = 0; c0 < n; c0 += 64) {
      int c = c0 + lane;
      float v = fill;
      for (int k = 0; k < K; ++k) {
        const int e = lane_i32(my_sel, k);
        const float w = lane_f32(wn, k);
        if (e == a0 + c) v = logf(w);
      }
      if (c < n) store_dt(p.router_probs, p.rp_dtype, (int64_t)t * n + c, v);
    }
    if (lane == 0) store_dt(p.weight_scale, p.rp_dtype, t, p.rsf * w_local);
  }
}


// ---------------------------------------------------------------------------------
// Row router: four tokens per wave, one per 16-lane row. Lane l of a row holds experts
// l, l + 16, l + 32, ... (EPL of them). Every reduction is the four in-row DPP steps, so a
// row's result reaches all of its lanes without leaving the row, and four tokens share
// each instruction. It covers the common configurations: no expert_ids, top_k <= 16,
// and either no groups or G = EPL / M groups of 16 M experts (E = 16 EPL), G <= 16. The
// selections are those of route_kernel (same keys, same k order for the weight sum);
// only the softmax denominator is summed in another order.
constexpr int kRowLanes = 16;
constexpr int kRowTokens = 4;  // tokens per wave

template <int CTRL>
__device__ __forceinline__ void key_score_step(uint64_t& k, float& s) {
  const uint64_t ok = dpp_u64<CTRL>(k);
  const float os = dpp_f32<CTRL>(s);
  if (ok > k) {
    k = ok;
    s = os;
  }
}

// Largest key of the row and the score carried with it, in every lane of the row.
__device__ __forceinline__ void row_max_key_score(uint64_t& k, float& s) {
  key_score_step<kDppSwap1>(k, s);
  key_score_step<kDppSwap2>(k, s);
  key_score_step<kDppHalfMirror>(k, s);
  key_score_step<kDppMirror>(k, s);
}

__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppSwap1>(v));
  v = max_u64(v, dpp_u64<kDppSwap2>(v));
  v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
  return max_u64(v, dpp_u64<kDppMirror>(v));
}

__device__ __forceinline__ float row_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f32<kDppMirror>(v));
}

// Same value in every lane of the row: each step adds two equal partial sums in either
// order, and float addition is commutative.
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_f32<kDppSwap1>(v);
  v += dpp_f32<kDppSwap2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  return v + dpp_f32<kDppMirror>(v);
}

__device__ __forceinline__ void row_top2(float& a1, float& a2) {
  top2_step<kDppSwap1>(a1, a2);
  top2_step<kDppSwap2>(a1, a2);
  top2_step<kDppHalfMirror>(a1, a2);
  top2_step<kDppMirror>(a1, a2);
}

// Value of lane src (0..63) of the wave, for every lane.
__device__ __forceinline__ int lane_fetch(int v, int src) {
  return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

// EPL experts per lane; M > 0: groups of 16 M experts (M per lane), G = EPL / M.
template <int EPL, int M>
__global__ __launch_bounds__(64 * kWavesPerBlock) void route_rows_kernel(RouteArgs p) {
  const int lane = threadIdx.x & 63;
  const int l = lane & (kRowLanes - 1), row0 = lane & ~(kRowLanes - 1);
  const int t0 = (blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * kRowTokens;
  if (t0 >= p.T) return;  // uniform per wave
  const int t = t0 + (lane >> 4);
  const bool live = t < p.T;  // rows past the last token compute on nothing
  const int E = p.E;
  const int64_t z0 = (int64_t)t * E;

  float s[EPL], u[EPL];
  bool valid[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) valid[j] = live && l + kRowLanes * j < E;
  load_logits<EPL, kRowLanes>(p, z0, l, valid, s);
  // ---- scoring, float32
  if (p.scoring == 0) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) m = fmaxf(m, s[j]);
    m = row_max_f32(m);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      s[j] = valid[j] ? expf(s[j] - m) : 0.f;
      sum += s[j];
    }
    sum = row_sum_f32(sum);
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] = s[j] / sum;
  } else if (p.scoring == 1) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] = valid[j] ? 1.0f / (1.0f + expf(-s[j])) : 0.f;
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      s[j] = valid[j] ? sqrtf(fmaxf(s[j], 0.f) + log1pf(expf(-fabsf(s[j])))) : 0.f;
  }
  add_bias<EPL, kRowLanes>(p, l, valid, s, u);

  bool elig[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) elig[j] = valid[j];
  if constexpr (M > 0) {
    // ---- group limit: group g = experts [16 M g, 16 M (g + 1)), slots j in [M g, M (g+1))
    constexpr int G = EPL / M;
    float my_gs = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
      for (int j = g * M; j < (g + 1) * M; ++j)
        if (valid[j]) {
          const float v = u[j];
          if (v > a1) {
            a2 = a1;
            a1 = v;
          } else if (v > a2) {
            a2 = v;
          }
        }
      row_top2(a1, a2);
      if (l == g) my_gs = p.bias ? a1 + a2 : a1;  // a group holds 16 M >= 2 experts
    }
    uint64_t gkey = l < G ? make_key(my_gs, l) : 0ull;
    uint32_t kept = 0;
    for (int i = 0; i < p.TG; ++i) {
      const int g = key_index(row_max_u64(gkey));
      kept |= 1u << g;
      if (l == g) gkey = 0ull;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) elig[j] = valid[j] && ((kept >> (j / M)) & 1u);
  }

  // ---- top-k: K rounds of a row-wide max; lane k of the row keeps the k-th pick
  uint64_t keys[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) keys[j] = elig[j] ? make_key(u[j], l + kRowLanes * j) : 0ull;
  const int K = p.K;
  int my_sel = 0;
  float my_w = 0.f, wsum = 0.f;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0ull;
    float best_s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (keys[j] > best) {
        best = keys[j];
        best_s = s[j];
      }
    row_max_key_score(best, best_s);
    const int e = key_index(best);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (l + kRowLanes * j == e) keys[j] = 0ull;
    wsum += best_s;
    if (l == k) {
      my_sel = e;
      my_w = best_s;
    }
  }

  const float wn = p.renormalize ? my_w / wsum : my_w;
  if (live && l < K) {
    p.topk_w[(int64_t)t * K + l] = wn * p.rsf;
    p.topk_ids[(int64_t)t * K + l] = my_sel;
  }

  // ---- expert-parallel router row and scale
  if (p.router_probs) {
    const int a0 = p.local_start, n = p.local_count;
    const float fill = p.rp_dtype == 2 ? -1.0e4f : -1.0e30f;
    float w_local = 0.f;  // k ascending
    for (int k = 0; k < K; ++k) {
      const int e = lane_fetch(my_sel, row0 + k);
      const float w = __int_as_float(lane_fetch(__float_as_int(wn), row0 + k));
      if (e >= a0 && e < a0 + n) w_local += w;
    }
    for (int c0 = 0; c0 < n; c0 += kRowLanes) {
      const int c = c0 + l;
      float v = fill;
      for (int k = 0; k < K; ++k) {
        const int e = lane_fetch(my_sel, row0 + k);
        const float w = __int_as_float(lane_fetch(__float_as_int(wn), row0 + k));
        if (e == a0 + c) v = logf(w);
      }
      if (live && c < n) store_dt(p.router_probs, p.rp_dtype, (int64_t)t * n + c, v);
    }
    if (live && l == 0) store_dt(p.weight_scale, p.rp_dtype, t, p.rsf * w_local);
  }
}

// false if this (EPL, m) has no instance (nothing launched).
template <int EPL>
bool launch_rows(const RouteArgs& a, int m, dim3 grid, dim3 block, hipStream_t s) {
  if (m == 0) {
    route_rows_kernel<EPL, 0><<<grid, block, 0, s>>>(a);
    return true;
  }
  if constexpr (EPL >= 8) {  // G = EPL / m groups, at most 16 (one per lane of a row)
    if constexpr (EPL <= kRowLanes) {
      if (m == 1) {
        route_rows_kernel<EPL, 1><<<grid, block, 0, s>>>(a);
        return true;
      }
    }
    if (m == 2) route_rows_kernel<EPL, 2><<<grid, block, 0, s>>>(a);
    else if (m == 4) route_rows_kernel<EPL, 4><<<grid, block, 0, s>>>(a);
    else return false;
    return true;
  }
  return false;
}

// Experts per lane of the row router for this configuration, or 0 when it does not apply.
// *m: experts per lane in one group (0 without groups).
// Below kRowsMinTokens the one-token-per-wave kernel is faster: with fewer waves than
// SIMDs, a token's serial latency decides the time, and a row lane holds 4x the experts.
constexpr int kRowsMinTokens = 1024;

int rows_epl(const RouteArgs& a, int* m) {
  *m = 0;
  if (a.T < kRowsMinTokens || a.expert_ids || a.K > kRowLanes || a.E > 512) return 0;
  const int epl = a.E <= 16 ? 1 : a.E <= 32 ? 2 : a.E <= 64 ? 4 : a.E <= 128 ? 8
                : a.E <= 256 ? 16 : 32;
  if (a.G <= 1) return epl;
  const int gsz = a.E / a.G;
  if (a.E != kRowLanes * epl || epl < 8 || gsz % kRowLanes) return 0;
  const int mm = gsz / kRowLanes;
  if ((mm != 1 && mm != 2 && mm != 4) || epl / mm > kRowLanes) return 0;
  *m = mm;
  return epl;
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  int m = 0;
  const int epl = rows_epl(a, &m);
  if (epl > 0) {
    const int per_block = kWavesPerBlock * kRowTokens;
    const dim3 grid((a.T + per_block - 1) / per_block), block(64 * kWavesPerBlock);
    bool launched = false;
    switch (epl) {
      case 1: launched = launch_rows<1>(a, m, grid, block, s); break;
      case 2: launched = launch_rows<2>(a, m, grid, block, s); break;
      case 4: launched = launch_rows<4>(a, m, grid, block, s); break;
      case 8: launched = launch_rows<8>(a, m, grid, block, s); break;
      case 16: launched = launch_rows<16>(a, m, grid, block, s); break;
      default: launched = launch_rows<32>(a, m, grid, block, s); break;
    }
    if (launched) return hipGetLastError();
    // no instance for this shape: the one-token-per-wave kernel below covers every case
  }
  dim3 grid((a.T + kWavesPerBlock - 1) / kWavesPerBlock), block(64 * kWavesPerBlock);
  if (a.E <= 64) route_kernel<1><<<grid, block, 0, s>>>(a);
  else if (a.E <= 128) route_kernel<2><<<grid, block, 0, s>>>(a);
  else if (a.E <= 256) route_kernel<4><<<grid, block, 0, s>>>(a);
  else route_kernel<8><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
