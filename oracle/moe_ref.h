/* Plain float64 CPU oracle of the routed Mixture-of-Experts FFN forward, in C.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg load the library built from moe_ref.c. The GPU library neither
 * includes this header nor links that library, and this code uses nothing of the GPU
 * library (no shared headers, helpers or tables).
 *
 * It is the second of the two oracles in this directory: moe_oracle.py writes the same
 * definitions in numpy; this one writes them as loops over tokens, experts and elements
 * (no BLAS), so it can be timed on every host core and checked against the numpy one.
 * The same pins (closed forms, brute force, page constants) run against both.
 *
 * Pages (cited by title and section):
 *   [MR]   ONNX Runtime pull request 32126, "[CUDA] Add MoERouter and SwiGLU contrib
 *          operators" (MoERouter, SwiGLU).
 *   [SPEC] ONNX Runtime pull request 25619, "Update MoE and qMoE spec" (SwiGLU
 *          Activation Function, Fusion Behavior).
 *   [TO]   TileOPs, "MoE Operators" (FusedTopKFwdOp, FusedMoEFwdOp, MoEGroupedGemmFwdOp,
 *          MoEPermuteAlignFwdOp, MoEPostPermuteFwdOp, SharedExpertMLPFwdOp,
 *          MoEGroupedGemmFP8FwdOp).
 *
 * Conventions: arrays are row-major and owned by the caller; every output array is
 * written in full. Input arrays of values carry a storage format code (moe_ref_fmt) and
 * are widened to double exactly, element by element. Functions return 0, or -1 for an
 * argument they cannot take (the message is in moe_ref_last_error()).
 */
#ifndef MOE_REF_H
#define MOE_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats: float64, float32, bfloat16 bits, float16 bits. */
enum moe_ref_fmt { MOE_REF_F64 = 0, MOE_REF_F32 = 1, MOE_REF_BF16 = 2, MOE_REF_F16 = 3 };
enum moe_ref_scoring { MOE_REF_SOFTMAX = 0, MOE_REF_SIGMOID = 1, MOE_REF_SQRT_SOFTPLUS = 2 };
/* Row order of a [2F, K] gate/up weight: gate rows then up rows, or 2j gate, 2j+1 up. */
enum moe_ref_layout { MOE_REF_STACKED = 0, MOE_REF_INTERLEAVED = 1 };
enum moe_ref_kind { MOE_REF_SWIGLU = 0, MOE_REF_GELU = 1 };

typedef struct {
  int32_t layout;  /* moe_ref_layout */
  int32_t kind;    /* moe_ref_kind */
  double alpha, beta, limit;
} moe_ref_act;

typedef struct {
  int64_t E, K;
  int32_t scoring;           /* moe_ref_scoring */
  int32_t renormalize;
  double routed_scaling_factor;
  int64_t num_expert_group;  /* 1: no group limit */
  int64_t topk_group;
} moe_ref_route_cfg;

const char* moe_ref_last_error(void);

/* Worker threads the token- and row-parallel functions use (1 by default; they split
 * independent tokens or rows, never a sum). Returns the count now in force. */
int moe_ref_set_threads(int n);

/* Round x to the nearest value of fmt, ties to even; overflow to infinity. F64: x. */
double moe_ref_round(double x, int32_t fmt);
void moe_ref_round_array(const double* x, int64_t n, int32_t fmt, double* out);
/* Widen n stored values (fmt) to double. */
void moe_ref_widen(const void* x, int32_t fmt, int64_t n, double* out);

/* [MR] MoERouter scoring over all E experts of each of T rows. */
int moe_ref_scores(const void* logits, int32_t logits_fmt, int64_t T, int64_t E,
                   int32_t scoring, double* scores);

/* Indices of n values ordered by value descending, equal values by index ascending. */
void moe_ref_ranked(const double* v, int64_t n, int64_t* order);

/* The router ([MR] MoERouter, [TO] FusedTopKFwdOp): scores, float32 selection keys
 * (bias added when correction_bias is given), the topk_group best groups of
 * num_expert_group, the top_k eligible experts by key (ties to the lower index), or the
 * given expert_ids [T, K] (hash routing, bias ignored); then weights from the unbiased
 * scores, renormalized when asked (wn), times routed_scaling_factor rounded to float32
 * (w). Diagnostics: keys [T, E], group_scores [T, G] (may be NULL), gap_sel and
 * gap_group [T] (smallest gap between consecutive keys among the top_k + 1 best
 * eligible experts; last kept minus first dropped group score; +inf when not defined).
 * scores may be NULL. correction_bias holds E values (float32 after rounding). */
int moe_ref_route(const moe_ref_route_cfg* c, const void* logits, int32_t logits_fmt,
                  int64_t T, const double* correction_bias, const int64_t* expert_ids,
                  double* scores, int64_t* topk_ids, double* wn, double* w, double* keys,
                  double* group_scores, double* gap_sel, double* gap_group);

/* [MR] MoERouter expert-parallel outputs for experts [start, start + count): log(wn) of
 * chosen local experts, fill elsewhere (-1e4 for float16, else -1e30), and
 * routed_scaling_factor * (sum of wn over chosen local experts); both rounded to fmt. */
int moe_ref_ep_outputs(const int64_t* topk_ids, const double* wn, int64_t T, int64_t K,
                       double routed_scaling_factor, int64_t start, int64_t count,
                       int32_t fmt, double* router_probs, double* weight_scale);

/* [MR] SwiGLU / [SPEC] SwiGLU Activation Function; [TO] gelu_and_mul (exact GELU). */
double moe_ref_gated(const moe_ref_act* a, double g, double l);
void moe_ref_gated_array(const moe_ref_act* a, const double* g, const double* l, int64_t n,
                         double* out);

/* One expert on rows x [M, H] (fmt): h = x Wgu^T (+ b_gu), a = act(h) stored in act_fmt,
 * y = a Wd^T (+ b_d), y unrounded. w_gate_up [2F, H], w_down [N, F] (N = H in a layer),
 * biases [2F] and [N] optional. a [M, F], y [M, N]. */
int moe_ref_expert_mlp(const void* x, int64_t M, int64_t H, int64_t F, int64_t N,
                       const void* w_gate_up, const void* w_down, const void* b_gate_up,
                       const void* b_down, int32_t fmt, const moe_ref_act* act,
                       int32_t act_fmt, double* a, double* y);

/* [TO] MoEGroupedGemmFwdOp on the contiguous layout: rows offsets[e] .. offsets[e+1]-1 of
 * a [M, K] times b[e]^T ([E, N, K]) plus bias[e] ([E, N], optional); with act, the gated
 * activation of each row's N values (N/2 outputs). Rows owned by no expert are 0.
 * Results rounded to out_fmt. */
int moe_ref_grouped_gemm(const void* a, int64_t M, int64_t K, const void* b, const void* bias,
                         int64_t E, int64_t N, const int64_t* offsets, int32_t fmt,
                         const moe_ref_act* act, int32_t out_fmt, double* out);

/* Expert-contiguous order of the T*K routes: counts, offsets [E+1], sorted routes
 * (ascending route index inside an expert), and each route's position. */
int moe_ref_permute(const int64_t* topk_ids, int64_t T, int64_t K, int64_t E,
                    int64_t* offsets, int64_t* sorted_route, int64_t* route_pos);

/* [TO] MoEPostPermuteFwdOp: out[t] = scale * sum_k w[t,k] y[route_pos[t K + k]], k
 * ascending, rounded to out_fmt; a negative position adds nothing. y [rows, H] (fmt). */
int moe_ref_combine(const void* y, int32_t fmt, int64_t rows, const double* topk_weights,
                    const int64_t* route_pos, int64_t T, int64_t K, int64_t H, double scale,
                    int32_t out_fmt, double* out);

/* [TO] SharedExpertMLPFwdOp: down(silu(x G^T) * (x U^T)), activation and result stored
 * in out_fmt. w_gate_up [2S, H] (gate rows, then up rows), w_down [H, S]. */
int moe_ref_shared_expert(const void* x, int64_t M, int64_t H, int64_t S,
                          const void* w_gate_up, const void* w_down, int32_t fmt,
                          int32_t out_fmt, double* out);

/* The layer for n_tokens chosen tokens ([TO] FusedMoEFwdOp, FusedMoESharedExpertFwdOp):
 * route each token (as moe_ref_route), then out[t] = sum_k w[t,k] y_k with y_k its k-th
 * expert's output (activation stored in dtype), rounded to dtype; shared_out[t] the
 * shared expert's output (when S > 0). hidden [T, H] and the weights are in fmt; w_gate_up
 * [E, 2F, H], w_down [E, H, F], b_gate_up [E, 2F], b_down [E, H] (optional). tokens NULL:
 * all T. topk_ids / topk_weights [n, K], out / shared_out [n, H]. */
typedef struct {
  int64_t H, F, S;
  moe_ref_route_cfg route;
  moe_ref_act act;
  int32_t fmt;    /* storage format of hidden, weights and biases */
  int32_t dtype;  /* storage format of the activation and the outputs */
} moe_ref_ffn_cfg;

int moe_ref_ffn_forward(const moe_ref_ffn_cfg* c, const void* hidden, int64_t T,
                        const void* logits, int32_t logits_fmt, const double* correction_bias,
                        const int64_t* expert_ids, const void* w_gate_up, const void* w_down,
                        const void* b_gate_up, const void* b_down, const void* shared_w_gate_up,
                        const void* shared_w_down, const int64_t* tokens, int64_t n_tokens,
                        int64_t* topk_ids, double* topk_weights, double* out, double* shared_out);

/* float8_e4m3fn codes to values (NaN only for the all-ones exponent and mantissa). */
void moe_ref_decode_e4m3fn(const uint8_t* codes, int64_t n, double* out);

/* [TO] MoEGroupedGemmFP8FwdOp: out[g, m, n] = sum over 128-wide K blocks kb of
 * (sum_k a b) * a_scale[g, m, kb] * b_scale[g, n / 128, kb], rounded to bfloat16, for
 * m < clamp(counts[g], 0, max_m); other rows NaN. a [E, max_m, K], b [E, N, K] codes;
 * the scales (float32 on the page) are passed widened to double. */
int moe_ref_grouped_gemm_fp8_masked(const uint8_t* a, const double* a_scale, const uint8_t* b,
                                    const double* b_scale, const int64_t* counts, int64_t E,
                                    int64_t max_m, int64_t N, int64_t K, double* out);

#ifdef __cplusplus
}
#endif
#endif
