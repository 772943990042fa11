/*
 * moe.h - C ABI of libmoe.so: the routed Mixture-of-Experts FFN forward on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [MR]   ONNX Runtime pull request 32126, "[CUDA] Add MoERouter and SwiGLU contrib
 *          operators".
 *   [CPU]  onnx-light-cpu, "MoE (CPU)" kernel schema.
 *   [SPEC] ONNX Runtime pull request 25619, "Update MoE and qMoE spec".
 *   [TO]   TileOPs, "MoE Operators" API page.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers (HBM) unless said otherwise; every row is
 *     contiguous ("row-major") and tensors are packed (no padding between rows).
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue work:
 *     they never synchronise the stream and never read device data on the host
 *     ([TO] MoEGroupedGemmFwdOp: metadata is not checked, since checking would
 *     synchronise). Device-side metadata (expert ids, offsets) outside its stated
 *     range is a precondition violation, not an error that is reported.
 *   - Ownership: the caller owns every buffer, including workspaces. The library
 *     allocates no device memory and keeps no mutable global state, apart from the
 *     fixed device scratch of moe_ffn_forward_noalloc; calls on one stream are
 *     ordered, calls on different streams must not share output buffers.
 *   - Errors: every argument check runs on the host before anything is enqueued; a
 *     call that returns an error has launched nothing and written nothing. An output
 *     that overlaps an input returns MOE_ERR_OVERLAP before any write ([TO]
 *     MoEPostPermuteFwdOp, MoEGroupedGemmFwdOp: overlap is rejected before writing).
 *   - Sizes of zero (T == 0, M == 0) return MOE_OK and launch nothing (moe_permute
 *     still writes its E+1 zero offsets); pointers to zero-sized buffers may be NULL.
 *   - dtypes: operands are MOE_F32, MOE_BF16 or MOE_F16 (the same dtype for activations
 *     and weights); router logits are float32, bfloat16 or float16 ([TO] FusedTopKFwdOp)
 *     and are read exactly into float32; routing weights are float32.
 *   - ABI version 2 (moe_abi_version): moe_route_cfg.logits_dtype and moe_act_cfg.kind
 *     were added at the ends of those structs, and logits became `const void*`.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null required pointer, bad size or bad option      */
  MOE_ERR_UNSUPPORTED = 2,  /* valid per the pages, not implemented here           */
  MOE_ERR_OVERLAP = 3,      /* an output overlaps an input                         */
  MOE_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the query returns */
  MOE_ERR_LAUNCH = 5        /* the HIP runtime refused a launch                    */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;

/* [MR] MoERouter scoring attribute; [TO] FusedTopKFwdOp scoring_func. */
typedef enum {
  MOE_SCORE_SOFTMAX = 0,       /* softmax over all E logits                       */
  MOE_SCORE_SIGMOID = 1,       /* 1 / (1 + exp(-z))                               */
  MOE_SCORE_SQRT_SOFTPLUS = 2  /* sqrt(log(1 + exp(z)))                           */
} moe_scoring;

/* Row order of a [.., 2F, H] gate/up weight ([SPEC] Fusion Behavior; [TO]
 * MoEGroupedGemmFwdOp): STACKED = F gate rows then F up rows; INTERLEAVED = row 2j is
 * gate j and row 2j+1 is up j. */
typedef enum { MOE_GU_STACKED = 0, MOE_GU_INTERLEAVED = 1 } moe_gu_layout;

typedef enum { MOE_BACKEND_AUTO = 0, MOE_BACKEND_STAGED = 1, MOE_BACKEND_INDEXED = 2 }
    moe_backend;

/* Expert row layouts of [TO] MoEGroupedGemmFwdOp's table:
 *   CONTIGUOUS  rows [M, .] grouped by expert; metadata [E] = segment ends (expert g owns
 *               rows end[g-1] .. end[g]-1, end[-1] = 0; segments may include padding)
 *   PER_ROW     rows [M, .] grouped by expert; metadata [M] = expert id of each row (ids
 *               outside [0, E) mark rows of no expert; each expert's rows form one run)
 *   MASKED      slabs [E, max_m, .]; metadata [E] = valid rows of each expert, read as
 *               max_m when larger and 0 when negative                               */
typedef enum { MOE_LAYOUT_CONTIGUOUS = 0, MOE_LAYOUT_PER_ROW = 1, MOE_LAYOUT_MASKED = 2 }
    moe_layout;

/* Router options ([MR] MoERouter attributes; [TO] FusedTopKFwdOp __init__ and forward).
 *   top_k                 experts per token, 1 <= top_k <= min(E, 32)
 *   scoring               moe_scoring
 *   renormalize           nonzero: divide the chosen scores by their sum
 *   routed_scaling_factor > 0, multiplies the returned weights once, after the
 *                         renormalization
 *   num_expert_group      G >= 1 groups of E/G consecutive experts (E % G == 0, G <= 64)
 *   topk_group            groups kept per token, 1 <= topk_group <= G, and the kept
 *                         groups must hold at least top_k experts
 *   local_expert_start/count  the expert-parallel slice [start, start+count) that
 *                         router_probs describes (0 <= start, start+count <= E)
 *   router_probs_dtype    moe_dtype of router_probs and weight_scale
 *   logits_dtype          moe_dtype of the logits (each value is converted exactly to
 *                         float32 before scoring)                                   */
typedef struct {
  int32_t top_k;
  int32_t scoring;
  int32_t renormalize;
  float routed_scaling_factor;
  int32_t num_expert_group;
  int32_t topk_group;
  int32_t local_expert_start;
  int32_t local_expert_count;
  int32_t router_probs_dtype;
  int32_t logits_dtype;
} moe_route_cfg;

/* Kind of gated activation: the SwiGLU family, or gelu_and_mul. */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GELU_AND_MUL = 1 } moe_act_kind;

/* Gated activation of the gate_up GEMM ([MR] SwiGLU; [SPEC] SwiGLU Activation
 * Function; [TO] MoEGroupedGemmFwdOp):
 *   kind MOE_ACT_SWIGLU: out_j = G * sigmoid(alpha * G) * (L + beta),
 *     G = min(gate_j, limit), L = clamp(up_j, -limit, limit); limit <= 0 turns both
 *     clamps off. silu_and_mul = {STACKED, 1, 0, 0, SWIGLU};
 *     swigluoai = {INTERLEAVED, 1.702, 1, 7, SWIGLU}.
 *   kind MOE_ACT_GELU_AND_MUL: out_j = gelu(gate_j) * up_j with the exact GELU
 *     x * Phi(x) (the pages name the activation only; the exact form is the reading
 *     taken); STACKED layout only; alpha, beta and limit are ignored. */
typedef struct {
  int32_t layout; /* moe_gu_layout */
  float alpha;
  float beta;
  float limit;
  int32_t kind;   /* moe_act_kind */
} moe_act_cfg;

/* Whole-layer configuration for moe_ffn_forward. F_shared = 0: no shared expert.
 * dtype: operand dtype of hidden, weights, biases and outputs. backend: moe_backend. */
typedef struct {
  moe_route_cfg route;
  moe_act_cfg act;
  int64_t T, H, E, F, F_shared;
  int32_t dtype;
  int32_t backend;
} moe_ffn_cfg;

/* Text of a status code. Host only; never fails. */
const char* moe_status_str(int status);

/* Library ABI version (this header: 2). Host only. */
int moe_abi_version(void);

/* ---------------------------------------------------------------------------------
 * moe_route - router: scores, selection, weights, expert-parallel outputs.
 * [MR] MoERouter; [TO] FusedTopKFwdOp and FusedMoEFwdOp (grouped routing).
 *
 * logits          [T, E] router logits in cfg->logits_dtype (float32, bfloat16 or
 *                 float16; [TO] FusedTopKFwdOp).
 * correction_bias [E] float32 or NULL. Added to the scores for the selection only
 *                 (noaux_tc); the weights use the unbiased scores.
 * expert_ids      [T, top_k] int32 or NULL. When given, it replaces the selection
 *                 (hash routing) and the bias and groups are ignored. Ids must lie in
 *                 [0, E); repeated ids in a row are a precondition violation.
 * Selection: the top_k experts with the largest float32 key (score + bias), ties to the
 * lower expert index; with G > 1, only inside the topk_group groups whose score is
 * largest (sum of the two best keys when a bias is given, else the best score; ties
 * to the lower group). Each topk_ids row is ordered by key descending, ties by index.
 * topk_weights    [T, top_k] float32 out: score of each chosen expert, divided by the
 *                 sum of the chosen scores when renormalize, times
 *                 routed_scaling_factor.
 * topk_ids        [T, top_k] int32 out.
 * router_probs    [T, local_expert_count] in router_probs_dtype, or NULL: log of the
 *                 normalized weight (before routed_scaling_factor) at a chosen expert of
 *                 the slice, -1e30 elsewhere (-1e4 for float16) [MR].
 * weight_scale    [T] in router_probs_dtype, or NULL (given together with
 *                 router_probs): routed_scaling_factor * sum of the normalized weights
 *                 of the chosen experts in the slice; exactly 0 with none [MR].
 * Errors: INVALID_ARG for null logits/topk outputs, E < 1, bad cfg fields;
 * UNSUPPORTED for E > 512 or T * max(E, top_k) >= 2^31;
 * OVERLAP if an output overlaps logits/bias/expert_ids or another output.
 * ------------------------------------------------------------------------------- */
int moe_route(const void* logits, int64_t T, int64_t E, const float* correction_bias,
              const int32_t* expert_ids, const moe_route_cfg* cfg, float* topk_weights,
              int32_t* topk_ids, void* router_probs, void* weight_scale, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_permute - expert-contiguous (tight, no padding) order of the R = T*top_k routes.
 * [TO] MoEPrePermuteFwdOp, MoEPermuteAlignFwdOp (here without padding), and the
 * contiguous layout of MoEGroupedGemmFwdOp.
 *
 * topk_ids        [T, K] int32 in [0, E); route r = t*K + k.
 * expert_offsets  [E+1] int32 out: routes of expert e occupy permuted rows
 *                 expert_offsets[e] .. expert_offsets[e+1]-1; expert_offsets[E] = R.
 * sorted_route    [R] int32 out: the route at each permuted row; inside one expert the
 *                 routes are in ascending r (a fixed order; the pages leave it open).
 * route_pos       [R] int32 out: inverse of sorted_route (permuted row of route r).
 * hidden, permuted  optional (both NULL or both given): permuted[m] =
 *                 hidden[sorted_route[m] / K], rows of H elements of dtype dt.
 * workspace       device scratch of at least moe_permute_workspace_size(T, K, E) bytes
 *                 (per-workgroup expert counts); contents on entry do not matter.
 * Limits: E <= 1024, R < 2^31. Errors: INVALID_ARG, OVERLAP, WORKSPACE.
 * moe_permute_workspace_size: host only; 0 for invalid sizes.
 * ------------------------------------------------------------------------------- */
size_t moe_permute_workspace_size(int64_t T, int64_t K, int64_t E);
int moe_permute(const int32_t* topk_ids, int64_t T, int64_t K, int64_t E,
                int32_t* expert_offsets, int32_t* sorted_route, int32_t* route_pos,
                const void* hidden, int64_t H, int32_t dt, void* permuted, void* workspace,
                size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_grouped_gemm_swiglu - grouped gate_up GEMM with the gated activation in its
 * epilogue; the [M, 2F] product is never written.
 * [TO] MoEGroupedGemmFwdOp (activation fused, bias [E, 2F] in b's row order added to
 * the float32 product before the activation), MoEExpertMLPFwdOp; [MR] SwiGLU.
 *
 * a               activations of dtype dt. If a_rows is NULL, a is [M, H] and row m of
 *                 the product uses a[m]; otherwise row m uses a[a_rows[m] / a_rows_div]
 *                 (a gather, e.g. hidden[T, H] with sorted_route and a_rows_div = K).
 * w_gate_up       [E, 2F, H] dt, rows in act->layout order.
 * b_gate_up       [E, 2F] dt or NULL.
 * expert_offsets  [E+1] int32: rows of expert e are expert_offsets[e] ..
 *                 expert_offsets[e+1]-1 (non-decreasing, expert_offsets[E] <= M).
 * out             [M, F] dt: act(a W_e^T + b_e) rounded to dt (ties to even). Rows not
 *                 covered by any expert are left unwritten.
 * Accumulation is float32. Limits: H % 8 == 0 for bf16/f16 (16-byte rows), E <= 1024;
 * for bf16/f16, M*H*2 and 2F*H*2 below 2^31 bytes (32-bit offsets; a gathered source
 * must also stay below 2^31 bytes). INVALID_ARG for gelu_and_mul with INTERLEAVED rows.
 * Errors: INVALID_ARG, UNSUPPORTED, OVERLAP (out vs a, weights, bias, offsets, a_rows).
 * With a gather, the rows read are named by a_rows on the device, which the host does
 * not read: OVERLAP covers a's first row only, and out must not overlap any gathered row
 * (a precondition, like the device metadata's ranges).
 * ------------------------------------------------------------------------------- */
int moe_grouped_gemm_swiglu(const void* a, const int32_t* a_rows, int32_t a_rows_div,
                            int64_t M, int64_t H, const void* w_gate_up,
                            const void* b_gate_up, int64_t E, int64_t F,
                            const int32_t* expert_offsets, int32_t dt,
                            const moe_act_cfg* act, void* out, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_grouped_gemm - plain grouped GEMM: out[rows of e] = a[rows of e] b[e]^T + bias[e].
 * [TO] MoEGroupedGemmFwdOp (contiguous layout, b is [E, N, K], float32 accumulation,
 * output in the operand dtype unless float32 is asked for).
 *
 * a, a_rows, a_rows_div  as in moe_grouped_gemm_swiglu, with K columns.
 * b               [E, N, K] dt.   bias  [E, N] dt or NULL.
 * out             [M, N] in out_dt (dt or MOE_F32). Rows outside every expert are left
 *                 unwritten.
 * Limits: K % 8 == 0 for bf16/f16, E <= 1024, M*K*2 and N*K*2 below 2^31 bytes for
 * bf16/f16 (32-bit offsets; a gathered source must also stay below 2^31 bytes).
 * Errors: INVALID_ARG, UNSUPPORTED, OVERLAP.
 * ------------------------------------------------------------------------------- */
int moe_grouped_gemm(const void* a, const int32_t* a_rows, int32_t a_rows_div, int64_t M,
                     int64_t K, const void* b, const void* bias, int64_t E, int64_t N,
                     const int32_t* expert_offsets, int32_t dt, int32_t out_dt, void* out,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * moe_grouped_gemm_layout - grouped GEMM over one of the layouts (moe_layout), with an
 * optional gated activation.
 * [TO] MoEGroupedGemmFwdOp (layout table; activation fused; bias added to the float32
 * product before the activation; output in the operand dtype or float32).
 *
 * a        CONTIGUOUS / PER_ROW: [M, K] dt.  MASKED: [E, max_m, K] dt (M is ignored).
 * b        [E, N, K] dt (with act: N = 2F gate/up rows in act->layout order).
 * bias     [E, N] dt or NULL.
 * layout_metadata  per layout (moe_layout), int32 on the device, not checked beyond
 *          clamping every expert's rows into the rows that exist.
 * act      NULL for a plain GEMM; else the gated activation (output width F = N/2).
 * out      rows like a ([M, N or F], or [E, max_m, N or F]) in out_dt (dt or MOE_F32):
 *          rows of an expert computed, rows of no expert (padding, masked rows past the
 *          count) left unwritten. A CONTIGUOUS segment's padding rows are computed with
 *          its expert's weights (their values are unspecified either way).
 * workspace  PER_ROW: moe_grouped_gemm_layout_workspace_size(E) bytes (each expert's run,
 *          found from the row ids); other layouts: may be NULL.
 * Limits and errors as moe_grouped_gemm; INVALID_ARG for an unknown layout, max_m < 0,
 * an odd N with act; WORKSPACE when PER_ROW lacks its workspace.
 * ------------------------------------------------------------------------------- */
size_t moe_grouped_gemm_layout_workspace_size(int64_t E);
int moe_grouped_gemm_layout(const void* a, int64_t M, int64_t K, const void* b,
                            const void* bias, int64_t E, int64_t N, int32_t layout,
                            const int32_t* layout_metadata, int64_t max_m,
                            const moe_act_cfg* act, int32_t dt, int32_t out_dt, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_permute_align - routes grouped by expert, each expert's range padded to a multiple
 * of block_size.
 * [TO] MoEPermuteAlignFwdOp. numel = T*K routes (route r = t*K + k), count[e] on expert e.
 *
 * sorted_token_ids  [numel + (E+1)(block_size-1)] int32 out: expert e's range (in expert
 *          order, length count[e] rounded up to block_size) holds its routes in ascending
 *          route index (the page leaves this order open), then numel; every entry past
 *          num_tokens_post_pad is numel.
 * expert_ids  [ceil(len(sorted_token_ids) / block_size)] int32 out: the owner of each
 *          block of the ranges, -1 past them.
 * num_tokens_post_pad  [1] int32 out: sum of the padded lengths.
 * workspace  moe_layout_workspace_size(T, K, E, block_size) bytes.
 * Limits: E <= 1024, block_size >= 1, numel + (E+1)(block_size-1) < 2^31.
 * Errors: INVALID_ARG, UNSUPPORTED, OVERLAP, WORKSPACE.
 * ------------------------------------------------------------------------------- */
size_t moe_layout_workspace_size(int64_t T, int64_t K, int64_t E, int64_t block_size);
int moe_permute_align(const int32_t* topk_ids, int64_t T, int64_t K, int64_t E,
                      int64_t block_size, int32_t* sorted_token_ids, int32_t* expert_ids,
                      int32_t* num_tokens_post_pad, void* workspace, size_t workspace_bytes,
                      void* stream);

/* ---------------------------------------------------------------------------------
 * moe_pre_permute - token rows materialised in an expert layout.
 * [TO] MoEPrePermuteFwdOp: (expert_input, layout_metadata, inverse_indices).
 *
 * hidden   [T, H] dt.   topk_ids [T, K] int32 in [0, E).
 * CONTIGUOUS / PER_ROW (rows of moe_permute_align with block_size; 1 = unpadded):
 *   expert_input  [T*K + E(block_size-1), H] dt: row m of the used length holds
 *                 hidden[r / K] for the route r placed there; padding and rows past the
 *                 used length are left unwritten.
 *   layout_metadata  CONTIGUOUS: [E] segment ends; PER_ROW: [T*K + E(block_size-1)]
 *                 expert id per row, -1 on padding and unused rows.
 * MASKED (block_size ignored):
 *   expert_input  [E, max_m, H] dt: slab row (e, j) holds the j-th route of expert e in
 *                 route order, for j < min(count[e], max_m); other rows unwritten.
 *   layout_metadata  [E] = min(count[e], max_m). A route ranked max_m or later in its
 *                 expert has no room (the pages leave capacity overflow open).
 * inverse_indices  [T*K] int32 out: the row of expert_input (flattened) holding route r,
 *          or -1 for a route without room; moe_combine takes it as route_pos.
 * workspace  moe_layout_workspace_size(T, K, E, block_size) bytes (1 for MASKED).
 * Errors: INVALID_ARG, UNSUPPORTED, OVERLAP, WORKSPACE.
 * ------------------------------------------------------------------------------- */
int moe_pre_permute(const void* hidden, int64_t T, int64_t H, int32_t dt,
                    const int32_t* topk_ids, int64_t K, int64_t E, int32_t layout,
                    int64_t block_size, int64_t max_m, void* expert_input,
                    int32_t* layout_metadata, int32_t* inverse_indices, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_combine - back to token order, routing weights applied, top-k reduced, cast.
 * [TO] MoEPostPermuteFwdOp (weights applied exactly once), FusedMoEExpertsFwdOp.
 *
 * y               [y_rows, H] in y_dt (MOE_F32 or the operand dtype): expert outputs in
 *                 any layout (a masked [E, max_m, H] slab is y_rows = E*max_m); every
 *                 non-negative route_pos entry must be below y_rows.
 * topk_weights    [T, K] float32.   route_pos [T*K] int32: the row of y holding each route
 *                 (moe_permute's route_pos, or moe_pre_permute's inverse_indices); a
 *                 negative entry contributes nothing.
 * out             [T, H] out_dt: scale * sum_k topk_weights[t,k] * y[route_pos[t*K+k]],
 *                 summed in float32 over k ascending, then rounded to out_dt.
 * Errors: INVALID_ARG, OVERLAP (out vs y, topk_weights, route_pos).
 * ------------------------------------------------------------------------------- */
int moe_combine(const void* y, int32_t y_dt, int64_t y_rows, const float* topk_weights,
                const int32_t* route_pos, int64_t T, int64_t K, int64_t H, float scale,
                void* out, int32_t out_dt, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_swiglu - standalone SwiGLU operator.
 * [MR] SwiGLU (float arithmetic whatever the storage type; optional up: without it gate
 * holds both halves of one [.., 2F] projection, gate first, then up); [SPEC] Fusion
 * Behavior (the fused projection may be interleaved instead).
 *
 * gate    [rows, F] in dt when up is given; else [rows, 2F] in dt, halves arranged per
 *         fusion: MOE_GU_STACKED = [gate | up], MOE_GU_INTERLEAVED = element 2j gate j,
 *         2j+1 up j.
 * up      [rows, F] in dt, or NULL.
 * out     [rows, F] in dt: G * sigmoid(alpha G) * (L + beta), G = min(gate, limit),
 *         L = clamp(up, -limit, limit) (limit <= 0: no clamps), rounded to dt once.
 * dt      MOE_F32, MOE_BF16 or MOE_F16 (inputs and output).
 * Errors: INVALID_ARG (null pointer with rows > 0, F < 1, bad fusion), UNSUPPORTED
 * (dtype, F >= 2^30), OVERLAP (out vs gate or up).
 * ------------------------------------------------------------------------------- */
int moe_swiglu(const void* gate, const void* up, int64_t rows, int64_t F, int32_t dt,
               int32_t fusion, float alpha, float beta, float limit, void* out,
               void* stream);

/* ---------------------------------------------------------------------------------
 * moe_ffn_workspace_size - bytes of device workspace moe_ffn_forward needs for cfg
 * (for either backend). Host only; returns 0 for an invalid cfg.
 * moe_ffn_backend - the backend moe_ffn_forward runs for cfg (MOE_BACKEND_STAGED or
 * MOE_BACKEND_INDEXED), has_bias = whether b_gate_up or b_down is given. AUTO follows
 * [TO] FusedMoEExpertsFwdOp: INDEXED when T*top_k <= 2E, the activation is
 * silu_and_mul, there is no bias, H % 128 == 0 and F % 256 == 0; STAGED otherwise.
 * Host only; returns -1 for an invalid cfg.
 * ------------------------------------------------------------------------------- */
size_t moe_ffn_workspace_size(const moe_ffn_cfg* cfg);
int moe_ffn_backend(const moe_ffn_cfg* cfg, int has_bias);

/* ---------------------------------------------------------------------------------
 * moe_ffn_forward - the routed MoE FFN layer, plus the optional shared expert.
 * [TO] FusedMoEFwdOp, FusedMoESharedExpertFwdOp, FusedMoEExpertsFwdOp,
 * IndexedExpertMLPFwdOp, SharedExpertMLPFwdOp; [MR] MoERouter.
 *
 * hidden [T, H] dt; logits [T, E] in cfg->route.logits_dtype; correction_bias [E]
 * float32 or NULL;
 * expert_ids [T, top_k] int32 or NULL (hash routing); w_gate_up [E, 2F, H] dt;
 * w_down [E, H, F] dt; b_gate_up [E, 2F] dt or NULL; b_down [E, H] dt or NULL;
 * shared_w_gate_up [2F_shared, H] dt (gate rows then up rows) and shared_w_down
 * [H, F_shared] dt, required when cfg->F_shared > 0.
 * out         [T, H] dt: sum_k w[t,k] (down_k(act(gate_up_k(h_t) + b_gu)) + b_down),
 *             w including routed_scaling_factor (applied once).
 * shared_out  [T, H] dt, or NULL when F_shared == 0: down(silu(h G^T) * (h U^T)),
 *             the activation rounded to dt before the down projection; not scaled.
 *             The caller adds out and shared_out when it needs the layer output.
 * topk_weights_out [T, top_k] float32 / topk_ids_out [T, top_k] int32: optional
 *             copies of the routing (NULL = not returned).
 * workspace   device buffer of at least moe_ffn_workspace_size(cfg) bytes, 256-byte
 *             aligned; its contents on entry do not matter.
 * The router_probs outputs of cfg->route are not produced here (use moe_route).
 * Errors: INVALID_ARG, UNSUPPORTED, OVERLAP, WORKSPACE.
 * ------------------------------------------------------------------------------- */
int moe_ffn_forward(const moe_ffn_cfg* cfg, const void* hidden, const void* logits,
                    const float* correction_bias, const int32_t* expert_ids,
                    const void* w_gate_up, const void* w_down, const void* b_gate_up,
                    const void* b_down, const void* shared_w_gate_up,
                    const void* shared_w_down, void* out, void* shared_out,
                    float* topk_weights_out, int32_t* topk_ids_out, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_ffn_forward_noalloc - moe_ffn_forward with the library's own fixed scratch in
 * place of the caller's workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). It allocates nothing: no hipMalloc, hipFree or allocating library call.
 *
 * Arguments, results and errors are those of moe_ffn_forward without the workspace.
 * The scratch is one static device array of MOE_FFN_NOALLOC_SCRATCH_BYTES in the
 * library, one copy per GPU, held until the process ends; its address is resolved once
 * per device on the first call made with that device current. A cfg whose
 * moe_ffn_workspace_size exceeds that size returns MOE_ERR_WORKSPACE before anything is
 * enqueued (64 MiB covers, e.g., decode batches of the DeepSeek-V3 shapes, the
 * DeepSeek-V3 shapes up to about 250 tokens and the Qwen3 shapes up to about 860).
 * Every call on a GPU uses the same array, and nothing in it needs to start at zero
 * (each call writes every region before reading it): calls that overlap in time on one
 * GPU (different streams, or different host threads) race on it and must be
 * serialised by the caller.
 * ------------------------------------------------------------------------------- */
#define MOE_FFN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_ffn_forward_noalloc(const moe_ffn_cfg* cfg, const void* hidden, const void* logits,
                            const float* correction_bias, const int32_t* expert_ids,
                            const void* w_gate_up, const void* w_down, const void* b_gate_up,
                            const void* b_down, const void* shared_w_gate_up,
                            const void* shared_w_down, void* out, void* shared_out,
                            float* topk_weights_out, int32_t* topk_ids_out, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_grouped_gemm_fp8_masked - block-scaled FP8 GEMM per expert over a masked slab:
 * out[g, :m_g] = a[g, :m_g] b[g]^T.
 * [TO] MoEGroupedGemmFP8FwdOp (float8_e4m3fn operands, per-row x 128 and per-128x128
 * float32 scales applied once per 128-wide K block, bfloat16 result).
 *
 * a        [E, max_m, K] float8_e4m3fn (OCP E4M3) bytes; expert g's rows are g*max_m ...
 * a_scale  [E, max_m, K/128] float32: one scale per row and 128 columns of a.
 * b        [E, N, K] float8_e4m3fn bytes (rows contiguous in K).
 * b_scale  [E, N/128, K/128] float32: one scale per 128 x 128 block of b.
 * counts   [E] int32 on the device: valid rows m_g of expert g, read as max_m when larger
 *          and as 0 when negative; not checked (a check would synchronise).
 * out      [E, max_m, N] bfloat16: for m < m_g, out[g, m, n] = sum over 128-wide K blocks
 *          kb of (sum_{k in kb} a[g,m,k] b[g,n,k]) * a_scale[g,m,kb] * b_scale[g,n/128,kb],
 *          accumulated in float32 and rounded once (ties to even). Rows at or past m_g are
 *          left unwritten.
 * Limits: K and N multiples of 128, E <= 1024, max_m*K and N*K below 2^31 bytes (32-bit
 * offsets within one expert). max_m == 0 does nothing.
 * Errors: INVALID_ARG (null pointer, non-positive size), UNSUPPORTED (K or N not a multiple
 * of 128, limits), OVERLAP (out vs a, a_scale, b, b_scale, counts).
 * ------------------------------------------------------------------------------- */
int moe_grouped_gemm_fp8_masked(const void* a, const float* a_scale, const void* b,
                                const float* b_scale, const int32_t* counts, int64_t E,
                                int64_t max_m, int64_t K, int64_t N, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
