/*
 * moe_mi355x.h -- C ABI of the MoE FFN forward pass for AMD MI355X (gfx950).
 *
 * The layer is split into four calls, run in this order on one HIP stream:
 *
 *   moe_route          per-token router: softmax top-k gate, or the fused
 *                      sigmoid + selection-bias top-k with sink lanes
 *   moe_build_indices  per-expert CSR of the token->expert assignments,
 *                      token permutation (and optional row gather / fp8
 *                      quantisation of the activations)
 *   moe_grouped_ffn    grouped gate_up GEMM with the gated activation fused
 *                      into its epilogue, then the grouped down GEMM
 *                      (moe_grouped_ffn_fused: both legs in one launch)
 *   moe_combine        router-weighted sum of each token's expert rows
 *   moe_shared_indices buckets of the shared (sink-lane) experts: all tokens each
 *
 * Sources (web pages, cited by title and section):
 *   [StackedMoE]  MAX Python API, max.nn.moe.StackedMoE: constructor
 *                 parameters, "Weight tensor shapes", transposed-weight
 *                 properties.
 *   [GatedAct]    MAX Python API, max.nn.moe.GatedActivation: fused_activation,
 *                 alpha, limit, kernel_parameters().
 *   [SinkRouter]  MAX Mojo API, nn.moe sink_gate_router_kernel: description,
 *                 Parameters and Args.
 *   [NeMoExperts] NeMo AutoModel, nemo_automodel.components.moe.experts:
 *                 GroupedExperts.forward, _permute_tokens_for_grouped_mm,
 *                 _apply_bias, the activation functions.
 *   [MegaFFN]     MAX Mojo API, builtin_kernels mega_ffn: per-leg expert
 *                 scales, clamp constants.
 *
 * Conventions shared by every call:
 *   - Every pointer named "device" is device memory owned by the caller; the
 *     library never allocates, frees, retains a pointer after returning, or
 *     synchronises.  Host scalars are passed by value inside the args struct.
 *   - Tensors are dense row-major; only `logits` has a leading dimension.
 *     bf16 tensors are uint16 bit patterns; fp8 tensors are OCP e4m3fn codes.
 *   - Every launch is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).
 *   - Argument errors are detected on the host before anything is launched:
 *     the call returns MOE_ERR_INVALID_ARGUMENT (or MOE_ERR_UNSUPPORTED for a
 *     valid but unimplemented combination, MOE_ERR_WORKSPACE_TOO_SMALL for a
 *     short workspace) and moe_last_error_message() says why.  MOE_ERR_HIP
 *     means a launch failed.  Data-dependent cases are defined behaviour, not
 *     errors: empty experts, expert ids outside the local slice (dropped),
 *     masked tokens (zero output).
 *   - Device pointers must be 16-byte aligned; row lengths in bytes must be
 *     multiples of 16 (so hidden_dim and moe_dim are multiples of 8).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

/* Router kinds. */
enum { MOE_ROUTER_SOFTMAX_TOPK = 0, MOE_ROUTER_SIGMOID_SINK = 1 };
/* [GatedAct] fused_activation. */
enum { MOE_ACT_SILU = 0, MOE_ACT_SWIGLUOAI = 1, MOE_ACT_GELU_TANH = 2 };
/* [StackedMoE] gate_up_format. */
enum { MOE_GATE_UP_CONCATENATED = 0, MOE_GATE_UP_INTERLEAVED = 1 };
/* Element types.  MOE_DTYPE_FP8_E4M3_TOKENS is a moe_build_indices form of
   the fp8 operand: every token quantised once (1x128 blocks), not permuted;
   moe_grouped_ffn then gathers the rows it needs through sorted_token.
   MX block formats ([StackedMoE] mxfp8_activations: MXFP4 experts run W4A8;
   formats of the OCP Microscaling specification): 32 consecutive elements
   along the reduction dimension share one E8M0 scale byte (2^(s-127)).
   MOE_DTYPE_MXFP4_W4A8 is a moe_grouped_ffn operand type: E2M1 weights
   (two per byte, element 2i in the low nibble of byte i) times MXFP8
   activations (e4m3 codes); MOE_DTYPE_MXFP8 / MOE_DTYPE_MXFP8_TOKENS are the
   moe_build_indices forms of those activations (permuted rows, or one row
   per token in token order).  MOE_DTYPE_MXFP4_W4A16 is the other MXFP4
   operand type: the same weights times bf16 activations (and a bf16
   intermediate A). */
enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_FP8_E4M3_BLOCK128 = 1, MOE_DTYPE_FP32 = 2,
       MOE_DTYPE_FP8_E4M3_TOKENS = 3, MOE_DTYPE_MXFP4_W4A8 = 4, MOE_DTYPE_MXFP8 = 5,
       MOE_DTYPE_MXFP8_TOKENS = 6, MOE_DTYPE_MXFP4_W4A16 = 7 };
/* Weight layouts: [StackedMoE] stacked [E, in_features, out_features]
   ("Weight tensor shapes"), or its transposed view
   [E, out_features, in_features] (gate_up_proj_transposed /
   down_proj_transposed). */
enum { MOE_WEIGHT_IN_OUT = 0, MOE_WEIGHT_OUT_IN = 1 };

/* ------------------------------------------------------------------------
 * moe_route -- [SinkRouter] description and Args; [StackedMoE] gate_cls,
 * router_dtype, num_experts_per_token.
 *
 * SOFTMAX_TOPK: logits z = x . w_gate^T (bf16 inputs, fp32 accumulate, fp32
 *   logits), or `logits` given directly.  Selects the k largest logits,
 *   largest first, equal logits to the lower expert index.  With renormalize
 *   != 0 the weights are the softmax over the k selected logits; otherwise the
 *   full-softmax probabilities of the selected experts.  n_shared_experts
 *   must be 0 and expert_bias NULL.
 * SIGMOID_SINK: key_e = sigmoid(z_e) + expert_bias[e] (float32; sigmoid is
 *   evaluated as 1/(1+exp(-z)) with exp rounded once to float32 and a
 *   correctly rounded add and divide); the k largest keys are selected,
 *   largest first, ties to the lower index.  The weights are the softmax over
 *   log-sigmoid of [the selected raw logits | the s sink logits, columns
 *   E..E+s-1].  k + s must be a power of two no greater than 64 (one
 *   wavefront).  Input is `logits` only.
 * Both: every weight (expert and sink) is multiplied by
 *   route_scale * global_scale[0].
 *
 * Arguments (device unless marked host):
 *   router_kind, num_tokens T >= 0, n_routed_experts E in [1, 1024],
 *   n_experts_per_tok k in [1, min(E, 64)], n_shared_experts s >= 0   host
 *   hidden_dim H                       host, softmax x-form only: a multiple
 *                                      of 8 in [8, 4194304]
 *   x          bf16 [T, H]             softmax x-form (logits == NULL), E <= 128
 *   w_gate     bf16 [E, H], or float32 [E, H] with router_dtype FP32: the
 *              gate linear layer (out, in)
 *   router_dtype host, x-form: MOE_DTYPE_BF16 (0, the default: bf16 gate) or
 *              MOE_DTYPE_FP32 ([StackedMoE] router_dtype float32: the gate is
 *              built in float32 and x is cast to float32, which is exact);
 *              ignored when logits are given
 *   logits     fp32 [T, logits_ld], logits_ld >= E + s; routed experts then
 *              sink lanes; a wider row's tail is not read
 *   logits_out fp32 [T, E] or NULL     softmax x-form: the computed logits
 *   expert_bias fp32 [E] or NULL (0)   sigmoid: selection only
 *   global_scale fp32 [1] or NULL (1.0)
 *   route_scale                        host float
 *   renormalize                        host int, softmax only
 *   expert_indices int32 [T, k]        out
 *   expert_weights fp32 [T, k]         out
 *   sink_weights   fp32 [T, s]         out, required when s > 0
 * ---------------------------------------------------------------------- */
typedef struct moe_route_args {
  int32_t router_kind;
  int32_t num_tokens;
  int32_t n_routed_experts;
  int32_t n_experts_per_tok;
  int32_t n_shared_experts;
  int32_t hidden_dim;
  const void* x;
  const void* w_gate;
  const float* logits;
  int64_t logits_ld;
  float* logits_out;
  const float* expert_bias;
  const float* global_scale;
  float route_scale;
  int32_t renormalize;
  int32_t* expert_indices;
  float* expert_weights;
  float* sink_weights;
  int32_t router_dtype;
} moe_route_args_t;

moe_status_t moe_route(const moe_route_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_build_indices -- [SinkRouter] moe_create_indices (bucketing needs every
 * token's assignment, hence its own launches); [NeMoExperts]
 * _permute_tokens_for_grouped_mm (sorted token ids, routing weights, counts,
 * cumulative offsets; n_local_experts / experts_start_idx; token_mask).
 *
 * Assignment (t, j) has flat slot t*k + j.  It is kept when
 * experts_start_idx <= expert_indices[t, j] < experts_start_idx +
 * n_local_experts and token_mask[t] != 0 (or token_mask is NULL); other
 * assignments are dropped.  Kept slots are bucketed by local expert; inside a
 * bucket they keep ascending slot order.
 *
 *   num_tokens T, n_experts_per_tok k, experts_start_idx,
 *   n_local_experts L in [1, 1024]                            host
 *   expert_indices int32 [T, k]
 *   expert_weights fp32 [T, k] or NULL
 *   token_mask     uint8 [T] or NULL
 *   expert_offsets int32 [L + 1]   out: exclusive prefix of bucket sizes;
 *                                  expert_offsets[L] = kept rows
 *   sorted_token   int32 [T*k]     out: token of CSR row p (p < kept)
 *   row_of_slot    int32 [T*k]     out: CSR row of slot t*k+j, -1 if dropped
 *   sorted_weight  fp32 [T*k] or NULL  out: expert_weights of CSR row p
 *   x              bf16 [T, H] or NULL   optional row gather:
 *   hidden_dim H                   host
 *   xperm_dtype    host: MOE_DTYPE_BF16 (copy rows) or
 *                  MOE_DTYPE_FP8_E4M3_BLOCK128 (per-token 1x128 e4m3 with
 *                  scale amax/448, 1 when amax = 0; H % 128 == 0), or
 *                  MOE_DTYPE_FP8_E4M3_TOKENS (the same quantisation, one row
 *                  per token in token order: x_perm [T, H], x_perm_scale
 *                  [T, H/128]; the gather is left to moe_grouped_ffn), or
 *                  MOE_DTYPE_MXFP8 / MOE_DTYPE_MXFP8_TOKENS (H % 32 == 0):
 *                  per 32 columns, shared exponent X = floor(log2 amax) - 8
 *                  (at least -127; 0 for an all-zero block), codes
 *                  e4m3(v * 2^-X) rounded to nearest even and saturating at
 *                  448, scale byte X + 127; permuted rows or one per token
 *   x_perm         [T*k, H] bf16 or uint8 out, rows p < kept written
 *                  ([T, H] for the _TOKENS forms)
 *   x_perm_scale   out, fp8 and MX only: fp32 [rows, H/128] (fp8) or E8M0
 *                  bytes [rows, H/32] (MX)
 *   workspace      device scratch of moe_build_indices_workspace_bytes()
 * Rows p >= expert_offsets[L] of the outputs are left unwritten.
 * ---------------------------------------------------------------------- */
typedef struct moe_index_args {
  int32_t num_tokens;
  int32_t n_experts_per_tok;
  int32_t experts_start_idx;
  int32_t n_local_experts;
  const int32_t* expert_indices;
  const float* expert_weights;
  const uint8_t* token_mask;
  int32_t* expert_offsets;
  int32_t* sorted_token;
  int32_t* row_of_slot;
  float* sorted_weight;
  const void* x;
  int32_t hidden_dim;
  int32_t xperm_dtype;
  void* x_perm;
  void* x_perm_scale;
  void* workspace;
  int64_t workspace_bytes;
} moe_index_args_t;

moe_status_t moe_build_indices(const moe_index_args_t* args, void* stream);
int64_t moe_build_indices_workspace_bytes(int32_t num_tokens, int32_t n_experts_per_tok,
                                          int32_t n_local_experts);

/* ------------------------------------------------------------------------
 * moe_build_indices_noalloc -- moe_build_indices for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what
 * moe_build_indices computes, with the same kernels, but its scratch (the
 * per-block expert counts) is a static device array of the library, one
 * copy per GPU, held until the process ends; it calls no allocating routine.
 *
 *   args           as for moe_build_indices, except that workspace must be
 *                  NULL and workspace_bytes 0
 * Errors: as moe_build_indices; MOE_ERR_WORKSPACE_TOO_SMALL when the call
 * needs more than MOE_BUILD_INDICES_NOALLOC_MAX_SCRATCH bytes of scratch
 * (moe_build_indices_workspace_bytes of its sizes), e.g. n_local_experts
 * 1024 with more than 2^21 routed slots.
 * The scratch needs no initial contents and keeps the last call's.  All
 * calls on one GPU share it: calls that overlap on one GPU (on different
 * streams, or from different host threads) race and give wrong results.
 * The first call on each GPU looks up that GPU's copy of the array (with
 * the device current); later calls reuse the address.
 * ---------------------------------------------------------------------- */
#define MOE_BUILD_INDICES_NOALLOC_MAX_SCRATCH (16 * 1024 * 1024)
moe_status_t moe_build_indices_noalloc(const moe_index_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_ffn -- [StackedMoE] weight shapes, gate_up_format, has_bias,
 * quant_config (FP8 block scaling); [GatedAct] fused_activation, alpha, limit;
 * [NeMoExperts] _apply_bias; [MegaFFN] per-leg expert scales.
 *
 * For every local expert e and every CSR row p in
 * [expert_offsets[e], expert_offsets[e+1]):
 *   h      = gate_up_expert_scales[e] * (x_p . W_gu[e]) + b_gate_up[e]   (fp32)
 *   gate, up = split(h): CONCATENATED [gate | up], INTERLEAVED gate = even
 *            columns, up = odd columns (the bias follows the same order)
 *   A[p]   = activation(gate, up)            stored bf16 (fp8 path: e4m3 with
 *            a per-row 1x128 scale amax/448; MX path: MXFP8, quantised as
 *            moe_build_indices does)
 *   O[p]   = down_expert_scales[e] * (A[p] . W_d[e]) + b_down[e]
 * activation (GatedAct): SILU silu(gate)*up, with limit > 0 gate=min(gate,limit)
 *   and up=clamp(up,-limit,limit) first; SWIGLUOAI g*sigmoid(alpha*g)*(u+1)
 *   with the same clamps (limit 0 = no clamp); GELU_TANH gelu(gate)*up,
 *   tanh approximation.  alpha must be 0 unless SWIGLUOAI; limit must be 0
 *   for GELU_TANH and >= 0 otherwise.
 *
 *   max_rows       host: rows allocated in x_perm / act / expert_out
 *                  (>= expert_offsets[L]); the row count itself is read on
 *                  the device, no host synchronisation
 *   hidden_dim H, moe_dim D, n_local_experts L in [1, 1024]       host
 *   expert_offsets int32 [L + 1]
 *   operand_dtype  host: MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3_BLOCK128,
 *                  MOE_DTYPE_MXFP4_W4A8 or MOE_DTYPE_MXFP4_W4A16 (MX: H % 128
 *                  == 0 and D % 128 == 0; OUT_IN weights only, whose packed
 *                  E2M1 rows run along K; W4A16 takes bf16 x_perm / x like
 *                  the bf16 path and keeps A in bf16)
 *   x_perm         [max_rows, H] bf16 (or e4m3 codes) -- or NULL to gather
 *                  rows straight from x through sorted_token (bf16 only)
 *   x_perm_scale   fp32 [max_rows, H/128] (fp8), E8M0 bytes [max_rows, H/32] (MX)
 *   x, sorted_token  bf16 [T, H], int32 [max_rows]   gather form; for fp8
 *                  x holds the per-token codes [T, H] and x_perm_scale the
 *                  per-token scales [T, H/128] (MOE_DTYPE_FP8_E4M3_TOKENS);
 *                  for MX the MOE_DTYPE_MXFP8_TOKENS codes and scales.
 *                  Size limits (the GEMMs address operands with buffer
 *                  loads of a 2 GiB range): bf16 and fp8 address x_perm and
 *                  the activation buffer from each tile's first row, so only
 *                  x in the gather form and one expert's weights must be
 *                  under 2 GiB; MX and moe_grouped_ffn_fused also need
 *                  x_perm and the activation buffer under 2 GiB
 *   num_tokens     host: rows of x in the gather form (T), used for its size
 *                  bound; 0 = not given, then max_rows x hidden_dim is taken
 *                  as x's size
 *   w_gate_up      bf16/e4m3: layout IN_OUT [L, H, 2D] (the [StackedMoE]
 *                  "Weight tensor shapes" themselves) or OUT_IN [L, 2D, H]
 *                  (its transposed view).  bf16 reads either layout
 *                  (w_gate_up_layout and w_down_layout chosen independently;
 *                  IN_OUT gate_up weights need the concatenated format, an
 *                  interleaved IN_OUT gate_up is MOE_ERR_UNSUPPORTED); fp8
 *                  and MX take OUT_IN only
 *   w_gate_up_scale fp32 [L, H/128, 2D/128] (IN_OUT) or [L, 2D/128, H/128];
 *                  MX: packed E2M1 w_gate_up [L, 2D, H/2] with E8M0 scale
 *                  bytes [L, 2D, H/32]
 *   b_gate_up      bf16 [L, 2D] or NULL
 *   w_down         layout IN_OUT [L, D, H] or OUT_IN [L, H, D]
 *   w_down_scale   fp32 [L, D/128, H/128] (IN_OUT) or [L, H/128, D/128];
 *                  MX: packed w_down [L, H, D/2] with scale bytes [L, H, D/32]
 *   b_down         bf16 [L, H] or NULL
 *   gate_up_expert_scales, down_expert_scales  fp32 [L] or NULL (1.0)
 *   act_workspace  device scratch of moe_ffn_workspace_bytes(): A, and for
 *                  bf16 the down GEMM's split-K partial tiles and arrival
 *                  counters (the gate_up launch clears the counters, so the
 *                  buffer needs no initialisation; calls sharing one buffer
 *                  must not overlap)
 *   out_dtype      host: MOE_DTYPE_FP32 or MOE_DTYPE_BF16
 *   expert_out     O [max_rows, H]; rows p >= expert_offsets[L] unwritten
 *   timing_events  NULL, or an array of 3 hipEvent_t created by the caller:
 *                  recorded on `stream` before the gate_up GEMM, between the
 *                  two GEMMs and after the down GEMM (per-kernel timing)
 * The weight pointers already point at the first local expert.
 * ---------------------------------------------------------------------- */
typedef struct moe_ffn_args {
  int32_t max_rows;
  int32_t hidden_dim;
  int32_t moe_dim;
  int32_t n_local_experts;
  const int32_t* expert_offsets;
  int32_t operand_dtype;
  const void* x_perm;
  const void* x_perm_scale;
  const void* x;
  const int32_t* sorted_token;
  const void* w_gate_up;
  int32_t w_gate_up_layout;
  const void* w_gate_up_scale;
  const void* b_gate_up;
  int32_t gate_up_format;
  const void* w_down;
  int32_t w_down_layout;
  const void* w_down_scale;
  const void* b_down;
  int32_t activation;
  float alpha;
  float limit;
  const float* gate_up_expert_scales;
  const float* down_expert_scales;
  void* act_workspace;
  int64_t act_workspace_bytes;
  int32_t out_dtype;
  void* expert_out;
  void* const* timing_events;
  int32_t num_tokens;
} moe_ffn_args_t;

moe_status_t moe_grouped_ffn(const moe_ffn_args_t* args, void* stream);
int64_t moe_ffn_workspace_bytes(int32_t max_rows, int32_t moe_dim, int32_t operand_dtype);

/* ------------------------------------------------------------------------
 * moe_grouped_ffn_fused -- [MegaFFN] the single-launch form: the gate_up
 * GEMM with the gated activation (L1) and the down GEMM (L2) in one launch,
 * pipelined across workgroups with per-row-block arrival counters and no
 * per-launch memset.  It computes what moe_grouped_ffn computes (same
 * arguments and results: A in bf16, or MXFP8 for W4A8; O in fp32 or bf16),
 * for bf16 operands and for MXFP4 weights with MXFP8 activations (the page's
 * block-scaled form, whose L1 re-quantises A) or with bf16 activations; it
 * pays off where the two-launch form is bound by weight streaming and launch
 * gaps (small batches, decode).
 *
 * Differences from moe_grouped_ffn:
 *   operand_dtype  MOE_DTYPE_BF16, MOE_DTYPE_MXFP4_W4A8 or
 *                  MOE_DTYPE_MXFP4_W4A16; hidden_dim % 64 == 0 (MX: % 128),
 *                  moe_dim % 128 == 0.  W4A8 takes x_perm (or the per-token
 *                  x) with x_perm_scale, W4A16 bf16 x_perm or x without it,
 *                  as moe_grouped_ffn does; both compute bit for bit what
 *                  moe_grouped_ffn's MX paths compute unless the down items
 *                  are split along K (below)
 *   act_workspace  moe_ffn_fused_workspace_bytes(max_rows, hidden_dim,
 *                  moe_dim, n_local_experts) bytes (the same for both
 *                  operand types), holding the launch's control words (work
 *                  queue, exit count, error word, a parts-done counter per
 *                  split down tile, and an arrival counter per 32-row block,
 *                  the last at the very end of the act_workspace_bytes the
 *                  caller passes), A from byte offset 1280 (bf16 [max_rows,
 *                  D]; W4A8: e4m3 codes [max_rows, D], then from byte offset
 *                  1280 + round_up(max_rows * D, 256) the E8M0 scale bytes
 *                  [max_rows, D/32]), and the fp32 partial tiles of the down
 *                  items split along K.  The
 *                  control words must be ZERO before the first call
 *                  (allocate the workspace zero-filled); every call leaves
 *                  them zero again.  So one workspace serves any call with
 *                  the same hidden_dim, moe_dim and n_local_experts and a
 *                  max_rows no larger than it was sized for, PROVIDED every
 *                  call passes the same act_workspace_bytes (the end of the
 *                  buffer anchors the arrival counters).  The error word
 *                  (the int32 at byte offset 8) becomes nonzero -- and
 *                  stays so -- when a call's results are wrong: 1 if a wait
 *                  for an arrival counter timed out (a scheduling fault), 2
 *                  if expert_offsets[n_local_experts] exceeded max_rows
 *                  (that call then computes nothing).
 *                  Calls sharing one workspace must not overlap; the launch
 *                  occupies one workgroup per CU (MX: two).
 *   expert_out     as for moe_grouped_ffn.  When the launch has at most 256
 *                  down tiles (32-row blocks x ceil(hidden_dim / 256)) and
 *                  moe_dim is at least 3 x hidden_dim, each down tile is
 *                  summed from round(moe_dim / (2 hidden_dim)) (at most 8) fp32
 *                  partial products over slices of K, always in the same
 *                  order: the result is deterministic, and within rounding of
 *                  moe_grouped_ffn's.
 *   timing_events  the first event before the launch, the other two after it
 * ---------------------------------------------------------------------- */
moe_status_t moe_grouped_ffn_fused(const moe_ffn_args_t* args, void* stream);
int64_t moe_ffn_fused_workspace_bytes(int32_t max_rows, int32_t hidden_dim, int32_t moe_dim, int32_t n_local_experts);

/* ------------------------------------------------------------------------
 * moe_combine -- [NeMoExperts] GroupedExperts.forward returns [T, dim]; the
 * down bias is weighted by the routing probability (_apply_bias), which this
 * form gives since the bias is inside O.
 *
 *   y[t] = sum over j = 0..k-1 with row_of_slot[t, j] >= 0 of
 *          expert_weights[t, j] * O[row_of_slot[t, j]]
 * summed in fp32 in ascending j, rounded to bf16; masked tokens give zero
 * rows.  Deterministic (a gather, no atomics).
 *
 * With shared experts ([StackedMoE] has_shared_experts; [SinkRouter] the
 * sink lanes are gated shared experts) the shared rows are added after the
 * routed slots, in ascending i:
 *   y[t] += sum over i = 0..n_shared-1 of shared_weights[t, i] * O_sh[i*T + t]
 *
 *   num_tokens T, n_experts_per_tok k, hidden_dim H               host
 *   expert_out     O [*, H], fp32 or bf16 (out_dtype, host)
 *   row_of_slot    int32 [T, k]
 *   expert_weights fp32 [T, k] or NULL (weight 1: router weight applied first)
 *   token_mask     uint8 [T] or NULL
 *   y              bf16 [T, H] out
 *   n_shared       host: shared experts, 0 for none
 *   shared_out     O_sh [n_shared * T, H], same dtype as expert_out (row i*T + t:
 *                  shared expert i on token t, as moe_grouped_ffn writes it
 *                  with the buckets of moe_shared_indices)
 *   shared_weights fp32 [T, n_shared] (the router's sink_weights) or NULL
 *                  (weight 1: always-on shared experts)
 * ---------------------------------------------------------------------- */
typedef struct moe_combine_args {
  int32_t num_tokens;
  int32_t n_experts_per_tok;
  int32_t hidden_dim;
  const void* expert_out;
  int32_t out_dtype;
  const int32_t* row_of_slot;
  const float* expert_weights;
  const uint8_t* token_mask;
  void* y;
  int32_t n_shared;
  const void* shared_out;
  const float* shared_weights;
} moe_combine_args_t;

moe_status_t moe_combine(const moe_combine_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_shared_indices -- buckets for the shared experts ([StackedMoE]
 * has_shared_experts, shared_experts_dim; [SinkRouter] the n_shared_experts
 * sink lanes are gated shared experts): every token goes to every shared
 * expert, so shared expert i is the bucket of rows [i*T, (i+1)*T) in token
 * order.  With these, moe_grouped_ffn (in its gather form, x + sorted_token)
 * runs the shared experts' MLPs, and moe_combine adds them.
 *
 *   num_tokens T, n_shared                                        host
 *   expert_offsets int32 [n_shared + 1] out: i * T
 *   sorted_token   int32 [n_shared * T] out: row i*T + t holds t
 * Errors: T < 0, n_shared < 1 or n_shared * T >= 2^31 -> INVALID_ARGUMENT.
 * ---------------------------------------------------------------------- */
moe_status_t moe_shared_indices(int32_t num_tokens, int32_t n_shared, int32_t* expert_offsets,
                                int32_t* sorted_token, void* stream);

/* ========================================================================
 * Backward pass (routed experts, bf16 operands).  With dy = dL/dy the
 * gradients follow the forward by the chain rule:
 *   moe_combine_backward      dO[p] = w[t,j] dy[t],  dw[t,j] = <dy[t], O[p]>
 *   moe_grouped_ffn_backward  dX, dW_gu, dW_d, db_gu, db_d from dO
 *   moe_combine (weights NULL, out_dtype FP32) on dX then gives dx[t].
 * The per-expert bias gradients are [NeMoExperts]' deterministic
 * bias-gradient reduction (_DeterministicBiasRepeatInterleave.backward,
 * _reduce_bias_grad_triton): one compensated fp32 sum per expert over its
 * contiguous rows, no atomics.  Every result is deterministic.
 * ===================================================================== */

/* ------------------------------------------------------------------------
 * moe_combine_backward -- backward of moe_combine ([NeMoExperts]
 * GroupedExperts.forward; the down bias sits inside the weighting,
 * _apply_bias):
 *   d_expert_out[row_of_slot[t,j]] = expert_weights[t,j] * dy[t]   (bf16)
 *   d_expert_weights[t,j]          = <dy[t], expert_out[row]>      (fp32)
 * for the kept slots of valid tokens; dropped slots and masked tokens get
 * d_expert_weights 0 and write no row.
 *
 *   num_tokens T, n_experts_per_tok k, hidden_dim H (multiple of 8)  host
 *   dy              bf16 [T, H]
 *   expert_out      O [*, H], fp32 or bf16 (out_dtype); read only when
 *                   d_expert_weights is not NULL
 *   row_of_slot     int32 [T, k]; expert_weights fp32 [T, k] or NULL (1)
 *   token_mask      uint8 [T] or NULL
 *   d_expert_out    bf16 [rows, H] out (the rows row_of_slot names)
 *   d_expert_weights fp32 [T, k] out, or NULL
 * ---------------------------------------------------------------------- */
typedef struct moe_combine_backward_args {
  int32_t num_tokens;
  int32_t n_experts_per_tok;
  int32_t hidden_dim;
  const void* dy;
  const void* expert_out;
  int32_t out_dtype;
  const int32_t* row_of_slot;
  const float* expert_weights;
  const uint8_t* token_mask;
  void* d_expert_out;
  float* d_expert_weights;
} moe_combine_backward_args_t;

moe_status_t moe_combine_backward(const moe_combine_backward_args_t* args, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_ffn_backward -- backward of moe_grouped_ffn for bf16 operands
 * ([StackedMoE] weight shapes; [GatedAct] activations; [MegaFFN] per-leg
 * expert scales, held constant; [NeMoExperts] bias reduction).  For each CSR
 * row p of local expert e, with h = s_gu (x . W_gu^T) + b_gu recomputed:
 *   dA    = s_d * dO . W_d                (bf16, in the workspace)
 *   dH    = [dA * dact/dgate, dA * dact/dup] in W_gu's column order (bf16;
 *           a clamp passes the gradient inside its closed range)
 *   d_x_perm[p]     = s_gu * dH . W_gu                        fp32 [max_rows, H]
 *   d_w_gate_up[e]  = s_gu * sum_p dH[p]^T x[p]               fp32 [L, 2D, H]
 *   d_w_down[e]     = s_d  * sum_p dO[p]^T A[p]               fp32 [L, H, D]
 *   d_b_gate_up[e]  = sum_p dH[p],  d_b_down[e] = sum_p dO[p] fp32, or NULL
 * The weight gradients have the OUT_IN layout of the forward's weights;
 * experts with no rows get zero gradients.
 *
 *   max_rows, hidden_dim H, moe_dim D (both multiples of 64), n_local_experts L  host
 *   expert_offsets  int32 [L+1], as for moe_grouped_ffn
 *   x + sorted_token (gather) or x_perm, bf16, as for moe_grouped_ffn
 *   w_gate_up       bf16 [L, 2D, H]  the forward's OUT_IN view
 *   w_gate_up_stacked bf16 [L, H, 2D] and w_down_stacked bf16 [L, D, H]:
 *                   the same weights in [StackedMoE]'s stacked shapes (see
 *                   moe_transpose_bf16); the forward's w_down is not needed
 *   b_gate_up       bf16 [L, 2D] or NULL; gate_up_format, activation, alpha,
 *                   limit, gate_up_expert_scales, down_expert_scales as for
 *                   the forward
 *   d_expert_out    dO, bf16 [max_rows, H] (moe_combine_backward's output)
 *   workspace       moe_ffn_backward_workspace_bytes(max_rows, H, D, L)
 *                   bytes, no initial contents: dA, the recomputed A, dH and
 *                   transposed copies of dO, A, dH and the rows of x (every
 *                   expert's rows padded to a multiple of 64)
 *   timing_events   NULL or 8 caller-created hipEvent_t recorded: start,
 *                   after dA, after the recompute, after dX, after the
 *                   transposes, after dW_d, after dW_gu, at the end
 * Errors as for moe_grouped_ffn; each buffer that goes through the GEMM
 * loads (the row buffers, their transposed copies, one expert's weights)
 * must be under 2 GiB.
 * ---------------------------------------------------------------------- */
typedef struct moe_ffn_backward_args {
  int32_t max_rows;
  int32_t hidden_dim;
  int32_t moe_dim;
  int32_t n_local_experts;
  const int32_t* expert_offsets;
  const void* x;
  const int32_t* sorted_token;
  const void* x_perm;
  const void* w_gate_up;
  const void* w_gate_up_stacked;
  const void* w_down_stacked;
  const void* b_gate_up;
  int32_t gate_up_format;
  int32_t activation;
  float alpha;
  float limit;
  const float* gate_up_expert_scales;
  const float* down_expert_scales;
  const void* d_expert_out;
  float* d_x_perm;
  float* d_w_gate_up;
  float* d_w_down;
  float* d_b_gate_up;
  float* d_b_down;
  void* workspace;
  int64_t workspace_bytes;
  void* timing_events;
} moe_ffn_backward_args_t;

moe_status_t moe_grouped_ffn_backward(const moe_ffn_backward_args_t* args, void* stream);
int64_t moe_ffn_backward_workspace_bytes(int32_t max_rows, int32_t hidden_dim, int32_t moe_dim,
                                         int32_t n_local_experts);

/* ------------------------------------------------------------------------
 * moe_transpose_bf16 -- dst[b][c][r] = src[b][r][c] for a [batch, rows, cols]
 * bf16 tensor: converts between [StackedMoE]'s stacked weight shapes and the
 * transposed (OUT_IN) views.  rows and cols are multiples of 64; src and dst
 * are distinct, 16-byte aligned device buffers.
 * ---------------------------------------------------------------------- */
moe_status_t moe_transpose_bf16(const void* src, void* dst, int32_t batch, int32_t rows, int32_t cols,
                                void* stream);

/* ------------------------------------------------------------------------
 * Measured ceilings (diagnostics; not part of the layer).  The GEMMs and the
 * bandwidth kernels are reported against the datasheet peaks and against
 * what these two probes reach on the same chip under the same clocks.
 *
 * moe_probe_mfma -- runs workgroups x 8 waves, each issuing iters x 8
 * independent matrix instructions on register operands: kind 0 is
 * v_mfma_f32_32x32x16_bf16 (32768 flops each), kind 1 is
 * v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 operands with unit scales
 * (131072 flops each).  out (device, fp32, workgroups x 8 elements) receives
 * one sum per wave so that the loop is kept; its values have no meaning.
 * workgroups and iters are >= 1; kind is 0 or 1.
 *
 * moe_probe_stream_copy -- copies `bytes` bytes from src to dst (device,
 * 16-byte aligned, not overlapping) with 16-byte loads and stores; bytes is a
 * multiple of 16 (0 launches nothing).
 *
 * moe_probe_stream_read -- reads `bytes` bytes of src (device, 16-byte
 * aligned; bytes a multiple of 16, 0 launches nothing) with 16-byte loads and
 * writes nothing else: the ceiling of a read-dominated kernel, and a way to
 * evict the caches without leaving dirty lines behind.  It launches
 * min(ceil(bytes / 32 KiB), out_len / 4) work-groups of 4 waves; wave w
 * writes out[w] (device, uint32) = the XOR of the 32-bit words it read, so
 * that the XOR of the written entries is the XOR of all words of src.
 * Entries past the launched waves are left as they are.  out_len >= 4.
 * ---------------------------------------------------------------------- */
moe_status_t moe_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, float* out, void* stream);
moe_status_t moe_probe_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);
moe_status_t moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* out, int32_t out_len, void* stream);

/* Helpers. */
const char* moe_status_string(moe_status_t status);
/* Message of the last failed call on this host thread ("" if none). */
const char* moe_last_error_message(void);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
