// Internal launchers of the HIP kernels (host side).  The public C ABI in
// include/moe_mi355x.h validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

hipError_t launch_router_softmax_logits(const float* logits, int64_t ld, int T, int E, int k,
                                        float scale, const float* gs, int renorm, int32_t* idx,
                                        float* w, hipStream_t st);
// wg: bf16 [E, H], or float32 [E, H] when w32 (the float32 gate)
hipError_t launch_router_softmax_x(const uint16_t* x, const void* wg, int w32, int T, int H, int E,
                                   int k, float scale, const float* gs, int renorm,
                                   float* logits_out, int32_t* idx, float* w, hipStream_t st);
hipError_t launch_router_sigmoid_sink(const float* logits, int64_t ld, const float* bias, int T,
                                      int E, int k, int s, float scale, const float* gs,
                                      int32_t* idx, float* w, float* sink_w, hipStream_t st);

int64_t csr_num_blocks(int64_t R);
hipError_t launch_build_indices(const int32_t* idx, const float* w, const uint8_t* mask, int T,
                                int k, int start, int L, int32_t* offsets, int32_t* sorted_token,
                                int32_t* row_of_slot, float* sorted_weight, int32_t* ws,
                                hipStream_t st);
// kind: 0 bf16 copy, 1 e4m3 with 1x128 fp32 scales, 2 MXFP8 (e4m3 with one
// E8M0 scale byte per 32 columns)
hipError_t launch_permute(const uint16_t* x, const int32_t* sorted_token, const int32_t* n_rows,
                          int64_t max_rows, int H, int kind, void* xp, void* xs, hipStream_t st);

struct FfnBf16Params {
  const int32_t* offsets;
  int L, H, D, max_rows;
  const uint16_t* x_perm;        // or nullptr: gather from x through sorted_token
  const uint16_t* x;
  const int32_t* sorted_token;
  const uint16_t* w_gate_up;     // OUT_IN [L, 2D, H], or IN_OUT [L, H, 2D] (gu_in_out)
  const uint16_t* b_gate_up;
  const uint16_t* w_down;        // OUT_IN [L, H, D], or IN_OUT [L, D, H] (d_in_out)
  const uint16_t* b_down;
  const float* gate_up_scales;
  const float* down_scales;
  int fmt, act_kind;
  int gu_in_out, d_in_out;       // the stacked layouts (gate_up: concatenated format only)
  float alpha, limit;
  uint16_t* act;                 // [max_rows, D]
  void* out;                     // [max_rows, H]
  int out_bf16;
  hipEvent_t const* events;      // optional: before gate_up, between, after down
  // split-K tail round of the down GEMM (all three null/0: off)
  int32_t* split_counters;       // SPLIT_COUNTERS ints
  float* split_partial;          // split_slots x SPLIT_TILE_FLOATS floats
  int split_slots;
};
constexpr int SPLIT_COUNTERS = 256;
constexpr int64_t SPLIT_TILE_FLOATS = 256 * 256;
// partial-tile slots the workspace provides for max_rows rows
inline int split_slots_for(int64_t max_rows) {
  const int64_t s = max_rows / 16;
  return (int)(s < SPLIT_COUNTERS ? s : SPLIT_COUNTERS);
}
hipError_t launch_ffn_bf16(const FfnBf16Params& p, hipStream_t st);

// One GEMM of the backward pass on the bf16 grouped-GEMM kernel:
//   rows   O[p] = escale[e] * A[p] . W[e]^T over the CSR rows (bf16 or fp32 out)
//   gate_up recompute: A[p] = act(h), dH[p] = dA[p] * d act (h = escale * x . W^T + bias)
//   wgrad  C[e] = escale[e] * A_e . B_e^T, K = the expert's padded segment
struct BwdGemm {
  const int32_t* offsets;
  int L, K, N, max_rows;
  const uint16_t* A;             // [rows, K] (nullptr for the gate_up recompute: gather X)
  const uint16_t* X;
  const int32_t* sorted_token;
  const uint16_t* W;             // [L][N, K] (wgrad: the B operand [N, Kpad], shared)
  int64_t w_estride, lda, ldb;
  const uint16_t* bias;          // gate_up recompute only: [L, 2N] or nullptr
  const float* escale;
  int act_kind, fmt;
  float alpha, limit;
  void* out;
  int64_t ldo;
  int out_bf16;
  const uint16_t* din;           // gate_up recompute: dA [rows, N]
  int64_t ld_din;
  void* out2;                    // gate_up recompute: dH [rows, 2N]
  int64_t ldo2;
  const int32_t* seg;            // wgrad: [L+1] padded segments
  int M;                         // wgrad: rows of the A operand
  int64_t out_estride;           // wgrad: elements between experts' outputs
};
// The backward of the routed-expert FFN (bf16 operands).
struct FfnBwdParams {
  const int32_t* offsets;
  int L, H, D, max_rows;
  const uint16_t* x;                  // bf16 [T, H] gathered through sorted_token, or
  const int32_t* sorted_token;
  const uint16_t* x_perm;             // bf16 [max_rows, H]
  const uint16_t* w_gate_up;          // OUT_IN [L, 2D, H]
  const uint16_t* w_gate_up_stacked;  // [L, H, 2D]
  const uint16_t* w_down_stacked;     // [L, D, H]
  const uint16_t* b_gate_up;
  int fmt, act_kind;
  float alpha, limit;
  const float* gate_up_scales;
  const float* down_scales;
  const uint16_t* d_out;              // dO bf16 [max_rows, H]
  float* d_x_perm;                    // [max_rows, H]
  float* d_w_gate_up;                 // [L, 2D, H]
  float* d_w_down;                    // [L, H, D]
  float* d_b_gate_up;                 // [L, 2D] or nullptr
  float* d_b_down;                    // [L, H] or nullptr
  void* ws;
  hipEvent_t const* events;           // optional, 8
};
// workspace byte offsets: segments, dA, A, dH, then the transposed operands
// dO^T [H, rp], A^T [D, rp], dH^T [2D, rp], x^T [H, rp]
struct FfnBwdLayout {
  int64_t rp;  // padded row width of the transposed operands
  int64_t seg_off, dA_off, A_off, dH_off, dOt_off, At_off, dHt_off, xt_off, bytes;
};
FfnBwdLayout ffn_bwd_layout(int64_t max_rows, int H, int D, int L);
hipError_t launch_ffn_backward(const FfnBwdParams& p, hipStream_t st);

struct CombineBwdParams {
  int T, k, H;
  const uint16_t* dy;
  const void* O;
  int o_bf16;
  const int32_t* row_of_slot;
  const float* w;
  const uint8_t* mask;
  uint16_t* dO;
  float* dw;
};
hipError_t launch_combine_backward(const CombineBwdParams& p, hipStream_t st);
hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int batch, int64_t rows, int64_t cols,
                                 hipStream_t st);

hipError_t launch_bwd_rows_gemm(const BwdGemm& b, hipStream_t st);
hipError_t launch_bwd_gate_up_gemm(const BwdGemm& b, hipStream_t st);
hipError_t launch_wgrad_gemm(const BwdGemm& b, hipStream_t st);

struct FfnFp8Params {
  const int32_t* offsets;
  int L, H, D, max_rows;
  const uint8_t* x_perm;         // e4m3 codes [max_rows, H], or per token [T, H] with sorted_token
  const float* x_scale;          // [max_rows, H/128] or [T, H/128]
  const int32_t* sorted_token;   // nullptr: rows already permuted
  const uint8_t* w_gate_up;      // OUT_IN [L, 2D, H]
  const float* w_gate_up_scale;  // [L, 2D/128, H/128]
  const uint8_t* w_down;         // OUT_IN [L, H, D]
  const float* w_down_scale;     // [L, H/128, D/128]
  const float* gate_up_scales;
  const float* down_scales;
  const uint16_t* b_gate_up;     // bf16 [L, 2D] (column order of fmt) or nullptr
  const uint16_t* b_down;        // bf16 [L, H] or nullptr
  int fmt;                       // 0 concatenated, 1 interleaved gate_up columns
  int act_kind;
  float alpha, limit;
  uint8_t* act;                  // e4m3 codes [max_rows, D]
  float* act_scale;              // [max_rows, D/128]
  void* out;                     // [max_rows, H] bf16 or fp32
  int out_bf16;
  hipEvent_t const* events;
};
hipError_t launch_ffn_fp8(const FfnFp8Params& p, hipStream_t st);

// MXFP4 weights x MXFP8 activations (W4A8); every scale is an E8M0 byte per
// 32 elements along K.
struct FfnMxParams {
  const int32_t* offsets;
  int L, H, D, max_rows;
  int fmt;                       // gate_up format
  const uint8_t* x_perm;         // e4m3 codes [max_rows, H], or per token [T, H] with sorted_token
  const uint8_t* x_scale;        // [max_rows, H/32] or [T, H/32]
  const int32_t* sorted_token;   // nullptr: rows already permuted
  const uint8_t* w_gate_up;      // packed e2m1, OUT_IN [L, 2D, H/2]
  const uint8_t* w_gate_up_scale;  // [L, 2D, H/32]
  const uint8_t* w_down;         // packed e2m1, OUT_IN [L, H, D/2]
  const uint8_t* w_down_scale;   // [L, H, D/32]
  const uint16_t* b_gate_up;     // bf16 [L, 2D] or nullptr
  const uint16_t* b_down;        // bf16 [L, H] or nullptr
  const float* gate_up_scales;
  const float* down_scales;
  int act_kind;
  float alpha, limit;
  uint8_t* act;                  // e4m3 codes [max_rows, D]
  uint8_t* act_scale;            // E8M0 [max_rows, D/32]
  void* out;                     // [max_rows, H] bf16 or fp32
  int out_bf16;
  hipEvent_t const* events;
};
hipError_t launch_ffn_mx(const FfnMxParams& p, hipStream_t st);
// MXFP4 weights x bf16 activations (W4A16): x_perm / act are bf16, no
// activation scales; the same weight fields.
hipError_t launch_ffn_w4a16(const FfnMxParams& p, hipStream_t st);

// Single-launch L1+L2 FFN for small batches (bf16, W4A8 or W4A16 operands): control words
// (queue, exit count, error, one arrival counter per 32-row block) at the
// start of the workspace, then A; zero when allocated, zero again after
// every launch.
// Workspace of the single-launch FFN, byte offsets from its start:
//   [0, act_off)          queue head, exit count, error word, unused, then one
//                         parts-done counter per split L2 tile
//   [act_off, part_off)   A: bf16 [max_rows, D], or (MX) e4m3 codes
//                         [max_rows, D] and, from act_scale_off, the E8M0
//                         scale bytes [max_rows, D/32]
//   [part_off, ...)       tiles_cap * S fp32 partial tiles of 32 x 256
//   the last row_blocks int32 of the caller's buffer: arrival counters
// The counters are zero between launches; the layout of a smaller max_rows
// with the same H, D, L lies inside that of a larger one.
struct FusedLayout {
  int64_t row_blocks;   // bound on the 32-row blocks of the launch
  int S;                // K parts of a split L2 tile (1: no split)
  int tiles_cap;        // L2 tiles the partial slots hold
  int64_t act_off, act_scale_off, part_off, bytes;
};
FusedLayout fused_layout(int64_t max_rows, int H, int D, int L);
// p.act is ignored: A lives in the workspace at act_off
hipError_t launch_ffn_fused(const FfnBf16Params& p, void* ws, int64_t ws_bytes, hipStream_t st);
// The same schedule for MXFP4 weights x MXFP8 activations (p.act and
// p.act_scale are ignored: A lives in the workspace).
hipError_t launch_ffn_fused_mx(const FfnMxParams& p, void* ws, int64_t ws_bytes, hipStream_t st);
// ... and for MXFP4 weights x bf16 activations (p.x_perm: bf16 rows or, with
// sorted_token, bf16 tokens; A bf16 in the workspace).
hipError_t launch_ffn_fused_w4a16(const FfnMxParams& p, void* ws, int64_t ws_bytes, hipStream_t st);

hipError_t launch_combine(const void* O, int o_bf16, const int32_t* row_of_slot, const float* w,
                          const uint8_t* mask, int T, int k, int H, uint16_t* y, int n_shared,
                          const void* O_shared, const float* w_shared, hipStream_t st);
hipError_t launch_shared_indices(int T, int n_shared, int32_t* offsets, int32_t* sorted_token,
                                 hipStream_t st);

}  // namespace moe
