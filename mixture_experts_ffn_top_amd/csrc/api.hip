// C ABI of the MoE FFN library: host-side argument validation (before any
// HIP call) and kernel dispatch.  See include/moe_mi355x.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "kernels.h"
#include "probe.h"

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

#define REQUIRE(cond, ...)                                                                         \
  do {                                                                                             \
    if (!(cond)) return fail(MOE_ERR_INVALID_ARGUMENT, __VA_ARGS__);                               \
  } while (0)

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error_message(void) { return g_err; }

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

// ---------------------------------------------------------------- route
moe_status_t moe_route(const moe_route_args_t* a, void* stream) {
  REQUIRE(a != nullptr, "moe_route: args is NULL");
  const int T = a->num_tokens, E = a->n_routed_experts, k = a->n_experts_per_tok,
            s = a->n_shared_experts;
  REQUIRE(T >= 0, "moe_route: num_tokens must be >= 0 (got %d)", T);
  REQUIRE(E >= 1 && E <= 1024, "moe_route: n_routed_experts must be in [1, 1024] (got %d)", E);
  REQUIRE(k >= 1 && k <= E && k <= 64,
          "moe_route: n_experts_per_tok must be in [1, min(n_routed_experts, 64)] (got %d)", k);
  REQUIRE(s >= 0, "moe_route: n_shared_experts must be >= 0 (got %d)", s);
  REQUIRE(std::isfinite(a->route_scale), "moe_route: route_scale must be finite");
  REQUIRE(T == 0 || (a->expert_indices && a->expert_weights),
          "moe_route: expert_indices and expert_weights are required");
  hipStream_t st = (hipStream_t)stream;
  if (a->router_kind == MOE_ROUTER_SOFTMAX_TOPK) {
    REQUIRE(s == 0, "moe_route: the softmax gate has no sink lanes (n_shared_experts must be 0)");
    REQUIRE(a->expert_bias == nullptr, "moe_route: expert_bias is only for the sigmoid router");
    const bool xform = a->logits == nullptr;
    if (xform) {
      REQUIRE(a->x != nullptr && a->w_gate != nullptr,
              "moe_route: softmax router needs logits, or x and w_gate");
      REQUIRE(E <= 128, "moe_route: the fused gate GEMM supports n_routed_experts <= 128 (got %d)", E);
      REQUIRE(a->hidden_dim >= 8 && a->hidden_dim % 8 == 0 && a->hidden_dim <= (1 << 22),
              "moe_route: hidden_dim must be a multiple of 8 in [8, 4194304] (got %d)", a->hidden_dim);
      REQUIRE(aligned16(a->x) && aligned16(a->w_gate), "moe_route: x and w_gate must be 16-byte aligned");
      REQUIRE(a->router_dtype == MOE_DTYPE_BF16 || a->router_dtype == MOE_DTYPE_FP32,
              "moe_route: router_dtype must be BF16 or FP32 (got %d)", a->router_dtype);
      return hip_status(moe::launch_router_softmax_x(
                            (const uint16_t*)a->x, a->w_gate, a->router_dtype == MOE_DTYPE_FP32, T,
                            a->hidden_dim, E, k,
                            a->route_scale, a->global_scale, a->renormalize, a->logits_out,
                            a->expert_indices, a->expert_weights, st),
                        "moe_route");
    }
    REQUIRE(a->x == nullptr, "moe_route: pass either logits or x/w_gate, not both");
    REQUIRE(a->logits_ld >= E, "moe_route: logits_ld must be >= n_routed_experts");
    return hip_status(moe::launch_router_softmax_logits(a->logits, a->logits_ld, T, E, k,
                                                        a->route_scale, a->global_scale,
                                                        a->renormalize, a->expert_indices,
                                                        a->expert_weights, st),
                      "moe_route");
  }
  if (a->router_kind == MOE_ROUTER_SIGMOID_SINK) {
    REQUIRE(a->logits != nullptr && a->x == nullptr, "moe_route: the sigmoid router takes logits");
    REQUIRE(is_pow2(k + s) && k + s <= 64,
            "moe_route: n_experts_per_tok + n_shared_experts must be a power of two <= 64 (got %d)",
            k + s);
    REQUIRE(a->logits_ld >= (int64_t)E + s,
            "moe_route: logits_ld must be >= n_routed_experts + n_shared_experts");
    REQUIRE(s == 0 || T == 0 || a->sink_weights != nullptr,
            "moe_route: sink_weights is required when n_shared_experts > 0");
    return hip_status(moe::launch_router_sigmoid_sink(a->logits, a->logits_ld, a->expert_bias, T, E,
                                                      k, s, a->route_scale, a->global_scale,
                                                      a->expert_indices, a->expert_weights,
                                                      a->sink_weights, st),
                      "moe_route");
  }
  return fail(MOE_ERR_INVALID_ARGUMENT, "moe_route: unknown router_kind %d", a->router_kind);
}

// ---------------------------------------------------------------- build indices
int64_t moe_build_indices_workspace_bytes(int32_t T, int32_t k, int32_t L) {
  if (T < 0 || k < 1 || L < 1) return 0;
  const int64_t nblk = moe::csr_num_blocks((int64_t)T * k);
  return round_up(nblk * L * (int64_t)sizeof(int32_t), 256);
}

}  // extern "C"

namespace {

// Checks every argument of moe_build_indices except the workspace, then
// launches on `workspace` (at least moe_build_indices_workspace_bytes).
moe_status_t build_indices_checked(const moe_index_args_t* a, int32_t* workspace, void* stream, const char* fn) {
  const int T = a->num_tokens, k = a->n_experts_per_tok, L = a->n_local_experts;
  const bool permute = a->x != nullptr;
  if (permute) {
    const int H = a->hidden_dim;
    REQUIRE(H >= 8 && H % 8 == 0, "%s: hidden_dim must be a positive multiple of 8 (got %d)", fn, H);
    REQUIRE(a->x_perm != nullptr, "%s: x_perm is required with x", fn);
    REQUIRE(aligned16(a->x) && aligned16(a->x_perm), "%s: x and x_perm must be 16-byte aligned", fn);
    if (a->xperm_dtype == MOE_DTYPE_FP8_E4M3_BLOCK128 || a->xperm_dtype == MOE_DTYPE_FP8_E4M3_TOKENS) {
      REQUIRE(H % 128 == 0, "%s: fp8 quantisation needs hidden_dim %% 128 == 0 (got %d)", fn, H);
      REQUIRE(a->x_perm_scale != nullptr, "%s: x_perm_scale is required for fp8", fn);
    } else if (a->xperm_dtype == MOE_DTYPE_MXFP8 || a->xperm_dtype == MOE_DTYPE_MXFP8_TOKENS) {
      REQUIRE(H % 32 == 0, "%s: MXFP8 quantisation needs hidden_dim %% 32 == 0 (got %d)", fn, H);
      REQUIRE(a->x_perm_scale != nullptr, "%s: x_perm_scale is required for MXFP8", fn);
    } else {
      REQUIRE(a->xperm_dtype == MOE_DTYPE_BF16,
              "%s: xperm_dtype must be BF16, FP8_E4M3_BLOCK128, FP8_E4M3_TOKENS, MXFP8 or MXFP8_TOKENS", fn);
    }
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = moe::launch_build_indices(a->expert_indices, a->expert_weights, a->token_mask, T, k,
                                           a->experts_start_idx, L, a->expert_offsets,
                                           a->sorted_token, a->row_of_slot, a->sorted_weight, workspace, st);
  if (e != hipSuccess) return hip_status(e, fn);
  if (permute) {
    const int dt = a->xperm_dtype;
    const bool tokens = dt == MOE_DTYPE_FP8_E4M3_TOKENS || dt == MOE_DTYPE_MXFP8_TOKENS;
    const int kind = dt == MOE_DTYPE_BF16 ? 0 : (dt == MOE_DTYPE_MXFP8 || dt == MOE_DTYPE_MXFP8_TOKENS) ? 2 : 1;
    e = moe::launch_permute((const uint16_t*)a->x, tokens ? nullptr : a->sorted_token,
                            a->expert_offsets + L, tokens ? (int64_t)T : (int64_t)T * k,
                            a->hidden_dim, kind, a->x_perm, a->x_perm_scale, st);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

moe_status_t build_indices_common_args(const moe_index_args_t* a, const char* fn) {
  REQUIRE(a != nullptr, "%s: args is NULL", fn);
  const int T = a->num_tokens, k = a->n_experts_per_tok, L = a->n_local_experts;
  REQUIRE(T >= 0, "%s: num_tokens must be >= 0 (got %d)", fn, T);
  REQUIRE(k >= 1 && k <= 1024, "%s: n_experts_per_tok must be in [1, 1024] (got %d)", fn, k);
  REQUIRE(L >= 1 && L <= 1024, "%s: n_local_experts must be in [1, 1024] (got %d)", fn, L);
  REQUIRE((int64_t)T * k < (int64_t)1 << 31, "%s: num_tokens * n_experts_per_tok must be < 2^31", fn);
  REQUIRE(a->expert_offsets != nullptr, "%s: expert_offsets is required", fn);
  REQUIRE(T == 0 || (a->expert_indices && a->sorted_token && a->row_of_slot),
          "%s: expert_indices, sorted_token and row_of_slot are required", fn);
  return MOE_OK;
}

// ---- the allocation-free form: its scratch (the per-block expert counts)
// is a file-scope device array, one copy per GPU the library runs on, held
// until the process ends.  Host code never passes the array's name (a host
// stand-in) to a kernel: the device address of each GPU's copy is looked up
// once, with that device current, and used from then on.
constexpr int64_t kNoallocScratchBytes = (int64_t)MOE_BUILD_INDICES_NOALLOC_MAX_SCRATCH;
static __device__ __align__(256) int32_t scratch[kNoallocScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (NULL with the
// message set on failure).
int32_t* noalloc_scratch(const char* fn, moe_status_t* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = hip_status(e, fn);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = fail(MOE_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices this form serves", fn, dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *st = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, fn);
      return nullptr;
    }
    g_scratch_ptr[dev] = (int32_t*)p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status_t moe_build_indices(const moe_index_args_t* a, void* stream) {
  const char* fn = "moe_build_indices";
  const moe_status_t c = build_indices_common_args(a, fn);
  if (c != MOE_OK) return c;
  const int64_t need = moe_build_indices_workspace_bytes(a->num_tokens, a->n_experts_per_tok, a->n_local_experts);
  if (a->workspace_bytes < need || (need > 0 && a->workspace == nullptr))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_build_indices: workspace needs %lld bytes (got %lld)",
                (long long)need, (long long)a->workspace_bytes);
  REQUIRE(aligned16(a->workspace), "moe_build_indices: workspace must be 16-byte aligned");
  return build_indices_checked(a, (int32_t*)a->workspace, stream, fn);
}

moe_status_t moe_build_indices_noalloc(const moe_index_args_t* a, void* stream) {
  const char* fn = "moe_build_indices_noalloc";
  const moe_status_t c = build_indices_common_args(a, fn);
  if (c != MOE_OK) return c;
  REQUIRE(a->workspace == nullptr && a->workspace_bytes == 0,
          "moe_build_indices_noalloc: workspace must be NULL and workspace_bytes 0 (the scratch is the library's)");
  const int64_t need = moe_build_indices_workspace_bytes(a->num_tokens, a->n_experts_per_tok, a->n_local_experts);
  if (need > kNoallocScratchBytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                "moe_build_indices_noalloc: this call needs %lld bytes of scratch; the static scratch holds %lld "
                "(use moe_build_indices with a workspace)", (long long)need, (long long)kNoallocScratchBytes);
  moe_status_t st = MOE_OK;
  int32_t* ws = noalloc_scratch(fn, &st);
  if (ws == nullptr) return st;
  return build_indices_checked(a, ws, stream, fn);
}

// ---------------------------------------------------------------- grouped FFN
}  // extern "C"

namespace {

// The gather form reads x [T, H] by token with 32-bit offsets from one base:
// x must be under 2 GiB.  T is num_tokens when given; otherwise every one of
// the max_rows rows is taken as a possible token (the bound before
// num_tokens was part of the arguments).
bool gather_rows_fit(const moe_ffn_args_t* a, int64_t elem_bytes) {
  const int64_t rows = a->num_tokens > 0 ? a->num_tokens : a->max_rows;
  return rows * a->hidden_dim * elem_bytes < ((int64_t)1 << 31);
}

const char* gather_bound_msg(const moe_ffn_args_t* a) {
  return a->num_tokens > 0 ? "x (num_tokens x hidden_dim) must be under 2 GiB in the gather form"
                           : "x must be under 2 GiB in the gather form; without num_tokens, max_rows x hidden_dim "
                             "is taken as its size (pass num_tokens)";
}

}  // namespace

extern "C" {

int64_t moe_ffn_workspace_bytes(int32_t max_rows, int32_t D, int32_t dtype) {
  if (max_rows < 0 || D < 1) return 0;
  if (dtype == MOE_DTYPE_FP8_E4M3_BLOCK128)
    return round_up((int64_t)max_rows * D, 256) + round_up((int64_t)max_rows * ((D + 127) / 128) * 4, 256);
  if (dtype == MOE_DTYPE_MXFP4_W4A8)  // A codes, then one E8M0 byte per 32 columns
    return round_up((int64_t)max_rows * D, 256) + round_up((int64_t)max_rows * ((D + 31) / 32), 256);
  if (dtype == MOE_DTYPE_MXFP4_W4A16)  // A in bf16
    return round_up((int64_t)max_rows * D * 2, 256);
  // bf16: A, then the down GEMM's split-K counters and partial tiles
  return round_up((int64_t)max_rows * D * 2, 256) + moe::SPLIT_COUNTERS * 4 +
         (int64_t)moe::split_slots_for(max_rows) * moe::SPLIT_TILE_FLOATS * 4;
}

moe_status_t moe_grouped_ffn(const moe_ffn_args_t* a, void* stream) {
  REQUIRE(a != nullptr, "moe_grouped_ffn: args is NULL");
  const int R = a->max_rows, H = a->hidden_dim, D = a->moe_dim, L = a->n_local_experts;
  REQUIRE(R >= 0, "moe_grouped_ffn: max_rows must be >= 0 (got %d)", R);
  REQUIRE(H >= 8 && H % 8 == 0, "moe_grouped_ffn: hidden_dim must be a positive multiple of 8 (got %d)", H);
  REQUIRE(D >= 8 && D % 8 == 0, "moe_grouped_ffn: moe_dim must be a positive multiple of 8 (got %d)", D);
  REQUIRE(L >= 1 && L <= 1024, "moe_grouped_ffn: n_local_experts must be in [1, 1024] (got %d)", L);
  REQUIRE(a->expert_offsets != nullptr, "moe_grouped_ffn: expert_offsets is required");
  REQUIRE(a->operand_dtype == MOE_DTYPE_BF16 || a->operand_dtype == MOE_DTYPE_FP8_E4M3_BLOCK128 ||
              a->operand_dtype == MOE_DTYPE_MXFP4_W4A8 || a->operand_dtype == MOE_DTYPE_MXFP4_W4A16,
          "moe_grouped_ffn: operand_dtype must be BF16, FP8_E4M3_BLOCK128, MXFP4_W4A8 or MXFP4_W4A16");
  REQUIRE(a->activation == MOE_ACT_SILU || a->activation == MOE_ACT_SWIGLUOAI ||
              a->activation == MOE_ACT_GELU_TANH,
          "moe_grouped_ffn: unknown activation %d", a->activation);
  REQUIRE(std::isfinite(a->alpha) && std::isfinite(a->limit), "moe_grouped_ffn: alpha and limit must be finite");
  REQUIRE(a->activation == MOE_ACT_SWIGLUOAI || a->alpha == 0.0f,
          "moe_grouped_ffn: alpha is the sigmoid scale of swigluoai and must be 0 for the other activations");
  REQUIRE(a->activation != MOE_ACT_GELU_TANH || a->limit == 0.0f,
          "moe_grouped_ffn: limit must be 0 for gelu_tanh");
  REQUIRE(a->limit >= 0.0f, "moe_grouped_ffn: limit must be >= 0");
  REQUIRE(a->gate_up_format == MOE_GATE_UP_CONCATENATED || a->gate_up_format == MOE_GATE_UP_INTERLEAVED,
          "moe_grouped_ffn: unknown gate_up_format %d", a->gate_up_format);
  REQUIRE(a->out_dtype == MOE_DTYPE_FP32 || a->out_dtype == MOE_DTYPE_BF16,
          "moe_grouped_ffn: out_dtype must be FP32 or BF16");
  REQUIRE(a->w_gate_up_layout == MOE_WEIGHT_IN_OUT || a->w_gate_up_layout == MOE_WEIGHT_OUT_IN,
          "moe_grouped_ffn: unknown w_gate_up_layout");
  REQUIRE(a->w_down_layout == MOE_WEIGHT_IN_OUT || a->w_down_layout == MOE_WEIGHT_OUT_IN,
          "moe_grouped_ffn: unknown w_down_layout");
  REQUIRE(a->w_gate_up && a->w_down, "moe_grouped_ffn: w_gate_up and w_down are required");
  REQUIRE(R == 0 || a->expert_out != nullptr, "moe_grouped_ffn: expert_out is required");
  const bool gather = a->x_perm == nullptr;
  if (gather) {
    REQUIRE(R == 0 || (a->x != nullptr && a->sorted_token != nullptr),
            "moe_grouped_ffn: pass x_perm, or x and sorted_token to gather rows");
  } else {
    REQUIRE(a->x == nullptr, "moe_grouped_ffn: pass either x_perm or x/sorted_token, not both");
  }
  REQUIRE(aligned16(a->x_perm) && aligned16(a->x) && aligned16(a->w_gate_up) && aligned16(a->w_down) &&
              aligned16(a->act_workspace) && aligned16(a->expert_out),
          "moe_grouped_ffn: tensors must be 16-byte aligned");
  const int64_t need = moe_ffn_workspace_bytes(R, D, a->operand_dtype);
  if (a->act_workspace_bytes < need || (need > 0 && a->act_workspace == nullptr))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_grouped_ffn: act_workspace needs %lld bytes (got %lld)",
                (long long)need, (long long)a->act_workspace_bytes);
  if (a->operand_dtype == MOE_DTYPE_MXFP4_W4A8 || a->operand_dtype == MOE_DTYPE_MXFP4_W4A16) {
    const bool a16 = a->operand_dtype == MOE_DTYPE_MXFP4_W4A16;
    REQUIRE(H % 128 == 0 && D % 128 == 0, "moe_grouped_ffn: MX needs hidden_dim and moe_dim multiples of 128");
    REQUIRE(a16 || (a->x_perm_scale != nullptr && (a->x_perm != nullptr || a->x != nullptr)),
            "moe_grouped_ffn: MX takes x_perm (or per-token x) and x_perm_scale, quantised by moe_build_indices");
    REQUIRE(!a16 || a->x_perm_scale == nullptr, "moe_grouped_ffn: W4A16 takes bf16 activations, no x_perm_scale");
    REQUIRE(a->w_gate_up_scale != nullptr && a->w_down_scale != nullptr,
            "moe_grouped_ffn: MXFP4 weights need w_gate_up_scale and w_down_scale");
    const int64_t es = a16 ? 2 : 1;   // bytes per activation element
    REQUIRE((int64_t)R * H * es < ((int64_t)1 << 31) && (int64_t)R * D * es < ((int64_t)1 << 31) &&
                (int64_t)D * H < ((int64_t)1 << 31),
            "moe_grouped_ffn: x_perm, the activation buffer and one expert's weights must each be under 2 GiB");
    REQUIRE(aligned16(a->b_gate_up) && aligned16(a->b_down), "moe_grouped_ffn: biases must be 16-byte aligned");
    if (a->w_gate_up_layout != MOE_WEIGHT_OUT_IN || a->w_down_layout != MOE_WEIGHT_OUT_IN)
      return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: MXFP4 weights must use the OUT_IN layout");
    if (R == 0) return ok();
    moe::FfnMxParams q{};
    q.offsets = a->expert_offsets;
    q.L = L;
    q.H = H;
    q.D = D;
    q.max_rows = R;
    q.fmt = a->gate_up_format;
    q.x_perm = (const uint8_t*)(a->x_perm ? a->x_perm : a->x);
    q.x_scale = (const uint8_t*)a->x_perm_scale;
    q.sorted_token = a->x_perm ? nullptr : a->sorted_token;
    q.w_gate_up = (const uint8_t*)a->w_gate_up;
    q.w_gate_up_scale = (const uint8_t*)a->w_gate_up_scale;
    q.w_down = (const uint8_t*)a->w_down;
    q.w_down_scale = (const uint8_t*)a->w_down_scale;
    q.b_gate_up = (const uint16_t*)a->b_gate_up;
    q.b_down = (const uint16_t*)a->b_down;
    q.gate_up_scales = a->gate_up_expert_scales;
    q.down_scales = a->down_expert_scales;
    q.act_kind = a->activation;
    q.alpha = a->alpha;
    q.limit = a->limit;
    q.act = (uint8_t*)a->act_workspace;
    q.act_scale = (uint8_t*)a->act_workspace + round_up((int64_t)R * D, 256);
    q.out = a->expert_out;
    q.out_bf16 = a->out_dtype == MOE_DTYPE_BF16;
    q.events = (hipEvent_t const*)a->timing_events;
    if (a16) return hip_status(moe::launch_ffn_w4a16(q, (hipStream_t)stream), "moe_grouped_ffn");
    return hip_status(moe::launch_ffn_mx(q, (hipStream_t)stream), "moe_grouped_ffn");
  }
  if (a->operand_dtype == MOE_DTYPE_FP8_E4M3_BLOCK128) {
    REQUIRE(H % 128 == 0 && D % 128 == 0, "moe_grouped_ffn: fp8 needs hidden_dim and moe_dim multiples of 128");
    REQUIRE(a->x_perm_scale != nullptr && (a->x_perm != nullptr || a->x != nullptr),
            "moe_grouped_ffn: fp8 takes x_perm (or per-token x) and x_perm_scale, quantised by moe_build_indices");
    REQUIRE(a->w_gate_up_scale != nullptr && a->w_down_scale != nullptr,
            "moe_grouped_ffn: fp8 weights need w_gate_up_scale and w_down_scale");
    // the GEMMs address permuted rows from each tile's first row and
    // gathered rows from x by token: the bounds are x [T, H] (gather) and
    // one expert's weights
    REQUIRE(!gather || gather_rows_fit(a, 1), "moe_grouped_ffn: %s", gather_bound_msg(a));
    REQUIRE((int64_t)2 * D * H < ((int64_t)1 << 31), "moe_grouped_ffn: one expert's weights must be under 2 GiB");
    REQUIRE(aligned16(a->b_gate_up) && aligned16(a->b_down), "moe_grouped_ffn: biases must be 16-byte aligned");
    if (a->w_gate_up_layout != MOE_WEIGHT_OUT_IN || a->w_down_layout != MOE_WEIGHT_OUT_IN)
      return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn: fp8 weights must use the OUT_IN layout");
    if (R == 0) return ok();
    moe::FfnFp8Params q{};
    q.offsets = a->expert_offsets;
    q.L = L;
    q.H = H;
    q.D = D;
    q.max_rows = R;
    q.x_perm = (const uint8_t*)(a->x_perm ? a->x_perm : a->x);
    q.x_scale = (const float*)a->x_perm_scale;
    q.sorted_token = a->x_perm ? nullptr : a->sorted_token;
    q.w_gate_up = (const uint8_t*)a->w_gate_up;
    q.w_gate_up_scale = (const float*)a->w_gate_up_scale;
    q.w_down = (const uint8_t*)a->w_down;
    q.w_down_scale = (const float*)a->w_down_scale;
    q.gate_up_scales = a->gate_up_expert_scales;
    q.down_scales = a->down_expert_scales;
    q.b_gate_up = (const uint16_t*)a->b_gate_up;
    q.b_down = (const uint16_t*)a->b_down;
    q.fmt = a->gate_up_format;
    q.act_kind = a->activation;
    q.alpha = a->alpha;
    q.limit = a->limit;
    q.act = (uint8_t*)a->act_workspace;
    q.act_scale = (float*)((uint8_t*)a->act_workspace + round_up((int64_t)R * D, 256));
    q.out = a->expert_out;
    q.out_bf16 = a->out_dtype == MOE_DTYPE_BF16;
    q.events = (hipEvent_t const*)a->timing_events;
    return hip_status(moe::launch_ffn_fp8(q, (hipStream_t)stream), "moe_grouped_ffn");
  }
  // the GEMMs address permuted rows from each tile's first row and
  // gathered rows from x by token: the bounds are x [T, H] (gather) and
  // one expert's weights
  REQUIRE(!gather || gather_rows_fit(a, 2), "moe_grouped_ffn: %s", gather_bound_msg(a));
  REQUIRE((int64_t)2 * D * H * 2 < ((int64_t)1 << 31), "moe_grouped_ffn: one expert's weights must be under 2 GiB");
  if (a->w_gate_up_layout == MOE_WEIGHT_IN_OUT && a->gate_up_format != MOE_GATE_UP_CONCATENATED)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_grouped_ffn: IN_OUT gate_up weights take the concatenated format (use OUT_IN for interleaved)");
  if (R == 0) return ok();
  moe::FfnBf16Params p{};
  p.gu_in_out = a->w_gate_up_layout == MOE_WEIGHT_IN_OUT;
  p.d_in_out = a->w_down_layout == MOE_WEIGHT_IN_OUT;
  p.offsets = a->expert_offsets;
  p.L = L;
  p.H = H;
  p.D = D;
  p.max_rows = R;
  p.x_perm = (const uint16_t*)a->x_perm;
  p.x = (const uint16_t*)a->x;
  p.sorted_token = a->sorted_token;
  p.w_gate_up = (const uint16_t*)a->w_gate_up;
  p.b_gate_up = (const uint16_t*)a->b_gate_up;
  p.w_down = (const uint16_t*)a->w_down;
  p.b_down = (const uint16_t*)a->b_down;
  p.gate_up_scales = a->gate_up_expert_scales;
  p.down_scales = a->down_expert_scales;
  p.fmt = a->gate_up_format;
  p.act_kind = a->activation;
  p.alpha = a->alpha;
  p.limit = a->limit;
  p.act = (uint16_t*)a->act_workspace;
  {
    uint8_t* split = (uint8_t*)a->act_workspace + round_up((int64_t)R * D * 2, 256);
    p.split_slots = moe::split_slots_for(R);
    p.split_counters = p.split_slots > 0 ? (int32_t*)split : nullptr;
    p.split_partial = p.split_slots > 0 ? (float*)(split + moe::SPLIT_COUNTERS * 4) : nullptr;
  }
  p.out = a->expert_out;
  p.out_bf16 = a->out_dtype == MOE_DTYPE_BF16;
  p.events = (hipEvent_t const*)a->timing_events;
  return hip_status(moe::launch_ffn_bf16(p, (hipStream_t)stream), "moe_grouped_ffn");
}

// ---------------------------------------------------------------- fused single launch
int64_t moe_ffn_fused_workspace_bytes(int32_t max_rows, int32_t H, int32_t D, int32_t L) {
  if (max_rows < 0 || H < 1 || D < 1 || L < 1) return 0;
  return moe::fused_layout(max_rows, H, D, L).bytes;
}

moe_status_t moe_grouped_ffn_fused(const moe_ffn_args_t* a, void* stream) {
  REQUIRE(a != nullptr, "moe_grouped_ffn_fused: args is NULL");
  const int R = a->max_rows, H = a->hidden_dim, D = a->moe_dim, L = a->n_local_experts;
  REQUIRE(R >= 0, "moe_grouped_ffn_fused: max_rows must be >= 0 (got %d)", R);
  REQUIRE(H >= 64 && H % 64 == 0, "moe_grouped_ffn_fused: hidden_dim must be a positive multiple of 64 (got %d)", H);
  REQUIRE(D >= 128 && D % 128 == 0, "moe_grouped_ffn_fused: moe_dim must be a positive multiple of 128 (got %d)", D);
  REQUIRE(L >= 1 && L <= 1024, "moe_grouped_ffn_fused: n_local_experts must be in [1, 1024] (got %d)", L);
  const bool a16 = a->operand_dtype == MOE_DTYPE_MXFP4_W4A16;
  const bool mx = a->operand_dtype == MOE_DTYPE_MXFP4_W4A8 || a16;
  REQUIRE(a->operand_dtype == MOE_DTYPE_BF16 || mx,
          "moe_grouped_ffn_fused: operand_dtype must be BF16, MXFP4_W4A8 or MXFP4_W4A16");
  REQUIRE(a->expert_offsets != nullptr, "moe_grouped_ffn_fused: expert_offsets is required");
  REQUIRE(a->activation == MOE_ACT_SILU || a->activation == MOE_ACT_SWIGLUOAI || a->activation == MOE_ACT_GELU_TANH,
          "moe_grouped_ffn_fused: unknown activation %d", a->activation);
  REQUIRE(std::isfinite(a->alpha) && std::isfinite(a->limit), "moe_grouped_ffn_fused: alpha and limit must be finite");
  REQUIRE(a->activation == MOE_ACT_SWIGLUOAI || a->alpha == 0.0f,
          "moe_grouped_ffn_fused: alpha is the sigmoid scale of swigluoai and must be 0 for the other activations");
  REQUIRE(a->activation != MOE_ACT_GELU_TANH || a->limit == 0.0f, "moe_grouped_ffn_fused: limit must be 0 for gelu_tanh");
  REQUIRE(a->limit >= 0.0f, "moe_grouped_ffn_fused: limit must be >= 0");
  REQUIRE(a->gate_up_format == MOE_GATE_UP_CONCATENATED || a->gate_up_format == MOE_GATE_UP_INTERLEAVED,
          "moe_grouped_ffn_fused: unknown gate_up_format %d", a->gate_up_format);
  REQUIRE(a->out_dtype == MOE_DTYPE_FP32 || a->out_dtype == MOE_DTYPE_BF16,
          "moe_grouped_ffn_fused: out_dtype must be FP32 or BF16");
  REQUIRE(a->w_gate_up && a->w_down, "moe_grouped_ffn_fused: w_gate_up and w_down are required");
  REQUIRE(R == 0 || a->expert_out != nullptr, "moe_grouped_ffn_fused: expert_out is required");
  const bool gather = a->x_perm == nullptr;
  if (gather)
    REQUIRE(R == 0 || (a->x != nullptr && a->sorted_token != nullptr),
            "moe_grouped_ffn_fused: pass x_perm, or x and sorted_token to gather rows");
  else
    REQUIRE(a->x == nullptr, "moe_grouped_ffn_fused: pass either x_perm or x/sorted_token, not both");
  REQUIRE(aligned16(a->x_perm) && aligned16(a->x) && aligned16(a->w_gate_up) && aligned16(a->w_down) &&
              aligned16(a->act_workspace) && aligned16(a->expert_out) && aligned16(a->b_gate_up) &&
              aligned16(a->b_down),
          "moe_grouped_ffn_fused: tensors must be 16-byte aligned");
  // bytes per activation element; one expert's gate_up weights: 2D rows of H elements
  const int64_t es = (mx && !a16) ? 1 : 2;
  const int64_t wbytes = mx ? (int64_t)D * H : (int64_t)2 * D * H * 2;
  const int64_t x_rows = gather && a->num_tokens > 0 ? a->num_tokens : R;
  REQUIRE(x_rows * H * es < ((int64_t)1 << 31) && (int64_t)R * D * es < ((int64_t)1 << 31) &&
              wbytes < ((int64_t)1 << 31),
          "moe_grouped_ffn_fused: x (or x_perm), the activation buffer and one expert's weights must each be under 2 GiB");
  if (mx) {
    REQUIRE(H % 128 == 0, "moe_grouped_ffn_fused: MX needs hidden_dim a multiple of 128 (got %d)", H);
    if (a16)
      REQUIRE(a->x_perm_scale == nullptr, "moe_grouped_ffn_fused: W4A16 takes bf16 activations, no x_perm_scale");
    else
      REQUIRE(a->x_perm_scale != nullptr,
              "moe_grouped_ffn_fused: W4A8 takes x_perm (or per-token x) and x_perm_scale, quantised by "
              "moe_build_indices");
    REQUIRE(a->w_gate_up_scale != nullptr && a->w_down_scale != nullptr,
            "moe_grouped_ffn_fused: MXFP4 weights need w_gate_up_scale and w_down_scale");
    REQUIRE(aligned16(a->x_perm_scale) && aligned16(a->w_gate_up_scale) && aligned16(a->w_down_scale),
            "moe_grouped_ffn_fused: scale tensors must be 16-byte aligned");
  }
  if (a->w_gate_up_layout != MOE_WEIGHT_OUT_IN || a->w_down_layout != MOE_WEIGHT_OUT_IN)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_ffn_fused: weights must use the OUT_IN layout");
  const int64_t need = moe_ffn_fused_workspace_bytes(R, H, D, L);
  if (a->act_workspace_bytes < need || (need > 0 && a->act_workspace == nullptr))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_grouped_ffn_fused: act_workspace needs %lld bytes (got %lld)",
                (long long)need, (long long)a->act_workspace_bytes);
  if (R == 0) return ok();
  if (mx) {
    moe::FfnMxParams q{};
    q.offsets = a->expert_offsets;
    q.L = L;
    q.H = H;
    q.D = D;
    q.max_rows = R;
    q.fmt = a->gate_up_format;
    q.x_perm = (const uint8_t*)(a->x_perm ? a->x_perm : a->x);
    q.x_scale = (const uint8_t*)a->x_perm_scale;
    q.sorted_token = a->x_perm ? nullptr : a->sorted_token;
    q.w_gate_up = (const uint8_t*)a->w_gate_up;
    q.w_gate_up_scale = (const uint8_t*)a->w_gate_up_scale;
    q.w_down = (const uint8_t*)a->w_down;
    q.w_down_scale = (const uint8_t*)a->w_down_scale;
    q.b_gate_up = (const uint16_t*)a->b_gate_up;
    q.b_down = (const uint16_t*)a->b_down;
    q.gate_up_scales = a->gate_up_expert_scales;
    q.down_scales = a->down_expert_scales;
    q.act_kind = a->activation;
    q.alpha = a->alpha;
    q.limit = a->limit;
    q.out = a->expert_out;
    q.out_bf16 = a->out_dtype == MOE_DTYPE_BF16;
    q.events = (hipEvent_t const*)a->timing_events;
    if (a16)
      return hip_status(moe::launch_ffn_fused_w4a16(q, a->act_workspace, a->act_workspace_bytes, (hipStream_t)stream),
                        "moe_grouped_ffn_fused");
    return hip_status(moe::launch_ffn_fused_mx(q, a->act_workspace, a->act_workspace_bytes, (hipStream_t)stream),
                      "moe_grouped_ffn_fused");
  }
  moe::FfnBf16Params p{};
  p.offsets = a->expert_offsets;
  p.L = L;
  p.H = H;
  p.D = D;
  p.max_rows = R;
  p.x_perm = (const uint16_t*)a->x_perm;
  p.x = (const uint16_t*)a->x;
  p.sorted_token = a->sorted_token;
  p.w_gate_up = (const uint16_t*)a->w_gate_up;
  p.b_gate_up = (const uint16_t*)a->b_gate_up;
  p.w_down = (const uint16_t*)a->w_down;
  p.b_down = (const uint16_t*)a->b_down;
  p.gate_up_scales = a->gate_up_expert_scales;
  p.down_scales = a->down_expert_scales;
  p.fmt = a->gate_up_format;
  p.act_kind = a->activation;
  p.alpha = a->alpha;
  p.limit = a->limit;
  p.out = a->expert_out;
  p.out_bf16 = a->out_dtype == MOE_DTYPE_BF16;
  p.events = (hipEvent_t const*)a->timing_events;
  return hip_status(moe::launch_ffn_fused(p, a->act_workspace, a->act_workspace_bytes, (hipStream_t)stream),
                    "moe_grouped_ffn_fused");
}

// ---------------------------------------------------------------- combine
moe_status_t moe_combine(const moe_combine_args_t* a, void* stream) {
  REQUIRE(a != nullptr, "moe_combine: args is NULL");
  const int T = a->num_tokens, k = a->n_experts_per_tok, H = a->hidden_dim;
  REQUIRE(T >= 0, "moe_combine: num_tokens must be >= 0 (got %d)", T);
  REQUIRE(k >= 1 && k <= 1024, "moe_combine: n_experts_per_tok must be in [1, 1024] (got %d)", k);
  REQUIRE(H >= 8 && H % 8 == 0, "moe_combine: hidden_dim must be a positive multiple of 8 (got %d)", H);
  REQUIRE(a->out_dtype == MOE_DTYPE_FP32 || a->out_dtype == MOE_DTYPE_BF16,
          "moe_combine: out_dtype must be FP32 or BF16");
  REQUIRE(T == 0 || (a->expert_out && a->row_of_slot && a->y),
          "moe_combine: expert_out, row_of_slot and y are required");
  REQUIRE(aligned16(a->expert_out) && aligned16(a->y), "moe_combine: expert_out and y must be 16-byte aligned");
  REQUIRE(a->n_shared >= 0 && a->n_shared <= 1024, "moe_combine: n_shared must be in [0, 1024] (got %d)",
          a->n_shared);
  REQUIRE(a->n_shared == 0 || T == 0 || a->shared_out != nullptr,
          "moe_combine: shared_out is required when n_shared > 0");
  REQUIRE(a->n_shared == 0 || aligned16(a->shared_out), "moe_combine: shared_out must be 16-byte aligned");
  return hip_status(moe::launch_combine(a->expert_out, a->out_dtype == MOE_DTYPE_BF16, a->row_of_slot,
                                        a->expert_weights, a->token_mask, T, k, H, (uint16_t*)a->y,
                                        a->n_shared, a->shared_out, a->shared_weights,
                                        (hipStream_t)stream),
                    "moe_combine");
}

// ---------------------------------------------------------------- shared-expert buckets
moe_status_t moe_shared_indices(int32_t T, int32_t n_shared, int32_t* expert_offsets,
                                int32_t* sorted_token, void* stream) {
  REQUIRE(T >= 0, "moe_shared_indices: num_tokens must be >= 0 (got %d)", T);
  REQUIRE(n_shared >= 1 && n_shared <= 1024, "moe_shared_indices: n_shared must be in [1, 1024] (got %d)",
          n_shared);
  REQUIRE((int64_t)T * n_shared < ((int64_t)1 << 31), "moe_shared_indices: n_shared * num_tokens must be < 2^31");
  REQUIRE(expert_offsets != nullptr && (T == 0 || sorted_token != nullptr),
          "moe_shared_indices: expert_offsets and sorted_token are required");
  return hip_status(moe::launch_shared_indices(T, n_shared, expert_offsets, sorted_token, (hipStream_t)stream),
                    "moe_shared_indices");
}

// ---------------------------------------------------------------- backward
moe_status_t moe_combine_backward(const moe_combine_backward_args_t* a, void* stream) {
  REQUIRE(a != nullptr, "moe_combine_backward: args is NULL");
  const int T = a->num_tokens, k = a->n_experts_per_tok, H = a->hidden_dim;
  REQUIRE(T >= 0, "moe_combine_backward: num_tokens must be >= 0 (got %d)", T);
  REQUIRE(k >= 1 && k <= 1024, "moe_combine_backward: n_experts_per_tok must be in [1, 1024] (got %d)", k);
  REQUIRE(H >= 8 && H % 8 == 0, "moe_combine_backward: hidden_dim must be a positive multiple of 8 (got %d)", H);
  REQUIRE(a->out_dtype == MOE_DTYPE_FP32 || a->out_dtype == MOE_DTYPE_BF16,
          "moe_combine_backward: out_dtype must be FP32 or BF16");
  REQUIRE(T == 0 || (a->dy && a->row_of_slot && a->d_expert_out),
          "moe_combine_backward: dy, row_of_slot and d_expert_out are required");
  REQUIRE(T == 0 || a->d_expert_weights == nullptr || a->expert_out != nullptr,
          "moe_combine_backward: expert_out is required for d_expert_weights");
  REQUIRE(aligned16(a->dy) && aligned16(a->expert_out) && aligned16(a->d_expert_out),
          "moe_combine_backward: dy, expert_out and d_expert_out must be 16-byte aligned");
  moe::CombineBwdParams q{};
  q.T = T;
  q.k = k;
  q.H = H;
  q.dy = (const uint16_t*)a->dy;
  q.O = a->expert_out;
  q.o_bf16 = a->out_dtype == MOE_DTYPE_BF16;
  q.row_of_slot = a->row_of_slot;
  q.w = a->expert_weights;
  q.mask = a->token_mask;
  q.dO = (uint16_t*)a->d_expert_out;
  q.dw = a->d_expert_weights;
  return hip_status(moe::launch_combine_backward(q, (hipStream_t)stream), "moe_combine_backward");
}

int64_t moe_ffn_backward_workspace_bytes(int32_t max_rows, int32_t H, int32_t D, int32_t L) {
  if (max_rows < 0 || H < 1 || D < 1 || L < 1) return 0;
  return moe::ffn_bwd_layout(max_rows, H, D, L).bytes;
}

moe_status_t moe_grouped_ffn_backward(const moe_ffn_backward_args_t* a, void* stream) {
  REQUIRE(a != nullptr, "moe_grouped_ffn_backward: args is NULL");
  const int R = a->max_rows, H = a->hidden_dim, D = a->moe_dim, L = a->n_local_experts;
  REQUIRE(R >= 0, "moe_grouped_ffn_backward: max_rows must be >= 0 (got %d)", R);
  REQUIRE(H >= 64 && H % 64 == 0, "moe_grouped_ffn_backward: hidden_dim must be a positive multiple of 64 (got %d)",
          H);
  REQUIRE(D >= 64 && D % 64 == 0, "moe_grouped_ffn_backward: moe_dim must be a positive multiple of 64 (got %d)", D);
  REQUIRE(L >= 1 && L <= 1024, "moe_grouped_ffn_backward: n_local_experts must be in [1, 1024] (got %d)", L);
  REQUIRE(a->activation == MOE_ACT_SILU || a->activation == MOE_ACT_SWIGLUOAI || a->activation == MOE_ACT_GELU_TANH,
          "moe_grouped_ffn_backward: unknown activation %d", a->activation);
  REQUIRE(std::isfinite(a->alpha) && std::isfinite(a->limit),
          "moe_grouped_ffn_backward: alpha and limit must be finite");
  REQUIRE(a->activation == MOE_ACT_SWIGLUOAI || a->alpha == 0.0f,
          "moe_grouped_ffn_backward: alpha is the sigmoid scale of swigluoai and must be 0 for the other activations");
  REQUIRE(a->activation != MOE_ACT_GELU_TANH || a->limit == 0.0f,
          "moe_grouped_ffn_backward: limit must be 0 for gelu_tanh");
  REQUIRE(a->limit >= 0.0f, "moe_grouped_ffn_backward: limit must be >= 0");
  REQUIRE(a->gate_up_format == MOE_GATE_UP_CONCATENATED || a->gate_up_format == MOE_GATE_UP_INTERLEAVED,
          "moe_grouped_ffn_backward: unknown gate_up_format %d", a->gate_up_format);
  REQUIRE(a->expert_offsets != nullptr, "moe_grouped_ffn_backward: expert_offsets is required");
  REQUIRE(a->w_gate_up && a->w_gate_up_stacked && a->w_down_stacked,
          "moe_grouped_ffn_backward: w_gate_up, w_gate_up_stacked and w_down_stacked are required");
  REQUIRE(a->d_w_gate_up && a->d_w_down, "moe_grouped_ffn_backward: d_w_gate_up and d_w_down are required");
  REQUIRE(R == 0 || (a->d_expert_out && a->d_x_perm),
          "moe_grouped_ffn_backward: d_expert_out and d_x_perm are required");
  const bool gather = a->x_perm == nullptr;
  if (gather)
    REQUIRE(R == 0 || (a->x != nullptr && a->sorted_token != nullptr),
            "moe_grouped_ffn_backward: pass x_perm, or x and sorted_token to gather rows");
  else
    REQUIRE(a->x == nullptr, "moe_grouped_ffn_backward: pass either x_perm or x/sorted_token, not both");
  REQUIRE(aligned16(a->x_perm) && aligned16(a->x) && aligned16(a->w_gate_up) && aligned16(a->w_gate_up_stacked) &&
              aligned16(a->w_down_stacked) && aligned16(a->b_gate_up) && aligned16(a->d_expert_out) &&
              aligned16(a->d_x_perm) && aligned16(a->d_w_gate_up) && aligned16(a->d_w_down) &&
              aligned16(a->workspace),
          "moe_grouped_ffn_backward: tensors must be 16-byte aligned");
  const moe::FfnBwdLayout f = moe::ffn_bwd_layout(R, H, D, L);
  const int64_t two_gib = (int64_t)1 << 31;
  REQUIRE((int64_t)R * H * 4 < two_gib && (int64_t)R * 2 * D * 2 < two_gib && (int64_t)2 * D * H * 2 < two_gib &&
              (int64_t)2 * D * f.rp * 2 < two_gib && (int64_t)H * f.rp * 2 < two_gib,
          "moe_grouped_ffn_backward: the row buffers, their transposed copies and one expert's weights must each be "
          "under 2 GiB");
  if (a->workspace_bytes < f.bytes || a->workspace == nullptr)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_grouped_ffn_backward: workspace needs %lld bytes (got %lld)",
                (long long)f.bytes, (long long)a->workspace_bytes);
  moe::FfnBwdParams q{};
  q.offsets = a->expert_offsets;
  q.L = L;
  q.H = H;
  q.D = D;
  q.max_rows = R;
  q.x = (const uint16_t*)a->x;
  q.sorted_token = a->sorted_token;
  q.x_perm = (const uint16_t*)a->x_perm;
  q.w_gate_up = (const uint16_t*)a->w_gate_up;
  q.w_gate_up_stacked = (const uint16_t*)a->w_gate_up_stacked;
  q.w_down_stacked = (const uint16_t*)a->w_down_stacked;
  q.b_gate_up = (const uint16_t*)a->b_gate_up;
  q.fmt = a->gate_up_format;
  q.act_kind = a->activation;
  q.alpha = a->alpha;
  q.limit = a->limit;
  q.gate_up_scales = a->gate_up_expert_scales;
  q.down_scales = a->down_expert_scales;
  q.d_out = (const uint16_t*)a->d_expert_out;
  q.d_x_perm = a->d_x_perm;
  q.d_w_gate_up = a->d_w_gate_up;
  q.d_w_down = a->d_w_down;
  q.d_b_gate_up = a->d_b_gate_up;
  q.d_b_down = a->d_b_down;
  q.ws = a->workspace;
  q.events = (hipEvent_t const*)a->timing_events;
  return hip_status(moe::launch_ffn_backward(q, (hipStream_t)stream), "moe_grouped_ffn_backward");
}

moe_status_t moe_transpose_bf16(const void* src, void* dst, int32_t batch, int32_t rows, int32_t cols, void* stream) {
  REQUIRE(batch >= 0 && rows >= 0 && cols >= 0, "moe_transpose_bf16: sizes must be >= 0");
  REQUIRE(rows % 64 == 0 && cols % 64 == 0, "moe_transpose_bf16: rows and cols must be multiples of 64 (got %d, %d)",
          rows, cols);
  REQUIRE((int64_t)batch * rows * cols == 0 || (src && dst), "moe_transpose_bf16: src and dst are required");
  REQUIRE(src != dst || (int64_t)batch * rows * cols == 0, "moe_transpose_bf16: src and dst must not be the same buffer");
  REQUIRE(aligned16(src) && aligned16(dst), "moe_transpose_bf16: src and dst must be 16-byte aligned");
  return hip_status(moe::launch_transpose_bf16((const uint16_t*)src, (uint16_t*)dst, batch, rows, cols,
                                               (hipStream_t)stream),
                    "moe_transpose_bf16");
}

// ---------------------------------------------------------------- measured ceilings
moe_status_t moe_probe_mfma(int32_t kind, int32_t workgroups, int32_t iters, float* out, void* stream) {
  REQUIRE(kind == 0 || kind == 1, "moe_probe_mfma: kind must be 0 (bf16) or 1 (fp8) (got %d)", kind);
  REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), "moe_probe_mfma: workgroups must be in [1, 1048576] (got %d)",
          workgroups);
  REQUIRE(iters >= 1, "moe_probe_mfma: iters must be >= 1 (got %d)", iters);
  REQUIRE(out != nullptr, "moe_probe_mfma: out is required");
  return hip_status(moe::launch_mfma_probe(kind, workgroups, iters, out, (hipStream_t)stream), "moe_probe_mfma");
}

moe_status_t moe_probe_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  REQUIRE(bytes >= 0 && bytes % 16 == 0, "moe_probe_stream_copy: bytes must be a multiple of 16 >= 0");
  if (bytes == 0) return ok();
  REQUIRE(src && dst, "moe_probe_stream_copy: src and dst are required");
  REQUIRE(aligned16(src) && aligned16(dst), "moe_probe_stream_copy: src and dst must be 16-byte aligned");
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  REQUIRE(s0 + (uintptr_t)bytes <= d0 || d0 + (uintptr_t)bytes <= s0,
          "moe_probe_stream_copy: src and dst must not overlap");
  return hip_status(moe::launch_stream_copy(src, dst, bytes / 16, (hipStream_t)stream), "moe_probe_stream_copy");
}

moe_status_t moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* out, int32_t out_len, void* stream) {
  REQUIRE(bytes >= 0 && bytes % 16 == 0, "moe_probe_stream_read: bytes must be a multiple of 16 >= 0");
  if (bytes == 0) return ok();
  REQUIRE(src && out, "moe_probe_stream_read: src and out are required");
  REQUIRE(aligned16(src), "moe_probe_stream_read: src must be 16-byte aligned");
  REQUIRE(out_len >= 4, "moe_probe_stream_read: out_len must be >= 4 (got %d)", out_len);
  return hip_status(moe::launch_stream_read(src, bytes / 16, out, out_len, (hipStream_t)stream),
                    "moe_probe_stream_read");
}

}  // extern "C"
