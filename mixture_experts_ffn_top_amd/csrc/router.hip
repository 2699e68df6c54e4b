// Routers: the softmax top-k gate (with its gate GEMM on MFMA) and the fused
// sigmoid + selection-bias top-k router with sink lanes
// (sink_gate_router_kernel page: description, Parameters, Args).
//
// Both run the selection as a wave64 arg-max repeated k times over packed
// (ordered float key, inverted expert index) u64 values, so the largest key
// wins and equal keys go to the lower expert index.
#include "common.h"
#include "kernels.h"

namespace moe {

// Selection over one token whose keys live in `key[j]` for expert
// lane + 64*j.  Lane i < k returns the i-th selected expert and its key.
template <int J>
__device__ __forceinline__ void wave_topk(const float (&key)[J], int E, int k, int lane,
                                          int& sel_idx, float& sel_key) {
  uint64_t cand[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int e = lane + MOE_WAVE * j;
    cand[j] = (e < E) ? pack_key(key[j], e) : 0ull;
  }
  sel_idx = -1;
  sel_key = 0.0f;
  for (int it = 0; it < k; ++it) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) best = cand[j] > best ? cand[j] : best;
    uint64_t w = wave_max_u64(best);
    if (lane == it) {
      sel_idx = unpack_idx(w);
      uint32_t u = (uint32_t)(w >> 32);
      u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
      sel_key = __uint_as_float(u);
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (cand[j] == w) cand[j] = 0ull;
  }
}

// Softmax weights of the selected lanes (lane < k holds its logit z).
__device__ __forceinline__ float softmax_selected(float z, int lane, int k) {
  float zmax = __shfl(z, 0, MOE_WAVE);  // slot 0 holds the largest logit
  float p = (lane < k) ? expf(z - zmax) : 0.0f;
  float s = wave_sum(p);
  return p / s;
}

// ------------------------------------------------------------ softmax, logits given
template <int J>
__global__ __launch_bounds__(256) void router_softmax_logits_kernel(
    const float* __restrict__ logits, int64_t ld, int T, int E, int k, float scale,
    const float* __restrict__ global_scale, int renorm, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int e = lane + MOE_WAVE * j;
    key[j] = (e < E) ? logits[(int64_t)t * ld + e] : 0.0f;
  }
  int sidx;
  float skey;
  wave_topk<J>(key, E, k, lane, sidx, skey);
  const float gs = global_scale ? global_scale[0] : 1.0f;
  float w;
  if (renorm) {
    w = softmax_selected(skey, lane, k);
  } else {
    float zmax = __shfl(skey, 0, MOE_WAVE);
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (lane + MOE_WAVE * j < E) part += expf(key[j] - zmax);
    float tot = wave_sum(part);
    w = expf(skey - zmax) / tot;
  }
  if (lane < k) {
    idx_out[(int64_t)t * k + lane] = sidx;
    w_out[(int64_t)t * k + lane] = w * scale * gs;
  }
}

// ------------------------------------------------------------ softmax, gate GEMM fused
// A workgroup owns 16 tokens; its 4 waves split the hidden dimension into
// quarters.  logits^T[e][t] = sum_h W[e][h] x[t][h] runs on
// v_mfma_f32_16x16x32_bf16 with W as the A operand (16 experts per tile) and
// x as the B operand (16 tokens); inside a wave, lane group g = lane/16 walks
// its own contiguous part of the wave's quarter, 8 elements per step, so
// every lane issues 16-byte loads.  The four partial sums meet in LDS, then
// each wave runs the top-k of 4 tokens.
template <int ETILES, int J>
__global__ __launch_bounds__(256) void router_softmax_x_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T, int H, int E, int k,
    float scale, const float* __restrict__ global_scale, int renorm, float* __restrict__ logits_out,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  constexpr int EP = ETILES * 16;
  __shared__ float s_part[4][16][EP + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16;
  const int col = lane & 15, grp = lane >> 4;
  const int chunks = H / 8;                          // 8-element chunks of a row
  const int per_wave = (chunks + 3) / 4;
  const int c_beg = wave * per_wave;
  const int c_end = min(chunks, c_beg + per_wave);
  const int per_grp = (per_wave + 3) / 4;
  const int tok = t0 + col;
  const bool tok_ok = tok < T;
  f32x4_t acc[ETILES];
#pragma unroll
  for (int i = 0; i < ETILES; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < per_grp; ++s) {
    const int c = c_beg + grp * per_grp + s;
    const bool c_ok = c < c_end;
    u32x4_t bv = {0u, 0u, 0u, 0u};
    if (tok_ok && c_ok) bv = *(const u32x4_t*)(x + (int64_t)tok * H + c * 8);
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
#pragma unroll
    for (int et = 0; et < ETILES; ++et) {
      const int e = et * 16 + col;
      u32x4_t av = {0u, 0u, 0u, 0u};
      if (e < E && c_ok) av = *(const u32x4_t*)(wg + (int64_t)e * H + c * 8);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
      acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[et], 0, 0, 0);
    }
  }
  // acc[et][i] = partial logit[token t0 + col][expert et*16 + 4*grp + i]
#pragma unroll
  for (int et = 0; et < ETILES; ++et)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[wave][col][et * 16 + grp * 4 + i] = acc[et][i];
  __syncthreads();
  const float gs = global_scale ? global_scale[0] : 1.0f;
  for (int tt = wave * 4; tt < wave * 4 + 4; ++tt) {
    const int t = t0 + tt;
    if (t >= T) break;
    float key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + MOE_WAVE * j;
      // fixed summation order over the four quarters
      key[j] = (e < E) ? ((s_part[0][tt][e] + s_part[1][tt][e]) + s_part[2][tt][e]) + s_part[3][tt][e] : 0.0f;
      if (logits_out && e < E) logits_out[(int64_t)t * E + e] = key[j];
    }
    int sidx;
    float skey;
    wave_topk<J>(key, E, k, lane, sidx, skey);
    float w;
    if (renorm) {
      w = softmax_selected(skey, lane, k);
    } else {
      float zmax = __shfl(skey, 0, MOE_WAVE);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (lane + MOE_WAVE * j < E) part += expf(key[j] - zmax);
      float tot = wave_sum(part);
      w = expf(skey - zmax) / tot;
    }
    if (lane < k) {
      idx_out[(int64_t)t * k + lane] = sidx;
      w_out[(int64_t)t * k + lane] = w * scale * gs;
    }
  }
}

// ------------------------------------------------------------ sigmoid + bias + sink lanes
template <int J>
__global__ __launch_bounds__(256) void router_sigmoid_sink_kernel(
    const float* __restrict__ logits, int64_t ld, const float* __restrict__ bias, int T, int E,
    int k, int s, float scale, const float* __restrict__ global_scale, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, float* __restrict__ sink_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* zrow = logits + (int64_t)t * ld;
  float key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    int e = lane + MOE_WAVE * j;
    if (e < E) {
      float b = bias ? bias[e] : 0.0f;
      key[j] = __fadd_rn(sigmoid_key_f32(zrow[e]), b);
    } else {
      key[j] = 0.0f;
    }
  }
  int sidx;
  float skey;
  wave_topk<J>(key, E, k, lane, sidx, skey);
  // lanes [0, k): selected routed experts' raw logits; lanes [k, k+s): sinks
  const int n = k + s;
  float v = 0.0f;
  if (lane < k) v = zrow[sidx];
  else if (lane < n) v = zrow[E + (lane - k)];
  float ls = (lane < n) ? log_sigmoid_f32(v) : -INFINITY;
  float m = wave_max(ls);
  float p = (lane < n) ? expf(ls - m) : 0.0f;
  float tot = wave_sum(p);
  const float gs = global_scale ? global_scale[0] : 1.0f;
  float w = p / tot * scale * gs;
  if (lane < k) {
    idx_out[(int64_t)t * k + lane] = sidx;
    w_out[(int64_t)t * k + lane] = w;
  } else if (lane < n) {
    sink_out[(int64_t)t * s + (lane - k)] = w;
  }
}

// ------------------------------------------------------------ launchers
static int pick_j(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

hipError_t launch_router_softmax_logits(const float* logits, int64_t ld, int T, int E, int k,
                                        float scale, const float* gs, int renorm, int32_t* idx,
                                        float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  switch (pick_j(E)) {
#define CASE(JJ)                                                                                   \
  case JJ:                                                                                         \
    router_softmax_logits_kernel<JJ><<<grid, block, 0, st>>>(logits, ld, T, E, k, scale, gs,       \
                                                             renorm, idx, w);                     \
    break;
    CASE(1) CASE(2) CASE(4) CASE(8) CASE(16)
#undef CASE
  }
  return hipGetLastError();
}

hipError_t launch_router_softmax_x(const uint16_t* x, const uint16_t* wg, int T, int H, int E,
                                   int k, float scale, const float* gs, int renorm,
                                   float* logits_out, int32_t* idx, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 15) / 16), block(256);
  const int et = (E + 15) / 16;
#define LAUNCH(ET, JJ)                                                                             \
  router_softmax_x_kernel<ET, JJ><<<grid, block, 0, st>>>(x, wg, T, H, E, k, scale, gs, renorm,     \
                                                          logits_out, idx, w)
  if (et <= 1) LAUNCH(1, 1);
  else if (et <= 2) LAUNCH(2, 1);
  else if (et <= 4) LAUNCH(4, 1);
  else LAUNCH(8, 2);
#undef LAUNCH
  return hipGetLastError();
}

hipError_t launch_router_sigmoid_sink(const float* logits, int64_t ld, const float* bias, int T,
                                      int E, int k, int s, float scale, const float* gs,
                                      int32_t* idx, float* w, float* sink_w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  switch (pick_j(E)) {
#define CASE(JJ)                                                                                   \
  case JJ:                                                                                         \
    router_sigmoid_sink_kernel<JJ><<<grid, block, 0, st>>>(logits, ld, bias, T, E, k, s, scale,    \
                                                           gs, idx, w, sink_w);                   \
    break;
    CASE(1) CASE(2) CASE(4) CASE(8) CASE(16)
#undef CASE
  }
  return hipGetLastError();
}

}  // namespace moe
