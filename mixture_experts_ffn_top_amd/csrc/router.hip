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
// Each round takes the wave maximum of the order-preserving 32-bit key
// images, then the lowest expert index holding it (first j whose ballot is
// non-empty, lowest lane in it), and removes that entry; 0 marks removed
// entries and experts past E (no float maps to 0).
template <int J>
__device__ __forceinline__ void wave_topk(const float (&key)[J], int E, int k, int lane,
                                          int& sel_idx, float& sel_key) {
  uint32_t cand[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + MOE_WAVE * j;
    cand[j] = (e < E) ? order_key(key[j]) : 0u;
  }
  sel_idx = -1;
  sel_key = 0.0f;
  for (int it = 0; it < k; ++it) {
    uint32_t best = cand[0];
#pragma unroll
    for (int j = 1; j < J; ++j) best = cand[j] > best ? cand[j] : best;
    const uint32_t m = wave_max_u32(best);
    int win = -1;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint64_t b = __ballot(cand[j] == m);
      if (win < 0 && b != 0) win = MOE_WAVE * j + (int)__builtin_ctzll(b);
    }
    if (lane == it) {
      sel_idx = win;
      sel_key = order_key_inv(m);
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (lane + MOE_WAVE * j == win) cand[j] = 0u;
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
// A workgroup owns 16 tokens.  logits^T[e][t] = sum_h W[e][h] x[t][h] runs on
// v_mfma_f32_16x16x32_bf16 with W as the A operand (16 experts per tile) and
// x as the B operand (16 tokens).  The hidden dimension is streamed in chunks
// of CC columns: the 16 token rows and the padded expert rows of a chunk go
// straight from HBM/L2 into LDS with buffer loads (no VGPRs, one 1 KB
// coalesced piece per instruction), NS chunks deep, so that many loads are
// in flight per CU; the kernel is bound by reading x once.  Inside a chunk
// wave w takes the 32-column k steps w, w+4, ...; the four partial sums meet
// in LDS, then each wave runs the top-k of 4 tokens.
//
// W32: the gate in float32 (StackedMoE page, router_dtype float32: the gate
// is built in float32 and its bf16 input cast to float32, which is exact).
// The expert rows of a chunk are then float32, the chunk 128 columns wide,
// and each 32-column k step runs as eight v_mfma_f32_16x16x4_f32: in MFMA m,
// lane group g supplies column 8g + m of the step (the same permutation of k
// for both operands), so each lane's 8 values stay contiguous in LDS.
//
// LDS row of a chunk: 16-byte pieces; piece p of row r sits at slot
// p ^ (r & 15): the 16 lanes of a fragment read (16 rows, one piece) then hit
// 16 different 16-byte bank groups.
static constexpr int RX_BUF_DWORD3 = 0x00020000;  // raw buffer resource word 3 (gfx9)

template <int ETILES, bool W32>
struct RxShape {
  static constexpr int EP = ETILES * 16;
  static constexpr int CC = W32 ? 128 : 256;                        // columns per chunk
  static constexpr int XRB = CC * 2;                                // bytes of a token row of a chunk
  static constexpr int WRB = CC * (W32 ? 4 : 2);                    // bytes of an expert row of a chunk
  static constexpr int XBLK = 16 * XRB / 1024;                      // 1 KB blocks of token rows
  static constexpr int STAGE = 16 * XRB + EP * WRB;                 // bytes per chunk
  // chunks in the pipeline: for E <= 32 few enough (<= 72 KB of LDS) that two
  // workgroups share a CU, so that at large T one's ramp and top-k overlap
  // the other's stream (at T = 32768, E = 8: 94 us against 110 with 8 chunks)
  static constexpr int NS = ETILES == 1 ? 4 : ETILES == 2 ? 3 : ETILES == 4 ? 3 : 2;
  static constexpr int LPW = STAGE / 1024 / 4;                      // 1 KB loads per wave per chunk
  static constexpr int PART = 4 * 16 * (EP + 1) * 4;                // partial-sum exchange
  static constexpr int LDS = NS * STAGE > PART ? NS * STAGE : PART;
  static_assert(STAGE % 4096 == 0, "a chunk is a whole number of 1 KB loads per wave");
};

// This wave's LPW loads of chunk c into the stage at `st`: 1 KB block
// g = wave * LPW + l, token rows for g < XBLK, expert rows after.
template <int ETILES, bool W32, int LPW>
__device__ __forceinline__ void rx_issue(char* st, int c, int wave, const uint32_t (&voff)[LPW],
                                         __amdgpu_buffer_rsrc_t x_rsrc, __amdgpu_buffer_rsrc_t w_rsrc) {
  using S = RxShape<ETILES, W32>;
#pragma unroll
  for (int l = 0; l < LPW; ++l) {
    const int g = wave * LPW + l;
    if (g < S::XBLK)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (lptr_t)(st + g * 1024), 16, voff[l], c * S::XRB, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lptr_t)(st + g * 1024), 16, voff[l], c * S::WRB, 0, 0);
  }
}

template <int ETILES, int J, bool W32>
__global__ __launch_bounds__(256) void router_softmax_x_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ wg, int T, int H, int E, int k,
    float scale, const float* __restrict__ global_scale, int renorm, float* __restrict__ logits_out,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  using S = RxShape<ETILES, W32>;
  constexpr int EP = S::EP, NS = S::NS, LPW = S::LPW, STAGE = S::STAGE, CC = S::CC;
  constexpr int XRB = S::XRB, WRB = S::WRB, XBLK = S::XBLK;
  constexpr int WEB = W32 ? 4 : 2;  // bytes per gate element
  __shared__ __attribute__((aligned(1024))) char smem[S::LDS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = blockIdx.x * 16;
  const int col = lane & 15, grp = lane >> 4;
  const int nrows = min(16, T - t0);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)t0 * H), (short)0, nrows * H * 2, RX_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)wg, (short)0, E * H * WEB, RX_BUF_DWORD3);
  // Load l of this wave moves 1 KB block g = wave * LPW + l of a chunk: token
  // rows for g < XBLK (XRB bytes each), then expert rows (WRB bytes each);
  // lane -> (row, slot).  Rows past the token or expert count read zeros
  // (buffer bounds).
  uint32_t voff[LPW];
#pragma unroll
  for (int l = 0; l < LPW; ++l) {
    const int g = wave * LPW + l;
    if (g < XBLK) {
      constexpr int PPR = XRB / 16;                // pieces per token row
      const int row = g * (1024 / XRB) + lane / PPR;
      const int piece = (lane % PPR) ^ (row & 15);
      voff[l] = (uint32_t)row * (uint32_t)H * 2u + (uint32_t)piece * 16u;
    } else {
      constexpr int PPR = WRB / 16;                // pieces per expert row
      const int row = (g - XBLK) * (1024 / WRB) + lane / PPR;
      const int piece = (lane % PPR) ^ (row & 15);
      voff[l] = (uint32_t)row * (uint32_t)H * (uint32_t)WEB + (uint32_t)piece * 16u;
    }
  }
  const int nchunk = (H + CC - 1) / CC;

#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nchunk) rx_issue<ETILES, W32, LPW>(smem + (c % NS) * STAGE, c, wave, voff, x_rsrc, w_rsrc);
  f32x4_t acc[ETILES];
#pragma unroll
  for (int i = 0; i < ETILES; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nchunk; ++c) {
    // chunk c landed (for this wave) once at most the loads of the chunks
    // issued after it are outstanding; the barrier publishes every wave's
    if (c + NS - 2 < nchunk) __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * LPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the buffer of chunk c-1 is free: every wave has passed the barrier
    if (c + NS - 1 < nchunk)
      rx_issue<ETILES, W32, LPW>(smem + ((c + NS - 1) % NS) * STAGE, c + NS - 1, wave, voff, x_rsrc, w_rsrc);
    const char* st = smem + (c % NS) * STAGE;
    const char* sw = st + 16 * XRB;                 // the expert rows of the chunk
    const int cols_left = H - c * CC;
#pragma unroll
    for (int jj = 0; jj < CC / 128; ++jj) {
      const int p = 4 * (wave + 4 * jj) + grp;     // this lane's 8 columns of 32-column k step wave + 4*jj
      u32x4_t bv = *(const u32x4_t*)(st + col * XRB + (p ^ col) * 16);
      if constexpr (!W32) {
        u32x4_t av[ETILES];
#pragma unroll
        for (int et = 0; et < ETILES; ++et)
          av[et] = *(const u32x4_t*)(sw + (et * 16 + col) * WRB + (p ^ col) * 16);
        if (p * 8 >= cols_left) {                   // past the end of the rows (last chunk)
          bv = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
          for (int et = 0; et < ETILES; ++et) av[et] = u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int et = 0; et < ETILES; ++et)
          acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[et]),
                                                            __builtin_bit_cast(bf16x8_t, bv), acc[et], 0, 0, 0);
      } else {
        // the 8 float32 gate values of these columns are pieces 2p and 2p + 1
        if (p * 8 >= cols_left) bv = u32x4_t{0u, 0u, 0u, 0u};
        float xf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xf[2 * i] = bf16_to_f32((uint16_t)(bv[i] & 0xffffu));
          xf[2 * i + 1] = bf16_to_f32((uint16_t)(bv[i] >> 16));
        }
#pragma unroll
        for (int et = 0; et < ETILES; ++et) {
          const char* wr = sw + (et * 16 + col) * WRB;
          f32x4_t a0 = *(const f32x4_t*)(wr + ((2 * p) ^ col) * 16);
          f32x4_t a1 = *(const f32x4_t*)(wr + ((2 * p + 1) ^ col) * 16);
          if (p * 8 >= cols_left) a0 = a1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[et] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[m], xf[m], acc[et], 0, 0, 0);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[et] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[m], xf[4 + m], acc[et], 0, 0, 0);
        }
      }
    }
  }
  // the exchange reuses the stage buffers once every wave is done with them
  __syncthreads();
  float (*s_part)[16][EP + 1] = (float (*)[16][EP + 1])smem;
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

hipError_t launch_router_softmax_x(const uint16_t* x, const void* wg, int w32, int T, int H, int E,
                                   int k, float scale, const float* gs, int renorm,
                                   float* logits_out, int32_t* idx, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 15) / 16), block(256);
  const int et = (E + 15) / 16;
#define LAUNCH(ET, JJ, W)                                                                          \
  router_softmax_x_kernel<ET, JJ, W><<<grid, block, 0, st>>>(x, wg, T, H, E, k, scale, gs, renorm,  \
                                                             logits_out, idx, w)
#define BY_E(W)                                                                                    \
  if (et <= 1) LAUNCH(1, 1, W);                                                                    \
  else if (et <= 2) LAUNCH(2, 1, W);                                                               \
  else if (et <= 4) LAUNCH(4, 1, W);                                                               \
  else LAUNCH(8, 2, W)
  if (w32) {
    BY_E(true);
  } else {
    BY_E(false);
  }
#undef BY_E
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
