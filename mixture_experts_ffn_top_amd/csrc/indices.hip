// Bucketing of token->expert assignments into a per-expert CSR
// (moe_create_indices on the sink_gate_router_kernel page: it needs every
// token's assignment, so it runs after the router as its own launches), and
// the row gather of the activations, optionally with the per-token 1x128
// e4m3 quantisation of the fp8 layer.
//
//   csr_hist    per block of IDX_SLOTS flat slots: LDS histogram over local
//               experts -> counts[e][block] (expert-major)
//   csr_scan    one workgroup: one flat exclusive scan of counts in that
//               order, which is at once the per-(expert, block) base and, at
//               block 0, the expert offset
//   csr_scatter per block: stable rank of each slot among same-expert slots
//               (wave ballots per distinct expert, LDS running counts) ->
//               sorted_token, row_of_slot, sorted_weight
//   permute     x_perm[p] = x[sorted_token[p]] (bf16 copy, or e4m3 + 1x128
//               fp32 scales, or MXFP8: e4m3 + one E8M0 byte per 32 columns)
// A batch of at most CSR_SMALL_MAX slots (decode) is bucketed by one
// workgroup in one launch instead (csr_small), the waves in the roles of the
// blocks, counts and running rows in LDS.
#include "common.h"
#include "kernels.h"

namespace moe {

static constexpr int IDX_SLOTS = 512;   // flat slots per workgroup

int64_t csr_num_blocks(int64_t R) { return (R + IDX_SLOTS - 1) / IDX_SLOTS; }

__device__ __forceinline__ int local_expert(const int32_t* idx, const uint8_t* mask, int64_t sl,
                                            int k, int start, int L) {
  int e = idx[sl] - start;
  bool ok = (unsigned)e < (unsigned)L;
  if (ok && mask) ok = mask[sl / k] != 0;
  return ok ? e : -1;
}

__global__ __launch_bounds__(256) void csr_hist_kernel(const int32_t* __restrict__ idx,
                                                       const uint8_t* __restrict__ mask, int64_t R,
                                                       int k, int start, int L, int nblk,
                                                       int32_t* __restrict__ counts) {
  extern __shared__ int32_t s_h[];
  for (int e = threadIdx.x; e < L; e += 256) s_h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * IDX_SLOTS;
  for (int i = threadIdx.x; i < IDX_SLOTS; i += 256) {
    const int64_t sl = base + i;
    if (sl >= R) break;
    const int e = local_expert(idx, mask, sl, k, start, L);
    if (e >= 0) atomicAdd(&s_h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += 256) counts[(int64_t)e * nblk + blockIdx.x] = s_h[e];
}

// One workgroup of 1024 threads.  Exclusive scan, in place, of the
// n = L * nblk counts in expert-major order: entry (e, b) becomes the first
// CSR row of expert e's slots in block b, and entry (e, 0) is expert e's
// offset.  Tiles of 16 words per thread (64 KB) are read coalesced, the next
// tile's loads in flight while the current one is scanned.
static constexpr int SCAN_PER = 16;
static constexpr int SCAN_TILE = 1024 * SCAN_PER;

__device__ __forceinline__ void scan_load(const int32_t* c, int64_t g0, int64_t n, int32_t (&v)[SCAN_PER]) {
  if (g0 + SCAN_PER <= n) {
#pragma unroll
    for (int q = 0; q < SCAN_PER / 4; ++q) {
      const int4 x = *(const int4*)(c + g0 + 4 * q);
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < SCAN_PER; ++i) v[i] = (g0 + i < n) ? c[g0 + i] : 0;
  }
}

__global__ __launch_bounds__(1024) void csr_scan_kernel(int32_t* __restrict__ counts, int L,
                                                        int nblk, int32_t* __restrict__ offsets) {
  __shared__ int32_t s_wave[16];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t n = (int64_t)L * nblk;
  int32_t carry = 0;
  int32_t v[SCAN_PER], nv[SCAN_PER];
  if (n > 0) scan_load(counts, (int64_t)t * SCAN_PER, n, v);
  for (int64_t t0 = 0; t0 < n; t0 += SCAN_TILE) {
    const int64_t g0 = t0 + (int64_t)t * SCAN_PER;
    if (t0 + SCAN_TILE < n) scan_load(counts, g0 + SCAN_TILE, n, nv);
    int32_t run = 0;
#pragma unroll
    for (int i = 0; i < SCAN_PER; ++i) {
      const int32_t x = v[i];
      v[i] = run;
      run += x;
    }
    int32_t inc = run;                       // inclusive scan of the thread sums in the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(inc, o, MOE_WAVE);
      if (lane >= o) inc += y;
    }
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int32_t wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int32_t x = s_wave[w];
      wpre += (w < wave) ? x : 0;
      tot += x;
    }
    const int32_t base = carry + wpre + (inc - run);
    if (g0 + SCAN_PER <= n) {
#pragma unroll
      for (int q = 0; q < SCAN_PER / 4; ++q)
        *(int4*)(counts + g0 + 4 * q) =
            make_int4(v[4 * q] + base, v[4 * q + 1] + base, v[4 * q + 2] + base, v[4 * q + 3] + base);
    } else {
#pragma unroll
      for (int i = 0; i < SCAN_PER; ++i)
        if (g0 + i < n) counts[g0 + i] = v[i] + base;
    }
    carry += tot;
    __syncthreads();                         // s_wave is rewritten by the next tile
#pragma unroll
    for (int i = 0; i < SCAN_PER; ++i) v[i] = nv[i];
  }
  // the barrier above (a workgroup-scope fence) makes the scanned words visible
  for (int e = t; e < L; e += 1024) offsets[e] = nblk > 0 ? counts[(int64_t)e * nblk] : 0;
  if (t == 0) offsets[L] = carry;
}

__global__ __launch_bounds__(256) void csr_scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const uint8_t* __restrict__ mask,
    int64_t R, int k, int start, int L, int nblk, const int32_t* __restrict__ base,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ row_of_slot,
    float* __restrict__ sorted_weight) {
  extern __shared__ int32_t sm[];
  int32_t* running = sm;       // [L]   next CSR row of each expert in this block
  int32_t* wcnt = sm + L;      // [4][L] this round's count per wave and expert
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < L; e += 256) {
    running[e] = base[(int64_t)e * nblk + blockIdx.x];
    wcnt[e] = wcnt[L + e] = wcnt[2 * L + e] = wcnt[3 * L + e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  const int64_t blk0 = (int64_t)blockIdx.x * IDX_SLOTS;
  for (int round = 0; round < IDX_SLOTS / 256; ++round) {
    const int64_t sl = blk0 + round * 256 + wave * 64 + lane;
    if (blk0 + round * 256 >= R) break;  // uniform across the block
    const int e = (sl < R) ? local_expert(idx, mask, sl, k, start, L) : -1;
    uint64_t pending = __ballot(e >= 0);
    int rank = 0;
    while (pending) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int le = __shfl(e, leader, MOE_WAVE);
      const uint64_t m = __ballot(e == le);
      if (e == le) rank = __popcll(m & lt_mask);
      if (lane == leader) wcnt[wave * L + le] = __popcll(m);
      pending &= ~m;
    }
    __syncthreads();
    if (e >= 0) {
      int pos = running[e] + rank;
      for (int w2 = 0; w2 < wave; ++w2) pos += wcnt[w2 * L + e];
      sorted_token[pos] = (int32_t)(sl / k);
      row_of_slot[sl] = pos;
      if (sorted_weight) sorted_weight[pos] = w[sl];
    } else if (sl < R) {
      row_of_slot[sl] = -1;
    }
    __syncthreads();
    if (e >= 0 && rank == 0) atomicAdd(&running[e], wcnt[wave * L + e]);
    __syncthreads();
    if (e >= 0 && rank == 0) wcnt[wave * L + e] = 0;
  }
}

// ---- one-workgroup form for small batches
// flat slots: one CU walks them at ~1 ns each after a fixed ~7 us, which
// beats the three launches up to a few thousand slots (measured: 9.6 against
// 23 us for 2048 slots over 256 experts, 16 against 17 us for 8192 over 8)
static constexpr int CSR_SMALL_MAX = 4096;
static constexpr int CSR_SMALL_NT = 1024;     // threads: 16 waves; one expert each in the scan (L <= 1024)
static constexpr int CSR_SMALL_W = CSR_SMALL_NT / 64;
static constexpr int CSR_SMALL_STEPS = CSR_SMALL_MAX / CSR_SMALL_NT;  // 64-slot steps per wave

// Lanes of the wave whose key equals this lane's, from one ballot per key
// bit (keys below 2^bits): the cost does not depend on how many keys differ.
__device__ __forceinline__ uint64_t wave_match(int key, int bits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < bits; ++b) {
    const bool set = (key >> b) & 1;
    const uint64_t bal = __ballot(set);
    m &= set ? bal : ~bal;
  }
  return m;
}

// The whole CSR of R <= CSR_SMALL_MAX slots in one workgroup, as the three
// kernels above do it across workgroups, with the 16 waves in the roles of
// their blocks: wave q owns the contiguous slots [q S, (q+1) S) (S a multiple
// of 64), walked 64 at a time, the expert ids kept in registers.
//   1. cnt[q][e] = slots of wave q for expert e (each step's group of equal
//      experts counted once, by its first lane, from the wave's match mask);
//   2. one scan in expert-major order: cnt[q][e] becomes expert e's first
//      row for wave q's slots, and the offsets follow;
//   3. the waves walk their slots again: a slot's row is its group's base
//      plus its rank among the group's earlier lanes.
__global__ __launch_bounds__(CSR_SMALL_NT) void csr_small_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const uint8_t* __restrict__ mask, int R,
    int k, int start, int L, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ row_of_slot, float* __restrict__ sorted_weight) {
  extern __shared__ int32_t cnt[];  // [CSR_SMALL_W][L]
  __shared__ int32_t s_wave[CSR_SMALL_W];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < CSR_SMALL_W * L; i += CSR_SMALL_NT) cnt[i] = 0;
  const int S = (R + CSR_SMALL_W * 64 - 1) / (CSR_SMALL_W * 64) * 64;  // slots per wave
  const int s0 = wave * S;
  const int steps = S / 64;
  // the slots' experts (and mask bytes and routing weights), every load
  // issued before any is used: addresses past R are clamped to slot R - 1
  // and the slot is dropped afterwards
  int ex[CSR_SMALL_STEPS];
  float wt[CSR_SMALL_STEPS];
  uint8_t mk[CSR_SMALL_STEPS];
  if (R > 0) {
#pragma unroll
    for (int j = 0; j < CSR_SMALL_STEPS; ++j) ex[j] = idx[min(s0 + j * 64 + lane, R - 1)];
    if (mask) {
#pragma unroll
      for (int j = 0; j < CSR_SMALL_STEPS; ++j) mk[j] = mask[min(s0 + j * 64 + lane, R - 1) / k];
    }
    if (sorted_weight) {
#pragma unroll
      for (int j = 0; j < CSR_SMALL_STEPS; ++j) wt[j] = w[min(s0 + j * 64 + lane, R - 1)];
    }
  }
#pragma unroll
  for (int j = 0; j < CSR_SMALL_STEPS; ++j) {
    const int sl = s0 + j * 64 + lane;
    const int e = ex[j] - start;
    const bool ok = j < steps && sl < R && (unsigned)e < (unsigned)L && (!mask || mk[j] != 0);
    ex[j] = ok ? e : -1;
  }
  __syncthreads();
  const int bits = 32 - __clz(L);  // keys 0 .. L (L: no local expert)
  int32_t* mine = cnt + wave * L;
#pragma unroll
  for (int j = 0; j < CSR_SMALL_STEPS; ++j) {
    if (j < steps) {
      const uint64_t m = wave_match(ex[j] >= 0 ? ex[j] : L, bits);
      if (ex[j] >= 0 && __popcll(m & ((1ull << lane) - 1ull)) == 0) mine[ex[j]] += __popcll(m);
    }
  }
  __syncthreads();
  // expert e = tid: its waves' counts in wave order, then the scan over experts
  int tot = 0;
  if (tid < L) {
    for (int q = 0; q < CSR_SMALL_W; ++q) {
      const int c = cnt[q * L + tid];
      cnt[q * L + tid] = tot;
      tot += c;
    }
  }
  int inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, MOE_WAVE);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int wpre = 0, total = 0;
#pragma unroll
  for (int q = 0; q < CSR_SMALL_W; ++q) {
    wpre += q < wave ? s_wave[q] : 0;
    total += s_wave[q];
  }
  if (tid < L) {
    const int off = wpre + inc - tot;
    offsets[tid] = off;
    for (int q = 0; q < CSR_SMALL_W; ++q) cnt[q * L + tid] += off;
  }
  if (tid == 0) offsets[L] = total;
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < CSR_SMALL_STEPS; ++j) {
    if (j < steps) {
      const int sl = s0 + j * 64 + lane;
      const int e = ex[j];
      const uint64_t m = wave_match(e >= 0 ? e : L, bits);
      const int rank = __popcll(m & lt_mask);
      if (e >= 0) {
        const int pos = mine[e] + rank;
        sorted_token[pos] = sl / k;
        row_of_slot[sl] = pos;
        if (sorted_weight) sorted_weight[pos] = wt[j];
      } else if (sl < R) {
        row_of_slot[sl] = -1;
      }
      // the group's first lane moves the wave's base past the group (its
      // read above came first in the wave's program order)
      if (e >= 0 && rank == 0) mine[e] += __popcll(m);
    }
  }
}

// x_perm[p] = x[sorted_token[p]] for p < offsets_end[0]; one wave per row.
__global__ __launch_bounds__(256) void permute_bf16_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ sorted_token,
                                                           const int32_t* __restrict__ n_rows,
                                                           int H, uint16_t* __restrict__ xp) {
  const int lane = threadIdx.x & 63;
  const int n = n_rows[0];
  const int chunks = H / 8;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < n; row += gridDim.x * 4) {
    const u32x4_t* src = (const u32x4_t*)(x + (int64_t)sorted_token[row] * H);
    u32x4_t* dst = (u32x4_t*)(xp + (int64_t)row * H);
    for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
  }
}

// Per-row, per-128-column e4m3 quantisation fused into the gather: one wave
// per row, 16 lanes own one 128-column group (8 elements each).  A wave
// issues the loads of PQ_U passes (4 groups each, 1 KB per load) before any
// arithmetic, so every lane has PQ_U 16-byte reads in flight.  With
// sorted_token == nullptr the rows are not permuted: row p of the output is
// token p (n_fixed rows), the per-token form the fp8 GEMM gathers from.
static constexpr int PQ_U = 4;

__global__ __launch_bounds__(256) void permute_fp8_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ sorted_token,
                                                          const int32_t* __restrict__ n_rows,
                                                          int n_fixed, int H,
                                                          uint8_t* __restrict__ xq,
                                                          float* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int n = sorted_token ? n_rows[0] : n_fixed;
  const int groups = H / 128;
  const int sub = lane & 15, gq = lane >> 4;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < n; row += gridDim.x * 4) {
    const uint16_t* src = x + (int64_t)(sorted_token ? sorted_token[row] : row) * H;
    uint8_t* dst = xq + (int64_t)row * H;
    for (int g0 = 0; g0 < groups; g0 += 4 * PQ_U) {
      u32x4_t v[PQ_U];
#pragma unroll
      for (int u = 0; u < PQ_U; ++u) {
        const int g = g0 + 4 * u + gq;
        v[u] = u32x4_t{0u, 0u, 0u, 0u};
        if (g < groups) v[u] = *(const u32x4_t*)(src + g * 128 + sub * 8);
      }
#pragma unroll
      for (int u = 0; u < PQ_U; ++u) {
        const int g = g0 + 4 * u + gq;
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_to_f32((uint16_t)(v[u][i] & 0xffffu));
          f[2 * i + 1] = bf16_to_f32((uint16_t)(v[u][i] >> 16));
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = row16_max(amax);  // a 128-column group is one row of 16 lanes
        const float s = (amax > 0.0f) ? __fdiv_rn(amax, 448.0f) : 1.0f;
        const SharedDivisor ds = shared_divisor(s);
        uint2 q;
        q.x = e4m3x4(div_rn(ds, f[0]), div_rn(ds, f[1]), div_rn(ds, f[2]), div_rn(ds, f[3]));
        q.y = e4m3x4(div_rn(ds, f[4]), div_rn(ds, f[5]), div_rn(ds, f[6]), div_rn(ds, f[7]));
        if (g < groups) {
          *(uint2*)(dst + g * 128 + sub * 8) = q;
          if (sub == 0) xs[(int64_t)row * groups + g] = s;
        }
      }
    }
  }
}

// Per-row MXFP8 quantisation fused into the gather (OCP MX: 32 columns share
// one E8M0 scale): one wave per row, 4 lanes own one 32-column block (8
// elements each, block max over the quad by DPP); a wave issues the loads of
// PQ_U passes (1 KB each) before any arithmetic.  Shared exponent
// X = floor(log2 amax) - 8 (at least -127; 0 for an all-zero block), codes
// e4m3(v * 2^-X) with round to nearest even and saturation, scale byte X+127.
// With sorted_token == nullptr row p is token p (n_fixed rows).
__global__ __launch_bounds__(256) void permute_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ sorted_token,
                                                            const int32_t* __restrict__ n_rows,
                                                            int n_fixed, int H,
                                                            uint8_t* __restrict__ xq,
                                                            uint8_t* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int n = sorted_token ? n_rows[0] : n_fixed;
  const int chunks = H / 8;          // 16-byte pieces of a row; 4 per block
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < n; row += gridDim.x * 4) {
    const uint16_t* src = x + (int64_t)(sorted_token ? sorted_token[row] : row) * H;
    uint8_t* dst = xq + (int64_t)row * H;
    for (int c0 = 0; c0 < chunks; c0 += 64 * PQ_U) {
      u32x4_t v[PQ_U];
#pragma unroll
      for (int u = 0; u < PQ_U; ++u) {
        const int c = c0 + 64 * u + lane;
        v[u] = u32x4_t{0u, 0u, 0u, 0u};
        if (c < chunks) v[u] = *(const u32x4_t*)(src + c * 8);
      }
#pragma unroll
      for (int u = 0; u < PQ_U; ++u) {
        const int c = c0 + 64 * u + lane;
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_to_f32((uint16_t)(v[u][i] & 0xffffu));
          f[2 * i + 1] = bf16_to_f32((uint16_t)(v[u][i] >> 16));
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __uint_as_float(dpp_u32<DPP_QP_XOR1>(__float_as_uint(amax), 0u)));
        amax = fmaxf(amax, __uint_as_float(dpp_u32<DPP_QP_XOR2>(__float_as_uint(amax), 0u)));
        const int ex = (int)((__float_as_uint(amax) >> 23) & 0xffu);
        const int X = amax == 0.0f ? 0 : max(ex - 127 - 8, -127);
        const float inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X
        uint2 q;
        q.x = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
        q.y = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
        if (c < chunks) {
          *(uint2*)(dst + c * 8) = q;
          if ((lane & 3) == 0) xs[(int64_t)row * (H / 32) + c / 4] = (uint8_t)(X + 127);
        }
      }
    }
  }
}

// Buckets of the shared experts: every token in each, in token order.
__global__ __launch_bounds__(256) void shared_indices_kernel(int T, int n_shared, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_token) {
  const int64_t n = (int64_t)T * n_shared;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n; p += (int64_t)gridDim.x * 256)
    sorted_token[p] = (int32_t)(p % T);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= n_shared; i += 256) offsets[i] = i * T;
}

hipError_t launch_shared_indices(int T, int n_shared, int32_t* offsets, int32_t* sorted_token,
                                 hipStream_t st) {
  int64_t blocks = ((int64_t)T * n_shared + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  shared_indices_kernel<<<(int)blocks, 256, 0, st>>>(T, n_shared, offsets, sorted_token);
  return hipGetLastError();
}

hipError_t launch_build_indices(const int32_t* idx, const float* w, const uint8_t* mask, int T,
                                int k, int start, int L, int32_t* offsets, int32_t* sorted_token,
                                int32_t* row_of_slot, float* sorted_weight, int32_t* ws,
                                hipStream_t st) {
  const int64_t R = (int64_t)T * k;
  if (R <= CSR_SMALL_MAX && L <= CSR_SMALL_NT) {
    const int lds = CSR_SMALL_W * L * (int)sizeof(int32_t);  // up to 64 KB
    const hipError_t err =
        hipFuncSetAttribute((const void*)csr_small_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    csr_small_kernel<<<1, CSR_SMALL_NT, lds, st>>>(idx, w, mask, (int)R, k, start, L, offsets, sorted_token,
                                                   row_of_slot, sorted_weight);
    return hipGetLastError();
  }
  const int nblk = (int)csr_num_blocks(R);
  if (nblk > 0) {
    csr_hist_kernel<<<nblk, 256, L * sizeof(int32_t), st>>>(idx, mask, R, k, start, L, nblk, ws);
  }
  csr_scan_kernel<<<1, 1024, 0, st>>>(ws, L, nblk, offsets);
  if (nblk > 0) {
    csr_scatter_kernel<<<nblk, 256, 5 * L * sizeof(int32_t), st>>>(
        idx, w, mask, R, k, start, L, nblk, ws, sorted_token, row_of_slot, sorted_weight);
  }
  return hipGetLastError();
}

hipError_t launch_permute(const uint16_t* x, const int32_t* sorted_token, const int32_t* n_rows,
                          int64_t max_rows, int H, int kind, void* xp, void* xs, hipStream_t st) {
  if (max_rows == 0) return hipSuccess;
  int64_t blocks = (max_rows + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (kind == 1)
    permute_fp8_kernel<<<(int)blocks, 256, 0, st>>>(x, sorted_token, n_rows, (int)max_rows, H,
                                                    (uint8_t*)xp, (float*)xs);
  else if (kind == 2)
    permute_mxfp8_kernel<<<(int)blocks, 256, 0, st>>>(x, sorted_token, n_rows, (int)max_rows, H,
                                                      (uint8_t*)xp, (uint8_t*)xs);
  else
    permute_bf16_kernel<<<(int)blocks, 256, 0, st>>>(x, sorted_token, n_rows, H, (uint16_t*)xp);
  return hipGetLastError();
}

}  // namespace moe
