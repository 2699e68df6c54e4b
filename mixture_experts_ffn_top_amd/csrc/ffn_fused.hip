// Single-launch expert FFN for small batches: the gate_up grouped GEMM with
// the gated activation (L1) and the down GEMM (L2) in one launch, pipelined
// across workgroups (mega_ffn page: one launch that fuses the L1 and L2 legs,
// cross-workgroup arrival counters, no per-launch memset).
//
// A persistent grid (one workgroup per CU) takes work items from one atomic
// queue: first every L1 item (expert, 32-row block, 128 outputs), then every
// L2 item (expert, 32-row block, 256 outputs, one of S parts of K).  An L2
// item needs the whole A row block, i.e. all D/128 L1 items of its (expert,
// row block); it waits for that block's arrival counter.  Because every L1
// item leaves the queue before any L2 item, the items an L2 item waits for
// are already held by running workgroups, which never wait themselves: the
// wait always ends.  It is bounded anyway (a few hundred ms); on timeout it
// sets an error word and goes on, so a broken schedule gives wrong numbers,
// not a hang.
//
// Balance.  An L1 item streams 256 weight rows of length H, an unsplit L2
// item 256 rows of length D; with D several times H (Mixtral: 3.5x) the few
// long L2 items would leave most CUs idle at the end.  So when the launch has
// few L2 tiles, each is split into S = round(D/2H) parts along K.  Every part
// writes its fp32 partial tile to the workspace and counts itself in; the
// last part to arrive adds the S partials in part order (its own from
// registers) and runs the epilogue, so the result does not depend on which
// part came last.  No part waits for another.
//
// Visibility follows the HIP memory model at agent scope: an L1 item's waves
// fence-release their A stores (write-back of the XCD's L2) before the
// counter increment; an L2 item acquires the counter and fence-acquires
// (invalidate) before loading A, whichever XCD either ran on.  The last
// workgroup to leave resets the queue, the exit count and the arrival
// counters, so the control words start at zero on the next launch; the
// caller zeroes them once, when the workspace is allocated.
//
// Tiles are 32 x 256 with 4 waves (32 x 64 each: the gate and up columns of
// 32 outputs for L1), k stages of 64 bf16, 4 stages deep in LDS through
// buffer loads: the batch is bound by streaming the weights.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int F_BM = 32, F_BN = 256, F_BK = 64;
constexpr int F_NS = 4;                             // LDS stages
constexpr int F_NW = 4;                             // waves, each 32 rows x 64 columns
constexpr int F_NT = 64 * F_NW;
constexpr int F_ROW = F_BK * 2;                     // bytes of one bf16 stage row (8 chunks)
constexpr int F_A_BYTES = F_BM * F_ROW;             // 4 KB
constexpr int F_B_BYTES = F_BN * F_ROW;             // 32 KB
constexpr int F_STAGE = F_A_BYTES + F_B_BYTES;      // 36 KB
constexpr int F_LPW_A = F_A_BYTES / 1024 / F_NW;    // 1 KB loads per wave per stage: 1
constexpr int F_LPW_B = F_B_BYTES / 1024 / F_NW;    // 8
constexpr int F_LOADS = F_LPW_A + F_LPW_B;
constexpr int F_PIPE = F_NS * F_STAGE;              // 144 KB
constexpr int F_BUF_DWORD3 = 0x00020000;            // raw buffer resource word 3 (gfx9)
constexpr uint32_t F_OOB = 0x80000000u;             // past every buffer range: zeros, no memory
constexpr int F_SPIN_LIMIT = 1 << 20;               // bounded wait: ~0.2 s of s_sleep 8
constexpr int F_MAX_TILES = 256;                    // L2 tiles a launch may split along K
constexpr int F_MAX_PARTS = 8;
constexpr int F_HDR_WORDS = 4 + F_MAX_TILES;        // queue, exits, error, unused, split counters
constexpr int64_t F_PART_FLOATS = F_BM * F_BN;      // one partial tile, 32 KB

// 128-byte rows, 8 chunks of 16 bytes: chunk c of row r at c ^ f(r).
__device__ __forceinline__ int f_swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int f_off(int row, int chunk) { return row * F_ROW + ((chunk ^ f_swz(row)) << 4); }

__device__ __forceinline__ void f_block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct FusedArgs {
  const int32_t* offsets;
  int L, H, D;
  const uint16_t* x;           // bf16 [T, H] gathered through sorted_token, or [R, H] rows (sorted_token null)
  const int32_t* sorted_token;
  const uint16_t* w_gu;        // OUT_IN [L, 2D, H]
  const uint16_t* w_d;         // OUT_IN [L, H, D]
  const uint16_t* b_gu;        // [L, 2D] or null
  const uint16_t* b_d;         // [L, H] or null
  const float* s_gu;           // [L] or null
  const float* s_d;
  float alpha, limit;
  uint16_t* act;               // A bf16 [R, D]
  void* out;                   // O [R, H]
  int32_t* ctl;                // [0] queue head, [1] exit count, [2] error, [4 + t] parts done of L2 tile t
  int32_t* arrive;             // [i] L1 items done of global row block i
  float* part;                 // [tile][part] partial tiles of F_PART_FLOATS, laid out by thread
  int S;                       // K parts of a split L2 tile
  int row_blocks;              // arrival counters the workspace holds
  int tiles_cap;               // split only when the launch has at most this many L2 tiles
};

template <int ACT, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(F_NT) void fused_ffn_kernel(const FusedArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_mbp = (int32_t*)(smem + F_PIPE);  // row-block prefix per expert, kept for the whole launch
  int32_t* s_item = s_mbp + p.L + 1;            // the current item, then the last-out flag
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int L = p.L;
  int32_t* queue = p.ctl;
  int32_t* exits = p.ctl + 1;
  int32_t* err = p.ctl + 2;
  int32_t* arrive = p.arrive;
  int32_t* tile_done = p.ctl + 4;

  if (wave == 0) {
    const int per = (L + 63) / 64;
    const int e0 = lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < L) sum += (p.offsets[e + 1] - p.offsets[e] + F_BM - 1) / F_BM;
    }
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, MOE_WAVE);
      if (lane >= o) inc += v;
    }
    int run = inc - sum;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < L) {
        s_mbp[e] = run;
        run += (p.offsets[e + 1] - p.offsets[e] + F_BM - 1) / F_BM;
      }
    }
    if (lane == 63) s_mbp[L] = inc;
  }
  __syncthreads();
  // more rows than max_rows: no counter may be touched, so do nothing
  const bool too_many = s_mbp[L] > p.row_blocks;
  if (too_many && tid == 0 && blockIdx.x == 0) __hip_atomic_store(p.ctl + 2, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int total_mb = too_many ? 0 : s_mbp[L];
  const int NB1 = p.D / 128, NB2 = (p.H + F_BN - 1) / F_BN;
  const int n2 = total_mb * NB2;
  const int S = (p.S > 1 && n2 <= p.tiles_cap) ? p.S : 1;
  const int n1 = total_mb * NB1, n_all = n1 + n2 * S;
  const int fr = lane & 31, fh = lane >> 5;

  for (;;) {
    if (tid == 0) s_item[0] = atomicAdd(queue, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item[0]);
    if (item >= n_all) break;
    const bool l2 = item >= n1;
    const int NB = l2 ? NB2 * S : NB1;
    const int it = l2 ? item - n1 : item;
    int lo = 0, hi = L - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_mbp[mid] * NB <= it) lo = mid;
      else hi = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    const int nmb = s_mbp[e + 1] - s_mbp[e];
    const int local = __builtin_amdgcn_readfirstlane(it - s_mbp[e] * NB);
    const int q_nb = local / nmb, mb = local % nmb;
    const int nb = l2 ? q_nb / S : q_nb;
    const int part = l2 ? q_nb % S : 0;
    const int gm = s_mbp[e] + mb;  // global row block: its arrival counter
    const int row_beg = __builtin_amdgcn_readfirstlane(p.offsets[e] + mb * F_BM);
    const int row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);

    if (l2) {
      // one thread spins on the counter (relaxed: no cache invalidation per
      // poll), then acquires once; the barrier orders the other waves' loads
      // of A after that acquire
      if (tid == 0) {
        int spins = 0;
        while (__hip_atomic_load(arrive + gm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < NB1) {
          __builtin_amdgcn_s_sleep(8);
          if (++spins > F_SPIN_LIMIT) {
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
    }

    // ---- operands of this item
    const int K = l2 ? p.D : p.H;
    const int parts = l2 ? S : 1;
    const int kt0 = part * (K / F_BK) / parts;
    const int KT = (part + 1) * (K / F_BK) / parts - kt0;  // k stages of this item
    const uint16_t* a_base = l2 ? p.act : p.x;
    const uint16_t* b_base = l2 ? p.w_d + (int64_t)e * p.H * p.D : p.w_gu + (int64_t)e * 2 * p.D * p.H;
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, 0x7fffffff, F_BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, 0x7fffffff, F_BUF_DWORD3);
    // A: wave w loads tile rows 8w .. 8w+7 (1 KB = 8 rows x 8 chunks); rows
    // past the expert's end read zeros.  B: wave w loads rows 64w .. 64w+63.
    uint32_t a_voff, b_voff[F_LPW_B];
    {
      const int trow = wave * 8 + (lane >> 3);
      const int r = row_beg + trow;
      if (r < row_end) {
        const uint32_t ar = (!l2 && p.sorted_token) ? (uint32_t)p.sorted_token[r] : (uint32_t)r;
        a_voff = ar * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ f_swz(trow)) * 16);
      } else {
        a_voff = F_OOB;
      }
    }
#pragma unroll
    for (int i = 0; i < F_LPW_B; ++i) {
      const int trow = (wave * F_LPW_B + i) * 8 + (lane >> 3);
      int wrow;
      if (l2) {
        wrow = min(nb * F_BN + trow, p.H - 1);
      } else {
        // wave column q: 32 gate rows, then the matching 32 up rows
        const int q = trow / 64, rr = trow % 64, isup = rr / 32, j = rr % 32;
        const int oc = nb * 128 + q * 32 + j;
        wrow = (FMT == 0) ? (isup ? p.D + oc : oc) : (2 * oc + isup);
      }
      b_voff[i] = (uint32_t)wrow * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ f_swz(trow)) * 16);
    }
    auto issue = [&](int kt) {
      uint8_t* st = smem + (kt % F_NS) * F_STAGE;
      const int soff = (kt0 + kt) * F_ROW;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(st + wave_s * 1024), 16, a_voff, soff, 0, 0);
#pragma unroll
      for (int i = 0; i < F_LPW_B; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(st + F_A_BYTES + (wave_s * F_LPW_B + i) * 1024), 16,
                                                 b_voff[i], soff, 0, 0);
    };

    f32x16_t acc[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ni][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < F_NS - 1; ++i)
      if (i < KT) issue(i);
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + F_NS - 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm((F_NS - 2) * F_LOADS));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      f_block_barrier();
      if (kt + F_NS - 1 < KT) issue(kt + F_NS - 1);
      const uint8_t* st = smem + (kt % F_NS) * F_STAGE;
#pragma unroll
      for (int s = 0; s < F_BK / 16; ++s) {
        // k16 step s: lane half fh holds k [16s + 8fh, +8) = chunk 2s + fh
        const bf16x8_t af = *(const bf16x8_t*)(st + f_off(fr, 2 * s + fh));
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const bf16x8_t bf = *(const bf16x8_t*)(st + F_A_BYTES + f_off(wave * 64 + ni * 32 + fr, 2 * s + fh));
          acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc[ni], 0, 0, 0);
        }
      }
    }

    // ---- epilogue.  acc[ni][4q + c] is C[row][col], row = fr, col = wave*64 + ni*32 + 8q + 4fh + c
    const int row = row_beg + fr;
    if (!l2) {
      const float sc = p.s_gu ? p.s_gu[e] : 1.0f;
      const uint16_t* bias = p.b_gu ? p.b_gu + (int64_t)e * 2 * p.D : nullptr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int oc = nb * 128 + wave * 32 + 8 * q + 4 * fh;  // first of 4 outputs
        float bg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, bu[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias) {
          if (FMT == 0) {
            const uint2 g2 = *(const uint2*)(bias + oc), u2 = *(const uint2*)(bias + p.D + oc);
            bg[0] = bf16_to_f32(g2.x & 0xffffu); bg[1] = bf16_to_f32(g2.x >> 16);
            bg[2] = bf16_to_f32(g2.y & 0xffffu); bg[3] = bf16_to_f32(g2.y >> 16);
            bu[0] = bf16_to_f32(u2.x & 0xffffu); bu[1] = bf16_to_f32(u2.x >> 16);
            bu[2] = bf16_to_f32(u2.y & 0xffffu); bu[3] = bf16_to_f32(u2.y >> 16);
          } else {
            const u32x4_t b4 = *(const u32x4_t*)(bias + 2 * oc);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              bg[c] = bf16_to_f32(b4[c] & 0xffffu);
              bu[c] = bf16_to_f32(b4[c] >> 16);
            }
          }
        }
        if (row < row_end) {
          float a[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            a[c] = gated_act<ACT>(acc[0][4 * q + c] * sc + bg[c], acc[1][4 * q + c] * sc + bu[c], p.alpha, p.limit);
          uint2 v;
          v.x = pack_bf16x2_rne(a[0], a[1]);
          v.y = pack_bf16x2_rne(a[2], a[3]);
          *(uint2*)(p.act + (int64_t)row * p.D + oc) = v;
        }
      }
      // publish this part of the row block.  The barrier orders every
      // wave's A stores before thread 0's release fence, which writes them
      // back once for the workgroup; the count then moves.
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(arrive + gm, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      if (S > 1) {
        // this part's partial tile, then count it in; acc[j/4][4(j%4) + c]
        // goes to float 4(j*F_NT + tid) + c of the slot, the same place in
        // every part
        const int t2 = gm * NB2 + nb;
        float* slots = p.part + (int64_t)t2 * S * F_PART_FLOATS;
        float* mine = slots + (int64_t)part * F_PART_FLOATS;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f32x4_t v = {acc[j / 4][4 * (j % 4)], acc[j / 4][4 * (j % 4) + 1], acc[j / 4][4 * (j % 4) + 2],
                             acc[j / 4][4 * (j % 4) + 3]};
          *(f32x4_t*)(mine + 4 * (j * F_NT + tid)) = v;
        }
        // release as for A; the last part acquires the others' partials
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          const int done = __hip_atomic_fetch_add(tile_done + t2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_item[1] = done == S - 1;
          if (done == S - 1) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            // every part has counted in: reset for the next launch
            __hip_atomic_store(tile_done + t2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        __syncthreads();
        if (!s_item[1]) {
          __syncthreads();
          continue;
        }
        // sum the parts in part order
        f32x16_t sum[2];
        for (int pp = 0; pp < S; ++pp) {
          if (pp == part) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
              for (int r = 0; r < 16; ++r) sum[ni][r] = pp ? sum[ni][r] + acc[ni][r] : acc[ni][r];
          } else {
            const float* src = slots + (int64_t)pp * F_PART_FLOATS;
            f32x4_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = *(const f32x4_t*)(src + 4 * (j * F_NT + tid));
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
              for (int c = 0; c < 4; ++c)
                sum[j / 4][4 * (j % 4) + c] = pp ? sum[j / 4][4 * (j % 4) + c] + v[j][c] : v[j][c];
          }
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[ni] = sum[ni];
      }
      const float sc = p.s_d ? p.s_d[e] : 1.0f;
      const uint16_t* bias = p.b_d ? p.b_d + (int64_t)e * p.H : nullptr;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb * F_BN + wave * 64 + ni * 32 + 8 * q + 4 * fh;
          if (n >= p.H || row >= row_end) continue;
          float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (bias) {
            const uint2 b2 = *(const uint2*)(bias + n);
            bd[0] = bf16_to_f32(b2.x & 0xffffu); bd[1] = bf16_to_f32(b2.x >> 16);
            bd[2] = bf16_to_f32(b2.y & 0xffffu); bd[3] = bf16_to_f32(b2.y >> 16);
          }
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = acc[ni][4 * q + c] * sc + bd[c];
          if (OUT_BF16) {
            uint2 w;
            w.x = pack_bf16x2_rne(v[0], v[1]);
            w.y = pack_bf16x2_rne(v[2], v[3]);
            *(uint2*)((uint16_t*)p.out + (int64_t)row * p.H + n) = w;
          } else {
            const f32x4_t w = {v[0], v[1], v[2], v[3]};
            *(f32x4_t*)((float*)p.out + (int64_t)row * p.H + n) = w;
          }
        }
    }
    __syncthreads();  // the stage buffers and the item word are reused by the next item
  }

  // the last workgroup out leaves the control words at zero for the next launch
  if (tid == 0)
    s_item[1] = __hip_atomic_fetch_add(exits, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
  __syncthreads();
  if (s_item[1]) {
    for (int i = tid; i < total_mb; i += F_NT) __hip_atomic_store(arrive + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // (the split counters were reset by their last parts)
    if (tid == 0) {
      __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(exits, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int fused_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

template <typename KernelT>
hipError_t launch_fused_kernel(KernelT kern, const FusedArgs& a, hipStream_t st) {
  const int lds = F_PIPE + (a.L + 4) * (int)sizeof(int32_t);
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int grid = fused_cu_count();
  if (grid <= 0) return hipErrorInvalidDevice;
  kern<<<grid, F_NT, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_fused_act(const FusedArgs& a, int fmt, int out_bf16, hipStream_t st) {
  if (fmt == 0)
    return out_bf16 ? launch_fused_kernel(fused_ffn_kernel<ACT, 0, true>, a, st)
                    : launch_fused_kernel(fused_ffn_kernel<ACT, 0, false>, a, st);
  return out_bf16 ? launch_fused_kernel(fused_ffn_kernel<ACT, 1, true>, a, st)
                  : launch_fused_kernel(fused_ffn_kernel<ACT, 1, false>, a, st);
}

}  // namespace

FusedLayout fused_layout(int64_t max_rows, int H, int D, int L) {
  FusedLayout f{};
  auto up256 = [](int64_t b) { return (b + 255) / 256 * 256; };
  const int64_t R = max_rows < 0 ? 0 : max_rows;
  // at most one partly filled 32-row block per expert that has rows
  f.row_blocks = (R + F_BM - 1) / F_BM + (L < R ? L : R);
  // a part of K about twice an L1 item's: each part also pays a partial tile
  // write and its share of the reduction (measured on the Mixtral decode
  // shape, D/H = 3.5: 2 parts 0.61 ms, 4 parts 0.63, unsplit 0.65)
  int S = H > 0 ? (D + H) / (2 * H) : 1;
  S = S < 1 ? 1 : (S > F_MAX_PARTS ? F_MAX_PARTS : S);
  if (S > D / F_BK) S = D / F_BK;
  const int64_t tiles = f.row_blocks * ((H + F_BN - 1) / F_BN);
  f.tiles_cap = S > 1 ? (int)(tiles < F_MAX_TILES ? tiles : F_MAX_TILES) : 0;
  f.S = f.tiles_cap > 0 ? S : 1;
  f.act_off = up256(F_HDR_WORDS * 4);
  f.part_off = f.act_off + up256(R * D * 2);
  f.bytes = f.part_off + (int64_t)f.tiles_cap * f.S * F_PART_FLOATS * 4 + up256(f.row_blocks * 4);
  return f;
}

hipError_t launch_ffn_fused(const FfnBf16Params& q, void* ws, int64_t ws_bytes, hipStream_t st) {
  hipError_t err;
  const FusedLayout f = fused_layout(q.max_rows, q.H, q.D, q.L);
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
  FusedArgs a{};
  a.offsets = q.offsets;
  a.L = q.L;
  a.H = q.H;
  a.D = q.D;
  a.x = q.x_perm ? q.x_perm : q.x;
  a.sorted_token = q.x_perm ? nullptr : q.sorted_token;
  a.w_gu = q.w_gate_up;
  a.w_d = q.w_down;
  a.b_gu = q.b_gate_up;
  a.b_d = q.b_down;
  a.s_gu = q.gate_up_scales;
  a.s_d = q.down_scales;
  a.alpha = q.alpha;
  a.limit = q.limit;
  a.act = (uint16_t*)((uint8_t*)ws + f.act_off);
  a.out = q.out;
  a.ctl = (int32_t*)ws;
  a.arrive = (int32_t*)((uint8_t*)ws + (ws_bytes & ~(int64_t)3)) - f.row_blocks;
  a.part = (float*)((uint8_t*)ws + f.part_off);
  a.S = f.S;
  a.tiles_cap = f.tiles_cap;
  a.row_blocks = (int)f.row_blocks;
  if (q.act_kind == ACT_SILU) err = launch_fused_act<ACT_SILU>(a, q.fmt, q.out_bf16, st);
  else if (q.act_kind == ACT_SWIGLUOAI) err = launch_fused_act<ACT_SWIGLUOAI>(a, q.fmt, q.out_bf16, st);
  else err = launch_fused_act<ACT_GELU_TANH>(a, q.fmt, q.out_bf16, st);
  if (err != hipSuccess) return err;
  // one launch: the middle event is recorded with the last
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;
  if (q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
