// Single-launch expert FFN for small batches: the gate_up grouped GEMM with
// the gated activation (L1) and the down GEMM (L2) in one launch, pipelined
// across workgroups (mega_ffn page: one launch that fuses the L1 and L2 legs,
// cross-workgroup arrival counters, no per-launch memset).
//
// A persistent grid (one or two workgroups per CU) takes work items from one atomic
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
// Visibility follows the HIP memory model at agent scope: after an L1 item's
// A stores, a workgroup barrier and a release fence (write-back of the XCD's
// L2) precede the counter increment; an L2 item acquires the counter and
// fence-acquires (invalidate) before loading A, whichever XCD either ran on.
// One fence publishes up to F_PUB L1 items of a workgroup at once; a
// workgroup publishes what it holds before it waits or leaves.  The last
// workgroup to leave resets the queue, the exit count and the arrival
// counters, so the control words start at zero on the next launch; the
// caller zeroes them once, when the workspace is allocated.
//
// Tiles are 32 x 256 with 4 waves (32 x 64 each: the gate and up columns of
// 32 outputs for L1).  Three operand kinds share the schedule, the tile and
// the epilogue arithmetic:
//   bf16:   k stages of 64 bf16, 4 stages deep in LDS through buffer loads,
//           one workgroup per CU;
//   W4A8:   MXFP4 weights x MXFP8 activations (the mega_ffn page's
//           block-scaled form), k stages of 128 on the scaled MFMA, 3 deep,
//           two workgroups per CU; L1 re-quantises A to MXFP8 before L2
//           reads it;
//   W4A16:  MXFP4 weights dequantised in registers x bf16 activations,
//           k stages of 128 on the bf16 MFMA, two workgroups per CU.
// Every kind is bound by streaming the weights.
#include "common.h"
#include "kernels.h"
#include "mx_common.h"
#include "mx_tile32.h"

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
constexpr int F_PUB = 4;                            // L1 items published per release fence
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

// ---------------------------------------------------------------- schedule
// Shared by both kernels: 256 threads, 32-row blocks.

// Prefix of 32-row blocks per expert into s_mbp[0 .. L] (wave 0), then a
// barrier.
__device__ __forceinline__ void fused_block_prefix(const int32_t* offsets, int L, int32_t* s_mbp) {
  if ((threadIdx.x >> 6) == 0) wave_expert_prefix(offsets, L, s_mbp, [](int rows) { return (rows + F_BM - 1) / F_BM; });
  __syncthreads();
}

struct FusedItem {
  bool l2;
  int e, nb, part;
  int gm;                // global row block: its arrival counter
  int row_beg, row_end;
};

// Work item `item` of the queue: first the n1 L1 items (expert, row block,
// one of NB1 blocks of 128 outputs), then the L2 items (expert, row block,
// one of NB2 blocks of 256 outputs, one of S parts of K); within an expert,
// output-block-major.  Every field is wave-uniform.
__device__ __forceinline__ FusedItem fused_item(int item, int n1, int NB1, int NB2, int S, int L,
                                                const int32_t* s_mbp, const int32_t* offsets) {
  FusedItem t;
  t.l2 = item >= n1;
  const int NB = t.l2 ? NB2 * S : NB1;
  const int it = t.l2 ? item - n1 : item;
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_mbp[mid] * NB <= it) lo = mid;
    else hi = mid - 1;
  }
  t.e = __builtin_amdgcn_readfirstlane(lo);
  const int nmb = s_mbp[t.e + 1] - s_mbp[t.e];
  const int local = __builtin_amdgcn_readfirstlane(it - s_mbp[t.e] * NB);
  const int q_nb = local / nmb, mb = local % nmb;
  t.nb = t.l2 ? q_nb / S : q_nb;
  t.part = t.l2 ? q_nb % S : 0;
  t.gm = s_mbp[t.e] + mb;
  t.row_beg = __builtin_amdgcn_readfirstlane(offsets[t.e] + mb * F_BM);
  t.row_end = __builtin_amdgcn_readfirstlane(offsets[t.e + 1]);
  return t;
}

// Waits until `counter` reaches `need`: one thread spins on it (relaxed: no
// cache invalidation per poll), then acquires once; the barrier orders the
// other waves' loads after that acquire.  The spin is bounded: on timeout it
// sets the error word and goes on.
__device__ __forceinline__ void fused_wait(const int32_t* counter, int need, int32_t* err) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
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

// L1 publication.  One release fence covers the A stores of up to F_PUB
// L1 items of a workgroup: thread 0 keeps their row blocks in s_pend
// ([0] the count, then the blocks) and counts them in together when the list
// is full, and before the workgroup takes an L2 item or leaves.  So a
// workgroup that waits holds nothing unpublished: every L1 item is published
// by a workgroup that does not wait, and each wait still ends.  (The fence
// writes back the XCD's whole L2; one per item cost up to 0.1 ms per launch.)
//
// Publishes the list (thread 0 only: no other thread reads it).
__device__ __forceinline__ void fused_flush0(int32_t* arrive, int32_t* s_pend) {
  if (s_pend[0] > 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    for (int i = 1; i <= s_pend[0]; ++i)
      __hip_atomic_fetch_add(arrive + s_pend[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_pend[0] = 0;
  }
}

// Called by every thread after a barrier that follows the stores (each
// wave's barrier waits for its own stores first).
__device__ __forceinline__ void fused_flush(int32_t* arrive, int32_t* s_pend) {
  if (threadIdx.x == 0) fused_flush0(arrive, s_pend);
}

// An L1 item's A stores are done: its row block joins the list, and a full
// list is published.
__device__ __forceinline__ void fused_count_in(int32_t* arrive, int gm, int32_t* s_pend) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n = s_pend[0] + 1;
    s_pend[n] = gm;
    s_pend[0] = n;
    if (n == F_PUB) fused_flush0(arrive, s_pend);
  }
}

// One part of a split L2 tile: writes the part's fp32 partial tile to its
// slot (acc[j/4][4(j%4) + c] goes to float 4(j*F_NT + tid) + c, the same
// place in every part) and counts it in at `done`.  The workgroup whose part
// comes last resets the counter for the next launch, adds the S parts in
// part order (its own from registers) into acc and returns true; the others
// return false.  No part waits for another.
__device__ __forceinline__ bool fused_split_reduce(f32x16_t (&acc)[2], float* slots, int part, int S, int32_t* done,
                                                   int32_t* s_flag) {
  const int tid = threadIdx.x;
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
    const int n = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[0] = n == S - 1;
    if (n == S - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // every part has counted in: reset for the next launch
      __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!s_flag[0]) return false;
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
  return true;
}

// The last workgroup out leaves the control words at zero for the next
// launch (the split counters were reset by their last parts).
__device__ __forceinline__ void fused_exit(int32_t* ctl, int32_t* arrive, int total_mb, int32_t* s_flag) {
  const int tid = threadIdx.x;
  if (tid == 0)
    s_flag[0] = __hip_atomic_fetch_add(ctl + 1, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
  __syncthreads();
  if (s_flag[0]) {
    for (int i = tid; i < total_mb; i += F_NT) __hip_atomic_store(arrive + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(ctl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctl + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------- bf16
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
  int max_rows;                // rows the A and O buffers hold
  int row_blocks;              // arrival counters the workspace holds
  int tiles_cap;               // split only when the launch has at most this many L2 tiles
};

template <int ACT, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(F_NT) void fused_ffn_kernel(const FusedArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_mbp = (int32_t*)(smem + F_PIPE);  // row-block prefix per expert, kept for the whole launch
  int32_t* s_item = s_mbp + p.L + 1;            // the current item, then the last-out flag
  int32_t* s_pend = s_item + 2;                 // L1 row blocks not yet published
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int L = p.L;
  int32_t* queue = p.ctl;
  int32_t* err = p.ctl + 2;
  int32_t* arrive = p.arrive;
  int32_t* tile_done = p.ctl + 4;

  if (tid == 0) s_pend[0] = 0;
  fused_block_prefix(p.offsets, L, s_mbp);
  // more rows than max_rows: neither A, O nor a counter may be touched, so do
  // nothing (at most max_rows rows also bound the row blocks by row_blocks)
  const bool too_many = p.offsets[L] > p.max_rows || s_mbp[L] > p.row_blocks;
  if (too_many && tid == 0 && blockIdx.x == 0) __hip_atomic_store(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    if (item >= n1) fused_flush(p.arrive, s_pend);  // before any wait, and before leaving
    if (item >= n_all) break;
    const FusedItem t = fused_item(item, n1, NB1, NB2, S, L, s_mbp, p.offsets);
    const bool l2 = t.l2;
    const int e = t.e, nb = t.nb, part = t.part, gm = t.gm, row_beg = t.row_beg, row_end = t.row_end;
    if (l2) fused_wait(arrive + gm, NB1, err);

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
          gate_up_bias_x4(bias, p.D, oc, FMT != 0, bg, bu);
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
      fused_count_in(arrive, gm, s_pend);  // this part of the row block is done
    } else {
      if (S > 1) {
        const int t2 = gm * NB2 + nb;
        if (!fused_split_reduce(acc, p.part + (int64_t)t2 * S * F_PART_FLOATS, part, S, tile_done + t2, s_item + 1)) {
          __syncthreads();
          continue;
        }
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
            bias_x4(bias + n, bd);
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

  fused_exit(p.ctl, arrive, total_mb, s_item + 1);
}

// ---------------------------------------------------------------- W4A8
// MXFP4 weights x MXFP8 activations on the 32 x 256 tile of mx_tile32.h, two
// workgroups per CU.
constexpr int M_WG_PER_CU = 2;
static_assert(T32_BM == F_BM && T32_BN == F_BN && T32_NT == F_NT, "the W4A8 tile is the schedule's tile");
static_assert(M_WG_PER_CU * (T32_PIPE + (1024 + 4) * 4) <= 160 * 1024, "two W4A8 workgroups share a CU");

struct FusedMxArgs {
  const int32_t* offsets;
  int L, H, D;
  const uint8_t* x;            // e4m3 [T, H] gathered through sorted_token, or [R, H] rows (sorted_token null)
  const uint8_t* x_scale;      // E8M0 [T or R, H/32]
  const int32_t* sorted_token;
  const uint8_t* w_gu;         // packed e2m1 OUT_IN [L, 2D, H/2]
  const uint8_t* w_gu_scale;   // E8M0 [L, 2D, H/32]
  const uint8_t* w_d;          // packed e2m1 OUT_IN [L, H, D/2]
  const uint8_t* w_d_scale;    // E8M0 [L, H, D/32]
  const uint16_t* b_gu;        // [L, 2D] or null
  const uint16_t* b_d;         // [L, H] or null
  const float* s_gu;           // [L] or null
  const float* s_d;
  float alpha, limit;
  uint8_t* act;                // A, e4m3 codes [R, D]
  uint8_t* act_scale;          // A, E8M0 [R, D/32]
  void* out;                   // O [R, H]
  int32_t* ctl;                // as FusedArgs
  int32_t* arrive;
  float* part;
  int S, max_rows, row_blocks, tiles_cap;
};

template <int ACT, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(F_NT) void fused_ffn_mx_kernel(const FusedMxArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_mbp = (int32_t*)(smem + T32_PIPE);  // row-block prefix per expert, kept for the whole launch
  int32_t* s_item = s_mbp + p.L + 1;            // the current item, then the last-part / last-out flag
  int32_t* s_pend = s_item + 2;                 // L1 row blocks not yet published
  const int tid = threadIdx.x;
  const int L = p.L;
  int32_t* err = p.ctl + 2;
  int32_t* tile_done = p.ctl + 4;

  if (tid == 0) s_pend[0] = 0;
  fused_block_prefix(p.offsets, L, s_mbp);
  // more rows than max_rows: do nothing (as the bf16 kernel)
  const bool too_many = p.offsets[L] > p.max_rows || s_mbp[L] > p.row_blocks;
  if (too_many && tid == 0 && blockIdx.x == 0) __hip_atomic_store(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int total_mb = too_many ? 0 : s_mbp[L];
  const int NB1 = p.D / 128, NB2 = (p.H + F_BN - 1) / F_BN;
  const int n2 = total_mb * NB2;
  const int S = (p.S > 1 && n2 <= p.tiles_cap) ? p.S : 1;
  const int n1 = total_mb * NB1, n_all = n1 + n2 * S;

  for (;;) {
    if (tid == 0) s_item[0] = atomicAdd(p.ctl, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item[0]);
    if (item >= n1) fused_flush(p.arrive, s_pend);  // before any wait, and before leaving
    if (item >= n_all) break;
    const FusedItem t = fused_item(item, n1, NB1, NB2, S, L, s_mbp, p.offsets);
    const bool l2 = t.l2;
    const int e = t.e, nb = t.nb, part = t.part, gm = t.gm, row_beg = t.row_beg, row_end = t.row_end;
    if (l2) fused_wait(p.arrive + gm, NB1, err);

    // ---- operands of this item: k stages kt0 .. kt0+KT-1 of the whole row
    const int K = l2 ? p.D : p.H;
    const int KS = K / MX_BK;
    const int parts = l2 ? S : 1;
    const int kt0 = part * KS / parts;
    const int KT = (part + 1) * KS / parts - kt0;
    Mx32Operands o;
    o.a = l2 ? p.act : p.x;
    o.a_scale = l2 ? p.act_scale : p.x_scale;
    o.gather = l2 ? nullptr : p.sorted_token;
    o.w = l2 ? p.w_d + (int64_t)e * p.H * (p.D / 2) : p.w_gu + (int64_t)e * 2 * p.D * (p.H / 2);
    o.w_scale = l2 ? p.w_d_scale + (int64_t)e * p.H * (p.D / 32) : p.w_gu_scale + (int64_t)e * 2 * p.D * (p.H / 32);
    o.K = K;
    o.row_beg = row_beg;
    o.row_end = row_end;
    o.kt0 = kt0;
    o.KT = KT;
    // weight row of tile row trow: L1 wave column q holds 32 gate rows, then
    // the matching 32 up rows; L2 256 consecutive rows (past H: the last)
    auto w_row = [&](int trow) -> int {
      if (l2) return min(nb * F_BN + trow, p.H - 1);
      const int q = trow / 64, rr = trow % 64, isup = rr / 32, j = rr % 32;
      const int oc = nb * 128 + q * 32 + j;
      return (FMT == 0) ? (isup ? p.D + oc : oc) : (2 * oc + isup);
    };
    f32x16_t acc[2];
    mx32_tile_loop(o, w_row, smem, acc);

    // ---- epilogue
    if (!l2) {
      mx32_store_a_mxfp8<ACT>(acc, p.s_gu ? p.s_gu[e] : 1.0f, p.b_gu ? p.b_gu + (int64_t)e * 2 * p.D : nullptr, p.D,
                              FMT != 0, p.alpha, p.limit, nb, row_beg, row_end, p.act, p.act_scale, smem);
      fused_count_in(p.arrive, gm, s_pend);  // this part of the row block is done
    } else {
      if (S > 1) {
        const int t2 = gm * NB2 + nb;
        if (!fused_split_reduce(acc, p.part + (int64_t)t2 * S * F_PART_FLOATS, part, S, tile_done + t2, s_item + 1)) {
          __syncthreads();
          continue;
        }
      }
      mx32_store_o_tile<OUT_BF16>(acc, p.s_d ? p.s_d[e] : 1.0f, p.b_d ? p.b_d + (int64_t)e * p.H : nullptr, p.H, nb,
                                  row_beg, row_end, p.out, smem);
    }
    __syncthreads();  // the stage buffers and the item word are reused by the next item
  }

  fused_exit(p.ctl, p.arrive, total_mb, s_item + 1);
}

// ---------------------------------------------------------------- W4A16
// MXFP4 weights x bf16 activations: the weights are dequantised to bf16 in
// registers per fragment (v_cvt_scalef32_pk_bf16_fp4, exact for every E8M0
// scale) and multiplied on v_mfma_f32_32x32x16_bf16, in the k order of the
// two-launch W4A16 GEMMs (mx_common.h); A stays bf16.  A k stage of 128:
// 8 KB of bf16 activation rows and 16 KB of packed e2m1 weight rows.  Two
// workgroups share a CU with two activation slots beside three weight slots
// (64 KB, plus the weight rows' scale dwords): each iteration issues the
// next stage's activations and then the weight stage after that, so the
// wait for a stage (loads retire in order per wave) leaves the next weight
// stage in flight.
constexpr int V_A_BYTES = F_BM * MX_A16_ROW;             // 8 KB
constexpr int V_B_BYTES = F_BN * MX_B_ROW;               // 16 KB
constexpr int V_NA = 2, V_NB = 3;                        // activation and weight slots
constexpr int V_LPW_A = V_A_BYTES / 1024 / F_NW;         // 1 KB loads per wave per stage: 2
constexpr int V_LPW_B = V_B_BYTES / 1024 / F_NW;         // 4
constexpr int V_B_OFF = V_NA * V_A_BYTES;
constexpr int V_BS_OFF = V_B_OFF + V_NB * V_B_BYTES;     // weight scales: 2 slots x 256 rows x 16 bytes
constexpr int V_PIPE = V_BS_OFF + 2 * F_BN * 16;         // 72 KB
constexpr int V_APITCH = 128 * 2 + 16;                   // staged A rows: 128 bf16 + bank skew
static_assert(V_NB * F_BN * 4 <= 2 * F_BN * 16, "single-stage scale slots fit");
static_assert(V_LPW_B < 64, "vmcnt range");
static_assert(M_WG_PER_CU * (V_PIPE + (1024 + 4) * 4) <= 160 * 1024, "two W4A16 workgroups share a CU");
static_assert(F_BM * V_APITCH <= V_BS_OFF, "staged A rows fit the stages");
static_assert(F_BM * (F_BN * 4 + 16) <= V_BS_OFF, "a staged fp32 output tile fits the stages");

struct FusedW4Args {
  const int32_t* offsets;
  int L, H, D;
  const uint16_t* x;           // bf16 [T, H] gathered through sorted_token, or [R, H] rows (sorted_token null)
  const int32_t* sorted_token;
  const uint8_t* w_gu;         // packed e2m1 OUT_IN [L, 2D, H/2]
  const uint8_t* w_gu_scale;   // E8M0 [L, 2D, H/32]
  const uint8_t* w_d;          // packed e2m1 OUT_IN [L, H, D/2]
  const uint8_t* w_d_scale;    // E8M0 [L, H, D/32]
  const uint16_t* b_gu;        // [L, 2D] or null
  const uint16_t* b_d;         // [L, H] or null
  const float* s_gu;           // [L] or null
  const float* s_d;
  float alpha, limit;
  uint16_t* act;               // A bf16 [R, D]
  void* out;                   // O [R, H]
  int32_t* ctl;                // as FusedArgs
  int32_t* arrive;
  float* part;
  int S, max_rows, row_blocks, tiles_cap;
};

template <int ACT, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(F_NT) void fused_ffn_w4a16_kernel(const FusedW4Args p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_mbp = (int32_t*)(smem + V_PIPE);  // row-block prefix per expert, kept for the whole launch
  int32_t* s_item = s_mbp + p.L + 1;            // the current item, then the last-part / last-out flag
  int32_t* s_pend = s_item + 2;                 // L1 row blocks not yet published
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int L = p.L;
  int32_t* err = p.ctl + 2;
  int32_t* tile_done = p.ctl + 4;

  if (tid == 0) s_pend[0] = 0;
  fused_block_prefix(p.offsets, L, s_mbp);
  // more rows than max_rows: do nothing (as the bf16 kernel)
  const bool too_many = p.offsets[L] > p.max_rows || s_mbp[L] > p.row_blocks;
  if (too_many && tid == 0 && blockIdx.x == 0) __hip_atomic_store(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int total_mb = too_many ? 0 : s_mbp[L];
  const int NB1 = p.D / 128, NB2 = (p.H + F_BN - 1) / F_BN;
  const int n2 = total_mb * NB2;
  const int S = (p.S > 1 && n2 <= p.tiles_cap) ? p.S : 1;
  const int n1 = total_mb * NB1, n_all = n1 + n2 * S;
  const int fr = lane & 31, fh = lane >> 5;

  for (;;) {
    if (tid == 0) s_item[0] = atomicAdd(p.ctl, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item[0]);
    if (item >= n1) fused_flush(p.arrive, s_pend);  // before any wait, and before leaving
    if (item >= n_all) break;
    const FusedItem t = fused_item(item, n1, NB1, NB2, S, L, s_mbp, p.offsets);
    const bool l2 = t.l2;
    const int e = t.e, nb = t.nb, part = t.part, gm = t.gm, row_beg = t.row_beg, row_end = t.row_end;
    if (l2) fused_wait(p.arrive + gm, NB1, err);

    // ---- operands of this item.  K stages ks = kt0 + kt of the whole row.
    const int K = l2 ? p.D : p.H;
    const int KS = K / MX_BK;
    const int parts = l2 ? S : 1;
    const int kt0 = part * KS / parts;
    const int KT = (part + 1) * KS / parts - kt0;
    const int G = (KS % 4 == 0 && kt0 % 4 == 0 && KT % 4 == 0) ? 4 : 1;
    const uint32_t srow = (uint32_t)K / 32u;
    const int32_t* gather = l2 ? nullptr : p.sorted_token;
    const uint16_t* a_base = l2 ? p.act : p.x;
    const uint8_t* b_base = l2 ? p.w_d + (int64_t)e * p.H * (p.D / 2) : p.w_gu + (int64_t)e * 2 * p.D * (p.H / 2);
    const uint8_t* bs_base =
        l2 ? p.w_d_scale + (int64_t)e * p.H * (p.D / 32) : p.w_gu_scale + (int64_t)e * 2 * p.D * (p.H / 32);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, 0x7fffffff, F_BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, 0x7fffffff, F_BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t bs_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)bs_base, (short)0, 0x7fffffff, F_BUF_DWORD3);
    auto w_row = [&](int trow) -> int {
      if (l2) return min(nb * F_BN + trow, p.H - 1);
      const int q = trow / 64, rr = trow % 64, isup = rr / 32, j = rr % 32;
      const int oc = nb * 128 + q * 32 + j;
      return (FMT == 0) ? (isup ? p.D + oc : oc) : (2 * oc + isup);
    };
    // A: wave w loads tile rows 8w .. 8w+7 as two 1 KB loads of 4 rows x 16
    // chunks (rows past the expert's end read zeros).  B: rows 64w .. 64w+63
    // (16 rows x 4 chunks per 1 KB) and their scale dwords, one row per lane.
    uint32_t a_voff[V_LPW_A], b_voff[V_LPW_B], bs_voff;
#pragma unroll
    for (int i = 0; i < V_LPW_A; ++i) {
      const int trow = (wave * V_LPW_A + i) * 4 + (lane >> 4);
      const int r = row_beg + trow;
      if (r < row_end) {
        const uint32_t ar = gather ? (uint32_t)gather[r] : (uint32_t)r;
        a_voff[i] = ar * (uint32_t)K * 2u + (uint32_t)(((lane & 15) ^ (trow & 15)) * 16);
      } else {
        a_voff[i] = F_OOB;
      }
    }
#pragma unroll
    for (int i = 0; i < V_LPW_B; ++i) {
      const int trow = (wave * V_LPW_B + i) * 16 + (lane >> 2);
      b_voff[i] = (uint32_t)w_row(trow) * ((uint32_t)K / 2u) + (uint32_t)(((lane & 3) ^ mx_fb(trow)) * 16);
    }
    bs_voff = (uint32_t)w_row(wave * 64 + lane) * srow;

    auto a_slot = [&](int kt) { return smem + (kt % V_NA) * V_A_BYTES; };
    auto b_slot = [&](int kt) { return smem + V_B_OFF + (kt % V_NB) * V_B_BYTES; };
    // scale group g = kt / 4 in slot g % 2 (rows 16 bytes apart), or stage
    // kt in slot kt % 3 (rows 4 bytes apart)
    auto bs_slot = [&](int kt) {
      return smem + V_BS_OFF + (G == 4 ? ((kt / 4) % 2) * (F_BN * 16) : (kt % V_NB) * (F_BN * 4));
    };
    auto issue_a = [&](int kt) {
#pragma unroll
      for (int i = 0; i < V_LPW_A; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(a_slot(kt) + (wave_s * V_LPW_A + i) * 1024), 16,
                                                 a_voff[i], (kt0 + kt) * MX_A16_ROW, 0, 0);
    };
    auto issue_b = [&](int kt) {
      const int ks = kt0 + kt;
      // the stage's scale group first (when it starts one), then its rows
      if (kt % G == 0) {
        if (G == 4)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lptr_t)(bs_slot(kt) + wave_s * 64 * 16), 16, bs_voff,
                                                   ks * 4, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lptr_t)(bs_slot(kt) + wave_s * 64 * 4), 4, bs_voff,
                                                   ks * 4, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < V_LPW_B; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(b_slot(kt) + (wave_s * V_LPW_B + i) * 1024), 16,
                                                 b_voff[i], ks * MX_B_ROW, 0, 0);
    };

    f32x16_t acc[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ni][r] = 0.0f;
    // Load order per wave: B(0), A(0), B(1), then per iteration kt: A(kt+1),
    // B(kt+2).  Iteration kt needs A(kt) and B(kt); only B(kt+1), issued
    // after A(kt), may still be in flight (its V_LPW_B row loads last).
    // A(kt+1) goes into the activation slot of stage kt-1 and B(kt+2) into
    // its weight slot, both free once every wave has passed iteration kt's
    // barrier.
    issue_b(0);
    issue_a(0);
    if (KT > 1) issue_b(1);
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(V_LPW_B));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      f_block_barrier();
      if (kt + 1 < KT) issue_a(kt + 1);
      if (kt + 2 < KT) issue_b(kt + 2);
      const uint8_t* ast = a_slot(kt);
      const uint8_t* bst = b_slot(kt);
      const uint8_t* bs_l = bs_slot(kt) + (kt % G) * 4;  // row r's scale dword at r * 4 G
#pragma unroll
      for (int half = 0; half < 2; ++half) {  // steps 4*half .. 4*half+3: one weight chunk, one MX block
        u32x4_t wq[2];
        float wsc[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int row = wave * 64 + ni * 32 + fr;
          wq[ni] = *(const u32x4_t*)(bst + mx_b_off(row, 2 * fh + half));
          wsc[ni] = e8m0_f32((*(const uint32_t*)(bs_l + row * 4 * G) >> (8 * (2 * fh + half))) & 0xffu);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int st = 4 * half + j;
          const bf16x8_t af = *(const bf16x8_t*)(ast + mx_a16_off(fr, 8 * fh + st));
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const uint32_t d = wq[ni][j];
            const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 0);
            const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 1);
            const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 2);
            const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 3);
            const bf16x8_t bw = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
            acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, af, acc[ni], 0, 0, 0);
          }
        }
      }
    }

    // ---- epilogue.  acc[ni][4q + c] is C[row][col], row = fr, col = wave*64 + ni*32 + 8q + 4fh + c
    if (!l2) {
      // block 0 holds the gate columns, block 1 the up columns of the wave's
      // 32 outputs; A in bf16, staged in LDS and stored as whole row pieces
      const float sc = p.s_gu ? p.s_gu[e] : 1.0f;
      const uint16_t* bias = p.b_gu ? p.b_gu + (int64_t)e * 2 * p.D : nullptr;
      __syncthreads();  // the stage buffers are free
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lc = wave * 32 + 8 * q + 4 * fh;  // first of 4 of the tile's 128 outputs
        float bg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, bu[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias) gate_up_bias_x4(bias, p.D, nb * 128 + lc, FMT != 0, bg, bu);
        float a[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          a[c] = gated_act<ACT>(acc[0][4 * q + c] * sc + bg[c], acc[1][4 * q + c] * sc + bu[c], p.alpha, p.limit);
        uint2 v;
        v.x = pack_bf16x2_rne(a[0], a[1]);
        v.y = pack_bf16x2_rne(a[2], a[3]);
        *(uint2*)(smem + fr * V_APITCH + lc * 2) = v;
      }
      __syncthreads();
      // 32 rows x 16 pieces of 16 bytes
      for (int i = tid; i < F_BM * 16; i += F_NT) {
        const int r = i >> 4, pc = i & 15;
        if (row_beg + r < row_end)
          *(u32x4_t*)(p.act + (int64_t)(row_beg + r) * p.D + nb * 128 + pc * 8) =
              *(const u32x4_t*)(smem + r * V_APITCH + pc * 16);
      }
      fused_count_in(p.arrive, gm, s_pend);  // this part of the row block is done
    } else {
      if (S > 1) {
        const int t2 = gm * NB2 + nb;
        if (!fused_split_reduce(acc, p.part + (int64_t)t2 * S * F_PART_FLOATS, part, S, tile_done + t2, s_item + 1)) {
          __syncthreads();
          continue;
        }
      }
      mx32_store_o_tile<OUT_BF16>(acc, p.s_d ? p.s_d[e] : 1.0f, p.b_d ? p.b_d + (int64_t)e * p.H : nullptr, p.H, nb,
                                  row_beg, row_end, p.out, smem);
    }
    __syncthreads();  // the stage buffers and the item word are reused by the next item
  }

  fused_exit(p.ctl, p.arrive, total_mb, s_item + 1);
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
  const int lds = F_PIPE + (a.L + 4 + F_PUB) * (int)sizeof(int32_t);
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

template <typename KernelT>
hipError_t launch_fused_mx_kernel(KernelT kern, const FusedMxArgs& a, hipStream_t st) {
  const int lds = T32_PIPE + (a.L + 4 + F_PUB) * (int)sizeof(int32_t);
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int grid = M_WG_PER_CU * fused_cu_count();
  if (grid <= 0) return hipErrorInvalidDevice;
  kern<<<grid, F_NT, lds, st>>>(a);
  return hipGetLastError();
}

template <typename KernelT>
hipError_t launch_fused_w4_kernel(KernelT kern, const FusedW4Args& a, hipStream_t st) {
  const int lds = V_PIPE + (a.L + 4 + F_PUB) * (int)sizeof(int32_t);
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int grid = M_WG_PER_CU * fused_cu_count();
  if (grid <= 0) return hipErrorInvalidDevice;
  kern<<<grid, F_NT, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_fused_w4_act(const FusedW4Args& a, int fmt, int out_bf16, hipStream_t st) {
  if (fmt == 0)
    return out_bf16 ? launch_fused_w4_kernel(fused_ffn_w4a16_kernel<ACT, 0, true>, a, st)
                    : launch_fused_w4_kernel(fused_ffn_w4a16_kernel<ACT, 0, false>, a, st);
  return out_bf16 ? launch_fused_w4_kernel(fused_ffn_w4a16_kernel<ACT, 1, true>, a, st)
                  : launch_fused_w4_kernel(fused_ffn_w4a16_kernel<ACT, 1, false>, a, st);
}

template <int ACT>
hipError_t launch_fused_mx_act(const FusedMxArgs& a, int fmt, int out_bf16, hipStream_t st) {
  if (fmt == 0)
    return out_bf16 ? launch_fused_mx_kernel(fused_ffn_mx_kernel<ACT, 0, true>, a, st)
                    : launch_fused_mx_kernel(fused_ffn_mx_kernel<ACT, 0, false>, a, st);
  return out_bf16 ? launch_fused_mx_kernel(fused_ffn_mx_kernel<ACT, 1, true>, a, st)
                  : launch_fused_mx_kernel(fused_ffn_mx_kernel<ACT, 1, false>, a, st);
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
  // A: bf16 [R, D], or MXFP8 codes [R, D] followed by the scale bytes [R, D/32]
  f.act_scale_off = f.act_off + up256(R * D);
  const int64_t act_bf16 = up256(R * D * 2), act_mx = up256(R * D) + up256(R * (D / 32));
  const int64_t act_bytes = act_bf16 > act_mx ? act_bf16 : act_mx;
  f.part_off = f.act_off + act_bytes;
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
  a.max_rows = q.max_rows;
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

hipError_t launch_ffn_fused_mx(const FfnMxParams& q, void* ws, int64_t ws_bytes, hipStream_t st) {
  hipError_t err;
  const FusedLayout f = fused_layout(q.max_rows, q.H, q.D, q.L);
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
  FusedMxArgs a{};
  a.offsets = q.offsets;
  a.L = q.L;
  a.H = q.H;
  a.D = q.D;
  a.x = q.x_perm;
  a.x_scale = q.x_scale;
  a.sorted_token = q.sorted_token;
  a.w_gu = q.w_gate_up;
  a.w_gu_scale = q.w_gate_up_scale;
  a.w_d = q.w_down;
  a.w_d_scale = q.w_down_scale;
  a.b_gu = q.b_gate_up;
  a.b_d = q.b_down;
  a.s_gu = q.gate_up_scales;
  a.s_d = q.down_scales;
  a.alpha = q.alpha;
  a.limit = q.limit;
  a.act = (uint8_t*)ws + f.act_off;
  a.act_scale = (uint8_t*)ws + f.act_scale_off;
  a.out = q.out;
  a.ctl = (int32_t*)ws;
  a.arrive = (int32_t*)((uint8_t*)ws + (ws_bytes & ~(int64_t)3)) - f.row_blocks;
  a.part = (float*)((uint8_t*)ws + f.part_off);
  a.S = f.S;
  a.tiles_cap = f.tiles_cap;
  a.max_rows = q.max_rows;
  a.row_blocks = (int)f.row_blocks;
  if (q.act_kind == ACT_SILU) err = launch_fused_mx_act<ACT_SILU>(a, q.fmt, q.out_bf16, st);
  else if (q.act_kind == ACT_SWIGLUOAI) err = launch_fused_mx_act<ACT_SWIGLUOAI>(a, q.fmt, q.out_bf16, st);
  else err = launch_fused_mx_act<ACT_GELU_TANH>(a, q.fmt, q.out_bf16, st);
  if (err != hipSuccess) return err;
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;
  if (q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

hipError_t launch_ffn_fused_w4a16(const FfnMxParams& q, void* ws, int64_t ws_bytes, hipStream_t st) {
  hipError_t err;
  const FusedLayout f = fused_layout(q.max_rows, q.H, q.D, q.L);
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
  FusedW4Args a{};
  a.offsets = q.offsets;
  a.L = q.L;
  a.H = q.H;
  a.D = q.D;
  a.x = (const uint16_t*)q.x_perm;
  a.sorted_token = q.sorted_token;
  a.w_gu = q.w_gate_up;
  a.w_gu_scale = q.w_gate_up_scale;
  a.w_d = q.w_down;
  a.w_d_scale = q.w_down_scale;
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
  a.max_rows = q.max_rows;
  a.row_blocks = (int)f.row_blocks;
  if (q.act_kind == ACT_SILU) err = launch_fused_w4_act<ACT_SILU>(a, q.fmt, q.out_bf16, st);
  else if (q.act_kind == ACT_SWIGLUOAI) err = launch_fused_w4_act<ACT_SWIGLUOAI>(a, q.fmt, q.out_bf16, st);
  else err = launch_fused_w4_act<ACT_GELU_TANH>(a, q.fmt, q.out_bf16, st);
  if (err != hipSuccess) return err;
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;
  if (q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
