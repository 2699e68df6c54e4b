// Grouped MX block-scaled expert GEMMs on gfx950: MXFP4 (E2M1) weights times
// MXFP8 (E4M3) activations, each with one E8M0 scale per 32 elements along K
// (StackedMoE page: MXFP4 weights run W4A8 with MXFP8 activations; the
// formats are those of the OCP Microscaling specification).  The scales go
// straight into v_mfma_scale_f32_32x32x64_f8f6f4, which applies them per 32
// K slots, so the main loop does no scale arithmetic at all.  The operand
// layout of that MFMA and the stage row formats are in mx_common.h.
//
// gate_up:  h = s_gu[e] * C + b_gu[e]; A = act(gate, up), re-quantised to
//           MXFP8 per row per 32 columns (shared exponent floor(log2 amax)-8,
//           unit scale for an all-zero block) -> codes + E8M0 scales, the
//           down GEMM's operand.
// down:     O = s_d[e] * C + b_d[e]  (bf16 or fp32 out)
//
// Tiling (batches of more than 32 rows per expert on average; smaller ones
// take the 32-row tiles further down): 256 x 256 workgroup tile, 8 waves in
// 2 x 4 (two per SIMD), each
// wave 128 x 64 = 4 x 2 MFMA blocks.  k stages of 128 go global -> LDS by
// buffer loads: the 32 KB of e4m3 activation rows (and their 4 scale bytes
// per row) double buffered by waves 0-3, the 16 KB of packed e2m1 weight
// rows (and theirs) four deep by waves 4-7.
#include "common.h"
#include "kernels.h"
#include "mx_common.h"
#include "mx_tile32.h"

namespace moe {

namespace {

enum { MX_GATE_UP = 0, MX_DOWN = 1 };

constexpr int X_BM = 256, X_BN = 256, X_BK = 128;         // BK in elements
constexpr int X_WAVES_M = 2, X_WAVES_N = 4;
constexpr int X_NT = 64 * X_WAVES_M * X_WAVES_N;           // 512 threads
constexpr int X_WTM = X_BM / X_WAVES_M, X_WTN = X_BN / X_WAVES_N;  // 128 x 64
constexpr int X_MI = X_WTM / 32, X_NI = X_WTN / 32;        // 4 x 2 MFMA blocks
static_assert(X_BK == MX_BK, "stage k of the MX row formats");
constexpr int X_A_ROW = MX_A_ROW;                          // bytes per e4m3 stage row
constexpr int X_B_ROW = MX_B_ROW;                          // bytes per packed e2m1 stage row
constexpr int X_A_BYTES = X_BM * X_A_ROW;                  // 32 KB
constexpr int X_B_BYTES = X_BN * X_B_ROW;                  // 16 KB
// LDS: activation slots of X_A_BYTES in a ring of 2, weight slots of
// X_B_BYTES in a ring of 4, then the scale dwords of the 256 activation rows
// and of the 256 weight rows in rings of 2 and 4 slots, each slot holding one
// group of up to 4 stages (16 bytes per row): 152 KB
constexpr int X_SC_SLOT = X_BM * 16;
constexpr int X_SC_A = 2 * X_A_BYTES + 4 * X_B_BYTES;
constexpr int X_SC_B = X_SC_A + 2 * X_SC_SLOT;
constexpr int X_LDS_PIPE = X_SC_B + 4 * X_SC_SLOT;
// the down epilogue stages its bf16 tile in LDS: rows of 512 bytes + 16 of
// bank skew (132 KB)
constexpr int X_LDS_OUT = X_BM * (X_BN * 2 + 16);
static_assert(X_LDS_OUT <= X_LDS_PIPE, "the staged output tile exceeds the pipeline's LDS");

constexpr int X_BUF_DWORD3 = 0x00020000;  // raw buffer resource word 3 (gfx9)
// A byte offset past every buffer's 0x7fffffff-byte range (also with a stage's
// k offset added): such a buffer load returns zeros without touching memory,
// and still counts as one load for the stage's vmcnt bookkeeping.
constexpr uint32_t X_OOB = 0x80000000u;


__device__ __forceinline__ void mx_block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct MxGemmArgs {
  const int32_t* offsets;
  int L;
  int K, N;                  // reduction length; output columns (gate_up D, down H)
  int fmt;                   // gate_up format (gate_up only)
  const uint8_t* A;          // e4m3 [rows, K] (or per token, gathered)
  const uint8_t* A_scale;    // E8M0 [rows, K/32]
  const int32_t* gather;     // row -> token, or nullptr
  const uint8_t* W;          // packed e2m1, OUT_IN per expert [w_rows, K/2]
  int64_t w_estride;         // bytes per expert
  const uint8_t* W_scale;    // E8M0 per expert [w_rows, K/32]
  int64_t ws_estride;        // bytes per expert
  const uint16_t* bias;      // bf16 per expert, or nullptr
  int64_t bias_estride;
  const float* escale;
  float alpha, limit;
  void* out;                 // gate_up: e4m3 [rows, D]; down: bf16 / fp32 [rows, H]
  uint8_t* out_scale;        // gate_up: E8M0 [rows, D/32]
};


struct MxTile {
  int e, nb, mb, row_beg, row_end;
};

// Maps this workgroup to its tile over the experts' BM-row blocks: the
// prefix of blocks per expert is built in LDS (wave 0), tiles are taken in
// expert-major, n-block, m-block order (m-blocks sharing a weight tile are
// neighbours), and each XCD (workgroups are dealt to the 8 XCDs round-robin)
// runs one contiguous range.  Called by the whole workgroup; false when the
// workgroup has no tile.  On return every wave has read the prefix, so the
// LDS may be overwritten.
template <int BM>
__device__ __forceinline__ bool mx_map_tile(const int32_t* offsets, int L, int NB, int32_t* s_mbp, MxTile& t) {
  const int wave = threadIdx.x >> 6;
  if (wave == 0) wave_expert_prefix(offsets, L, s_mbp, [](int rows) { return (rows + BM - 1) / BM; });
  __syncthreads();
  const int total = s_mbp[L] * NB;
  const int per_xcd = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return false;
  const int tile = (blockIdx.x & 7) * per_xcd + slot;
  if (tile >= total) return false;
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_mbp[mid] * NB <= tile) lo = mid;
    else hi = mid - 1;
  }
  t.e = __builtin_amdgcn_readfirstlane(lo);
  const int nmb = s_mbp[t.e + 1] - s_mbp[t.e];
  const int local = __builtin_amdgcn_readfirstlane(tile - s_mbp[t.e] * NB);
  t.nb = local / nmb;
  t.mb = local % nmb;
  t.row_beg = __builtin_amdgcn_readfirstlane(offsets[t.e] + t.mb * BM);
  t.row_end = __builtin_amdgcn_readfirstlane(offsets[t.e + 1]);
  __syncthreads();
  return true;
}

// Grid of a launch: enough workgroups for every tile whatever the split of
// max_rows over the experts (each non-empty expert adds at most one partial
// m-block), rounded to a multiple of the 8 XCDs.
inline int64_t mx_grid(int max_rows, int L, int BM, int N, int NBO) {
  const int64_t nonempty = (int64_t)max_rows < L ? max_rows : L;
  const int64_t mblocks = (max_rows + BM - 1) / BM + nonempty;
  const int64_t NB = (N + NBO - 1) / NBO;
  return ((mblocks * NB + 7) / 8) * 8;
}

template <int MODE, int ACT, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(X_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_mx_kernel(const MxGemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_mbp = (int32_t*)smem;  // m-block prefix, before the stage buffers are filled

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / X_WAVES_N, wn = wave % X_WAVES_N;
  constexpr int NBO = (MODE == MX_GATE_UP) ? X_BN / 2 : X_BN;  // output columns per tile
  const int NB = (p.N + NBO - 1) / NBO;
  MxTile t;
  if (!mx_map_tile<X_BM>(p.offsets, p.L, NB, s_mbp, t)) return;
  const int e = t.e, nb = t.nb, row_beg = t.row_beg, row_end = t.row_end;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm_s = wave_s / X_WAVES_N;
  const int KT = p.K / X_BK;        // K is a multiple of 128
  const uint32_t srow = (uint32_t)p.K / 32u;  // scale bytes per row

  // weight row of B tile row trow: wave column q owns 32 gate rows then the
  // matching 32 up rows (gate_up), or 64 consecutive rows (down)
  auto w_row = [&](int trow) {
    if (MODE == MX_DOWN) return min(nb * X_BN + trow, p.N - 1);
    const int q = trow / X_WTN, rr = trow % X_WTN, isup = rr / (X_WTN / 2), j = rr % (X_WTN / 2);
    const int oc = min(nb * NBO + q * (X_WTN / 2) + j, p.N - 1);
    return (FMT == 0) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
  };

  // ---- loader.  A: 1 KB = 8 rows x 8 chunks per instruction; B: 16 rows x
  // 4 chunks.  Per-lane offsets fixed for the tile, the k offset of a stage in
  // the scalar offset, the LDS destination in M0.  A rows past the expert's
  // last row read zeros; weight rows past N repeat the last one.  Neither
  // result is ever stored.
  // Loader roles: waves 0-3 fetch the activation rows (and their scales)
  // into a ring of 2 stages, waves 4-7 the weight rows (and theirs) into a
  // ring of 4.  A wave's vmcnt then counts one stream only, so the weight
  // stream keeps three stages in flight while the activations, re-read from
  // L2 by the neighbouring n-blocks, keep one.
  constexpr int A_SLOT = X_A_BYTES, B_SLOT = X_B_BYTES;
  constexpr int NA = 2, NB4 = 4, B_RING = NA * A_SLOT;
  constexpr int LB = X_B_BYTES / 1024 / 4;  // row loads per weight-role wave per stage
  // The scale dwords of G consecutive stages (G = 4 when the stage count
  // allows, else 1) come in one load per role wave: 16 contiguous bytes of
  // each row instead of 4 bytes of each row per stage, a quarter of the
  // cache lines.  Group g sits in scale slot g % 2 (activations) or g % 4
  // (weights), rows 4 G bytes apart.
  const int G = (KT % 4 == 0) ? 4 : 1;
  const bool a_role = wave_s < 4;
  const int rw = wave_s & 3;
  const uint8_t* Wexp = p.W + (int64_t)e * p.w_estride;
  const uint8_t* WSexp = p.W_scale + (int64_t)e * p.ws_estride;
  uint32_t voff[8];
  uint32_t s_voff;
  if (a_role) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int trow = (rw * 8 + i) * 8 + (lane >> 3);
      const int r = row_beg + trow;
      if (r < row_end) {
        const uint32_t ar = p.gather ? (uint32_t)p.gather[r] : (uint32_t)r;
        voff[i] = ar * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ mx_fa(trow)) * 16);
      } else {
        voff[i] = X_OOB;
      }
    }
    const int a_sr = min(row_beg + rw * 64 + lane, row_end - 1);
    s_voff = (p.gather ? (uint32_t)p.gather[a_sr] : (uint32_t)a_sr) * srow;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int trow = (rw * 4 + i) * 16 + (lane >> 2);
      voff[i] = (uint32_t)w_row(trow) * ((uint32_t)p.K / 2u) + (uint32_t)(((lane & 3) ^ mx_fb(trow)) * 16);
    }
#pragma unroll
    for (int i = 4; i < 8; ++i) voff[i] = 0;
    s_voff = (uint32_t)w_row(rw * 64 + lane) * srow;
  }
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, 0x7fffffff, X_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Wexp, (short)0, 0x7fffffff, X_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t as_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.A_scale, (short)0, 0x7fffffff, X_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t bs_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)WSexp, (short)0, 0x7fffffff, X_BUF_DWORD3);

  auto a_slot = [&](int kt) { return smem + (kt % NA) * A_SLOT; };
  auto b_slot = [&](int kt) { return smem + B_RING + (kt % NB4) * B_SLOT; };
  auto as_slot = [&](int kt) { return smem + X_SC_A + ((kt / G) % 2) * X_SC_SLOT; };
  auto bs_slot = [&](int kt) { return smem + X_SC_B + ((kt / G) % 4) * X_SC_SLOT; };
  // a stage's scale group first (when the stage starts one), then its rows
  auto issue_scales = [&](const __amdgpu_buffer_rsrc_t& rsrc, uint8_t* slot, int kt) {
    if (kt % G != 0) return;
    if (G == 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lptr_t)(slot + rw * 64 * 16), 16, s_voff, kt * 4, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lptr_t)(slot + rw * 64 * 4), 4, s_voff, kt * 4, 0, 0);
  };
  auto issue_a = [&](int kt) {
    issue_scales(as_rsrc, as_slot(kt), kt);
    uint8_t* st = a_slot(kt);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(st + (rw * 8 + i) * 1024), 16, voff[i], kt * X_A_ROW, 0, 0);
  };
  auto issue_b = [&](int kt) {
    issue_scales(bs_rsrc, bs_slot(kt), kt);
    uint8_t* st = b_slot(kt);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(st + (rw * 4 + i) * 1024), 16, voff[i], kt * X_B_ROW, 0, 0);
  };

  const int fr = lane & 31, fh = lane >> 5;
  f32x16_t acc[X_MI][X_NI];
#pragma unroll
  for (int mi = 0; mi < X_MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < X_NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int live_mi = min(max((row_end - (row_beg + wm_s * X_WTM) + 31) / 32, 0), X_MI);

  // ---- main loop.  Iteration kt: each role waits for its own loads of stage
  // kt (the weight waves leave stages kt+1 and kt+2 in flight: at least LB
  // loads each, one more where a stage starts a scale group), the barrier
  // publishes the stage, then the activation waves issue stage kt+1 into the
  // activation slot of stage kt-1 and the weight waves stage kt+3 into the
  // weight slot of stage kt-1 (both free: every wave has passed the barrier
  // after computing stage kt-1), and the stage's 16 MFMAs per wave run
  if (a_role) {
    issue_a(0);
  } else {
    issue_b(0);
    if (KT > 1) issue_b(1);
    if (KT > 2) issue_b(2);
  }
  for (int kt = 0; kt < KT; ++kt) {
    if (a_role || kt + 1 >= KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    else if (kt + 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LB));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(LB));
    mx_block_barrier();
    if (a_role) {
      if (kt + 1 < KT) issue_a(kt + 1);
    } else {
      if (kt + 3 < KT) issue_b(kt + 3);
    }
    const uint8_t* ast = a_slot(kt);
    const uint8_t* bst = b_slot(kt);
    // this stage's scale dword of row r: r * 4 G + (kt % G) * 4 in its group slot
    const uint8_t* as_l = as_slot(kt) + (kt % G) * 4;
    const uint8_t* bs_l = bs_slot(kt) + (kt % G) * 4;
    i32x8_t bq[X_NI][2];
    int bsc[X_NI][2];
#pragma unroll
    for (int ni = 0; ni < X_NI; ++ni) {
      const int row = wn * X_WTN + ni * 32 + fr;
      const uint32_t s4 = *(const uint32_t*)(bs_l + row * 4 * G);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bq[ni][kk] = mx_frag_b(bst, row, kk, fh);
        bsc[ni][kk] = (int)((s4 >> (8 * (2 * kk + fh))) & 0xffu);
      }
    }
#pragma unroll
    for (int mi = 0; mi < X_MI; ++mi) {
      if (mi < live_mi) {
        const int row = wm * X_WTM + mi * 32 + fr;
        const uint32_t s4 = *(const uint32_t*)(as_l + row * 4 * G);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const i32x8_t aq = mx_frag_a(ast, row, kk, fh);
          const int asc = (int)((s4 >> (8 * (2 * kk + fh))) & 0xffu);
#pragma unroll
          for (int ni = 0; ni < X_NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bq[ni][kk], aq, acc[mi][ni], 4, 0, 0,
                                                                          bsc[ni][kk], 0, asc);
        }
      }
    }
  }

  // ---- epilogue.  acc[mi][ni][4q + c] is C[row][col] with
  //   row = wm*128 + mi*32 + fr,  col = wn*64 + ni*32 + 8q + 4fh + c
  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if (MODE == MX_GATE_UP) {
    // block 0 holds the gate columns, block 1 the up columns of the wave's 32
    // outputs, which are one MX block of each row: the 16 values of a lane and
    // the 16 of lane xor 32
    uint8_t* out = (uint8_t*)p.out;
    float bg[4][4], bu[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int oc = nb * NBO + wn * 32 + 8 * q + 4 * fh;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bg[q][c] = 0.0f;
        bu[q][c] = 0.0f;
      }
      if (bias_e) {
        gate_up_bias_x4(bias_e, p.N, oc, FMT != 0, bg[q], bu[q]);
      }
    }
#pragma unroll
    for (int mi = 0; mi < X_MI; ++mi) {
      const int row = row_beg + wm * X_WTM + mi * 32 + fr;
      float a[16];
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        a[r] = gated_act<ACT>(acc[mi][0][r] * sc + bg[r / 4][r % 4], acc[mi][1][r] * sc + bu[r / 4][r % 4],
                              p.alpha, p.limit);
        m = fmaxf(m, fabsf(a[r]));
      }
      m = fmaxf(m, __shfl_xor(m, 32, MOE_WAVE));
      if (row >= row_end) continue;
      const int X = mx_shared_exp(m);
      const float inv = mx_inv_scale(X);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int oc = nb * NBO + wn * 32 + 8 * q + 4 * fh;
        *(uint32_t*)(out + (int64_t)row * p.N + oc) =
            e4m3x4(a[4 * q] * inv, a[4 * q + 1] * inv, a[4 * q + 2] * inv, a[4 * q + 3] * inv);
      }
      if (fh == 0) p.out_scale[(int64_t)row * (p.N / 32) + (nb * NBO + wn * 32) / 32] = (uint8_t)(X + 127);
    }
  } else if (OUT_BF16) {
    // The tile's bf16 outputs go through LDS (row pitch 528 bytes: 4 banks of
    // skew per row) so that each store moves whole 512-byte row pieces: a
    // lane's own accumulators cover 8 bytes of each of 16 rows, which as
    // direct stores would touch every output line 8 times.
    constexpr int PITCH = X_LDS_OUT / X_BM;
    __syncthreads();  // the stage buffers are free
#pragma unroll
    for (int ni = 0; ni < X_NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lc = wn * X_WTN + ni * 32 + 8 * q + 4 * fh;  // first of 4 tile columns
        const int n = nb * X_BN + lc;
        float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias_e && n < p.N) {
          bias_x4(bias_e + n, bd);
        }
#pragma unroll
        for (int mi = 0; mi < X_MI; ++mi) {
          const int lr = wm * X_WTM + mi * 32 + fr;
          uint2 w;
          w.x = pack_bf16x2_rne(acc[mi][ni][4 * q + 0] * sc + bd[0], acc[mi][ni][4 * q + 1] * sc + bd[1]);
          w.y = pack_bf16x2_rne(acc[mi][ni][4 * q + 2] * sc + bd[2], acc[mi][ni][4 * q + 3] * sc + bd[3]);
          *(uint2*)(smem + lr * PITCH + lc * 2) = w;
        }
      }
    __syncthreads();
    // 64 lanes store two rows of 32 x 16 bytes; wave w takes rows 32 w .. 32 w + 31
    const int cpart = lane & 31;
    const int n = nb * X_BN + cpart * 8;
#pragma unroll 4
    for (int j = 0; j < X_BM / (2 * X_WAVES_M * X_WAVES_N); ++j) {
      const int lr = wave * (X_BM / (X_WAVES_M * X_WAVES_N)) + 2 * j + (lane >> 5);
      const int row = row_beg + lr;
      if (row < row_end && n < p.N)
        *(u32x4_t*)((uint16_t*)p.out + (int64_t)row * p.N + n) = *(const u32x4_t*)(smem + lr * PITCH + cpart * 16);
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < X_NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb * X_BN + wn * X_WTN + ni * 32 + 8 * q + 4 * fh;  // first of 4 columns
        if (n >= p.N) continue;
        float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias_e) {
          bias_x4(bias_e + n, bd);
        }
#pragma unroll
        for (int mi = 0; mi < X_MI; ++mi) {
          const int row = row_beg + wm * X_WTM + mi * 32 + fr;
          if (row >= row_end) continue;
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = acc[mi][ni][4 * q + c] * sc + bd[c];
          if (OUT_BF16) {
            uint2 w;
            w.x = pack_bf16x2_rne(v[0], v[1]);
            w.y = pack_bf16x2_rne(v[2], v[3]);
            *(uint2*)((uint16_t*)p.out + (int64_t)row * p.N + n) = w;
          } else {
            const f32x4_t w = {v[0], v[1], v[2], v[3]};
            *(f32x4_t*)((float*)p.out + (int64_t)row * p.N + n) = w;
          }
        }
      }
  }
}

// ------------------------------------------------------------------ W4A16
// MXFP4 weights with bf16 activations: the weights are dequantised to bf16 in
// registers, per MFMA fragment, by v_cvt_scalef32_pk_bf16_fp4 (two E2M1 codes
// of a byte times an fp32 scale -> two bf16, exact for every E8M0 scale), and
// the product runs on v_mfma_f32_32x32x16_bf16.  Tile 128 x 256 (the format
// serves weight-bound batches first), 8 waves in 2 x 4, each 64 x 64 = 2 x 2
// MFMA blocks; k stages of 128 triple buffered in LDS: 32 KB of bf16 rows
// and 16 KB of packed e2m1 rows.  The weight rows' scale bytes (4 per row
// per stage) come four stages at a time where the stage count allows: 16
// contiguous bytes of each row instead of 4 bytes of each row per stage, a
// quarter of the cache lines (per stage they were as many lines as the
// weight codes).
//
// The k16 steps of a stage take k in the order mx_common.h gives for W4A16.
// Two shapes, both 3 stages deep: 128-row tiles with 8 waves (2 x 4), and,
// for batches of a few rows per expert (decode), 32-row tiles with 4 waves
// whose 75 KB of LDS let two workgroups share a CU.  Such a batch is bound by
// streaming the weights; with one 4-wave workgroup per CU each SIMD has a
// single wave, which serialises its LDS reads, conversions and MFMAs, and
// the second workgroup hides them (measured: 6 stages with one workgroup per
// CU, or 2 stages with three, were slower).
constexpr int W_BN = 256, W_BK = 128;
constexpr int W_A_ROW = W_BK * 2;                                   // bytes per bf16 stage row
constexpr int W_B_ROW = W_BK / 2;
constexpr int W_B_BYTES = W_BN * W_B_ROW;                           // 16 KB

template <int BM>
struct W4Shape {
  static constexpr int WAVES_M = BM >= 64 ? 2 : 1, WAVES_N = 4, NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NWAVES;
  static constexpr int NS = 3;                                       // stages
  static constexpr int WTM = BM / WAVES_M, WTN = W_BN / WAVES_N;    // wave tile, WTN = 64
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int A_BYTES = BM * W_A_ROW;
  static constexpr int STAGE = A_BYTES + W_B_BYTES;
  // scale slots after the stages: groups of 4 stages (16 bytes per row) in a
  // ring of 2, or single stages (4 bytes per row) in a ring of 3
  static constexpr int BS_OFF = NS * STAGE;
  static constexpr int LPW_A = A_BYTES / 1024 / NWAVES, LPW_B = W_B_BYTES / 1024 / NWAVES;
  static constexpr int BS_RPW = W_BN / NWAVES;                      // weight scale rows per wave
  static constexpr int LOADS = LPW_A + LPW_B;                       // row loads per wave per stage
  static constexpr int LDS = BS_OFF + 2 * W_BN * 16;
  static_assert(LPW_A >= 1 && LPW_B >= 1 && BS_RPW <= 64, "W4A16 tile shape");
  static_assert((NS - 2) * LOADS < 64, "vmcnt range");
  static_assert(BM != 32 || 2 * LDS <= 160 * 1024, "two 32-row workgroups share a CU");
};

static_assert(W_A_ROW == MX_A16_ROW, "the bf16 activation rows of mx_common.h");

struct W4GemmArgs {
  const int32_t* offsets;
  int L;
  int K, N;
  const uint16_t* A;         // bf16 [rows, K] (or per token, gathered)
  const int32_t* gather;
  const uint8_t* W;          // packed e2m1, OUT_IN per expert [w_rows, K/2]
  int64_t w_estride;
  const uint8_t* W_scale;    // E8M0 per expert [w_rows, K/32]
  int64_t ws_estride;
  const uint16_t* bias;
  int64_t bias_estride;
  const float* escale;
  float alpha, limit;
  void* out;                 // gate_up: bf16 [rows, D]; down: bf16 / fp32 [rows, H]
};


template <int MODE, int ACT, int FMT, bool OUT_BF16, int W_BM>
__global__ __launch_bounds__(W4Shape<W_BM>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_w4a16_kernel(const W4GemmArgs p) {
  constexpr int W_WAVES_N = W4Shape<W_BM>::WAVES_N, W_WTM = W4Shape<W_BM>::WTM, W_WTN = W4Shape<W_BM>::WTN;
  constexpr int W_MI = W4Shape<W_BM>::MI, W_NI = W4Shape<W_BM>::NI, W_NS = W4Shape<W_BM>::NS;
  constexpr int W_A_BYTES = W4Shape<W_BM>::A_BYTES, W_BS_OFF = W4Shape<W_BM>::BS_OFF, W_STAGE = W4Shape<W_BM>::STAGE;
  constexpr int W_LPW_A = W4Shape<W_BM>::LPW_A, W_LPW_B = W4Shape<W_BM>::LPW_B, W_LOADS = W4Shape<W_BM>::LOADS;
  constexpr int W_BS_RPW = W4Shape<W_BM>::BS_RPW;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / W_WAVES_N, wn = wave % W_WAVES_N;
  constexpr int NBO = (MODE == MX_GATE_UP) ? W_BN / 2 : W_BN;
  const int NB = (p.N + NBO - 1) / NBO;
  MxTile t;
  if (!mx_map_tile<W_BM>(p.offsets, p.L, NB, (int32_t*)smem, t)) return;
  const int e = t.e, nb = t.nb, row_beg = t.row_beg, row_end = t.row_end;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm_s = wave_s / W_WAVES_N;
  const int KT = p.K / W_BK;
  const uint32_t srow = (uint32_t)p.K / 32u;

  auto w_row = [&](int trow) {
    if (MODE == MX_DOWN) return min(nb * W_BN + trow, p.N - 1);
    const int q = trow / W_WTN, rr = trow % W_WTN, isup = rr / (W_WTN / 2), j = rr % (W_WTN / 2);
    const int oc = min(nb * NBO + q * (W_WTN / 2) + j, p.N - 1);
    return (FMT == 0) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
  };

  // ---- loader.  A: 1 KB = 4 rows x 16 chunks; B: 16 rows x 4 chunks; the
  // weight rows' scale dwords: lanes 0..31 of wave w, rows 32w + lane.
  const uint8_t* Wexp = p.W + (int64_t)e * p.w_estride;
  const uint8_t* WSexp = p.W_scale + (int64_t)e * p.ws_estride;
  // fixed-size arrays (the lambdas below capture them; an array whose size
  // depends on the template argument there stops clang from emitting the
  // kernel's host stub)
  static_assert(W_LPW_A <= 4 && W_LPW_B <= 4, "load counts");
  uint32_t a_voff[4], b_voff[4];
#pragma unroll
  for (int i = 0; i < W_LPW_A; ++i) {
    const int trow = (wave * W_LPW_A + i) * 4 + (lane >> 4);
    const int r = row_beg + trow;
    if (r < row_end) {
      const uint32_t ar = p.gather ? (uint32_t)p.gather[r] : (uint32_t)r;
      a_voff[i] = ar * (uint32_t)p.K * 2u + (uint32_t)(((lane & 15) ^ (trow & 15)) * 16);
    } else {
      a_voff[i] = X_OOB;   // past the expert's rows: reads zeros, moves no memory
    }
  }
#pragma unroll
  for (int i = 0; i < W_LPW_B; ++i) {
    const int trow = (wave * W_LPW_B + i) * 16 + (lane >> 2);
    b_voff[i] = (uint32_t)w_row(trow) * ((uint32_t)p.K / 2u) + (uint32_t)(((lane & 3) ^ mx_fb(trow)) * 16);
  }
  const uint32_t bs_voff = (uint32_t)w_row(wave * W_BS_RPW + lane % W_BS_RPW) * srow;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, 0x7fffffff, X_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Wexp, (short)0, 0x7fffffff, X_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t bs_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)WSexp, (short)0, 0x7fffffff, X_BUF_DWORD3);

  auto stage_base = [&](int kt) { return smem + (kt % W_NS) * W_STAGE; };
  const int G = (KT % 4 == 0) ? 4 : 1;
  auto bs_slot = [&](int kt) {
    return smem + W_BS_OFF + (G == 4 ? ((kt / 4) % 2) * (W_BN * 16) : (kt % W_NS) * (W_BN * 4));
  };
  auto issue = [&](int kt) {
    // the stage's scale group first (when it starts one), then its rows
    if (lane < W_BS_RPW && kt % G == 0) {
      if (G == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lptr_t)(bs_slot(kt) + wave_s * W_BS_RPW * 16), 16, bs_voff,
                                                 kt * 4, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lptr_t)(bs_slot(kt) + wave_s * W_BS_RPW * 4), 4, bs_voff,
                                                 kt * 4, 0, 0);
    }
    uint8_t* st = stage_base(kt);
#pragma unroll
    for (int i = 0; i < W_LPW_A; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(st + (wave_s * W_LPW_A + i) * 1024), 16, a_voff[i],
                                               kt * W_A_ROW, 0, 0);
#pragma unroll
    for (int i = 0; i < W_LPW_B; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(st + W_A_BYTES + (wave_s * W_LPW_B + i) * 1024), 16,
                                               b_voff[i], kt * W_B_ROW, 0, 0);
  };

  const int fr = lane & 31, fh = lane >> 5;
  f32x16_t acc[W_MI][W_NI];
#pragma unroll
  for (int mi = 0; mi < W_MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < W_NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
  const int live_mi = min(max((row_end - (row_beg + wm_s * W_WTM) + 31) / 32, 0), W_MI);

  // stages 0 .. NS-2 in the prologue; iteration kt waits for stage kt (at
  // most the NS-2 stages issued after it outstanding: at least W_LOADS row
  // loads each), publishes it, and issues stage kt+NS-1 into the buffer of
  // stage kt-1
#pragma unroll
  for (int i = 0; i < W_NS - 1; ++i)
    if (i < KT) issue(i);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + W_NS - 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm((W_NS - 2) * W_LOADS));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    mx_block_barrier();
    if (kt + W_NS - 1 < KT) issue(kt + W_NS - 1);
    const uint8_t* st = stage_base(kt);
    const uint8_t* bs_l = bs_slot(kt) + (kt % G) * 4;  // row r's scale dword at r * 4 G
#pragma unroll
    for (int half = 0; half < 2; ++half) {     // steps 4*half .. 4*half+3: one weight chunk, one MX block
      u32x4_t wq[W_NI];
      float wsc[W_NI];
#pragma unroll
      for (int ni = 0; ni < W_NI; ++ni) {
        const int row = wn * W_WTN + ni * 32 + fr;
        wq[ni] = *(const u32x4_t*)(st + W_A_BYTES + mx_b_off(row, 2 * fh + half));
        wsc[ni] = e8m0_f32((*(const uint32_t*)(bs_l + row * 4 * G) >> (8 * (2 * fh + half))) & 0xffu);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = 4 * half + j;
        bf16x8_t bw[W_NI];
#pragma unroll
        for (int ni = 0; ni < W_NI; ++ni) {
          const uint32_t d = wq[ni][j];
          const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 0);
          const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 1);
          const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 2);
          const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, wsc[ni], 3);
          bw[ni] = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        }
#pragma unroll
        for (int mi = 0; mi < W_MI; ++mi) {
          if (mi < live_mi) {
            const int row = wm * W_WTM + mi * 32 + fr;
            const bf16x8_t af = *(const bf16x8_t*)(st + mx_a16_off(row, 8 * fh + s));
#pragma unroll
            for (int ni = 0; ni < W_NI; ++ni)
              acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw[ni], af, acc[mi][ni], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue.  acc[mi][ni][4q + c] is C[row][col] with
  //   row = wm*64 + mi*32 + fr,  col = wn*64 + ni*32 + 8q + 4fh + c
  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if (MODE == MX_GATE_UP) {
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int oc = nb * NBO + wn * 32 + 8 * q + 4 * fh;  // first of 4 outputs
      float bg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, bu[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (bias_e) {
        gate_up_bias_x4(bias_e, p.N, oc, FMT != 0, bg, bu);
      }
#pragma unroll
      for (int mi = 0; mi < W_MI; ++mi) {
        const int row = row_beg + wm * W_WTM + mi * 32 + fr;
        if (row >= row_end) continue;
        float a[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          a[c] = gated_act<ACT>(acc[mi][0][4 * q + c] * sc + bg[c], acc[mi][1][4 * q + c] * sc + bu[c], p.alpha,
                                p.limit);
        uint2 v;
        v.x = pack_bf16x2_rne(a[0], a[1]);
        v.y = pack_bf16x2_rne(a[2], a[3]);
        *(uint2*)(out + (int64_t)row * p.N + oc) = v;
      }
    }
  } else {
    // The tile's outputs go through LDS (rows of 256 outputs plus 16 bytes
    // of bank skew) so that each store moves whole rows: a lane's own
    // accumulators cover 4 columns of each of its rows, which as direct
    // stores would touch every output line 8 or 16 times.
    constexpr int ES = OUT_BF16 ? 2 : 4;
    constexpr int PITCH = W_BN * ES + 16;
    static_assert(W_BM * PITCH <= W4Shape<W_BM>::LDS, "staged output tile exceeds LDS");
    __syncthreads();  // the stage buffers are free
#pragma unroll
    for (int ni = 0; ni < W_NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lc = wn * W_WTN + ni * 32 + 8 * q + 4 * fh;  // first of 4 tile columns
        const int n = nb * W_BN + lc;
        float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias_e && n < p.N) {
          bias_x4(bias_e + n, bd);
        }
#pragma unroll
        for (int mi = 0; mi < W_MI; ++mi) {
          uint8_t* dst = smem + (wm * W_WTM + mi * 32 + fr) * PITCH + lc * ES;
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = acc[mi][ni][4 * q + c] * sc + bd[c];
          if (OUT_BF16) {
            uint2 w;
            w.x = pack_bf16x2_rne(v[0], v[1]);
            w.y = pack_bf16x2_rne(v[2], v[3]);
            *(uint2*)dst = w;
          } else {
            *(f32x4_t*)dst = f32x4_t{v[0], v[1], v[2], v[3]};
          }
        }
      }
    __syncthreads();
    // a row is W_BN * ES bytes: 32 (bf16) or 64 (fp32) lanes of 16 bytes
    constexpr int LPR = W_BN * ES / 16, RPI = 64 / LPR;  // lanes per row, rows per store
    constexpr int NWAVES = W4Shape<W_BM>::NWAVES;
    const int cpart = lane % LPR;
    const int n = nb * W_BN + cpart * (16 / ES);
    for (int r = wave * RPI + lane / LPR; r < W_BM; r += NWAVES * RPI) {
      const int row = row_beg + r;
      if (row < row_end && n < p.N)
        *(u32x4_t*)((uint8_t*)p.out + ((int64_t)row * p.N + n) * ES) = *(const u32x4_t*)(smem + r * PITCH + cpart * 16);
    }
  }
}

template <int BM, typename KernelT>
hipError_t launch_w4(KernelT kern, const W4GemmArgs& a, int max_rows, int NBO, hipStream_t st) {
  const int prefix = (a.L + 1) * (int)sizeof(int32_t);
  const int lds = W4Shape<BM>::LDS > prefix ? W4Shape<BM>::LDS : prefix;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t grid = mx_grid(max_rows, a.L, BM, a.N, NBO);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, W4Shape<BM>::NT, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT, int BM>
hipError_t launch_w4_gate_up(const W4GemmArgs& g, int fmt, int max_rows, hipStream_t st) {
  if (fmt == 0)
    return launch_w4<BM>(grouped_gemm_w4a16_kernel<MX_GATE_UP, ACT, 0, true, BM>, g, max_rows, W_BN / 2, st);
  return launch_w4<BM>(grouped_gemm_w4a16_kernel<MX_GATE_UP, ACT, 1, true, BM>, g, max_rows, W_BN / 2, st);
}

template <typename KernelT>
hipError_t launch_mx(KernelT kern, const MxGemmArgs& a, int max_rows, int NBO, hipStream_t st) {
  const int prefix = (a.L + 1) * (int)sizeof(int32_t);
  const int lds = X_LDS_PIPE > prefix ? X_LDS_PIPE : prefix;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t grid = mx_grid(max_rows, a.L, X_BM, a.N, NBO);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, X_NT, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_mx_gate_up(const MxGemmArgs& g, int fmt, int max_rows, hipStream_t st) {
  if (fmt == 0) return launch_mx(grouped_gemm_mx_kernel<MX_GATE_UP, ACT, 0, false>, g, max_rows, X_BN / 2, st);
  return launch_mx(grouped_gemm_mx_kernel<MX_GATE_UP, ACT, 1, false>, g, max_rows, X_BN / 2, st);
}

// ------------------------------------------------------------------ W4A8, 32-row tiles
// For batches of a few rows per expert (decode) the 256-row tiles above are
// mostly empty.  These GEMMs run the 32 x 256 tile of mx_tile32.h instead
// (4 waves, 69 KB of LDS, two workgroups per CU), with the same MFMA
// sequence per output element and the same epilogue arithmetic as the
// 256-row kernels, so their results are bit-identical.
template <int MODE, int ACT, int FMT, bool OUT_BF16>
__global__ __launch_bounds__(T32_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_mx32_kernel(const MxGemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NBO = (MODE == MX_GATE_UP) ? T32_BN / 2 : T32_BN;  // output columns per tile
  const int NB = (p.N + NBO - 1) / NBO;
  MxTile t;
  if (!mx_map_tile<T32_BM>(p.offsets, p.L, NB, (int32_t*)smem, t)) return;
  const int e = t.e, nb = t.nb;
  Mx32Operands o;
  o.a = p.A;
  o.a_scale = p.A_scale;
  o.gather = p.gather;
  o.w = p.W + (int64_t)e * p.w_estride;
  o.w_scale = p.W_scale + (int64_t)e * p.ws_estride;
  o.K = p.K;
  o.row_beg = t.row_beg;
  o.row_end = t.row_end;
  o.kt0 = 0;
  o.KT = p.K / MX_BK;
  // weight row of tile row trow: wave column q owns 32 gate rows then the
  // matching 32 up rows (gate_up), or 64 consecutive rows (down)
  auto w_row = [&](int trow) -> int {
    if (MODE == MX_DOWN) return min(nb * T32_BN + trow, p.N - 1);
    const int q = trow / 64, rr = trow % 64, isup = rr / 32, j = rr % 32;
    const int oc = min(nb * NBO + q * 32 + j, p.N - 1);
    return (FMT == 0) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
  };
  f32x16_t acc[2];
  mx32_tile_loop(o, w_row, smem, acc);
  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if (MODE == MX_GATE_UP)
    mx32_store_a_mxfp8<ACT>(acc, sc, bias_e, p.N, FMT != 0, p.alpha, p.limit, nb, t.row_beg, t.row_end,
                            (uint8_t*)p.out, p.out_scale, smem);
  else
    mx32_store_o_tile<OUT_BF16>(acc, sc, bias_e, p.N, nb, t.row_beg, t.row_end, p.out, smem);
}

template <typename KernelT>
hipError_t launch_mx32(KernelT kern, const MxGemmArgs& a, int max_rows, int NBO, hipStream_t st) {
  const int prefix = (a.L + 1) * (int)sizeof(int32_t);
  const int lds = T32_PIPE > prefix ? T32_PIPE : prefix;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t grid = mx_grid(max_rows, a.L, T32_BM, a.N, NBO);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, T32_NT, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT>
hipError_t launch_mx32_gate_up(const MxGemmArgs& g, int fmt, int max_rows, hipStream_t st) {
  if (fmt == 0) return launch_mx32(grouped_gemm_mx32_kernel<MX_GATE_UP, ACT, 0, false>, g, max_rows, T32_BN / 2, st);
  return launch_mx32(grouped_gemm_mx32_kernel<MX_GATE_UP, ACT, 1, false>, g, max_rows, T32_BN / 2, st);
}

template <int BM>
hipError_t launch_ffn_w4a16_bm(const FfnMxParams& q, hipStream_t st) {
  hipError_t err;
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
  W4GemmArgs g{};
  g.offsets = q.offsets;
  g.L = q.L;
  g.K = q.H;
  g.N = q.D;
  g.A = (const uint16_t*)q.x_perm;
  g.gather = q.sorted_token;
  g.W = q.w_gate_up;
  g.w_estride = (int64_t)2 * q.D * (q.H / 2);
  g.W_scale = q.w_gate_up_scale;
  g.ws_estride = (int64_t)2 * q.D * (q.H / 32);
  g.bias = q.b_gate_up;
  g.bias_estride = (int64_t)2 * q.D;
  g.escale = q.gate_up_scales;
  g.alpha = q.alpha;
  g.limit = q.limit;
  g.out = q.act;
  if (q.act_kind == ACT_SILU) err = launch_w4_gate_up<ACT_SILU, BM>(g, q.fmt, q.max_rows, st);
  else if (q.act_kind == ACT_SWIGLUOAI) err = launch_w4_gate_up<ACT_SWIGLUOAI, BM>(g, q.fmt, q.max_rows, st);
  else err = launch_w4_gate_up<ACT_GELU_TANH, BM>(g, q.fmt, q.max_rows, st);
  if (err != hipSuccess) return err;
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;
  W4GemmArgs d{};
  d.offsets = q.offsets;
  d.L = q.L;
  d.K = q.D;
  d.N = q.H;
  d.A = (const uint16_t*)q.act;
  d.W = q.w_down;
  d.w_estride = (int64_t)q.H * (q.D / 2);
  d.W_scale = q.w_down_scale;
  d.ws_estride = (int64_t)q.H * (q.D / 32);
  d.bias = q.b_down;
  d.bias_estride = q.H;
  d.escale = q.down_scales;
  d.out = q.out;
  if (q.out_bf16)
    err = launch_w4<BM>(grouped_gemm_w4a16_kernel<MX_DOWN, ACT_SILU, 0, true, BM>, d, q.max_rows, W_BN, st);
  else
    err = launch_w4<BM>(grouped_gemm_w4a16_kernel<MX_DOWN, ACT_SILU, 0, false, BM>, d, q.max_rows, W_BN, st);
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace

// 32-row tiles when the batch averages at most 32 rows per expert
hipError_t launch_ffn_w4a16(const FfnMxParams& q, hipStream_t st) {
  if ((int64_t)q.max_rows <= (int64_t)32 * q.L) return launch_ffn_w4a16_bm<32>(q, st);
  return launch_ffn_w4a16_bm<128>(q, st);
}

// 32-row tiles when the batch averages at most 32 rows per expert
hipError_t launch_ffn_mx(const FfnMxParams& q, hipStream_t st) {
  hipError_t err;
  const bool small = (int64_t)q.max_rows <= (int64_t)32 * q.L;
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
  MxGemmArgs g{};
  g.offsets = q.offsets;
  g.L = q.L;
  g.K = q.H;
  g.N = q.D;
  g.fmt = q.fmt;
  g.A = q.x_perm;
  g.A_scale = q.x_scale;
  g.gather = q.sorted_token;
  g.W = q.w_gate_up;
  g.w_estride = (int64_t)2 * q.D * (q.H / 2);
  g.W_scale = q.w_gate_up_scale;
  g.ws_estride = (int64_t)2 * q.D * (q.H / 32);
  g.bias = q.b_gate_up;
  g.bias_estride = (int64_t)2 * q.D;
  g.escale = q.gate_up_scales;
  g.alpha = q.alpha;
  g.limit = q.limit;
  g.out = q.act;
  g.out_scale = q.act_scale;
  if (q.act_kind == ACT_SILU)
    err = small ? launch_mx32_gate_up<ACT_SILU>(g, q.fmt, q.max_rows, st)
                : launch_mx_gate_up<ACT_SILU>(g, q.fmt, q.max_rows, st);
  else if (q.act_kind == ACT_SWIGLUOAI)
    err = small ? launch_mx32_gate_up<ACT_SWIGLUOAI>(g, q.fmt, q.max_rows, st)
                : launch_mx_gate_up<ACT_SWIGLUOAI>(g, q.fmt, q.max_rows, st);
  else
    err = small ? launch_mx32_gate_up<ACT_GELU_TANH>(g, q.fmt, q.max_rows, st)
                : launch_mx_gate_up<ACT_GELU_TANH>(g, q.fmt, q.max_rows, st);
  if (err != hipSuccess) return err;
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;
  MxGemmArgs d{};
  d.offsets = q.offsets;
  d.L = q.L;
  d.K = q.D;
  d.N = q.H;
  d.A = q.act;
  d.A_scale = q.act_scale;
  d.W = q.w_down;
  d.w_estride = (int64_t)q.H * (q.D / 2);
  d.W_scale = q.w_down_scale;
  d.ws_estride = (int64_t)q.H * (q.D / 32);
  d.bias = q.b_down;
  d.bias_estride = q.H;
  d.escale = q.down_scales;
  d.out = q.out;
  if (small)
    err = q.out_bf16 ? launch_mx32(grouped_gemm_mx32_kernel<MX_DOWN, ACT_SILU, 0, true>, d, q.max_rows, T32_BN, st)
                     : launch_mx32(grouped_gemm_mx32_kernel<MX_DOWN, ACT_SILU, 0, false>, d, q.max_rows, T32_BN, st);
  else if (q.out_bf16)
    err = launch_mx(grouped_gemm_mx_kernel<MX_DOWN, ACT_SILU, 0, true>, d, q.max_rows, X_BN, st);
  else
    err = launch_mx(grouped_gemm_mx_kernel<MX_DOWN, ACT_SILU, 0, false>, d, q.max_rows, X_BN, st);
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
