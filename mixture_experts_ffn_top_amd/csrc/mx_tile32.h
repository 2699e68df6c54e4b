// One 32 x 256 tile of the MXFP4 x MXFP8 (W4A8) product for batches of a few
// rows per expert, shared by the single-launch FFN and the 32-row grouped
// GEMMs: 4 waves of 32 x 64 (in gate_up, the gate and up columns of 32
// outputs), k stages of 128 on v_mfma_scale_f32_32x32x64_f8f6f4 (the operand
// layout of mx_common.h).  A stage is 4 KB of e4m3 activation rows and 16 KB
// of packed e2m1 weight rows, 3 deep, plus the rows' scale dwords, which come
// four stages per 16-byte load where the stages allow (else one stage per
// 4-byte load).  With 69 KB of LDS two workgroups share a CU, so each SIMD
// holds a second wave that covers the first one's LDS reads and MFMAs while
// both wait on the weight stream.
#pragma once

#include "common.h"
#include "mx_common.h"

namespace moe {

constexpr int T32_BM = 32, T32_BN = 256, T32_NW = 4, T32_NT = 64 * T32_NW;
constexpr int T32_NS = 3;
constexpr int T32_A_BYTES = T32_BM * MX_A_ROW;            // 4 KB
constexpr int T32_B_BYTES = T32_BN * MX_B_ROW;            // 16 KB
constexpr int T32_STAGE = T32_A_BYTES + T32_B_BYTES;
constexpr int T32_LPW_B = T32_B_BYTES / 1024 / T32_NW;    // 1 KB weight row loads per wave per stage: 4
constexpr int T32_LOADS = 1 + T32_LPW_B;                  // row loads per wave per stage
constexpr int T32_AS_OFF = T32_NS * T32_STAGE;            // activation scales: 2 slots x 32 rows x 16 bytes
constexpr int T32_BS_OFF = T32_AS_OFF + 2 * T32_BM * 16;  // weight scales: 2 slots x 256 rows x 16 bytes
constexpr int T32_PIPE = T32_BS_OFF + 2 * T32_BN * 16;    // 69 KB
constexpr int T32_CPITCH = 128 + 16;                      // staged A codes: 128 bytes per row + bank skew
constexpr int T32_BUF_DWORD3 = 0x00020000;                // raw buffer resource word 3 (gfx9)
constexpr uint32_t T32_OOB = 0x80000000u;                 // past every buffer range: zeros, no memory
static_assert(T32_NS * T32_BM * 4 <= 2 * T32_BM * 16 && T32_NS * T32_BN * 4 <= 2 * T32_BN * 16,
              "single-stage scale slots fit");
static_assert((T32_NS - 2) * T32_LOADS < 64, "vmcnt range");
static_assert(T32_BM * T32_CPITCH + T32_BM * 4 <= T32_NS * T32_STAGE, "staged A codes and scales fit the stages");
static_assert(T32_BM * (T32_BN * 4 + 16) <= T32_NS * T32_STAGE, "a staged fp32 output tile fits the stages");

// The operands of one tile.  A rows row_beg .. row_beg+31 (those at or past
// row_end read zeros) are rows gather[r] (or r) of a and a_scale; w and
// w_scale are one expert's packed weights [w_rows, K/2] and E8M0 scales
// [w_rows, K/32].  The tile contracts k stages kt0 .. kt0+KT-1 of K/128.
struct Mx32Operands {
  const uint8_t* a;
  const uint8_t* a_scale;
  const int32_t* gather;
  const uint8_t* w;
  const uint8_t* w_scale;
  int K, row_beg, row_end, kt0, KT;
};

__device__ __forceinline__ void t32_block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// acc[ni][4q + c] = C[fr][wave*64 + ni*32 + 8q + 4fh + c] of the tile, fr =
// lane & 31, fh = lane >> 5; w_row(trow) is the weight row of tile row trow.
// Called by the whole workgroup; the LDS pipeline is free on entry and on
// return (every load has landed and been read).
template <typename WRow>
__device__ __forceinline__ void mx32_tile_loop(const Mx32Operands& o, WRow w_row, uint8_t* smem, f32x16_t (&acc)[2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int fr = lane & 31, fh = lane >> 5;
  const int K = o.K, KS = K / MX_BK, kt0 = o.kt0, KT = o.KT;
  // scale groups of 4 stages: 16-byte aligned rows (KS % 4 == 0) and whole
  // groups inside these stages
  const int G = (KS % 4 == 0 && kt0 % 4 == 0 && KT % 4 == 0) ? 4 : 1;
  const uint32_t srow = (uint32_t)K / 32u;  // scale bytes per row
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)o.a, (short)0, 0x7fffffff, T32_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t as_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)o.a_scale, (short)0, 0x7fffffff, T32_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)o.w, (short)0, 0x7fffffff, T32_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t bs_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)o.w_scale, (short)0, 0x7fffffff, T32_BUF_DWORD3);
  // A: wave w loads tile rows 8w .. 8w+7 (1 KB = 8 rows x 8 chunks; rows
  // past the end read zeros) and, by lanes 0-7, their scale dwords (rows
  // past the end repeat the last one; never used).  B: wave w loads rows
  // 64w .. 64w+63 (16 rows x 4 chunks per 1 KB) and their scale dwords, one
  // row per lane.
  uint32_t a_voff, as_voff, b_voff[T32_LPW_B], bs_voff;
  {
    const int trow = wave * 8 + (lane >> 3);
    const int r = o.row_beg + trow;
    if (r < o.row_end) {
      const uint32_t ar = o.gather ? (uint32_t)o.gather[r] : (uint32_t)r;
      a_voff = ar * (uint32_t)K + (uint32_t)(((lane & 7) ^ mx_fa(trow)) * 16);
    } else {
      a_voff = T32_OOB;
    }
    const int sr = min(o.row_beg + wave * 8 + (lane & 7), o.row_end - 1);
    as_voff = (o.gather ? (uint32_t)o.gather[sr] : (uint32_t)sr) * srow;
  }
#pragma unroll
  for (int i = 0; i < T32_LPW_B; ++i) {
    const int trow = (wave * T32_LPW_B + i) * 16 + (lane >> 2);
    b_voff[i] = (uint32_t)w_row(trow) * ((uint32_t)K / 2u) + (uint32_t)(((lane & 3) ^ mx_fb(trow)) * 16);
  }
  bs_voff = (uint32_t)w_row(wave * 64 + lane) * srow;

  // scale group g = kt / 4 in slot g % 2 (rows 16 bytes apart), or stage kt
  // in slot kt % 3 (rows 4 bytes apart): row r's dword of stage kt at
  // r * 4 G + (kt % G) * 4
  auto as_slot = [&](int kt) {
    return smem + T32_AS_OFF + (G == 4 ? ((kt / 4) % 2) * (T32_BM * 16) : (kt % T32_NS) * (T32_BM * 4));
  };
  auto bs_slot = [&](int kt) {
    return smem + T32_BS_OFF + (G == 4 ? ((kt / 4) % 2) * (T32_BN * 16) : (kt % T32_NS) * (T32_BN * 4));
  };
  auto issue = [&](int kt) {
    const int ks = kt0 + kt;
    // the stage's scale group first (when it starts one), then its rows
    if (kt % G == 0) {
      if (G == 4) {
        if (lane < 8)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rsrc, (lptr_t)(as_slot(kt) + wave_s * 8 * 16), 16, as_voff,
                                                   ks * 4, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lptr_t)(bs_slot(kt) + wave_s * 64 * 16), 16, bs_voff,
                                                 ks * 4, 0, 0);
      } else {
        if (lane < 8)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rsrc, (lptr_t)(as_slot(kt) + wave_s * 8 * 4), 4, as_voff,
                                                   ks * 4, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lptr_t)(bs_slot(kt) + wave_s * 64 * 4), 4, bs_voff,
                                                 ks * 4, 0, 0);
      }
    }
    uint8_t* st = smem + (kt % T32_NS) * T32_STAGE;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(st + wave_s * 1024), 16, a_voff, ks * MX_A_ROW, 0, 0);
#pragma unroll
    for (int i = 0; i < T32_LPW_B; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(st + T32_A_BYTES + (wave_s * T32_LPW_B + i) * 1024), 16,
                                               b_voff[i], ks * MX_B_ROW, 0, 0);
  };

#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[ni][r] = 0.0f;
  // stages 0 .. NS-2 in the prologue; iteration kt waits for stage kt (the
  // stage after it may stay in flight: at least T32_LOADS loads), publishes
  // it, and issues stage kt+2 into the buffer of stage kt-1
#pragma unroll
  for (int i = 0; i < T32_NS - 1; ++i)
    if (i < KT) issue(i);
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + T32_NS - 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm((T32_NS - 2) * T32_LOADS));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    t32_block_barrier();
    if (kt + T32_NS - 1 < KT) issue(kt + T32_NS - 1);
    const uint8_t* st = smem + (kt % T32_NS) * T32_STAGE;
    const int sg = (kt % G) * 4;
    const uint32_t as4 = *(const uint32_t*)(as_slot(kt) + sg + fr * 4 * G);
    uint32_t bs4[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bs4[ni] = *(const uint32_t*)(bs_slot(kt) + sg + (wave * 64 + ni * 32 + fr) * 4 * G);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // k step kk covers MX blocks 2kk and 2kk+1; lane half fh passes block 2kk+fh's scale
      const i32x8_t aq = mx_frag_a(st, fr, kk, fh);
      const int asc = (int)((as4 >> (8 * (2 * kk + fh))) & 0xffu);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const i32x8_t bq = mx_frag_b(st + T32_A_BYTES, wave * 64 + ni * 32 + fr, kk, fh);
        const int bsc = (int)((bs4[ni] >> (8 * (2 * kk + fh))) & 0xffu);
        acc[ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bq, aq, acc[ni], 4, 0, 0, bsc, 0, asc);
      }
    }
  }
}

// gate_up epilogue: A = act(s * C + bias) of the tile's 128 outputs (output
// block nb of D), re-quantised to MXFP8 as the 256-row MX gate_up does
// (shared exponent floor(log2 amax) - 8 per 32 outputs of a row, codes RNE):
// block 0 holds the gate columns, block 1 the up columns of each wave's 32
// outputs, one MX block per row, the 16 values of a lane and the 16 of lane
// xor 32.  Codes and scale bytes are staged in LDS and stored as whole row
// pieces: codes [rows, D], scales [rows, D/32].  Called by the whole
// workgroup; smem must be free.
template <int ACT>
__device__ __forceinline__ void mx32_store_a_mxfp8(const f32x16_t (&acc)[2], float sc, const uint16_t* bias, int D,
                                                   bool interleaved, float alpha, float limit, int nb, int row_beg,
                                                   int row_end, uint8_t* codes, uint8_t* scales, uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, fr = lane & 31, fh = lane >> 5;
  float a[16];
  float m = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int oc = nb * 128 + wave * 32 + 8 * q + 4 * fh;  // first of 4 outputs
    float bg[4] = {0.0f, 0.0f, 0.0f, 0.0f}, bu[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (bias) gate_up_bias_x4(bias, D, oc, interleaved, bg, bu);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      a[4 * q + c] = gated_act<ACT>(acc[0][4 * q + c] * sc + bg[c], acc[1][4 * q + c] * sc + bu[c], alpha, limit);
      m = fmaxf(m, fabsf(a[4 * q + c]));
    }
  }
  m = fmaxf(m, __shfl_xor(m, 32, MOE_WAVE));
  const int X = mx_shared_exp(m);
  const float inv = mx_inv_scale(X);
  uint8_t* s_codes = smem;
  uint8_t* s_scales = smem + T32_BM * T32_CPITCH;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *(uint32_t*)(s_codes + fr * T32_CPITCH + wave * 32 + 8 * q + 4 * fh) =
        e4m3x4(a[4 * q] * inv, a[4 * q + 1] * inv, a[4 * q + 2] * inv, a[4 * q + 3] * inv);
  if (fh == 0) s_scales[fr * 4 + wave] = (uint8_t)(X + 127);
  __syncthreads();
  const int r = tid >> 3, pc = tid & 7;  // 32 rows x 8 pieces of 16 bytes
  if (row_beg + r < row_end)
    *(u32x4_t*)(codes + (int64_t)(row_beg + r) * D + nb * 128 + pc * 16) =
        *(const u32x4_t*)(s_codes + r * T32_CPITCH + pc * 16);
  if (tid < T32_BM && row_beg + tid < row_end)
    *(uint32_t*)(scales + (int64_t)(row_beg + tid) * (D / 32) + nb * 4) = *(const uint32_t*)(s_scales + tid * 4);
}

// down epilogue: O = s * C + bias for the tile's 256 columns (column block nb
// of H), staged in LDS (rows of 256 outputs + 16 bytes of bank skew) and
// stored as whole row pieces of O [rows, H] (bf16 or fp32).  Called by the
// whole workgroup; smem must be free.
template <bool OUT_BF16>
__device__ __forceinline__ void mx32_store_o_tile(const f32x16_t (&acc)[2], float sc, const uint16_t* bias, int H, int nb,
                                                  int row_beg, int row_end, void* out, uint8_t* smem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, fr = lane & 31, fh = lane >> 5;
  constexpr int ES = OUT_BF16 ? 2 : 4;
  constexpr int PITCH = T32_BN * ES + 16;
  __syncthreads();
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lc = wave * 64 + ni * 32 + 8 * q + 4 * fh;  // first of 4 tile columns
      const int n = nb * T32_BN + lc;
      float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (bias && n < H) bias_x4(bias + n, bd);
      float v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = acc[ni][4 * q + c] * sc + bd[c];
      uint8_t* dst = smem + fr * PITCH + lc * ES;
      if (OUT_BF16) {
        uint2 w;
        w.x = pack_bf16x2_rne(v[0], v[1]);
        w.y = pack_bf16x2_rne(v[2], v[3]);
        *(uint2*)dst = w;
      } else {
        *(f32x4_t*)dst = f32x4_t{v[0], v[1], v[2], v[3]};
      }
    }
  __syncthreads();
  // a row is T32_BN * ES bytes: 32 (bf16) or 64 (fp32) lanes of 16 bytes
  constexpr int LPR = T32_BN * ES / 16, RPI = 64 / LPR;  // lanes per row, rows per store
  const int cpart = lane % LPR;
  const int n = nb * T32_BN + cpart * (16 / ES);
  for (int r = wave * RPI + lane / LPR; r < T32_BM; r += T32_NW * RPI) {
    const int row = row_beg + r;
    if (row < row_end && n < H)
      *(u32x4_t*)((uint8_t*)out + ((int64_t)row * H + n) * ES) = *(const u32x4_t*)(smem + r * PITCH + cpart * 16);
  }
}

}  // namespace moe
