// Grouped fp8 (OCP e4m3fn) block-scaled expert GEMMs on gfx950 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4; its E8M0 operand scales carry the
// power-of-two part of the block scales).
//
// Operands carry software scales (StackedMoE page: FP8 quantization with
// block scaling; the fp8 layer's weights have one fp32 scale per 128 x 128
// block, its activations one per token per 128 columns):
//   x_perm  codes [rows, H] with xs [rows, H/128]
//   W       codes [L, N, K] (OUT_IN) with ws [L, N/128, K/128]
// so that
//   C[m, n] = sum over 128-wide k blocks kb of xs[m, kb] ws[n/128, kb] P_kb[m, n]
// where P_kb is the product of the raw codes over block kb.  The two scales
// are arbitrary fp32 values.  Each is split exactly as s = 2^(e - 127) * m,
// e its float32 exponent field clamped to [1, 253] and m = s * 2^(127 - e)
// (in [1, 4) for a normal s, [2^-23, 1) for a subnormal one).  The exponent
// bytes ride in the matrix instruction's E8M0 operand scales, which scale the
// block product by 2^(ex + ew - 254) in hardware; the running sum is kept in
// units of the current block's software factor u_kb = mx mw:
//   acc <- acc * (u_{kb-1} / u_kb) + 2^(ex + ew - 254) P_kb,   C = acc * u_last
// which needs no second set of accumulators.  The factors stay within
// [2^-46, 16), so neither the reciprocal nor the rescale can overflow however
// small the scales are, and a block whose scaled product falls below the
// float32 range adds nothing, as it should.  A zero scale keeps the previous
// unit and zeroes the operand codes it scales, so its block adds nothing.
//
// gate_up:  h = s_gu[e] * C, A = act(gate, up), then A is re-quantised per
//           row per 128 columns (scale amax/448, 1 when amax = 0) -> codes +
//           scales, the down GEMM's operand (the "re-quant" of the L1 leg on
//           the mega_ffn page).
// down:     O = s_d[e] * C  (bf16 or fp32 out)
//
// Tiling (the layout of the bf16 kernel): 256 x 256 workgroup tile, 8 waves
// in 2 x 4 (two per SIMD), each wave 128 x 64 = 4 x 2 MFMA blocks with 128
// fp32 accumulators per lane.  k stages of 128 fp8 (one scale block) go
// global -> LDS by buffer loads, double buffered, with the 256 activation
// scales and the tile's two weight scales of the stage.
// The weight fragment is the MFMA's first operand, so a lane's accumulators
// are four consecutive output columns of one row per group of four.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

enum { F8_GATE_UP = 0, F8_DOWN = 1 };
enum { F8_CONCAT = 0, F8_INTERLEAVED = 1 };  // gate_up column order (StackedMoE gate_up_format)

constexpr int Q_BM = 256, Q_BN = 256, Q_BK = 128;        // BK in fp8 elements (= bytes)
constexpr int Q_NSTAGE = 2;
constexpr int Q_WAVES_M = 2, Q_WAVES_N = 4;
constexpr int Q_NT = 64 * Q_WAVES_M * Q_WAVES_N;          // 512 threads
constexpr int Q_WTM = Q_BM / Q_WAVES_M, Q_WTN = Q_BN / Q_WAVES_N;  // 128 x 64
constexpr int Q_MI = Q_WTM / 32, Q_NI = Q_WTN / 32;       // 4 x 2 MFMA blocks
constexpr int Q_A_BYTES = Q_BM * Q_BK;                    // 32 KB
constexpr int Q_B_BYTES = Q_BN * Q_BK;                    // 32 KB
constexpr int Q_WS_BYTES = 16;                            // the tile's two weight scales (+ pad)
constexpr int Q_STAGE_BYTES = Q_A_BYTES + Q_B_BYTES + Q_WS_BYTES;
constexpr int Q_LPW_A = Q_A_BYTES / 1024 / (Q_WAVES_M * Q_WAVES_N);  // 4
constexpr int Q_LPW_B = Q_B_BYTES / 1024 / (Q_WAVES_M * Q_WAVES_N);  // 4
constexpr int Q_ROW_LOADS = Q_LPW_A + Q_LPW_B;             // row loads per wave per stage
// the activation scales of a group of up to 4 stages (16 bytes per row), in
// a ring of 2 after the stage buffers
constexpr int Q_XS_SLOT = Q_BM * 16;
constexpr int Q_XS_OFF = Q_NSTAGE * Q_STAGE_BYTES;
constexpr int Q_LDS_PIPE = Q_XS_OFF + 2 * Q_XS_SLOT;      // 128 KB + 8 KB of scales
constexpr int Q_LDS_OUT = Q_BM * (Q_BN * 2 + 16);         // the down tile's bf16 outputs (132 KB)

// Buffer resource word 3 for raw (unformatted) dword accesses on gfx9 parts.
constexpr int F8_BUF_DWORD3 = 0x00020000;
// A load offset beyond the 0x7fffffff-byte range of the buffer resources
// (with room for any k offset added to it): out-of-range buffer loads return
// zeros without touching memory.
constexpr uint32_t F8_OOB_OFFSET = 0xC0000000u;

// 128-byte rows, 8 chunks of 16 bytes; chunk c of row r sits at c ^ f(r)
// (fragment reads of 32 consecutive rows hit distinct banks).
__device__ __forceinline__ int f8_swz_f(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int f8_swz(int row, int chunk) { return row * Q_BK + ((chunk ^ f8_swz_f(row)) << 4); }

// Workgroup barrier that publishes LDS (ds writes and the loads into LDS this
// wave waited for) without __syncthreads()'s full wait for the loads into
// LDS still in flight; the clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void f8_block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s = 2^(e - 127) * m exactly: e (returned) is the exponent field clamped to
// [1, 253], the E8M0 byte of the matrix instruction's operand scale; m =
// s * 2^(127 - e).  Zero gives m = 0; a non-finite s gives a non-finite m.
__device__ __forceinline__ int f8_split_scale(float s, float& m) {
  const uint32_t ef = (__builtin_bit_cast(uint32_t, s) >> 23) & 0xffu;
  const int e = (int)min(max(ef, 1u), 253u);
  m = __builtin_amdgcn_ldexpf(s, 127 - e);
  return e;
}

struct Fp8GemmArgs {
  const int32_t* offsets;
  int L;
  int K, N;                  // reduction length; output columns (gate_up D, down H)
  const uint8_t* A;          // [rows, K] codes (or per token, gathered)
  const float* A_scale;      // [rows, K/128]
  const int32_t* gather;     // row -> token, or nullptr
  const uint8_t* W;          // OUT_IN per expert [w_rows, K]
  int64_t w_estride;         // bytes per expert
  const float* W_scale;      // per expert [w_rows/128, K/128]
  int64_t ws_estride;        // floats per expert
  const float* escale;
  float alpha, limit;
  void* out;                 // gate_up: codes [rows, D]; down: bf16 / fp32 [rows, H]
  float* out_scale;          // gate_up: [rows, D/128]
  const uint16_t* bias;      // bf16 per expert (gate_up [2D] in the column order of fmt, down [H]) or nullptr
  int64_t bias_estride;
  int fmt;                   // gate_up: F8_CONCAT or F8_INTERLEAVED
};

template <int MODE, int ACT, bool OUT_BF16>
__global__ __launch_bounds__(Q_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_fp8_kernel(const Fp8GemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  // the m-block prefix only maps this workgroup to its tile; it shares LDS
  // with the stage buffers, which are filled after that
  int32_t* s_mbp = (int32_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Q_WAVES_N, wn = wave % Q_WAVES_N;
  const int L = p.L;

  // ---- prefix of 256-row blocks per expert (wave 0), in LDS
  if (wave == 0) wave_expert_prefix(p.offsets, L, s_mbp, [](int rows) { return (rows + Q_BM - 1) / Q_BM; });
  __syncthreads();

  constexpr int NBO = (MODE == F8_GATE_UP) ? Q_BN / 2 : Q_BN;  // output columns per tile
  const int NB = (p.N + NBO - 1) / NBO;
  const int total = s_mbp[L] * NB;
  const int per_xcd = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return;
  const int tile = (blockIdx.x & 7) * per_xcd + slot;
  if (tile >= total) return;
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_mbp[mid] * NB <= tile) lo = mid;
    else hi = mid - 1;
  }
  // uniform by construction; made scalar so that the address bases live in SGPRs
  const int e = __builtin_amdgcn_readfirstlane(lo);
  const int nmb = s_mbp[e + 1] - s_mbp[e];
  const int local = __builtin_amdgcn_readfirstlane(tile - s_mbp[e] * NB);
  const int nb = local / nmb, mb = local % nmb;
  const int row_beg = __builtin_amdgcn_readfirstlane(p.offsets[e] + mb * Q_BM);
  const int row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm_s = wave_s / Q_WAVES_N, wn_s = wave_s % Q_WAVES_N;
  const int KT = p.K / Q_BK;       // K is a multiple of 128: every stage is one scale block
  __syncthreads();  // every wave has read the prefix before the loads overwrite it

  // ---- loader: buffer loads straight into LDS, 1 KB = 8 rows x 8 chunks per
  // instruction; per-lane offsets fixed for the tile, the k offset of a stage
  // in the scalar offset, the destination in M0
  const int lrow = lane >> 3;
  const uint8_t* Wexp = p.W + (int64_t)e * p.w_estride;
  uint32_t a_voff[Q_LPW_A], b_voff[Q_LPW_B];
  // A wave whose 32 activation rows all lie past the expert's last row (in
  // its last m-block) points their loads past the end of the buffer range,
  // where they fetch nothing: an output row depends on its own activation
  // row only, and rows past the end are neither computed nor stored.
  const bool a_live = row_beg + wave * 32 < row_end;
#pragma unroll
  for (int i = 0; i < Q_LPW_A; ++i) {
    const int trow = (wave * Q_LPW_A + i) * 8 + lrow;
    const int r = min(row_beg + trow, row_end - 1);
    const uint32_t ar = p.gather ? (uint32_t)p.gather[r] : (uint32_t)(r - row_beg);
    a_voff[i] = a_live ? ar * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ f8_swz_f(trow)) * 16) : F8_OOB_OFFSET;
  }
#pragma unroll
  for (int i = 0; i < Q_LPW_B; ++i) {
    const int trow = (wave * Q_LPW_B + i) * 8 + lrow;
    int wrow;
    if (MODE == F8_DOWN) {
      wrow = min(nb * Q_BN + trow, p.N - 1);
    } else {
      // B rows of wave column q: 32 gate rows, then the matching 32 up rows
      const int q = trow / Q_WTN, rr = trow % Q_WTN, isup = rr / (Q_WTN / 2), j = rr % (Q_WTN / 2);
      const int oc = min(nb * NBO + q * (Q_WTN / 2) + j, p.N - 1);
      wrow = (p.fmt == F8_CONCAT) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
    }
    b_voff[i] = (uint32_t)wrow * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ f8_swz_f(trow)) * 16);
  }
  // activation scales: wave w fetches the scales of 32 rows into scale slots
  // 32w .. 32w+31, those of G consecutive stages at once (G = 4 when the
  // stage count allows, else 1): 16 contiguous bytes of each row instead of
  // 4 bytes of each row per stage, a quarter of the cache lines.  With G = 4
  // slot p holds tile row p, and a lane reads its four rows' scales with
  // four reads whose lanes step 16 bytes; with G = 1 slot p holds tile row
  // (p/128)*128 + (p%4)*32 + (p%128)/4, so the four rows a lane's MFMA
  // blocks use (wm*128 + 32 mi + fr, mi = 0..3) are the one 16-byte piece of
  // slots wm*128 + 4 fr .. + 3.
  const int G = (KT % 4 == 0) ? 4 : 1;
  const int xs_p = wave * 32 + (lane & 31);
  const int xs_t = (G == 4) ? xs_p : (xs_p & ~127) + (xs_p & 3) * 32 + ((xs_p & 127) >> 2);
  const int xs_r = min(row_beg + xs_t, row_end - 1);
  const uint32_t xs_row = p.gather ? (uint32_t)p.gather[xs_r] : (uint32_t)(xs_r - row_beg);
  const uint32_t xs_voff = xs_row * (uint32_t)KT * 4u;
  // weight scales: a tile uses two 128 x 128 scale blocks per stage, fetched
  // into the stage's scale slots 0 and 1 by lanes 0 and 1 of wave 0.
  // down: the tile's 256 columns are blocks 2 nb and 2 nb + 1 (the last one
  // clamped at an N tail); gate_up: the gate and the up block of output
  // block nb (concatenated), or blocks 2 nb and 2 nb + 1 (interleaved:
  // output oc's gate and up rows are 2 oc and 2 oc + 1, so the tile's first 64
  // outputs sit in block 2 nb, the next 64 in 2 nb + 1).
  const int ws_j = lane & 1;
  const int ws_b = (MODE == F8_DOWN)      ? min(2 * nb + ws_j, p.N / 128 - 1)
                   : (p.fmt == F8_CONCAT) ? (ws_j == 0 ? nb : p.N / 128 + nb)
                                          : 2 * nb + ws_j;
  const uint32_t ws_voff = (uint32_t)ws_b * (uint32_t)KT * 4u;
  // slot of each of the wave's two 32-column blocks
  int ws_slot[Q_NI];
#pragma unroll
  for (int ni = 0; ni < Q_NI; ++ni)
    ws_slot[ni] = (MODE == F8_DOWN || p.fmt != F8_CONCAT) ? (wn_s >= Q_WAVES_N / 2 ? 1 : 0) : ni;
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.W_scale + (int64_t)e * p.ws_estride), (short)0, 0x7fffffff, F8_BUF_DWORD3);
  // permuted rows (and their scales): the buffer resources start at the
  // tile's first row, so the row buffers may exceed 2 GiB; gathered rows are
  // addressed from the per-token codes by token
  const int64_t rb = p.gather ? 0 : (int64_t)row_beg;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.A + rb * p.K), (short)0, 0x7fffffff, F8_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Wexp, (short)0, 0x7fffffff, F8_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t s_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.A_scale + rb * KT), (short)0, 0x7fffffff, F8_BUF_DWORD3);

  auto stage_base = [&](int kt) { return smem + (kt % Q_NSTAGE) * Q_STAGE_BYTES; };
  auto xs_slot = [&](int kt) { return smem + Q_XS_OFF + ((kt / G) % 2) * Q_XS_SLOT; };
  // the group's scales, by the stage that starts it (lanes 0-31)
  auto issue_xs = [&](int kt) {
    if (kt % G != 0) return;
    if (G == 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lptr_t)(xs_slot(kt) + wave_s * 32 * 16), 16, xs_voff, kt * 4, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lptr_t)(xs_slot(kt) + wave_s * 32 * 4), 4, xs_voff, kt * 4, 0, 0);
  };
  // a wave's loads of stage kt in three parts (part 0: activation rows 0-1
  // and weight rows 0-1, part 1: the other rows, part 2: the scales), so
  // that they can be issued between the MFMA blocks of the stage before
  auto issue_part = [&](int kt, int part) {
    uint8_t* st = stage_base(kt);
    const int kb = kt * Q_BK;
    if (part < 2) {
#pragma unroll
      for (int i = part * Q_LPW_A / 2; i < (part + 1) * Q_LPW_A / 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(st + (wave_s * Q_LPW_A + i) * 1024), 16, a_voff[i], kb, 0, 0);
#pragma unroll
      for (int i = part * Q_LPW_B / 2; i < (part + 1) * Q_LPW_B / 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(st + Q_A_BYTES + (wave_s * Q_LPW_B + i) * 1024), 16, b_voff[i], kb, 0, 0);
    } else {
      if (lane < 32)
        issue_xs(kt);
      if (wave_s == 0 && lane < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lptr_t)(st + Q_A_BYTES + Q_B_BYTES), 4, ws_voff, kt * 4, 0, 0);
    }
  };
  auto issue = [&](int kt) {
    issue_part(kt, 0);
    issue_part(kt, 1);
    issue_part(kt, 2);
  };

  const int fr = lane & 31, fk = lane >> 5;
  f32x16_t acc[Q_MI][Q_NI];
#pragma unroll
  for (int mi = 0; mi < Q_MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < Q_NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // Fragments: one 32-row block and a 64-wide k step is 32 bytes per lane =
  // chunks 4kk+2fk and 4kk+2fk+1 of the lane's row.  The weight fragments of
  // a stage (both 32-column blocks, both k steps) stay in registers for the
  // stage; the activation fragments are read one 32-row block ahead.
  auto frag = [&](const uint8_t* base, int row, int kk) {
    const u32x4_t lo4 = *(const u32x4_t*)(base + f8_swz(row, kk * 4 + fk * 2));
    const u32x4_t hi4 = *(const u32x4_t*)(base + f8_swz(row, kk * 4 + fk * 2 + 1));
    return i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
  };
  auto read_b = [&](int kt, i32x8_t (&bq)[Q_NI][2]) {
    const uint8_t* bs = stage_base(kt) + Q_A_BYTES;
#pragma unroll
    for (int ni = 0; ni < Q_NI; ++ni)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) bq[ni][kk] = frag(bs, wn * Q_WTN + ni * 32 + fr, kk);
  };
  auto read_xs = [&](int kt) {
    if (G == 1) return *(const f32x4_t*)(xs_slot(kt) + (wm * Q_WTM + fr * 4) * 4);
    const uint8_t* g = xs_slot(kt) + (kt % 4) * 4 + (wm * Q_WTM + fr) * 16;
    f32x4_t v;
#pragma unroll
    for (int mi = 0; mi < Q_MI; ++mi) v[mi] = *(const float*)(g + mi * 32 * 16);
    return v;
  };
  auto read_ws = [&](int kt) { return *(const f32x2_t*)(stage_base(kt) + Q_A_BYTES + Q_B_BYTES); };
  auto read_a = [&](int kt, int mi, i32x8_t (&aq)[2]) {
    const uint8_t* as = stage_base(kt);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) aq[kk] = frag(as, wm * Q_WTM + mi * 32 + fr, kk);
  };

  // 32-row blocks of this wave holding rows of the expert (the empty blocks
  // of an expert's last m-block skip their MFMAs)
  const int live_mi = min(max((row_end - (row_beg + wm_s * Q_WTM) + 31) / 32, 0), Q_MI);

  // ---- scales.  Lane row of block mi: wm*128 + mi*32 + fr; weight-scale
  float unit[Q_MI][Q_NI];  // scale of the accumulator units
#pragma unroll
  for (int mi = 0; mi < Q_MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < Q_NI; ++ni) unit[mi][ni] = 1.0f;

  // ---- main loop.  Stage kt: per 32-row block mi, move its accumulators to
  // the stage's scale units, then 4 MFMAs (2 column blocks x 2 k steps)
  // while the next block's activation fragments are read.  After the last
  // block: wait for stage kt+1, barrier, refill stage kt's buffer with stage
  // kt+2 (issued two stages ahead), read stage kt+1's first fragments.
  i32x8_t bq[Q_NI][2], aq[2][2];
  issue(0);
  if (KT > 1) issue(1);
  // stage 0 landed: stage 1 issued at least its Q_ROW_LOADS row loads after it
  if (KT > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(Q_ROW_LOADS));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  f8_block_barrier();
  read_b(0, bq);
  f32x4_t xs4 = read_xs(0);
  f32x2_t ws2 = read_ws(0);
  if (live_mi > 0) read_a(0, 0, aq[0]);
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  for (int kt = 0; kt < KT; ++kt) {
    // a zero scale keeps the previous unit and zeroes the codes it scales
    float wm_[Q_NI];
    int we[Q_NI];
#pragma unroll
    for (int ni = 0; ni < Q_NI; ++ni) {
      const float w = ws_slot[ni] ? ws2[1] : ws2[0];
      we[ni] = f8_split_scale(w, wm_[ni]);
      if (__builtin_bit_cast(uint32_t, w) << 1 == 0u) {
        asm volatile("");
        bq[ni][0] = bq[ni][1] = i32x8_t{};
      }
    }
#pragma unroll
    for (int mi = 0; mi < Q_MI; ++mi) {
      const int c = mi & 1;
      if (mi + 1 < Q_MI && mi + 1 < live_mi) read_a(kt, mi + 1, aq[c ^ 1]);
      if (mi < live_mi) {
        const float x = xs4[mi];
        if (__builtin_amdgcn_ballot_w64(x == 0.0f) != 0) {
          asm volatile("");
          if (x == 0.0f) aq[c][0] = aq[c][1] = i32x8_t{};
        }
        float xm;
        const int xe = f8_split_scale(x, xm);
#pragma unroll
        for (int ni = 0; ni < Q_NI; ++ni) {
          float u = xm * wm_[ni];
          u = (u != 0.0f) ? u : unit[mi][ni];
          const float ratio = unit[mi][ni] * __builtin_amdgcn_rcpf(u);
          unit[mi][ni] = u;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mi][ni][r] *= ratio;
        }
        // the exponent bytes: the weight operand's (first) is uniform, the
        // activation operand's is this lane's row's (lanes r and 32 + r hold
        // the two K halves of row r and pass the same byte)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int ni = 0; ni < Q_NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bq[ni][kk], aq[c][kk], acc[mi][ni], 0, 0, 0,
                                                                          we[ni], 0, xe);
      }
      // stage kt+1's loads (its buffer was freed by the barrier that began
      // this stage), spread over the first three blocks: issued all at once
      // they would queue behind each other and hold up the waves' next reads
      if (mi < 3 && kt >= 1 && kt + 1 < KT) issue_part(kt + 1, mi);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    }
    if (kt + 1 < KT) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      f8_block_barrier();
      read_b(kt + 1, bq);
      xs4 = read_xs(kt + 1);
      ws2 = read_ws(kt + 1);
      if (live_mi > 0) read_a(kt + 1, 0, aq[0]);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    }
  }

  // ---- epilogue.  acc[mi][ni][4q + c] is C[row][col] in units unit[mi][ni] with
  //   row = wm*128 + mi*32 + fr,  col = wn*64 + ni*32 + 8q + 4fk + c
  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if (MODE == F8_GATE_UP) {
    // block 0 holds gate columns, block 1 the up columns of the same 32
    // outputs; the 128 outputs of a row (one re-quantisation block) are spread
    // over the four wave columns, whose row maxima meet in LDS.  The biases
    // of this lane's 16 outputs (gate and up), in the column order of fmt:
    float bg[16], bu[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int oc = nb * NBO + wn * 32 + 8 * q + 4 * fk;
#pragma unroll
      for (int c = 0; c < 4; ++c) bg[4 * q + c] = bu[4 * q + c] = 0.0f;
      if (bias_e && oc < p.N) {
        gate_up_bias_x4(bias_e, p.N, oc, p.fmt != F8_CONCAT, bg + 4 * q, bu + 4 * q);
      }
    }
    float a[Q_MI][16];
    float amax[Q_MI];
#pragma unroll
    for (int mi = 0; mi < Q_MI; ++mi) {
      const float ug = unit[mi][0] * sc, uu = unit[mi][1] * sc;
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        a[mi][r] = gated_act<ACT>(acc[mi][0][r] * ug + bg[r], acc[mi][1][r] * uu + bu[r], p.alpha, p.limit);
        m = fmaxf(m, fabsf(a[mi][r]));
      }
      amax[mi] = fmaxf(m, __shfl_xor(m, 32, MOE_WAVE));
    }
    __syncthreads();  // the stage buffers are free
    float* red = (float*)smem;  // [256 rows][4 wave columns]
    if (fk == 0) {
#pragma unroll
      for (int mi = 0; mi < Q_MI; ++mi) red[(wm * Q_WTM + mi * 32 + fr) * 4 + wn] = amax[mi];
    }
    __syncthreads();
    uint8_t* out = (uint8_t*)p.out;
#pragma unroll
    for (int mi = 0; mi < Q_MI; ++mi) {
      const int lrw = wm * Q_WTM + mi * 32 + fr;
      const int row = row_beg + lrw;
      if (row >= row_end) continue;
      const f32x4_t r4 = *(const f32x4_t*)(red + lrw * 4);
      const float m = fmaxf(fmaxf(r4[0], r4[1]), fmaxf(r4[2], r4[3]));
      const float s = (m > 0.0f) ? __fdiv_rn(m, 448.0f) : 1.0f;
      const SharedDivisor ds = shared_divisor(s);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int oc = nb * NBO + wn * 32 + 8 * q + 4 * fk;
        const uint32_t w = e4m3x4(div_rn(ds, a[mi][4 * q + 0]), div_rn(ds, a[mi][4 * q + 1]),
                                  div_rn(ds, a[mi][4 * q + 2]), div_rn(ds, a[mi][4 * q + 3]));
        *(uint32_t*)(out + (int64_t)row * p.N + oc) = w;
      }
      if (wn == 0 && fk == 0) p.out_scale[(int64_t)row * (p.N / 128) + nb] = s;
    }
  } else if (OUT_BF16) {
    // The tile's bf16 outputs go through LDS (row pitch 528 bytes: 4 banks of
    // skew per row) so that each store moves whole 512-byte row pieces: a
    // lane's own accumulators cover 8 bytes of each of 16 rows, which as
    // direct stores would touch every output line 8 times.
    constexpr int PITCH = Q_LDS_OUT / Q_BM;
    __syncthreads();  // the stage buffers are free
#pragma unroll
    for (int ni = 0; ni < Q_NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lc = wn * Q_WTN + ni * 32 + 8 * q + 4 * fk;  // first of 4 tile columns
        const int n = nb * Q_BN + lc;
        float bb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias_e && n < p.N) {
          bias_x4(bias_e + n, bb);
        }
#pragma unroll
        for (int mi = 0; mi < Q_MI; ++mi) {
          const int lr = wm * Q_WTM + mi * 32 + fr;
          const float u = unit[mi][ni] * sc;
          uint2 w;
          w.x = pack_bf16x2_rne(acc[mi][ni][4 * q + 0] * u + bb[0], acc[mi][ni][4 * q + 1] * u + bb[1]);
          w.y = pack_bf16x2_rne(acc[mi][ni][4 * q + 2] * u + bb[2], acc[mi][ni][4 * q + 3] * u + bb[3]);
          *(uint2*)(smem + lr * PITCH + lc * 2) = w;
        }
      }
    __syncthreads();
    // 64 lanes store two rows of 32 x 16 bytes; wave w takes rows 2 j + ... of its 32
    const int cpart = lane & 31;
    const int n = nb * Q_BN + cpart * 8;
#pragma unroll 4
    for (int j = 0; j < Q_BM / (2 * Q_WAVES_M * Q_WAVES_N); ++j) {
      const int lr = wave * (Q_BM / (Q_WAVES_M * Q_WAVES_N)) + 2 * j + (lane >> 5);
      const int row = row_beg + lr;
      if (row < row_end && n < p.N)
        *(u32x4_t*)((uint16_t*)p.out + (int64_t)row * p.N + n) = *(const u32x4_t*)(smem + lr * PITCH + cpart * 16);
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < Q_NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nb * Q_BN + wn * Q_WTN + ni * 32 + 8 * q + 4 * fk;  // first of 4 columns
        if (n >= p.N) continue;
#pragma unroll
        for (int mi = 0; mi < Q_MI; ++mi) {
          const int row = row_beg + wm * Q_WTM + mi * 32 + fr;
          if (row >= row_end) continue;
          const float u = unit[mi][ni] * sc;
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = acc[mi][ni][4 * q + c] * u;
          if (bias_e) {
            float bb[4];
            bias_x4(bias_e + n, bb);
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] += bb[c];
          }
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

template <typename KernelT>
hipError_t launch_fp8(KernelT kern, const Fp8GemmArgs& a, int max_rows, int NBO, hipStream_t st) {
  const int prefix = (a.L + 1) * (int)sizeof(int32_t);
  const int pipe = Q_LDS_PIPE > Q_LDS_OUT ? Q_LDS_PIPE : Q_LDS_OUT;
  const int lds = pipe > prefix ? pipe : prefix;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t nonempty = (int64_t)max_rows < a.L ? max_rows : a.L;
  const int64_t mblocks = (max_rows + Q_BM - 1) / Q_BM + nonempty;
  const int64_t NB = (a.N + NBO - 1) / NBO;
  const int64_t grid = ((mblocks * NB + 7) / 8) * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, Q_NT, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_fp8(const FfnFp8Params& q, hipStream_t st) {
  hipError_t err;
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
  Fp8GemmArgs g{};
  g.offsets = q.offsets;
  g.L = q.L;
  g.K = q.H;
  g.N = q.D;
  g.A = q.x_perm;
  g.A_scale = q.x_scale;
  g.gather = q.sorted_token;
  g.W = q.w_gate_up;
  g.w_estride = (int64_t)2 * q.D * q.H;
  g.W_scale = q.w_gate_up_scale;
  g.ws_estride = (int64_t)(2 * q.D / 128) * (q.H / 128);
  g.escale = q.gate_up_scales;
  g.alpha = q.alpha;
  g.limit = q.limit;
  g.out = q.act;
  g.out_scale = q.act_scale;
  g.bias = q.b_gate_up;
  g.bias_estride = 2 * (int64_t)q.D;
  g.fmt = q.fmt;
  if (q.act_kind == ACT_SILU)
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_GATE_UP, ACT_SILU, false>, g, q.max_rows, Q_BN / 2, st);
  else if (q.act_kind == ACT_SWIGLUOAI)
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_GATE_UP, ACT_SWIGLUOAI, false>, g, q.max_rows, Q_BN / 2, st);
  else
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_GATE_UP, ACT_GELU_TANH, false>, g, q.max_rows, Q_BN / 2, st);
  if (err != hipSuccess) return err;
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;
  Fp8GemmArgs d{};
  d.offsets = q.offsets;
  d.L = q.L;
  d.K = q.D;
  d.N = q.H;
  d.A = q.act;
  d.A_scale = q.act_scale;
  d.W = q.w_down;
  d.w_estride = (int64_t)q.D * q.H;
  d.W_scale = q.w_down_scale;
  d.ws_estride = (int64_t)(q.H / 128) * (q.D / 128);
  d.escale = q.down_scales;
  d.out = q.out;
  d.bias = q.b_down;
  d.bias_estride = q.H;
  if (q.out_bf16)
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_DOWN, ACT_SILU, true>, d, q.max_rows, Q_BN, st);
  else
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_DOWN, ACT_SILU, false>, d, q.max_rows, Q_BN, st);
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
