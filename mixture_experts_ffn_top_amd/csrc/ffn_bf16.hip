// Grouped bf16 expert GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// gate_up:  A[p, :] = act( s_gu[e] * (X[p, :] . W_gu[e]) + b_gu[e] )   (bf16 out)
// down:     O[p, :] = s_d[e] * (A[p, :] . W_d[e]) + b_d[e]             (fp32/bf16 out)
// for every CSR row p of local expert e (StackedMoE page weight shapes;
// GatedActivation page activations; mega_ffn page per-leg expert scales).
//
// Tiling: 256 x 256 workgroup tile, 8 waves in 2 x 4 (two per SIMD), each
// wave a 128 x 64 sub-tile of 4 x 2 MFMA blocks (128 fp32 accumulators per
// lane); while one wave of a SIMD waits at a barrier or on LDS the other
// issues MFMAs.  Both operands go straight from global memory into LDS
// (direct-to-LDS loads, no register staging) in 64-wide k stages, double
// buffered: the loads of stage k+1 are in flight while stage k runs on the
// matrix cores, and the MFMA fragments of the next 16-wide k step are read
// from LDS while the current step's MFMAs issue.
//
// The per-expert row counts live only on the device.  Every workgroup reads
// expert_offsets, builds the prefix of 256-row blocks per expert in LDS and
// maps its id to (expert, n-block, m-block).  Tiles are ordered expert-major,
// then n-block, then m-block, so the m-blocks that share one weight tile are
// neighbours; the id is remapped so that each XCD (workgroups are dealt to
// the 8 XCDs round-robin) runs one contiguous range of tiles and the shared
// weight tile is fetched into that XCD's L2 once.
//
// For gate_up the 256 weight rows of a tile are 128 gate rows and the 128
// matching up rows (concatenated [gate | up] or interleaved even/odd columns
// are resolved while loading), arranged so that each wave's accumulator
// block 0 holds 32 gate columns and block 1 the up columns of the same 32
// outputs: the activation runs in registers.
#include "common.h"
#include "kernels.h"

namespace moe {

enum { MODE_GATE_UP = 0, MODE_DOWN = 1 };
enum { FMT_CONCAT = 0, FMT_INTERLEAVED = 1 };

static constexpr int BM = 256, BN = 256, BK = 64;
static constexpr int NSTAGE = 2;                                 // LDS pipeline depth (power of two)
static constexpr int WAVES_M = 2, WAVES_N = 4;                   // 8 waves, 2 per SIMD
static constexpr int NTHREADS = 64 * WAVES_M * WAVES_N;
static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;     // wave tile 128 x 64
static constexpr int MI = WTM / 32, NI = WTN / 32;               // 32x32 MFMA blocks per wave
static constexpr int CPR = BK / 8;                               // 16-byte chunks per tile row
static constexpr int RPB = 1024 / (BK * 2);                      // tile rows per 1 KB load block
static constexpr int LPW = (BM * BK * 2 / 1024) / (WAVES_M * WAVES_N);  // 1 KB loads per wave per operand
static constexpr int KKS = BK / 16;                              // 16-wide k steps per stage
static constexpr int TILE_ELEMS = BM * BK;                       // bf16 elements per operand stage
static constexpr int LDS_BYTES_TILES = NSTAGE * 2 * TILE_ELEMS * 2;  // 4 stages x 2 operands

struct GemmArgs {
  const int32_t* offsets;
  int L;
  int K;          // reduction length
  int N;          // output columns: gate_up D, down H
  const uint16_t* A;   // [rows, K] (x_perm or act) or nullptr to gather from X
  const uint16_t* X;   // gather source [T, K]
  const int32_t* sorted_token;
  const uint16_t* W;   // OUT_IN per expert: [w_rows, K]
  int64_t w_estride;   // elements per expert
  const uint16_t* bias;
  int64_t bias_estride;
  const float* escale;
  float alpha, limit;
  void* out;
  int64_t ldo;
  int64_t lda, ldb;    // row pitch (elements) of the A rows and of the weight rows
};

// LDS layout of one operand stage: 256 rows x BK bf16, CPR 16-byte chunks
// per row.  Chunk c of row r sits at physical chunk c ^ f(r), chosen so that
// the 16-byte fragment reads of an MFMA (32 consecutive rows, one chunk) hit
// distinct banks both when 8 lanes share a 128-byte bank cycle and when 16
// lanes share a 256-byte one:
//   64-byte rows:  f(r) = ((r>>1 ^ r>>3) & 1) | ((r>>2 & 1) << 1)
//   128-byte rows: f(r) = (r ^ r>>3) & 7
__device__ __forceinline__ int swz_f(int r) {
  if (CPR == 4) return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
  return (r ^ (r >> 3)) & 7;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_f(row)) << 3); }

template <int MODE, int ACT, int FMT, bool GATHER, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_bf16_kernel(const GemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* As = (uint16_t*)smem;
  uint16_t* Bs = As + NSTAGE * TILE_ELEMS;
  int32_t* s_mbp = (int32_t*)(smem + LDS_BYTES_TILES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int L = p.L;

  // ---- prefix of 256-row blocks per expert (wave 0), in LDS
  if (wave == 0) {
    const int per = (L + 63) / 64;
    const int e0 = lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < L) sum += (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
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
        run += (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
      }
    }
    if (lane == 63) s_mbp[L] = inc;
  }
  __syncthreads();

  constexpr int NBO = (MODE == MODE_GATE_UP) ? BN / 2 : BN;  // output columns per tile
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
  const int e = lo;
  const int nmb = s_mbp[e + 1] - s_mbp[e];
  const int local = tile - s_mbp[e] * NB;
  const int nb = local / nmb, mb = local % nmb;
  const int row_beg = p.offsets[e] + mb * BM;
  const int row_end = p.offsets[e + 1];

  // ---- loader: direct global -> LDS (global_load_lds_dwordx4), no VGPR
  // staging.  One instruction moves a 1 KB block of RPB tile rows x CPR
  // chunks; lane l lands at row RPB*blk + l/CPR, physical chunk l%CPR, so it
  // fetches the logical chunk (l%CPR) ^ f(row).  Wave w moves blocks
  // LPW*w .. LPW*w+LPW-1 of both operands.
  const int lrow = lane / CPR;
  const char* a_base = GATHER ? (const char*)p.X : (const char*)p.A;
  const char* b_base = (const char*)(p.W + (int64_t)e * p.w_estride);
  const int64_t a_row_bytes = p.lda * 2, b_row_bytes = p.ldb * 2;
  uint32_t a_off[LPW], b_off[LPW];  // byte offset of this lane's row
  int lchunk[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int trow = (wave * LPW + i) * RPB + lrow;  // tile row 0..255
    lchunk[i] = (lane % CPR) ^ swz_f(trow);
    const int r = min(row_beg + trow, row_end - 1);
    const int64_t arow = GATHER ? (int64_t)p.sorted_token[r] : (int64_t)r;
    a_off[i] = (uint32_t)(arow * a_row_bytes);
    int wrow;
    if (MODE == MODE_DOWN) {
      wrow = min(nb * BN + trow, p.N - 1);
    } else {
      // B rows of wave column q: WTN/2 gate rows, then the matching up rows
      const int q = trow / WTN, rr = trow % WTN, isup = rr / (WTN / 2), j = rr % (WTN / 2);
      const int oc = min(nb * NBO + q * (WTN / 2) + j, p.N - 1);
      wrow = (FMT == FMT_CONCAT) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
    }
    b_off[i] = (uint32_t)(wrow * b_row_bytes);
  }
  const int KT = (p.K + BK - 1) / BK;
  auto issue = [&](int kt) {
    const int buf = kt & (NSTAGE - 1);
    uint16_t* as = As + buf * TILE_ELEMS + wave * LPW * 512;
    uint16_t* bs = Bs + buf * TILE_ELEMS + wave * LPW * 512;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      // the last stage of a ragged K is clamped to stay inside the row; its
      // A chunks past K are zeroed in LDS before the stage is published
      const uint32_t kb = (uint32_t)min(kt * BK + lchunk[i] * 8, p.K - 8) * 2u;
      __builtin_amdgcn_global_load_lds((gptr_t)(a_base + a_off[i] + kb), (lptr_t)(as + i * 512), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const uint32_t kb = (uint32_t)min(kt * BK + lchunk[i] * 8, p.K - 8) * 2u;
      __builtin_amdgcn_global_load_lds((gptr_t)(b_base + b_off[i] + kb), (lptr_t)(bs + i * 512), 16, 0, 0);
    }
  };
  // wait until this wave's loads of stage `kt` have landed: the loads of the
  // stages issued after it (at most NSTAGE-2 of them, 2*LPW each) may still fly
  auto wait_stage = [&](int kt) {
    const int newer = min(KT - 1, kt + NSTAGE - 2) - kt;
    if (NSTAGE > 3 && newer >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * LPW));
    else if (NSTAGE > 2 && newer >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  };
  // ragged K: after this wave's loads of stage kt landed, overwrite the A
  // chunks it fetched past K with zeros (B there holds finite weights); the
  // barrier that publishes the stage orders these writes
  auto zero_tail = [&](int kt) {
    if (kt * BK + BK > p.K) {
      uint16_t* as = As + (kt & (NSTAGE - 1)) * TILE_ELEMS + wave * LPW * 512;
      const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        if (kt * BK + lchunk[i] * 8 >= p.K) *(u32x4_t*)(as + i * 512 + lane * 8) = z;
    }
  };

  const int fr = lane & 31, fk = lane >> 5;
  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  auto read_frags = [&](int kt, int kk, bf16x8_t (&af)[MI], bf16x8_t (&bfr)[NI]) {
    const uint16_t* as = As + (kt & (NSTAGE - 1)) * TILE_ELEMS;
    const uint16_t* bs = Bs + (kt & (NSTAGE - 1)) * TILE_ELEMS;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      af[mi] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(as + swz(wm * WTM + mi * 32 + fr, kk * 2 + fk)));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      bfr[ni] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(bs + swz(wn * WTN + ni * 32 + fr, kk * 2 + fk)));
  };
  auto mfmas = [&](const bf16x8_t (&af)[MI], const bf16x8_t (&bfr)[NI]) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
  };

  // ---- main loop.  The KKS 16-wide k steps of stage kt run as
  //   [fragments (kt,kk+1) | MFMAs (kt,kk)]   for kk < KKS-1, then
  //   wait stage kt+1, barrier, issue stage kt+NSTAGE into kt's buffer,
  //   [fragments (kt+1,0) | MFMAs (kt,KKS-1)]
  // so every fragment read overlaps a block of MFMAs and the global loads of
  // the next NSTAGE-1 stages are in flight; two waves per SIMD cover each
  // other's barrier and dependency stalls.
  for (int s = 0; s < NSTAGE && s < KT; ++s) issue(s);
  wait_stage(0);
  zero_tail(0);
  __syncthreads();
  bf16x8_t fa[2][MI], fb[2][NI];
  read_frags(0, 0, fa[0], fb[0]);
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
    for (int kk = 0; kk < KKS; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < KKS) {
        read_frags(kt, kk + 1, fa[c ^ 1], fb[c ^ 1]);
      } else {
        if (kt + 1 < KT) {
          wait_stage(kt + 1);
          zero_tail(kt + 1);
        }
        __syncthreads();
        if (kt + NSTAGE < KT) issue(kt + NSTAGE);
        if (kt + 1 < KT) read_frags(kt + 1, 0, fa[c ^ 1], fb[c ^ 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(fa[c], fb[c]);
      __builtin_amdgcn_sched_barrier(0);
      // retire the reads that overlapped this MFMA block, so that the next
      // step's reads never leave more LDS operations outstanding than the
      // compiler tracks precisely
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    }
  }

  // ---- epilogue.  acc[mi][ni][r] is C[row][col] with
  //   row = wm*WTM + mi*32 + 8*(r/4) + 4*fk + r%4,  col = wn*WTN + ni*32 + fr
  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if (MODE == MODE_GATE_UP) {
    // blocks ni < NI/2 hold gate columns, ni + NI/2 the up columns of the same outputs
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int ni = 0; ni < NI / 2; ++ni) {
      const int oc = nb * NBO + wn * (WTN / 2) + ni * 32 + fr;
      if (oc >= p.N) continue;
      float bg = 0.0f, bu = 0.0f;
      if (bias_e) {
        const int gi = (FMT == FMT_CONCAT) ? oc : 2 * oc;
        const int ui = (FMT == FMT_CONCAT) ? p.N + oc : 2 * oc + 1;
        bg = bf16_to_f32(bias_e[gi]);
        bu = bf16_to_f32(bias_e[ui]);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_beg + wm * WTM + mi * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
          if (row < row_end) {
            const float g = acc[mi][ni][r] * sc + bg;
            const float u = acc[mi][ni + NI / 2][r] * sc + bu;
            out[(int64_t)row * p.ldo + oc] = f32_to_bf16(gated_act<ACT>(g, u, p.alpha, p.limit));
          }
        }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = nb * BN + wn * WTN + ni * 32 + fr;
      if (n >= p.N) continue;
      const float bd = bias_e ? bf16_to_f32(bias_e[n]) : 0.0f;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_beg + wm * WTM + mi * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
          if (row < row_end) {
            const float v = acc[mi][ni][r] * sc + bd;
            if (OUT_BF16) ((uint16_t*)p.out)[(int64_t)row * p.ldo + n] = f32_to_bf16(v);
            else ((float*)p.out)[(int64_t)row * p.ldo + n] = v;
          }
        }
    }
  }
}

template <typename KernelT>
static hipError_t launch_gemm(KernelT kern, const GemmArgs& a, int max_rows, int NBO,
                              hipStream_t st) {
  const int lds = LDS_BYTES_TILES + (a.L + 1) * (int)sizeof(int32_t);
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t nonempty = (int64_t)max_rows < a.L ? max_rows : a.L;
  const int64_t mblocks = (max_rows + BM - 1) / BM + nonempty;
  const int64_t NB = (a.N + NBO - 1) / NBO;
  const int64_t max_tiles = mblocks * NB;
  const int64_t grid = ((max_tiles + 7) / 8) * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, NTHREADS, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT, int FMT, bool GATHER>
static hipError_t gate_up_dispatch(const GemmArgs& a, int max_rows, hipStream_t st) {
  return launch_gemm(grouped_gemm_bf16_kernel<MODE_GATE_UP, ACT, FMT, GATHER, true>, a, max_rows, BN / 2, st);
}

hipError_t launch_ffn_bf16(const FfnBf16Params& q, hipStream_t st) {
  GemmArgs g{};
  g.offsets = q.offsets;
  g.L = q.L;
  g.K = q.H;
  g.N = q.D;
  g.A = q.x_perm;
  g.X = q.x;
  g.sorted_token = q.sorted_token;
  g.W = q.w_gate_up;
  g.w_estride = (int64_t)2 * q.D * q.H;
  g.bias = q.b_gate_up;
  g.bias_estride = 2 * (int64_t)q.D;
  g.escale = q.gate_up_scales;
  g.alpha = q.alpha;
  g.limit = q.limit;
  g.out = q.act;
  g.ldo = q.D;
  g.lda = q.H;
  g.ldb = q.H;
  const bool gather = (q.x_perm == nullptr);
  hipError_t err;
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
#define GU(ACTV, FMTV)                                                                             \
  err = gather ? gate_up_dispatch<ACTV, FMTV, true>(g, q.max_rows, st)                             \
               : gate_up_dispatch<ACTV, FMTV, false>(g, q.max_rows, st)
  if (q.fmt == FMT_CONCAT) {
    if (q.act_kind == ACT_SILU) GU(ACT_SILU, FMT_CONCAT);
    else if (q.act_kind == ACT_SWIGLUOAI) GU(ACT_SWIGLUOAI, FMT_CONCAT);
    else GU(ACT_GELU_TANH, FMT_CONCAT);
  } else {
    if (q.act_kind == ACT_SILU) GU(ACT_SILU, FMT_INTERLEAVED);
    else if (q.act_kind == ACT_SWIGLUOAI) GU(ACT_SWIGLUOAI, FMT_INTERLEAVED);
    else GU(ACT_GELU_TANH, FMT_INTERLEAVED);
  }
#undef GU
  if (err != hipSuccess) return err;
  if (q.events && (err = hipEventRecord(q.events[1], st)) != hipSuccess) return err;

  GemmArgs d{};
  d.offsets = q.offsets;
  d.L = q.L;
  d.K = q.D;
  d.N = q.H;
  d.A = q.act;
  d.W = q.w_down;
  d.w_estride = (int64_t)q.D * q.H;
  d.bias = q.b_down;
  d.bias_estride = q.H;
  d.escale = q.down_scales;
  d.out = q.out;
  d.ldo = q.H;
  d.lda = q.D;
  d.ldb = q.D;
  if (q.out_bf16)
    err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, true>, d, q.max_rows, BN, st);
  else
    err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, false>, d, q.max_rows, BN, st);
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
