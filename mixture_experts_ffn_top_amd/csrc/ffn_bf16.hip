// Grouped bf16 expert GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// gate_up:  A[p, :] = act( s_gu[e] * (X[p, :] . W_gu[e]) + b_gu[e] )   (bf16 out)
// down:     O[p, :] = s_d[e] * (A[p, :] . W_d[e]) + b_d[e]             (fp32/bf16 out)
// for every CSR row p of local expert e (StackedMoE page weight shapes;
// GatedActivation page activations; mega_ffn page per-leg expert scales).
//
// Tiling: 256 x 256 x 64 workgroup tile, 4 waves in 2 x 2, each wave a
// 128 x 128 sub-tile of 4 x 4 MFMA blocks (256 fp32 accumulators per lane).
// Both operands are staged through LDS with a 16-byte-chunk XOR swizzle and
// double buffering; global loads of tile k+1 are in flight while tile k runs
// on the matrix cores.
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
// blocks 0,1 hold gate columns and blocks 2,3 the up columns of the same
// outputs: the activation runs in registers.
#include "common.h"
#include "kernels.h"

namespace moe {

enum { MODE_GATE_UP = 0, MODE_DOWN = 1 };
enum { FMT_CONCAT = 0, FMT_INTERLEAVED = 1 };

static constexpr int BM = 256, BN = 256, BK = 64;
static constexpr int TILE_ELEMS = BM * BK;                       // bf16 elements per operand tile
static constexpr int LDS_BYTES_TILES = 2 * 2 * TILE_ELEMS * 2;    // 2 operands x 2 stages

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
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

template <int MODE, int ACT, int FMT, bool GATHER, bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_bf16_kernel(const GemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* As = (uint16_t*)smem;
  uint16_t* Bs = As + 2 * TILE_ELEMS;
  int32_t* s_mbp = (int32_t*)(smem + LDS_BYTES_TILES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
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

  // ---- loader setup: thread owns chunk c16 of rows r0 + 32 i (i < 8)
  const int c16 = tid & 7, r0 = tid >> 3;
  const uint16_t* a_ptr[8];
  const uint16_t* b_ptr[8];
  const uint16_t* We = p.W + (int64_t)e * p.w_estride;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = min(row_beg + r0 + 32 * i, row_end - 1);
    if (GATHER) a_ptr[i] = p.X + (int64_t)p.sorted_token[r] * p.K + c16 * 8;
    else a_ptr[i] = p.A + (int64_t)r * p.K + c16 * 8;
    const int n = r0 + 32 * i;
    int wrow;
    if (MODE == MODE_DOWN) {
      wrow = min(nb * BN + n, p.N - 1);
    } else {
      const int half = n >> 7, rr = n & 127, isup = rr >> 6, j = rr & 63;
      const int oc = min(nb * NBO + half * 64 + j, p.N - 1);
      wrow = (FMT == FMT_CONCAT) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
    }
    b_ptr[i] = We + (int64_t)wrow * p.K + c16 * 8;
  }

  u32x4_t ra[8], rb[8];
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int kt) {
    const int kof = kt * BK;
    const bool kok = (kof + c16 * 8) < p.K;
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = kok ? *(const u32x4_t*)(a_ptr[i] + kof) : zero4;
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[i] = kok ? *(const u32x4_t*)(b_ptr[i] + kof) : zero4;
  };
  auto lstore = [&](int buf) {
    uint16_t* as = As + buf * TILE_ELEMS;
    uint16_t* bs = Bs + buf * TILE_ELEMS;
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)(as + swz(r0 + 32 * i, c16)) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)(bs + swz(r0 + 32 * i, c16)) = rb[i];
  };

  const int fr = lane & 31, fk = lane >> 5;
  f32x16_t acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  const int KT = (p.K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint16_t* as = As + cur * TILE_ELEMS;
    const uint16_t* bs = Bs + cur * TILE_ELEMS;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        af[mi] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(as + swz(wm * 128 + mi * 32 + fr, kk * 2 + fk)));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfr[ni] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(bs + swz(wn * 128 + ni * 32 + fr, kk * 2 + fk)));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  acc[mi][ni][r] is C[row][col] with
  //   row = wm*128 + mi*32 + 8*(r/4) + 4*fk + r%4,  col = wn*128 + ni*32 + fr
  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if (MODE == MODE_GATE_UP) {
    uint16_t* out = (uint16_t*)p.out;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int oc = nb * NBO + wn * 64 + ni * 32 + fr;
      if (oc >= p.N) continue;
      float bg = 0.0f, bu = 0.0f;
      if (bias_e) {
        const int gi = (FMT == FMT_CONCAT) ? oc : 2 * oc;
        const int ui = (FMT == FMT_CONCAT) ? p.N + oc : 2 * oc + 1;
        bg = bf16_to_f32(bias_e[gi]);
        bu = bf16_to_f32(bias_e[ui]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_beg + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
          if (row < row_end) {
            const float g = acc[mi][ni][r] * sc + bg;
            const float u = acc[mi][ni + 2][r] * sc + bu;
            out[(int64_t)row * p.ldo + oc] = f32_to_bf16(gated_act<ACT>(g, u, p.alpha, p.limit));
          }
        }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int n = nb * BN + wn * 128 + ni * 32 + fr;
      if (n >= p.N) continue;
      const float bd = bias_e ? bf16_to_f32(bias_e[n]) : 0.0f;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_beg + wm * 128 + mi * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
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
  kern<<<(unsigned)grid, 256, lds, st>>>(a);
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
  if (q.out_bf16)
    err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, true>, d, q.max_rows, BN, st);
  else
    err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, false>, d, q.max_rows, BN, st);
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
