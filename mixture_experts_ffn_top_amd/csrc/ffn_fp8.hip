// Grouped fp8 (OCP e4m3fn) block-scaled expert GEMMs on gfx950 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit hardware scales).
//
// Operands carry software scales (StackedMoE page: FP8 quantization with
// block scaling; the fp8 layer's weights have one fp32 scale per 128 x 128
// block, its activations one per token per 128 columns):
//   x_perm  codes [rows, H] with xs [rows, H/128]
//   W       codes [L, N, K] (OUT_IN) with ws [L, N/128, K/128]
// For every 128-wide k block kb the MFMAs accumulate the raw code products
// into a partial sum P, which is folded into the output accumulator as
//   acc += P * xs[row, kb] * ws[n/128, kb]
// (the two scales cannot enter the MFMA, being arbitrary fp32 values).
//
// gate_up:  h = s_gu[e] * acc, A = act(gate, up), then A is re-quantised per
//           row per 128 columns (scale amax/448, 1 when amax = 0) -> codes +
//           scales, the down GEMM's operand (the "re-quant" of the L1 leg on
//           the mega_ffn page).
// down:     O = s_d[e] * acc  (bf16 or fp32 out)
//
// Tiling: 128 rows x 256 weight rows per workgroup, 8 waves in 2 x 4 (two
// per SIMD), each wave a 64 x 64 sub-tile of 2 x 2 MFMA blocks with an
// output accumulator and a per-block partial (64 + 64 fp32 per lane).
// k stages of 128 fp8 (one scale block) go global -> LDS by direct-to-LDS
// loads, three stages deep, together with the 128 activation scales of the
// stage.  For gate_up the 256 weight rows are 128 gate rows and the matching
// 128 up rows, so one tile produces 128 whole output columns -- exactly one
// re-quantisation block per row.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

enum { F8_GATE_UP = 0, F8_DOWN = 1 };

constexpr int F_BM = 128, F_BN = 256, F_BK = 128;        // BK in fp8 elements (= bytes)
constexpr int F_NSTAGE = 3;
constexpr int F_WAVES_M = 2, F_WAVES_N = 4;
constexpr int F_NT = 64 * F_WAVES_M * F_WAVES_N;          // 512 threads
constexpr int F_WTM = F_BM / F_WAVES_M, F_WTN = F_BN / F_WAVES_N;  // 64 x 64
constexpr int F_MI = F_WTM / 32, F_NI = F_WTN / 32;       // 2 x 2 MFMA blocks
constexpr int F_A_BYTES = F_BM * F_BK;                    // 16 KB
constexpr int F_B_BYTES = F_BN * F_BK;                    // 32 KB
constexpr int F_XS_BYTES = F_BM * 4;                      // 512 B of activation scales
constexpr int F_STAGE_BYTES = F_A_BYTES + F_B_BYTES;      // operand bytes per stage
constexpr int F_LPW_A = F_A_BYTES / 1024 / (F_WAVES_M * F_WAVES_N);  // 2
constexpr int F_LPW_B = F_B_BYTES / 1024 / (F_WAVES_M * F_WAVES_N);  // 4
constexpr int F_LOADS = F_LPW_A + F_LPW_B + 1;            // per wave per stage (+1 scales)
constexpr int F_XS_BUFS = 4;                              // scale buffers (see main loop)
constexpr int F_LDS_PIPE = F_NSTAGE * F_STAGE_BYTES + F_XS_BUFS * F_XS_BYTES;
constexpr int F_EPI_PITCH = 132;                          // floats per row of the epilogue tile

// 128-byte rows, 8 chunks of 16 bytes; chunk c of row r sits at c ^ f(r)
// (fragment reads of 32 consecutive rows hit distinct banks).
__device__ __forceinline__ int f8_swz_f(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int f8_swz(int row, int chunk) { return row * F_BK + ((chunk ^ f8_swz_f(row)) << 4); }

// Buffer resource word 3 for raw (unformatted) dword accesses on gfx9 parts.
constexpr int F8_BUF_DWORD3 = 0x00020000;

// Workgroup barrier that publishes LDS (ds writes and the loads into LDS this
// wave waited for) without __syncthreads()'s full wait for the loads into
// LDS still in flight; the clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void f8_block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
};

template <int MODE, int ACT, bool OUT_BF16>
__global__ __launch_bounds__(F_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_fp8_kernel(const Fp8GemmArgs p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int32_t* s_mbp = (int32_t*)(smem + F_LDS_PIPE);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / F_WAVES_N, wn = wave % F_WAVES_N;
  const int L = p.L;

  // ---- prefix of 128-row blocks per expert (wave 0), in LDS
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

  constexpr int NBO = (MODE == F8_GATE_UP) ? F_BN / 2 : F_BN;
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
  const int row_beg = __builtin_amdgcn_readfirstlane(p.offsets[e] + mb * F_BM);
  const int row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wn_s = wave_s % F_WAVES_N;
  const int KT = p.K / F_BK;       // K is a multiple of 128
  const int KB = KT;               // scale blocks along K

  // ---- loader: 1 KB direct-to-LDS blocks of 8 rows x 8 chunks
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ f8_swz_f(lrow);  // rows 8*blk + lrow: f depends on lrow and blk
  const uint8_t* Wexp = p.W + (int64_t)e * p.w_estride;
  uint32_t a_off[F_LPW_A], b_off[F_LPW_B];
  int a_chunk[F_LPW_A], b_chunk[F_LPW_B];
#pragma unroll
  for (int i = 0; i < F_LPW_A; ++i) {
    const int trow = (wave * F_LPW_A + i) * 8 + lrow;
    a_chunk[i] = (lane & 7) ^ f8_swz_f(trow);
    const int r = min(row_beg + trow, row_end - 1);
    const int64_t ar = p.gather ? (int64_t)p.gather[r] : (int64_t)r;
    a_off[i] = (uint32_t)(ar * p.K);
  }
#pragma unroll
  for (int i = 0; i < F_LPW_B; ++i) {
    const int trow = (wave * F_LPW_B + i) * 8 + lrow;
    b_chunk[i] = (lane & 7) ^ f8_swz_f(trow);
    int wrow;
    if (MODE == F8_DOWN) {
      wrow = min(nb * F_BN + trow, p.N - 1);
    } else {
      const int q = trow / F_WTN, rr = trow % F_WTN, isup = rr / (F_WTN / 2), j = rr % (F_WTN / 2);
      const int oc = min(nb * NBO + q * (F_WTN / 2) + j, p.N - 1);
      wrow = isup ? p.N + oc : oc;
    }
    b_off[i] = (uint32_t)((int64_t)wrow * p.K);
  }
  (void)lchunk;
  // activation scales of 16 tile rows per wave (lanes 0..15)
  const int xs_r = min(row_beg + wave * 16 + (lane & 15), row_end - 1);
  const int64_t xs_row = p.gather ? (int64_t)p.gather[xs_r] : (int64_t)xs_r;
  const float* xs_src = p.A_scale + xs_row * KB;

  // Buffer loads straight into LDS: per-lane offsets fixed for the tile, the
  // k offset of a stage in the scalar offset, the destination in M0.
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, 0x7fffffff, F8_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)Wexp, (short)0, 0x7fffffff, F8_BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.A_scale, (short)0, 0x7fffffff, F8_BUF_DWORD3);
  uint32_t a_voff[F_LPW_A], b_voff[F_LPW_B];
#pragma unroll
  for (int i = 0; i < F_LPW_A; ++i) a_voff[i] = a_off[i] + (uint32_t)a_chunk[i] * 16u;
#pragma unroll
  for (int i = 0; i < F_LPW_B; ++i) b_voff[i] = b_off[i] + (uint32_t)b_chunk[i] * 16u;
  const uint32_t xs_voff = (uint32_t)(xs_row * KB) * 4u;

  auto stage_a = [&](int kt) { return smem + (kt % F_NSTAGE) * F_STAGE_BYTES; };
  auto stage_xs = [&](int kt) { return (float*)(smem + F_NSTAGE * F_STAGE_BYTES + (kt % F_XS_BUFS) * F_XS_BYTES); };
  auto issue = [&](int kt) {
    uint8_t* as = stage_a(kt) + wave_s * F_LPW_A * 1024;
    uint8_t* bs = stage_a(kt) + F_A_BYTES + wave_s * F_LPW_B * 1024;
    const int kb = kt * F_BK;
#pragma unroll
    for (int i = 0; i < F_LPW_A; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)(as + i * 1024), 16, a_voff[i], kb, 0, 0);
#pragma unroll
    for (int i = 0; i < F_LPW_B; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)(bs + i * 1024), 16, b_voff[i], kb, 0, 0);
    if (lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lptr_t)(stage_xs(kt) + wave_s * 16), 4, xs_voff, kt * 4, 0, 0);
  };
  auto wait_stage = [&](int kt) {
    const int newer = min(KT - 1, kt + F_NSTAGE - 2) - kt;
    if (newer >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(F_LOADS));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  };

  const int fr = lane & 31, fk = lane >> 5;
  f32x16_t acc[F_MI][F_NI], part[F_MI][F_NI];
#pragma unroll
  for (int mi = 0; mi < F_MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < F_NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // fragment of one 32-row block for the 64-wide k step kk: 32 bytes = chunks 4kk+2fk, +1
  auto read_frags = [&](int kt, int kk, i32x8_t (&af)[F_MI], i32x8_t (&bfr)[F_NI]) {
    const uint8_t* as = stage_a(kt);
    const uint8_t* bs = stage_a(kt) + F_A_BYTES;
#pragma unroll
    for (int mi = 0; mi < F_MI; ++mi) {
      const int row = wm * F_WTM + mi * 32 + fr;
      const u32x4_t lo4 = *(const u32x4_t*)(as + f8_swz(row, kk * 4 + fk * 2));
      const u32x4_t hi4 = *(const u32x4_t*)(as + f8_swz(row, kk * 4 + fk * 2 + 1));
      af[mi] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
    }
#pragma unroll
    for (int ni = 0; ni < F_NI; ++ni) {
      const int row = wn * F_WTN + ni * 32 + fr;
      const u32x4_t lo4 = *(const u32x4_t*)(bs + f8_swz(row, kk * 4 + fk * 2));
      const u32x4_t hi4 = *(const u32x4_t*)(bs + f8_swz(row, kk * 4 + fk * 2 + 1));
      bfr[ni] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
    }
  };
  auto mfmas = [&](const i32x8_t (&af)[F_MI], const i32x8_t (&bfr)[F_NI], bool first) {
#pragma unroll
    for (int mi = 0; mi < F_MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < F_NI; ++ni) {
        const f32x16_t c = first ? f32x16_t{} : part[mi][ni];
        part[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bfr[ni], c, 0, 0, 0, 127, 0, 127);
      }
  };
  // weight-scale block rows of this wave's two 32-column blocks
  int ws_blk[F_NI];
#pragma unroll
  for (int ni = 0; ni < F_NI; ++ni) {
    if (MODE == F8_DOWN) ws_blk[ni] = min((nb * F_BN + wn_s * F_WTN) / 128, p.N / 128 - 1);
    else ws_blk[ni] = (ni == 0) ? nb : (p.N / 128 + nb);  // gate block, up block
  }
  // read through the scalar cache: uniform per wave, and a vector load here
  // would make the wait for it drain the loads into LDS still in flight
  typedef const __attribute__((address_space(4))) float* scalar_f32_ptr;
  const scalar_f32_ptr wsc = (scalar_f32_ptr)(p.W_scale + (int64_t)e * p.ws_estride);
  auto rescale = [&](int kt) {
    const float* xs = stage_xs(kt);
    float sw[F_NI];
#pragma unroll
    for (int ni = 0; ni < F_NI; ++ni) sw[ni] = wsc[(int64_t)ws_blk[ni] * KB + kt];
#pragma unroll
    for (int mi = 0; mi < F_MI; ++mi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // rows wm*64 + mi*32 + 8g + 4fk + (0..3)
        const f32x4_t s4 = *(const f32x4_t*)(xs + wm * F_WTM + mi * 32 + 8 * g + 4 * fk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int ni = 0; ni < F_NI; ++ni)
            acc[mi][ni][4 * g + i] = fmaf(part[mi][ni][4 * g + i], s4[i] * sw[ni], acc[mi][ni][4 * g + i]);
      }
  };

  // ---- main loop: stage kt = two 64-wide k steps and one scale block
  for (int s = 0; s < F_NSTAGE && s < KT; ++s) issue(s);
  wait_stage(0);
  f8_block_barrier();
  i32x8_t fa[2][F_MI], fb[2][F_NI];
  read_frags(0, 0, fa[0], fb[0]);
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  for (int kt = 0; kt < KT; ++kt) {
    read_frags(kt, 1, fa[1], fb[1]);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa[0], fb[0], true);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    if (kt + 1 < KT) wait_stage(kt + 1);
    f8_block_barrier();
    // stage kt's operands are all in registers: refill its buffer.  The
    // scales use F_XS_BUFS > F_NSTAGE buffers, so stage kt's scales survive
    // until the rescale below.
    if (kt + F_NSTAGE < KT) issue(kt + F_NSTAGE);
    if (kt + 1 < KT) read_frags(kt + 1, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(fa[1], fb[1], false);
    __builtin_amdgcn_sched_barrier(0);
    rescale(kt);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  }

  const float sc = p.escale ? p.escale[e] : 1.0f;
  if (MODE == F8_GATE_UP) {
    // activation into an fp32 tile in LDS (the pipeline buffers are free),
    // then each row's 128 outputs are re-quantised by 4 threads
    __syncthreads();
    float* t = (float*)smem;
#pragma unroll
    for (int mi = 0; mi < F_MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * F_WTM + mi * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
        const float g = acc[mi][0][r] * sc, u = acc[mi][1][r] * sc;
        t[row * F_EPI_PITCH + wn * 32 + fr] = gated_act<ACT>(g, u, p.alpha, p.limit);
      }
    __syncthreads();
    const int row = tid >> 2, part4 = tid & 3;
    const float* src = t + row * F_EPI_PITCH + part4 * 32;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4_t q = *(const f32x4_t*)(src + 4 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[4 * i + j] = q[j];
        amax = fmaxf(amax, fabsf(q[j]));
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, MOE_WAVE));
    amax = fmaxf(amax, __shfl_xor(amax, 2, MOE_WAVE));
    const float s = (amax > 0.0f) ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const int grow = row_beg + row;
    const int ocol = nb * NBO + part4 * 32;
    if (grow < row_end && ocol < p.N) {
      u32x4_t w0, w1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t x0 = 0, x1 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x0 |= (uint32_t)f32_to_e4m3(__fdiv_rn(v[4 * i + j], s)) << (8 * j);
          x1 |= (uint32_t)f32_to_e4m3(__fdiv_rn(v[16 + 4 * i + j], s)) << (8 * j);
        }
        w0[i] = x0;
        w1[i] = x1;
      }
      uint8_t* dst = (uint8_t*)p.out + (int64_t)grow * p.N + ocol;
      *(u32x4_t*)dst = w0;
      *(u32x4_t*)(dst + 16) = w1;
      if (part4 == 0) p.out_scale[(int64_t)grow * (p.N / 128) + nb] = s;
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < F_NI; ++ni) {
      const int n = nb * F_BN + wn * F_WTN + ni * 32 + fr;
      if (n >= p.N) continue;
#pragma unroll
      for (int mi = 0; mi < F_MI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_beg + wm * F_WTM + mi * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
          if (row < row_end) {
            const float v = acc[mi][ni][r] * sc;
            if (OUT_BF16) ((uint16_t*)p.out)[(int64_t)row * p.N + n] = f32_to_bf16(v);
            else ((float*)p.out)[(int64_t)row * p.N + n] = v;
          }
        }
    }
  }
}

template <typename KernelT>
hipError_t launch_fp8(KernelT kern, const Fp8GemmArgs& a, int max_rows, int NBO, hipStream_t st) {
  const int epi = F_BM * F_EPI_PITCH * 4;
  const int pipe = F_LDS_PIPE > epi ? F_LDS_PIPE : epi;
  const int lds = pipe + (a.L + 1) * (int)sizeof(int32_t);
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t nonempty = (int64_t)max_rows < a.L ? max_rows : a.L;
  const int64_t mblocks = (max_rows + F_BM - 1) / F_BM + nonempty;
  const int64_t NB = (a.N + NBO - 1) / NBO;
  const int64_t grid = ((mblocks * NB + 7) / 8) * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, F_NT, lds, st>>>(a);
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
  if (q.act_kind == ACT_SILU)
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_GATE_UP, ACT_SILU, false>, g, q.max_rows, F_BN / 2, st);
  else if (q.act_kind == ACT_SWIGLUOAI)
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_GATE_UP, ACT_SWIGLUOAI, false>, g, q.max_rows, F_BN / 2, st);
  else
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_GATE_UP, ACT_GELU_TANH, false>, g, q.max_rows, F_BN / 2, st);
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
  if (q.out_bf16)
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_DOWN, ACT_SILU, true>, d, q.max_rows, F_BN, st);
  else
    err = launch_fp8(grouped_gemm_fp8_kernel<F8_DOWN, ACT_SILU, false>, d, q.max_rows, F_BN, st);
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

}  // namespace moe
