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
// (buffer loads with an LDS destination, no register staging) in 64-wide k
// stages: the activation rows double buffered, the weight rows triple
// buffered, so the loads of the next stages are in flight while a stage runs
// on the matrix cores, and the MFMA fragments of the next 16-wide k step are
// read from LDS while the current step's MFMAs issue.
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

// MODE_GATE_UP_BWD recomputes the gate_up product of the backward pass: its
// epilogue stores A again and dH = dA * d act (dA read from `din`).
// MODE_WGRAD computes per-expert weight gradients C[e] = A_e . B_e^T, where
// A and B are [M or N rows, K] operands whose K columns are the expert's
// padded row segment seg[e] .. seg[e+1] (a multiple of 64, zero padded).
enum { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_GATE_UP_BWD = 2, MODE_WGRAD = 3 };
enum { FMT_CONCAT = 0, FMT_INTERLEAVED = 1 };

static constexpr int BM = 256, BN = 256, BK = 64;
static constexpr int NSTAGE_A = 2, NSTAGE_B = 3;                 // LDS buffers per operand
static constexpr int WAVES_M = 2, WAVES_N = 4;                   // 8 waves, 2 per SIMD
static constexpr int NTHREADS = 64 * WAVES_M * WAVES_N;
static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;     // wave tile 128 x 64
static constexpr int MI = WTM / 32, NI = WTN / 32;               // 32x32 MFMA blocks per wave
static constexpr int CPR = BK / 8;                               // 16-byte chunks per tile row
static constexpr int RPB = 1024 / (BK * 2);                      // tile rows per 1 KB load block
static constexpr int LPW_A = (BM * BK * 2 / 1024) / (WAVES_M * WAVES_N);  // 1 KB loads per wave, A
static constexpr int LPW_B = (BN * BK * 2 / 1024) / (WAVES_M * WAVES_N);  // 1 KB loads per wave, B
static constexpr int KKS = BK / 16;                              // 16-wide k steps per stage
static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;       // bf16 elements per operand stage
static constexpr int LDS_BYTES_TILES = (NSTAGE_A * A_ELEMS + NSTAGE_B * B_ELEMS) * 2;  // 160 KB

// Buffer resource word 3 for raw (unformatted) dword accesses on gfx9 parts.
static constexpr int BUF_DWORD3 = 0x00020000;
// A load offset beyond the 0x7fffffff-byte range of the buffer resources
// (with room for any k offset added to or taken from it): out-of-range
// buffer loads return zeros without touching memory.
static constexpr uint32_t OOB_OFFSET = 0xC0000000u;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;

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
  // split-K of the last, partly filled round of tiles (nullptr: off)
  float* partial;      // split_slots tiles of BM x BN fp32 partial sums
  int32_t* counters;   // one arrival counter per split tile, zero on entry
  int split_slots;     // capacity of `partial` in tiles
  int G;               // workgroups resident at once (one per CU)
  int32_t* zero;       // counters this launch clears for the next one (or nullptr)
  int n_zero;
  // MODE_GATE_UP_BWD
  const uint16_t* din;  // dA, bf16 [rows, N]
  int64_t ld_din;
  void* out2;           // dH, bf16 [rows, 2N] in W_gu's column order
  int64_t ldo2;
  // MODE_WGRAD
  const int32_t* seg;   // [L+1] padded K segment of each expert
  int M;                // rows of the A operand
  int64_t out_estride;  // elements between experts' outputs
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

// Workgroup barrier that publishes this wave's LDS writes (ds_write and the
// buffer loads into LDS it has already waited for) without draining the
// loads still in flight: __syncthreads() would add a full vmcnt(0) wait for
// the outstanding loads into LDS.  The memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// B_IO: the weights in the StackedMoE page's stacked layout, each expert
// [K, N_total] with the output columns contiguous (IN_OUT), instead of the
// transposed [N, K] view (OUT_IN).  A weight stage is then 64 k-rows of the
// tile's 256 columns (512 bytes each), whose 64-byte spans are XOR-swizzled
// by (k-row & 7); the MFMA fragments (8 consecutive k of one column per lane)
// are read with two transposing LDS reads (ds_read_b64_tr_b16) each.
template <int MODE, int ACT, int FMT, bool GATHER, bool OUT_BF16, bool B_IO = false>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm_bf16_kernel(const GemmArgs p) {
  static_assert(!B_IO || MODE == MODE_DOWN || (MODE == MODE_GATE_UP && FMT == FMT_CONCAT),
                "stacked (IN_OUT) weights: the forward GEMMs, concatenated gate_up");
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* As = (uint16_t*)smem;
  uint16_t* Bs = As + NSTAGE_A * A_ELEMS;
  // the m-block prefix is only needed to map this workgroup to its tile; it
  // shares LDS with the operand buffers, which are filled after that
  int32_t* s_mbp = (int32_t*)smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int L = p.L;
  if (p.zero && blockIdx.x == 0)
    for (int i = tid; i < p.n_zero; i += NTHREADS) p.zero[i] = 0;

  constexpr bool GU = (MODE == MODE_GATE_UP || MODE == MODE_GATE_UP_BWD);
  constexpr int NBO = GU ? BN / 2 : BN;  // output columns per tile
  // the tile: expert e, column block nb, row block mb over rows [row_beg, row_end)
  int e, nb, mb, row_beg, row_end, K;
  int tile = 0, part = 0, S = 1, full = 0;
  bool split = false;
  const char* a_base;
  const char* b_base;
  if constexpr (MODE == MODE_WGRAD) {
    // fixed M x N per expert: tiles expert-major, then column block, then
    // row block, each XCD one contiguous range
    const int nmb_w = (p.M + BM - 1) / BM, per_e = nmb_w * ((p.N + BN - 1) / BN);
    const int total = L * per_e, per_xcd = (total + 7) >> 3, slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return;
    const int t = (blockIdx.x & 7) * per_xcd + slot;
    if (t >= total) return;
    e = __builtin_amdgcn_readfirstlane(t / per_e);
    // within an expert: bands of 8 row blocks, each walked column block by
    // column block, so that the 32 tiles one XCD runs together are 8 row
    // blocks x 4 column blocks and share both operands in its L2
    const int local = t % per_e, NBW = (p.N + BN - 1) / BN;
    const int full_rows = nmb_w / 8 * 8;
    int nb_, mb_;
    if (local < full_rows * NBW) {
      const int band = local / (8 * NBW), r = local % (8 * NBW);
      nb_ = r / 8;
      mb_ = band * 8 + r % 8;
    } else {
      const int r = local - full_rows * NBW, h = nmb_w - full_rows;
      nb_ = r / h;
      mb_ = full_rows + r % h;
    }
    nb = __builtin_amdgcn_readfirstlane(nb_);
    mb = __builtin_amdgcn_readfirstlane(mb_);
    row_beg = mb * BM;
    row_end = p.M;
    // the segment, clipped to the padded width of the operands (it only
    // exceeds it if the row offsets exceed the rows the buffers were sized for)
    const int width = (int)p.lda;
    const int seg0 = __builtin_amdgcn_readfirstlane(min(p.seg[e], width));
    K = __builtin_amdgcn_readfirstlane(max(min(p.seg[e + 1], width) - seg0, 0));
    a_base = (const char*)(p.A + seg0);
    b_base = (const char*)(p.W + seg0);
  } else {

  // ---- prefix of 256-row blocks per expert (wave 0), in LDS
  if (wave == 0) wave_expert_prefix(p.offsets, L, s_mbp, [](int rows) { return (rows + BM - 1) / BM; });
  __syncthreads();

  const int NB = (p.N + NBO - 1) / NBO;
  const int total = s_mbp[L] * NB;
  // Tiles run in rounds of G (one workgroup per CU).  When the last round is
  // at most half full, its `rem` tiles are split along K into S parts each
  // so that it fills the chip; the last part to finish adds the S partial
  // sums in a fixed order and runs the epilogue.
  int rem = 0;
  if (p.partial && p.G > 0) {
    const int r = total % p.G;
    if (r > 0 && 2 * r <= p.G) {
      S = min(min(4, p.G / r), p.split_slots / r);
      S = min(S, (p.K + BK - 1) / BK / 4);  // at least 4 k stages per part
      if (S >= 2) rem = r;
      else S = 1;
    }
  }
  full = total - rem;  // a multiple of G (and of 8) when splitting
  const int slot = blockIdx.x >> 3;
  if (rem == 0) {
    const int per_xcd = (total + 7) >> 3;
    if (slot >= per_xcd) return;
    tile = (blockIdx.x & 7) * per_xcd + slot;
    if (tile >= total) return;
  } else {
    // each XCD runs its share of the whole tiles, then all the parts of its
    // share of the split tiles (the parts of one tile meet in one L2)
    const int full_x = full >> 3, parts_x = ((rem + 7) >> 3) * S;
    if (slot >= full_x + parts_x) return;
    if (slot < full_x) {
      tile = (blockIdx.x & 7) * full_x + slot;
    } else {
      const int j = (blockIdx.x & 7) * parts_x + (slot - full_x);
      if (j >= rem * S) return;
      tile = full + j / S;
      part = j % S;
    }
  }
  split = tile >= full && rem > 0;

  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_mbp[mid] * NB <= tile) lo = mid;
    else hi = mid - 1;
  }
  // uniform by construction; made scalar so that every address base below
  // lives in SGPRs
  e = __builtin_amdgcn_readfirstlane(lo);
  const int nmb = s_mbp[e + 1] - s_mbp[e];
  const int local = __builtin_amdgcn_readfirstlane(tile - s_mbp[e] * NB);
  nb = local / nmb;
  mb = local % nmb;
  row_beg = __builtin_amdgcn_readfirstlane(p.offsets[e] + mb * BM);
  row_end = __builtin_amdgcn_readfirstlane(p.offsets[e + 1]);
  K = p.K;
  // permuted rows: the buffer resource starts at the tile's first row (a
  // 64-bit base), so the 32-bit offsets span one tile and the row buffer
  // itself may exceed the 2 GiB a buffer resource addresses; gathered rows
  // are addressed from x by token
  a_base = GATHER ? (const char*)p.X : (const char*)p.A + (int64_t)row_beg * p.lda * 2;
  b_base = (const char*)(p.W + (int64_t)e * p.w_estride);
  __syncthreads();  // every wave has read the prefix before the loads overwrite it
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // ---- loader: buffer loads straight into LDS (buffer_load_dwordx4 ... lds),
  // no VGPR staging.  One instruction moves a 1 KB block of RPB tile rows x
  // CPR chunks; lane l lands at row RPB*blk + l/CPR, physical chunk l%CPR,
  // so it fetches the logical chunk (l%CPR) ^ f(row).  Wave w moves blocks
  // LPW*w .. LPW*w+LPW-1 of both operands.  The per-lane byte offset (row and
  // swizzled chunk) is fixed for the tile; the k offset of a stage goes in
  // the scalar offset and the LDS destination in M0, so a load costs no
  // vector instruction.
  const int lrow = lane / CPR;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, 0x7fffffff, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, 0x7fffffff, BUF_DWORD3);
  const uint32_t a_row_bytes = (uint32_t)p.lda * 2u, b_row_bytes = (uint32_t)p.ldb * 2u;
  // the swizzled chunk this lane fetches for load block i (recomputed where
  // needed rather than kept in registers)
  auto a_chunk = [&](int i) { return (lane % CPR) ^ swz_f((wave * LPW_A + i) * RPB + lrow); };
  auto b_chunk = [&](int i) { return (lane % CPR) ^ swz_f((wave * LPW_B + i) * RPB + lrow); };
  // byte offset of this lane's row plus its chunk, fixed for the tile
  uint32_t a_voff[LPW_A], b_voff[LPW_B];
  // A wave whose activation rows (one 32-row block) all lie past the tile's
  // last row points their loads past the end of the buffer range, where they
  // fetch nothing: an output row depends on its own activation row only, and
  // rows past the end are neither computed nor stored.
  const bool a_live = row_beg + wave * LPW_A * RPB < row_end;
#pragma unroll
  for (int i = 0; i < LPW_A; ++i) {
    const int trow = (wave * LPW_A + i) * RPB + lrow;  // tile row
    const int r = min(row_beg + trow, row_end - 1);
    // row offset from the base: the token (gathered), the row within the
    // tile (permuted rows, rebased), or the weight-gradient operand's row
    const uint32_t arow = GATHER ? (uint32_t)p.sorted_token[r] : (uint32_t)(r - (MODE == MODE_WGRAD ? 0 : row_beg));
    a_voff[i] = a_live ? arow * a_row_bytes + (uint32_t)a_chunk(i) * 16u : OOB_OFFSET;
  }
#pragma unroll
  for (int i = 0; i < LPW_B; ++i) {
    if constexpr (B_IO) {
      // 1 KB = 2 k-rows of 32 chunks: lane l lands at k-row 2*blk + l/32,
      // physical chunk l%32, and fetches the tile columns of logical chunk
      // (l%32) ^ ((k-row & 7) << 2)
      const int r = 2 * (wave * LPW_B + i) + (lane >> 5);
      const int t = ((lane & 31) ^ ((r & 7) << 2)) * 8;  // first tile column of the chunk
      int gcol;
      if (MODE == MODE_DOWN) {
        gcol = min(nb * BN + t, p.N - 8);
      } else {
        // concatenated: wave column q holds WTN/2 gate columns, then the matching up columns
        const int q = t / WTN, rr = t % WTN, isup = rr / (WTN / 2), j = rr % (WTN / 2);
        const int oc = min(nb * NBO + q * (WTN / 2) + j, p.N - 8);
        gcol = isup ? p.N + oc : oc;
      }
      b_voff[i] = (uint32_t)r * b_row_bytes + (uint32_t)gcol * 2u;
      continue;
    }
    const int trow = (wave * LPW_B + i) * RPB + lrow;  // tile row
    int wrow;
    if (MODE == MODE_DOWN || MODE == MODE_WGRAD) {
      wrow = min(nb * BN + trow, p.N - 1);
    } else {
      // B rows of wave column q: WTN/2 gate rows, then the matching up rows
      const int q = trow / WTN, rr = trow % WTN, isup = rr / (WTN / 2), j = rr % (WTN / 2);
      const int oc = min(nb * NBO + q * (WTN / 2) + j, p.N - 1);
      wrow = (FMT == FMT_CONCAT) ? (isup ? p.N + oc : oc) : (2 * oc + isup);
    }
    b_voff[i] = (uint32_t)wrow * b_row_bytes + (uint32_t)b_chunk(i) * 16u;
  }
  const int KTF = K / BK;              // full k stages
  const int KT_ALL = (K + BK - 1) / BK;  // all k stages (the last may be ragged)
  // this workgroup's k stages [KB, KT): all of them, or one part of a split tile
  const int KB = split ? part * KT_ALL / S : 0;
  const int KT = split ? (part + 1) * KT_ALL / S : KT_ALL;

  // A (activation rows) is double buffered, B (weight rows) triple buffered.
  // Stage kt's A goes to buffer kt % 2 and its B to buffer kt % 3.
  auto issue_a = [&](int kt) {
    lptr_t dst = (lptr_t)(As + (kt % NSTAGE_A) * A_ELEMS + wave_s * LPW_A * 512);
    if (kt < KTF) {
#pragma unroll
      for (int i = 0; i < LPW_A; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)((char*)dst + i * 1024), 16, a_voff[i], kt * (BK * 2), 0, 0);
    } else {
      // the ragged last stage is clamped to stay inside each row; its A
      // chunks past K are zeroed in LDS before the stage is published
#pragma unroll
      for (int i = 0; i < LPW_A; ++i) {
        const int c = a_chunk(i);
        const uint32_t kb = (uint32_t)min(kt * BK + c * 8, K - 8) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lptr_t)((char*)dst + i * 1024), 16,
                                                 a_voff[i] - (uint32_t)c * 16u + kb, 0, 0, 0);
      }
    }
  };
  auto issue_b = [&](int kt) {
    lptr_t dst = (lptr_t)(Bs + (kt % NSTAGE_B) * B_ELEMS + wave_s * LPW_B * 512);
    if constexpr (B_IO) {
      if (kt < KTF) {
#pragma unroll
        for (int i = 0; i < LPW_B; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)((char*)dst + i * 1024), 16, b_voff[i],
                                                   (uint32_t)kt * BK * b_row_bytes, 0, 0);
      } else {
        // the ragged last stage: k-rows past K read row K - 1 (finite weights
        // under the zeroed A chunks)
#pragma unroll
        for (int i = 0; i < LPW_B; ++i) {
          const uint32_t r = 2u * (uint32_t)(wave_s * LPW_B + i) + ((uint32_t)lane >> 5);
          const uint32_t kr = (uint32_t)min(kt * BK + (int)r, K - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)((char*)dst + i * 1024), 16,
                                                   b_voff[i] - r * b_row_bytes + kr * b_row_bytes, 0, 0, 0);
        }
      }
      return;
    }
    if (kt < KTF) {
#pragma unroll
      for (int i = 0; i < LPW_B; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)((char*)dst + i * 1024), 16, b_voff[i], kt * (BK * 2), 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < LPW_B; ++i) {
        const int c = b_chunk(i);
        const uint32_t kb = (uint32_t)min(kt * BK + c * 8, K - 8) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lptr_t)((char*)dst + i * 1024), 16,
                                                 b_voff[i] - (uint32_t)c * 16u + kb, 0, 0, 0);
      }
    }
  };
  // Issue order: A0 B0 B1 A1 B2 | in iteration kt: A(kt+2) B(kt+3).  When
  // stage kt+1 is needed (end of iteration kt) the only loads issued after
  // A(kt+1) are B(kt+2), so vmcnt(LPW_B) means A(kt+1) and B(kt+1) landed.
  auto wait_next = [&](int kt) {
    if (kt + 2 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW_B));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  };
  // ragged K: after this wave's loads of stage kt landed, overwrite the A
  // chunks it fetched past K with zeros (B there holds finite weights); the
  // barrier that publishes the stage orders these writes
  auto zero_tail = [&](int kt) {
    if (kt * BK + BK > K) {
      uint16_t* as = As + (kt % NSTAGE_A) * A_ELEMS + wave_s * LPW_A * 512;
      const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < LPW_A; ++i)
        if (kt * BK + a_chunk(i) * 8 >= K) *(u32x4_t*)(as + i * 512 + lane * 8) = z;
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
    const uint16_t* as = As + (kt % NSTAGE_A) * A_ELEMS;
    const uint16_t* bs = Bs + (kt % NSTAGE_B) * B_ELEMS;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      af[mi] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(as + swz(wm * WTM + mi * 32 + fr, kk * 2 + fk)));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      if constexpr (B_IO) {
        // lane l holds column l%32 of the block, k rows 8(l/32) .. +8: in
        // each 16-lane group g, lane i addresses k-row 8(g>>1) + (i>>2) (and
        // + 4) at columns 16(g&1) + 4(i&3) .. +4, and the transposing read
        // hands it 4 consecutive k of column 16(g&1) + i
        const int g = lane >> 4, i = lane & 15;
        const int r0 = kk * 16 + 8 * (g >> 1) + (i >> 2);
        const int col = wn * WTN + ni * 32 + 16 * (g & 1) + 4 * (i & 3);
        auto at = [&](int r) {
          return (lds_v4i16_ptr)(bs + r * BN + (((col >> 3) ^ ((r & 7) << 2)) << 3) + (col & 7));
        };
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(r0));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(at(r0 + 4));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        bfr[ni] = __builtin_bit_cast(bf16x8_t, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
      } else {
        bfr[ni] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(bs + swz(wn * WTN + ni * 32 + fr, kk * 2 + fk)));
      }
    }
  };
  // 32-row blocks of this wave that hold rows of the expert: the last m-block
  // of an expert is usually partly empty, and its empty blocks skip their
  // MFMAs (nothing is stored for those rows)
  const int wm_s = wave_s / WAVES_N;
  const int live_mi = min(max((row_end - (row_beg + wm_s * WTM) + 31) / 32, 0), MI);
  auto mfmas = [&](const bf16x8_t (&af)[MI], const bf16x8_t (&bfr)[NI], auto full) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      if (FULL || mi < live_mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
  };

  // ---- main loop.  The KKS 16-wide k steps of stage kt run as
  //   [MFMAs (kt,kk) interleaved with the fragment reads of (kt,kk+1)]
  // for kk < KKS-1, then
  //   wait for stage kt+1, barrier, fragment reads (kt+1,0),
  //   [MFMAs (kt,KKS-1) interleaved with the loads of A(kt+2), B(kt+3)]
  // so that neither the LDS reads nor the load issue ever hold up the matrix
  // pipe; two waves per SIMD cover each other's barrier and wait stalls.
  // Iterations whose loads are all full stages run without branches.
  bf16x8_t fa[2][MI], fb[2][NI];
  // LDS read instructions per k step: one per fragment, two per weight
  // fragment read transposed
  constexpr int NREADS = MI + (B_IO ? 2 : 1) * NI;
  auto iteration = [&](int kt, auto steady, auto full) {
    constexpr bool STEADY = decltype(steady)::value;
#pragma unroll
    for (int kk = 0; kk < KKS; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < KKS) {
        read_frags(kt, kk + 1, fa[c ^ 1], fb[c ^ 1]);
        mfmas(fa[c], fb[c], full);
#pragma unroll
        for (int j = 0; j < MI * NI; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (j < NREADS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
      } else {
        if (STEADY) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW_B));
        } else if (kt + 1 < KT) {
          wait_next(kt);
          zero_tail(kt + 1);
        }
        block_barrier();
        if (STEADY || kt + 1 < KT) read_frags(kt + 1, 0, fa[c ^ 1], fb[c ^ 1]);
        if (STEADY || kt + 2 < KT) issue_a(kt + 2);
        if (STEADY || kt + 3 < KT) issue_b(kt + 3);
        mfmas(fa[c], fb[c], full);
        __builtin_amdgcn_sched_group_barrier(0x100, NREADS, 0);  // DS reads first
#pragma unroll
        for (int j = 0; j < MI * NI; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // buffer load
        }
      }
      // no wait here: the compiler waits for each fragment where an MFMA
      // first uses it, so the next step's early MFMAs overlap the tail of
      // this step's reads
    }
  };

  const int NK = KT - KB;  // stages of this workgroup (0 only for an empty weight-gradient segment)
  if (NK > 0) {
  issue_a(KB);
  issue_b(KB);
  if (NK > 1) issue_b(KB + 1);
  if (NK > 1) issue_a(KB + 1);
  if (NK > 2) issue_b(KB + 2);
  if (NK > 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPW_B + LPW_A));
  else if (NK > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW_B + LPW_A));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  zero_tail(KB);
  block_barrier();
  read_frags(KB, 0, fa[0], fb[0]);
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  const int k_steady = min(KTF, KT) - 3;  // iterations whose loads are all full stages
  int kt = KB;
  if (live_mi == MI) {
    for (; kt < k_steady; ++kt) iteration(kt, std::true_type{}, std::true_type{});
    for (; kt < KT; ++kt) iteration(kt, std::false_type{}, std::true_type{});
  } else {
    for (; kt < k_steady; ++kt) iteration(kt, std::true_type{}, std::false_type{});
    for (; kt < KT; ++kt) iteration(kt, std::false_type{}, std::false_type{});
  }
  }

  // ---- epilogue.  The weight fragment is the MFMA's first operand, so the
  // accumulators hold the transposed block: acc[mi][ni][r] is C[row][col] with
  //   row = wm*WTM + mi*32 + fr,  col = wn*WTN + ni*32 + 8*(r/4) + 4*fk + r%4
  // and every lane owns four consecutive columns of one row per r/4, written
  // with one 8-byte (bf16) or 16-byte (fp32) store.  Column counts and row
  // pitches are multiples of 8, so these stores are aligned.
  if (split) {
    // publish this part's partial sums, then let the last part of the tile
    // (in arrival order) add all parts in part order
    float* mine = p.partial + ((int64_t)(tile - full) * S + part) * (BM * BN);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v = {acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]};
          *(f32x4_t*)(mine + ((((mi * NI + ni) * 4 + q) * NTHREADS) + tid) * 4) = v;
        }
    // The barrier orders every wave's partial stores before thread 0's
    // agent-scope release (one L2 write-back for the workgroup); the last
    // part's thread 0 acquires once, and the barrier orders the other waves'
    // partial loads after it.
    __syncthreads();
    int32_t* s_flag = (int32_t*)smem;
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int old = __hip_atomic_fetch_add(&p.counters[tile - full], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag[0] = (old == S - 1);
      if (old == S - 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        // every part has counted in: ready for the next launch
        __hip_atomic_store(&p.counters[tile - full], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (s_flag[0] == 0) return;
    const float* first = p.partial + (int64_t)(tile - full) * S * (BM * BN);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t idx = ((((mi * NI + ni) * 4 + q) * NTHREADS) + tid) * 4;
          f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)(first + idx));
          for (int t = 1; t < S; ++t) v += __builtin_nontemporal_load((const f32x4_t*)(first + (int64_t)t * (BM * BN) + idx));
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[mi][ni][4 * q + c] = v[c];
        }
  }

  const float sc = p.escale ? p.escale[e] : 1.0f;
  const uint16_t* bias_e = p.bias ? p.bias + (int64_t)e * p.bias_estride : nullptr;
  if constexpr (GU) {
    // Blocks ni < NI/2 hold gate columns, ni + NI/2 the up columns of the
    // same outputs.  The bf16 results go through LDS so that they leave as
    // whole tile rows: first A (256 rows x 128 outputs), then, for the
    // backward recompute, dH (256 rows x 256 columns in W_gu's order), its
    // gradients recomputed from the accumulators still in registers.
    uint16_t* stg = (uint16_t*)smem;
    constexpr int AROW = NBO + 8, HROW = 2 * NBO + 8;  // staged row pitches (bf16), padded
    static_assert(BM * HROW * 2 <= LDS_BYTES_TILES, "staged epilogue exceeds LDS");
    auto bias_of = [&](int oc, float (&bg)[4], float (&bu)[4]) {
      for (int c = 0; c < 4; ++c) bg[c] = bu[c] = 0.0f;
      if (!bias_e) return;
      gate_up_bias_x4(bias_e, p.N, oc, FMT != FMT_CONCAT, bg, bu);
    };
    // ---- A
    __syncthreads();  // the operand tiles are no longer read
#pragma unroll
    for (int ni = 0; ni < NI / 2; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ocl = wn * (WTN / 2) + ni * 32 + 8 * q + 4 * fk;  // tile output of 4
        const int oc = nb * NBO + ocl;
        float bg[4], bu[4];
        if (oc < p.N) bias_of(oc, bg, bu);  // N is a multiple of 8: all 4 are in range
        else for (int c = 0; c < 4; ++c) bg[c] = bu[c] = 0.0f;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          float a[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            a[c] = gated_act<ACT>(acc[mi][ni][4 * q + c] * sc + bg[c], acc[mi][ni + NI / 2][4 * q + c] * sc + bu[c],
                                  p.alpha, p.limit);
          uint2 v;
          v.x = pack_bf16x2_rne(a[0], a[1]);
          v.y = pack_bf16x2_rne(a[2], a[3]);
          *(uint2*)(stg + (wm * WTM + mi * 32 + fr) * AROW + ocl) = v;
        }
      }
    __syncthreads();
    {
      uint16_t* out = (uint16_t*)p.out;
      const int oc = nb * NBO + (lane & 15) * 8;  // 16 lanes per 256-byte row
      for (int r = wave * 4 + (lane >> 4); r < BM; r += 4 * WAVES_M * WAVES_N) {
        const int row = row_beg + r;
        if (row < row_end && oc < p.N)
          *(u32x4_t*)(out + (int64_t)row * p.ldo + oc) = *(const u32x4_t*)(stg + r * AROW + (lane & 15) * 8);
      }
    }
    if (MODE == MODE_GATE_UP_BWD) {
      // ---- dH = dA * d act, staged in W_gu's column order for this tile:
      // concatenated [128 gate | 128 up], interleaved gate/up pairs
      __syncthreads();
#pragma unroll
      for (int ni = 0; ni < NI / 2; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ocl = wn * (WTN / 2) + ni * 32 + 8 * q + 4 * fk;
          const int oc = nb * NBO + ocl;
          float bg[4], bu[4];
          if (oc < p.N) bias_of(oc, bg, bu);
          else for (int c = 0; c < 4; ++c) bg[c] = bu[c] = 0.0f;
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            const int rl = wm * WTM + mi * 32 + fr;
            const int row = row_beg + rl;
            float da[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (row < row_end && oc < p.N) {
              const uint2 d2 = *(const uint2*)(p.din + (int64_t)row * p.ld_din + oc);
              da[0] = bf16_to_f32(d2.x & 0xffffu); da[1] = bf16_to_f32(d2.x >> 16);
              da[2] = bf16_to_f32(d2.y & 0xffffu); da[3] = bf16_to_f32(d2.y >> 16);
            }
            float a, dg[4], du[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              gated_act_grad<ACT>(acc[mi][ni][4 * q + c] * sc + bg[c], acc[mi][ni + NI / 2][4 * q + c] * sc + bu[c],
                                  p.alpha, p.limit, a, dg[c], du[c]);
              dg[c] *= da[c];
              du[c] *= da[c];
            }
            uint16_t* srow = stg + rl * HROW;
            if (FMT == FMT_CONCAT) {
              uint2 g2, u2;
              g2.x = pack_bf16x2_rne(dg[0], dg[1]);
              g2.y = pack_bf16x2_rne(dg[2], dg[3]);
              u2.x = pack_bf16x2_rne(du[0], du[1]);
              u2.y = pack_bf16x2_rne(du[2], du[3]);
              *(uint2*)(srow + ocl) = g2;
              *(uint2*)(srow + NBO + ocl) = u2;
            } else {
              const u32x4_t w4 = {pack_bf16x2_rne(dg[0], du[0]), pack_bf16x2_rne(dg[1], du[1]),
                                  pack_bf16x2_rne(dg[2], du[2]), pack_bf16x2_rne(dg[3], du[3])};
              *(u32x4_t*)(srow + 2 * ocl) = w4;
            }
          }
        }
      __syncthreads();
      // 512-byte staged rows, 32 lanes each; staged column j holds
      //   concatenated: gate (j < NBO) or up (j >= NBO) of output j mod NBO
      //   interleaved:  column 2 * nb * NBO + j of dH
      uint16_t* dh = (uint16_t*)p.out2;
      const int j = (lane & 31) * 8;
      const int oc = nb * NBO + (FMT == FMT_CONCAT ? j % NBO : j / 2);  // first output these 8 columns belong to
      const int64_t col = (FMT == FMT_CONCAT) ? (j < NBO ? (int64_t)nb * NBO + j : (int64_t)p.N + nb * NBO + j - NBO)
                                              : (int64_t)2 * nb * NBO + j;
      for (int r = wave * 2 + (lane >> 5); r < BM; r += 2 * WAVES_M * WAVES_N) {
        const int row = row_beg + r;
        if (row < row_end && oc < p.N)
          *(u32x4_t*)(dh + (int64_t)row * p.ldo2 + col) = *(const u32x4_t*)(stg + r * HROW + j);
      }
    }
  } else if constexpr (!OUT_BF16) {
    // fp32 output through LDS, one 128-row half of the tile at a time: the
    // wave row that owns the half writes its accumulators into LDS, then
    // every wave stores whole 1 KB output rows (one contiguous 16 bytes per
    // lane), instead of 32-byte pieces of 32 rows per store instruction.
    // A weight gradient goes to its expert's block of the output.
    float* out_e = (float*)p.out + (MODE == MODE_WGRAD ? (int64_t)e * p.out_estride : 0);
    float* stage = (float*)smem;  // [WTM][SROW]; the padding spreads the rows over the banks
    constexpr int SROW = BN + 4;
    static_assert(WTM * SROW * 4 <= LDS_BYTES_TILES, "staged epilogue exceeds LDS");
#pragma unroll
    for (int half = 0; half < WAVES_M; ++half) {
      __syncthreads();  // the tiles (or the previous half) are no longer read
      if (wm == half) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = wn * WTN + ni * 32 + 8 * q + 4 * fk;  // tile column of 4
            const int n = nb * BN + nl;
            float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (bias_e && n < p.N) {
              bias_x4(bias_e + n, bd);
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
              const f32x4_t v = {acc[mi][ni][4 * q] * sc + bd[0], acc[mi][ni][4 * q + 1] * sc + bd[1],
                                 acc[mi][ni][4 * q + 2] * sc + bd[2], acc[mi][ni][4 * q + 3] * sc + bd[3]};
              *(f32x4_t*)(stage + (mi * 32 + fr) * SROW + nl) = v;
            }
          }
      }
      __syncthreads();
      const int n = nb * BN + lane * 4;
      for (int rr = wave; rr < WTM; rr += WAVES_M * WAVES_N) {
        const int row = row_beg + half * WTM + rr;
        if (row < row_end && n < p.N)
          *(f32x4_t*)(out_e + (int64_t)row * p.ldo + n) = *(const f32x4_t*)(stage + rr * SROW + lane * 4);
      }
    }
  } else {
    // bf16 output through LDS (row pitch 528 bytes: 4 banks of skew per
    // row), so that each store moves whole 512-byte row pieces instead of 8
    // bytes of each of 32 rows per store instruction.
    constexpr int PITCH = BN * 2 + 16;
    static_assert(BM * PITCH <= LDS_BYTES_TILES, "staged epilogue exceeds LDS");
    uint8_t* stg = (uint8_t*)smem;
    __syncthreads();  // the operand tiles are no longer read
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * WTN + ni * 32 + 8 * q + 4 * fk;  // tile column of 4
        const int n = nb * BN + nl;
        float bd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias_e && n < p.N) {
          bias_x4(bias_e + n, bd);
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          uint2 w;
          w.x = pack_bf16x2_rne(acc[mi][ni][4 * q] * sc + bd[0], acc[mi][ni][4 * q + 1] * sc + bd[1]);
          w.y = pack_bf16x2_rne(acc[mi][ni][4 * q + 2] * sc + bd[2], acc[mi][ni][4 * q + 3] * sc + bd[3]);
          *(uint2*)(stg + (wm * WTM + mi * 32 + fr) * PITCH + nl * 2) = w;
        }
      }
    __syncthreads();
    uint16_t* out_e = (uint16_t*)p.out;
    const int n = nb * BN + (lane & 31) * 8;  // 32 lanes per 512-byte row
    for (int r = wave * 2 + (lane >> 5); r < BM; r += 2 * WAVES_M * WAVES_N) {
      const int row = row_beg + r;
      if (row < row_end && n < p.N)
        *(u32x4_t*)(out_e + (int64_t)row * p.ldo + n) = *(const u32x4_t*)(stg + r * PITCH + (lane & 31) * 16);
    }
  }
}

template <typename KernelT>
static hipError_t launch_gemm(KernelT kern, const GemmArgs& a, int max_rows, int NBO,
                              hipStream_t st) {
  const int prefix = (a.L + 1) * (int)sizeof(int32_t);
  const int lds = LDS_BYTES_TILES > prefix ? LDS_BYTES_TILES : prefix;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t nonempty = (int64_t)max_rows < a.L ? max_rows : a.L;
  const int64_t mblocks = (max_rows + BM - 1) / BM + nonempty;
  const int64_t NB = (a.N + NBO - 1) / NBO;
  const int64_t max_tiles = mblocks * NB;
  // with the split tail round each XCD runs at most G/8 + 4 more workgroups
  const int64_t extra = a.partial ? a.G / 8 + 4 : 0;
  const int64_t grid = ((max_tiles + 7) / 8 + extra) * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, NTHREADS, lds, st>>>(a);
  return hipGetLastError();
}

template <int ACT, int FMT, bool GATHER>
static hipError_t gate_up_dispatch(const GemmArgs& a, bool in_out, int max_rows, hipStream_t st) {
  if constexpr (FMT == FMT_CONCAT) {
    if (in_out)
      return launch_gemm(grouped_gemm_bf16_kernel<MODE_GATE_UP, ACT, FMT, GATHER, true, true>, a, max_rows, BN / 2, st);
  }
  return launch_gemm(grouped_gemm_bf16_kernel<MODE_GATE_UP, ACT, FMT, GATHER, true>, a, max_rows, BN / 2, st);
}

// Compute units of the current device (one GEMM workgroup each), cached per device.
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = n;
  return n;
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
  g.ldb = q.gu_in_out ? 2 * (int64_t)q.D : q.H;  // weight row pitch: [H, 2D] stacked or [2D, H]
  g.zero = q.split_counters;  // the down GEMM's arrival counters start at zero
  g.n_zero = q.split_counters ? SPLIT_COUNTERS : 0;
  const bool gather = (q.x_perm == nullptr);
  hipError_t err;
  if (q.events && (err = hipEventRecord(q.events[0], st)) != hipSuccess) return err;
#define GU(ACTV, FMTV)                                                                             \
  err = gather ? gate_up_dispatch<ACTV, FMTV, true>(g, q.gu_in_out != 0, q.max_rows, st)          \
               : gate_up_dispatch<ACTV, FMTV, false>(g, q.gu_in_out != 0, q.max_rows, st)
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
  d.ldb = q.d_in_out ? q.H : q.D;  // weight row pitch: [D, H] stacked or [H, D]
  if (q.split_partial && q.split_slots > 0) {
    d.partial = q.split_partial;
    d.counters = q.split_counters;
    d.split_slots = q.split_slots < SPLIT_COUNTERS ? q.split_slots : SPLIT_COUNTERS;
    d.G = cu_count();
  }
  if (q.d_in_out) {
    if (q.out_bf16)
      err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, true, true>, d, q.max_rows, BN, st);
    else
      err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, false, true>, d, q.max_rows, BN, st);
  } else if (q.out_bf16) {
    err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, true>, d, q.max_rows, BN, st);
  } else {
    err = launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, false>, d, q.max_rows, BN, st);
  }
  if (err == hipSuccess && q.events) err = hipEventRecord(q.events[2], st);
  return err;
}

// ---------------------------------------------------------------- backward GEMMs

static GemmArgs bwd_args(const BwdGemm& b) {
  GemmArgs g{};
  g.offsets = b.offsets;
  g.L = b.L;
  g.K = b.K;
  g.N = b.N;
  g.A = b.A;
  g.X = b.X;
  g.sorted_token = b.sorted_token;
  g.W = b.W;
  g.w_estride = b.w_estride;
  g.lda = b.lda;
  g.ldb = b.ldb;
  g.bias = b.bias;
  g.bias_estride = 2 * (int64_t)b.N;
  g.escale = b.escale;
  g.alpha = b.alpha;
  g.limit = b.limit;
  g.out = b.out;
  g.ldo = b.ldo;
  g.din = b.din;
  g.ld_din = b.ld_din;
  g.out2 = b.out2;
  g.ldo2 = b.ldo2;
  g.seg = b.seg;
  g.M = b.M;
  g.out_estride = b.out_estride;
  return g;
}

hipError_t launch_bwd_rows_gemm(const BwdGemm& b, hipStream_t st) {
  const GemmArgs g = bwd_args(b);
  if (b.out_bf16)
    return launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, true>, g, b.max_rows, BN, st);
  return launch_gemm(grouped_gemm_bf16_kernel<MODE_DOWN, ACT_SILU, FMT_CONCAT, false, false>, g, b.max_rows, BN, st);
}

template <int ACT, int FMT>
static hipError_t gate_up_bwd_dispatch(const GemmArgs& g, bool gather, int max_rows, hipStream_t st) {
  if (gather)
    return launch_gemm(grouped_gemm_bf16_kernel<MODE_GATE_UP_BWD, ACT, FMT, true, true>, g, max_rows, BN / 2, st);
  return launch_gemm(grouped_gemm_bf16_kernel<MODE_GATE_UP_BWD, ACT, FMT, false, true>, g, max_rows, BN / 2, st);
}

hipError_t launch_bwd_gate_up_gemm(const BwdGemm& b, hipStream_t st) {
  const GemmArgs g = bwd_args(b);
  const bool gather = b.A == nullptr;
  if (b.fmt == FMT_CONCAT) {
    if (b.act_kind == ACT_SILU) return gate_up_bwd_dispatch<ACT_SILU, FMT_CONCAT>(g, gather, b.max_rows, st);
    if (b.act_kind == ACT_SWIGLUOAI) return gate_up_bwd_dispatch<ACT_SWIGLUOAI, FMT_CONCAT>(g, gather, b.max_rows, st);
    return gate_up_bwd_dispatch<ACT_GELU_TANH, FMT_CONCAT>(g, gather, b.max_rows, st);
  }
  if (b.act_kind == ACT_SILU) return gate_up_bwd_dispatch<ACT_SILU, FMT_INTERLEAVED>(g, gather, b.max_rows, st);
  if (b.act_kind == ACT_SWIGLUOAI) return gate_up_bwd_dispatch<ACT_SWIGLUOAI, FMT_INTERLEAVED>(g, gather, b.max_rows, st);
  return gate_up_bwd_dispatch<ACT_GELU_TANH, FMT_INTERLEAVED>(g, gather, b.max_rows, st);
}

hipError_t launch_wgrad_gemm(const BwdGemm& b, hipStream_t st) {
  const GemmArgs g = bwd_args(b);
  auto kern = grouped_gemm_bf16_kernel<MODE_WGRAD, ACT_SILU, FMT_CONCAT, false, false>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES_TILES);
  if (err != hipSuccess) return err;
  const int64_t tiles = (int64_t)b.L * ((b.M + BM - 1) / BM) * ((b.N + BN - 1) / BN);
  const int64_t grid = (tiles + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<(unsigned)grid, NTHREADS, LDS_BYTES_TILES, st>>>(g);
  return hipGetLastError();
}

}  // namespace moe
