// MX block-scaled operands on gfx950 (OCP Microscaling formats: E2M1 and E4M3
// elements, one E8M0 scale per 32 elements along K), shared by the grouped MX
// GEMMs and the single-launch MX FFN.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 with the e2m1 operand
// first and the e4m3 operand second (measured with one-wave probes on
// gfx950): lane l = 32h + r holds row r.  Its 32 e2m1 codes all fall in the
// first 32 K slots (h = 0) or the last 32 (h = 1); of its 32 e4m3 bytes,
// bytes 0-15 fall in the first 32 slots and bytes 16-31 in the last 32.
// e2m1 code p of half 0 meets e4m3 byte p of half 0 (p < 16) or byte p-16 of
// half 1; e2m1 code p of half 1 meets e4m3 byte 16+p of half 0 (p < 16) or
// byte p of half 1.  The scale of the first 32 slots is lane r's, of the last
// 32 lane 32+r's.  So for the 64-wide k step kk, whose MX blocks are 2kk and
// 2kk+1:
//   e2m1 lane h: k [64kk+32h, +32)            = 16-byte chunk 2kk+h of the row
//   e4m3 lane h: k [64kk+16h, +16), [64kk+32+16h, +16) = chunks 4kk+h, 4kk+2+h
//   both pass the scale byte of block 2kk+h.
// (e2m1 element 2i is the low nibble of byte i, as the MFMA reads it.)
//
// k stages are 128 elements: an e4m3 stage row is 128 bytes (8 chunks of
// 16), a packed e2m1 stage row 64 bytes (4 chunks), and a row's 4 scale
// bytes of the stage form one dword.
#pragma once

#include "common.h"

namespace moe {

constexpr int MX_BK = 128;            // k elements per stage
constexpr int MX_A_ROW = MX_BK;       // bytes per e4m3 stage row
constexpr int MX_B_ROW = MX_BK / 2;   // bytes per packed e2m1 stage row

// e4m3 rows: chunk c of row r at c ^ fa(r).
__device__ __forceinline__ int mx_fa(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int mx_a_off(int row, int chunk) { return row * MX_A_ROW + ((chunk ^ mx_fa(row)) << 4); }
// e2m1 rows: chunk c of row r at c ^ fb(r), which puts the rows r, r+4, r+8,
// r+12 that share banks on four different chunks (the fragment reads of 32
// consecutive rows are conflict-free).
__device__ __forceinline__ int mx_fb(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }
__device__ __forceinline__ int mx_b_off(int row, int chunk) { return row * MX_B_ROW + ((chunk ^ mx_fb(row)) << 4); }

// The e4m3 fragment of k step kk for a lane of half h (see above).
__device__ __forceinline__ i32x8_t mx_frag_a(const uint8_t* st, int row, int kk, int h) {
  const u32x4_t lo4 = *(const u32x4_t*)(st + mx_a_off(row, 4 * kk + h));
  const u32x4_t hi4 = *(const u32x4_t*)(st + mx_a_off(row, 4 * kk + 2 + h));
  return i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
}
// The e2m1 fragment of k step kk (its 32 codes in the low 16 bytes).
__device__ __forceinline__ i32x8_t mx_frag_b(const uint8_t* st, int row, int kk, int h) {
  const u32x4_t c4 = *(const u32x4_t*)(st + mx_b_off(row, 2 * kk + h));
  return i32x8_t{(int)c4[0], (int)c4[1], (int)c4[2], (int)c4[3], 0, 0, 0, 0};
}

// W4A16 (MXFP4 weights, bf16 activations on v_mfma_f32_32x32x16_bf16): a k
// stage of 128 holds bf16 activation rows of 256 bytes (16 chunks) beside
// the same packed e2m1 weight rows.  Inside a stage the 8 k16 steps need not
// walk k in order, only the same way for both operands: at step s lane
// 32h + r takes k [64h + 8s, +8).  Its 8 weights then come from one MX block
// (2h + s/4), from dword s%4 of the 16-byte chunk 2h + s/4 of its weight
// row, and its 8 activations are chunk 8h + s of the activation row.
constexpr int MX_A16_ROW = MX_BK * 2;  // bytes per bf16 stage row
// bf16 rows: chunk c of row r at c ^ (r & 15).
__device__ __forceinline__ int mx_a16_off(int row, int chunk) { return row * MX_A16_ROW + ((chunk ^ (row & 15)) << 4); }

// Shared exponent of an MXFP8 block with largest magnitude m (>= 0):
// floor(log2 m) - 8, at least -127; 0 for m = 0.
__device__ __forceinline__ int mx_shared_exp(float m) {
  const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);
  return m == 0.0f ? 0 : max(e - 127 - 8, -127);
}
// 2^-X for X in [-127, 120]: a normal float built from its exponent field.
__device__ __forceinline__ float mx_inv_scale(int X) { return __uint_as_float((uint32_t)(127 - X) << 23); }

// E8M0 byte -> the fp32 2^(s-127) (s = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_f32(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

}  // namespace moe
