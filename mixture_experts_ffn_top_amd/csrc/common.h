// Shared device helpers for the gfx950 MoE kernels: number formats, wave64
// reductions, activation math, MFMA vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

namespace moe {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Two floats to packed bf16 with one v_cvt_pk_bf16_f32 (round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------- experts
// Exclusive prefix over the L experts of blocks(rows of e), rows = offsets[e+1]
// - offsets[e]: out[e] for e < L and the total in out[L].  Run by one whole
// wave; lane i takes ceil(L/64) consecutive experts.
template <typename Blocks>
__device__ __forceinline__ void wave_expert_prefix(const int32_t* offsets, int L, int32_t* out, Blocks blocks) {
  const int lane = threadIdx.x & 63;
  const int per = (L + 63) / 64;
  const int e0 = lane * per;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < L) sum += blocks(offsets[e + 1] - offsets[e]);
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
      out[e] = run;
      run += blocks(offsets[e + 1] - offsets[e]);
    }
  }
  if (lane == 63) out[L] = inc;
}

// ---------------------------------------------------------------- biases
// The bf16 biases of four consecutive outputs at p (8-byte aligned), as floats.
__device__ __forceinline__ void bias_x4(const uint16_t* p, float* b) {
  const uint2 v = *(const uint2*)p;
  b[0] = bf16_to_f32(v.x & 0xffffu);
  b[1] = bf16_to_f32(v.x >> 16);
  b[2] = bf16_to_f32(v.y & 0xffffu);
  b[3] = bf16_to_f32(v.y >> 16);
}
// Gate and up biases of the outputs oc .. oc+3 of a gate_up bias row of 2N
// values: concatenated (gate at oc, up at N + oc) or interleaved (the gate of
// output j at 2j, its up at 2j+1; the row 16-byte aligned).
__device__ __forceinline__ void gate_up_bias_x4(const uint16_t* row, int N, int oc, bool interleaved, float* bg,
                                                float* bu) {
  if (!interleaved) {
    bias_x4(row + oc, bg);
    bias_x4(row + N + oc, bu);
  } else {
    const u32x4_t b4 = *(const u32x4_t*)(row + 2 * oc);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bg[c] = bf16_to_f32(b4[c] & 0xffffu);
      bu[c] = bf16_to_f32(b4[c] >> 16);
    }
  }
}

// ---------------------------------------------------------------- e4m3fn
// float -> OCP e4m3fn code, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint8_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint8_t)(sign | 0x7fu);   // NaN
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);  // >= 448 (and inf): saturate
  float af = __uint_as_float(a);
  int e = (int)(a >> 23) - 127;                            // unbiased exponent
  if (e < -6) {
    // subnormal range: value / 2^-9, rounded to nearest even integer in [0, 8]
    float q = rintf(af * 512.0f);                          // exact scaling
    return (uint8_t)(sign | (uint32_t)q);                  // q == 8 is the code of 2^-6
  }
  // normal: keep 3 mantissa bits, round to nearest even on the 20 dropped bits
  uint32_t m = a & 0x7fffffu;
  uint32_t rest = m & 0xfffffu;
  uint32_t keep = m >> 20;
  uint32_t half = 0x80000u;
  if (rest > half || (rest == half && (keep & 1u))) keep += 1;
  uint32_t ef = (uint32_t)(e + 7);
  if (keep == 8) { keep = 0; ef += 1; }
  (void)af;
  return (uint8_t)(sign | (ef << 3) | keep);
}

// Four floats -> four e4m3fn codes (byte i from v[i]), the same codes as
// f32_to_e4m3.  v_cvt_pk_fp8_f32 rounds to nearest even into OCP e4m3fn;
// for inputs first clamped to +-448 its codes equal f32_to_e4m3's for every
// non-NaN float (verified over all 2^32 bit patterns on gfx950).  A group
// holding a NaN takes the software encoder, which keeps NaN -> 0x7f | sign.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  if (__builtin_expect((a != a) | (b != b) | (c != c) | (d != d), 0))
    return (uint32_t)f32_to_e4m3(a) | ((uint32_t)f32_to_e4m3(b) << 8) |
           ((uint32_t)f32_to_e4m3(c) << 16) | ((uint32_t)f32_to_e4m3(d) << 24);
  auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}

// x / s in float32, correctly rounded like __fdiv_rn, for one divisor shared
// by many dividends: y = RN(1/s) once, then per dividend q0 = RN(x y),
// r = x - s q0 by one fma (exact), q = RN(q0 + r y) by another.  With y the
// correctly rounded reciprocal and no underflow on the way this correction is
// correctly rounded (Markstein's theorem, binary floating point, round to
// nearest); the fast form is used only for normal s >= 2^-92, which keeps r
// normal wherever a quotient can reach an e4m3 code other than zero, and
// x's sign is copied so that -0 stays -0.  Other divisors take __fdiv_rn.
struct SharedDivisor {
  float s, y;
  bool fast;
};
__device__ __forceinline__ SharedDivisor shared_divisor(float s) {
  SharedDivisor d;
  d.s = s;
  d.fast = s >= 0x1p-92f && s < __builtin_inff();
  d.y = d.fast ? __fdiv_rn(1.0f, s) : 0.0f;
  return d;
}
__device__ __forceinline__ float div_rn(const SharedDivisor& d, float x) {
#pragma clang fp contract(off)
  if (!d.fast) return __fdiv_rn(x, d.s);
  const float q0 = x * d.y;
  const float r = __builtin_fmaf(-q0, d.s, x);
  return __builtin_copysignf(__builtin_fmaf(r, d.y, q0), x);
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t ef = (c >> 3) & 0xfu;
  uint32_t m = c & 7u;
  float v;
  if (ef == 0) v = (float)m * (1.0f / 512.0f);
  else v = __uint_as_float(((ef + 120u) << 23) | (m << 20));
  if (ef == 15 && m == 7) v = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(v) | s);
}

// ---------------------------------------------------------------- wave64 reductions
// All-lanes reductions over a full wave (all 64 lanes active).  Inside each
// row of 16 lanes they run on DPP moves (quad_perm xor 1, xor 2, then
// row_half_mirror and row_mirror: after each step every lane holds the
// reduction of its quad, half-row, row); the four row results are then read
// with v_readlane and combined in a fixed order, so every lane gets the same
// value and no LDS round trip is taken.
static constexpr int DPP_QP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
static constexpr int DPP_QP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
static constexpr int DPP_ROW_HALF_MIRROR = 0x141;
static constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t row_lane(uint32_t v, int r) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 16 * r);
}

__device__ __forceinline__ float wave_max(float v) {
  const uint32_t ninf = 0xff800000u;
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_QP_XOR1>(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_QP_XOR2>(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(__float_as_uint(v), ninf)));
  const uint32_t u = __float_as_uint(v);
  return fmaxf(fmaxf(__uint_as_float(row_lane(u, 0)), __uint_as_float(row_lane(u, 1))),
               fmaxf(__uint_as_float(row_lane(u, 2)), __uint_as_float(row_lane(u, 3))));
}
// Maximum over each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float row16_max(float v) {
  const uint32_t ninf = 0xff800000u;
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_QP_XOR1>(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_QP_XOR2>(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(__float_as_uint(v), ninf)));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp_u32<DPP_QP_XOR1>(__float_as_uint(v), 0u));
  v += __uint_as_float(dpp_u32<DPP_QP_XOR2>(__float_as_uint(v), 0u));
  v += __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(__float_as_uint(v), 0u));
  v += __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(__float_as_uint(v), 0u));
  const uint32_t u = __float_as_uint(v);
  return (__uint_as_float(row_lane(u, 0)) + __uint_as_float(row_lane(u, 1))) +
         (__uint_as_float(row_lane(u, 2)) + __uint_as_float(row_lane(u, 3)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint64_t w = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32), 0u) << 32) | dpp_u32<CTRL>((uint32_t)v, 0u);
  return w > v ? w : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_QP_XOR1>(v, 0u));
  v = max(v, dpp_u32<DPP_QP_XOR2>(v, 0u));
  v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v, 0u));
  v = max(v, dpp_u32<DPP_ROW_MIRROR>(v, 0u));
  return max(max(row_lane(v, 0), row_lane(v, 1)), max(row_lane(v, 2), row_lane(v, 3)));
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<DPP_QP_XOR1>(v);
  v = dpp_max_u64<DPP_QP_XOR2>(v);
  v = dpp_max_u64<DPP_ROW_HALF_MIRROR>(v);
  v = dpp_max_u64<DPP_ROW_MIRROR>(v);
  uint64_t r = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t x = ((uint64_t)row_lane((uint32_t)(v >> 32), q) << 32) | row_lane((uint32_t)v, q);
    r = x > r ? x : r;
  }
  return r;
}

// Order-preserving map of a float key to uint32 (-0 is taken as +0), packed
// with the expert index so that the u64 maximum is the largest key and, among
// equal keys, the lowest index.
__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
  uint32_t u = __float_as_uint(key);
  if (u == 0x80000000u) u = 0;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ int unpack_idx(uint64_t p) { return (int)(0xffffffffu - (uint32_t)p); }

// The key half of pack_key alone (never 0 for a float), and its inverse.
__device__ __forceinline__ uint32_t order_key(float key) { return (uint32_t)(pack_key(key, 0) >> 32); }
__device__ __forceinline__ float order_key_inv(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// The router's float32 sigmoid: exp(-z) rounded once to float32, then a
// correctly rounded add and divide.
__device__ __forceinline__ float sigmoid_key_f32(float z) {
  float e = (float)exp(-(double)z);
  return __fdiv_rn(1.0f, __fadd_rn(1.0f, e));
}

__device__ __forceinline__ float log_sigmoid_f32(float v) {
  return fminf(v, 0.0f) - log1pf(expf(-fabsf(v)));
}

// ---------------------------------------------------------------- activations
enum { ACT_SILU = 0, ACT_SWIGLUOAI = 1, ACT_GELU_TANH = 2 };

// 1 / (1 + e^-x) with the hardware exp2 and reciprocal (about 1 ulp each):
// ample for an activation whose result is stored in 16 or 8 bits.
__device__ __forceinline__ float sigmoid_f32(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

template <int ACT>
__device__ __forceinline__ float gated_act(float g, float u, float alpha, float limit) {
  if (ACT == ACT_SILU || ACT == ACT_SWIGLUOAI) {
    if (limit > 0.0f) {
      g = fminf(g, limit);
      u = fminf(fmaxf(u, -limit), limit);
    }
  }
  if (ACT == ACT_SILU) return g * sigmoid_f32(g) * u;
  if (ACT == ACT_SWIGLUOAI) return g * sigmoid_f32(alpha * g) * (u + 1.0f);
  // gelu_tanh
  const float c = 0.7978845608028654f, a = 0.044715f;
  float t = tanhf(c * (g + a * g * g * g));
  return 0.5f * g * (1.0f + t) * u;
}

// The activation (the same float steps as gated_act) and its partial
// derivatives with respect to the unclamped gate and up.  A clamp passes the
// gradient where its input lies inside the closed range and blocks it outside.
template <int ACT>
__device__ __forceinline__ void gated_act_grad(float g0, float u0, float alpha, float limit, float& a, float& dg,
                                               float& du) {
  float g = g0, u = u0, mg = 1.0f, mu = 1.0f;
  if ((ACT == ACT_SILU || ACT == ACT_SWIGLUOAI) && limit > 0.0f) {
    g = fminf(g0, limit);
    u = fminf(fmaxf(u0, -limit), limit);
    mg = (g0 <= limit) ? 1.0f : 0.0f;
    mu = (u0 >= -limit && u0 <= limit) ? 1.0f : 0.0f;
  }
  if (ACT == ACT_SILU) {
    const float s = sigmoid_f32(g);
    a = g * s * u;
    dg = mg * (s * (1.0f + g * (1.0f - s)) * u);
    du = mu * (g * s);
  } else if (ACT == ACT_SWIGLUOAI) {
    const float s = sigmoid_f32(alpha * g);
    a = g * s * (u + 1.0f);
    dg = mg * ((s + alpha * g * s * (1.0f - s)) * (u + 1.0f));
    du = mu * (g * s);
  } else {
    const float c = 0.7978845608028654f, k = 0.044715f;
    const float t = tanhf(c * (g + k * g * g * g));
    const float gelu = 0.5f * g * (1.0f + t);
    a = gelu * u;
    dg = (0.5f * (1.0f + t) + 0.5f * g * (1.0f - t * t) * c * (1.0f + 3.0f * k * g * g)) * u;
    du = gelu;
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]) that wait on one counter only.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }
constexpr int waitcnt_lgkm(int n) { return 0xf | (0x3 << 14) | (0x7 << 4) | ((n & 0xf) << 8); }

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

}  // namespace moe
