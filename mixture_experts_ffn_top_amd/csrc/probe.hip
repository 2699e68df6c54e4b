// Measured ceilings, reported next to the datasheet peaks:
//  * MFMA: a loop of independent matrix instructions on every CU, two waves
//    per SIMD, eight accumulators per wave, operands in registers.  No memory
//    traffic beyond one result per wave (kept so that the loop is not
//    removed).  The rate it reaches under the chip's power management is the
//    practical ceiling of the GEMMs.
//  * HBM: a streaming copy, 16-byte loads and stores, four in flight per lane,
//    each byte read once and written once.
#include "common.h"
#include "probe.h"

namespace moe {

namespace {

constexpr int PROBE_NT = 512;  // 8 waves: two per SIMD

__global__ __launch_bounds__(PROBE_NT) void mfma_probe_bf16_kernel(int iters, float seed, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  // operands that depend on the seed, so that nothing folds at compile time
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(lane + i));
    b[i] = (__bf16)(seed * (float)(lane - i));
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[blockIdx.x * (PROBE_NT / 64) + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(PROBE_NT) void mfma_probe_fp8_kernel(int iters, float seed, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  i32x8_t a, b;
  const int base = (int)(seed * 1000.0f);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((base + lane + i) & 0x03030303);  // small finite e4m3 codes
    b[i] = 0x30303030 ^ ((base + lane - i) & 0x03030303);
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane == 0) out[blockIdx.x * (PROBE_NT / 64) + (threadIdx.x >> 6)] = s;
}

constexpr int COPY_NT = 256;
constexpr int COPY_UNROLL = 4;

__global__ __launch_bounds__(COPY_NT) void stream_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                              int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * (COPY_NT * COPY_UNROLL) + threadIdx.x;
  uint4 v[COPY_UNROLL];
#pragma unroll
  for (int u = 0; u < COPY_UNROLL; ++u) {
    const int64_t i = base + (int64_t)u * COPY_NT;
    if (i < n) v[u] = src[i];
  }
#pragma unroll
  for (int u = 0; u < COPY_UNROLL; ++u) {
    const int64_t i = base + (int64_t)u * COPY_NT;
    if (i < n) dst[i] = v[u];
  }
}

constexpr int READ_NT = 256;
constexpr int READ_UNROLL = 8;

// Each wave XORs the 32-bit words it reads and lane 0 writes the result, so
// that the loads are kept and the XOR of all outputs is that of all words.
__global__ __launch_bounds__(READ_NT) void stream_read_kernel(const uint4* __restrict__ src, int64_t n,
                                                              uint32_t* __restrict__ out) {
  const int64_t step = (int64_t)gridDim.x * (READ_NT * READ_UNROLL);
  uint32_t x = 0;
  for (int64_t base = (int64_t)blockIdx.x * (READ_NT * READ_UNROLL) + threadIdx.x; base < n; base += step) {
    uint4 v[READ_UNROLL];
#pragma unroll
    for (int u = 0; u < READ_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * READ_NT;
      v[u] = i < n ? src[i] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < READ_UNROLL; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (READ_NT / 64) + (threadIdx.x >> 6)] = x;
}

}  // namespace

int probe_waves(int workgroups) { return workgroups * (PROBE_NT / 64); }

hipError_t launch_mfma_probe(int fp8, int workgroups, int iters, float* out, hipStream_t st) {
  if (workgroups <= 0 || iters <= 0) return hipErrorInvalidValue;
  if (fp8)
    mfma_probe_fp8_kernel<<<workgroups, PROBE_NT, 0, st>>>(iters, 0.001f, out);
  else
    mfma_probe_bf16_kernel<<<workgroups, PROBE_NT, 0, st>>>(iters, 0.001f, out);
  return hipGetLastError();
}

int64_t stream_read_workgroups(int64_t n16, int32_t out_len) {
  const int64_t per_block = READ_NT * READ_UNROLL;
  const int64_t want = (n16 + per_block - 1) / per_block;
  const int64_t cap = out_len / (READ_NT / 64);
  return want < cap ? want : cap;
}

hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* out, int32_t out_len, hipStream_t st) {
  if (n16 <= 0) return hipSuccess;
  const int64_t grid = stream_read_workgroups(n16, out_len);
  if (grid < 1) return hipErrorInvalidValue;
  // entries past the grid's waves stay as they are; the used ones are all written
  stream_read_kernel<<<dim3((unsigned)grid), READ_NT, 0, st>>>((const uint4*)src, n16, out);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t st) {
  if (n16 <= 0) return hipSuccess;
  const int64_t per_block = COPY_NT * COPY_UNROLL;
  const int64_t grid = (n16 + per_block - 1) / per_block;
  stream_copy_kernel<<<dim3((unsigned)grid), COPY_NT, 0, st>>>((const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError();
}

}  // namespace moe
