// Router-weighted combine: y[t] = sum_j w[t, j] * O[row_of_slot[t, j]]
// + sum_i ws[t, i] * O_sh[i*T + t] (the shared experts, if any), fp32 sums in
// ascending j then i, bf16 out.  One wave per (token, 512-column slice), 8
// columns per lane, 16-byte loads and stores: a batch of a few thousand
// tokens still puts tens of waves on every CU, enough loads in flight to
// stream O from HBM.  A gather with a fixed order, so the result is
// deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool O_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ O,
                                                      const int32_t* __restrict__ row_of_slot,
                                                      const float* __restrict__ w,
                                                      const uint8_t* __restrict__ mask, int T,
                                                      int k, int H, uint16_t* __restrict__ y,
                                                      int n_shared, const void* __restrict__ Osh,
                                                      const float* __restrict__ wsh) {
  const int lane = threadIdx.x & 63;
  const int S = (H + 511) / 512;                        // column slices per token
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = __builtin_amdgcn_readfirstlane((int)(gw / S));
  if (t >= T) return;
  const int c = __builtin_amdgcn_readfirstlane((int)(gw % S)) * 512 + lane * 8;
  const bool valid = mask ? (mask[t] != 0) : true;
  if (c < H) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    auto add_row = [&](const void* base, int64_t r, float wt) {
      if (O_BF16) {
        const u32x4_t v = *(const u32x4_t*)((const uint16_t*)base + r * H + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += wt * bf16_to_f32((uint16_t)(v[i] & 0xffffu));
          acc[2 * i + 1] += wt * bf16_to_f32((uint16_t)(v[i] >> 16));
        }
      } else {
        const f32x4_t* src = (const f32x4_t*)((const float*)base + r * H + c);
        const f32x4_t a = src[0], b = src[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += wt * a[i];
          acc[4 + i] += wt * b[i];
        }
      }
    };
    if (valid) {
      for (int j = 0; j < k; ++j) {
        const int r = row_of_slot[(int64_t)t * k + j];
        if (r < 0) continue;
        add_row(O, r, w ? w[(int64_t)t * k + j] : 1.0f);
      }
      for (int i = 0; i < n_shared; ++i)
        add_row(Osh, (int64_t)i * T + t, wsh ? wsh[(int64_t)t * n_shared + i] : 1.0f);
    }
    u32x4_t out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(u32x4_t*)(y + (int64_t)t * H + c) = out;
  }
}

hipError_t launch_combine(const void* O, int o_bf16, const int32_t* row_of_slot, const float* w,
                          const uint8_t* mask, int T, int k, int H, uint16_t* y, int n_shared,
                          const void* O_shared, const float* w_shared, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t waves = (int64_t)T * ((H + 511) / 512);
  if ((waves + 3) / 4 > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (o_bf16)
    combine_kernel<true><<<grid, block, 0, st>>>(O, row_of_slot, w, mask, T, k, H, y, n_shared, O_shared, w_shared);
  else
    combine_kernel<false><<<grid, block, 0, st>>>(O, row_of_slot, w, mask, T, k, H, y, n_shared, O_shared, w_shared);
  return hipGetLastError();
}

}  // namespace moe
