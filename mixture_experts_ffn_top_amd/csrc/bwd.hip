// Backward pass of the routed-expert FFN (the chain rule through the
// router-weighted combine, the two expert GEMMs and the gated activation of
// the StackedMoE / GatedActivation pages; the down bias inside the router
// weighting of _apply_bias and the deterministic per-expert bias-gradient
// reduction of the nemo_automodel experts page).
//
//   combine backward  dO[p] = w[t, j] dy[t] (bf16), dw[t, j] = <dy[t], O[p]>
//   dA       = s_d  * dO . W_d          rows GEMM on the stacked [L, D, H] view
//   recompute h = s_gu * x . W_gu^T + b_gu; store A = act(h) and
//            dH = dA * d act / d(gate, up) in W_gu's column order
//   dX       = s_gu * dH . W_gu         rows GEMM on the stacked [L, H, 2D] view
//   dW_d[e]  = s_d  * dO_e^T . A_e      weight-gradient GEMM, [H, D] per expert
//   dW_gu[e] = s_gu * dH_e^T . x_e      weight-gradient GEMM, [2D, H] per expert
//   db_d[e]  = sum of dO_e rows, db_gu[e] = sum of dH_e rows (compensated fp32)
//
// The weight-gradient GEMMs contract over an expert's rows.  Their operands
// are transposed first into [columns, padded rows] copies in which every
// expert's rows form one segment that starts on a multiple of 64 and is
// zero padded to one, so the contraction runs on the same K-contiguous MFMA
// tiles as the forward GEMMs; the bias sums read the same copies.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int TT = 64;  // transpose tile

// seg[e] = sum over e' < e of round_up(rows of e', 64); seg[L] = the total
__global__ __launch_bounds__(64) void seg_offsets_kernel(const int32_t* __restrict__ offsets, int L,
                                                         int32_t* __restrict__ seg) {
  wave_expert_prefix(offsets, L, seg, [](int rows) { return (rows + TT - 1) / TT * TT; });
}

// dst[c, q] for the padded row q of column block blockIdx.x, q block
// blockIdx.y: the source row of q (through `gather` if given), or zero in an
// expert's padding.  src is [rows, C] bf16 with row pitch ld_src; dst is
// [C, Rp].  C is a multiple of 64.
__global__ __launch_bounds__(256) void seg_transpose_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                            const int32_t* __restrict__ gather,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ seg, int L, int C,
                                                            uint16_t* __restrict__ dst, int64_t Rp) {
  __shared__ uint16_t tile[TT][TT + 2];
  const int q0 = blockIdx.y * TT;
  if (q0 >= seg[L] || q0 + TT > Rp) return;  // (the second only if offsets exceed max_rows)
  int lo = 0, hi = L - 1;  // the expert whose segment holds q0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg[mid] <= q0) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int p_base = offsets[e] + (q0 - seg[e]);
  const int n_valid = offsets[e + 1] - p_base;  // rows of this block that exist (may be <= 0)
  const int c0 = blockIdx.x * TT;
  const int t = threadIdx.x;
  {
    const int j = t >> 2, cg = (t & 3) * 16;  // row j, 16 columns from cg
    u32x4_t v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (j < n_valid) {
      const int64_t row = gather ? (int64_t)gather[p_base + j] : (int64_t)(p_base + j);
      const u32x4_t* s = (const u32x4_t*)(src + row * ld_src + c0 + cg);
      v0 = s[0];
      v1 = s[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[j][cg + 2 * i] = (uint16_t)(v0[i] & 0xffffu);
      tile[j][cg + 2 * i + 1] = (uint16_t)(v0[i] >> 16);
      tile[j][cg + 8 + 2 * i] = (uint16_t)(v1[i] & 0xffffu);
      tile[j][cg + 8 + 2 * i + 1] = (uint16_t)(v1[i] >> 16);
    }
  }
  __syncthreads();
  {
    const int c = t >> 2, jg = (t & 3) * 16;  // column c, 16 rows from jg
    u32x4_t w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = (uint32_t)tile[jg + 2 * i][c] | ((uint32_t)tile[jg + 2 * i + 1][c] << 16);
      w1[i] = (uint32_t)tile[jg + 8 + 2 * i][c] | ((uint32_t)tile[jg + 8 + 2 * i + 1][c] << 16);
    }
    u32x4_t* d = (u32x4_t*)(dst + (int64_t)(c0 + c) * Rp + q0 + jg);
    d[0] = w0;
    d[1] = w1;
  }
}

// out[e, c] = sum over q in seg[e] .. seg[e+1] of srcT[c, q]: one wave per
// (expert, column), each lane a compensated (Kahan) fp32 sum of every 256th
// group of 4, then a fixed-order tree over the lanes: deterministic.
__global__ __launch_bounds__(256) void bias_grad_kernel(const uint16_t* __restrict__ srcT, int64_t Rp,
                                                        const int32_t* __restrict__ seg, int L, int C,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= (int64_t)L * C) return;
  const int e = (int)(gid / C), c = (int)(gid % C);
  // both multiples of 64; clipped to the padded width (exceeded only if the
  // row offsets exceed the rows the buffers were sized for)
  const int q0 = (int)min((int64_t)seg[e], Rp), q1 = (int)min((int64_t)seg[e + 1], Rp);
  const uint16_t* row = srcT + (int64_t)c * Rp;
  float s = 0.0f, comp = 0.0f;
  for (int q = q0 + lane * 4; q < q1; q += 256) {
    const uint2 v = *(const uint2*)(row + q);
    const float x[4] = {bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xffffu),
                        bf16_to_f32(v.y >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = x[i] - comp;
      const float tt = s + y;
      comp = (tt - s) - y;
      s = tt;
    }
  }
  s -= comp;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, MOE_WAVE);
  if (lane == 0) out[(int64_t)e * C + c] = s;
}

// Backward of the combine, one workgroup per token: for each slot j with a
// row, dO[row] = w dy[t] in bf16 and dw[t, j] = <dy[t], O[row]> (fp32, a
// fixed-order reduction); dropped slots and masked tokens get dw = 0.
template <bool O_BF16>
__global__ __launch_bounds__(256) void combine_backward_kernel(const uint16_t* __restrict__ dy,
                                                               const void* __restrict__ O,
                                                               const int32_t* __restrict__ row_of_slot,
                                                               const float* __restrict__ w,
                                                               const uint8_t* __restrict__ mask, int k, int H,
                                                               uint16_t* __restrict__ dO, float* __restrict__ dw) {
  __shared__ float s_part[4];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool valid = mask ? (mask[t] != 0) : true;
  for (int j = 0; j < k; ++j) {
    const int r = row_of_slot[(int64_t)t * k + j];
    const bool live = valid && r >= 0;
    const float wt = w ? w[(int64_t)t * k + j] : 1.0f;
    float dot = 0.0f;
    if (live) {
      for (int c = tid * 8; c < H; c += 256 * 8) {
        const u32x4_t d = *(const u32x4_t*)(dy + (int64_t)t * H + c);
        float dv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dv[2 * i] = bf16_to_f32(d[i] & 0xffffu);
          dv[2 * i + 1] = bf16_to_f32(d[i] >> 16);
        }
        u32x4_t o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2_rne(wt * dv[2 * i], wt * dv[2 * i + 1]);
        *(u32x4_t*)(dO + (int64_t)r * H + c) = o;
        if (dw) {
          float ov[8];
          if (O_BF16) {
            const u32x4_t v = *(const u32x4_t*)((const uint16_t*)O + (int64_t)r * H + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ov[2 * i] = bf16_to_f32(v[i] & 0xffffu);
              ov[2 * i + 1] = bf16_to_f32(v[i] >> 16);
            }
          } else {
            const f32x4_t a = *(const f32x4_t*)((const float*)O + (int64_t)r * H + c);
            const f32x4_t b = *(const f32x4_t*)((const float*)O + (int64_t)r * H + c + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ov[i] = a[i];
              ov[4 + i] = b[i];
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) dot += dv[i] * ov[i];
        }
      }
    }
    if (dw) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, MOE_WAVE);
      if (lane == 0) s_part[wave] = dot;
      __syncthreads();
      if (tid == 0) dw[(int64_t)t * k + j] = live ? ((s_part[0] + s_part[1]) + (s_part[2] + s_part[3])) : 0.0f;
      __syncthreads();
    }
  }
}

// dst[b][c][r] = src[b][r][c] for a [batch, rows, cols] bf16 tensor; rows and
// cols are multiples of 64.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst, int64_t rows,
                                                             int64_t cols) {
  __shared__ uint16_t tile[TT][TT + 2];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * TT, c0 = (int64_t)blockIdx.x * TT;
  const uint16_t* s = src + b * rows * cols;
  uint16_t* d = dst + b * rows * cols;
  const int t = threadIdx.x;
  {
    const int j = t >> 2, cg = (t & 3) * 16;
    const u32x4_t* p = (const u32x4_t*)(s + (r0 + j) * cols + c0 + cg);
    const u32x4_t v0 = p[0], v1 = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[j][cg + 2 * i] = (uint16_t)(v0[i] & 0xffffu);
      tile[j][cg + 2 * i + 1] = (uint16_t)(v0[i] >> 16);
      tile[j][cg + 8 + 2 * i] = (uint16_t)(v1[i] & 0xffffu);
      tile[j][cg + 8 + 2 * i + 1] = (uint16_t)(v1[i] >> 16);
    }
  }
  __syncthreads();
  {
    const int c = t >> 2, jg = (t & 3) * 16;
    u32x4_t w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = (uint32_t)tile[jg + 2 * i][c] | ((uint32_t)tile[jg + 2 * i + 1][c] << 16);
      w1[i] = (uint32_t)tile[jg + 8 + 2 * i][c] | ((uint32_t)tile[jg + 8 + 2 * i + 1][c] << 16);
    }
    u32x4_t* q = (u32x4_t*)(d + (c0 + c) * rows + r0 + jg);
    q[0] = w0;
    q[1] = w1;
  }
}

int64_t up256(int64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

FfnBwdLayout ffn_bwd_layout(int64_t R, int H, int D, int L) {
  FfnBwdLayout f{};
  const int64_t nonempty = R < L ? R : L;
  f.rp = (R + 63 * nonempty + TT - 1) / TT * TT;
  int64_t o = 0;
  f.seg_off = o;
  o += up256((int64_t)(L + 1) * 4);
  f.dA_off = o;
  o += up256(R * D * 2);
  f.A_off = o;
  o += up256(R * D * 2);
  f.dH_off = o;
  o += up256(R * 2 * D * 2);
  f.dOt_off = o;
  o += up256((int64_t)H * f.rp * 2);
  f.At_off = o;
  o += up256((int64_t)D * f.rp * 2);
  f.dHt_off = o;
  o += up256((int64_t)2 * D * f.rp * 2);
  f.xt_off = o;
  o += up256((int64_t)H * f.rp * 2);
  f.bytes = o;
  return f;
}

static hipError_t seg_transpose(const uint16_t* src, int64_t ld, const int32_t* gather, const FfnBwdParams& q,
                                const int32_t* seg, int C, uint16_t* dst, int64_t Rp, hipStream_t st) {
  const dim3 grid((unsigned)(C / TT), (unsigned)(Rp / TT));
  seg_transpose_kernel<<<grid, 256, 0, st>>>(src, ld, gather, q.offsets, seg, q.L, C, dst, Rp);
  return hipGetLastError();
}

static hipError_t bias_grad(const uint16_t* srcT, int64_t Rp, const int32_t* seg, int L, int C, float* out,
                            hipStream_t st) {
  const int64_t waves = (int64_t)L * C;
  bias_grad_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(srcT, Rp, seg, L, C, out);
  return hipGetLastError();
}

hipError_t launch_ffn_backward(const FfnBwdParams& q, hipStream_t st) {
  const FfnBwdLayout f = ffn_bwd_layout(q.max_rows, q.H, q.D, q.L);
  uint8_t* ws = (uint8_t*)q.ws;
  int32_t* seg = (int32_t*)(ws + f.seg_off);
  uint16_t* dA = (uint16_t*)(ws + f.dA_off);
  uint16_t* A = (uint16_t*)(ws + f.A_off);
  uint16_t* dH = (uint16_t*)(ws + f.dH_off);
  uint16_t* dOt = (uint16_t*)(ws + f.dOt_off);
  uint16_t* At = (uint16_t*)(ws + f.At_off);
  uint16_t* dHt = (uint16_t*)(ws + f.dHt_off);
  uint16_t* xt = (uint16_t*)(ws + f.xt_off);
  const int H = q.H, D = q.D, L = q.L;
  const bool gather = q.x_perm == nullptr;
  hipError_t err;
  auto ev = [&](int i) { return q.events ? hipEventRecord(q.events[i], st) : hipSuccess; };
  if ((err = ev(0)) != hipSuccess) return err;
  seg_offsets_kernel<<<1, 64, 0, st>>>(q.offsets, L, seg);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  // dA = s_d * dO . W_d
  BwdGemm b{};
  b.offsets = q.offsets;
  b.L = L;
  b.max_rows = q.max_rows;
  b.K = H;
  b.N = D;
  b.A = q.d_out;
  b.W = q.w_down_stacked;
  b.w_estride = (int64_t)D * H;
  b.lda = H;
  b.ldb = H;
  b.escale = q.down_scales;
  b.out = dA;
  b.ldo = D;
  b.out_bf16 = 1;
  if ((err = launch_bwd_rows_gemm(b, st)) != hipSuccess || (err = ev(1)) != hipSuccess) return err;

  // recompute h: A = act(h), dH = dA * d act
  BwdGemm g{};
  g.offsets = q.offsets;
  g.L = L;
  g.max_rows = q.max_rows;
  g.K = H;
  g.N = D;
  g.A = gather ? nullptr : q.x_perm;
  g.X = q.x;
  g.sorted_token = q.sorted_token;
  g.W = q.w_gate_up;
  g.w_estride = (int64_t)2 * D * H;
  g.lda = H;
  g.ldb = H;
  g.bias = q.b_gate_up;
  g.escale = q.gate_up_scales;
  g.act_kind = q.act_kind;
  g.fmt = q.fmt;
  g.alpha = q.alpha;
  g.limit = q.limit;
  g.out = A;
  g.ldo = D;
  g.out_bf16 = 1;
  g.din = dA;
  g.ld_din = D;
  g.out2 = dH;
  g.ldo2 = 2 * (int64_t)D;
  if ((err = launch_bwd_gate_up_gemm(g, st)) != hipSuccess || (err = ev(2)) != hipSuccess) return err;

  // dX = s_gu * dH . W_gu
  BwdGemm x{};
  x.offsets = q.offsets;
  x.L = L;
  x.max_rows = q.max_rows;
  x.K = 2 * D;
  x.N = H;
  x.A = dH;
  x.W = q.w_gate_up_stacked;
  x.w_estride = (int64_t)2 * D * H;
  x.lda = 2 * (int64_t)D;
  x.ldb = 2 * (int64_t)D;
  x.escale = q.gate_up_scales;
  x.out = q.d_x_perm;
  x.ldo = H;
  x.out_bf16 = 0;
  if ((err = launch_bwd_rows_gemm(x, st)) != hipSuccess || (err = ev(3)) != hipSuccess) return err;

  // the weight-gradient operands, transposed into padded expert segments
  const int64_t Rp = f.rp;
  if (Rp > 0) {
    if ((err = seg_transpose(q.d_out, H, nullptr, q, seg, H, dOt, Rp, st)) != hipSuccess) return err;
    if ((err = seg_transpose(A, D, nullptr, q, seg, D, At, Rp, st)) != hipSuccess) return err;
    if ((err = seg_transpose(dH, 2 * D, nullptr, q, seg, 2 * D, dHt, Rp, st)) != hipSuccess) return err;
    if ((err = seg_transpose(gather ? q.x : q.x_perm, H, gather ? q.sorted_token : nullptr, q, seg, H, xt, Rp,
                             st)) != hipSuccess)
      return err;
  }
  if ((err = ev(4)) != hipSuccess) return err;

  // dW_d[e] = s_d * dO_e^T . A_e  ([H, D]),  dW_gu[e] = s_gu * dH_e^T . x_e  ([2D, H])
  BwdGemm w{};
  w.L = L;
  w.seg = seg;
  w.M = H;
  w.N = D;
  w.A = dOt;
  w.W = At;
  w.lda = Rp;
  w.ldb = Rp;
  w.escale = q.down_scales;
  w.out = q.d_w_down;
  w.ldo = D;
  w.out_estride = (int64_t)H * D;
  if ((err = launch_wgrad_gemm(w, st)) != hipSuccess || (err = ev(5)) != hipSuccess) return err;
  w.M = 2 * D;
  w.N = H;
  w.A = dHt;
  w.W = xt;
  w.escale = q.gate_up_scales;
  w.out = q.d_w_gate_up;
  w.ldo = H;
  w.out_estride = (int64_t)2 * D * H;
  if ((err = launch_wgrad_gemm(w, st)) != hipSuccess || (err = ev(6)) != hipSuccess) return err;

  // per-expert bias gradients
  if (q.d_b_down && (err = bias_grad(dOt, Rp, seg, L, H, q.d_b_down, st)) != hipSuccess) return err;
  if (q.d_b_gate_up && (err = bias_grad(dHt, Rp, seg, L, 2 * D, q.d_b_gate_up, st)) != hipSuccess) return err;
  return ev(7);
}

hipError_t launch_combine_backward(const CombineBwdParams& q, hipStream_t st) {
  if (q.T == 0) return hipSuccess;
  if (q.o_bf16)
    combine_backward_kernel<true><<<q.T, 256, 0, st>>>(q.dy, q.O, q.row_of_slot, q.w, q.mask, q.k, q.H, q.dO, q.dw);
  else
    combine_backward_kernel<false><<<q.T, 256, 0, st>>>(q.dy, q.O, q.row_of_slot, q.w, q.mask, q.k, q.H, q.dO, q.dw);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, int batch, int64_t rows, int64_t cols,
                                 hipStream_t st) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)(cols / TT), (unsigned)(rows / TT), (unsigned)batch);
  transpose_bf16_kernel<<<grid, 256, 0, st>>>(src, dst, rows, cols);
  return hipGetLastError();
}

}  // namespace moe
