// Launchers of the measured-ceiling probes (MFMA loop, streaming copy, streaming read).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// waves a probe launch of `workgroups` work-groups runs
int probe_waves(int workgroups);
// fp8 = 0: v_mfma_f32_32x32x16_bf16; fp8 = 1: v_mfma_scale_f32_32x32x64_f8f6f4
// (e4m3 operands, unit scales).  Each wave issues iters * 8 instructions and
// writes one float to out[wave].
hipError_t launch_mfma_probe(int fp8, int workgroups, int iters, float* out, hipStream_t st);
// copies n16 16-byte units from src to dst
hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, hipStream_t st);
// workgroups (4 waves each) a streaming read of n16 16-byte units launches
// with out_len output entries: one per 32 KiB, at most out_len / 4
int64_t stream_read_workgroups(int64_t n16, int32_t out_len);
// reads n16 16-byte units of src; out[wave] = XOR of the 32-bit words the wave read
hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* out, int32_t out_len, hipStream_t st);

}  // namespace moe
