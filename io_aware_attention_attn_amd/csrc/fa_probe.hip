// fa_probe.hip — the matrix cores' sustained bf16 rate, measured in place.
//
// A measurement helper, not an operation of attention: every workgroup slot runs a long
// loop of independent v_mfma_f32_32x32x16_bf16 on operands loaded once from a buffer
// of random bf16 values, with no other memory traffic.  Each wave keeps four
// accumulators and feeds every instruction a different (A, B) pair, in the accumulator
// form the attention kernels compile to (VGPR results).  The rate this loop sustains
// under the board's power limit is the ceiling the prefill's MFMA work can approach;
// the benchmark reports it beside the prefill's own rate.
#include "fa_device.h"
#include "fa_internal.h"
#include "fa.h"

namespace fa {
namespace {

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2))) void
mfma_probe_kernel(const u32x4* __restrict__ in, float* __restrict__ out, int iters) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, in[gid * 8 + i]);
    b[i] = __builtin_bit_cast(bf16x8, in[gid * 8 + 4 + i]);
  }
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + 1) & 3], acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[gid] = s;
}

}  // namespace
}  // namespace fa

extern "C" {

size_t fa_probe_mfma_bf16_operand_bytes(int blocks) {
  return blocks > 0 ? (size_t)blocks * 256 * 8 * 16 : 0;
}

int fa_probe_mfma_bf16(const void* operands, size_t operand_bytes, float* out, int blocks,
                       int iters, hipStream_t stream) {
  if (!operands || !out) return FA_ERR_NULL;
  if (blocks <= 0 || iters <= 0 || blocks > (1 << 20)) return FA_ERR_SHAPE;
  if (operand_bytes < fa_probe_mfma_bf16_operand_bytes(blocks)) return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 15u) != 0)
    return FA_ERR_ALIGN;
  hipLaunchKernelGGL(fa::mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const fa::u32x4*>(operands), out, iters);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
