// fa_probe.hip — two ceilings measured in place: the matrix cores' sustained bf16 rate
// and the HBM streaming-read rate.
//
// Measurement helpers, not operations of attention.
//
// Matrix cores: every workgroup slot runs a long loop of independent
// v_mfma_f32_32x32x16_bf16 on operands loaded once from a buffer of random bf16 values,
// with no other memory traffic.  Each wave keeps four accumulators and feeds every
// instruction a different (A, B) pair, in the accumulator form the attention kernels
// compile to (VGPR results).  The rate this loop sustains under the board's power limit
// is the ceiling the prefill's MFMA work can approach.
//
// Streaming read: the workgroups walk a buffer once, 16 bytes per lane per load (each wave
// instruction reads 1 KB contiguous), with the non-temporal cache policy the decode's K/V
// loads use, eight loads in flight per lane, and fold what they read into a per-thread
// XOR so that no load can be dropped.  Its rate is the ceiling the decode's K/V stream
// can approach.  The benchmark reports both beside the kernels' own rates.
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

constexpr uint32_t kStreamChunk = 256 * 16 * 8;  // bytes one workgroup reads per pass
constexpr int kStreamPolicy = 2;                  // non-temporal, as the decode's K/V loads

// Pass p of workgroup w reads the chunk at byte (p * blocks + w) * kStreamChunk: load u of
// thread t at chunk + 4096 u + 16 t.  Loads at or past `bytes` return zero (the
// descriptor's range check), so a ragged last chunk needs no branch.
__global__ __launch_bounds__(256) void stream_probe_kernel(const void* __restrict__ buf,
                                                           uint32_t bytes,
                                                           uint32_t* __restrict__ out,
                                                           uint32_t stride) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(buf), (short)0, (int)bytes, 0x00020000);
  const uint32_t lane_off = threadIdx.x * 16u;
  uint32_t x = 0;
  for (uint32_t base = blockIdx.x * kStreamChunk; base < bytes; base += stride) {
    u32x4 r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      r[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + 4096u * u + lane_off, 0,
                                                   kStreamPolicy);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = x;
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

int fa_probe_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks,
                         hipStream_t stream) {
  if (!buf || !out) return FA_ERR_NULL;
  if (blocks <= 0 || blocks > (1 << 16) || bytes == 0 || bytes > (size_t(1) << 31) ||
      bytes % 16 != 0)
    return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
    return FA_ERR_ALIGN;
  // blocks * kStreamChunk <= 2^31, so base + stride stays below 2^32
  hipLaunchKernelGGL(fa::stream_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, buf,
                     (uint32_t)bytes, out, (uint32_t)blocks * fa::kStreamChunk);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
