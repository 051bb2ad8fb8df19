// fa_internal.h — argument blocks and launchers shared between the C ABI (fa_api.hip)
// and the kernel translation units.  Not part of the public interface (include/fa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Prefill forward: Q [B,Nq,Hq,d], K/V [B,Nk,Hkv,d], O [B,Nq,Hq,d] fp32, LSE [B,Hq,Nq] fp32.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  // variable-length packed batch (cu_q != nullptr): Nq / Nk = longest query / key sequence;
  // q/k/v rows `*_stride` elements apart, O [total_q, Hq, d], LSE [Hq, total_q]
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0, q_stride = 0, kv_stride = 0;
};

// Split-KV decode: q [B,Hq,d], caches [B,Nk_max,Hkv,d], seqlens [B] (device),
// O [B,Hq,d] fp32, LSE [B,Hq] fp32, workspace = partial O [B,Hq,P,d] fp32 followed by
// partial LSE [B,Hq,P] fp32 with P = max_pieces = ceil(ceil(Nk_max / 64) / (chunk / 64)) + 1,
// the most pieces one (batch, K/V head) can be cut into.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens;
  float* o;
  float* lse;
  float* part_o;
  float* part_lse;
  int B, Hq, Hkv, Nk_max, d, chunk, max_pieces;
  float scale;
  // paged caches (block_table != nullptr): k, v are [num_pages, page_size, Hkv, d] and
  // Nk_max = max_pages * page_size
  const int* block_table = nullptr;
  int page_size = 0, max_pages = 0, num_pages = 0;
};

// Backward: q, dout [B,Nq,Hq,d] bf16, k, v [B,Nk,Hkv,d] bf16, o [B,Nq,Hq,d] fp32 and
// lse [B,Hq,Nq] fp32 from the forward; dq [B,Nq,Hq,d], dk, dv [B,Nk,Hkv,d] fp32.
// Workspace: dsum = D_i and lse2 = LSE_i log2(e), each [B,Hq,Nq] fp32.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* o;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  float* dsum;
  float* lse2;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
};

inline size_t backward_vec_bytes(int B, int Hq, int Nq) {
  size_t n = (size_t)B * Hq * Nq * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

// FP8 forward: q [B,Nq,Hq,d], k, v [B,Nk,Hkv,d] as OCP E4M3 codes; value = code * descale.
struct Fp8Args {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  float q_descale, k_descale, v_descale;
};

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);
hipError_t launch_prefill_fp8(const Fp8Args& a, hipStream_t s);
// Compute units of the current device (queried once per device; 256 if the query fails).
int device_cus();

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode_splitkv(const DecodeArgs& a, hipStream_t s);

// Workspace split used by both the size query and the launcher.
inline size_t decode_part_o_bytes(int B, int Hq, int max_pieces, int d) {
  size_t n = (size_t)B * Hq * max_pieces * d * sizeof(float);
  return (n + 255) & ~(size_t)255;
}
inline size_t decode_part_lse_bytes(int B, int Hq, int max_pieces) {
  size_t n = (size_t)B * Hq * max_pieces * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

}  // namespace fa
