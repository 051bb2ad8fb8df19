// fa_api.hip — the C ABI declared in include/fa.h: host-side validation, kernel
// selection and launch.  Validation happens before any HIP call; nothing here
// allocates or synchronises.  The only state is the per-device address of the fixed
// scratch array that fa_decode_splitkv_noalloc uses in place of a workspace.
#include "fa.h"

#include <limits.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa_internal.h"

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Shared checks for the two prefill entry points.
int check_prefill(const void* q, const void* k, const void* v, const float* o, const float* lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // Row indices and the 1-D grid are 32-bit: keep B*N*H and the block count in range.
  if ((long long)B * Nq * Hq > INT_MAX || (long long)B * Nk * Hkv > INT_MAX) return FA_ERR_SHAPE;
  if ((long long)B * Hq * ((Nq + 15) / 16) > INT_MAX) return FA_ERR_SHAPE;
  // Buffer addressing inside one batch's slice uses 32-bit byte offsets.
  if ((long long)(Nq + 256) * Hq * d * 4 > INT_MAX || (long long)(Nk + 256) * Hkv * d * 4 > INT_MAX)
    return FA_ERR_SHAPE;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  return FA_OK;
}

// Most pieces one (batch, K/V head) of the decode can be cut into: its steps of 64 keys
// are split over consecutive waves in runs of at least chunk / 64 steps, and a run
// boundary can fall on either side of the segment.
int max_pieces_of(int Nk_max, int chunk) {
  const int steps = (Nk_max + 63) / 64;
  const int rmin = chunk / 64;
  return (steps + rmin - 1) / rmin + 1;
}

int check_decode_sizes(int B, int Hq, int Hkv, int Nk_max, int d, int chunk) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nk_max <= 0 || d <= 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if ((long long)B * Nk_max * Hkv > INT_MAX) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (chunk <= 0 || chunk % 64 != 0) return FA_ERR_UNSUPPORTED;
  // the split kernel counts all 64-key steps of all (batch, K/V head, head group)
  // segments in 32-bit integers; Hkv * ceil((Hq / Hkv) / 16) <= Hq bounds the segment count
  const long long steps = (long long)B * Hq * ((Nk_max + 63) / 64);
  if (steps > 0x3fffffffLL || Hq > 65535 || B > 65535) return FA_ERR_SHAPE;
  return FA_OK;
}

// Validation shared by the two contiguous-cache decode entry points (everything but
// the workspace).
int check_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                         const int* seqlens_k, const float* o, const float* lse, int B, int Hq,
                         int Hkv, int Nk_max, int d, int chunk) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !o || !lse) return FA_ERR_NULL;
  const int st = check_decode_sizes(B, Hq, Hkv, Nk_max, d, chunk);
  if (st != FA_OK) return st;
  // one sequence's K or V rows are addressed with 32-bit byte offsets
  if ((long long)(Nk_max + 64) * Hkv * d * 2 > INT_MAX) return FA_ERR_SHAPE;
  if (misaligned(q) || misaligned(k_cache) || misaligned(v_cache) || misaligned(o) ||
      (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return FA_ERR_ALIGN;
  return FA_OK;
}

// Split + merge kernels of a contiguous-cache decode with the partial results in
// `workspace` (large enough, 16-byte aligned: checked by the callers).
int launch_decode_contiguous(const void* q, const void* k_cache, const void* v_cache,
                             const int* seqlens_k, float* o, float* lse, int B, int Hq, int Hkv,
                             int Nk_max, int d, float scale, int chunk, void* workspace,
                             hipStream_t stream) {
  const int mp = max_pieces_of(Nk_max, chunk);
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             fa::decode_part_o_bytes(B, Hq, mp, d));
  fa::DecodeArgs a{q, k_cache, v_cache, seqlens_k, o, lse, part_o, part_lse,
                   B, Hq, Hkv, Nk_max, d, chunk, mp, scale};
  return fa::launch_decode_splitkv(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Device scratch of fa_decode_splitkv_noalloc: the split kernel's partial results live
// here instead of in a caller workspace.  Every GPU the library runs on holds its own
// copy of the array (at its own address) until the process ends.  In host code the
// name `scratch` is only a host-side stand-in for the symbol, never a device address;
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)80 << 20;  // 80 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's copy of `scratch` (looked up on the first call
// on that device, with that device current, and kept), or nullptr if the lookup fails.
void* scratch_of_current_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream) {
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal);
  if (st != FA_OK) return st;
  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0};
  return fa::launch_prefill_bf16(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   hipStream_t stream) {
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal);
  if (st != FA_OK) return st;
  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0};
  return fa::launch_prefill_f32(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                      const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                      int max_seqlen_q, int max_seqlen_k, int total_q, int total_k, int d,
                      float scale, int causal, int q_row_stride, int k_row_stride,
                      int v_row_stride, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || max_seqlen_q <= 0 || max_seqlen_k < 0 || total_q <= 0 ||
      total_k < 0 || d <= 0)
    return FA_ERR_SHAPE;
  if (Hq % Hkv != 0 || max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // token rows must hold all heads and start on 16-byte boundaries; K and V share one stride
  if (q_row_stride < Hq * d || k_row_stride < Hkv * d || k_row_stride != v_row_stride)
    return FA_ERR_SHAPE;
  if (q_row_stride % 8 != 0 || k_row_stride % 8 != 0) return FA_ERR_ALIGN;
  // 32-bit grid, and 32-bit byte offsets inside one sequence's rows (reads may run one
  // block past its end; each sequence is addressed from its own first token)
  if ((long long)B * Hq * ((max_seqlen_q + 127) / 128) > INT_MAX) return FA_ERR_SHAPE;
  if ((long long)(max_seqlen_q + 256) * q_row_stride * 2 > INT_MAX ||
      (long long)(max_seqlen_k + 256) * k_row_stride * 2 > INT_MAX)
    return FA_ERR_SHAPE;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
    return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_ALIGN;
  fa::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, scale,
                    causal ? 1 : 0};
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.q_stride = q_row_stride;
  a.kv_stride = k_row_stride;
  return fa::launch_prefill_bf16(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_fp8(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   float q_descale, float k_descale, float v_descale, hipStream_t stream) {
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal);
  if (st != FA_OK) return st;
  // descales must be positive finite numbers (NaN fails every comparison)
  if (!(q_descale > 0.f && q_descale < 3.0e38f) || !(k_descale > 0.f && k_descale < 3.0e38f) ||
      !(v_descale > 0.f && v_descale < 3.0e38f))
    return FA_ERR_SHAPE;
  fa::Fp8Args a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0,
                q_descale, k_descale, v_descale};
  return fa::launch_prefill_fp8(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_backward_workspace_bytes(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  return 2 * fa::backward_vec_bytes(B, Hq, Nq);
}

int fa_backward(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int Nq,
                int Nk, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  const int st = check_prefill(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal);
  if (st != FA_OK) return st;
  if ((long long)B * Hkv * ((Nk + 127) / 128) > INT_MAX) return FA_ERR_SHAPE;
  if (misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv)) return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, Hq, Nq))
    return FA_ERR_WORKSPACE;
  if (misaligned(workspace)) return FA_ERR_ALIGN;
  fa::BackwardArgs a{q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr,
                     B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0};
  a.dsum = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    fa::backward_vec_bytes(B, Hq, Nq));
  return fa::launch_backward(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_splitkv_workspace_bytes(int B, int Hq, int Nk_max, int d, int chunk) {
  if (check_decode_sizes(B, Hq, 1, Nk_max, d, chunk) != FA_OK) return 0;
  const int mp = max_pieces_of(Nk_max, chunk);
  return fa::decode_part_o_bytes(B, Hq, mp, d) + fa::decode_part_lse_bytes(B, Hq, mp);
}

int fa_decode_splitkv(const void* q, const void* k_cache, const void* v_cache,
                      const int* seqlens_k, float* o, float* lse, int B, int Hq, int Hkv,
                      int Nk_max, int d, float scale, int chunk, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const int st = check_decode_splitkv(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nk_max,
                                      d, chunk);
  if (st != FA_OK) return st;
  const int mp = max_pieces_of(Nk_max, chunk);
  const size_t need = fa::decode_part_o_bytes(B, Hq, mp, d) + fa::decode_part_lse_bytes(B, Hq, mp);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (misaligned(workspace)) return FA_ERR_ALIGN;
  return launch_decode_contiguous(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nk_max, d,
                                  scale, chunk, workspace, stream);
}

int fa_decode_splitkv_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seqlens_k, float* o, float* lse, int B, int Hq, int Hkv,
                              int Nk_max, int d, float scale, int chunk, hipStream_t stream) {
  const int st = check_decode_splitkv(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nk_max,
                                      d, chunk);
  if (st != FA_OK) return st;
  const int mp = max_pieces_of(Nk_max, chunk);
  const size_t need = fa::decode_part_o_bytes(B, Hq, mp, d) + fa::decode_part_lse_bytes(B, Hq, mp);
  if (need > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = scratch_of_current_device();
  if (ws == nullptr) return FA_ERR_HIP;
  return launch_decode_contiguous(q, k_cache, v_cache, seqlens_k, o, lse, B, Hq, Hkv, Nk_max, d,
                                  scale, chunk, ws, stream);
}

int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                    const int* block_table, const int* seqlens_k, float* o, float* lse, int B,
                    int Hq, int Hkv, int num_pages, int page_size, int max_pages, int d,
                    float scale, int chunk, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seqlens_k || !o || !lse) return FA_ERR_NULL;
  if (num_pages <= 0 || page_size <= 0 || max_pages <= 0) return FA_ERR_SHAPE;
  if (page_size % 64 != 0) return FA_ERR_UNSUPPORTED;
  if ((long long)max_pages * page_size > INT_MAX) return FA_ERR_SHAPE;
  const int Nk_max = max_pages * page_size;
  const int st = check_decode_sizes(B, Hq, Hkv, Nk_max, d, chunk);
  if (st != FA_OK) return st;
  // one page of one K/V head is addressed with 32-bit offsets; the page index with 64
  if ((long long)page_size * Hkv * d * 2 > INT_MAX || (long long)B * max_pages > INT_MAX)
    return FA_ERR_SHAPE;
  if (misaligned(q) || misaligned(k_pages) || misaligned(v_pages) || misaligned(o) ||
      (reinterpret_cast<uintptr_t>(seqlens_k) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return FA_ERR_ALIGN;
  const int mp = max_pieces_of(Nk_max, chunk);
  const size_t need = fa::decode_part_o_bytes(B, Hq, mp, d) + fa::decode_part_lse_bytes(B, Hq, mp);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (misaligned(workspace)) return FA_ERR_ALIGN;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             fa::decode_part_o_bytes(B, Hq, mp, d));
  fa::DecodeArgs a{q, k_pages, v_pages, seqlens_k, o, lse, part_o, part_lse,
                   B, Hq, Hkv, Nk_max, d, chunk, mp, scale};
  a.block_table = block_table;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  return fa::launch_decode_splitkv(a, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes (non-positive, Hq % Hkv != 0, causal "
                              "with Nq > Nk, a packed row stride too small, a descale not positive, or too large "
                              "for 32-bit indexing)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128; decode chunk "
                                    "and page size must be positive multiples of 64";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a tensor pointer is not 16-byte aligned (or a "
                              "packed row stride is not a multiple of 8 elements)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: the decode's partial results would not fit the "
                                "library's fixed 80 MiB device scratch (fa_decode_splitkv_noalloc); "
                                "use fa_decode_splitkv with a workspace";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
