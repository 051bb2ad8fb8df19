// fa_prefill_fp8.hip — FlashAttention forward with FP8 (OCP E4M3) Q, K, V for gfx950.
//
// The same tile loop as the bf16 prefill ("flash-attn" notes §3-§5.2; "LLM 기초 —
// Attention부터 FlashAttention까지" ③-5): per (batch, query head, 128 query rows) the K/V
// blocks stream through LDS and the online softmax keeps a running exponent reference and
// row sums.  The FP8 forward of "FlashAttention-3 (FA-3)" (§3 names FP8 low precision)
// is the model for the precisions: both products take FP8 operands and accumulate in
// fp32; the probabilities P are rounded to E4M3 for P.V.  Per-tensor descale factors
// turn the stored FP8 codes back into values (x = code * descale): q and k descales fold
// into the exponent scale, the v descale into the final normalisation.
//
// gfx950 specifics:
//   * v_mfma_f32_32x32x64_f8f6f4 (format E4M3 for both operands): a lane of each operand
//     holds 32 consecutive k bytes; the same (lane half, byte) pairs meet in the sum.
//   * S^T = K Q^T takes its A rows in a permuted key order, so that after the product a
//     lane already holds the P^T values of keys 32*half .. 32*half + 31 in the order the
//     second product needs: no cross-lane exchange.
//   * V^T for O^T = V^T P^T comes from the row-major V tile through ds_read_b64_tr_b8
//     (each 16-lane group reads 8 rows x 16 bytes and every lane receives one column).
//   * O is normalised by the sum of the E4M3-rounded weights, formed by one more MFMA
//     against a block of ones (gfx950 has no FP8 dot instruction); the LSE uses the fp32
//     sum of the unrounded weights.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBN8 = 64;            // keys per K/V block
constexpr float kSumCap8 = 256.f;   // largest per-lane block sum of exp2(S*c - m_ref)
constexpr int kOnesE4M3 = 0x38383838;  // four E4M3 1.0 codes

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
typedef __attribute__((address_space(3))) void lds8_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc8(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Key row (within the 64-key block) that lane l32 feeds as A row of the S^T product for
// key half kb: l32 = 8a + 4b + c -> key 32b + 8a + 4kb + c.  The product's register r of
// lane half hi then holds key 32hi + 8(r/4) + 4kb + r%4.
__device__ __forceinline__ int a_row_key(int l32, int kb) {
  return 32 * ((l32 >> 2) & 1) + 8 * (l32 >> 3) + 4 * kb + (l32 & 3);
}

// XOR of the 16-byte chunk index within a tile row (rows of D bytes).
// K rows are read 32 bytes per lane in the permuted order above: the 16 rows a 16-lane
// group reads at one chunk land on distinct bank groups.  V rows are read transposed:
// the two 16-lane groups of a half-wave read the same 8 consecutive rows at the adjacent
// chunks 2c and 2c + 1, and the swizzle (even values only) keeps all 16 (row, chunk)
// pairs on distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k8(int row) {
  return D == 128 ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 5) & 1) << 2))
                  : (((row >> 3) & 1) | (((row >> 5) & 1) << 1));
}
template <int D>
__device__ __forceinline__ int swz_v8(int row) {
  return D == 128 ? (((row >> 1) & 3) << 1) : (((row >> 2) & 1) << 1);
}

// LDS-DMA of one 64-row block (D bytes per row) in 16-byte pieces, swizzled.
template <int D>
struct Tile8 {
  static constexpr int CH = D / 16;                 // 16-byte chunks per row
  static constexpr int PER_WAVE = kBN8 * CH / 64 / 4;  // instructions per wave (4 waves)
};

template <int D, bool IS_V>
__device__ __forceinline__ void tile8_offsets(uint32_t* off, uint32_t row_bytes, int wave,
                                              int lane) {
#pragma unroll
  for (int i = 0; i < Tile8<D>::PER_WAVE; ++i) {
    const int lin = (wave * Tile8<D>::PER_WAVE + i) * 64 + lane;
    const int row = lin / Tile8<D>::CH;
    const int pos = lin % Tile8<D>::CH;
    const int c = pos ^ (IS_V ? swz_v8<D>(row) : swz_k8<D>(row));
    off[i] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
  }
}

template <int D>
__device__ __forceinline__ void tile8_issue(__amdgpu_buffer_rsrc_t rs, const uint32_t* off,
                                            uint32_t soff, uint8_t* tile, int wave) {
#pragma unroll
  for (int i = 0; i < Tile8<D>::PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds8_void_t*)(tile + (wave * Tile8<D>::PER_WAVE + i) * 1024), 16, off[i], soff, 0,
        0);
}

// four fp32 -> four E4M3 codes in one dword (byte i = x_i), round to nearest even.  The
// first conversion writes the low half only and keeps the high half of `old`, which the
// second overwrites: passing the dword's previous (dead) contents saves a register clear.
__device__ __forceinline__ int pack_e4m3x4(float x0, float x1, float x2, float x3, int old) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, old, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(2, 2))) void
prefill_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                   const uint8_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                   int B, int Hq, int Hkv, int Nq, int Nk, float c, float v_descale,
                   int n_mblocks) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int BM = 128;
  constexpr int PW = Tile8<D>::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[kBN8 * D];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[kBN8 * D];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[kBN8 * D];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[kBN8 * D];
  uint8_t* const ks[2] = {ks0, ks1};
  uint8_t* const vs[2] = {vs0, vs1};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // work order as the bf16 prefill: bundles of one query block of one (batch, K/V head)
  // group's G query heads, heaviest (last) query block first, spread over the XCDs by
  // xcd_work
  const int G = Hq / Hkv;
  const XcdWork w = xcd_work((int)blockIdx.x, G, B * Hkv, n_mblocks);
  const int hg = w.sub;
  const int mb = n_mblocks - 1 - w.level;
  const int bk = w.group;
  const int kvh = bk % Hkv;
  const int b = bk / Hkv;
  const int hq = kvh * G + hg;
  const int m0 = mb * BM;

  const uint32_t q_row_bytes = (uint32_t)Hq * D;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D;
  const __amdgpu_buffer_rsrc_t rq =
      rsrc8(Q + ((size_t)b * Nq * Hq + hq) * D, (uint32_t)(Nq - 1) * q_row_bytes + D);
  const __amdgpu_buffer_rsrc_t rk =
      rsrc8(K + ((size_t)b * Nk * Hkv + kvh) * D, (uint32_t)(Nk - 1) * kv_row_bytes + D);
  const __amdgpu_buffer_rsrc_t rv =
      rsrc8(V + ((size_t)b * Nk * Hkv + kvh) * D, (uint32_t)(Nk - 1) * kv_row_bytes + D);

  const int diag = Nk - Nq;
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(m0 + BM, Nq) - 1 + diag + 1);
  const int n = (kend + kBN8 - 1) / kBN8;

  // Q^T fragments (B of S^T): lane = query row, bytes 64s + 32hi .. +31 (zeros past Nq)
  const int qrow = m0 + wave * 32 + l32;
  i32x8 qf[D / 64];
#pragma unroll
  for (int s = 0; s < D / 64; ++s) {
    const uint32_t off = (uint32_t)qrow * q_row_bytes + (uint32_t)(64 * s + 32 * hi);
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    const u32x4 up = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
    qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                  (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
  }

  // LDS byte offsets of the K operand reads: row a_row_key(l32, kb), chunks 4s + 2hi, +1
  uint32_t koff[2][D / 64][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = a_row_key(l32, kb);
#pragma unroll
    for (int s = 0; s < D / 64; ++s)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        koff[kb][s][e] = (uint32_t)(row * D + (((4 * s + 2 * hi + e) ^ swz_k8<D>(row)) * 16));
  }
  // LDS byte offsets of the transposed V reads: lane (group g, p = 2i + e) points at row
  // 32h + 8j + i, columns 32db + 16(g & 1) + 8e .. +7; the lane receives column
  // 32db + l32 of rows 32h + 8j .. +7 (keys of this lane half, in order)
  uint32_t voff[D / 32][4];
  {
    const int g = lane >> 4, p = lane & 15;
    const int i = p >> 1, e = p & 1, h = g >> 1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = 32 * h + 8 * jj + i;
        const int col = 32 * db + 16 * (g & 1) + 8 * e;
        voff[db][jj] = (uint32_t)(row * D + (((col >> 4) ^ swz_v8<D>(row)) * 16) + (col & 15));
      }
  }
  uint32_t kvo[PW], vvo[PW];
  tile8_offsets<D, false>(kvo, kv_row_bytes, wave, lane);
  tile8_offsets<D, true>(vvo, kv_row_bytes, wave, lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  f32x16 lsum = {};         // row sums of the E4M3 weights (every register holds the sum)
  float m_ref = kNegInf;    // exponent reference, base 2
  float neg_m = 0.f;        // -m_ref, or 0 while the reference is still -inf
  // this lane's share of the row sum of the fp32 weights, in two independent chains
  float ls_a = 0.f, ls_b = 0.f;
  float lim = kSumCap8;     // that sum after the last block, plus kSumCap8
  i32x8 ones = {kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3,
                      kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3};

  auto qk = [&](const uint8_t* kt, f32x16* s) __attribute__((always_inline)) {
    const char* kb8 = reinterpret_cast<const char*>(kt);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 64; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kb8 + koff[kb][st][0]);
        const u32x4 up = *reinterpret_cast<const u32x4*>(kb8 + koff[kb][st][1]);
        const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
        s[kb] = mfma8(a, qf[st], s[kb]);
      }
  };

  // -inf for keys past the end or (causal) past this row's last visible key.
  auto mask = [&](f32x16* s, int j) __attribute__((always_inline)) {
    const int rel = qrow + diag - (j * kBN8 + 32 * hi);  // last visible key, minus 32hi
    const int relk = Nk - 1 - (j * kBN8 + 32 * hi);      // last existing key, minus 32hi
    const int lim = CAUSAL ? min(rel, relk) : relk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * kb + (r & 3);
        s[kb][r] = (key > lim) ? kNegInf : s[kb][r];
      }
  };

  auto row_max = [&](const f32x16* s) __attribute__((always_inline)) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return xor32_max(mx) * c;
  };

  auto rescale_to = [&](float m_blk) __attribute__((always_inline)) {
    const float m_new = fmaxf(m_ref, m_blk);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_ref - m_new);
    ls_a *= alpha;
    ls_b *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum[r] *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    m_ref = m_new;
    neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
  };

  // P^T = exp2(S^T c - m_ref) packed as the B operand of the second product: dword 2a
  // holds keys 32hi + 8a + 0..3 (registers 4a.. of s[0]), dword 2a+1 keys 32hi + 8a + 4..7
  // (registers 4a.. of s[1]); the fp32 weights are added to the running sums ea, eb.
  auto exp_pack = [&](const f32x16* s, i32x8& pf, float& ea, float& eb)
      __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) p[t] = fast_exp2(fmaf(s[kb][4 * a + t], c, neg_m));
        ea += p[0] + p[1];
        eb += p[2] + p[3];
        pf[2 * a + kb] = pack_e4m3x4(p[0], p[1], p[2], p[3], pf[2 * a + kb]);
      }
  };

  // O^T += V^T P^T and the E4M3 row sums (ones^T P^T)
  auto pv = [&](const uint8_t* vt, const i32x8& pf) __attribute__((always_inline)) {
    const __attribute__((address_space(3))) uint8_t* vb =
        (const __attribute__((address_space(3))) uint8_t*)(vt);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      i32x2 r[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        r[jj] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vb + voff[db][jj]));
      const i32x8 a = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
      acc[db] = mfma8(a, pf, acc[db]);
    }
    lsum = mfma8(ones, pf, lsum);
  };

  // block j needs the mask if it runs past the last key, or (causal) past the last key
  // visible from this wave's first row
  const int wrow0 = m0 + wave * 32;
  auto need_mask = [&](int j) __attribute__((always_inline)) {
    return (j * kBN8 + kBN8 > Nk) || (CAUSAL && (j * kBN8 + kBN8 - 1 > wrow0 + diag));
  };

  // a block's softmax with the rare reference move (see the bf16 prefill): taken when a
  // lane's fp32 sum grew by more than kSumCap8 over the block
  auto softmax = [&](f32x16* s, i32x8& pf, float ea, float eb) __attribute__((always_inline)) {
    float tot = ea + eb;
    if (__builtin_amdgcn_ballot_w64(!(tot <= lim)) != 0) {
      rescale_to(row_max(s));
      ea = ls_a;
      eb = ls_b;
      exp_pack(s, pf, ea, eb);
      tot = ea + eb;
    }
    ls_a = ea;
    ls_b = eb;
    lim = tot + kSumCap8;
  };

  f32x16 s_a[2], s_b[2];
  i32x8 pf = {};  // P^T of the block in flight (each block's packing overwrites it)
  if (n > 0) {
    tile8_issue<D>(rk, kvo, 0, ks[0], wave);
    tile8_issue<D>(rv, vvo, 0, vs[0], wave);
    if (n > 1) tile8_issue<D>(rk, kvo, kBN8 * kv_row_bytes, ks[1], wave);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    qk(ks[0], s_a);
    if (need_mask(0)) mask(s_a, 0);
    m_ref = row_max(s_a);
    neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
  }

  // iteration j: MFMA S(j+1) | VALU softmax of block j; then MFMA O += V(j)^T P(j)^T
  auto step_next = [&](auto stage_c, int j, f32x16* s_cur, f32x16* s_nxt)
      __attribute__((always_inline)) {
    constexpr int sc = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (j + 2 < n)
      tile8_issue<D>(rk, kvo, (uint32_t)(j + 2) * kBN8 * kv_row_bytes, ks[sc], wave);
    tile8_issue<D>(rv, vvo, (uint32_t)(j + 1) * kBN8 * kv_row_bytes, vs[1 - sc], wave);
    qk(ks[1 - sc], s_nxt);
    float ea = ls_a, eb = ls_b;
    exp_pack(s_cur, pf, ea, eb);
    asm volatile("" ::"v"(pf), "v"(ea), "v"(eb));
    if (need_mask(j + 1)) mask(s_nxt, j + 1);
    softmax(s_cur, pf, ea, eb);
    pv(vs[sc], pf);
  };
  auto step_last = [&](auto stage_c, f32x16* s_cur) __attribute__((always_inline)) {
    constexpr int sc = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    float ea = ls_a, eb = ls_b;
    exp_pack(s_cur, pf, ea, eb);
    softmax(s_cur, pf, ea, eb);
    pv(vs[sc], pf);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int j = 0;
  for (; j + 2 < n; j += 2) {
    // the block of ones stays in its eight registers across the loop (left to itself the
    // compiler rebuilds it with seven v_mov before every row-sum product)
    asm volatile("" : "+v"(ones));
    step_next(S0{}, j, s_a, s_b);
    step_next(S1{}, j + 1, s_b, s_a);
  }
  if (j + 1 < n) {
    step_next(S0{}, j, s_a, s_b);
    step_last(S1{}, s_b);
  } else if (n > 0) {
    step_last(S0{}, s_a);
  }

  // O = v_descale * acc / (sum of E4M3 weights), LSE = ln2 (m_ref + log2(sum of fp32 weights))
  const float l_ex = xor32_sum(ls_a + ls_b);
  const float inv = v_descale / lsum[0];
  if (qrow < Nq) {
    float* Orow = O + (((size_t)b * Nq + qrow) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(Orow + 32 * db + 8 * g + 4 * hi) =
            f32x4{acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                  acc[db][4 * g + 3] * inv};
    if (hi == 0) LSE[((size_t)b * Hq + hq) * Nq + qrow] = (m_ref + fast_log2(l_ex)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch8(const Fp8Args& a, hipStream_t s) {
  const int n_mblocks = (a.Nq + 127) / 128;
  const float c = a.scale * a.q_descale * a.k_descale * kLog2e;
  hipLaunchKernelGGL((prefill_fp8_kernel<D, CAUSAL>), dim3((unsigned)(n_mblocks * a.B * a.Hq)),
                     dim3(256), 0, s, static_cast<const uint8_t*>(a.q),
                     static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.o,
                     a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk, c, a.v_descale, n_mblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_fp8(const Fp8Args& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch8<64, true>(a, s) : launch8<64, false>(a, s);
  return a.causal ? launch8<128, true>(a, s) : launch8<128, false>(a, s);
}

}  // namespace fa
