// fa_decode.hip — split-KV decode attention over a padded KV cache, plus the LSE merge.
//
// What is computed ([LLM-basics] = "LLM 기초 — Attention부터 FlashAttention까지",
// ②-3/②-4: one new query per sequence attends to that sequence's whole KV cache,
// so decode reads every cached key and value once and is bound by memory traffic;
// ②-7: Hq/Hkv query heads share one K/V head.  [FA3-entry] = "FlashAttention-3
// (FA-3)", itpe.jackerlab.com, §4 names a dedicated decode kernel.  [FA-notes] =
// "flash-attn" notes, minjae-portfolio.vercel.app, §4 gives the two-block merge
// that combines the pieces):
//   kernel 1, one workgroup per (chunk of `chunk` keys, K/V head, batch): all the
//     query heads of that K/V head's group attend to the chunk's keys; it writes
//     the chunk-normalised output O_c and lse_c for each of those heads.  Every
//     K/V byte of the valid keys is read from HBM exactly once.
//   kernel 2, one workgroup per (query head, batch): LSE = M + ln sum_c e^(lse_c - M)
//     with M = max_c lse_c, O = sum_c e^(lse_c - LSE) O_c.
//
// gfx950 mapping of kernel 1
//   * 256 threads = 4 wave64s; each wave takes 64-key pieces of the chunk and keeps
//     its own running (m, l, acc); the four waves are merged through LDS at the end.
//   * Scores S^T = K q^T with v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 d read
//     straight from HBM into VGPRs (16-byte loads), B = the group's query heads
//     (up to 16, zero-padded) held in VGPRs.  The matrix cores are far from busy
//     here; they are used because the group's 8 query heads make the per-byte
//     arithmetic too high for plain fp32 VALU at HBM speed.
//   * O^T = V^T P^T with the same instruction: V is transposed through the wave's
//     own LDS slice, in the permuted key order in which the score layout hands P
//     to the second product.
//   * Keys at or beyond the sequence length are never loaded (zero in registers and
//     -inf in the scores), so poisoned cache padding cannot leak in.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kSub = 64;   // keys per wave piece
constexpr int kVPad = 8;   // bf16 padding per transposed V row

// Position of 4-key run starting at key kk (multiple of 4, 0..63) in a transposed
// V row.  Inside each 32-key half, lane group g of the score layout holds keys
// 4g..4g+3 of the first 16 and of the second 16; the P fragment slots 8g..8g+7
// take them in that order, so runs are stored 0,4,1,5,2,6,3,7 (by run index).
__device__ __forceinline__ int dvt_pos(int kk) {
  const int half = kk >> 5;
  const int sub = (kk & 31) >> 2;
  return half * 32 + (sub & 3) * 8 + (sub >> 2) * 4;
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int* __restrict__ seqlens, float* __restrict__ part_o,
    float* __restrict__ part_lse, int Hq, int Hkv, int Nk_max, int chunk, int max_chunks,
    int n_qgroups, float c) {
  constexpr int VT_BYTES = kWaves * D * (kSub + kVPad) * 2;
  constexpr int MERGE_BYTES = kWaves * 16 * (D + 4) * 4 + 3 * kWaves * 16 * 4;
  constexpr int SMEM = VT_BYTES > MERGE_BYTES ? VT_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];

  const int chunk_id = blockIdx.x;
  const int kvh = blockIdx.y / n_qgroups;
  const int qg = blockIdx.y % n_qgroups;
  const int b = blockIdx.z;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Nk_max ? Nk_max : L);
  const int c0 = chunk_id * chunk;
  if (c0 >= L) return;  // uniform across the workgroup
  const int c1 = min(c0 + chunk, L);

  const int G = Hq / Hkv;
  const int hq0 = kvh * G + qg * 16;
  const int nq = min(16, G - qg * 16);  // query heads handled here

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  const size_t kv_stride = (size_t)Hkv * D;
  const uint16_t* Kb = Kc + ((size_t)b * Nk_max * Hkv + kvh) * D;
  const uint16_t* Vb = Vc + ((size_t)b * Nk_max * Hkv + kvh) * D;

  // q^T fragments: lane holds query head hq0 + l16, d = 32*s + 8*grp .. +7.
  bf16x8 qf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (l16 < nq) w = ldg128(Qd + ((size_t)b * Hq + hq0 + l16) * D + 32 * s + 8 * grp);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  uint16_t* vt = reinterpret_cast<uint16_t*>(smem) + wave * D * (kSub + kVPad);

  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{};
  // l_run sums the bf16-rounded weights (O's normaliser), l_lse the unrounded ones.
  float m_run = kNegInf, l_run = 0.f, l_lse = 0.f;

  // V loading: a lane owns column chunk vcc (8 d) of 4-key runs kq, kq+KQ, ...
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int KQ = 64 / CPR;        // lanes per column chunk (4 or 8)
  constexpr int RUNS = 16 / KQ;       // 4-key runs per lane (4 or 2)
  const int vcc = lane % CPR;
  const int vkq = lane / CPR;

  for (int n0 = c0 + wave * kSub; n0 < c1; n0 += kWaves * kSub) {
    // K fragments straight from HBM, V rows into registers.
    u32x4 kf[4][D / 32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = n0 + kb * 16 + l16;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < c1) w = ldg128(Kb + (size_t)key * kv_stride + 32 * s + 8 * grp);
        kf[kb][s] = w;
      }
    }
    u32x4 vr[RUNS][4];
#pragma unroll
    for (int ru = 0; ru < RUNS; ++ru)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = n0 + (vkq + ru * KQ) * 4 + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < c1) w = ldg128(Vb + (size_t)key * kv_stride + vcc * 8);
        vr[ru][r] = w;
      }

    // Transpose V into this wave's LDS slice.
#pragma unroll
    for (int ru = 0; ru < RUNS; ++ru) {
      const int pos = dvt_pos((vkq + ru * KQ) * 4);
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int sh = (cc & 1) * 16;
        const uint32_t e0 = (vr[ru][0][cc >> 1] >> sh) & 0xffffu;
        const uint32_t e1 = (vr[ru][1][cc >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (vr[ru][2][cc >> 1] >> sh) & 0xffffu;
        const uint32_t e3 = (vr[ru][3][cc >> 1] >> sh) & 0xffffu;
        u32x2 w = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *reinterpret_cast<u32x2*>(&vt[(vcc * 8 + cc) * (kSub + kVPad) + pos]) = w;
      }
    }

    // S^T = K q^T: four 16-key blocks.
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int st = 0; st < D / 32; ++st)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kb][st]),
                                                        qf[st], s[kb], 0, 0, 0);
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = n0 + kb * 16 + 4 * grp + r;
        const float t = (key < c1) ? s[kb][r] * c : kNegInf;
        s[kb][r] = t;
        mx = fmaxf(mx, t);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float ex = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kb][r] = fast_exp2(s[kb][r] - m_use);
        ex += s[kb][r];
      }
    l_lse = l_lse * alpha + ex;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;

    // P rounded to bf16 for the second product; the row sum adds those same rounded
    // weights, so the chunk output is a true weighted mean of V.
    bf16x8 pf[2];
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 w = {pack_bf16x2(s[2 * u][0], s[2 * u][1]), pack_bf16x2(s[2 * u][2], s[2 * u][3]),
                 pack_bf16x2(s[2 * u + 1][0], s[2 * u + 1][1]),
                 pack_bf16x2(s[2 * u + 1][2], s[2 * u + 1][3])};
#pragma unroll
      for (int t = 0; t < 4; ++t) rs = sum_bf16x2(w[t], rs);
      pf[u] = __builtin_bit_cast(bf16x8, w);
    }
    l_run = l_run * alpha + rs;
    // The wave's own LDS writes must land before its lanes read each other's data.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &vt[(db * 16 + l16) * (kSub + kVPad) + 32 * u + 8 * grp]);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[u], acc[db], 0, 0, 0);
      }
    __builtin_amdgcn_wave_barrier();
  }

  // Row sums across the four lane groups that share a query.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  l_lse += __shfl_xor(l_lse, 16);
  l_lse += __shfl_xor(l_lse, 32);

  // Merge the four waves through LDS (the V slices are dead by now).
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);                 // [4][16][D+4]
  float* mm = mo + kWaves * 16 * (D + 4);                     // [4][16]
  float* ml = mm + kWaves * 16;                               // [4][16]
  float* mle = ml + kWaves * 16;                              // [4][16]
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<f32x4*>(&mo[(wave * 16 + l16) * (D + 4) + db * 16 + 4 * grp]) = acc[db];
  if (grp == 0) {
    mm[wave * 16 + l16] = m_run;
    ml[wave * 16 + l16] = l_run;
    mle[wave * 16 + l16] = l_lse;
  }
  __syncthreads();

  constexpr int TPQ = kThreads / 16;  // threads per query head (16)
  constexpr int DPT = D / TPQ;        // d per thread (8 or 4)
  const int qi = tid / TPQ;
  const int d0 = (tid % TPQ) * DPT;
  if (qi < nq) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mm[w * 16 + qi]);
    float wsc[kWaves];
    float Lsum = 0.f, Lex = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wsc[w] = fast_exp2(mm[w * 16 + qi] - M);  // 0 for a wave that saw no key
      Lsum += wsc[w] * ml[w * 16 + qi];
      Lex += wsc[w] * mle[w * 16 + qi];
    }
    const float inv = 1.f / Lsum;
    const int hq = hq0 + qi;
    float* dst = part_o + (((size_t)b * Hq + hq) * max_chunks + chunk_id) * D + d0;
#pragma unroll
    for (int i = 0; i < DPT; i += 4) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&mo[(w * 16 + qi) * (D + 4) + d0 + i]);
        o += x * wsc[w];
      }
      *reinterpret_cast<f32x4*>(dst + i) = o * inv;
    }
    if (d0 == 0)
      part_lse[((size_t)b * Hq + hq) * max_chunks + chunk_id] = (M + fast_log2(Lex)) * kLn2;
  }
}

// Kernel 2: merge the chunks of one (query head, batch).  One thread per d column.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const int* __restrict__ seqlens,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         float* __restrict__ O,
                                                         float* __restrict__ LSE, int Hq,
                                                         int Nk_max, int chunk, int max_chunks) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Nk_max ? Nk_max : L);
  const int nc = (L + chunk - 1) / chunk;
  const size_t row = (size_t)b * Hq + hq;
  const float* pl = part_lse + row * max_chunks;
  const float* po = part_o + row * max_chunks * D + d;

  float M = kNegInf;
  for (int ci = 0; ci < nc; ++ci) M = fmaxf(M, pl[ci]);
  float ssum = 0.f, acc = 0.f;
  for (int ci = 0; ci < nc; ++ci) {
    const float w = fast_exp2((pl[ci] - M) * kLog2e);
    ssum += w;
    acc = fmaf(w, po[(size_t)ci * D], acc);
  }
  O[row * D + d] = (nc > 0) ? acc / ssum : 0.f;
  if (d == 0) LSE[row] = (nc > 0) ? M + fast_log2(ssum) * kLn2 : kNegInf;
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int n_qgroups = (G + 15) / 16;
  hipLaunchKernelGGL((decode_split_kernel<D>),
                     dim3((unsigned)a.max_chunks, (unsigned)(a.Hkv * n_qgroups), (unsigned)a.B),
                     dim3(kThreads), 0, s, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     a.seqlens, a.part_o, a.part_lse, a.Hq, a.Hkv, a.Nk_max, a.chunk,
                     a.max_chunks, n_qgroups, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(D), 0, s,
                     a.seqlens, a.part_o, a.part_lse, a.o, a.lse, a.Hq, a.Nk_max, a.chunk,
                     a.max_chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_splitkv(const DecodeArgs& a, hipStream_t s) {
  return a.d == 64 ? launch<64>(a, s) : launch<128>(a, s);
}

}  // namespace fa
