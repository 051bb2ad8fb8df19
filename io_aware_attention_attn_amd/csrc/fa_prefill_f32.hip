// fa_prefill_f32.hip — FlashAttention forward with fp32 inputs, everything in fp32.
//
// Same algorithm as the bf16 path ([FA-notes] = "flash-attn" notes,
// minjae-portfolio.vercel.app, §4 online softmax and §5.2 forward sketch): a
// workgroup owns a block of query rows, streams 32-key K/V blocks through LDS and
// keeps the running row max, row sum and output accumulator.  No value is ever
// rounded below fp32, so this path meets a 1e-5 absolute bound; it is plain
// VALU code (fp32 has no dense-matrix speed advantage at these sizes).
//
// Work split: each query row is handled by D/16 consecutive lanes, each lane
// owning 16 of the row's d columns.  A score is a 16-term partial dot product
// per lane, summed across the row's lanes with xor shuffles.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBNf = 32;  // keys per block

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
    float c, int n_mblocks) {
  constexpr int TPR = D / 16;            // lanes per query row
  constexpr int RB = kThreads / TPR;     // query rows per workgroup
  __shared__ float ks[kBNf][D + 4];
  __shared__ float vs[kBNf][D + 4];

  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int rloc = tid / TPR;
  const int bh_count = B * Hq;
  const int mb = n_mblocks - 1 - (int)blockIdx.x / bh_count;
  const int bh = (int)blockIdx.x % bh_count;
  const int hq = bh % Hq;
  const int b = bh / Hq;
  const int kvh = hq / (Hq / Hkv);
  const int m0 = mb * RB;
  const int row = m0 + rloc;

  const size_t q_stride = (size_t)Hq * D;
  const size_t kv_stride = (size_t)Hkv * D;
  const float* Kb = K + ((size_t)b * Nk * Hkv + kvh) * D;
  const float* Vb = V + ((size_t)b * Nk * Hkv + kvh) * D;

  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    q[i] = (row < Nq) ? Q[((size_t)b * Nq + row) * q_stride + (size_t)hq * D + part * 16 + i] : 0.f;

  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  const int diag = Nk - Nq;

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(m0 + RB, Nq) - 1 + diag + 1);

  for (int n0 = 0; n0 < kend; n0 += kBNf) {
    __syncthreads();
    for (int idx = tid; idx < kBNf * D / 4; idx += kThreads) {
      const int key = idx / (D / 4);
      const int col = (idx % (D / 4)) * 4;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (n0 + key < Nk) {
        kv = *reinterpret_cast<const f32x4*>(Kb + (size_t)(n0 + key) * kv_stride + col);
        vv = *reinterpret_cast<const f32x4*>(Vb + (size_t)(n0 + key) * kv_stride + col);
      }
      *reinterpret_cast<f32x4*>(&ks[key][col]) = kv;
      *reinterpret_cast<f32x4*>(&vs[key][col]) = vv;
    }
    __syncthreads();

    float t[kBNf];
#pragma unroll
    for (int j = 0; j < kBNf; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) dot = fmaf(q[i], ks[j][part * 16 + i], dot);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) dot += __shfl_xor(dot, off);
      const int key = n0 + j;
      const bool dead = (key >= Nk) || (CAUSAL && key > row + diag);
      t[j] = dead ? kNegInf : dot * c;
    }
    float mx = t[0];
#pragma unroll
    for (int j = 1; j < kBNf; ++j) mx = fmaxf(mx, t[j]);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kBNf; ++j) {
      t[j] = fast_exp2(t[j] - m_use);
      rs += t[j];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = acc[i] * alpha;
#pragma unroll
      for (int j = 0; j < kBNf; ++j) a = fmaf(t[j], vs[j][part * 16 + i], a);
      acc[i] = a;
    }
  }

  if (row < Nq) {
    const float inv = 1.f / l_run;
    float* Orow = O + ((size_t)b * Nq + row) * q_stride + (size_t)hq * D + part * 16;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      f32x4 w = {acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv};
      *reinterpret_cast<f32x4*>(Orow + i) = w;
    }
    if (part == 0) LSE[((size_t)b * Hq + hq) * Nq + row] = (m_run + fast_log2(l_run)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  constexpr int RB = kThreads / (D / 16);
  const int n_mblocks = (a.Nq + RB - 1) / RB;
  const long long blocks = (long long)n_mblocks * a.B * a.Hq;
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                     a.scale * kLog2e, n_mblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
  return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
}

}  // namespace fa
