// fa_prefill_bf16.hip — FlashAttention forward (prefill), bf16 in, fp32 accumulate, gfx950.
//
// What is computed ([FA-notes] = "flash-attn" notes, minjae-portfolio.vercel.app,
// §3 tiling / §4 online softmax / §5.2 forward kernel sketch; [LLM-basics] =
// "LLM 기초 — Attention부터 FlashAttention까지", ③-2 online softmax, ③-5 tile loop):
// one workgroup owns a block of query rows of one (batch, query head).  It keeps
// that Q block in registers and streams the K/V blocks of the matching K/V head
// through LDS.  For each K/V block it forms the scores, updates the running row
// maximum m and row sum l with the two-block merge (m_new = max(m_old, m_blk);
// old sums and the output accumulator scaled by exp(m_old - m_new)), and adds
// P V to the accumulator.  S and P live only in registers.  At the end
// O = acc / l and LSE = m + ln l are written.
//
// gfx950 mapping
//   * 256 threads = 4 wave64s; each wave owns 32 query rows, the workgroup 128.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = 32 keys x 16 d from LDS, B = Q^T fragment held in VGPRs for the whole
//     loop.  In the 32x32 result every lane holds 16 keys of ONE query row
//     (row = lane % 32), so a row maximum is an in-lane max over 32 values plus
//     a single exchange between the two wave halves (v_permlane32_swap).
//   * O^T = V^T P^T with the same instruction: A = V^T from LDS, B = P^T taken
//     straight from the score registers (rounded to bf16).  The output lanes
//     again hold one query row each, so the rescale by exp2(m_old - m_new) is a
//     per-lane multiply.  The keys of the P fragment come in the order the score
//     layout produces them; the transposed V tile in LDS is stored in that same
//     permuted key order, so the contraction pairs the right key with the right
//     value.
//   * Scores are taken to base 2 with scale*log2(e) folded into one multiply,
//     so every exponential is one v_exp_f32.
//   * K/V blocks of 64 keys: the next block is fetched from HBM into registers
//     while the current one is multiplied; K is stored row-major with a 16-byte
//     row pad (conflict-free 128-bit reads), V is transposed in registers and
//     stored [d][key].
//   * Causal: key blocks wholly in the future of the workgroup's rows are never
//     visited; only blocks that cross the diagonal (or the ragged end of the key
//     sequence) are masked.  Workgroups are issued heaviest-first.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per K/V block
constexpr int kThreads = 256;  // four wave64s
constexpr int kPad = 8;        // bf16 elements of padding per LDS row (16 bytes)

template <int D>
struct Smem {
  uint16_t k[kBN][D + kPad];   // K block, [key][d]
  uint16_t vt[D][kBN + kPad];  // V block transposed, [d][permuted key]
};

// Position of key `kk` (a multiple of 4 inside the block) in a transposed V row.
// Within each 16-key group the four 4-key runs are stored in the order 0, 2, 1, 3,
// which is the order in which the score layout hands keys to the P fragment
// (wave half 0 supplies keys 0-3 and 8-11, half 1 supplies 4-7 and 12-15).
__device__ __forceinline__ int vt_pos(int kk) {
  const int sub = (kk & 15) >> 2;
  return (kk & ~15) + (sub & 1) * 8 + (sub >> 1) * 4;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE, int B,
    int Hq, int Hkv, int Nq, int Nk, float c, int n_mblocks) {
  static_assert(D == 64 || D == 128, "head dim");
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Workgroup -> (query block, head, batch).  Query blocks are issued from the last
  // (the most keys under a causal mask) to the first.
  const int bh_count = B * Hq;
  const int bid = blockIdx.x;
  const int mb = n_mblocks - 1 - bid / bh_count;
  const int bh = bid % bh_count;
  const int hq = bh % Hq;
  const int b = bh / Hq;
  const int kvh = hq / (Hq / Hkv);
  const int m0 = mb * kBM;

  const size_t q_stride = (size_t)Hq * D;
  const size_t kv_stride = (size_t)Hkv * D;
  const uint16_t* Qb = Q + ((size_t)b * Nq * Hq + hq) * D;
  const uint16_t* Kb = K + ((size_t)b * Nk * Hkv + kvh) * D;
  const uint16_t* Vb = V + ((size_t)b * Nk * Hkv + kvh) * D;

  // Q^T fragments: lane holds query row qrow, d = 16*s + 8*hi .. +7.
  const int qrow = m0 + wave * 32 + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < Nq) w = ldg128(Qb + (size_t)qrow * q_stride + 16 * s + 8 * hi);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  // Keys this workgroup must visit: all of them, or under the causal mask up to the
  // last key visible from its last valid row.
  int kend = Nk;
  if (CAUSAL) {
    const int last_row = min(m0 + kBM, Nq) - 1;
    kend = min(Nk, last_row + (Nk - Nq) + 1);
  }
  const int n_tiles = (kend + kBN - 1) / kBN;

  // Register staging of one K/V block.
  constexpr int KCH = kBN * D / 8 / kThreads;  // 16-byte K chunks per thread
  constexpr int CW = D / 16;                   // V columns per thread (4 keys x CW)
  constexpr int VCC = D / CW;                  // column chunks per key row (16)
  const int v_kg = tid / VCC;                  // 4-key group 0..15
  const int v_cc = tid % VCC;
  u32x4 kreg[KCH];
  uint32_t vreg[4][CW / 2];

  auto load_block = [&](int n0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = i * kThreads + tid;
      const int key = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (n0 + key < Nk) w = ldg128(Kb + (size_t)(n0 + key) * kv_stride + col);
      kreg[i] = w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = n0 + v_kg * 4 + r;
      const uint16_t* src = Vb + (size_t)key * kv_stride + v_cc * CW;
      if constexpr (CW == 8) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key < Nk) w = ldg128(src);
#pragma unroll
        for (int t = 0; t < 4; ++t) vreg[r][t] = w[t];
      } else {
        u32x2 w = {0u, 0u};
        if (key < Nk) w = *reinterpret_cast<const u32x2*>(src);
        vreg[r][0] = w[0];
        vreg[r][1] = w[1];
      }
    }
  };

  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int id = i * kThreads + tid;
      const int key = id / (D / 8);
      const int col = (id % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[key][col]) = kreg[i];
    }
    const int pos = vt_pos(v_kg * 4);
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
      const int sh = (cc & 1) * 16;
      const uint32_t e0 = (vreg[0][cc >> 1] >> sh) & 0xffffu;
      const uint32_t e1 = (vreg[1][cc >> 1] >> sh) & 0xffffu;
      const uint32_t e2 = (vreg[2][cc >> 1] >> sh) & 0xffffu;
      const uint32_t e3 = (vreg[3][cc >> 1] >> sh) & 0xffffu;
      u32x2 w = {e0 | (e1 << 16), e2 | (e3 << 16)};
      *reinterpret_cast<u32x2*>(&sm.vt[v_cc * CW + cc][pos]) = w;
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = kNegInf;  // running row max, base-2 units
  float l_run = 0.f;      // this lane's share of the running row sum

  const int diag = Nk - Nq;  // key j visible from row i iff j <= i + diag

  if (n_tiles > 0) load_block(0);
  for (int j = 0; j < n_tiles; ++j) {
    const int n0 = j * kBN;
    __syncthreads();
    store_block();
    __syncthreads();
    if (j + 1 < n_tiles) load_block(n0 + kBN);

    // S^T = K Q^T for two 32-key halves.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[kb * 32 + l32][16 * st + 8 * hi]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
    }

    // Scale into base-2 units; mask the ragged end and the causal diagonal.
    const bool need_mask = (n0 + kBN > Nk) || (CAUSAL && (n0 + kBN - 1 > m0 + diag));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] *= c;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool dead = (key >= Nk) || (CAUSAL && key > qrow + diag);
          s[kb][r] = dead ? kNegInf : s[kb][r];
        }
    }

    // Online softmax update ([FA-notes] §4): m_new = max(m_old, block max).
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[kb][r] - m_use);
        s[kb][r] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

    // P^T fragments: 16 keys per MFMA step, eight consecutive score registers each.
    bf16x8 pf[kBN / 16];
#pragma unroll
    for (int u = 0; u < kBN / 16; ++u) {
      const int kb = u >> 1;
      const int base = 8 * (u & 1);
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(s[kb][base + 2 * t], s[kb][base + 2 * t + 1]);
      pf[u] = __builtin_bit_cast(bf16x8, w);
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int u = 0; u < kBN / 16; ++u) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&sm.vt[db * 32 + l32][16 * u + 8 * hi]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], acc[db], 0, 0, 0);
      }
  }

  // Epilogue: O = acc / l, LSE = ln2 * (m + log2 l).
  const float l_tot = xor32_sum(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < Nq) {
    float* Orow = O + ((size_t)(b * Nq + qrow) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                   acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(Orow + 32 * db + 8 * g + 4 * hi) = w;
      }
    if (hi == 0) LSE[((size_t)b * Hq + hq) * Nq + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  const int n_mblocks = (a.Nq + kBM - 1) / kBM;
  const long long blocks = (long long)n_mblocks * a.B * a.Hq;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                     a.scale * kLog2e, n_mblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
  return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
}

}  // namespace fa
