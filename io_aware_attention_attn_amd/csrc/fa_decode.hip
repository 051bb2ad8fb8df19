// fa_decode.hip — split-KV decode attention over a padded KV cache, plus the LSE merge.
//
// What is computed ([LLM-basics] = "LLM 기초 — Attention부터 FlashAttention까지",
// ②-3/②-4: one new query per sequence attends to that sequence's whole KV cache,
// so decode reads every cached key and value once and is bound by memory traffic;
// ②-7: Hq/Hkv query heads share one K/V head.  [FA3-entry] = "FlashAttention-3
// (FA-3)", itpe.jackerlab.com, §4 names a dedicated decode kernel.  [FA-notes] =
// "flash-attn" notes, minjae-portfolio.vercel.app, §4 gives the two-block merge
// that combines the pieces):
//   kernel 1: the keys of every (batch, K/V head) are cut into pieces; for each piece
//     all the query heads of that K/V head's group attend to the piece's keys, and
//     the piece-normalised output O_p and lse_p of each of those heads are written.
//     Every K/V byte of the valid keys is read from HBM exactly once.
//   kernel 2, one workgroup per (query head, batch): LSE = M + ln sum_p e^(lse_p - M)
//     with M = max_p lse_p, O = sum_p e^(lse_p - LSE) O_p.
//
// gfx950 mapping of kernel 1
//   * Every wave is an independent, persistent worker.  The (batch, K/V head, head
//     group) segments are laid end to end in 64-key steps, T steps in all, and wave w
//     takes the contiguous steps [w R, (w+1) R) with R = max(ceil(T / W), chunk / 64)
//     (W = waves in the grid): every wave streams the same number of bytes whatever
//     the length mix.  A wave writes one partial result (O_p, lse_p) for each piece of
//     a segment that its range covers, so a segment of n steps has at most
//     ceil(n / R) + 1 pieces and the merge reads a few records per query head.
//   * Software pipeline over the wave's steps: while step s is computed, the K and V
//     rows of step s+1 are in flight into registers.  Each load instruction fetches
//     whole head rows (4 rows x 256 bytes at d = 128): fetched 16 keys x 64 bytes per
//     instruction, the layout the score product wants in registers, the same bytes
//     stream about 9% slower.  A landed step is written to the wave's own LDS slice and
//     the MFMA operands are read from there; K and V are written out one after the
//     other and each half's next loads leave as soon as its registers are free, so a
//     wave never drains its loads at a step boundary.
//   * Scores S^T = K q^T with v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 d read as rows
//     from LDS, B = the group's query heads (up to 16, zero-padded).
//     The matrix cores are far from busy; they are used because the group's query
//     heads make the per-byte arithmetic too high for plain fp32 VALU at HBM speed.
//   * O^T = V^T P^T with the same instruction; V^T comes from the row-major V slice
//     through transposed LDS reads (ds_read_b64_tr_b16), in the key order in which
//     the score layout hands P to the product.
//   * Buffer loads clip at the sequence length, so cache rows at or beyond it read
//     as zeros (and get -inf scores): poisoned padding cannot leak in.
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;  // four independent wave workers per workgroup
constexpr int kWaves = 4;
constexpr int kStep = 64;      // keys per step
constexpr int kNT = 2;         // cache policy of the K/V loads: non-temporal

typedef __attribute__((address_space(3))) void dlds_void_t;
typedef __bf16 dbf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dbf16x4 dlds_bf16x4_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dmake_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// XOR swizzle of the 16-byte chunk index in a V row: a half-wave's transposed read
// touches 8 consecutive rows x 2 adjacent chunks, which then fall in distinct banks.
template <int D>
__device__ __forceinline__ int dswz(int row) {
  return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3);
}

// Where a wave is: batch b, K/V head kvh, head group qg of segment `seg` (= kvh * QG +
// qg) of that batch, step i (keys [64 i, 64 i + 64) clipped at the length L, nb steps
// in the segment), and S, the global index of the segment's first step (it names the
// segment).
struct Pos {
  int b, kvh, qg, L, nb, seg, i, S;
  int page;  // paged caches: physical page holding the step's keys
};

// Paged KV cache ([LLM-basics] ②-8, PagedAttention): the keys of sequence b are kept in
// pages of page_size keys, [num_pages, page_size, Hkv, d]; table[b * max_pages + j] is
// the physical page of the sequence's logical page j.  page_size is a multiple of 64, so
// a 64-key step never straddles two pages.  Unused by the contiguous-cache kernel.
struct Paging {
  const int* table;
  int max_pages, page_size, num_pages;
};

// Steps per wave, computed identically by both kernels from the total step count T.
__device__ __forceinline__ int steps_per_wave(int T, int W, int rmin) {
  return max((T + W - 1) / W, rmin);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ Qd, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, const int* __restrict__ seqlens, float* __restrict__ part_o,
    float* __restrict__ part_lse, int B, int Hq, int Hkv, int Nk_max, int rmin, int max_pieces,
    int QG, float c, Paging pg) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int RPI = 64 / CH;           // cache rows per load instruction (whole rows)
  constexpr int NI = kStep / RPI;        // load instructions per step, K and V each (= CH)
  constexpr int DB = D / 16;             // 16-row d blocks of O^T
  constexpr int KS = D / 32;             // 32-wide d steps of the score product
  // Each wave stages one step of K and of V in its own LDS slice (no barrier needed):
  // the cache rows arrive in registers with whole 256-byte head rows per load instruction
  // (the access pattern HBM serves fastest) and are written to LDS, from where the MFMA
  // operands are read: K rows directly, V^T through transposed reads.
  __shared__ __attribute__((aligned(1024))) uint16_t kst[kWaves][kStep * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vst[kWaves][kStep * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int G = Hq / Hkv;
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;

  // ---- per-lane fixed offsets
  // Loads: instruction i of a step covers rows RPI i .. RPI i + RPI - 1; lane -> row
  // lane / CH, chunk lane % CH.
  const int ld_row = lane / CH;
  const int ld_chunk = lane % CH;
  const uint32_t ld_off = (uint32_t)ld_row * row_bytes + (uint32_t)ld_chunk * 16u;
  // LDS byte offsets the lane writes its chunk to (row RPI i + ld_row): K rows swizzled so
  // the 16 rows of one K operand read fall in 16 different bank groups, V rows as the
  // transposed reads need.  The swizzles depend on the row only through ld_row's low bits
  // and RPI i, and RPI i is a multiple of 4 (D = 128) or 8 (D = 64).
  uint32_t kw_off[NI], vw_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = RPI * i + ld_row;
    const int ksw = D == 128 ? (row & 15) : ((row >> 1) & 7);
    kw_off[i] = (uint32_t)(row * D * 2 + ((ld_chunk ^ ksw) * 16));
    vw_off[i] = (uint32_t)(row * D * 2 + ((ld_chunk ^ dswz<D>(row)) * 16));
  }
  // K fragment reads (A of S^T): key 16 kb + l16 of the step, d = 32 st + 8 g.
  uint32_t kr_off[KS];
  {
    const int ksw = D == 128 ? (l16 & 15) : ((l16 >> 1) & 7);  // rows 16 kb + l16
#pragma unroll
    for (int st = 0; st < KS; ++st)
      kr_off[st] = (uint32_t)(l16 * D * 2 + (((4 * st + g) ^ ksw) * 16));
  }
  // Transposed V reads: in 16-lane group g, lane p points at row 32u + 4g + p/4 (+16
  // for the second half of the slots) and columns 16*db + 4*(p%4); the group receives
  // V[row0 + i][16*db + p], i = 0..3.
  uint32_t tr_off[DB];
  {
    const int rowl = 4 * g + (l16 >> 2);
    const int sw = dswz<D>(rowl);  // rows differ from rowl by multiples of 16 only
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 16 * db + 4 * (l16 & 3);
      tr_off[db] = (uint32_t)(rowl * D * 2 + (((col >> 3) ^ sw) * 16) + (col & 7) * 2);
    }
  }

  // ---- work range of this wave
  const int W = gridDim.x * kWaves;
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wave);
  const int per_b = Hkv * QG;  // segments per sequence
  // Sequence lengths are read with scalar loads (constant address space, uniform
  // index): they complete on their own counter, so reading one never waits for the
  // vector loads already in flight.
  const __attribute__((address_space(4))) int* sl =
      (const __attribute__((address_space(4))) int*)seqlens;
  // For up to 64 sequences the lengths are also kept one per lane, so a lookup is a
  // register read instead of a memory round trip.
  const int sl_lane = (B <= 64 && lane < B) ? sl[lane] : 0;
  auto seqlen = [&](int bb) __attribute__((always_inline)) {
    const int ub = __builtin_amdgcn_readfirstlane(bb);
    int L = (B <= 64) ? __builtin_amdgcn_readlane(sl_lane, ub) : sl[ub];
    L = L < 0 ? 0 : (L > Nk_max ? Nk_max : L);
    return __builtin_amdgcn_readfirstlane(L);
  };
  int T = 0;
  for (int bb = 0; bb < B; ++bb) T += ((seqlen(bb) + kStep - 1) / kStep) * per_b;
  T = __builtin_amdgcn_readfirstlane(T);
  const int R = __builtin_amdgcn_readfirstlane(steps_per_wave(T, W, rmin));
  const long long g_begin = (long long)w * R;
  if (g_begin >= T) return;
  const int g_end = (int)min((long long)T, g_begin + R);
  int gs = (int)g_begin;  // global index of the current step

  // Position of step i of segment seg of sequence bb (all arguments wave-uniform).
  auto make_pos = [&](int bb, int L, int nb, int seg, int i, int S) __attribute__((always_inline)) {
    Pos p;
    p.b = __builtin_amdgcn_readfirstlane(bb);
    p.L = __builtin_amdgcn_readfirstlane(L);
    p.nb = __builtin_amdgcn_readfirstlane(nb);
    p.seg = __builtin_amdgcn_readfirstlane(seg);
    p.i = __builtin_amdgcn_readfirstlane(i);
    p.S = __builtin_amdgcn_readfirstlane(S);
    p.kvh = __builtin_amdgcn_readfirstlane(seg / QG);
    p.qg = __builtin_amdgcn_readfirstlane(seg % QG);
    p.page = 0;
    if constexpr (PAGED) {
      // scalar load through the constant address space; entries are clamped into the
      // pool so a bad table entry cannot address outside it
      const __attribute__((address_space(4))) int* tb =
          (const __attribute__((address_space(4))) int*)pg.table;
      const int lp = __builtin_amdgcn_readfirstlane((i * kStep) / pg.page_size);
      int e = tb[__builtin_amdgcn_readfirstlane(bb * pg.max_pages + lp)];
      e = e < 0 ? 0 : (e >= pg.num_pages ? pg.num_pages - 1 : e);
      p.page = __builtin_amdgcn_readfirstlane(e);
    }
    return p;
  };
  // Position of global step g (0 <= g < T): skip whole sequences, then split the rest.
  auto locate = [&](int g) __attribute__((always_inline)) {
    int base = 0, bb = 0;
    int nb = (seqlen(0) + kStep - 1) / kStep;
    while (g >= base + nb * per_b) {
      base += nb * per_b;
      ++bb;
      nb = (seqlen(bb) + kStep - 1) / kStep;
    }
    const int r = g - base;
    const int seg = r / nb;
    return make_pos(bb, seqlen(bb), nb, seg, r % nb, base + seg * nb);
  };

  Pos cur = locate(gs), nxt = cur;

  u32x4 kreg[NI], vreg[NI];  // one step of K and V rows on their way to LDS
  bf16x8 qf[KS];
  f32x4 acc[DB];
  float m_run = kNegInf, l_run = 0.f, l_lse = 0.f;

  // Buffer descriptors of one sequence's K or V slice, clipped after key L - 1.  Built
  // from values forced into scalar registers so the loads need no per-lane loop.
  auto rsrc_of = [&](const uint16_t* base, const Pos& it) __attribute__((always_inline)) {
    const uint64_t a = reinterpret_cast<uint64_t>(base + ((size_t)it.b * Nk_max * Hkv + it.kvh) * D);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t nrec = __builtin_amdgcn_readfirstlane((uint32_t)(it.L - 1) * row_bytes + D * 2);
    return dmake_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), nrec);
  };
  // Paged caches: descriptor of the step's page for K/V head kvh, clipped after the
  // page's last key inside the sequence (`valid` >= 1 keys).
  auto page_rsrc = [&](const uint16_t* base, int page, int kvh, int valid)
      __attribute__((always_inline)) {
    const uint64_t a =
        reinterpret_cast<uint64_t>(base + ((size_t)page * pg.page_size * Hkv + kvh) * D);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t nrec = __builtin_amdgcn_readfirstlane((uint32_t)(valid - 1) * row_bytes + D * 2);
    return dmake_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), nrec);
  };
  // Where the rows of step `it` come from: the K and V descriptors and the byte offset of
  // the step's first key row inside them.
  struct Src {
    __amdgpu_buffer_rsrc_t rk, rv;
    uint32_t soff;
  };
  auto source = [&](const Pos& it) __attribute__((always_inline)) {
    const int n0 = it.i * kStep;
    Src src;
    if constexpr (PAGED) {
      const int p0 = __builtin_amdgcn_readfirstlane((n0 / pg.page_size) * pg.page_size);
      const int valid = min(pg.page_size, it.L - p0);
      src.rk = page_rsrc(Kc, it.page, it.kvh, valid);
      src.rv = page_rsrc(Vc, it.page, it.kvh, valid);
      src.soff = (uint32_t)(n0 - p0) * row_bytes;
    } else {
      src.rk = rsrc_of(Kc, it);
      src.rv = rsrc_of(Vc, it);
      src.soff = (uint32_t)n0 * row_bytes;
    }
    return src;
  };
  // Issue the K (or V) loads of a step into kreg (vreg).  Every cache byte is read once,
  // so the loads are marked non-temporal.
  auto issue_k = [&](const Src& src) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(
          src.rk, ld_off + (uint32_t)(RPI * i) * row_bytes, src.soff, kNT);
  };
  auto issue_v = [&](const Src& src) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(
          src.rv, ld_off + (uint32_t)(RPI * i) * row_bytes, src.soff, kNT);
  };
  // The landed K (or V) rows of a step into this wave's LDS slice.
  auto stage_k = [&]() __attribute__((always_inline)) {
    char* kb8 = reinterpret_cast<char*>(kst[wave]);
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(kb8 + kw_off[i]) = kreg[i];
  };
  auto stage_v = [&]() __attribute__((always_inline)) {
    char* vb8 = reinterpret_cast<char*>(vst[wave]);
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(vb8 + vw_off[i]) = vreg[i];
  };

  auto item_begin = [&](const Pos& it) __attribute__((always_inline)) {
    const int hq0 = it.kvh * G + it.qg * 16;
    const int nq = min(16, G - it.qg * 16);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (l16 < nq) w = ldg128(Qd + ((size_t)it.b * Hq + hq0 + l16) * D + 32 * st + 8 * g);
      qf[st] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x4{};
    m_run = kNegInf;
    l_run = 0.f;
    l_lse = 0.f;
  };

  // Partial result of the piece of segment `it` that this wave covered: record
  // w - S / R of that segment (the pieces of a segment go to consecutive waves).
  auto item_end = [&](const Pos& it) __attribute__((always_inline)) {
    float lr = l_run, le = l_lse;
    lr += __shfl_xor(lr, 16);
    lr += __shfl_xor(lr, 32);
    le += __shfl_xor(le, 16);
    le += __shfl_xor(le, 32);
    const int hq0 = it.kvh * G + it.qg * 16;
    const int nq = min(16, G - it.qg * 16);
    if (l16 < nq) {
      const int hq = hq0 + l16;
      const int pc = w - it.S / R;
      const float inv = 1.f / lr;
      float* dst = part_o + (((size_t)it.b * Hq + hq) * max_pieces + pc) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = acc[db] * inv;
      if (g == 0)
        part_lse[((size_t)it.b * Hq + hq) * max_pieces + pc] = (m_run + fast_log2(le)) * kLn2;
    }
  };

  // One 64-key step: scores, online softmax, P V.
  auto compute = [&](const Pos& it) __attribute__((always_inline)) {
    const int n0 = it.i * kStep;
    const char* kb8 = reinterpret_cast<const char*>(kst[wave]);
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb8 + kr_off[st] + kb * 16 * D * 2);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
    }
    float mx = kNegInf;
    const int lim = it.L - 1 - (n0 + 4 * g);  // last valid key, relative to this lane's keys
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tv = (kb * 16 + r > lim) ? kNegInf : s[kb][r] * c;
        s[kb][r] = tv;
        mx = fmaxf(mx, tv);
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
    m_run = m_new;
    l_lse = l_lse * alpha + ex;
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    // P rounded to bf16 for the second product; the row sum for O adds those same
    // rounded weights, so the chunk output is a true weighted mean of V.
    bf16x8 pf[2];
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 w = {pack_bf16x2(s[2 * u][0], s[2 * u][1]), pack_bf16x2(s[2 * u][2], s[2 * u][3]),
                 pack_bf16x2(s[2 * u + 1][0], s[2 * u + 1][1]),
                 pack_bf16x2(s[2 * u + 1][2], s[2 * u + 1][3])};
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) rs = sum_bf16x2(w[q4], rs);
      pf[u] = __builtin_bit_cast(bf16x8, w);
    }
    l_run = l_run * alpha + rs;
    const __attribute__((address_space(3))) char* vb =
        (const __attribute__((address_space(3))) char*)(vst[wave]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const dbf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (dlds_bf16x4_t*)(vb + tr_off[db] + (32 * u) * D * 2));
        const dbf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (dlds_bf16x4_t*)(vb + tr_off[db] + (32 * u + 16) * D * 2));
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[u], acc[db], 0, 0, 0);
      }
  };

  // The step after `it` in this wave's range: the next step of the segment, or the
  // first step of the next segment with keys.  Returns false at the end of the range.
  auto advance = [&](const Pos& it, Pos& nt) __attribute__((always_inline)) -> bool {
    if (gs + 1 >= g_end) return false;
    gs = __builtin_amdgcn_readfirstlane(gs + 1);
    int bb = it.b, L = it.L, nb = it.nb, seg = it.seg, i = it.i + 1, S = it.S;
    if (i == nb) {
      i = 0;
      S += nb;
      ++seg;
      if (seg == per_b) {
        // next sequence with at least one key (one exists: gs < g_end <= T)
        seg = 0;
        do {
          ++bb;
          L = seqlen(bb);
        } while (L == 0);
        nb = (L + kStep - 1) / kStep;
      }
    }
    nt = make_pos(bb, L, nb, seg, i, S);
    return true;
  };

  // ---- pipeline: while step s is computed from LDS, the rows of step s+1 are in flight
  // into kreg / vreg.  K and V are staged one after the other, and each half's loads for
  // step s+1 go out as soon as its registers are free, so the wave never drains its
  // loads: the next K rows are on their way while this step's V rows are still landing
  // (vector loads complete in issue order; the register uses below wait for exactly the
  // loads they need).
  item_begin(cur);
  {
    const Src src = source(cur);
    issue_k(src);
    issue_v(src);
  }
  while (true) {
    stage_k();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): written; kreg free again
    const bool more = advance(cur, nxt);
    // After the last step the loads still go out, on an empty descriptor (no memory access,
    // zeros back): with the same loads in flight on both paths the compiler's wait counts
    // for the V rows below stay exact instead of falling back to the shorter path's.
    Src src = {dmake_rsrc(Kc, 0u), dmake_rsrc(Vc, 0u), 0u};
    if (more) src = source(nxt);
    issue_k(src);
    stage_v();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // vreg free again
    issue_v(src);
    compute(cur);
    if (!more || nxt.S != cur.S) {
      item_end(cur);
      if (more) item_begin(nxt);
    }
    if (!more) break;
    cur = nxt;
  }
}

// Kernel 2: merge the pieces of one (query head, batch).  The workgroup first finds
// the segment's global start S and length n (sums over the sequence lengths, split
// over the threads) and from them, with the split kernel's R, the number of pieces
// (S + n - 1) / R - S / R + 1.  The four waves then take every fourth piece; each
// lane owns D/64 columns.  Per wave: running maximum, weights and weighted sums with
// several piece rows in flight; the four partial results are then combined through
// LDS with the same merge rule.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const int* __restrict__ seqlens, const float* __restrict__ part_o,
    const float* __restrict__ part_lse, float* __restrict__ O, float* __restrict__ LSE, int B,
    int Hq, int Hkv, int QG, int Nk_max, int W, int rmin, int max_pieces) {
  constexpr int NW = kMergeThreads / 64;
  constexpr int DPL = D / 64;  // columns per lane
  __shared__ float s_m[NW], s_l[NW];
  __shared__ float s_acc[NW][D];
  __shared__ int s_tot[NW], s_pre[NW];
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int per_b = Hkv * QG;
  const size_t row = (size_t)b * Hq + hq;
  const float* pl = part_lse + row * max_pieces;
  const float* po = part_o + row * max_pieces * D + lane * DPL;
  // The first kSpec pieces of each wave (pieces wave, wave + NW, ...) are read before the
  // piece count is known, so these reads overlap the length reads below.  Slots at or past
  // the count (inside the workspace row) hold whatever earlier calls left there; they are
  // dropped by the count test and never enter the arithmetic.
  constexpr int kSpec = 4;
  float lv[kSpec], ov[kSpec][DPL];
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int ci = wave + u * NW;
    lv[u] = kNegInf;
#pragma unroll
    for (int i = 0; i < DPL; ++i) ov[u][i] = 0.f;
    if (ci < max_pieces) {
      lv[u] = pl[ci];
#pragma unroll
      for (int i = 0; i < DPL; ++i) ov[u][i] = po[(size_t)ci * D + i];
    }
  }
  auto nsteps = [&](int bb) {
    int L = seqlens[bb];
    L = L < 0 ? 0 : (L > Nk_max ? Nk_max : L);
    return (L + 63) / 64;
  };
  const int nb = nsteps(b);  // read now, beside the other lengths
  // T = all steps, pre = steps of the sequences before b: with at most 64 sequences every
  // wave sums the lengths itself (one per lane), otherwise the workgroup shares the sum
  int T = 0, base = 0;
  if (B <= 64) {
    const int n = lane < B ? nsteps(lane) * per_b : 0;
    int tot = n, pre = lane < b ? n : 0;
    for (int off = 32; off > 0; off >>= 1) {
      tot += __shfl_xor(tot, off);
      pre += __shfl_xor(pre, off);
    }
    T = tot;
    base = pre;
  } else {
    int tot = 0, pre = 0;
    for (int bb = threadIdx.x; bb < B; bb += kMergeThreads) {
      const int n = nsteps(bb) * per_b;
      tot += n;
      pre += (bb < b) ? n : 0;
    }
    for (int off = 32; off > 0; off >>= 1) {
      tot += __shfl_xor(tot, off);
      pre += __shfl_xor(pre, off);
    }
    if (lane == 0) {
      s_tot[wave] = tot;
      s_pre[wave] = pre;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      T += s_tot[i];
      base += s_pre[i];
    }
  }
  const int R = steps_per_wave(T, W, rmin);
  const int G = Hq / Hkv;
  const int seg = (hq / G) * QG + (hq % G) / 16;
  const int S = base + seg * nb;
  const int nc = nb > 0 ? (S + nb - 1) / R - S / R + 1 : 0;
  // Wave-level maximum and weighted sums over this wave's pieces (every lane reads the
  // same lse values); pieces beyond the first kSpec per wave (long segments) are read here.
  float M = kNegInf;
#pragma unroll
  for (int u = 0; u < kSpec; ++u)
    if (wave + u * NW < nc) M = fmaxf(M, lv[u]);
  for (int ci = wave + kSpec * NW; ci < nc; ci += NW) M = fmaxf(M, pl[ci]);
  float ssum = 0.f;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  const float Mref = (M == kNegInf) ? 0.f : M;
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    if (wave + u * NW < nc) {
      const float w = fast_exp2((lv[u] - Mref) * kLog2e);
      ssum += w;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = fmaf(w, ov[u][i], acc[i]);
    }
  }
  for (int ci = wave + kSpec * NW; ci < nc; ci += NW) {
    const float w = fast_exp2((pl[ci] - Mref) * kLog2e);
    ssum += w;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = fmaf(w, po[(size_t)ci * D + i], acc[i]);
  }
  if (lane == 0) {
    s_m[wave] = M;
    s_l[wave] = ssum;
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) s_acc[wave][lane * DPL + i] = acc[i];
  __syncthreads();

  // Combine the four waves (a wave that had no piece contributes weight 0).
  float Mt = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) Mt = fmaxf(Mt, s_m[w]);
  const float Mtr = (Mt == kNegInf) ? 0.f : Mt;
  float wsc[NW], St = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wsc[w] = (s_m[w] == kNegInf) ? 0.f : fast_exp2((s_m[w] - Mtr) * kLog2e);
    St += wsc[w] * s_l[w];
  }
  for (int d = threadIdx.x; d < D; d += kMergeThreads) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o = fmaf(wsc[w], s_acc[w][d], o);
    O[row * D + d] = (nc > 0) ? o / St : 0.f;
  }
  if (threadIdx.x == 0) LSE[row] = (nc > 0) ? Mtr + fast_log2(St) * kLn2 : kNegInf;
}

template <int D, bool PAGED>
hipError_t launch(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int QG = (G + 15) / 16;
  // Persistent wave workers: one workgroup (4 workers, 128 KB of LDS) per CU.
  const int cus = device_cus();
  const int rmin = a.chunk / kStep;  // a piece has at least `chunk` keys' worth of steps
  const Paging pg{a.block_table, a.max_pages, a.page_size, a.num_pages};
  hipLaunchKernelGGL((decode_split_kernel<D, PAGED>), dim3((unsigned)cus), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.seqlens, a.part_o, a.part_lse, a.B,
                     a.Hq, a.Hkv, a.Nk_max, rmin, a.max_pieces, QG, a.scale * kLog2e, pg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)a.Hq, (unsigned)a.B),
                     dim3(kMergeThreads), 0, s, a.seqlens, a.part_o, a.part_lse, a.o, a.lse,
                     a.B, a.Hq, a.Hkv, QG, a.Nk_max, cus * kWaves, rmin, a.max_pieces);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device, queried once per device and kept (the value
// never changes while the process runs; racing first calls store the same number).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_decode_splitkv(const DecodeArgs& a, hipStream_t s) {
  if (a.block_table != nullptr)
    return a.d == 64 ? launch<64, true>(a, s) : launch<128, true>(a, s);
  return a.d == 64 ? launch<64, false>(a, s) : launch<128, false>(a, s);
}

}  // namespace fa
