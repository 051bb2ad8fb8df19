// fa_prefill_bf16.hip — FlashAttention forward (prefill), bf16 in, fp32 accumulate, gfx950.
//
// What is computed ([FA-notes] = "flash-attn" notes, minjae-portfolio.vercel.app,
// §3 tiling / §4 online softmax / §5.2 forward kernel sketch; [LLM-basics] =
// "LLM 기초 — Attention부터 FlashAttention까지", ③-2 online softmax, ③-5 tile loop):
// one workgroup owns a block of query rows of one (batch, query head).  It keeps
// that Q block in registers and streams the K/V blocks of the matching K/V head
// through LDS.  For each K/V block it forms the scores, updates the running row
// maximum and row sum with the two-block merge, rescales the output accumulator,
// and adds P V to it.  S and P live only in registers.  At the end O = acc / l
// and LSE = m + ln l are written.
//
// gfx950 mapping
//   * WAVES wave64s per workgroup, 32 query rows each.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = 32 keys x 16 d read from LDS, B = the Q^T fragment kept in VGPRs for the
//     whole loop.  In the 32x32 result a lane holds 16 keys of ONE query row
//     (row = lane % 32), so a row maximum is an in-lane max plus one exchange
//     between the wave halves (v_permlane32_swap).
//   * O^T = V^T P^T with the same instruction: B = P^T straight from the score
//     registers (rounded to bf16), A = V^T read from the row-major V block with
//     ds_read_b64_tr_b16 (the LDS unit transposes 4x4 blocks of 16-bit values in
//     flight).  The keys of the P fragment come in the order the score layout
//     produces them, and the transposed reads fetch V rows in that same order.
//   * K/V blocks of 64 keys go from HBM straight into LDS (buffer_load ... lds, no
//     VGPR staging), double-buffered.  K block j+2 and V block j+1 are in flight
//     while block j is processed, so each iteration needs one barrier.
//   * The scores of block j+1 (MFMA) are issued before the softmax of block j
//     (VALU) so the two can overlap.
//   * Row chunks in LDS are XOR-swizzled so the MFMA operand reads are free of
//     bank conflicts.
//   * exp2 with scale*log2(e) folded into one FMA per score.  The exponent
//     reference is the first block's row maximum, and it is moved (to a half
//     block's row maximum, with the accumulator rescale) only when that half
//     block's exponentials add up to more than kSumCap in some lane: the
//     online-softmax identity holds for any common reference value, and the cap
//     keeps every weight <= 2^8.  The common case therefore computes no row
//     maximum and no rescale at all; the rare half block that trips the cap is
//     recomputed after the move.
//   * The softmax of each block is done in two 32-key halves: the first overlaps
//     the next block's score MFMAs, the second the first half's P.V MFMAs.
//   * Buffer loads clip at the end of each (batch, head) slice, so rows past Nq
//     or Nk read as zeros without branches.
//   * Workgroups find their work from the XCD they run on (each XCD has its own
//     L2): an XCD owns whole (batch, K/V head) groups where they divide over the
//     XCDs, runs them from the last query block (most keys under a causal mask) to
//     the first with the GQA group's query heads adjacent, so workgroups sharing
//     K/V run together on one XCD; otherwise the bundles are dealt out in a snake
//     so every XCD gets equal work (xcd_work).
//   * Causal: key blocks wholly in the future of the workgroup's rows are never
//     visited; only blocks crossing the diagonal or the ragged end are masked.
//   * Small grids (at most two workgroups per CU): the workgroup
//     has two key groups of WAVES waves on the same query rows, taking alternate key
//     blocks; group 1 hands its state to group 0 through LDS at the end, and group 0
//     merges the two states by the two-block rule before the epilogue.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBN = 64;        // keys per K/V block
constexpr float kSumCap = 256.f;  // largest per-lane half-block sum of exp2(S*c - m_ref)

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// XOR swizzles of the 16-byte chunk index inside an LDS row of D bf16.
template <int D>
struct Swz {
  // K: 16 consecutive rows read at the same chunk land in 16 different bank groups.
  static __device__ __forceinline__ int k(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
  }
  // V: the 4 rows x 4 chunks a half-wave touches in one transposed read are distinct.
  static __device__ __forceinline__ int v(int row) {
    return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
  }
};

// Loads of one 64-key block (all D columns) straight into LDS.  Each instruction
// fills 1 KB of LDS in lane order; the global chunk a lane fetches is chosen so the
// LDS copy ends up swizzled.  The per-lane byte offsets are fixed (block_offsets);
// the block's row offset goes in the scalar offset (issue_block).
template <int D, int WAVES>
struct BlockShape {
  static constexpr int CH = D / 8;
  static constexpr int INSTS = kBN * CH / 64;
  static constexpr int PER_WAVE = INSTS / WAVES;
  static_assert(PER_WAVE * WAVES == INSTS, "block split");
};

template <int D, int WAVES, bool IS_V>
__device__ __forceinline__ void block_offsets(uint32_t* voff, uint32_t row_bytes, int wave,
                                              int lane) {
  using S = BlockShape<D, WAVES>;
#pragma unroll
  for (int i = 0; i < S::PER_WAVE; ++i) {
    const int lin = (wave * S::PER_WAVE + i) * 64 + lane;
    const int row = lin / S::CH;
    const int pos = lin % S::CH;
    const int c = pos ^ (IS_V ? Swz<D>::v(row) : Swz<D>::k(row));
    voff[i] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
  }
}

template <int D, int WAVES>
__device__ __forceinline__ void issue_block(__amdgpu_buffer_rsrc_t rs, const uint32_t* voff,
                                            uint32_t soff, uint16_t* tile, int wave) {
  using S = BlockShape<D, WAVES>;
#pragma unroll
  for (int i = 0; i < S::PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)(tile + (wave * S::PER_WAVE + i) * 512), 16, voff[i], soff, 0, 0);
}

__device__ __forceinline__ int xcd_remap(int g, int T) {
  const int q = T / kXcds, r = T % kXcds;
  const int x = g % kXcds, i = g / kXcds;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Variable-length batches packed along the token axis ([FA3-entry] §2): sequence b owns
// query rows cu_q[b] .. cu_q[b+1] - 1 and key rows cu_k[b] .. cu_k[b+1] - 1 (offsets are
// clamped into [0, total], lengths to the kernel's Nq / Nk, which then hold the longest
// query and key sequence); consecutive tokens are `*_stride` elements apart, which also
// lets Q/K/V be views into one packed QKV tensor.  O is [total_q, Hq, d], LSE [Hq, total_q].
struct Varlen {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int q_stride, kv_stride;
};

// KSPLIT: two groups of WAVES waves share the workgroup's query rows and split its key
// blocks between them (group g takes blocks g, g+2, g+4, ...), each with its own LDS
// stages; at the end group 1 hands its running state (reference, sums, accumulator)
// through LDS and group 0 merges it with its own by the two-block rule ([FA-notes] §4)
// before the epilogue.  For grids too small to fill the GPU: the key loop of a workgroup
// halves and each SIMD gets a second wave.
template <int D, int WAVES, bool CAUSAL, bool VARLEN, bool KSPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(WAVES * 64 * (KSPLIT ? 2 : 1),
                                                      WAVES * 64 * (KSPLIT ? 2 : 1)),
                          amdgpu_waves_per_eu(2, 2))) void
prefill_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, float* __restrict__ O,
                    float* __restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk, float c,
                    int n_mblocks, Varlen vl) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int BM = 32 * WAVES;
  constexpr int NG = KSPLIT ? 2 : 1;  // key groups
  // One array per stage: the compiler's wait insertion can then tell an LDS-DMA
  // write into one stage from reads of the other, and does not stall the reads of
  // the current block on the prefetch of the next one.  With key groups each stage
  // holds one block per group.
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[NG * kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t ks1[NG * kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[NG * kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs1[NG * kBN * D];
  uint16_t* const ks[2] = {ks0, ks1};
  uint16_t* const vs[2] = {vs0, vs1};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = KSPLIT ? wave_all / WAVES : 0;  // key group
  const int wave = KSPLIT ? wave_all % WAVES : wave_all;  // row wave within the group
  const uint32_t goff = (uint32_t)grp * kBN * D;  // this group's block inside a stage (elements)
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- which work item: XCD-aware order, heavy query blocks first
  const int G = Hq / Hkv;
  const int T = n_mblocks * B * Hq;
  int hg, mb, kvh, b;
  if (!VARLEN) {
    // equal sequences: bundles are one query block of one (batch, K/V head) group's G
    // query heads, heaviest (last) query block first
    const XcdWork w = xcd_work((int)blockIdx.x, G, B * Hkv, n_mblocks);
    hg = w.sub;
    mb = n_mblocks - 1 - w.level;
    kvh = w.group % Hkv;
    b = w.group / Hkv;
  } else if (Hkv % kXcds == 0) {
    // unequal sequences: K/V head major, so each XCD's contiguous slice holds whole K/V
    // heads of every sequence (equal work per XCD), the group's heads adjacent
    const int lam = xcd_remap((int)blockIdx.x, T);
    hg = lam % G;
    const int rest = lam / G;
    mb = n_mblocks - 1 - rest % n_mblocks;
    const int bk = rest / n_mblocks;
    b = bk % B;
    kvh = bk / B;
  } else {
    // fewer K/V heads than XCDs: query head major (balanced when Hq is a multiple of 8)
    const int lam = xcd_remap((int)blockIdx.x, T);
    mb = n_mblocks - 1 - lam % n_mblocks;
    const int rest = lam / n_mblocks;
    b = rest % B;
    const int h = rest / B;
    hg = h % G;
    kvh = h / G;
  }
  const int hq = kvh * G + hg;
  const int m0 = mb * BM;

  // ---- this sequence's rows: fixed-length batch, or a slice of the packed batch
  uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const uint16_t* Qb = Q + ((size_t)b * Nq * Hq + hq) * D;
  const uint16_t* Kb = K + ((size_t)b * Nk * Hkv + kvh) * D;
  const uint16_t* Vb = V + ((size_t)b * Nk * Hkv + kvh) * D;
  size_t o_row0 = (size_t)b * Nq;                 // O row of this sequence's query 0
  size_t lse0 = ((size_t)b * Hq + hq) * Nq;      // LSE index of this sequence's query 0
  if constexpr (VARLEN) {
    const __attribute__((address_space(4))) int* cq = (const __attribute__((address_space(4))) int*)vl.cu_q;
    const __attribute__((address_space(4))) int* ck = (const __attribute__((address_space(4))) int*)vl.cu_k;
    const int q0 = min(max(cq[b], 0), vl.total_q);
    const int q1 = min(max(cq[b + 1], q0), vl.total_q);
    const int k0 = min(max(ck[b], 0), vl.total_k);
    const int k1 = min(max(ck[b + 1], k0), vl.total_k);
    Nq = __builtin_amdgcn_readfirstlane(min(q1 - q0, Nq));
    Nk = __builtin_amdgcn_readfirstlane(min(k1 - k0, Nk));
    if (m0 >= Nq) return;  // the whole block is past this sequence's end
    q_row_bytes = (uint32_t)vl.q_stride * 2;
    kv_row_bytes = (uint32_t)vl.kv_stride * 2;
    Qb = Q + (size_t)q0 * vl.q_stride + (size_t)hq * D;
    Kb = K + (size_t)k0 * vl.kv_stride + (size_t)kvh * D;
    Vb = V + (size_t)k0 * vl.kv_stride + (size_t)kvh * D;
    o_row0 = (size_t)q0;
    lse0 = (size_t)hq * vl.total_q + q0;
  }
  // ---- key blocks to visit
  const int diag = Nk - Nq;  // key j visible from row i iff j <= i + diag
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(m0 + BM, Nq) - 1 + diag + 1);
  const int n_all = (kend + kBN - 1) / kBN;
  // this group's blocks: absolute block index j * NG + grp for j = 0 .. n - 1
  const int n = KSPLIT ? (n_all - grp + 1) / 2 : n_all;
  auto absj = [&](int j) __attribute__((always_inline)) { return j * NG + grp; };
  if constexpr (VARLEN) {
    if (n_all <= 0) {
      // no key visible from any row of the block (no keys, or causal with more queries
      // than keys): the rows' softmax is empty -> O = 0, LSE = -inf
      const int r = m0 + tid / 2;  // two threads per row, D/2 columns each
      if (tid < 2 * BM && r < Nq) {
        float* Orow = O + ((o_row0 + r) * Hq + hq) * D + (tid & 1) * (D / 2);
#pragma unroll
        for (int i = 0; i < D / 2; i += 4) *reinterpret_cast<f32x4*>(Orow + i) = f32x4{};
        if ((tid & 1) == 0) LSE[lse0 + r] = kNegInf;
      }
      return;
    }
  }
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qb, (uint32_t)(Nq - 1) * q_row_bytes + D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb, (uint32_t)(Nk - 1) * kv_row_bytes + D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vb, (uint32_t)(Nk - 1) * kv_row_bytes + D * 2);

  // ---- Q^T fragments: lane holds query row qrow, d = 16*s + 8*hi .. +7 (zeros past Nq)
  const int qrow = m0 + wave * 32 + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        rq, (uint32_t)qrow * q_row_bytes + (uint32_t)(16 * s + 8 * hi) * 2, 0, 0);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  // ---- per-lane LDS byte offsets of the MFMA operand reads
  // K (A of S^T): row kb*32 + l32, logical chunk 2*st + hi.
  uint32_t koff[D / 16];
  {
    const int sk = Swz<D>::k(l32);  // (kb*32 + l32) has the same swizzle for both kb
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      koff[st] = goff * 2 + (uint32_t)(l32 * D * 2 + (((2 * st + hi) ^ sk) * 16));
  }
  // V (A of O^T) through transposed reads: in each 16-lane group, lane p points at
  // row key0 + p/4 and columns d0 + 4*(p%4) .. +3; the group then receives
  // V[key0 + i][d0 + p] for i = 0..3.
  uint32_t voff[D / 32];
  {
    const int p = lane & 15;
    const int g = lane >> 4;
    const int rowl = 4 * hi + (p >> 2);        // row inside the 16-key step (+16u + 8e)
    const int sv = Swz<D>::v(rowl);            // rows differ by multiples of 4 only
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int dcol = 32 * db + 16 * (g & 1) + 4 * (p & 3);
      voff[db] = goff * 2 + (uint32_t)(rowl * D * 2 + (((dcol >> 3) ^ sv) * 16) + (dcol & 7) * 2);
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_ref = kNegInf;  // exponent reference (running max, possibly lagging), base 2
  float neg_m = 0.f;      // -m_ref, or 0 while the reference is still -inf
  // This lane's share of the row sums, each in two independent chains: the unrounded
  // weights (for the LSE) and the bf16-rounded ones (O's normaliser).
  float ls_a = 0.f, ls_b = 0.f;
  float lr_a = 0.f, lr_b = 0.f;
  float lim = kSumCap;    // the unrounded sum after the last half block, plus kSumCap

  uint32_t kvo[BlockShape<D, WAVES>::PER_WAVE], vvo[BlockShape<D, WAVES>::PER_WAVE];
  block_offsets<D, WAVES, false>(kvo, kv_row_bytes, wave, lane);
  block_offsets<D, WAVES, true>(vvo, kv_row_bytes, wave, lane);

  // S^T of one block: 16 MFMAs over two independent 32-key accumulators.
  auto qk = [&](const uint16_t* kt, f32x16* s) __attribute__((always_inline)) {
    const char* kb8 = reinterpret_cast<const char*>(kt);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb8 + koff[st] + kb * 32 * D * 2);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
  };

  // -inf for keys past the end or (causal) past this row's last visible key.
  auto mask = [&](f32x16* s, int j) __attribute__((always_inline)) {
    const int rel = qrow + diag - (j * kBN + 4 * hi);  // last visible key, block-relative
    const int relk = Nk - 1 - (j * kBN + 4 * hi);        // last existing key, block-relative
    const int lim = CAUSAL ? min(rel, relk) : relk;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + (r & 3);
        s[kb][r] = (key > lim) ? kNegInf : s[kb][r];
      }
  };

  // Maximum of each row over keys 32h .. 32h + 31 of the block, base-2 units (c > 0).
  auto row_max = [&](const f32x16* s, int h) __attribute__((always_inline)) {
    float mx = s[h][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[h][r]);
    return xor32_max(mx) * c;
  };

  // Move the exponent reference up to the block's row max (online-softmax merge,
  // [FA-notes] §4): old sums and accumulator scale by exp2(m_old - m_new).
  auto rescale_to = [&](float m_blk) __attribute__((always_inline)) {
    const float m_new = fmaxf(m_ref, m_blk);
    // a row that has seen no visible key yet keeps alpha = 1
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_ref - m_new);
    ls_a *= alpha;
    ls_b *= alpha;
    lr_a *= alpha;
    lr_b *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    m_ref = m_new;
    neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
  };

  // P = exp2(S*c - m_ref) for keys 32h .. 32h + 31 of the block (score registers s[h],
  // P fragments pf[2h], pf[2h + 1]), with this lane's weights added to the running sums
  // passed in: ea/eb the fp32 weights (for the LSE), ra/rb the bf16-rounded ones (v_dot2
  // with (1, 1)); O's normaliser adds up exactly the rounded weights, so O = acc / l is a
  // true weighted mean of V whatever the reference.
  auto exp_pack = [&](f32x16* s, bf16x8* pf, int h, float& ea, float& eb, float& ra, float& rb)
      __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = 2 * h + uu;
      const int kb = h;
      const int base = 8 * uu;
      u32x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p0 = fast_exp2(fmaf(s[kb][base + 2 * t], c, neg_m));
        const float p1 = fast_exp2(fmaf(s[kb][base + 2 * t + 1], c, neg_m));
        ea += p0;
        eb += p1;
        w[t] = pack_bf16x2(p0, p1);
        if (t & 1) rb = sum_bf16x2(w[t], rb);
        else ra = sum_bf16x2(w[t], ra);
      }
      pf[u] = __builtin_bit_cast(bf16x8, w);
    }
  };

  // Fold one half block's weights into the running sums (exp_pack has already added them
  // to the copies ea..rb).  A lane whose unrounded sum grew by more than kSumCap over the
  // half block (a score well above the reference, or a reference still at -inf) sends the
  // wave through the rare path: reference moved to the half block's row max (the part of
  // O already accumulated is rescaled with the sums), half block recomputed.  NaN sums
  // take that path too and then propagate.
  auto commit_half = [&](f32x16* s, bf16x8* pf, int h, float ea, float eb, float ra, float rb)
      __attribute__((always_inline)) {
    float tot = ea + eb;
    if (__builtin_amdgcn_ballot_w64(!(tot <= lim)) != 0) {
      rescale_to(row_max(s, h));
      ea = ls_a;
      eb = ls_b;
      ra = lr_a;
      rb = lr_b;
      exp_pack(s, pf, h, ea, eb, ra, rb);
      tot = ea + eb;
    }
    ls_a = ea;
    ls_b = eb;
    lr_a = ra;
    lr_b = rb;
    lim = tot + kSumCap;
  };

  // O^T += V^T P^T over keys 32h .. 32h + 31 of the block, V^T through transposed LDS
  // reads.
  auto pv = [&](const uint16_t* vt, const bf16x8* pf, int h) __attribute__((always_inline)) {
    const __attribute__((address_space(3))) char* vb =
        (const __attribute__((address_space(3))) char*)(vt);
#pragma unroll
    for (int u = 2 * h; u < 2 * h + 2; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_t*)(vb + voff[db] + (16 * u) * D * 2));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4_t*)(vb + voff[db] + (16 * u + 8) * D * 2));
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], acc[db], 0, 0, 0);
      }
  };

  // Block j needs the mask if it runs past the last key, or (causal) past the last key
  // visible from this wave's first row.
  const int wrow0 = m0 + wave * 32;
  auto need_mask = [&](int j) __attribute__((always_inline)) {
    return (j * kBN + kBN > Nk) || (CAUSAL && (j * kBN + kBN - 1 > wrow0 + diag));
  };

  // ---- prologue: K(0), V(0), K(1) in flight; S(0), its mask and max
  f32x16 s_a[2], s_b[2];
  if (!KSPLIT || n > 0) {
    issue_block<D, WAVES>(rk, kvo, (uint32_t)absj(0) * kBN * kv_row_bytes, ks[0] + goff, wave);
    issue_block<D, WAVES>(rv, vvo, (uint32_t)absj(0) * kBN * kv_row_bytes, vs[0] + goff, wave);
    if (n > 1)
      issue_block<D, WAVES>(rk, kvo, (uint32_t)absj(1) * kBN * kv_row_bytes, ks[1] + goff, wave);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    qk(ks[0], s_a);
    if (need_mask(absj(0))) mask(s_a, absj(0));
    m_ref = fmaxf(row_max(s_a, 0), row_max(s_a, 1));  // first reference (acc, sums still 0)
    neg_m = (m_ref == kNegInf) ? 0.f : -m_ref;
  }

  // ---- software pipeline.  Iteration j (scores of block j already masked):
  //   phase 1: MFMA S(j+1) = K(j+1) Q^T          | VALU softmax of keys 0..31 of block j
  //   (diagonal or ragged block j+1 only: mask)
  //   phase 2: MFMA O^T += V(j)^T P(j)^T, keys 0..31 | VALU softmax of keys 32..63
  //   phase 3: MFMA O^T += V(j)^T P(j)^T, keys 32..63
  // with the rare reference move (half block redone) after either softmax half.
  // Each phase is one basic block, so the scheduler can interleave that phase's MFMA
  // with its VALU work (one wave issues its instructions in order).
  auto step_next = [&](auto stage_c, int j, f32x16* s_cur, f32x16* s_nxt)
      __attribute__((always_inline)) {
    constexpr int sc = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // this wave's K(j+1), V(j) have landed
    __syncthreads();                      // ... and everyone's; stage sc of K is free
    if (j + 2 < n)
      issue_block<D, WAVES>(rk, kvo, (uint32_t)absj(j + 2) * kBN * kv_row_bytes, ks[sc] + goff,
                            wave);
    issue_block<D, WAVES>(rv, vvo, (uint32_t)absj(j + 1) * kBN * kv_row_bytes, vs[1 - sc] + goff,
                          wave);
    bf16x8 pf[kBN / 16];
    qk(ks[1 - sc], s_nxt);
    float ea = ls_a, eb = ls_b, ra = lr_a, rb = lr_b;
    exp_pack(s_cur, pf, 0, ea, eb, ra, rb);
    // Keep the exp/pack work in this block: without a use here the compiler would sink
    // it past the mask branch, next to its only consumer, and nothing would overlap.
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pf[0])), "v"(__builtin_bit_cast(u32x4, pf[1])),
                 "v"(ea), "v"(eb), "v"(ra), "v"(rb));
    if (need_mask(absj(j + 1))) mask(s_nxt, absj(j + 1));
    commit_half(s_cur, pf, 0, ea, eb, ra, rb);
    pv(vs[sc], pf, 0);
    ea = ls_a, eb = ls_b, ra = lr_a, rb = lr_b;
    exp_pack(s_cur, pf, 1, ea, eb, ra, rb);
    commit_half(s_cur, pf, 1, ea, eb, ra, rb);
    pv(vs[sc], pf, 1);
  };
  auto step_last = [&](auto stage_c, f32x16* s_cur) __attribute__((always_inline)) {
    constexpr int sc = decltype(stage_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    bf16x8 pf[kBN / 16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float ea = ls_a, eb = ls_b, ra = lr_a, rb = lr_b;
      exp_pack(s_cur, pf, h, ea, eb, ra, rb);
      commit_half(s_cur, pf, h, ea, eb, ra, rb);
      pv(vs[sc], pf, h);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  int j = 0;
  for (; j + 2 < n; j += 2) {
    step_next(S0{}, j, s_a, s_b);
    step_next(S1{}, j + 1, s_b, s_a);
  }
  if (j + 1 < n) {
    step_next(S0{}, j, s_a, s_b);
    step_last(S1{}, s_b);
  } else if (!KSPLIT || n > 0) {
    step_last(S0{}, s_a);
  }

  float l_run = lr_a + lr_b;  // this lane's share of the row sum of the bf16-rounded weights
  float l_lse = ls_a + ls_b;  // ... and of the unrounded weights (for the LSE)
  if constexpr (KSPLIT) {
    // every wave passes the same number of barriers: group 0 has n0 + 1 of them (prologue
    // and one per block), group 1 one fewer when the block count is odd, none if it got
    // no block
    const int n0 = (n_all + 1) / 2;
    const int mine = n > 0 ? n + 1 : 0;
    for (int i = mine; i < n0 + 1; ++i) __syncthreads();
    __syncthreads();  // every wave is past its last read of the stage arrays
    // group 1 hands over its state: accumulator in its own part of the stage arrays
    // (one array per row wave), reference and sums in mst
    __shared__ float mst[WAVES][3][64];
    uint16_t* const arr = wave == 0 ? ks0 : wave == 1 ? ks1 : wave == 2 ? vs0 : vs1;
    float* dump = reinterpret_cast<float*>(arr + kBN * D);  // group 1's block of that array
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dump[(db * 16 + r) * 64 + lane] = acc[db][r];
      mst[wave][0][lane] = m_ref;
      mst[wave][1][lane] = l_run;
      mst[wave][2][lane] = l_lse;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = mst[wave][0][lane];
    const float mn = fmaxf(m_ref, m1);
    const float a0 = (m_ref == kNegInf) ? 0.f : fast_exp2(m_ref - mn);
    const float a1 = (m1 == kNegInf) ? 0.f : fast_exp2(m1 - mn);
    l_run = l_run * a0 + mst[wave][1][lane] * a1;
    l_lse = l_lse * a0 + mst[wave][2][lane] * a1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[db][r] = fmaf(acc[db][r], a0, dump[(db * 16 + r) * 64 + lane] * a1);
    m_ref = mn;
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l)
  const float l_tot = xor32_sum(l_run);
  const float l_ex = xor32_sum(l_lse);
  // a row that saw no key (packed batches only: an empty sequence, or causal rows ahead
  // of every key) has l = 0 and acc = 0: O = 0, LSE = -inf
  const float inv = (!VARLEN || l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qrow < Nq) {
    float* Orow = O + ((o_row0 + qrow) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                   acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(Orow + 32 * db + 8 * g + 4 * hi) = w;
      }
    if (hi == 0) LSE[lse0 + qrow] = (l_ex > 0.f) ? (m_ref + fast_log2(l_ex)) * kLn2 : kNegInf;
  }
}

template <int D, int WAVES, bool CAUSAL, bool VARLEN>
hipError_t launch(const PrefillArgs& a, hipStream_t s) {
  constexpr int BM = 32 * WAVES;
  // varlen: Nq / Nk are the longest query / key sequence (Nq sizes the grid)
  const int n_mblocks = (a.Nq + BM - 1) / BM;
  const long long blocks = (long long)n_mblocks * a.B * a.Hq;
  const Varlen vl{a.cu_q, a.cu_k, a.total_q, a.total_k, a.q_stride, a.kv_stride};
  // a grid of at most two workgroups per CU (the two-waves-per-SIMD occupancy of the
  // plain kernel) leaves the GPU waiting on the key loops of its heaviest blocks: two key
  // groups halve them and give every SIMD a second wave
  if (blocks <= 2LL * device_cus() && a.Nk > 2 * kBN) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, WAVES, CAUSAL, VARLEN, true>),
                       dim3((unsigned)blocks), dim3(2 * WAVES * 64), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq,
                       a.Nk, a.scale * kLog2e, n_mblocks, vl);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((prefill_bf16_kernel<D, WAVES, CAUSAL, VARLEN, false>),
                     dim3((unsigned)blocks), dim3(WAVES * 64), 0, s,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), a.o, a.lse, a.B, a.Hq, a.Hkv, a.Nq, a.Nk,
                     a.scale * kLog2e, n_mblocks, vl);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  if (a.cu_q != nullptr) {
    if (a.d == 64) return a.causal ? launch<64, 4, true, true>(a, s) : launch<64, 4, false, true>(a, s);
    return a.causal ? launch<128, 4, true, true>(a, s) : launch<128, 4, false, true>(a, s);
  }
  if (a.d == 64) return a.causal ? launch<64, 4, true, false>(a, s) : launch<64, 4, false, false>(a, s);
  return a.causal ? launch<128, 4, true, false>(a, s) : launch<128, 4, false, false>(a, s);
}

}  // namespace fa
