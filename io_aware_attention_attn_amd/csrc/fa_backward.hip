// fa_backward.hip — attention backward pass for gfx950 (bf16 MFMA, fp32 softmax math).
//
// Sources: the backward sketch of the "flash-attn" notes, §5.2 (P rebuilt on chip from
// Q, K and the forward's softmax statistics instead of being read back; dV = P^T dO,
// dP = dO V^T), the recomputation note of "LLM 기초 — Attention부터 FlashAttention까지"
// ③-5, and the derivative of the row softmax for the steps the sketch leaves out:
//   D_i = sum_j P_ij dP_ij = sum_c dO_ic O_ic,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// P = exp(scale S - LSE) comes straight from the stored log-sum-exp: no row max and no
// normaliser are recomputed.
//
// Three kernels, in stream order, none of them with atomics (results are bitwise
// reproducible):
//   bwd_prep_kernel   D_i = sum_c dO_ic O_ic and lse2_i = LSE_i * log2(e), per (b, h, i).
//   bwd_dkdv_kernel   one workgroup per 256 keys of one (batch, K/V head), 8 waves of
//                     32 keys, two waves per SIMD: K of those keys sits in LDS and -V in
//                     registers while the Q and dO tiles of every query head of the GQA
//                     group stream through LDS; dK and dV accumulate in registers and
//                     are written once.
//   bwd_dq_kernel     one workgroup per 128 query rows of one (batch, query head): Q and
//                     dO rows stay in registers while K and V tiles stream through LDS;
//                     dQ accumulates in registers.
// S and dP are therefore formed twice (once per output side), which trades 40% more
// MFMA work for having no cross-workgroup reduction at all.
//
// MFMA layouts of the dQ kernel (v_mfma_f32_32x32x16_bf16, D = A B): the A operand of
// lane l is row l%32, k = 8(l/32) .. +7; B is column l%32, the same k; D holds column
// l%32, rows 8(r/4) + 4(l/32) + r%4 in register r.  The dK/dV kernel uses
// v_mfma_f32_16x16x32_bf16: A lane l is row l%16, k = 8(l/16) .. +7; B column l%16, the
// same k; D column l%16, rows 4(l/16) + r.  Tiles in LDS are read both as rows (16-byte
// reads) and transposed (ds_read_b64_tr_b16), so one XOR swizzle per kernel serves both.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kTile = 64;  // rows per LDS tile (keys for dQ, query rows for dK/dV)

typedef __attribute__((address_space(3))) void blds_void_t;
typedef __bf16 bbf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bbf16x4 blds_bf16x4_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// XOR applied to the 16-byte chunk index of a tile row.  Row reads: 16 consecutive rows
// at one logical chunk fall on 16 different bank groups.  Transposed reads: the 4
// consecutive rows x 4 chunks one half-wave touches are all distinct.
template <int D>
__device__ __forceinline__ int bswz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// One 64-row tile (all D columns) of a [rows, H, D] bf16 tensor straight into LDS:
// each instruction fills 1 KB in lane order, the global chunk a lane fetches is the one
// that belongs at its swizzled LDS position.
template <int D>
struct TileShape {
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int PER_WAVE = kTile * CH / 64 / 4;  // instructions per wave (4 waves)
};

template <int D>
__device__ __forceinline__ void tile_offsets(uint32_t* off, uint32_t row_bytes, int wave,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < TileShape<D>::PER_WAVE; ++i) {
    const int lin = (wave * TileShape<D>::PER_WAVE + i) * 64 + lane;
    const int row = lin / TileShape<D>::CH;
    const int pos = lin % TileShape<D>::CH;
    off[i] = (uint32_t)row * row_bytes + (uint32_t)(pos ^ bswz<D>(row)) * 16u;
  }
}

template <int D>
__device__ __forceinline__ void tile_issue(__amdgpu_buffer_rsrc_t rs, const uint32_t* off,
                                           uint32_t soff, uint16_t* tile, int wave) {
#pragma unroll
  for (int i = 0; i < TileShape<D>::PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (blds_void_t*)(tile + (wave * TileShape<D>::PER_WAVE + i) * 512), 16, off[i], soff,
        0, 0);
}

// LDS byte offset of the 16-byte chunk (2*st + hi) of tile row `row` (row reads).
template <int D>
__device__ __forceinline__ uint32_t row_chunk(int row, int chunk) {
  return (uint32_t)(row * D * 2 + ((chunk ^ bswz<D>(row)) * 16));
}

// Per-lane LDS byte offsets of the transposed reads that form an A operand X^T[32 d x 16
// rows] from a row-major tile: in each 16-lane group, lane p points at row r0 + p/4 and
// columns d0 + 4(p%4) .. +3, and the group receives X[r0 + i][d0 + p], i = 0..3.  Rows
// 16u + 8e + 4hi + p/4; the swizzle does not depend on u, so toff[db][e] plus 16u rows.
template <int D>
__device__ __forceinline__ void tr_offsets(uint32_t (*toff)[2], int lane) {
  const int p = lane & 15;
  const int g = lane >> 4;
  const int hi = (lane >> 5) & 1;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = 8 * e + 4 * hi + (p >> 2);
      const int dcol = 32 * db + 16 * (g & 1) + 4 * (p & 3);
      toff[db][e] = (uint32_t)(row * D * 2 + (((dcol >> 3) ^ bswz<D>(row)) * 16) + (dcol & 7) * 2);
    }
}

// A operand X^T[32 d (block db) x 16 rows (step u)] from a tile through transposed reads.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, const uint32_t (*toff)[2],
                                             int db, int u) {
  const __attribute__((address_space(3))) char* base =
      (const __attribute__((address_space(3))) char*)(tile);
  const bbf16x4 lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((blds_bf16x4_t*)(base + toff[db][0] + 16 * u * D * 2));
  const bbf16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((blds_bf16x4_t*)(base + toff[db][1] + 16 * u * D * 2));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic and lse2_i = LSE_i log2(e).  D/8 lanes per row, 8 columns each.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ O,
                                                       const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       float* __restrict__ Dws,
                                                       float* __restrict__ L2ws, int B, int Hq,
                                                       int Nq) {
  constexpr int LPR = D / 8;
  const long long rows = (long long)B * Nq * Hq;
  const long long r = (long long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (r < rows) {
    const float* o = O + r * D + part * 8;
    const u32x4 w = ldg128(dO + r * D + part * 8);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(o);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(o + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = fmaf(__uint_as_float(w[t] << 16), (t < 2 ? o0[2 * t] : o1[2 * t - 4]), acc);
      acc = fmaf(__uint_as_float(w[t] & 0xffff0000u), (t < 2 ? o0[2 * t + 1] : o1[2 * t - 3]),
                 acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (r < rows && part == 0) {
    const int h = (int)(r % Hq);
    const long long bi = r / Hq;
    const int i = (int)(bi % Nq);
    const int b = (int)(bi / Nq);
    const size_t idx = ((size_t)b * Hq + h) * Nq + i;
    Dws[idx] = acc;
    L2ws[idx] = LSE[idx] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------
// dK, dV for 256 keys of one (batch, K/V head): 8 waves of 32 keys (two groups of 16),
// two waves per SIMD.  The workgroup's K block sits in LDS and is read as the B operand of
// S = Q K^T; -V stays in registers as the B operand of D - dP.  The dK and dV accumulators
// (32 keys x D each) take half of the wave's 256 registers, which is why a wave holds 32
// keys and not 64, and why K lives in LDS rather than in registers.
//
// With v_mfma_f32_16x16x32_bf16 a lane's S / dP accumulators hold one key (the column)
// and four query rows, which is exactly the k slice the B operand of the dV^T += dO^T P
// and (-dK)^T += Q^T (-dS) products needs from that lane: P and -dS go from the score
// registers to the next product without a lane exchange.  The A operands of those two
// products (dO^T, Q^T) are read transposed from the same tiles, with rows gathered in the
// order the score layout produces them (4g .. 4g+3 and 16+4g .. 16+4g+3 of a 32-row
// block for lane group g).
constexpr int kKeysDKV = 256;  // keys per dK/dV workgroup

// Chunk swizzle of this kernel's tiles (Q, dO and the K block).  ds_read_b128 serves 16
// lanes per pass, the lanes of quads {0,3,5,6} (or {1,2,4,7}) of a half-wave together,
// and the transposed reads serve a half-wave per pass (LDS bank structure measured with
// the SQ_LDS_BANK_CONFLICT counter on gfx950).  The row reads here put 16 rows at one
// logical chunk per 16-lane group, the transposed reads 8 rows x 2 chunks per half-wave;
// with this XOR both patterns hit 16 distinct bank groups per pass.  (The dQ kernel's
// swizzle, made for the 32x32 operand shapes, leaves 2-way conflicts on both.)
template <int D>
__device__ __forceinline__ int dkv_swz(int row) {
  return D == 128 ? ((row & 7) << 1) : (row & 6);
}

template <int D>
__device__ __forceinline__ uint32_t dkv_row_chunk(int row, int chunk) {
  return (uint32_t)(row * D * 2 + ((chunk ^ dkv_swz<D>(row)) * 16));
}

template <int D>
struct DkvShape {
  static constexpr int CH = D / 8;                            // 16-byte chunks per row
  static constexpr int PER_WAVE = kTile * CH / 64 / 8;        // Q / dO tile, per wave
  static constexpr int K_PER_WAVE = kKeysDKV * CH / 64 / 8;   // K block, per wave
};

// One 64-row Q or dO tile into LDS, 8 waves: each instruction fills 1 KB in lane order.
template <int D>
__device__ __forceinline__ void dkv_tile_offsets(uint32_t* off, uint32_t row_bytes, int wave,
                                                 int lane) {
#pragma unroll
  for (int i = 0; i < DkvShape<D>::PER_WAVE; ++i) {
    const int lin = (wave * DkvShape<D>::PER_WAVE + i) * 64 + lane;
    const int row = lin / DkvShape<D>::CH;
    const int pos = lin % DkvShape<D>::CH;
    off[i] = (uint32_t)row * row_bytes + (uint32_t)(pos ^ dkv_swz<D>(row)) * 16u;
  }
}

template <int D>
__device__ __forceinline__ void dkv_tile_issue(__amdgpu_buffer_rsrc_t rs, const uint32_t* off,
                                               uint32_t soff, uint16_t* tile, int wave) {
#pragma unroll
  for (int i = 0; i < DkvShape<D>::PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (blds_void_t*)(tile + (wave * DkvShape<D>::PER_WAVE + i) * 512), 16, off[i], soff,
        0, 0);
}

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512),
                          amdgpu_waves_per_eu(2, 2))) void
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ Dws, const float* __restrict__ L2ws,
                float* __restrict__ dK, float* __restrict__ dV, int B, int Hq, int Hkv, int Nq,
                int Nk, float c, float scale, int n_kblocks) {
  constexpr int PW = DkvShape<D>::PER_WAVE;
  constexpr int KPW = DkvShape<D>::K_PER_WAVE;
  constexpr int CH = DkvShape<D>::CH;
  constexpr int KS = D / 32;  // 32-wide d steps of the S and dP products
  constexpr int DB = D / 16;  // 16-row d blocks of dK^T and dV^T
  __shared__ __attribute__((aligned(1024))) uint16_t qs0[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t qs1[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t os0[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t os1[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t kls[kKeysDKV * D];
  __shared__ __attribute__((aligned(16))) float ls[2][2][kTile];  // [stage][lse2, D][row]
  // stage buffers picked with a select (a runtime-indexed array of LDS pointers would
  // need a static initializer the target cannot express)
  auto qs = [&](int st) __attribute__((always_inline)) { return st ? qs1 : qs0; };
  auto os = [&](int st) __attribute__((always_inline)) { return st ? os1 : os0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p16 = lane & 15;  // key within a 16-key group (column of S, dP)
  const int g = lane >> 4;    // lane group: rows 4g .. 4g+3 of every 16-row block

  const int G = Hq / Hkv;
  // one workgroup per bundle; key block 0 (seen by the most query rows) is the heaviest
  const XcdWork w = xcd_work((int)blockIdx.x, 1, B * Hkv, n_kblocks);
  const int kblk = w.level;
  const int bk = w.group;
  const int kvh = bk % Hkv;
  const int b = bk / Hkv;
  const int n0 = kblk * kKeysDKV;
  const int kw0 = n0 + wave * 32;  // first key of this wave; its keys are kw0 + 16 kg + p16
  const int diag = Nk - Nq;        // key j visible from row i iff j <= i + diag

  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;

  // the workgroup's K block straight into LDS (rows past Nk read as zeros)
  {
    const __amdgpu_buffer_rsrc_t rk =
        brsrc(K + ((size_t)b * Nk * Hkv + kvh) * D, (uint32_t)(Nk - 1) * kv_row_bytes + D * 2);
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int lin = (wave * KPW + i) * 64 + lane;
      const int row = lin / CH;
      const int pos = lin % CH;
      const uint32_t off =
          (uint32_t)(n0 + row) * kv_row_bytes + (uint32_t)(pos ^ dkv_swz<D>(row)) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (blds_void_t*)(kls + (wave * KPW + i) * 512),
                                               16, off, 0, 0, 0);
    }
  }
  // -V^T B operands of this lane's two keys, d = 32 s + 8 g .. +7 (zeros past Nk).  V
  // enters negated (exact in bf16) so that the dP product, started from D instead of 0,
  // yields D - dP directly: the softmax gradient needs no subtraction, and dK comes out
  // negated.
  bf16x8 vf[2][KS];
  {
    const __amdgpu_buffer_rsrc_t rv =
        brsrc(V + ((size_t)b * Nk * Hkv + kvh) * D, (uint32_t)(Nk - 1) * kv_row_bytes + D * 2);
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint32_t off =
            (uint32_t)(kw0 + 16 * kg + p16) * kv_row_bytes + (uint32_t)(32 * s + 8 * g) * 2;
        vf[kg][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0) ^ 0x80008000u);
      }
  }

  // query tiles that can see any of the 256 keys: rows >= n0 - diag under the causal
  // mask; tiles from row n0 + 255 - diag on see all of them and need no mask
  const int n_mt = (Nq + kTile - 1) / kTile;
  const int m_first = CAUSAL ? min(max(0, n0 - diag) / kTile, n_mt) : 0;
  const int m_full =
      CAUSAL ? min((max(0, n0 + kKeysDKV - 1 - diag) + kTile - 1) / kTile, n_mt) : 0;
  const int n_it = (n_mt - m_first) * G;
  const int n_open = (n_mt - m_full) * G;  // the first n_open iterations are unmasked

  f32x4 dkt[2][DB], dvt[2][DB];
#pragma unroll
  for (int kg = 0; kg < 2; ++kg)
#pragma unroll
    for (int i = 0; i < DB; ++i) {
      dkt[kg][i] = f32x4{};
      dvt[kg][i] = f32x4{};
    }

  // row reads (A operands of S and dP, B operands from the K block): row 16x + p16,
  // chunk 4s + g; the swizzle depends on the row's low four bits only, so the 16-row
  // block and the key group enter as immediate offsets
  uint32_t roff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) roff[s] = dkv_row_chunk<D>(p16, 4 * s + g);
  // transposed reads: lane p16 of group g points at row 4g + p16/4 and columns
  // 16 db + 4 (p16 % 4) .. +3, and the group receives X[row0 + i][16 db + p16].  The
  // offset for d block db is block 0's with 32 db XORed in: the swizzle permutes chunks,
  // and block db's two chunks differ from block 0's only in bits 1.. of the chunk index.
  uint32_t toff0;
  {
    const int row = 4 * g + (p16 >> 2);
    const int dcol = 4 * (p16 & 3);
    toff0 = (uint32_t)(row * D * 2 + (((dcol >> 3) ^ dkv_swz<D>(row)) * 16) + (dcol & 7) * 2);
  }
  uint32_t tl[PW];
  dkv_tile_offsets<D>(tl, q_row_bytes, wave, lane);
  const char* kt = reinterpret_cast<const char*>(kls) + wave * 32 * D * 2;

  // iteration t -> query tile n_mt-1 - t/G, query head t%G of the group: the workgroups of
  // one K/V head that run together all start at the last tile and step through the same
  // Q and dO tiles in the same order, so each tile is fetched from HBM about once per
  // XCD and then hit in its L2
  auto tile_of = [&](int t) __attribute__((always_inline)) { return n_mt - 1 - t / G; };
  auto issue = [&](int t, int stage) __attribute__((always_inline)) {
    const int hq = kvh * G + t % G;
    const int m = tile_of(t) * kTile;
    const __amdgpu_buffer_rsrc_t rq =
        brsrc(Q + ((size_t)b * Nq * Hq + hq) * D, (uint32_t)(Nq - 1) * q_row_bytes + D * 2);
    const __amdgpu_buffer_rsrc_t ro =
        brsrc(dO + ((size_t)b * Nq * Hq + hq) * D, (uint32_t)(Nq - 1) * q_row_bytes + D * 2);
    dkv_tile_issue<D>(rq, tl, (uint32_t)m * q_row_bytes, qs(stage), wave);
    dkv_tile_issue<D>(ro, tl, (uint32_t)m * q_row_bytes, os(stage), wave);
    if (wave < 2) {
      // rows past Nq read as 0: lse2 = 0 and D = 0 there, and Q, dO rows are 0 too, so
      // those rows add nothing to dK or dV
      const float* src = (wave == 0 ? L2ws : Dws) + ((size_t)b * Hq + hq) * Nq;
      const __amdgpu_buffer_rsrc_t rl = brsrc(src, (uint32_t)Nq * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (blds_void_t*)(&ls[stage][wave][0]), 4,
                                               (uint32_t)lane * 4, (uint32_t)m * 4, 0, 0);
    }
  };

  // one iteration, with or without the causal mask.  The stage is a runtime value: with
  // the two stages unrolled into one loop body the compiler renames the 32 accumulator
  // registers between the copies and runs out of registers.
  auto step = [&](auto MASK, int t) __attribute__((always_inline)) {
    const int st = t & 1;
    constexpr bool masked = decltype(MASK)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // this wave's part of tile t has landed
    __syncthreads();                      // ... everyone's; stage st^1 is free again
    if (t + 1 < n_it) issue(t + 1, st ^ 1);
    const char* qt = reinterpret_cast<const char*>(qs(st));
    const char* ot = reinterpret_cast<const char*>(os(st));
    const __attribute__((address_space(3))) char* ob =
        (const __attribute__((address_space(3))) char*)(os(st));
    const __attribute__((address_space(3))) char* qb =
        (const __attribute__((address_space(3))) char*)(qs(st));
    // tile row r sees key kw0 + 16 kg + p16 iff r >= kmin + 16 kg
    const int kmin = kw0 + p16 - diag - tile_of(t) * kTile;

#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      u32x4 pw[2], dw[2];  // P and -dS of the 32-row block kb2 as B operands, per key group
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rb = 2 * kb2 + h;
        // S = Q K^T and D - dP = D + dO (-V)^T for rows 16 rb .. +15
        const f32x4 dd = *reinterpret_cast<const f32x4*>(&ls[st][1][16 * rb + 4 * g]);
        f32x4 s[2] = {f32x4{}, f32x4{}};
        f32x4 dp[2] = {dd, dd};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qt + roff[ks] + rb * 16 * D * 2);
          const bf16x8 ao = *reinterpret_cast<const bf16x8*>(ot + roff[ks] + rb * 16 * D * 2);
#pragma unroll
          for (int kg = 0; kg < 2; ++kg) {
            const bf16x8 kk = *reinterpret_cast<const bf16x8*>(kt + roff[ks] + kg * 16 * D * 2);
            s[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kk, s[kg], 0, 0, 0);
            dp[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, vf[kg][ks], dp[kg], 0, 0, 0);
          }
        }
        // P = 2^(S c - lse2) and -dS = P (D - dP), packed to bf16
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&ls[st][0][16 * rb + 4 * g]);
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          float pv[4], dv4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float pp = fast_exp2(fmaf(s[kg][i], c, -l2[i]));
            if (masked) pp = (16 * rb + 4 * g + i >= kmin + 16 * kg) ? pp : 0.f;
            pv[i] = pp;
            dv4[i] = pp * dp[kg][i];
          }
          pw[kg][2 * h] = pack_bf16x2(pv[0], pv[1]);
          pw[kg][2 * h + 1] = pack_bf16x2(pv[2], pv[3]);
          dw[kg][2 * h] = pack_bf16x2(dv4[0], dv4[1]);
          dw[kg][2 * h + 1] = pack_bf16x2(dv4[2], dv4[3]);
        }
      }
      // dV^T += dO^T P and (-dK)^T += Q^T (-dS) over the 32 rows of block kb2
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t tdb = toff0 ^ (uint32_t)(32 * db);
        const bbf16x4 o0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (blds_bf16x4_t*)(ob + tdb + (32 * kb2) * D * 2));
        const bbf16x4 o1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (blds_bf16x4_t*)(ob + tdb + (32 * kb2 + 16) * D * 2));
        const bbf16x4 q0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (blds_bf16x4_t*)(qb + tdb + (32 * kb2) * D * 2));
        const bbf16x4 q1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (blds_bf16x4_t*)(qb + tdb + (32 * kb2 + 16) * D * 2));
        const bf16x8 ao = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
        const bf16x8 aq = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
          dvt[kg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              ao, __builtin_bit_cast(bf16x8, pw[kg]), dvt[kg][db], 0, 0, 0);
          dkt[kg][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              aq, __builtin_bit_cast(bf16x8, dw[kg]), dkt[kg][db], 0, 0, 0);
        }
        // issue each d block's four reads just ahead of its four products: left free, the
        // compiler hoists all 32 reads and spills
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  using Open = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, CAUSAL>;
  if (n_it > 0) issue(0, 0);
  int t = 0;
  for (; t < n_open; ++t) step(Open{}, t);
  for (; t < n_it; ++t) step(Masked{}, t);

  // dK = scale * (Q^T dS)^T (the accumulator holds -Q^T dS), dV = (dO^T P)^T; lane = key,
  // registers hold d = 16 db + 4g .. +3
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const int key = kw0 + 16 * kg + p16;
    if (key < Nk) {
      float* krow = dK + (((size_t)b * Nk + key) * Hkv + kvh) * D;
      float* vrow = dV + (((size_t)b * Nk + key) * Hkv + kvh) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int col = 16 * db + 4 * g;
        *reinterpret_cast<f32x4*>(krow + col) = dkt[kg][db] * -scale;
        *reinterpret_cast<f32x4*>(vrow + col) = dvt[kg][db];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// dQ for 128 query rows (32 per wave) of one (batch, query head).
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(2, 2))) void
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ Dws, const float* __restrict__ L2ws,
              float* __restrict__ dQ, int B, int Hq, int Hkv, int Nq, int Nk, float c,
              float scale, int n_mblocks) {
  constexpr int PW = TileShape<D>::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) uint16_t ks0[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t ks1[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs0[kTile * D];
  __shared__ __attribute__((aligned(1024))) uint16_t vs1[kTile * D];
  auto ks = [&](int st) __attribute__((always_inline)) { return st ? ks1 : ks0; };
  auto vs = [&](int st) __attribute__((always_inline)) { return st ? vs1 : vs0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // work order as in the forward: bundles of one query block of one (batch, K/V head)
  // group's G query heads, heaviest (last) query block first
  const int G = Hq / Hkv;
  const XcdWork w = xcd_work((int)blockIdx.x, G, B * Hkv, n_mblocks);
  const int hg = w.sub;
  const int mb = n_mblocks - 1 - w.level;
  const int bk = w.group;
  const int kvh = bk % Hkv;
  const int b = bk / Hkv;
  const int hq = kvh * G + hg;
  const int m0 = mb * 128;
  const int qrow = m0 + wave * 32 + l32;  // this lane's query row (column of S^T, dP^T)
  const int diag = Nk - Nq;

  const uint32_t q_row_bytes = (uint32_t)Hq * D * 2;
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;

  // Q and dO rows of this lane (B operands; zeros past Nq), and its lse2 / D
  bf16x8 qf[D / 16], of[D / 16];
  float l2 = 0.f, dd = 0.f;
  {
    const __amdgpu_buffer_rsrc_t rq =
        brsrc(Q + ((size_t)b * Nq * Hq + hq) * D, (uint32_t)(Nq - 1) * q_row_bytes + D * 2);
    const __amdgpu_buffer_rsrc_t ro =
        brsrc(dO + ((size_t)b * Nq * Hq + hq) * D, (uint32_t)(Nq - 1) * q_row_bytes + D * 2);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const uint32_t off = (uint32_t)qrow * q_row_bytes + (uint32_t)(16 * st + 8 * hi) * 2;
      qf[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      of[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
    }
    if (qrow < Nq) {
      const size_t idx = ((size_t)b * Hq + hq) * Nq + qrow;
      l2 = L2ws[idx];
      dd = Dws[idx];
    }
  }

  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(m0 + 128, Nq) - 1 + diag + 1);
  const int n = (kend + kTile - 1) / kTile;

  const __amdgpu_buffer_rsrc_t rk =
      brsrc(K + ((size_t)b * Nk * Hkv + kvh) * D, (uint32_t)(Nk - 1) * kv_row_bytes + D * 2);
  const __amdgpu_buffer_rsrc_t rv =
      brsrc(V + ((size_t)b * Nk * Hkv + kvh) * D, (uint32_t)(Nk - 1) * kv_row_bytes + D * 2);
  uint32_t tl[PW];
  tile_offsets<D>(tl, kv_row_bytes, wave, lane);
  uint32_t toff[D / 32][2];
  tr_offsets<D>(toff, lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  // -D of this lane's row in every accumulator register: the dP^T products start from it,
  // so they end at dP - D with no subtraction per score
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = -dd;

  // key tiles every row of the block sees in full (and that lie inside Nk) need no mask
  const int n_open =
      min(n, (CAUSAL ? min(m0 + diag, Nk - 1) + 1 : Nk) / kTile);

  if (n > 0) {
    tile_issue<D>(rk, tl, 0, ks(0), wave);
    tile_issue<D>(rv, tl, 0, vs(0), wave);
  }
  // one key tile on LDS stage ST (compile-time, so LDS addresses fold into immediates),
  // with or without the causal / key-range mask
  auto step = [&](auto ST, auto MASK, int j) __attribute__((always_inline)) {
    constexpr int st = decltype(ST)::value;
    constexpr bool masked = decltype(MASK)::value;
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (j + 1 < n) {
      tile_issue<D>(rk, tl, (uint32_t)(j + 1) * kTile * kv_row_bytes, ks(st ^ 1), wave);
      tile_issue<D>(rv, tl, (uint32_t)(j + 1) * kTile * kv_row_bytes, vs(st ^ 1), wave);
    }
    const char* kt = reinterpret_cast<const char*>(ks(st));
    const char* vt = reinterpret_cast<const char*>(vs(st));

    // per 32-key half: S^T = K Q^T and dP^T - D = V dO^T - D (lane = query row), then dS^T, then
    // dQ^T += K^T dS^T; half 1's products overlap half 0's VALU work
    f32x16 s[2], dp[2];
    bf16x8 dsp[4];
    const int lim = CAUSAL ? min(qrow + diag, Nk - 1) - j * kTile - 4 * hi
                           : Nk - 1 - j * kTile - 4 * hi;
    auto sdp = [&](int kb) __attribute__((always_inline)) {
      s[kb] = f32x16{};
      dp[kb] = negd;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int row = 32 * kb + l32;
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kt + row_chunk<D>(row, 2 * kk + hi));
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(vt + row_chunk<D>(row, 2 * kk + hi));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[kk], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, of[kk], dp[kb], 0, 0, 0);
      }
    };
    auto grad = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 2 * kb; u < 2 * kb + 2; ++u) {
        const int base = 8 * (u & 1);
        u32x4 w;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float v2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = base + 2 * t + e;
            const int kl = kb * 32 + 8 * (r >> 2) + (r & 3);
            float p = fast_exp2(fmaf(s[kb][r], c, -l2));
            if (masked) p = (kl <= lim) ? p : 0.f;
            v2[e] = p * dp[kb][r];  // P (dP - D)
          }
          w[t] = pack_bf16x2(v2[0], v2[1]);
        }
        dsp[u] = __builtin_bit_cast(bf16x8, w);
      }
    };
    auto accum = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 2 * kb; u < 2 * kb + 2; ++u)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 a = tr_operand<D>(ks(st), toff, db, u);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsp[u], acc[db], 0, 0, 0);
        }
    };
    sdp(0);
    sdp(1);
    grad(0);
    accum(0);
    grad(1);
    accum(1);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Open = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  int j = 0;
  for (; j + 1 < (n_open & ~1); j += 2) {
    step(S0{}, Open{}, j);
    step(S1{}, Open{}, j + 1);
  }
  for (; j + 1 < n; j += 2) {
    step(S0{}, Masked{}, j);
    step(S1{}, Masked{}, j + 1);
  }
  if (j < n) step(S0{}, Masked{}, j);

  if (qrow < Nq) {
    float* row = dQ + (((size_t)b * Nq + qrow) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(row + 32 * db + 8 * g + 4 * hi) =
            f32x4{acc[db][4 * g] * scale, acc[db][4 * g + 1] * scale, acc[db][4 * g + 2] * scale,
                  acc[db][4 * g + 3] * scale};
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BackwardArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.Nq * a.Hq;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256),
                     0, s, a.o, static_cast<const uint16_t*>(a.dout), a.lse, a.dsum, a.lse2,
                     a.B, a.Hq, a.Nq);
  const float c = a.scale * kLog2e;
  const int n_kblocks = (a.Nk + kKeysDKV - 1) / kKeysDKV;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(n_kblocks * a.B * a.Hkv)),
                     dim3(512), 0, s, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const uint16_t*>(a.dout), a.dsum, a.lse2, a.dk, a.dv, a.B, a.Hq,
                     a.Hkv, a.Nq, a.Nk, c, a.scale, n_kblocks);
  const int n_mblocks = (a.Nq + 127) / 128;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(n_mblocks * a.B * a.Hq)),
                     dim3(256), 0, s, static_cast<const uint16_t*>(a.q),
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const uint16_t*>(a.dout), a.dsum, a.lse2, a.dq, a.B, a.Hq,
                     a.Hkv, a.Nq, a.Nk, c, a.scale, n_mblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
  return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
}

}  // namespace fa
