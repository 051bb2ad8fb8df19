// fa_device.h — small gfx950 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (l ^ 32): the two halves of the wave swap their registers.
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 values rounded to nearest-even bf16 and packed (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t packed, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), one, acc, false);
}

__device__ __forceinline__ u32x4 ldg128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Work order over the XCDs.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup g runs on XCD g % 8 as that XCD's (g / 8)-th), and each XCD has its own L2.
// The grid is NBK groups (a (batch, K/V head) pair: workgroups that stream the same K/V)
// x n_blk block levels (level 0 the heaviest under the causal mask) x `per` workgroups per
// bundle (one level of one group).  Where the groups divide over the XCDs, each XCD owns
// whole groups and runs its share level by level, heaviest first; where they do not but
// the bundles do, the bundles, heaviest first, are dealt to the XCDs in a snake (0..7,
// 7..0, ...), so no XCD gets only the heavy blocks of a group; otherwise each XCD takes a
// contiguous slice of the group-major list.
constexpr int kXcds = 8;

struct XcdWork {
  int level;  // 0 = heaviest block
  int group;  // (batch, K/V head) index
  int sub;    // workgroup within the bundle
};

__device__ __forceinline__ XcdWork xcd_work(int g, int per, int NBK, int n_blk) {
  const int x = g % kXcds, i = g / kXcds;  // workgroup i of XCD x
  const int NB = n_blk * NBK;
  XcdWork w;
  if (NBK % kXcds == 0) {
    const int gpx = NBK / kXcds;  // groups per XCD
    const int r = i / per;
    w.sub = i % per;
    w.level = r / gpx;
    w.group = x * gpx + r % gpx;
  } else if (NB % kXcds == 0) {
    const int j = i / per;
    w.sub = i % per;
    const int gb = j * kXcds + ((j & 1) ? kXcds - 1 - x : x);
    w.level = gb / NBK;
    w.group = gb % NBK;
  } else {
    const int T = NB * per;
    const int q = T / kXcds, rm = T % kXcds;
    const int lam = (x < rm) ? x * (q + 1) + i : rm * (q + 1) + (x - rm) * q + i;
    w.sub = lam % per;
    const int rest = lam / per;
    w.level = rest % n_blk;
    w.group = rest / n_blk;
  }
  return w;
}

}  // namespace fa
