// Device-side helpers shared by the CSA2 kernels (gfx950 / CDNA4, wave64).
//
// Number formats follow "FP4 Main KV Cache To Halve Storage Again" (E2M1 main KV) in the
// DeepSeek V4.1 Flash paper notes and 3.5 of the Chinese reading (E4M3 scales); the
// indexer's fp8 keys are OCP E4M3 ("FN").  Every codec here is exact: the tests compare
// its bytes with an independent host implementation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
#define CSA2_MAX_D_DEV 512
#define CSA2_MAX_WINDOW_DEV 128
#define CSA2_MAX_K_DEV 2048
#define CSA2_MAX_DK_DEV 256
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------- formats
// E2M1 magnitude of y by round-to-nearest, ties to the even code, saturating at 6:
// the seven decision points sit halfway between consecutive magnitudes
// (0 .5 1 1.5 2 3 4 6); at a tie the comparison picks the even code.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  const float a = fabsf(y);
  uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
               (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(y) >> 28) & 8u);
}

__device__ __forceinline__ float e2m1_value(uint32_t code) {
  // magnitudes by code: 0 .5 1 1.5 2 3 4 6 (exact in fp32)
  const uint32_t m = code & 7u;
  float mag = (m < 2u) ? 0.5f * (float)m : __uint_as_float(((m >> 1) + 126u) << 23 | (m & 1u) << 22);
  return (code & 8u) ? -mag : mag;
}

// OCP E4M3 of y: round-to-nearest-even on the 3-bit mantissa, saturating at 448.
// Normal range (|y| >= 2^-6): round the fp32 mantissa at bit 20 and rebias the exponent
// (a mantissa carry moves into the exponent).  Below 2^-6 the grid is uniform with step
// 2^-9, so the code is rint(|y| * 512) (exact scaling; rint is ties-to-even).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a <= 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    code = (u >> 20) - (120u << 3);
  }
  return code | sign;
}

// The same code with both cases computed and one selected (no branch; the subnormal case
// adds 2^14, whose fp32 ulp is 2^-9, so the hardware add rounds |y| to a multiple of 2^-9
// ties-to-even and the low bits of the sum are the code).  Cheaper where a wave's values
// fall on both sides of 2^-6, dearer where they do not; equal to e4m3_encode for every
// fp32 input.
__device__ __forceinline__ uint32_t e4m3_encode_select(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  const uint32_t u = __float_as_uint(a);
  const uint32_t nrm = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  const uint32_t sub = __float_as_uint(a + 16384.0f) - 0x46800000u;  // 0x46800000 = 2^14
  uint32_t code = a < 0.015625f ? sub : nrm;
  code = a <= 448.0f ? code : 0x7Eu;
  return code | sign;
}

// x / s correctly rounded (round to nearest even) for many x and one divisor s > 0, finite
// inputs: r = 1/s correctly rounded once, then per quotient q0 = x r and one exact-residual
// correction q = q0 + (x - q0 s) r with fused multiply-adds (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res. Dev. 1990: with
// r the rounded reciprocal, the corrected quotient is the rounded quotient).  The residual
// must not underflow, so a divisor below 2^-92 is scaled with x by 2^64 first (exact).  The
// sign is taken from x, which also keeps the sign of a zero quotient.
struct ExactQuotient {
  float k, s, r;
  ExactQuotient() = default;
  __device__ __forceinline__ explicit ExactQuotient(float div) {
    k = div < 0x1p-92f ? 0x1p64f : 1.0f;
    s = div * k;
    r = 1.0f / s;
  }
  __device__ __forceinline__ float operator()(float x) const {
    const float xs = x * k;
    const float q0 = xs * r;
    return copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, xs), r, q0), x);
  }
};

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = (e == 0u) ? (float)m * 0.001953125f : __uint_as_float((e + 120u) << 23 | m << 20);
  return (c & 0x80u) ? -mag : mag;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// ---------------------------------------------------------------------------- ordering
// Order-preserving 32-bit key of a visible score (larger score -> larger key); -0 and +0
// map to the same key so that equal scores tie exactly as real numbers do.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ bool visible(float s) { return s > kNegInf; }  // false for NaN

constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
__device__ __forceinline__ uint32_t hist_bin(uint32_t key) { return key >> (32 - kHistBits); }

// ---------------------------------------------------------------------------- reductions
// Cross-lane reductions with DPP (a few cycles each) instead of LDS permutes (~100+
// cycles each, and chained).  A DPP row is 16 lanes; after the quad swaps (xor 1, xor 2),
// the half-row mirror and the row mirror every lane of the row holds the row's total,
// combined in the same order on every lane.  Whole-wave results combine the four row
// totals read back as scalars.  Call from wave-uniform control flow only.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppMirror>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  return v + dpp_mov<kDppMirror>(v);
}
// unsigned minimum / maximum over the 64 lanes of the wave (DPP within rows, then the
// four row results by readlane)
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  v = min(v, dpp_mov_u<kDppXor1>(v));
  v = min(v, dpp_mov_u<kDppXor2>(v));
  v = min(v, dpp_mov_u<kDppHalfMirror>(v));
  v = min(v, dpp_mov_u<kDppMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  v = max(v, dpp_mov_u<kDppXor1>(v));
  v = max(v, dpp_mov_u<kDppXor2>(v));
  v = max(v, dpp_mov_u<kDppHalfMirror>(v));
  v = max(v, dpp_mov_u<kDppMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}
// inclusive suffix sum within each 16-lane row (lane i: lanes i..15 of its row), by
// Hillis-Steele steps with DPP row shifts toward lower lanes (lanes past the row end add 0)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shift_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row16_suffix(uint32_t x) {
  x += dpp_shift_u<0x101>(x);  // row_shl:1
  x += dpp_shift_u<0x102>(x);  // row_shl:2
  x += dpp_shift_u<0x104>(x);  // row_shl:4
  x += dpp_shift_u<0x108>(x);  // row_shl:8
  return x;
}
// inclusive suffix sum over the 64 lanes of the wave
__device__ __forceinline__ uint32_t wave_suffix(uint32_t x) {
  x = row16_suffix(x);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t t3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t add = (row == 0) ? t1 + t2 + t3 : (row == 1) ? t2 + t3 : (row == 2) ? t3 : 0u;
  return x + add;
}
// number of lanes below this one whose bit is set in mask
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}
// Reserve consecutive slots of an LDS counter for the lanes whose pred is set: one atomic
// per wave (lanes keep their order); returns this lane's slot (meaningful where pred).
// Every lane of the wave must call it.
__device__ __forceinline__ uint32_t wave_reserve(uint32_t* counter, bool pred) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return 0;
  const int lane = threadIdx.x & 63;
  const int leader = __builtin_ctzll(mask);
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(mask));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  return base + lanes_below(mask);
}
// the value of lane l ^ 32 (v_permlane32_swap exchanges the two 32-lane halves; a VALU
// op, unlike a shuffle through LDS)
__device__ __forceinline__ float swap_halves(float v) {
  const int b = __builtin_bit_cast(int, v);
  const auto pr = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? pr[0] : pr[1]);
}
__device__ __forceinline__ float lane_read(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

}  // namespace csa2
