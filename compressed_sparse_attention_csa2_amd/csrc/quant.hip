// Write side: FP4 (E2M1, per-channel fp32 scale, or one E4M3 scale per 16 channels of each
// entry) main-KV pack and E4M3 per-row quantise.
// "FP4 Main KV Cache To Halve Storage Again" (paper notes) / 3.5 of the Chinese reading:
// the main KV is stored as E2M1 and dequantised before attention.  The per-channel scale
// is the absmax over the sequence's rows divided by 6 (the largest E2M1 magnitude).
//
// HBM-bound streaming kernels: 16-byte coalesced row reads where the shape allows (else one
// 32-bit word or one byte of codes per thread), absmax by an order-preserving atomicMax on
// the fp32 bit pattern (abs values are non-negative, so unsigned order == float order; the
// max does not depend on order).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace csa2 {

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// 16-byte stores (p 16-byte aligned, n a multiple of 4)
__global__ void k_fill_u32x4(uint4* p, int64_t n4, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(v, v, v, v);
}

// absmax over rows of each channel: grid (ceil(D/256), row chunks, B)
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4_absmax(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                    int rows_per_block, uint32_t* __restrict__ amax_bits) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.z;
  if (c >= D) return;
  const int t0 = blockIdx.y * rows_per_block;
  const int t1 = min(T, t0 + rows_per_block);
  float m = 0.0f;
  const XT* xp = x + b * xsb + c;
  for (int t = t0; t < t1; ++t) m = fmaxf(m, fabsf(load_as_f32(xp + t * xst)));
  atomicMax(&amax_bits[(int64_t)b * D + c], __float_as_uint(m));
}

__global__ void k_fp4_finalize_scales(int64_t n, float* scales) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) scales[i] = __uint_as_float(__float_as_uint(scales[i])) / 6.0f;
}

// pack: one thread per 8 channels (one 32-bit word of codes) of one row
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4_pack(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                  const int32_t* __restrict__ n0, int64_t n_max,
                                                  uint8_t* __restrict__ codes, const float* __restrict__ scales) {
  const int words = D / 8;
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (g >= (int64_t)T * words) return;
  const int t = (int)(g / words), w8 = (int)(g % words);
  const int64_t row = (int64_t)(n0 ? n0[b] : 0) + t;
  if (row < 0 || row >= n_max) return;
  const XT* xr = x + b * xsb + t * xst + w8 * 8;
  const float* s = scales + (int64_t)b * D + w8 * 8;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float si = s[i];
    const uint32_t code = (si != 0.0f) ? e2m1_encode(load_as_f32(xr + i) / si) : 0u;
    word |= code << (4 * i);
  }
  *reinterpret_cast<uint32_t*>(codes + ((int64_t)b * n_max + row) * (D / 2) + w8 * 4) = word;
}

// One 16-byte chunk of x as fp32: 4 channels of fp32 input, 8 of bf16.
template <typename XT>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int C = 4;
  template <bool NT>
  __device__ __forceinline__ static void load(const float* p, float (&v)[C]) {
    const v4f a = NT ? __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p)) : *reinterpret_cast<const v4f*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
};
template <>
struct Chunk<uint16_t> {
  static constexpr int C = 8;
  template <bool NT>
  __device__ __forceinline__ static void load(const uint16_t* p, float (&v)[C]) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u a = NT ? __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p)) : *reinterpret_cast<const v4u*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
  }
};

// Vector forms for rows of D channels in 16-byte chunks, where the chunks per row divide 256
// and rows start 16-byte aligned.  Thread i of a 256-thread block reads chunk i % chunks of
// rows r + i / chunks, stepping 256 / chunks rows, so every wave load is one contiguous
// kilobyte.  absmax: each block walks a run of `rpb` rows with kAbsUnroll loads in flight
// and few blocks (each adds one atomic per channel); pack: groups of kPackUnroll steps are
// dealt to the blocks round robin.
constexpr int kAbsUnroll = 8, kPackUnroll = 4;

// absmax: per-thread maxima, reduced per channel in LDS (as unsigned: the bits of
// non-negative fp32 values order like the values), then one global atomic per channel and block.
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4_absmax_v(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                      int rpb, uint32_t* __restrict__ amax_bits) {
  constexpr int C = Chunk<XT>::C;
  __shared__ uint32_t s_m[CSA2_MAX_D_DEV];
  const int chunks = D / C, lanes_r = 256 / chunks;
  const int w = threadIdx.x % chunks, rl = threadIdx.x / chunks;
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < D; i += 256) s_m[i] = 0u;
  float m[C];
#pragma unroll
  for (int i = 0; i < C; ++i) m[i] = 0.0f;
  const int t0 = blockIdx.x * rpb, t1 = min(T, t0 + rpb);
  const XT* xb = x + b * xsb + C * w;
  int t = t0 + rl;
  for (; t + (kAbsUnroll - 1) * lanes_r < t1; t += kAbsUnroll * lanes_r) {
    float v[kAbsUnroll][C];
#pragma unroll
    for (int u = 0; u < kAbsUnroll; ++u) Chunk<XT>::template load<false>(xb + (int64_t)(t + u * lanes_r) * xst, v[u]);
#pragma unroll
    for (int u = 0; u < kAbsUnroll; ++u)
#pragma unroll
      for (int i = 0; i < C; ++i) m[i] = fmaxf(m[i], fabsf(v[u][i]));
  }
  for (; t < t1; t += lanes_r) {
    float v[C];
    Chunk<XT>::template load<false>(xb + (int64_t)t * xst, v);
#pragma unroll
    for (int i = 0; i < C; ++i) m[i] = fmaxf(m[i], fabsf(v[i]));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C; ++i) atomicMax(&s_m[C * w + i], __float_as_uint(m[i]));
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += 256) {
    const uint32_t v = s_m[i];
    if (v) atomicMax(&amax_bits[(int64_t)b * D + i], v);
  }
}

// Codes of one chunk: C / 2 bytes (fp32 input: 16 bits, bf16: 32 bits).
template <int C>
struct ChunkCodes;
template <>
struct ChunkCodes<4> {
  using T = uint16_t;
};
template <>
struct ChunkCodes<8> {
  using T = uint32_t;
};

// pack: each thread quantises its chunk's channels for every row it visits.  The quotient
// x / s_c is one correctly rounded reciprocal per channel plus a fused-multiply-add
// correction per value (ExactQuotient: the same value as the division); a scale that is not
// positive and finite, or a quotient that overflows, takes the division itself.  The loads
// are the last use of x, so they bypass the caches' retention.
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4_pack_v(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                    const int32_t* __restrict__ n0, int64_t n_max,
                                                    uint8_t* __restrict__ codes, const float* __restrict__ scales) {
  constexpr int C = Chunk<XT>::C;
  using CT = typename ChunkCodes<C>::T;
  const int chunks = D / C, lanes_r = 256 / chunks;
  const int w = threadIdx.x % chunks, rl = threadIdx.x / chunks;
  const int b = blockIdx.y;
  float sc[C];
  bool fast[C];
  ExactQuotient eq[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    sc[i] = scales[(int64_t)b * D + C * w + i];
    fast[i] = sc[i] > 0.0f && sc[i] <= 3.0e38f;
    eq[i] = ExactQuotient(fast[i] ? sc[i] : 1.0f);
  }
  const int64_t base = n0 ? n0[b] : 0;
  const XT* xb = x + b * xsb + C * w;
  uint8_t* cb = codes + (int64_t)b * n_max * (D / 2) + (C / 2) * w;
  auto encode = [&](const float (&v)[C]) -> CT {
    CT word = 0;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      uint32_t code = 0u;
      if (sc[i] != 0.0f) {
        float y = fast[i] ? eq[i](v[i]) : v[i] / sc[i];
        if (!(fabsf(y) <= 3.4e38f)) y = v[i] / sc[i];
        code = e2m1_encode(y);
      }
      word |= (CT)(code << (4 * i));
    }
    return word;
  };
  auto store = [&](int tt, CT word) {
    const int64_t row = base + tt;
    if (row >= 0 && row < n_max) *reinterpret_cast<CT*>(cb + row * (D / 2)) = word;
  };
  const int R = kPackUnroll * lanes_r;  // rows per group
  for (int g = blockIdx.x; (int64_t)g * R < T; g += gridDim.x) {
    int t = g * R + rl;
    if ((g + 1) * (int64_t)R <= T) {
      float v[kPackUnroll][C];
#pragma unroll
      for (int u = 0; u < kPackUnroll; ++u) Chunk<XT>::template load<true>(xb + (int64_t)(t + u * lanes_r) * xst, v[u]);
#pragma unroll
      for (int u = 0; u < kPackUnroll; ++u) store(t + u * lanes_r, encode(v[u]));
    } else {
      for (; t < T; t += lanes_r) {
        float v[C];
        Chunk<XT>::template load<true>(xb + (int64_t)t * xst, v);
        store(t, encode(v));
      }
    }
  }
}

// pack for D not a multiple of 8: one thread per byte (two channels)
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4_pack_bytes(int T, int D, const XT* __restrict__ x, int64_t xsb,
                                                        int64_t xst, const int32_t* __restrict__ n0, int64_t n_max,
                                                        uint8_t* __restrict__ codes, const float* __restrict__ scales) {
  const int bytes = D / 2;
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (g >= (int64_t)T * bytes) return;
  const int t = (int)(g / bytes), i = (int)(g % bytes);
  const int64_t row = (int64_t)(n0 ? n0[b] : 0) + t;
  if (row < 0 || row >= n_max) return;
  const XT* xr = x + b * xsb + t * xst + 2 * i;
  const float* s = scales + (int64_t)b * D + 2 * i;
  const uint32_t lo = (s[0] != 0.0f) ? e2m1_encode(load_as_f32(xr) / s[0]) : 0u;
  const uint32_t hi = (s[1] != 0.0f) ? e2m1_encode(load_as_f32(xr + 1) / s[1]) : 0u;
  codes[((int64_t)b * n_max + row) * bytes + i] = (uint8_t)(lo | hi << 4);
}

// The pages' layout: one E4M3 scale per 16 channels of each entry, no global scale.  One
// thread per (row, group of 16 channels): sc = E4M3(fl32(amax / 6)), codes E2M1(fl32(x /
// value(sc))).  Consecutive threads take consecutive groups, so the 64 B reads and the 8 B
// code writes are contiguous across a wave.
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4g16_pack(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                     const int32_t* __restrict__ n0, int64_t n_max,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ gscales) {
  const int groups = D / 16;
  const int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (gi >= (int64_t)T * groups) return;
  const int t = (int)(gi / groups), g = (int)(gi % groups);
  const int64_t row = (int64_t)(n0 ? n0[b] : 0) + t;
  if (row < 0 || row >= n_max) return;
  const XT* xr = x + b * xsb + t * xst + 16 * g;
  float v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = load_as_f32(xr + i);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const uint32_t sc = e4m3_encode(amax / 6.0f);
  const float sv = e4m3_value(sc);
  uint32_t w[2] = {0u, 0u};
  if (sv != 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_encode(v[i] / sv) << (4 * (i & 7));
  }
  const int64_t orow = (int64_t)b * n_max + row;
  *reinterpret_cast<uint2*>(codes + orow * (D / 2) + 8 * g) = make_uint2(w[0], w[1]);
  gscales[orow * groups + g] = (uint8_t)sc;
}

// E4M3 per row: one wave per row, lanes stride over the row's D values.
// Vector form of the per-row E4M3 quantise for rows of D channels in 16-byte chunks whose
// count per row divides 64: the chunks of one row sit in adjacent lanes of one wave, so the
// row absmax is a butterfly over those lanes.  Groups of kPackUnroll block steps are dealt
// to the blocks round robin; rows past T load a clamped row and store nothing, so every
// lane takes part in every butterfly.  One ExactQuotient per row replaces the per-value
// division (same quotient), with the division kept for scales it does not cover.
template <typename XT>
__global__ __launch_bounds__(256) void k_fp8_rows_v(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                    const int32_t* __restrict__ n0, int64_t n_max,
                                                    uint8_t* __restrict__ codes, float* __restrict__ scales) {
  constexpr int C = Chunk<XT>::C;
  using CT = typename std::conditional<C == 4, uint32_t, uint64_t>::type;
  const int chunks = D / C, lanes_r = 256 / chunks;
  const int w = threadIdx.x % chunks, rl = threadIdx.x / chunks;
  const int b = blockIdx.y;
  const int64_t base = n0 ? n0[b] : 0;
  const XT* xb = x + b * xsb + C * w;
  const int R = kPackUnroll * lanes_r;
  for (int g = blockIdx.x; (int64_t)g * R < T; g += gridDim.x) {
    float v[kPackUnroll][C];
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
      const int t = min(g * R + rl + u * lanes_r, T - 1);
      Chunk<XT>::template load<true>(xb + (int64_t)t * xst, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < C; ++i) m = fmaxf(m, fabsf(v[u][i]));
      for (int off = chunks >> 1; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float sc = m / 448.0f;
      const bool fast = sc > 0.0f && sc <= 3.0e38f;
      const ExactQuotient eq(fast ? sc : 1.0f);
      CT word = 0;
#pragma unroll
      for (int i = 0; i < C; ++i) {
        uint32_t code = 0u;
        if (sc != 0.0f) {
          float y = fast ? eq(v[u][i]) : v[u][i] / sc;
          if (!(fabsf(y) <= 3.4e38f)) y = v[u][i] / sc;
          code = e4m3_encode(y);
        }
        word |= (CT)code << (8 * i);
      }
      const int t = g * R + rl + u * lanes_r;
      const int64_t row = base + t;
      if (t < T && row >= 0 && row < n_max) {
        *reinterpret_cast<CT*>(codes + ((int64_t)b * n_max + row) * D + C * w) = word;
        if (w == 0) scales[(int64_t)b * n_max + row] = sc;
      }
    }
  }
}

template <typename XT>
__global__ __launch_bounds__(256) void k_fp8_rows(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                  const int32_t* __restrict__ n0, int64_t n_max,
                                                  uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (t >= T) return;
  const int64_t row = (int64_t)(n0 ? n0[b] : 0) + t;
  if (row < 0 || row >= n_max) return;
  const XT* xr = x + b * xsb + t * xst;
  float m = 0.0f;
  for (int d = lane; d < D; d += 64) m = fmaxf(m, fabsf(load_as_f32(xr + d)));
  m = wave_max(m);
  const float s = m / 448.0f;
  uint8_t* out = codes + ((int64_t)b * n_max + row) * D;
  for (int d = lane; d < D; d += 64) out[d] = (uint8_t)(s != 0.0f ? e4m3_encode(load_as_f32(xr + d) / s) : 0u);
  if (lane == 0) scales[(int64_t)b * n_max + row] = s;
}

// E2M1 per row (4-bit indexer keys): one wave per row; s = absmax/6, lanes take pairs of
// dims and write one byte each (the lower dim in the low nibble).
template <typename XT>
__global__ __launch_bounds__(256) void k_fp4_rows(int T, int D, const XT* __restrict__ x, int64_t xsb, int64_t xst,
                                                  const int32_t* __restrict__ n0, int64_t n_max,
                                                  uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (t >= T) return;
  const int64_t row = (int64_t)(n0 ? n0[b] : 0) + t;
  if (row < 0 || row >= n_max) return;
  const XT* xr = x + b * xsb + t * xst;
  float m = 0.0f;
  for (int d = lane; d < D; d += 64) m = fmaxf(m, fabsf(load_as_f32(xr + d)));
  m = wave_max(m);
  const float s = m / 6.0f;
  uint8_t* out = codes + ((int64_t)b * n_max + row) * (D / 2);
  for (int i = lane; i < D / 2; i += 64) {
    const uint32_t lo = s != 0.0f ? e2m1_encode(load_as_f32(xr + 2 * i) / s) : 0u;
    const uint32_t hi = s != 0.0f ? e2m1_encode(load_as_f32(xr + 2 * i + 1) / s) : 0u;
    out[i] = (uint8_t)(lo | hi << 4);
  }
  if (lane == 0) scales[(int64_t)b * n_max + row] = s;
}

int launch_quantize_fp4_rows(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                             const int32_t* n0, int64_t n_max, uint8_t* codes, float* scales, hipStream_t st) {
  dim3 g((T + 3) / 4, B);
  if (bf16)
    hipLaunchKernelGGL(k_fp4_rows<uint16_t>, g, dim3(256), 0, st, T, D, (const uint16_t*)x, xsb, xst, n0, n_max,
                       codes, scales);
  else
    hipLaunchKernelGGL(k_fp4_rows<float>, g, dim3(256), 0, st, T, D, (const float*)x, xsb, xst, n0, n_max, codes,
                       scales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return 0;
  if ((reinterpret_cast<uintptr_t>(p) & 15) == 0 && n % 4 == 0) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_fill_u32x4, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<uint4*>(p), n / 4, v);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename XT>
static int quantize_fp4_t(bool compute, int B, int T, int D, const XT* x, int64_t xsb, int64_t xst, const int32_t* n0,
                          int64_t n_max, uint8_t* codes, float* scales, hipStream_t st) {
  // vector kernels: 16-byte chunks whose count per row divides 256, 16-byte aligned rows
  constexpr int C = Chunk<XT>::C;
  const int chunks = D / C;
  const bool vec = D % C == 0 && D <= CSA2_MAX_D_DEV && 256 % chunks == 0 &&
                   (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (xst * sizeof(XT)) % 16 == 0 &&
                   (xsb * sizeof(XT)) % 16 == 0;
  if (vec) {
    // absmax: about 512 blocks in all, runs of at least 4 unrolled steps
    const int lanes_r = 256 / chunks;
    int64_t rpb = ((int64_t)T * B + 511) / 512;
    rpb = ((rpb + lanes_r - 1) / lanes_r) * lanes_r;
    if (rpb < 4 * kAbsUnroll * lanes_r) rpb = 4 * kAbsUnroll * lanes_r;
    if (compute) {
      if (launch_fill_u32(reinterpret_cast<uint32_t*>(scales), (int64_t)B * D, 0u, st)) return -1;
      hipLaunchKernelGGL(k_fp4_absmax_v<XT>, dim3((unsigned)((T + rpb - 1) / rpb), B), dim3(256), 0, st, T, D, x, xsb,
                         xst, (int)rpb, reinterpret_cast<uint32_t*>(scales));
      const int64_t n = (int64_t)B * D;
      hipLaunchKernelGGL(k_fp4_finalize_scales, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, scales);
    }
    // pack: about 8192 blocks in all, at most one per group of rows
    const int64_t groups = ((int64_t)T + kPackUnroll * lanes_r - 1) / (kPackUnroll * lanes_r);
    const int64_t per_seq = std::max<int64_t>(1, 8192 / B);
    hipLaunchKernelGGL(k_fp4_pack_v<XT>, dim3((unsigned)std::min(groups, per_seq), B), dim3(256), 0, st, T, D, x, xsb,
                       xst, n0, n_max, codes, scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (compute) {
    if (launch_fill_u32(reinterpret_cast<uint32_t*>(scales), (int64_t)B * D, 0u, st)) return -1;
    const int rows_per_block = 256;
    dim3 g((D + 255) / 256, (T + rows_per_block - 1) / rows_per_block, B);
    hipLaunchKernelGGL(k_fp4_absmax<XT>, g, dim3(256), 0, st, T, D, x, xsb, xst, rows_per_block,
                       reinterpret_cast<uint32_t*>(scales));
    const int64_t n = (int64_t)B * D;
    hipLaunchKernelGGL(k_fp4_finalize_scales, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, scales);
  }
  if (D % 8 == 0) {
    const int64_t work = (int64_t)T * (D / 8);
    hipLaunchKernelGGL(k_fp4_pack<XT>, dim3((unsigned)((work + 255) / 256), B), dim3(256), 0, st, T, D, x, xsb, xst,
                       n0, n_max, codes, scales);
  } else {
    const int64_t work = (int64_t)T * (D / 2);
    hipLaunchKernelGGL(k_fp4_pack_bytes<XT>, dim3((unsigned)((work + 255) / 256), B), dim3(256), 0, st, T, D, x, xsb,
                       xst, n0, n_max, codes, scales);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_fp4(bool compute, bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                        const int32_t* n0, int64_t n_max, uint8_t* codes, float* scales, hipStream_t st) {
  if (bf16)
    return quantize_fp4_t(compute, B, T, D, (const uint16_t*)x, xsb, xst, n0, n_max, codes, scales, st);
  return quantize_fp4_t(compute, B, T, D, (const float*)x, xsb, xst, n0, n_max, codes, scales, st);
}

int launch_quantize_fp4_g16(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                            const int32_t* n0, int64_t n_max, uint8_t* codes, uint8_t* gscales, hipStream_t st) {
  const int64_t work = (int64_t)T * (D / 16);
  dim3 g((unsigned)((work + 255) / 256), B);
  if (bf16)
    hipLaunchKernelGGL(k_fp4g16_pack<uint16_t>, g, dim3(256), 0, st, T, D, (const uint16_t*)x, xsb, xst, n0, n_max,
                       codes, gscales);
  else
    hipLaunchKernelGGL(k_fp4g16_pack<float>, g, dim3(256), 0, st, T, D, (const float*)x, xsb, xst, n0, n_max, codes,
                       gscales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_fp8(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst, const int32_t* n0,
                        int64_t n_max, uint8_t* codes, float* scales, hipStream_t st) {
  const int C = bf16 ? Chunk<uint16_t>::C : Chunk<float>::C;
  const int esz = bf16 ? 2 : 4;
  const int chunks = D / C;
  if (D % C == 0 && 64 % chunks == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (xst * esz) % 16 == 0 &&
      (xsb * esz) % 16 == 0 && (reinterpret_cast<uintptr_t>(codes) & 7) == 0) {
    // about 8192 blocks in all, at most one per group of rows
    const int64_t groups = ((int64_t)T + kPackUnroll * (256 / chunks) - 1) / (kPackUnroll * (256 / chunks));
    const dim3 gv((unsigned)std::min<int64_t>(groups, std::max(1, 8192 / B)), B);
    if (bf16)
      hipLaunchKernelGGL(k_fp8_rows_v<uint16_t>, gv, dim3(256), 0, st, T, D, (const uint16_t*)x, xsb, xst, n0, n_max,
                         codes, scales);
    else
      hipLaunchKernelGGL(k_fp8_rows_v<float>, gv, dim3(256), 0, st, T, D, (const float*)x, xsb, xst, n0, n_max, codes,
                         scales);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  dim3 g((T + 3) / 4, B);
  if (bf16)
    hipLaunchKernelGGL(k_fp8_rows<uint16_t>, g, dim3(256), 0, st, T, D, (const uint16_t*)x, xsb, xst, n0, n_max,
                       codes, scales);
  else
    hipLaunchKernelGGL(k_fp8_rows<float>, g, dim3(256), 0, st, T, D, (const float*)x, xsb, xst, n0, n_max, codes,
                       scales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
