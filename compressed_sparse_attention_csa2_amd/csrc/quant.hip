// Write side: FP4 (E2M1, per-channel fp32 scale, or one E4M3 scale per 16 channels of each
// entry) main-KV pack and E4M3 per-row quantise.
// "FP4 Main KV Cache To Halve Storage Again" (paper notes) / 3.5 of the Chinese reading:
// the main KV is stored as E2M1 and dequantised before attention.  The per-channel scale
// is the absmax over the sequence's rows divided by 6 (the largest E2M1 magnitude).
//
// HBM-bound streaming kernels: coalesced row reads, one 32-bit word of packed codes per
// thread, absmax by an order-preserving atomicMax on the fp32 bit pattern (abs values
// are non-negative, so unsigned order == float order; the max does not depend on order).
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
