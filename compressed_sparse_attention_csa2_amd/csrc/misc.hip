// Gather + dequantise, coarse keys of the two-level indexer, candidate expansion.
#include "common.hpp"
#include "launch.hpp"

namespace csa2 {

typedef int v4i_t __attribute__((ext_vector_type(4)));

// out[r][k][c] = fl32(E2M1(code) * s_c) of cache row idx[r][k] (G16: the scale of the
// entry's 16-channel group, E4M3); 0 for rows outside [0, n_max).  One thread per 8
// channels.  (The stored FP4 entries are turned back into real values before the
// attention uses them: "FP4 Main KV Cache To Halve Storage Again", paper notes.)
template <bool G16>
__global__ __launch_bounds__(256) void k_gather_dequant(int T, int K, int D, const uint8_t* __restrict__ codes,
                                                        const void* __restrict__ scales_v, int64_t n_max,
                                                        const int32_t* __restrict__ idx, float* __restrict__ out,
                                                        int64_t total_words) {
  const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (g >= total_words) return;
  const int words = D / 8;
  const int64_t rk = g / words;           // (b*T + t)*K + k
  const int w8 = (int)(g % words);
  const int b = (int)(rk / ((int64_t)T * K));
  const int32_t j = idx[rk];
  float v[8];
  if (j >= 0 && j < n_max) {
    const int64_t row = (int64_t)b * n_max + j;
    const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + row * (D / 2) + w8 * 4);
    if (G16) {
      const float s = e4m3_value(static_cast<const uint8_t*>(scales_v)[row * (D / 16) + w8 / 2]);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = e2m1_value((word >> (4 * i)) & 15u) * s;
    } else {
      const float* s = static_cast<const float*>(scales_v) + (int64_t)b * D + w8 * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = e2m1_value((word >> (4 * i)) & 15u) * s[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float4* o = reinterpret_cast<float4*>(out + rk * D + w8 * 8);
  o[0] = make_float4(v[0], v[1], v[2], v[3]);
  o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Coarse keys: one wave per (sequence, block).  Lane c sums fl32(sk_j * E4M3(k8_jc)) over
// the block's rows in row order in fp32 (each partial sum rounded), divides by the row
// count, then the block's 64 means are re-quantised to E4M3 with their own max/448.
__global__ __launch_bounds__(256) void k_coarse_keys(int64_t n_max, const int32_t* __restrict__ n_keys, int dk,
                                                     int block, int64_t nb_max, const uint8_t* __restrict__ k8,
                                                     const float* __restrict__ k_scale, uint8_t* __restrict__ kb8,
                                                     float* __restrict__ kb_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = blockIdx.x * 4LL + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (blk >= nb_max) return;
  int64_t nk = n_keys[b];
  if (nk > n_max) nk = n_max;
  const int64_t j0 = blk * block;
  const int64_t j1 = (j0 + block < nk) ? j0 + block : nk;
  const int64_t orow = (int64_t)b * nb_max + blk;
  if (j1 <= j0) {
    for (int c = lane; c < dk; c += 64) kb8[orow * dk + c] = 0;
    if (lane == 0) kb_scale[orow] = 0.0f;
    return;
  }
  float mean[CSA2_MAX_DK_DEV / 64];
  float amax = 0.0f;
  for (int ci = 0; ci * 64 < dk; ++ci) {
    const int c = ci * 64 + lane;
    float sum = 0.0f;
    if (c < dk) {
      for (int64_t j = j0; j < j1; ++j) {
        const int64_t row = (int64_t)b * n_max + j;
        const float v = k_scale[row] * e4m3_value(k8[row * dk + c]);
        sum = sum + v;
      }
    }
    mean[ci] = sum / (float)(j1 - j0);
    if (c < dk) amax = fmaxf(amax, fabsf(mean[ci]));
  }
  amax = wave_max(amax);
  const float s = amax / 448.0f;
  for (int ci = 0; ci * 64 < dk; ++ci) {
    const int c = ci * 64 + lane;
    if (c < dk) kb8[orow * dk + c] = (uint8_t)(s != 0.0f ? e4m3_encode(mean[ci] / s) : 0u);
  }
  if (lane == 0) kb_scale[orow] = s;
}

int launch_gather_dequant(bool g16, int B, int T, int K, int D, const uint8_t* codes, const void* scales,
                          int64_t n_max, const int32_t* idx, float* out, hipStream_t st) {
  const int64_t total = (int64_t)B * T * K * (D / 8);
  if (total == 0) return 0;
  const dim3 g((unsigned)((total + 255) / 256));
  if (g16)
    hipLaunchKernelGGL(k_gather_dequant<true>, g, dim3(256), 0, st, T, K, D, codes, scales, n_max, idx, out, total);
  else
    hipLaunchKernelGGL(k_gather_dequant<false>, g, dim3(256), 0, st, T, K, D, codes, scales, n_max, idx, out, total);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ void k_causal_limits(int R, int T, const int32_t* __restrict__ n_keys, int32_t* __restrict__ q_limit) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < R) q_limit[r] = n_keys[r / T] - T + r % T;
}

int launch_causal_limits(int B, int T, const int32_t* n_keys, int32_t* q_limit, hipStream_t st) {
  const int R = B * T;
  hipLaunchKernelGGL(k_causal_limits, dim3((R + 255) / 256), dim3(256), 0, st, R, T, n_keys, q_limit);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_coarse_keys(int B, int64_t n_max, const int32_t* n_keys, int dk, int block, const uint8_t* k8,
                       const float* k_scale, uint8_t* kb8, float* kb_scale, hipStream_t st) {
  const int64_t nb = (n_max + block - 1) / block;
  hipLaunchKernelGGL(k_coarse_keys, dim3((unsigned)((nb + 3) / 4), B), dim3(256), 0, st, n_max, n_keys, dk, block, nb,
                     k8, k_scale, kb8, kb_scale);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Read-stream ceiling probe: the grid sweeps `n16` 16-byte chunks with nontemporal loads,
// eight in flight per lane, and folds them into one word per thread.  The word is stored
// only when it equals a value the caller's data never produces, so the kernel's memory
// traffic is the read alone.
__global__ __launch_bounds__(256) void k_stream_read(const v4i_t* __restrict__ p, int64_t n16, uint32_t never,
                                                     uint32_t* __restrict__ sink) {
  constexpr int U = 8;  // 16-byte loads in flight per lane
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = blockIdx.x * 256LL + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4i_t a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= (uint32_t)(a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3]);
  }
  for (; i < n16; i += stride) {
    const v4i_t a = __builtin_nontemporal_load(p + i);
    acc ^= (uint32_t)(a[0] ^ a[1] ^ a[2] ^ a[3]);
  }
  if (acc == never) sink[0] = acc;
}

int launch_stream_read(const void* p, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(256), 0, st, static_cast<const v4i_t*>(p), bytes / 16,
                     0x9E3779B9u, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
