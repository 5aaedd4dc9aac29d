// Sparse softmax attention over the selected FP4 entries (gather + dequant + attention).
// "Compressed Sparse Attention 2 Or CSA2 In Simple Terms": only the selected entries are
// attended; "FP4 Main KV Cache To Halve Storage Again": entries are dequantised back
// before attention; "Model Setup Numbers Without Jargon": 64 heads of dim 512.  The whole
// dequantised entry is both key and value.
//
// MFMA path (bf16 queries, Hq % 16 == 0, D % 128 == 0).  One block = 16 heads x up to
// 128 selected entries (4 waves x 32).  The per-channel scale s_c factors out of both
// contractions: logits use q' = q * s (fp32, split into bf16 hi + lo so that q' keeps
// ~16 significant bits) against the exact E2M1 values e (bf16); the output is
// s_c * sum_j p_j e_jc, with p in fp16 and e exact in fp16.  Each FP4 row is read
// straight from HBM into MFMA operand layout (no LDS staging): for QK lane (entry n,
// group g) takes 16 contiguous bytes per 128 channels; for PV lane (channel block n,
// entry group g) takes one 32-bit word (8 channels) of each of 8 entries, so the 8
// MFMAs of a k-step cover 8 interleaved channel sets.  Entries are split over blocks
// (split-K); the last block of a (row, head group) to finish merges the partial results
// by log-sum-exp.
//
// fp32 path (fp32 queries): plain VALU, one block per (row, head), fp32 throughout.
#include "common.hpp"
#include "launch.hpp"

namespace csa2 {

constexpr int kAttHeads = 16;    // heads per block (MFMA M)
constexpr int kAttEntries = 128; // entries per block (4 waves x 32)

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xFFFFu) | (hi16 << 16); }

// E2M1 pair in byte BS of `word` -> two fp16 / bf16 values (exact; scale 1).
template <int BS>
__device__ __forceinline__ uint32_t cvt_pair_f16(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, BS));
}
template <int BS>
__device__ __forceinline__ uint32_t cvt_pair_bf16(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, BS));
}

// 8 E2M1 codes of one 32-bit word -> 8 bf16 values (exact), in nibble order.
__device__ __forceinline__ v8bf decode8_bf16(uint32_t word) {
  const uint4 u = make_uint4(cvt_pair_bf16<0>(word), cvt_pair_bf16<1>(word), cvt_pair_bf16<2>(word),
                             cvt_pair_bf16<3>(word));
  return __builtin_bit_cast(v8bf, u);
}

template <int D>
__global__ __launch_bounds__(256) void k_attend_mfma(int T, int Hq, int K, int splits, const uint16_t* __restrict__ q,
                                                     const uint8_t* __restrict__ codes,
                                                     const float* __restrict__ scales, int64_t n_max,
                                                     const int32_t* __restrict__ idx, float softmax_scale,
                                                     void* __restrict__ out, int out_bf16, float* __restrict__ lse,
                                                     float* __restrict__ part_o, float* __restrict__ part_ml,
                                                     uint32_t* __restrict__ counters) {
  constexpr int kRowBytes = D / 2;
  constexpr int kChunks = D / 128;
  constexpr int kApad = D + 8;         // bf16 elements per A row (pad against bank conflicts)
  constexpr int kPpad = kAttEntries + 8;
  __shared__ float s_scale[D];
  __shared__ uint16_t s_ahi[kAttHeads * kApad];
  __shared__ uint16_t s_alo[kAttHeads * kApad];
  __shared__ uint16_t s_p[kAttHeads * kPpad];
  __shared__ int32_t s_idx[kAttEntries];
  __shared__ float s_red[4][kAttHeads];
  __shared__ float s_m[kAttHeads], s_l[kAttHeads];
  __shared__ uint32_t s_last;

  const int split = blockIdx.x, hg = blockIdx.y, r = blockIdx.z;
  const int b = r / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int per_split = (K + splits - 1) / splits;
  const int e0 = split * per_split;
  const int ecount = max(0, min(per_split, K - e0));

  // ---- phase 0: scales, indices, q' = q * s split into bf16 hi + lo
  for (int i = tid; i < D; i += 256) s_scale[i] = scales[(int64_t)b * D + i];
  for (int i = tid; i < kAttEntries; i += 256) {
    int32_t j = (i < ecount) ? idx[(int64_t)r * K + e0 + i] : -1;
    s_idx[i] = (j >= 0 && j < n_max) ? j : -1;
  }
  __syncthreads();
  const uint16_t* qb = q + ((int64_t)r * Hq + hg * kAttHeads) * D;
  for (int i = tid; i < kAttHeads * D / 8; i += 256) {
    const int h = i / (D / 8), c = (i % (D / 8)) * 8;
    const uint4 raw = *reinterpret_cast<const uint4*>(qb + (int64_t)h * D + c);
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      uint32_t hh[2], ll[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float qv = bf16_to_f32((uint16_t)(wds[k2] >> (16 * e)));
        const float qs = qv * s_scale[c + 2 * k2 + e];
        const uint16_t h16 = bf16_rne(qs);
        hh[e] = h16;
        ll[e] = bf16_rne(qs - bf16_to_f32(h16));
      }
      hi[k2] = pack2(hh[0], hh[1]);
      lo[k2] = pack2(ll[0], ll[1]);
    }
    *reinterpret_cast<uint4*>(&s_ahi[h * kApad + c]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(&s_alo[h * kApad + c]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  __syncthreads();

  // ---- phase 1: logits for this wave's 32 entries (two 16-entry tiles)
  float logit[2][4];
  const uint8_t* cb = codes + (int64_t)b * n_max * kRowBytes;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int el = wave * 32 + nt * 16 + n16;
    const int32_t j = s_idx[el];
    uint4 kw[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      kw[i] = (j >= 0) ? *reinterpret_cast<const uint4*>(cb + (int64_t)j * kRowBytes + 64 * i + 16 * g)
                       : make_uint4(0, 0, 0, 0);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t wd[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const v8bf bv = decode8_bf16(wd[sub]);
        const int c = 128 * i + 32 * g + 8 * sub;
        const v8bf ah = *reinterpret_cast<const v8bf*>(&s_ahi[n16 * kApad + c]);
        const v8bf al = *reinterpret_cast<const v8bf*>(&s_alo[n16 * kApad + c]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) logit[nt][rr] = (j >= 0) ? acc[rr] * softmax_scale : kNegInf;
  }

  // ---- phase 2: softmax statistics over the block's entries (heads 4g + rr of this lane)
  float mx[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float v = fmaxf(logit[0][rr], logit[1][rr]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    mx[rr] = v;
  }
  if (n16 == 0)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) s_red[wave][4 * g + rr] = mx[rr];
  __syncthreads();
  if (tid < kAttHeads) s_m[tid] = fmaxf(fmaxf(s_red[0][tid], s_red[1][tid]), fmaxf(s_red[2][tid], s_red[3][tid]));
  __syncthreads();
  float psum[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int h = 4 * g + rr;
    const float m = s_m[h];
    float v = 0.0f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float p = (m == kNegInf) ? 0.0f : __expf(logit[nt][rr] - m);
      const _Float16 ph = (_Float16)p;
      s_p[h * kPpad + wave * 32 + nt * 16 + n16] = __builtin_bit_cast(uint16_t, ph);
      v += p;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    psum[rr] = v;
  }
  __syncthreads();
  if (n16 == 0)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) s_red[wave][4 * g + rr] = psum[rr];
  __syncthreads();
  if (tid < kAttHeads) s_l[tid] = (s_red[0][tid] + s_red[1][tid]) + (s_red[2][tid] + s_red[3][tid]);
  __syncthreads();

  // ---- phase 3: o[h][c] = sum_j p[h][j] e[j][c]; wave w covers channel tiles w, w+4, ...
  const bool single = (splits == 1);
  for (int ct = wave; ct < kChunks; ct += 4) {
    v4f acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kAttEntries / 32; ++ks) {
      const v8h pa = *reinterpret_cast<const v8h*>(&s_p[n16 * kPpad + 32 * ks + 8 * g]);
      uint32_t wd[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int32_t j = s_idx[32 * ks + 8 * g + jj];
        wd[jj] = (j >= 0) ? *reinterpret_cast<const uint32_t*>(cb + (int64_t)j * kRowBytes + 64 * ct + 4 * n16) : 0u;
      }
      // cv[jj][bsel] = channels (2 bsel, 2 bsel + 1) of entry jj as two fp16
      uint32_t cv[8][4];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        cv[jj][0] = cvt_pair_f16<0>(wd[jj]);
        cv[jj][1] = cvt_pair_f16<1>(wd[jj]);
        cv[jj][2] = cvt_pair_f16<2>(wd[jj]);
        cv[jj][3] = cvt_pair_f16<3>(wd[jj]);
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int bs = m >> 1, hi = m & 1;
        uint32_t bw[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const uint32_t x0 = hi ? (cv[2 * q2][bs] >> 16) : cv[2 * q2][bs];
          const uint32_t x1 = hi ? (cv[2 * q2 + 1][bs] >> 16) : cv[2 * q2 + 1][bs];
          bw[q2] = pack2(x0, x1);
        }
        const v8h bv = __builtin_bit_cast(v8h, make_uint4(bw[0], bw[1], bw[2], bw[3]));
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bv, acc[m], 0, 0, 0);
      }
    }
    // lane holds heads 4g + rr, channel 128 ct + 8 n16 + m
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = 4 * g + rr;
      const float l = s_l[h];
      const float inv = (l > 0.0f) ? 1.0f / l : 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int c = 128 * ct + 8 * n16 + m;
        const float o = acc[m][rr] * inv * s_scale[c];
        const int64_t oh = (int64_t)r * Hq + hg * kAttHeads + h;
        if (single) {
          if (out_bf16)
            reinterpret_cast<uint16_t*>(out)[oh * D + c] = bf16_rne(o);
          else
            reinterpret_cast<float*>(out)[oh * D + c] = o;
        } else {
          part_o[(((int64_t)r * splits + split) * Hq + hg * kAttHeads + h) * D + c] = o;
        }
      }
    }
  }
  if (single) {
    if (lse && tid < kAttHeads) {
      const float l = s_l[tid];
      lse[(int64_t)r * Hq + hg * kAttHeads + tid] = (l > 0.0f) ? s_m[tid] + __logf(l) : kNegInf;
    }
    return;
  }
  if (tid < kAttHeads) {
    float* ml = part_ml + (((int64_t)r * splits + split) * Hq + hg * kAttHeads + tid) * 2;
    ml[0] = s_m[tid];
    ml[1] = s_l[tid];
  }

  // ---- phase 4: the last split block of (r, hg) merges all splits by log-sum-exp
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&counters[(int64_t)r * (Hq / kAttHeads) + hg], 1u) == (uint32_t)splits - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid < kAttHeads) {
    const int h = tid;
    float M = kNegInf;
    for (int s = 0; s < splits; ++s) {
      const float* ml = part_ml + (((int64_t)r * splits + s) * Hq + hg * kAttHeads + h) * 2;
      if (ml[1] > 0.0f) M = fmaxf(M, ml[0]);
    }
    float Z = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const float* ml = part_ml + (((int64_t)r * splits + s) * Hq + hg * kAttHeads + h) * 2;
      if (ml[1] > 0.0f) Z += ml[1] * __expf(ml[0] - M);
    }
    s_m[h] = M;
    s_l[h] = Z;
    if (lse) lse[(int64_t)r * Hq + hg * kAttHeads + h] = (Z > 0.0f) ? M + __logf(Z) : kNegInf;
  }
  __syncthreads();
  for (int i = tid; i < kAttHeads * D; i += 256) {
    const int h = i / D, c = i % D;
    const float M = s_m[h], Z = s_l[h];
    float o = 0.0f;
    if (Z > 0.0f) {
      for (int s = 0; s < splits; ++s) {
        const int64_t base = ((int64_t)r * splits + s) * Hq + hg * kAttHeads + h;
        const float* ml = part_ml + base * 2;
        if (ml[1] > 0.0f) o = fmaf(ml[1] * __expf(ml[0] - M) / Z, part_o[base * D + c], o);
      }
    }
    const int64_t oh = (int64_t)r * Hq + hg * kAttHeads + h;
    if (out_bf16)
      reinterpret_cast<uint16_t*>(out)[oh * D + c] = bf16_rne(o);
    else
      reinterpret_cast<float*>(out)[oh * D + c] = o;
  }
}

// fp32 path: one block per (row, head)
__global__ __launch_bounds__(256) void k_attend_f32(int T, int Hq, int D, int K, const float* __restrict__ q,
                                                    const uint8_t* __restrict__ codes,
                                                    const float* __restrict__ scales, int64_t n_max,
                                                    const int32_t* __restrict__ idx, float softmax_scale,
                                                    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float s_q[CSA2_MAX_D_DEV];
  __shared__ float s_scale[CSA2_MAX_D_DEV];
  __shared__ float s_logit[CSA2_MAX_K_DEV];
  __shared__ int32_t s_idx[CSA2_MAX_K_DEV];
  __shared__ float s_red[8];
  const int h = blockIdx.x, r = blockIdx.y, b = r / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* qh = q + ((int64_t)r * Hq + h) * D;
  for (int c = tid; c < D; c += 256) {
    s_q[c] = qh[c];
    s_scale[c] = scales[(int64_t)b * D + c];
  }
  for (int e = tid; e < K; e += 256) {
    const int32_t j = idx[(int64_t)r * K + e];
    s_idx[e] = (j >= 0 && j < n_max) ? j : -1;
  }
  __syncthreads();
  const int rowb = D / 2;
  const uint8_t* cb = codes + (int64_t)b * n_max * rowb;
  for (int e = wave; e < K; e += 4) {
    const int32_t j = s_idx[e];
    float dot = 0.0f;
    if (j >= 0) {
      for (int c = lane; c < D; c += 64) {
        const uint32_t byte = cb[(int64_t)j * rowb + c / 2];
        const float v = e2m1_value((c & 1) ? (byte >> 4) : (byte & 15u)) * s_scale[c];
        dot = fmaf(s_q[c], v, dot);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) s_logit[e] = (j >= 0) ? dot * softmax_scale : kNegInf;
  }
  __syncthreads();
  float m = kNegInf;
  for (int e = tid; e < K; e += 256) m = fmaxf(m, s_logit[e]);
  m = wave_max(m);
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float z = 0.0f;
  for (int e = tid; e < K; e += 256) {
    const float p = (m == kNegInf) ? 0.0f : expf(s_logit[e] - m);
    s_logit[e] = p;
    z += p;
  }
  z = wave_sum(z);
  if (lane == 0) s_red[4 + wave] = z;
  __syncthreads();
  z = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);
  const float inv = (z > 0.0f) ? 1.0f / z : 0.0f;
  for (int c = tid; c < D; c += 256) {
    float o = 0.0f;
    for (int e = 0; e < K; ++e) {
      const int32_t j = s_idx[e];
      if (j < 0) continue;
      const uint32_t byte = cb[(int64_t)j * rowb + c / 2];
      const float v = e2m1_value((c & 1) ? (byte >> 4) : (byte & 15u)) * s_scale[c];
      o = fmaf(s_logit[e], v, o);
    }
    out[((int64_t)r * Hq + h) * D + c] = o * inv;
  }
  if (lse && tid == 0) lse[(int64_t)r * Hq + h] = (z > 0.0f) ? m + logf(z) : kNegInf;
}

int attend_entries_per_split() { return kAttEntries; }

int launch_attend(const AttendArgs& a, hipStream_t st) {
  const int R = a.B * a.T;
  if (!a.q_bf16) {
    hipLaunchKernelGGL(k_attend_f32, dim3(a.Hq, R), dim3(256), 0, st, a.T, a.Hq, a.D, a.K, (const float*)a.q,
                       a.codes, a.scales, a.n_max, a.idx, a.softmax_scale, (float*)a.out, a.lse);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (a.splits > 1 && launch_fill_u32(a.counters, (int64_t)R * (a.Hq / kAttHeads), 0u, st)) return -1;
  dim3 g(a.splits, a.Hq / kAttHeads, R);
#define CSA2_ATT(DD)                                                                                               \
  hipLaunchKernelGGL(k_attend_mfma<DD>, g, dim3(256), 0, st, a.T, a.Hq, a.K, a.splits, (const uint16_t*)a.q,     \
                     a.codes, a.scales, a.n_max, a.idx, a.softmax_scale, a.out, (int)a.out_bf16, a.lse, a.part_o, \
                     a.part_ml, a.counters)
  switch (a.D) {
    case 128: CSA2_ATT(128); break;
    case 256: CSA2_ATT(256); break;
    case 384: CSA2_ATT(384); break;
    case 512: CSA2_ATT(512); break;
    default: return -1;
  }
#undef CSA2_ATT
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
