// Device helpers shared by the indexer score kernels and the Top-K selection's fallback,
// which re-scores the columns of a block whose candidate list cannot be trusted with exactly
// the score kernel's arithmetic (same query operand, same MFMA, same epilogue order), so
// that a re-scored column has the bit-identical score.
// "Compressed Sparse Attention 2 Or CSA2 In Simple Terms": the score is the head-weighted
// sum of per-head dot products of the low-bit query and key.
#pragma once

#include "common.hpp"

namespace csa2 {

// Visible rows of query row r: [0, lim].  n_keys counts cache rows; with key_div > 1 the
// columns are blocks of key_div rows (coarse keys) and a block is visible iff it holds at
// least one visible row.
__device__ __forceinline__ int64_t visible_limit(int b, int r, int64_t n_max, const int32_t* n_keys,
                                                 const int32_t* q_limit, int key_div) {
  int64_t nk = n_keys[b];
  if (key_div > 1) nk = (nk + key_div - 1) / key_div;
  int64_t lim = (nk < n_max ? nk : n_max) - 1;
  if (q_limit && q_limit[r] < lim) lim = q_limit[r];
  return lim;
}

// Quantise lane's half of head (lane%32) of the query row to E4M3 and return the MFMA
// A operand (byte j of the 32 = dim 32*(lane/32) + j), plus sq for that head.  SEL picks
// the branch-free encoder: short candidate scans wait on this prologue and run faster with
// it, long streaming scans hide it behind their loads and run faster without.
template <typename QT, bool SEL>
__device__ __forceinline__ v8i quantize_query_operand(const QT* __restrict__ qrow, int lane, float& sq_out) {
  // two passes over the (cache-resident) 32 values so that few registers are live while
  // the first key tiles are in flight: absmax, then encode
  const int hq = lane & 31, half = lane >> 5;
  const QT* p = qrow + hq * 64 + half * 32;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(load_as_f32(p + i)));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const float sq = amax / 448.0f;
  const ExactQuotient div(sq);
  const uint32_t keep = sq != 0.0f ? ~0u : 0u;  // an all-zero head encodes to zero bytes
  v8i a;
#pragma unroll
  for (int wd = 0; wd < 8; ++wd) {
    uint32_t word = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const float y = div(load_as_f32(p + wd * 4 + bb));
      word |= (SEL ? e4m3_encode_select(y) : e4m3_encode(y)) << (8 * bb);
    }
    a[wd] = (int)(word & keep);
  }
  sq_out = sq;
  return a;
}

// The 4-bit variant: the head's 32 values of this lane as E2M1 (sq = absmax/6), packed
// two per byte with the lower dim in the low nibble, in the first four operand dwords
// (an FP4 operand of the 32x32x64 MFMA takes 16 bytes per lane).
template <typename QT>
__device__ __forceinline__ v8i quantize_query_operand_fp4(const QT* __restrict__ qrow, int lane, float& sq_out) {
  const int hq = lane & 31, half = lane >> 5;
  const QT* p = qrow + hq * 64 + half * 32;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(load_as_f32(p + i)));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const float sq = amax / 6.0f;
  const ExactQuotient div(sq);
  const uint32_t keep = sq != 0.0f ? ~0u : 0u;
  v8i a = {};
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    uint32_t word = 0;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) word |= e2m1_encode(div(load_as_f32(p + wd * 8 + nb))) << (4 * nb);
    a[wd] = (int)(word & keep);
  }
  sq_out = sq;
  return a;
}

// One 32-key tile: the 32 x 32 x 64 MFMA of the query operand A (32 heads) and the key
// operand B (lane l: key l % 32, bytes 32 (l / 32) .. + 31 of fp8 keys, or 16 (l / 32) .. + 15
// of FP4 keys), then the head-weighted sum: 16 in-lane FMAs over this lane's heads (cvec =
// their c_h = w_h sq_h) in a fixed order, plus lane l ^ 32's 16.  Invisible keys score -inf.
// tile_mfma and tile_epilogue split it so that several tiles' MFMAs can issue back to back.
template <bool F4>
__device__ __forceinline__ v16f tile_mfma(const v8i& A, const v8i& B) {
  v16f acc = {};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, F4 ? 4 : 0, F4 ? 4 : 0, 0, 0, 0, 0);
}
__device__ __forceinline__ float tile_epilogue(const v16f& acc, const float (&cvec)[16], bool visible_key,
                                               float key_scale) {
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) part = fmaf(cvec[j], acc[j], part);
  const float total = part + __shfl_xor(part, 32);
  return visible_key ? total * key_scale : kNegInf;
}
template <bool F4>
__device__ __forceinline__ float tile_score(const v8i& A, const v8i& B, const float (&cvec)[16], bool visible_key,
                                            float key_scale) {
  return tile_epilogue(tile_mfma<F4>(A, B), cvec, visible_key, key_scale);
}

// c_h of the 16 heads whose results lane l holds in a tile's accumulator (s_c: the 32 c_h)
__device__ __forceinline__ void tile_head_factors(const float* s_c, int half, float (&cvec)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) cvec[i] = s_c[8 * (i >> 2) + 4 * half + (i & 3)];
}

}  // namespace csa2
