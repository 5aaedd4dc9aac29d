// Indexer scoring.  "Compressed Sparse Attention 2 Or CSA2 In Simple Terms" (paper notes):
// each layer's indexer (32 query heads, "Model Setup Numbers Without Jargon") scores every
// visible past entry; the score is the head-weighted sum of per-head dot products.
//
// fp8 path (decode): per 32-key tile one v_mfma_f32_32x32x64_f8f6f4 computes all
// 32 heads x 32 keys x 64 dims (A = the E4M3-quantised query, kept in registers for the
// whole kernel; B = 32 keys streamed from HBM).  Lane l of the result holds key l%32 and
// 16 of the 32 heads, so the head-weighted sum is 16 in-lane FMAs plus one exchange
// with lane l^32.  The kernel is HBM-bound (68 B per key against 8 kFLOP of fp8 MFMA);
// each wave keeps 8 KB of key loads in flight.  Optionally it also builds a per-row
// histogram of the scores' top bits for the Top-K select that follows.
#include "common.hpp"
#include "launch.hpp"

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

// ---------------------------------------------------------------------------- fp32 path
// One thread per column; the query row is staged in LDS.  score = sum_h w_h (q_h . k_j),
// accumulated in a fixed order with fmaf.
template <bool CAND>
__global__ __launch_bounds__(256) void k_score_f32(int T, int H, int dk, int64_t ncols, const float* __restrict__ q,
                                                   const float* __restrict__ w, const float* __restrict__ k,
                                                   int64_t n_max, const int32_t* __restrict__ n_keys,
                                                   const int32_t* __restrict__ q_limit,
                                                   const int32_t* __restrict__ cand, float* __restrict__ scores,
                                                   uint32_t* __restrict__ hist, int key_div) {
  extern __shared__ float smem[];
  float* qs = smem;                 // [H][dk]
  float* ws = smem + H * dk;        // [H]
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y, b = r / T;
  for (int i = threadIdx.x; i < H * dk; i += 256) qs[i] = q[(int64_t)r * H * dk + i];
  for (int i = threadIdx.x; i < H; i += 256) ws[i] = w[(int64_t)r * H + i];
  if (hist)
    for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  __syncthreads();
  const int64_t lim = visible_limit(b, r, n_max, n_keys, q_limit, key_div);
  const int64_t col = blockIdx.x * 256LL + threadIdx.x;
  if (col < ncols) {
    const int64_t row = CAND ? (int64_t)cand[r * ncols + col] : col;
    float s = kNegInf;
    if (row >= 0 && row <= lim) {
      const float* kr = k + ((int64_t)b * n_max + row) * dk;
      float total = 0.0f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.0f;
        for (int d = 0; d < dk; ++d) dot = fmaf(qs[h * dk + d], kr[d], dot);
        total = fmaf(ws[h], dot, total);
      }
      s = total;
    }
    scores[r * ncols + col] = s;
    if (hist && visible(s)) atomicAdd(&lhist[hist_bin(order_key(s))], 1u);
  }
  if (hist) {
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&hist[(int64_t)r * kHistBins + i], v);
    }
  }
}

// ---------------------------------------------------------------------------- fp8 path
constexpr int kScoreWaves = 4;
constexpr int kTilesPerStep = 4;  // 32-key tiles per wave per step (8 x 16 B loads in flight per lane)

// Quantise lane's half of head (lane%32) of the query row to E4M3 and return the MFMA
// A operand (byte j of the 32 = dim 32*(lane/32) + j), plus sq for that head.
template <typename QT>
__device__ __forceinline__ v8i quantize_query_operand(const QT* __restrict__ qrow, int lane, float& sq_out) {
  const int hq = lane & 31, half = lane >> 5;
  const QT* p = qrow + hq * 64 + half * 32;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = load_as_f32(p + i);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  const float sq = amax / 448.0f;
  v8i a;
#pragma unroll
  for (int wd = 0; wd < 8; ++wd) {
    uint32_t word = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const uint32_t code = (sq != 0.0f) ? e4m3_encode(v[wd * 4 + bb] / sq) : 0u;
      word |= code << (8 * bb);
    }
    a[wd] = (int)word;
  }
  sq_out = sq;
  return a;
}

template <typename QT, bool CAND>
__global__ __launch_bounds__(256) void k_score_fp8(int T, int64_t ncols, int cols_per_block,
                                                   const QT* __restrict__ q, const float* __restrict__ w,
                                                   const uint8_t* __restrict__ k8, const float* __restrict__ ks,
                                                   int64_t n_max, const int32_t* __restrict__ n_keys,
                                                   const int32_t* __restrict__ q_limit,
                                                   const int32_t* __restrict__ cand, float* __restrict__ scores,
                                                   uint32_t* __restrict__ hist, int key_div) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y, b = r / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  if (hist)
    for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;

  float sq;
  const v8i A = quantize_query_operand(q + (int64_t)r * 32 * 64, lane, sq);
  const float c_own = w[(int64_t)r * 32 + (lane & 31)] * sq;
  float cvec[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) cvec[i] = __shfl(c_own, 8 * (i >> 2) + 4 * half + (i & 3));
  const int64_t lim = visible_limit(b, r, n_max, n_keys, q_limit, key_div);
  if (hist) __syncthreads();

  const int64_t c0 = (int64_t)blockIdx.x * cols_per_block;
  const int64_t c1 = (c0 + cols_per_block < ncols) ? c0 + cols_per_block : ncols;
  const int ntiles = (int)((c1 - c0 + 31) / 32);
  const uint8_t* kb = k8 + (int64_t)b * n_max * 64 + half * 32;
  const float* ksb = ks + (int64_t)b * n_max;
  float* srow = scores + (int64_t)r * ncols;

  for (int t0 = wave; t0 < ntiles; t0 += kScoreWaves * kTilesPerStep) {
    uint4 ka[kTilesPerStep], kc[kTilesPerStep];
    float skv[kTilesPerStep];
    bool vis[kTilesPerStep];
    int64_t col[kTilesPerStep];
#pragma unroll
    for (int u = 0; u < kTilesPerStep; ++u) {
      const int tt = t0 + u * kScoreWaves;
      col[u] = c0 + (int64_t)tt * 32 + (lane & 31);
      const bool in = tt < ntiles && col[u] < c1;
      int64_t row = -1;
      if (in) row = CAND ? (int64_t)cand[(int64_t)r * ncols + col[u]] : col[u];
      vis[u] = in && row >= 0 && row <= lim;
      if (vis[u]) {
        const uint4* src = reinterpret_cast<const uint4*>(kb + row * 64);
        ka[u] = src[0];
        kc[u] = src[1];
        skv[u] = ksb[row];
      } else {
        ka[u] = make_uint4(0, 0, 0, 0);
        kc[u] = make_uint4(0, 0, 0, 0);
        skv[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kTilesPerStep; ++u) {
      const int tt = t0 + u * kScoreWaves;
      if (tt >= ntiles) break;
      v8i B;
      B[0] = (int)ka[u].x; B[1] = (int)ka[u].y; B[2] = (int)ka[u].z; B[3] = (int)ka[u].w;
      B[4] = (int)kc[u].x; B[5] = (int)kc[u].y; B[6] = (int)kc[u].z; B[7] = (int)kc[u].w;
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 0, 0, 0, 0, 0, 0);
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) part = fmaf(cvec[i], acc[i], part);
      const float total = part + __shfl_xor(part, 32);
      const float s = vis[u] ? total * skv[u] : kNegInf;
      if (half == 0 && col[u] < c1) {
        srow[col[u]] = s;
        if (hist && visible(s)) atomicAdd(&lhist[hist_bin(order_key(s))], 1u);
      }
    }
  }
  if (hist) {
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&hist[(int64_t)r * kHistBins + i], v);
    }
  }
}

int score_cols_per_block(int64_t ncols) {
  // enough blocks per row to fill the chip at decode batch sizes, >= 4 tiles per wave
  if (ncols >= 65536) return 2048;
  if (ncols >= 8192) return 1024;
  return 512;
}

int launch_score(const ScoreArgs& a, hipStream_t st) {
  const int R = a.B * a.T;
  if (a.prec == 0) {
    dim3 g((unsigned)((a.ncols + 255) / 256), R);
    const size_t sh = sizeof(float) * ((size_t)a.H * a.dk + a.H);
    if (a.cand)
      hipLaunchKernelGGL(k_score_f32<true>, g, dim3(256), sh, st, a.T, a.H, a.dk, a.ncols, (const float*)a.q, a.w,
                         (const float*)a.k, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist, a.key_div);
    else
      hipLaunchKernelGGL(k_score_f32<false>, g, dim3(256), sh, st, a.T, a.H, a.dk, a.ncols, (const float*)a.q, a.w,
                         (const float*)a.k, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist, a.key_div);
  } else {
    const int cpb = score_cols_per_block(a.ncols);
    dim3 g((unsigned)((a.ncols + cpb - 1) / cpb), R);
#define CSA2_SCORE_LAUNCH(QT, CAND)                                                                              \
  hipLaunchKernelGGL((k_score_fp8<QT, CAND>), g, dim3(256), 0, st, a.T, a.ncols, cpb, (const QT*)a.q, a.w,      \
                     (const uint8_t*)a.k, a.k_scale, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist,    \
                     a.key_div)
    if (a.q_bf16) {
      if (a.cand) CSA2_SCORE_LAUNCH(uint16_t, true); else CSA2_SCORE_LAUNCH(uint16_t, false);
    } else {
      if (a.cand) CSA2_SCORE_LAUNCH(float, true); else CSA2_SCORE_LAUNCH(float, false);
    }
#undef CSA2_SCORE_LAUNCH
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
