// Top-K selection.  "Compressed Sparse Attention 2 Or CSA2 In Simple Terms" (paper notes):
// the indexer keeps the 512 highest-scoring entries.  Order: higher score first, ties to
// the lower position (a strict total order, so the selected set is unique); the result is
// written in ascending position order, -1 padded.
//
// Distributed radix select, no grid-wide barrier:
//   1. the score kernel (or k_topk_hist) adds every visible score's top 11 key bits to a
//      per-row histogram;
//   2. every block of k_topk_select derives from the histogram the bin that holds the
//      K-th largest score, and appends the (key, position) pairs of its column chunk that
//      fall in that bin or above to a per-row candidate list (one atomic per block);
//   3. the last block of a row to finish (atomic counter after a release fence) runs an
//      exact 8-bit-digit radix select over the candidates on the 64-bit composite
//      key = (score key << 32) | ~position, then sorts the winners by position.
// Candidates per row are typically ~2K for K = 512 of 131072; all-equal scores degrade to
// every visible column (correct, slower).
#include "common.hpp"
#include "launch.hpp"

namespace csa2 {

constexpr int kSelThreads = 256;
constexpr int kSelColsPerBlock = 2048;

// inclusive suffix sum over the 256 threads of a block: sum of v over threads >= tid
__device__ __forceinline__ uint32_t block_suffix_sum(uint32_t v, uint32_t* sh4) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(x, o);
    if (lane + o < 64) x += y;
  }
  if (lane == 0) sh4[wave] = x;
  __syncthreads();
  uint32_t add = 0;
  for (int w2 = wave + 1; w2 < kSelThreads / 64; ++w2) add += sh4[w2];
  __syncthreads();
  return x + add;
}

template <bool CAND>
__global__ __launch_bounds__(256) void k_topk_hist(int64_t ncols, const float* __restrict__ scores,
                                                   const int32_t* __restrict__ cand, uint32_t* __restrict__ hist) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kSelColsPerBlock;
  for (int64_t c = c0 + threadIdx.x; c < c0 + kSelColsPerBlock && c < ncols; c += 256) {
    const float s = scores[(int64_t)r * ncols + c];
    const bool ok = visible(s) && (!CAND || cand[(int64_t)r * ncols + c] >= 0);
    if (ok) atomicAdd(&lhist[hist_bin(order_key(s))], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&hist[(int64_t)r * kHistBins + i], v);
  }
}

template <bool CAND>
__global__ __launch_bounds__(256) void k_topk_select(int64_t ncols, const float* __restrict__ scores,
                                                     const int32_t* __restrict__ cand, int K,
                                                     const uint32_t* __restrict__ hist, RowCtl* __restrict__ ctl,
                                                     uint2* __restrict__ candbuf, int32_t* __restrict__ idx_out,
                                                     float* __restrict__ val_out) {
  __shared__ uint2 stage[kSelColsPerBlock];  // candidates of this block; reused by the final sort
  __shared__ uint32_t sh4[4];
  __shared__ uint32_t s_misc[8];
  __shared__ uint32_t h256[256];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;

  // ---- 1. threshold bin from the row histogram (thread t owns bins 8t .. 8t+7)
  const uint32_t* hrow = hist + (int64_t)r * kHistBins;
  uint32_t hb[8];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hb[i] = hrow[tid * 8 + i];
    local += hb[i];
  }
  const uint32_t suf = block_suffix_sum(local, sh4);  // visible scores in bins >= 8*tid
  if (tid == 0) s_misc[0] = suf;                      // total visible
  __syncthreads();
  const uint32_t total = s_misc[0];
  const uint32_t keff = total < (uint32_t)K ? total : (uint32_t)K;
  if (tid == 0) s_misc[1] = kHistBins;  // no candidates unless set below
  __syncthreads();
  if (keff > 0 && suf >= keff && suf - local < keff) {
    // the K-th largest lies in one of this thread's bins; walk them from the top
    uint32_t acc = suf - local;
    for (int i = 7; i >= 0; --i) {
      acc += hb[i];
      if (acc >= keff) {
        s_misc[1] = tid * 8 + i;
        break;
      }
    }
  }
  if (tid == 0) s_misc[2] = 0;
  __syncthreads();
  const uint32_t beta = s_misc[1];

  // ---- 2. append this block's candidates (bin >= beta)
  const int64_t c0 = (int64_t)blockIdx.x * kSelColsPerBlock;
  if (beta < (uint32_t)kHistBins) {
    for (int64_t c = c0 + tid; c < c0 + kSelColsPerBlock && c < ncols; c += kSelThreads) {
      const float s = scores[(int64_t)r * ncols + c];
      const int32_t pos = CAND ? cand[(int64_t)r * ncols + c] : (int32_t)c;
      if (visible(s) && pos >= 0) {
        const uint32_t key = order_key(s);
        if (hist_bin(key) >= beta) {
          const uint32_t slot = atomicAdd(&s_misc[2], 1u);
          stage[slot] = make_uint2(key, (uint32_t)pos);
        }
      }
    }
  }
  __syncthreads();
  const uint32_t nloc = s_misc[2];
  if (tid == 0) s_misc[3] = nloc ? atomicAdd(&ctl[r].ncand, nloc) : 0u;
  __syncthreads();
  uint2* crow = candbuf + (int64_t)r * ncols;
  for (uint32_t i = tid; i < nloc; i += kSelThreads) crow[s_misc[3] + i] = stage[i];

  // ---- 3. the last block of the row finishes the selection
  __threadfence();
  __syncthreads();
  if (tid == 0) s_misc[4] = (atomicAdd(&ctl[r].done, 1u) == gridDim.x - 1) ? 1u : 0u;
  __syncthreads();
  if (!s_misc[4]) return;
  __threadfence();
  const uint32_t M = __hip_atomic_load(&ctl[r].ncand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // radix select of the keff-th largest composite over 8-bit digits, most significant first
  uint64_t prefix = 0, mask = 0;
  uint32_t need = keff;
  for (int shift = 56; shift >= 0 && need > 0; shift -= 8) {
    h256[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < M; i += kSelThreads) {
      const uint2 c = crow[i];
      const uint64_t comp = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      if ((comp & mask) == prefix) atomicAdd(&h256[(comp >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t mine = h256[tid];
    const uint32_t sfx = block_suffix_sum(mine, sh4);
    if (sfx >= need && sfx - mine < need) {
      s_misc[5] = tid;
      s_misc[6] = sfx - mine;  // strictly above this digit
      s_misc[7] = mine;
    }
    __syncthreads();
    const uint32_t v = s_misc[5];
    need -= s_misc[6];
    prefix |= (uint64_t)v << shift;
    mask |= (uint64_t)255u << shift;
    const bool done = (s_misc[7] == need);
    __syncthreads();
    if (done) break;
  }

  // winners: (comp & mask) >= prefix
  if (tid == 0) s_misc[2] = 0;
  __syncthreads();
  if (keff > 0) {
    for (uint32_t i = tid; i < M; i += kSelThreads) {
      const uint2 c = crow[i];
      const uint64_t comp = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      if ((comp & mask) >= prefix) {
        const uint32_t slot = atomicAdd(&s_misc[2], 1u);
        if (slot < (uint32_t)K) stage[slot] = make_uint2(c.y, c.x);  // (position, key)
      }
    }
  }
  __syncthreads();
  // bitonic sort of the winners by position (padding sorts last)
  int P = 1;
  while (P < (int)keff) P <<= 1;
  for (int i = (int)keff + tid; i < P; i += kSelThreads) stage[i] = make_uint2(0x7FFFFFFFu, 0u);
  __syncthreads();
  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kSelThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint2 x = stage[i], y = stage[ixj];
          const bool up = (i & kk) == 0;
          if (((int)x.x > (int)y.x) == up) {
            stage[i] = y;
            stage[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < K; i += kSelThreads) {
    const bool have = i < (int)keff;
    idx_out[(int64_t)r * K + i] = have ? (int32_t)stage[i].x : -1;
    if (val_out) val_out[(int64_t)r * K + i] = have ? key_to_float(stage[i].y) : kNegInf;
  }
}

int launch_topk_hist(int R, int64_t ncols, const float* scores, const int32_t* cand, uint32_t* hist, hipStream_t st) {
  dim3 g((unsigned)((ncols + kSelColsPerBlock - 1) / kSelColsPerBlock), R);
  if (cand)
    hipLaunchKernelGGL(k_topk_hist<true>, g, dim3(256), 0, st, ncols, scores, cand, hist);
  else
    hipLaunchKernelGGL(k_topk_hist<false>, g, dim3(256), 0, st, ncols, scores, cand, hist);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_topk_select(int R, int64_t ncols, const float* scores, const int32_t* cand, int K, const uint32_t* hist,
                       RowCtl* ctl, uint2* candbuf, int32_t* idx_out, float* val_out, hipStream_t st) {
  dim3 g((unsigned)((ncols + kSelColsPerBlock - 1) / kSelColsPerBlock), R);
  if (cand)
    hipLaunchKernelGGL(k_topk_select<true>, g, dim3(kSelThreads), 0, st, ncols, scores, cand, K, hist, ctl, candbuf,
                       idx_out, val_out);
  else
    hipLaunchKernelGGL(k_topk_select<false>, g, dim3(kSelThreads), 0, st, ncols, scores, cand, K, hist, ctl,
                       candbuf, idx_out, val_out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
