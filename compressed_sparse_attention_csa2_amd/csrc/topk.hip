// Top-K selection.  "Compressed Sparse Attention 2 Or CSA2 In Simple Terms" (paper notes):
// the indexer keeps the 512 highest-scoring entries.  Order: higher score first, ties to
// the lower position (a strict total order, so the selected set is unique); the result is
// written in ascending position order, -1 padded.
//
// Distributed radix select over three launches, no fence or grid-wide wait inside a
// kernel (on MI355X an agent-scope release writes back the XCD's whole L2, which made
// in-kernel hand-offs between blocks cost tens of microseconds, and blocks polling a
// counter with device-scope loads slowed the score blocks still streaming up to 4x):
//   1. the score kernel (or k_topk_hist) adds every visible score's top 11 key bits to a
//      per-row histogram (LDS histogram per block, then one atomic per non-empty bin);
//   2. k_topk_filter: every block derives from the complete histogram the bin holding the
//      K-th largest score and writes the (key, position) pairs of its column chunk in
//      that bin or above to its own region of the row's candidate list, plus their count
//      (no cross-block reservation, so no atomic round trip on the critical path); scores
//      in the threshold bin also feed a second-level histogram of the next 11 key bits;
//   3. finalize_row (topk_dev.hpp) selects the exact K among the candidates - in
//      k_topk_finalize, or inside the attention kernel of an indexing layer.
// Candidates per row are typically ~1K for K = 512 of 131072 N(0,1)-like scores; all-equal
// scores degrade to every visible column (correct, slower).
#include "common.hpp"
#include "launch.hpp"
#include "select_dev.hpp"
#include "topk_dev.hpp"

namespace csa2 {

constexpr int kFiltThreads = 256;
constexpr int kHistColsPerBlock = 2048;
constexpr int kFinThreads = 1024;

// inclusive suffix sum over the 256 threads of a block: sum of v over threads >= tid
__device__ __forceinline__ uint32_t block_suffix_sum(uint32_t v, uint32_t* sh4) {
  return block_suffix<kFiltThreads, kFiltThreads>(v, sh4);
}

template <bool CAND>
__global__ __launch_bounds__(256) void k_topk_hist(int64_t ncols, const float* __restrict__ scores,
                                                   const int32_t* __restrict__ cand, uint32_t* __restrict__ hist) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kHistColsPerBlock;
  for (int64_t c = c0 + threadIdx.x; c < c0 + kHistColsPerBlock && c < ncols; c += 256) {
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

// The threshold bin of a row from its first-level histogram: beta, the visible scores
// above it, keff = min(K, visible).  Block-wide (256 threads, thread t owns bins 8t..8t+7);
// result in s_misc[0] (visible total), [1] (beta; kHistBins if nothing is visible),
// [4] (above).
// The same from this thread's bins hb = hrow[8 tid .. 8 tid + 7], already loaded.
__device__ __forceinline__ void row_threshold_of(const uint32_t (&hb)[8], int K, uint32_t* sh4, uint32_t* s_misc) {
  const int tid = threadIdx.x;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) local += hb[i];
  const uint32_t suf = block_suffix_sum(local, sh4);  // visible scores in bins >= 8*tid
  if (tid == 0) {
    s_misc[0] = suf;
    s_misc[1] = kHistBins;
    s_misc[4] = 0;
  }
  __syncthreads();
  const uint32_t total = s_misc[0];
  const uint32_t keff = total < (uint32_t)K ? total : (uint32_t)K;
  if (keff > 0 && suf >= keff && suf - local < keff) {
    uint32_t acc = suf - local;
    for (int i = 7; i >= 0; --i) {
      if (acc + hb[i] >= keff) {
        s_misc[1] = tid * 8 + i;
        s_misc[4] = acc;  // visible scores in bins above beta
        break;
      }
      acc += hb[i];
    }
  }
  __syncthreads();
}

// 16-byte loads of this thread's 8 bins (a row's histogram is 8 KB, 16-byte aligned)
__device__ __forceinline__ void load_bins(const uint32_t* __restrict__ hrow, uint32_t (&hb)[8]) {
  const uint4 a = reinterpret_cast<const uint4*>(hrow)[2 * threadIdx.x];
  const uint4 b = reinterpret_cast<const uint4*>(hrow)[2 * threadIdx.x + 1];
  hb[0] = a.x; hb[1] = a.y; hb[2] = a.z; hb[3] = a.w;
  hb[4] = b.x; hb[5] = b.y; hb[6] = b.z; hb[7] = b.w;
}

__device__ __forceinline__ void row_threshold(const uint32_t* __restrict__ hrow, int K, uint32_t* sh4,
                                              uint32_t* s_misc) {
  uint32_t hb[8];
  load_bins(hrow, hb);
  row_threshold_of(hb, K, sh4, s_misc);
}

// Many rows (chunked prefill): one block per row derives the row's threshold once, so
// that the filter blocks read 16 bytes of it instead of the 8 KB histogram each.
__global__ __launch_bounds__(kFiltThreads) void k_topk_threshold(int K, const uint32_t* __restrict__ hist,
                                                                RowCtl* __restrict__ ctl) {
  __shared__ uint32_t sh4[4];
  __shared__ uint32_t s_misc[8];
  const int r = blockIdx.x;
  row_threshold(hist + (int64_t)r * kHistBins, K, sh4, s_misc);
  if (threadIdx.x == 0) {
    const uint32_t total = s_misc[0];
    ctl[r].beta = s_misc[1];
    ctl[r].above = s_misc[4];
    ctl[r].keff = total < (uint32_t)K ? total : (uint32_t)K;
  }
}

// CTL: the row's threshold was computed by k_topk_threshold (read ctl); otherwise every
// block derives it from the histogram and block 0 of the row writes ctl.
// Regions: kFilterColsPerBlock columns with CTL (many rows), kFilterColsNarrow otherwise
// (twice the blocks for the few rows of a decode step).
template <bool CAND, bool CTL>
__global__ __launch_bounds__(256) void k_topk_filter(int64_t ncols, const float* __restrict__ scores,
                                                     const int32_t* __restrict__ cand, int K,
                                                     const uint32_t* __restrict__ hist, uint32_t* __restrict__ hist2,
                                                     RowCtl* __restrict__ ctl, uint2* __restrict__ candbuf,
                                                     uint32_t* __restrict__ cnt, uint4* __restrict__ clear,
                                                     int64_t clear_n4) {
  constexpr int kWaves = kFiltThreads / 64;
  constexpr int kCols = CTL ? kFilterColsPerBlock : kFilterColsNarrow;
  constexpr int kPer = kCols / kFiltThreads;  // 16 or 8 columns per thread
  __shared__ uint32_t lhist2[kHistBins];
  __shared__ uint32_t sh4[kWaves];
  __shared__ uint32_t s_misc[8];
  __shared__ uint32_t s_off[kPer * kWaves];  // candidates before (column pass i, wave w)
  static_assert(kPer * kWaves <= 64, "one wave scans the (pass, wave) counts");
  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the next selection's histograms and control words, idle until then, are cleared here
  // (the caller's fill then clears only the first selection's)
  for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kFiltThreads + tid; i < clear_n4;
       i += (int64_t)gridDim.x * gridDim.y * kFiltThreads)
    clear[i] = make_uint4(0u, 0u, 0u, 0u);

  // the scores of this block's columns (all loads first, branch-free, clamped); pass i,
  // wave w, lane l holds column c0 + 256 i + 64 w + l, so (i, w, l) order is column order
  const int64_t c0 = (int64_t)blockIdx.x * kCols;
  const float* srow = scores + (int64_t)r * ncols;
  const int32_t* prow = CAND ? cand + (int64_t)r * ncols : nullptr;
  // the row's histogram bins first: the threshold is derived while the scores are in flight
  uint32_t hb[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if (!CTL) load_bins(hist + (int64_t)r * kHistBins, hb);
  __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the score loads (the counter retires in order)
  float sv[kPer];
  int32_t pv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t c = c0 + tid + (int64_t)i * kFiltThreads;
    const int64_t cc = c < ncols ? c : ncols - 1;
    sv[i] = srow[cc];
    pv[i] = CAND ? prow[cc] : (int32_t)cc;
    if (c >= ncols) sv[i] = kNegInf;
  }

  // threshold bin
  for (int i = tid; i < kHistBins; i += kFiltThreads) lhist2[i] = 0;
  uint32_t beta;
  if (CTL) {
    beta = ctl[r].beta;
    __syncthreads();  // lhist2 zeroed before any block thread adds to it
  } else {
    row_threshold_of(hb, K, sh4, s_misc);
    beta = s_misc[1];
    if (blockIdx.x == 0 && tid == 0) {
      const uint32_t total = s_misc[0];
      ctl[r].beta = beta;
      ctl[r].above = s_misc[4];
      ctl[r].keff = total < (uint32_t)K ? total : (uint32_t)K;
    }
  }
  const int nreg = (int)gridDim.x;
  if (beta >= (uint32_t)kHistBins) {  // nothing visible in this row (uniform per block)
    if (tid == 0) cnt[(int64_t)r * nreg + blockIdx.x] = 0;
    return;
  }

  // candidates: visible, first-level bin >= beta.  Compacted in column order (ballot
  // counts per (pass, wave), an exclusive scan over them, then each lane's rank in its
  // ballot), so that without a candidate map a row's list is sorted by position.
  uint64_t bal[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool vis = visible(sv[i]) && pv[i] >= 0;
    const uint32_t key = order_key(sv[i]);
    const uint32_t b1 = hist_bin(key);
    const bool take = vis && b1 >= beta;
    bal[i] = __ballot(take);
    if (take && b1 == beta) atomicAdd(&lhist2[hist2_bin(key)], 1u);
  }
  if (lane < kPer) {
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i == lane) n = (uint32_t)__builtin_popcountll(bal[i]);
    s_off[lane * kWaves + wave] = n;
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan over the kPer * kWaves (64 or 32) counts in (pass, wave) order
    const uint32_t v = (lane < kPer * kWaves) ? s_off[lane] : 0u;
    const uint32_t sfx = wave_suffix(v);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
    if (lane < kPer * kWaves) s_off[lane] = tot - sfx;
    if (lane == 0) s_misc[2] = tot;
  }
  __syncthreads();
  const uint32_t nloc = s_misc[2];
  if (tid == 0) cnt[(int64_t)r * nreg + blockIdx.x] = nloc;
  if (nloc == 0) return;
  uint2* creg = candbuf + ((int64_t)r * nreg + blockIdx.x) * kCols;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if ((bal[i] >> lane) & 1ull) {
      const uint32_t slot = s_off[i * kWaves + wave] + lanes_below(bal[i]);
      creg[slot] = make_uint2(order_key(sv[i]), (uint32_t)pv[i]);
    }
  }
  for (int i = tid; i < kHistBins; i += kFiltThreads) {
    const uint32_t v = lhist2[i];
    if (v) atomicAdd(&hist2[(int64_t)r * kHistBins + i], v);
  }
}

// EXPAND (two-level select, candidate pool): the selected columns are blocks of `block`
// positions; the kernel also writes the blocks' positions in order, -1 past a sequence's
// n_keys or for padding (the candidate list of the fine stage).  idx_out and val_out may be
// null.  With rps > 1 query rows per sequence, row t of a sequence stops at n_keys - (rps -
// 1 - t).
template <bool SORTED, bool EXPAND>
__global__ __launch_bounds__(kFinThreads) void k_topk_finalize(int nreg, int rstride, int K, const RowCtl* __restrict__ ctl,
                                                               const uint32_t* __restrict__ hist2,
                                                               const uint2* __restrict__ candbuf,
                                                               const uint32_t* __restrict__ cnt,
                                                               int32_t* __restrict__ idx_out,
                                                               float* __restrict__ val_out, int block,
                                                               const int32_t* __restrict__ n_keys,
                                                               int32_t* __restrict__ expand_out, int rps) {
  __shared__ FinalizeSmem sm;
  __shared__ int32_t s_pos[CSA2_MAX_K_DEV];
  __shared__ uint32_t s_key[CSA2_MAX_K_DEV];
  const int r = blockIdx.x;
  const RowCtl c = ctl[r];
  const int keff = finalize_row<kFinThreads, SORTED>(candbuf + (int64_t)r * nreg * rstride,
                                                     cnt + (int64_t)r * nreg, nreg, rstride, hist2 + (int64_t)r * kHistBins,
                                                     c.beta, c.above, c.keff, sm, s_pos, s_key);
  for (int i = threadIdx.x; i < K; i += kFinThreads) {
    const bool have = i < keff;
    if (idx_out) idx_out[(int64_t)r * K + i] = have ? s_pos[i] : -1;
    if (val_out) val_out[(int64_t)r * K + i] = have ? key_to_float(s_key[i]) : kNegInf;
  }
  if (EXPAND) {
    // rows_per_seq (rps) query rows share a sequence; row t of it sees its first
    // n_keys - (rps - 1 - t) positions (multi-token decode).  K * block fits in int32 (the
    // expansion is bounded by the Top-K column limit).
    const int64_t nk = (int64_t)n_keys[r / rps] - (rps - 1 - r % rps);
    int32_t* dst = expand_out + (int64_t)r * K * block;
    // one selected block per thread and pass: its `block` positions, four per store when
    // the block size allows
    const bool vec = block % 4 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
    for (int e = threadIdx.x; e < K; e += kFinThreads) {
      const int64_t base = (e < keff) ? (int64_t)s_pos[e] * block : -1;
      auto pos = [&](int k) -> int32_t { return (base >= 0 && base + k < nk) ? (int32_t)(base + k) : -1; };
      int32_t* d = dst + (int64_t)e * block;
      if (vec) {
        for (int k = 0; k < block; k += 4) *reinterpret_cast<int4*>(d + k) = make_int4(pos(k), pos(k + 1), pos(k + 2), pos(k + 3));
      } else {
        for (int k = 0; k < block; ++k) d[k] = pos(k);
      }
    }
  }
}

// Candidate pool of a Full layer: the largest score of every block of `block` consecutive
// positions (-inf where none is visible), plus the first-level histogram of those maxima
// for the pool's Top-K.  kBmPer blocks of positions per thread, 256 threads per workgroup;
// blocks of 8 positions (the pages' size) read each block with two 16-byte loads.
constexpr int kBmPer = 4;

template <bool B8>
__global__ __launch_bounds__(256) void k_block_max(int64_t ncols, int block, int64_t nb,
                                                   const float* __restrict__ scores, float* __restrict__ bmax,
                                                   uint32_t* __restrict__ hist) {
  __shared__ uint32_t lhist[kHistBins];
  const int r = blockIdx.y;
  for (int i = threadIdx.x; i < kHistBins; i += 256) lhist[i] = 0;
  const float* srow = scores + (int64_t)r * ncols;
  float m[kBmPer];
#pragma unroll
  for (int j = 0; j < kBmPer; ++j) {
    const int64_t k = (blockIdx.x * (int64_t)kBmPer + j) * 256 + threadIdx.x;
    m[j] = kNegInf;
    if (k >= nb) continue;
    if (B8 && k * 8 + 8 <= ncols) {
      const float4 a = *reinterpret_cast<const float4*>(srow + k * 8);
      const float4 c = *reinterpret_cast<const float4*>(srow + k * 8 + 4);
      m[j] = fmaxf(fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)), fmaxf(fmaxf(c.x, c.y), fmaxf(c.z, c.w)));
    } else {
      const int64_t n = (ncols - k * block < block) ? ncols - k * block : block;
      for (int64_t i = 0; i < n; ++i) m[j] = fmaxf(m[j], srow[k * block + i]);  // scores are never NaN
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBmPer; ++j) {
    const int64_t k = (blockIdx.x * (int64_t)kBmPer + j) * 256 + threadIdx.x;
    if (k >= nb) continue;
    bmax[(int64_t)r * nb + k] = m[j];
    if (visible(m[j])) atomicAdd(&lhist[hist_bin(order_key(m[j]))], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&hist[(int64_t)r * kHistBins + i], v);
  }
}

int launch_block_max(int R, int64_t ncols, int block, const float* scores, float* bmax, uint32_t* hist,
                     hipStream_t st) {
  const int64_t nb = (ncols + block - 1) / block;
  const dim3 g((unsigned)((nb + 256 * kBmPer - 1) / (256 * kBmPer)), R);
  // 16-byte loads need 16-byte aligned rows
  if (block == 8 && ncols % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0)
    hipLaunchKernelGGL(k_block_max<true>, g, dim3(256), 0, st, ncols, block, nb, scores, bmax, hist);
  else
    hipLaunchKernelGGL(k_block_max<false>, g, dim3(256), 0, st, ncols, block, nb, scores, bmax, hist);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_topk_hist(int R, int64_t ncols, const float* scores, const int32_t* cand, uint32_t* hist, hipStream_t st) {
  dim3 g((unsigned)((ncols + kHistColsPerBlock - 1) / kHistColsPerBlock), R);
  if (cand)
    hipLaunchKernelGGL(k_topk_hist<true>, g, dim3(256), 0, st, ncols, scores, cand, hist);
  else
    hipLaunchKernelGGL(k_topk_hist<false>, g, dim3(256), 0, st, ncols, scores, cand, hist);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One workgroup per row (select_row): idx_out [R][K] ascending (SORTED; otherwise ranked by
// position), -1 padded; val_out (nullable) their scores.  clear: as in k_topk_filter (words of
// a later selection zeroed on the side).
template <bool SORTED, int NT, int MAXREG>
__global__ __launch_bounds__(NT) void k_topk_select(SelectIn in, int32_t* __restrict__ idx_out,
                                                    float* __restrict__ val_out, uint4* __restrict__ clear,
                                                    int64_t clear_n4) {
  __shared__ SelectSmem sm;
  __shared__ int32_t s_pos[CSA2_MAX_K_DEV];
  __shared__ uint32_t s_key[CSA2_MAX_K_DEV];
  const int r = blockIdx.x, tid = threadIdx.x;
  for (int64_t i = (int64_t)r * NT + tid; i < clear_n4; i += (int64_t)gridDim.x * NT)
    clear[i] = make_uint4(0u, 0u, 0u, 0u);
  const int keff = (int)select_row<SORTED, NT, MAXREG>(in, r, sm, s_pos, s_key);
  const int K = in.K;
  for (int i = tid; i < K; i += NT) {
    const bool have = i < keff;
    if (idx_out) idx_out[(int64_t)r * K + i] = have ? s_pos[i] : -1;
    if (val_out) val_out[(int64_t)r * K + i] = have ? key_to_float(s_key[i]) : kNegInf;
  }
  if (in.expand_out) {  // the winners are blocks: write their positions (the fine candidates)
    const int blk = in.expand_block;
    const int64_t nk = in.n_keys[r / in.T];
    int32_t* dst = in.expand_out + (int64_t)r * K * blk;
    for (int64_t i = tid; i < (int64_t)K * blk; i += NT) {
      const int e = (int)(i / blk);
      const int64_t p = e < keff ? (int64_t)s_pos[e] * blk + i % blk : -1;
      dst[i] = (p >= 0 && p < nk) ? (int32_t)p : -1;
    }
  }
}

int launch_topk_select(const ScoreArgs& a, int K, bool sorted, int nreg, int32_t* idx_out, float* val_out,
                       hipStream_t st, uint32_t* clear, int64_t clear_words, int expand_block,
                       int32_t* expand_out) {
  if (nreg > kSelMaxRegions) return -1;
  if (a.prec != 1 && a.prec != 2) return -1;  // the re-score covers the fp8 and FP4 indexers
  if (a.H != 32 || a.dk != 64) return -1;
  if (clear && ((reinterpret_cast<uintptr_t>(clear) & 15) || clear_words % 4)) return -1;
  uint4* clear4 = clear ? reinterpret_cast<uint4*>(clear) : nullptr;
  const int64_t clear_n4 = clear ? clear_words / 4 : 0;
  const int R = a.B * a.T;
  const LocalCand& lc = a.lc;
  SelectIn in{};
  in.nreg = nreg;
  in.stride = lc.stride;
  in.rcols = lc.rcols;
  in.ncols = a.ncols;
  in.K = K;
  in.candbuf = lc.cand;
  in.cnt = lc.cnt;
  in.cut = lc.cut;
  in.vis = lc.vis;
  in.scores = a.scores;
  in.cand = a.cand;
  in.q = a.q;
  in.q_bf16 = a.q_bf16 ? 1 : 0;
  in.f4 = a.prec == 2 ? 1 : 0;
  in.w = a.w;
  in.k = static_cast<const uint8_t*>(a.k);
  in.ks = a.k_scale;
  in.n_max = a.n_max;
  in.n_keys = a.n_keys;
  in.q_limit = a.q_limit;
  in.key_div = a.key_div;
  in.T = a.T;
  // the lists' cap for a row whose columns are all visible (shorter rows list more per
  // region and, past spec, take the general path), rounded up to a power of two
  const int64_t cap = list_cap(a.lc.K, a.lc.rcols, a.ncols, kListMargin, a.lc.stride);
  int spec = 1;
  while (spec < cap && 2 * spec <= a.lc.stride) spec *= 2;
  in.spec = spec;
  in.expand_out = expand_out;
  in.expand_block = expand_block;
#define CSA2_SELECT(S, NT, MR) \
  hipLaunchKernelGGL((k_topk_select<S, NT, MR>), dim3(R), dim3(NT), 0, st, in, idx_out, val_out, clear4, clear_n4)
  // one region count per thread covers rows of up to kSelThreads regions (2M columns at
  // 2048 per region) and keeps the per-thread region state in few registers
  if (nreg <= kSelThreads) {
    if (sorted) CSA2_SELECT(true, kSelThreads, kSelThreads); else CSA2_SELECT(false, kSelThreads, kSelThreads);
  } else {
    if (sorted) CSA2_SELECT(true, kSelThreads, kSelMaxRegions); else CSA2_SELECT(false, kSelThreads, kSelMaxRegions);
  }
#undef CSA2_SELECT
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Rows from which the threshold is computed once per row in its own kernel rather than
// in every filter block (many rows: the histogram re-reads would cost more than a launch);
// those filter blocks also take the wider regions.
constexpr int kThresholdKernelRows = 64;

int topk_region_cols(int R) { return R >= kThresholdKernelRows ? kFilterColsPerBlock : kFilterColsNarrow; }
int topk_regions(int R, int64_t ncols) {
  const int c = topk_region_cols(R);
  return (int)((ncols + c - 1) / c);
}

int launch_topk_filter(int R, int64_t ncols, const float* scores, const int32_t* cand, int K, const uint32_t* hist,
                       uint32_t* hist2, RowCtl* ctl, uint2* candbuf, uint32_t* cnt, hipStream_t st,
                       uint32_t* clear, int64_t clear_words) {
  if (clear && ((reinterpret_cast<uintptr_t>(clear) & 15) || clear_words % 4)) return -1;
  uint4* clear4 = clear ? reinterpret_cast<uint4*>(clear) : nullptr;
  const int64_t clear_n4 = clear ? clear_words / 4 : 0;
  dim3 g((unsigned)topk_regions(R, ncols), R);
  const bool pre = R >= kThresholdKernelRows;
  if (pre) hipLaunchKernelGGL(k_topk_threshold, dim3(R), dim3(kFiltThreads), 0, st, K, hist, ctl);
#define CSA2_FILTER(C, P)                                                                                      \
  hipLaunchKernelGGL((k_topk_filter<C, P>), g, dim3(kFiltThreads), 0, st, ncols, scores, cand, K, hist, hist2, ctl, \
                     candbuf, cnt, clear4, clear_n4)
  if (cand) {
    if (pre) CSA2_FILTER(true, true); else CSA2_FILTER(true, false);
  } else {
    if (pre) CSA2_FILTER(false, true); else CSA2_FILTER(false, false);
  }
#undef CSA2_FILTER
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_topk_finalize(int R, int64_t ncols, int K, bool sorted, const RowCtl* ctl, const uint32_t* hist2,
                         const uint2* candbuf, const uint32_t* cnt, int32_t* idx_out, float* val_out, hipStream_t st,
                         int block, const int32_t* n_keys, int32_t* expand_out, int rps) {
  const int nreg = topk_regions(R, ncols);
#define CSA2_FIN(S, E)                                                                                          \
  hipLaunchKernelGGL((k_topk_finalize<S, E>), dim3(R), dim3(kFinThreads), 0, st, nreg, topk_region_cols(R), K, ctl, \
                     hist2, candbuf, cnt,                                                                        \
                     idx_out, val_out, block, n_keys, expand_out, rps)
  if (expand_out) {
    if (!sorted) return -1;  // block selections come from a list without a candidate map
    CSA2_FIN(true, true);
  } else if (sorted) {
    CSA2_FIN(true, false);
  } else {
    CSA2_FIN(false, false);
  }
#undef CSA2_FIN
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
