// Exact Top-K finalisation of one query row from its candidate list (block-wide device
// function, shared by the standalone select kernel and the attention kernel, which runs
// it redundantly per block instead of paying a kernel boundary).
//
// Inputs prepared by the filter kernel: every visible score whose first-level bin (top
// 11 key bits) is >= beta is a candidate (order key, position); `above` of them lie in
// bins > beta and are winners; inside bin beta the filter built a second-level histogram
// of the next 11 key bits.  The finaliser
//   1. finds in that histogram the second-level bin beta2 holding the remaining need,
//   2. collects the few candidates tied at (beta, beta2),
//   3. finds among them the threshold of the exact order (score desc, position asc) on
//      the 64-bit composite (key << 32 | ~position): rank counting when few, an MSB-first
//      radix select otherwise (e.g. many equal scores),
//   4. compacts the winners (above (beta, beta2), or tied with composite >= threshold)
//      in list order.  The filter writes the list in position order when there is no
//      candidate map, so the winners come out ascending; with a candidate map they are
//      ranked by position afterwards.
#pragma once

#include "common.hpp"

namespace csa2 {

constexpr int kFinStage = 8192;   // candidates staged in LDS; longer lists are read from global memory
constexpr int kFinCap = 1024;     // tied candidates held in LDS; more are re-read from the list
constexpr int kFinRankMax = 256;  // tied sets up to this size are resolved by rank counting
constexpr int kFinMaxRegions = 8192;
constexpr int kFilterColsPerBlock = 4096;  // columns (and candidate slots) per filter block, many rows
constexpr int kFilterColsNarrow = 2048;    // the same for a few (decode) rows: twice the blocks

__device__ __forceinline__ uint32_t hist2_bin(uint32_t key) { return (key >> (32 - 2 * kHistBits)) & (kHistBins - 1); }

struct FinalizeSmem {
  uint32_t h256[256];
  uint32_t misc[16];
  uint32_t wsum[16];
  uint32_t start[kFinMaxRegions + 1];  // exclusive prefix of the per-region counts
  uint2 stage[kFinStage];
  uint2 tied[kFinCap];
  alignas(16) uint32_t win_pos[CSA2_MAX_K_DEV];
  uint32_t win_key[CSA2_MAX_K_DEV];
};

// A row's candidates: the filter block b of the row wrote cnt[b] pairs at regions +
// b * stride (the columns a filter block covers); `start` (LDS) is the exclusive prefix of
// the counts.
struct CandList {
  const uint2* regions;
  const uint32_t* start;
  int nreg;
  int stride;
  __device__ __forceinline__ uint2 get(uint32_t i) const {
    int lo = 0, hi = nreg - 1;  // last region whose start <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return regions[(int64_t)lo * stride + (i - start[lo])];
  }
};

// inclusive suffix sum of v over threads tid..T-1 (T a multiple of 64, <= block size);
// threads >= T contribute and receive 0.  Contains two block barriers.
template <int NT, int T>
__device__ __forceinline__ uint32_t block_suffix(uint32_t v, uint32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_suffix((tid < T) ? v : 0u);
  if (lane == 0) wsum[wave] = x;
  __syncthreads();
  uint32_t add = 0;
#pragma unroll
  for (int w2 = 1; w2 < T / 64; ++w2) add += (w2 > wave) ? wsum[w2] : 0u;  // independent reads
  __syncthreads();
  return (tid < T) ? x + add : 0u;
}

// The tie test: same first- and second-level bins as the threshold.
__device__ __forceinline__ bool is_tied(uint32_t key, uint32_t beta, uint32_t beta2) {
  return hist_bin(key) == beta && hist2_bin(key) == beta2;
}

// The composite threshold among the tied candidates: exactly `need` (>= 1) of them have
// composite >= the returned value.  src[0..n) holds the tied candidates (FILTERED =
// false), or is the row's whole candidate list from which the tied ones are picked by
// is_tied.  Ends with a block barrier; every thread gets the value.
template <int NT, bool FILTERED, typename SRC, typename SM>
__device__ __forceinline__ uint64_t tied_threshold(const SRC& src, uint32_t n, uint32_t need, uint32_t beta, uint32_t beta2, SM& sm) {
  const int tid = threadIdx.x;
  if (!FILTERED && n <= (uint32_t)kFinRankMax) {
    for (uint32_t i = tid; i < n; i += NT) {  // ranks are distinct: positions are
      const uint2 c = src(i);
      const uint64_t ci = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      uint32_t rank = 0;
      for (uint32_t j = 0; j < n; ++j) {
        const uint2 d = src(j);
        const uint64_t cj = ((uint64_t)d.x << 32) | (uint32_t)(~d.y);
        rank += (cj > ci) ? 1u : 0u;
      }
      if (rank == need - 1) {
        sm.misc[12] = (uint32_t)ci;
        sm.misc[13] = (uint32_t)(ci >> 32);
      }
    }
    __syncthreads();
    return ((uint64_t)sm.misc[13] << 32) | sm.misc[12];
  }
  // radix select over 8-bit digits of the composite, most significant first; the
  // selected ones are those with (comp & mask) >= prefix, i.e. comp >= prefix
  uint64_t prefix = 0, mask = 0;
  uint32_t rem = need;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) sm.h256[tid] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += NT) {
      const uint2 c = src(i);
      if (FILTERED && !is_tied(c.x, beta, beta2)) continue;
      const uint64_t comp = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      if ((comp & mask) == prefix) atomicAdd(&sm.h256[(comp >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t mine = (tid < 256) ? sm.h256[tid] : 0u;
    const uint32_t sfx = block_suffix<NT, 256>(mine, sm.wsum);
    if (tid < 256 && sfx >= rem && sfx - mine < rem) {
      sm.misc[8] = tid;
      sm.misc[9] = sfx - mine;
      sm.misc[10] = mine;
    }
    __syncthreads();
    rem -= sm.misc[9];
    prefix |= (uint64_t)sm.misc[8] << shift;
    mask |= (uint64_t)255u << shift;
    const bool done = (sm.misc[10] == rem);
    __syncthreads();
    if (done) break;
  }
  return prefix;
}

// Writes the keff winners' positions (ascending) to out_pos[0..keff) and, if out_key !=
// nullptr, their order keys; returns keff.  All threads of the block must call it.
// The candidates are in `nreg` regions of `rstride` pairs (counts in cnt);
// SORTED: the list is in ascending position order (no candidate map).
template <int NT, bool SORTED>
__device__ __forceinline__ int finalize_row(const uint2* __restrict__ regions, const uint32_t* __restrict__ cnt, int nreg,
                            int rstride, const uint32_t* __restrict__ h2row, uint32_t beta, uint32_t above, uint32_t keff,
                            FinalizeSmem& sm, int32_t* out_pos, uint32_t* out_key) {
  constexpr int kWaves = NT / 64;
  constexpr int kCompPer = 64 / kWaves;  // list items per thread and compaction pass
  static_assert(kCompPer * kWaves == 64 && kCompPer >= 1, "one wave scans the (pass, wave) counts");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the second-level histogram is loaded first (before anything waits for the row's
  // control values): its latency overlaps the count prefix
  constexpr int kPer = (kHistBins / NT > 0) ? kHistBins / NT : 1;  // bins per thread
  constexpr int kT = kHistBins / kPer;                               // threads holding bins
  uint32_t hb[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) hb[i] = (tid < kT) ? h2row[tid * kPer + i] : 0u;
  if (keff == 0) return 0;
  // 0. region starts: exclusive prefix of the per-region counts (one wave when there are
  //    at most 64 regions, else one load per thread per pass; nreg <= kFinMaxRegions)
  if (nreg <= 64) {
    if (wave == 0) {
      const uint32_t v = (lane < nreg) ? cnt[lane] : 0u;
      const uint32_t sfx = wave_suffix(v);  // counts of regions >= lane
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
      if (lane < nreg) sm.start[lane] = tot - sfx;
      if (lane == 0) sm.misc[4] = tot;
    }
    __syncthreads();
  } else {
    uint32_t carry = 0;
    for (int base = 0; base < nreg; base += NT) {
      const int rg = base + tid;
      const uint32_t v = (rg < nreg) ? cnt[rg] : 0u;
      const uint32_t suf = block_suffix<NT, NT>(v, sm.wsum);  // sum over threads >= tid
      if (tid == 0) sm.misc[4] = suf;                         // pass total
      __syncthreads();
      const uint32_t total = sm.misc[4];
      if (rg < nreg) sm.start[rg] = carry + (total - suf);
      carry += total;
      __syncthreads();
    }
    if (tid == 0) sm.misc[4] = carry;
    __syncthreads();
  }
  const uint32_t M = sm.misc[4];
  const CandList list{regions, sm.start, nreg, rstride};
  // 1. issue the loads that stage the candidates in LDS (all in flight, clamped,
  //    branch-free); they are stored after the second-level scan, which hides them
  constexpr int kStagePer = kFinStage / NT;
  const bool staged = M <= (uint32_t)kFinStage;
  uint2 sv[kStagePer];
  if (staged) {
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const uint32_t i = tid + u * NT;
      if (u * NT < (int)M) sv[u] = list.get(i < M ? i : M - 1);  // uniform guard
    }
  }
  // 2. second-level threshold inside bin beta
  const uint32_t need1 = keff - above;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) local += hb[i];
  if (tid == 0) {
    sm.misc[0] = 0;  // beta2
    sm.misc[1] = 0;  // candidates of bin beta above beta2
    sm.misc[2] = 0;  // tied count
  }
  const uint32_t suf = block_suffix<NT, kT>(local, sm.wsum);
  if (tid < kT && suf >= need1 && suf - local < need1) {
    uint32_t acc = suf - local;
    for (int i = kPer - 1; i >= 0; --i) {
      if (acc + hb[i] >= need1) {
        sm.misc[0] = tid * kPer + i;
        sm.misc[1] = acc;
        break;
      }
      acc += hb[i];
    }
  }
  if (staged) {
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const uint32_t i = tid + u * NT;
      if (i < M) sm.stage[i] = sv[u];
    }
  }
  __syncthreads();
  const uint32_t beta2 = sm.misc[0];
  const uint32_t need3 = need1 - sm.misc[1];  // >= 1: bin (beta, beta2) holds the K-th
  // 3. collect the candidates tied at (beta, beta2)
  for (uint32_t base = 0; base < M; base += NT) {  // uniform trip count: wave_reserve needs every lane
    const uint32_t i = base + tid;
    const bool valid = i < M;
    const uint2 c = valid ? (staged ? sm.stage[i] : list.get(i)) : make_uint2(0u, 0u);
    const bool tie = valid && is_tied(c.x, beta, beta2);
    const uint32_t ts = wave_reserve(&sm.misc[2], tie);
    if (tie && ts < (uint32_t)kFinCap) sm.tied[ts] = c;
  }
  __syncthreads();
  // 4. the composite threshold among them (held in LDS, or - rare, e.g. many equal
  //    scores - picked out of the whole candidate list again)
  const uint32_t ntied = sm.misc[2];
  uint64_t thr;
  if (ntied <= (uint32_t)kFinCap) {
    const uint2* tl = sm.tied;
    thr = tied_threshold<NT, false>([tl](uint32_t i) { return tl[i]; }, ntied, need3, beta, beta2, sm);
  } else if (staged) {
    const uint2* st = sm.stage;
    thr = tied_threshold<NT, true>([st](uint32_t i) { return st[i]; }, M, need3, beta, beta2, sm);
  } else {
    thr = tied_threshold<NT, true>([list](uint32_t i) { return list.get(i); }, M, need3, beta, beta2, sm);
  }
  // 5. compact the winners in list order: item base + 64 (kWaves u + wave) + lane goes to
  //    its (pass u, wave) count's exclusive prefix plus its rank in the ballot
  int32_t* dst_pos = SORTED ? out_pos : reinterpret_cast<int32_t*>(sm.win_pos);
  uint32_t* dst_key = SORTED ? out_key : sm.win_key;
  uint32_t carry = 0;
  for (uint32_t base = 0; base < M; base += 64 * 64) {
    uint64_t bal[kCompPer];
    uint2 cv[kCompPer];
#pragma unroll
    for (int u = 0; u < kCompPer; ++u) {
      const uint32_t i = base + 64 * (kWaves * u + wave) + lane;
      const bool valid = i < M;
      const uint2 c = valid ? (staged ? sm.stage[i] : list.get(i)) : make_uint2(0u, 0u);
      const uint32_t b1 = hist_bin(c.x), b2 = hist2_bin(c.x);
      const uint64_t comp = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      const bool win = valid && (b1 > beta || (b1 == beta && (b2 > beta2 || (b2 == beta2 && comp >= thr))));
      bal[u] = __ballot(win);
      cv[u] = c;
    }
    if (lane < kCompPer) {
      uint32_t n = 0;
#pragma unroll
      for (int u = 0; u < kCompPer; ++u)
        if (u == lane) n = (uint32_t)__builtin_popcountll(bal[u]);
      sm.h256[lane * kWaves + wave] = n;
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t v = sm.h256[lane];
      const uint32_t sfx = wave_suffix(v);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
      sm.h256[64 + lane] = carry + tot - sfx;
      if (lane == 0) sm.misc[5] = tot;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kCompPer; ++u) {
      if ((bal[u] >> lane) & 1ull) {
        const uint32_t slot = sm.h256[64 + u * kWaves + wave] + lanes_below(bal[u]);
        if (slot < (uint32_t)CSA2_MAX_K_DEV) {
          dst_pos[slot] = (int32_t)cv[u].y;
          if (!SORTED || out_key) dst_key[slot] = cv[u].x;
        }
      }
    }
    carry += sm.misc[5];
    __syncthreads();
  }
  if (!SORTED) {
    // rank the winners by position (distinct positions): each counts the smaller ones,
    // reading the list four at a time (broadcast LDS reads)
    for (uint32_t i = tid; i < keff; i += NT) {
      const uint32_t p = sm.win_pos[i];
      uint32_t rank = 0;
      const uint32_t k4 = keff & ~3u;
#pragma unroll 8
      for (uint32_t j = 0; j < k4; j += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.win_pos[j]);
        rank += (v.x < p) + (v.y < p) + (v.z < p) + (v.w < p);
      }
      for (uint32_t j = k4; j < keff; ++j) rank += (sm.win_pos[j] < p) ? 1u : 0u;
      out_pos[rank] = (int32_t)p;
      if (out_key) out_key[rank] = sm.win_key[i];
    }
    __syncthreads();
  }
  return (int)keff;
}

}  // namespace csa2
