// Exact Top-K finalisation of one query row from its candidate list (block-wide device
// function, shared by the standalone select kernel and the attention kernel, which runs
// it redundantly per block instead of paying a kernel boundary).
//
// Inputs prepared by the filter kernel: every visible score whose first-level bin (top
// 11 key bits) is >= beta is a candidate (order key, position); `above` of them lie in
// bins > beta and are winners; inside bin beta the filter built a second-level histogram
// of the next 11 key bits.  The finaliser
//   1. finds in that histogram the second-level bin beta2 holding the remaining need,
//   2. keeps every candidate above (beta, beta2) and collects the few tied at (beta, beta2),
//   3. picks the remaining need among the tied ones by the exact order (score desc,
//      position asc) - rank counting when few, an MSB-first radix select on the 64-bit
//      composite (key << 32 | ~position) otherwise (e.g. many equal scores),
//   4. ranks the winners by position (ascending output).
#pragma once

#include "common.hpp"

namespace csa2 {

constexpr int kFinStage = 4096;   // candidates staged in LDS; longer lists are read from global memory
constexpr int kFinCap = 1024;     // tied candidates held in LDS; more are re-read from the list
constexpr int kFinRankMax = 256;  // tied sets up to this size are resolved by rank counting
constexpr int kFinMaxRegions = 4096;
constexpr int kFilterColsPerBlock = 4096;  // columns (and candidate slots) per filter block

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
// b * kFilterColsPerBlock; `start` (LDS) is the exclusive prefix of the counts.
struct CandList {
  const uint2* regions;
  const uint32_t* start;
  int nreg;
  __device__ __forceinline__ uint2 get(uint32_t i) const {
    int lo = 0, hi = nreg - 1;  // last region whose start <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return regions[(int64_t)lo * kFilterColsPerBlock + (i - start[lo])];
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
  for (int w2 = wave + 1; w2 < T / 64; ++w2) add += wsum[w2];
  __syncthreads();
  return (tid < T) ? x + add : 0u;
}

// The tie test: same first- and second-level bins as the threshold.
__device__ __forceinline__ bool is_tied(uint32_t key, uint32_t beta, uint32_t beta2) {
  return hist_bin(key) == beta && hist2_bin(key) == beta2;
}

// Select `need` of the tied candidates by the exact order and append them to the winner
// list (slot counter misc[3]).  src[0..n) holds the tied candidates (FILTERED = false), or
// is the row's whole candidate list from which the tied ones are picked by is_tied.
template <int NT, bool FILTERED, typename SRC>
__device__ void select_tied(const SRC& src, uint32_t n, uint32_t need, uint32_t beta, uint32_t beta2,
                            FinalizeSmem& sm) {
  const int tid = threadIdx.x;
  if (need == 0) return;
  if (!FILTERED && n <= (uint32_t)kFinRankMax) {
    for (uint32_t i = tid; i < n; i += NT) {
      const uint2 c = src(i);
      const uint64_t ci = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      uint32_t rank = 0;
      for (uint32_t j = 0; j < n; ++j) {
        const uint2 d = src(j);
        const uint64_t cj = ((uint64_t)d.x << 32) | (uint32_t)(~d.y);
        rank += (cj > ci) ? 1u : 0u;
      }
      if (rank < need) {
        const uint32_t slot = atomicAdd(&sm.misc[3], 1u);
        if (slot < (uint32_t)CSA2_MAX_K_DEV) {
          sm.win_pos[slot] = c.y;
          sm.win_key[slot] = c.x;
        }
      }
    }
    __syncthreads();
    return;
  }
  // radix select over 8-bit digits of the composite, most significant first
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
  for (uint32_t i = tid; i < n; i += NT) {
    const uint2 c = src(i);
    if (FILTERED && !is_tied(c.x, beta, beta2)) continue;
    const uint64_t comp = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
    if ((comp & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&sm.misc[3], 1u);
      if (slot < (uint32_t)CSA2_MAX_K_DEV) {
        sm.win_pos[slot] = c.y;
        sm.win_key[slot] = c.x;
      }
    }
  }
  __syncthreads();
}

// Writes the keff winners' positions (ascending) to out_pos[0..keff) and, if out_key !=
// nullptr, their order keys; returns keff.  All threads of the block must call it.
// The candidates are in `nreg` regions of kFilterColsPerBlock pairs (counts in cnt).
template <int NT>
__device__ int finalize_row(const uint2* __restrict__ regions, const uint32_t* __restrict__ cnt, int nreg,
                            const uint32_t* __restrict__ h2row, uint32_t beta, uint32_t above, uint32_t keff,
                            FinalizeSmem& sm, int32_t* out_pos, uint32_t* out_key) {
  const int tid = threadIdx.x;
  if (keff == 0) return 0;
  // 0. region starts: exclusive prefix of the per-region counts (one load per thread per
  //    pass; nreg <= kFinMaxRegions)
  {
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
  const CandList list{regions, sm.start, nreg};
  // 1. stage the candidates in LDS (four loads in flight per thread, clamped, branch-free)
  const bool staged = M <= (uint32_t)kFinStage;
  if (staged) {
    for (uint32_t base = tid; base < M; base += 4 * NT) {
      uint2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = base + u * NT;
        v[u] = list.get(i < M ? i : M - 1);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t i = base + u * NT;
        if (i < M) sm.stage[i] = v[u];
      }
    }
  }
  // 2. second-level threshold inside bin beta
  const uint32_t need1 = keff - above;
  constexpr int kPer = (kHistBins / NT > 0) ? kHistBins / NT : 1;  // bins per thread
  constexpr int kT = kHistBins / kPer;                               // threads holding bins
  uint32_t hb[kPer];
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    hb[i] = (tid < kT) ? h2row[tid * kPer + i] : 0u;
    local += hb[i];
  }
  if (tid == 0) {
    sm.misc[0] = 0;  // beta2
    sm.misc[1] = 0;  // candidates of bin beta above beta2
    sm.misc[2] = 0;  // tied count
    sm.misc[3] = 0;  // winner count
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
  __syncthreads();
  const uint32_t beta2 = sm.misc[0];
  const uint32_t need3 = need1 - sm.misc[1];
  // 3. classify: winners above (beta, beta2), tied at (beta, beta2)
  for (uint32_t base = 0; base < M; base += NT) {  // uniform trip count: wave_reserve needs every lane
    const uint32_t i = base + tid;
    const bool valid = i < M;
    const uint2 c = valid ? (staged ? sm.stage[i] : list.get(i)) : make_uint2(0u, 0u);
    const uint32_t b1 = hist_bin(c.x);
    const uint32_t b2 = hist2_bin(c.x);
    const bool win = valid && (b1 > beta || (b1 == beta && b2 > beta2));
    const bool tie = valid && b1 == beta && b2 == beta2;
    const uint32_t ws = wave_reserve(&sm.misc[3], win);
    const uint32_t ts = wave_reserve(&sm.misc[2], tie);
    if (win && ws < (uint32_t)CSA2_MAX_K_DEV) {
      sm.win_pos[ws] = c.y;
      sm.win_key[ws] = c.x;
    }
    if (tie && ts < (uint32_t)kFinCap) sm.tied[ts] = c;
  }
  __syncthreads();
  // 4. the remaining need among the tied candidates (held in LDS, or - rare, e.g. many
  //    equal scores - picked out of the whole candidate list again)
  const uint32_t ntied = sm.misc[2];
  if (ntied <= (uint32_t)kFinCap) {
    const uint2* tl = sm.tied;
    select_tied<NT, false>([tl](uint32_t i) { return tl[i]; }, ntied, need3, beta, beta2, sm);
  } else if (staged) {
    const uint2* st = sm.stage;
    select_tied<NT, true>([st](uint32_t i) { return st[i]; }, M, need3, beta, beta2, sm);
  } else {
    select_tied<NT, true>([list](uint32_t i) { return list.get(i); }, M, need3, beta, beta2, sm);
  }
  // 5. rank the winners by position (distinct positions): each counts the smaller ones,
  //    reading the list four at a time (broadcast LDS reads)
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
  return (int)keff;
}

}  // namespace csa2
