// Exact Top-K of one query row from the candidate lists its score blocks wrote (one
// workgroup per row, k_topk_select).
//
// Every score block of a row lists the visible scores of its columns that lie in first-level
// bins (top 11 order-key bits) above a block-local cut, the lowest bin such that the bins
// above hold at most a few times the winners a block holds on average; it also records its
// cut and how many visible scores it has (all of them listed: a complete block).  Let tau be
// the K-th largest (score, lower position first) among the listed candidates and beta its
// bin.  If every incomplete block's cut lies below beta, every unlisted score is in a bin
// below beta, hence below tau, and the listed candidates hold the whole Top-K: the K-th of
// the candidates is the K-th overall.  Otherwise (clustered scores, many equal scores, a
// block holding more winners than it listed) the failing blocks are re-read whole from the
// row's scores and the selection runs again over the enlarged list, in which no block can
// fail any more (enlarging the list only raises tau).
//
// The selection itself is a radix select on the composite (key << 32 | ~position): the
// threshold bin beta from the first-level histogram, the second-level bin inside it (the
// next 11 key bits), the few candidates tied at both, their exact composite threshold
// (rank counting, or an 8-bit-digit radix select), then an ordered compaction.  Lists are in
// column order, so without a candidate map the winners come out by ascending position.
#pragma once

#include "score_dev.hpp"
#include "topk_dev.hpp"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelMaxRegions = 8192;

struct SelectSmem {
  // h1 and h2 (16 KB, contiguous) also hold the staging owner map (uint16 region of each
  // list item) before the histograms are built
  alignas(16) uint32_t h1[kHistBins];  // read 16 bytes at a time
  alignas(16) uint32_t h2[kHistBins];
  uint32_t h256[256];
  uint32_t misc[16];
  uint32_t wsum[16];
  uint32_t start[kSelMaxRegions + 1];  // exclusive prefix of the region sizes
  uint32_t raw[kSelMaxRegions / 32];   // bit per region: re-read whole from the scores (fallback)
  uint2 stage[kFinStage];
  uint2 tied[kFinCap];
  alignas(16) uint32_t win_pos[CSA2_MAX_K_DEV];
  uint32_t win_key[CSA2_MAX_K_DEV];
};

// A row's candidates as one list in column order: region b holds start[b+1] - start[b]
// items, either its listed (key, position) pairs, or (raw[b]) its whole column range read
// from the row's scores (key 0 = not visible).
struct RowList {
  const uint2* regions;   // [nreg][stride]
  const uint32_t* start;  // LDS
  const uint32_t* raw;    // LDS bit mask
  int nreg;
  int stride;             // slots per region
  int rcols;              // columns per region
  const float* srow;      // the row's re-scored scores (raw regions)
  const int32_t* prow;    // the row's candidate positions (nullable: position = column)
  // item k of region b
  __device__ __forceinline__ uint2 get_in(int b, uint32_t k) const {
    if (!((raw[b >> 5] >> (b & 31)) & 1u)) return regions[(int64_t)b * stride + k];
    const int64_t col = (int64_t)b * rcols + k;
    const float sc = __builtin_nontemporal_load(srow + col);  // written by this workgroup (re-score)
    const int32_t pos = prow ? prow[col] : (int32_t)col;
    return make_uint2((visible(sc) && pos >= 0) ? order_key(sc) : 0u, (uint32_t)pos);
  }
  __device__ __forceinline__ uint2 get(uint32_t i) const {
    int lo = 0, hi = nreg - 1;  // last region whose start <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return get_in(lo, i - start[lo]);
  }
};

// Wave 0 finds the bin of a 2048-bin LDS histogram that holds the need-th largest item (bins
// counted from the top) and writes it to *bin_out (kHistBins if the histogram holds fewer
// than need), the items in higher bins to *above_out and, if count_out != nullptr, the items
// in that bin to *count_out (0 without one).  Lane l sums bins 32 l .. 32 l + 31;
// one suffix scan finds the group of 32 bins, a second one (a bin per lane) the bin.  One
// wave's scans instead of block-wide ones: the other waves only meet it at the caller's next
// barrier.
__device__ __forceinline__ void wave0_threshold_bin(const uint32_t* h, uint32_t need, uint32_t* bin_out,
                                                    uint32_t* above_out, uint32_t* count_out = nullptr) {
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63;
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = *reinterpret_cast<const uint4*>(&h[32 * lane + 4 * q]);
    local += v.x + v.y + v.z + v.w;
  }
  const uint32_t suf = wave_suffix(local);  // items in bins >= 32 lane
  const uint64_t grp = __ballot(need > 0 && suf >= need && suf - local < need);
  if (grp == 0) {
    if (lane == 0) {
      *bin_out = kHistBins;
      *above_out = 0;
      if (count_out) *count_out = 0;
    }
    return;
  }
  const int g = __builtin_ctzll(grp);
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(suf - local), g);  // items above group g
  const uint32_t hv = lane < 32 ? h[32 * g + lane] : 0u;
  const uint32_t s2 = base + wave_suffix(hv);  // lane < 32: items in bins >= 32 g + lane
  if (lane < 32 && s2 >= need && s2 - hv < need) {  // one lane (hv > 0 there)
    *bin_out = 32 * g + lane;
    *above_out = s2 - hv;
    if (count_out) *count_out = hv;
  }
}

// The first-level threshold over the list: sm.misc[0] = beta (kHistBins if fewer than keff
// visible items), sm.misc[1] = visible items in bins above beta.  BUILD: count the list into
// sm.h1 here (cleared here); otherwise the caller did, cleared h1 and h2 and synchronised.
// Also clears sm.h2 for select_winners (BUILD) and resets the tied count.  src(i) gives item i.
template <int NT, bool BUILD, typename SRC>
__device__ __forceinline__ void select_first_level(const SRC& src, uint32_t M, uint32_t keff, SelectSmem& sm) {
  const int tid = threadIdx.x;
  if (BUILD) {
    for (int i = tid; i < kHistBins; i += NT) {
      sm.h1[i] = 0;
      sm.h2[i] = 0;
    }
    __syncthreads();
    for (uint32_t i = tid; i < M; i += NT) {
      const uint32_t key = src(i).x;
      if (key) atomicAdd(&sm.h1[hist_bin(key)], 1u);
    }
    __syncthreads();
  }
  wave0_threshold_bin(sm.h1, keff, &sm.misc[0], &sm.misc[1]);
  if (tid == 0) sm.misc[4] = 0;  // tied count
  __syncthreads();
}

// The winners (composite >= thr: exactly keff items) of the list in list order, their
// positions to out_pos (SORTED: ascending) and, if out_key != nullptr, their order keys.
// Item base + 64 (kWaves u + wave) + lane goes to its (pass u, wave) count's exclusive
// prefix plus its rank in the ballot.  Without SORTED the winners are then ranked by position.
template <int NT, bool SORTED, typename SRC>
__device__ __forceinline__ void compact_winners(const SRC& src, uint32_t M, uint32_t keff, uint64_t thr,
                                                SelectSmem& sm, int32_t* out_pos, uint32_t* out_key) {
  constexpr int kWaves = NT / 64;
  constexpr int kCompPer = 64 / kWaves;  // list items per thread and compaction pass
  static_assert(kCompPer * kWaves == 64 && kCompPer >= 1, "one wave scans the (pass, wave) counts");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
      const uint2 c = valid ? src(i) : make_uint2(0u, 0u);
      const uint64_t comp = ((uint64_t)c.x << 32) | (uint32_t)(~c.y);
      bal[u] = __ballot(valid && c.x && comp >= thr);
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
    // every wave scans the 64 (pass, wave) counts itself (no second barrier): the offset of
    // (u, wave) is the suffix's complement at lane kWaves u + wave
    const uint32_t sfx = wave_suffix(sm.h256[lane]);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
    const uint32_t off = carry + tot - sfx;
#pragma unroll
    for (int u = 0; u < kCompPer; ++u) {
      const uint32_t base_u = (uint32_t)__builtin_amdgcn_readlane((int)off, u * kWaves + wave);
      if ((bal[u] >> lane) & 1ull) {
        const uint32_t slot = base_u + lanes_below(bal[u]);
        if (slot < (uint32_t)CSA2_MAX_K_DEV) {
          dst_pos[slot] = (int32_t)cv[u].y;
          if (!SORTED || out_key) dst_key[slot] = cv[u].x;
        }
      }
    }
    carry += tot;
    __syncthreads();  // every wave has read the counts before the next pass (or the caller) reuses h256
  }
  if (!SORTED) {
    // rank the winners by position (distinct positions): each counts the smaller ones
    for (uint32_t i = tid; i < keff; i += NT) {
      const uint32_t p = sm.win_pos[i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < keff; ++j) rank += (sm.win_pos[j] < p) ? 1u : 0u;
      out_pos[rank] = (int32_t)p;
      if (out_key) out_key[rank] = sm.win_key[i];
    }
    __syncthreads();
  }
}

// Given the first-level threshold (beta, above) of the list, the keff winners' positions in
// list order (SORTED: ascending) to out_pos and, if out_key != nullptr, their order keys.
template <int NT, bool SORTED, typename SRC>
__device__ __forceinline__ void select_winners(const SRC& src, uint32_t M, uint32_t keff, uint32_t beta, uint32_t above,
                               SelectSmem& sm, int32_t* out_pos, uint32_t* out_key) {
  const int tid = threadIdx.x;
  // 1. second-level histogram of bin beta (h2 cleared before the first-level barrier) and
  //    its threshold
  for (uint32_t i = tid; i < M; i += NT) {
    const uint32_t key = src(i).x;
    if (key && hist_bin(key) == beta) atomicAdd(&sm.h2[hist2_bin(key)], 1u);
  }
  __syncthreads();
  const uint32_t need1 = keff - above;
  wave0_threshold_bin(sm.h2, need1, &sm.misc[2], &sm.misc[3]);
  __syncthreads();
  const uint32_t beta2 = sm.misc[2];
  const uint32_t need3 = need1 - sm.misc[3];  // >= 1: bin (beta, beta2) holds the K-th
  // 2. the candidates tied at (beta, beta2)
  for (uint32_t base = 0; base < M; base += NT) {  // uniform trip count: wave_reserve needs every lane
    const uint32_t i = base + tid;
    const bool valid = i < M;
    const uint2 c = valid ? src(i) : make_uint2(0u, 0u);
    const bool tie = valid && c.x && is_tied(c.x, beta, beta2);
    const uint32_t ts = wave_reserve(&sm.misc[4], tie);
    if (tie && ts < (uint32_t)kFinCap) sm.tied[ts] = c;
  }
  __syncthreads();
  // 3. their composite threshold (held in LDS, or - many equal scores - picked out of the
  //    whole list again)
  const uint32_t ntied = sm.misc[4];
  uint64_t thr;
  if (ntied <= (uint32_t)kFinCap) {
    const uint2* tl = sm.tied;
    thr = tied_threshold<NT, false>([tl](uint32_t i) { return tl[i]; }, ntied, need3, beta, beta2, sm);
  } else {
    thr = tied_threshold<NT, true>(src, M, need3, beta, beta2, sm);
  }
  compact_winners<NT, SORTED>(src, M, keff, thr, sm, out_pos, out_key);
}

// The exact Top-K of row r from its score blocks' candidate lists (LocalCand), by the NT
// threads of a workgroup (rows of at most MAXREG regions): the region counts' prefix, the
// candidates staged in LDS, the first-level threshold and the check that every incomplete
// block's cut lies below it (else those blocks are re-read from the scores and the selection
// runs on the enlarged list), then the winners in list order.  Writes the keff = min(K,
// visible) winners' positions to out_pos (ascending with SORTED, else ranked by position)
// and, if out_key != nullptr, their order keys; returns keff.  Every thread must call it.
// Fast path (at most 64 regions whose slots fit the LDS staging: the decode rows and both
// stages of the two-level select): the region counts and every slot of every region are
// loaded in one round, their prefix is one wave's scan and a histogram over the listed
// keys' own range is counted from registers.
struct SelectIn {
  int nreg, stride;       // regions per row; candidate slots per region
  int spec;               // slots per region loaded with the counts (a power of two): the lists'
                          // expected cap, rounded up
  int rcols;              // columns per region (a score block's columns)
  int64_t ncols;
  int K;
  const uint2* candbuf;   // [R][nreg][stride]
  const uint32_t* cnt;    // [R][nreg]
  const int32_t* cut;
  const uint32_t* vis;
  float* scores;          // [R][ncols]: a re-scored region's scores (written and read only there)
  const int32_t* cand;    // [R][ncols] candidate positions, or nullptr (position = column)
  // the scan's inputs, for the re-score (32 heads x 64 dims)
  const void* q;          // [R][32][64] bf16 (q_bf16) or fp32
  int q_bf16, f4;         // f4: the FP4 indexer (32-byte keys), else E4M3 (64-byte keys)
  const float* w;         // [R][32]
  const uint8_t* k;       // [B][n_max][64 or 32]
  const float* ks;        // [B][n_max]
  int64_t n_max;
  const int32_t* n_keys;
  const int32_t* q_limit;
  int key_div, T;
  // optional expansion of the winners (columns = blocks of expand_block positions) into
  // their positions, [R][K * expand_block], -1 past the sequence's n_keys or for padding
  int32_t* expand_out;
  int expand_block;
};

// Re-score every region of row r marked in sm.raw into in.scores, with the score kernel's
// arithmetic (score_dev.hpp: the same query operand, MFMA and epilogue order, so each score
// is bit-identical to the one the scan computed), then make the stores visible to the
// workgroup.  Uses sm.h2 (the query row) and sm.h256 (the head factors), which the
// selection rebuilds afterwards.  Every thread must call it.
template <int NT>
__device__ __forceinline__ void rescore_raw_regions(const SelectIn& in, int r, SelectSmem& sm) {
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int b = r / in.T;
  // the query row into LDS, the head weights into registers
  const int qbytes = in.q_bf16 ? 32 * 64 * 2 : 32 * 64 * 4;
  for (int i = tid; i < qbytes / 16; i += NT)
    reinterpret_cast<uint4*>(sm.h2)[i] =
        reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(in.q) + (int64_t)r * qbytes)[i];
  const float wv = tid < 32 ? in.w[(int64_t)r * 32 + tid] : 0.0f;
  __syncthreads();
  float sq;
  v8i A;
  if (in.f4) {
    A = in.q_bf16 ? quantize_query_operand_fp4(reinterpret_cast<const uint16_t*>(sm.h2), lane, sq)
                  : quantize_query_operand_fp4(reinterpret_cast<const float*>(sm.h2), lane, sq);
  } else {
    A = in.q_bf16 ? quantize_query_operand<uint16_t, false>(reinterpret_cast<const uint16_t*>(sm.h2), lane, sq)
                  : quantize_query_operand<float, false>(reinterpret_cast<const float*>(sm.h2), lane, sq);
  }
  float* s_c = reinterpret_cast<float*>(sm.h256);
  if (wave == 0 && lane < 32) s_c[lane] = sq;
  __syncthreads();
  if (tid < 32) s_c[tid] = wv * s_c[tid];
  __syncthreads();
  float cvec[16];
  tile_head_factors(s_c, half, cvec);
  const int64_t lim = visible_limit(b, r, in.n_max, in.n_keys, in.q_limit, in.key_div);
  const int kb = in.f4 ? 32 : 64;  // key bytes
  const uint8_t* kbase = in.k + (int64_t)b * in.n_max * kb + (in.f4 ? 16 : 32) * half;
  const float* ksb = in.ks + (int64_t)b * in.n_max;
  const int32_t* crow = in.cand ? in.cand + (int64_t)r * in.ncols : nullptr;
  float* srow = in.scores + (int64_t)r * in.ncols;
  const int tiles = in.rcols / 32;
  for (int rg = 0; rg < in.nreg; ++rg) {
    if (!((sm.raw[rg >> 5] >> (rg & 31)) & 1u)) continue;  // uniform
    for (int t = wave; t < tiles; t += kWaves) {             // uniform per wave
      const int64_t col = (int64_t)rg * in.rcols + (int64_t)t * 32 + (lane & 31);
      int64_t pos = -1;
      if (col < in.ncols) pos = crow ? (int64_t)crow[col] : col;
      const bool v = pos >= 0 && pos <= lim;
      const int64_t rr = v ? pos : 0;
      const v4i* src = reinterpret_cast<const v4i*>(kbase + rr * kb);
      const v4i x0 = src[0];
      v4i x1 = {0, 0, 0, 0};
      if (!in.f4) x1 = src[1];
      const v8i B = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const float skl = ksb[rr];
      const float sc = in.f4 ? tile_score<true>(A, B, cvec, v, skl) : tile_score<false>(A, B, cvec, v, skl);
      if (half == 0 && col < in.ncols) srow[col] = sc;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <bool SORTED, int NT, int MAXREG>
__device__ __forceinline__ uint32_t select_row(const SelectIn& in, int r, SelectSmem& sm, int32_t* out_pos,
                                               uint32_t* out_key) {
  static_assert(MAXREG <= kSelMaxRegions && MAXREG >= 64, "region bound");
  constexpr int kRP = (MAXREG + NT - 1) / NT;  // regions per thread (region tid + NT j)
  constexpr int kSP = kFinStage / NT;         // staged items per thread
  constexpr int kWaves = NT / 64;
  constexpr int kFastRegions = 64;            // fast path: one wave's scan of the region counts,
  constexpr int kFastPer = kFinStage / NT;    //   every slot of every region loaded with the counts
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nreg = in.nreg, stride = in.stride, rcols = in.rcols, K = in.K;
  const int64_t ncols = in.ncols;
  const uint2* __restrict__ candbuf = in.candbuf;
  const uint32_t* __restrict__ cnt = in.cnt;
  const int32_t* __restrict__ cut = in.cut;
  const uint32_t* __restrict__ vis = in.vis;
  const float* scores = in.scores;  // written by the re-score, read after it
  const int32_t* __restrict__ cand = in.cand;
  const int spec = in.spec, ssh = __builtin_ctz((unsigned)spec);
  const int slots = nreg * spec;  // < kFinStage on the fast path
  const bool few = nreg <= kFastRegions && nreg * (int64_t)spec <= kFinStage;
  // 0. every load issued together: (few regions) the first spec slots of every region,
  //    whatever their counts turn out to be, then the region counts, cuts and visible counts,
  //    masked only after all are issued (a value used or spilled right after its load is
  //    waited for there, and with it every load issued before: the slots go first)
  uint2 fv[kFastPer];  // fast path: item tid + NT u = slot (i & (spec - 1)) of region (i >> ssh)
  if (few) {  // uniform
    const uint2* crow = candbuf + (int64_t)r * nreg * stride;
#pragma unroll
    for (int u = 0; u < kFastPer; ++u) {
      const int i = tid + NT * u;
      const int ic = i < slots ? i : slots - 1;
      if (NT * u < slots) fv[u] = crow[(int64_t)(ic >> ssh) * stride + (ic & (spec - 1))];  // uniform bound
    }
  }
  uint32_t rcv[kRP], rvv[kRP];
  int32_t rcutv[kRP];
  // (unconditional loads from clamped addresses, masked afterwards: a load behind a branch
  // is waited for where the branch joins)
#pragma unroll
  for (int j = 0; j < kRP; ++j) {
    const int rg = tid + NT * j;
    if (NT * j >= nreg) {  // uniform
      rcv[j] = rvv[j] = 0u;
      rcutv[j] = -1;
      continue;
    }
    const int64_t o = (int64_t)r * nreg + (rg < nreg ? rg : nreg - 1);
    rcv[j] = cnt[o];
    rvv[j] = vis[o];
    rcutv[j] = cut[o];
  }
#pragma unroll
  for (int j = 0; j < kRP; ++j) {
    if (tid + NT * j >= nreg) {
      rcv[j] = rvv[j] = 0u;
      rcutv[j] = -1;
    }
  }
  for (int i = tid; i < kSelMaxRegions / 32; i += NT) sm.raw[i] = 0u;
  for (int i = tid; i < kHistBins; i += NT) {
    sm.h1[i] = 0u;
    sm.h2[i] = 0u;
  }
  // region starts (exclusive prefix of the sizes: the listed count, or the region's columns
  // when it is re-read whole); sm.start[nreg] = the total
  auto prefix = [&](bool with_raw) -> uint32_t {
    uint32_t carry = 0;
#pragma unroll
    for (int j = 0; j < kRP; ++j) {
      if (NT * j >= nreg) break;  // uniform
      const int rg = tid + NT * j;
      uint32_t v = rcv[j];
      if (with_raw && rg < nreg && ((sm.raw[rg >> 5] >> (rg & 31)) & 1u)) {
        const int64_t left = ncols - (int64_t)rg * rcols;
        v = (uint32_t)(left < rcols ? left : rcols);
      }
      const uint32_t suf = block_suffix<NT, NT>(v, sm.wsum);
      if (tid == 0) sm.misc[8] = suf;
      __syncthreads();
      const uint32_t tot = sm.misc[8];
      if (rg < nreg) sm.start[rg] = carry + tot - suf;
      carry += tot;
      __syncthreads();
    }
    if (tid == 0) sm.start[nreg] = carry;
    return carry;
  };
  // 1. visible total and starts
  uint32_t V, M = 0;
  bool fast = false;
  if (few) {
    if (wave == 0) {  // regions are lanes: one wave's scans
      const uint32_t c = rcv[0];
      const uint32_t sfx = wave_suffix(c);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
      const uint32_t vsfx = wave_suffix(rvv[0]);
      if (lane < nreg) sm.start[lane] = tot - sfx;
      if (lane == 0) {
        sm.start[nreg] = tot;
        sm.misc[9] = (uint32_t)__builtin_amdgcn_readlane((int)vsfx, 0);
        sm.misc[11] = __ballot(c > (uint32_t)spec) ? 0u : 1u;
      }
    }
    __syncthreads();
    V = sm.misc[9];
    fast = sm.misc[11] != 0;  // every listed candidate was loaded
    M = sm.start[nreg];
  } else {
    uint32_t vloc = 0;
#pragma unroll
    for (int j = 0; j < kRP; ++j) vloc += rvv[j];
    const uint32_t vsuf = block_suffix<NT, NT>(vloc, sm.wsum);
    if (tid == 0) sm.misc[9] = vsuf;
    __syncthreads();
    V = sm.misc[9];
  }
  const uint32_t keff = V < (uint32_t)K ? V : (uint32_t)K;
  RowList L{candbuf + (int64_t)r * nreg * stride, sm.start, sm.raw, nreg, stride, rcols, scores + (int64_t)r * ncols,
            cand ? cand + (int64_t)r * ncols : nullptr};
  const uint2* st = sm.stage;
  int pass = 0;
  if (keff > 0 && fast) {
    // 2. stage the listed candidates from registers, and the range [lo, hi] of their keys
    //    over the row
    bool have[kFastPer];
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int u = 0; u < kFastPer; ++u) {
      const int i = tid + NT * u;
      have[u] = false;
      if (NT * u < slots && i < slots) {
        const int b = i >> ssh, k = i & (spec - 1);
        const uint32_t s0 = sm.start[b];
        have[u] = (uint32_t)k < sm.start[b + 1] - s0;
        if (have[u]) {
          sm.stage[s0 + k] = fv[u];
          kmn = min(kmn, fv[u].x);
          kmx = max(kmx, fv[u].x);
        }
      }
    }
    kmn = wave_min_u(kmn);
    kmx = wave_max_u(kmx);
    if (lane == 0) {
      sm.h256[wave] = kmn;
      sm.h256[kWaves + wave] = kmx;
    }
    __syncthreads();
    // 3. a histogram over the keys' own range, bins of 2^sh keys (at most 2048 bins): the
    //    listed keys sit in a few first-level bins, so counting them there would make every
    //    atomic of a bin wait for the others; spread over their range they rarely collide
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lo = min(lo, sm.h256[w]);
      hi = max(hi, sm.h256[kWaves + w]);
    }
    const uint32_t span = hi - lo;  // M >= keff >= 1 items, so lo <= hi
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    const int sh = bits > kHistBits ? bits - kHistBits : 0;
#pragma unroll
    for (int u = 0; u < kFastPer; ++u)
      if (have[u]) atomicAdd(&sm.h1[(fv[u].x - lo) >> sh], 1u);
    __syncthreads();
    wave0_threshold_bin(sm.h1, keff, &sm.misc[0], &sm.misc[1], &sm.misc[2]);
    if (tid == 0) sm.misc[4] = 0;  // tied count
    __syncthreads();
    const uint32_t tb = sm.misc[0], above = sm.misc[1], ntied = sm.misc[2];
    if (tb >= (uint32_t)kHistBins) {  // uniform: fewer listed than keff, every incomplete block is re-read
      if (wave == 0) {
        const uint64_t bal = __ballot(lane < nreg && rvv[0] > rcv[0]);
        if (lane < 2) sm.raw[lane] = (uint32_t)(bal >> (32 * lane));
      }
      __syncthreads();
      pass = 1;
    } else if (ntied <= (uint32_t)kFinCap) {  // uniform
      // 4. the candidates in bin tb (the K-th among them), their exact composite threshold
#pragma unroll
      for (int u = 0; u < kFastPer; ++u) {
        const bool tie = have[u] && ((fv[u].x - lo) >> sh) == tb;
        const uint32_t ts = wave_reserve(&sm.misc[4], tie);
        if (tie) sm.tied[ts] = fv[u];
      }
      __syncthreads();
      const uint2* tl = sm.tied;
      const uint64_t thr = tied_threshold<NT, false>([tl](uint32_t i) { return tl[i]; }, ntied, keff - above, 0u, 0u, sm);
      // 5. the check (regions are lanes of wave 0): every incomplete block's cut must lie
      //    below the first-level bin of the K-th score; the flag is read after the
      //    compaction's barriers
      const uint32_t beta = hist_bin((uint32_t)(thr >> 32));
      if (wave == 0) {
        const bool bad = lane < nreg && rvv[0] > rcv[0] && rcutv[0] >= (int32_t)beta;
        const uint64_t bal = __ballot(bad);
        if (lane < 2) sm.raw[lane] = (uint32_t)(bal >> (32 * lane));
        if (lane == 0) sm.misc[14] = bal ? 1u : 0u;
      }
      auto src = [&](uint32_t i) -> uint2 { return st[i]; };
      compact_winners<NT, SORTED>(src, M, keff, thr, sm, out_pos, out_key);
      pass = sm.misc[14] ? 1 : 2;
    } else {
      // many equal keys: the first-level selection over the staged list
      auto src = [&](uint32_t i) -> uint2 { return st[i]; };
      select_first_level<NT, true>(src, M, keff, sm);
      const uint32_t beta = sm.misc[0], ab = sm.misc[1];
      if (wave == 0) {
        const bool bad = lane < nreg && rvv[0] > rcv[0] && (beta >= (uint32_t)kHistBins || rcutv[0] >= (int32_t)beta);
        const uint64_t bal = __ballot(bad);
        if (lane < 2) sm.raw[lane] = (uint32_t)(bal >> (32 * lane));
        if (lane == 0) sm.misc[14] = bal ? 1u : 0u;
      }
      __syncthreads();
      if (!sm.misc[14]) {
        select_winners<NT, SORTED>(src, M, keff, beta, ab, sm, out_pos, out_key);
        pass = 2;
      } else {
        pass = 1;
      }
    }
    if (pass == 1) {  // the fallback over the enlarged list
      rescore_raw_regions<NT>(in, r, sm);
      M = prefix(true);
      __syncthreads();
    }
  } else if (keff > 0) {
    M = prefix(false);
    __syncthreads();
  }
  for (; pass < 2 && keff > 0; ++pass) {  // generic path; pass 1: the fallback over the enlarged list
    const bool staged = M <= (uint32_t)kFinStage;
    if (staged) {
      // owner map (the region of every item), then every item's load in flight at once
      uint16_t* owner = reinterpret_cast<uint16_t*>(sm.h1);
      for (int b = wave; b < nreg; b += kWaves) {
        const uint32_t s0 = sm.start[b], n = sm.start[b + 1] - s0;
        for (uint32_t k = lane; k < n; k += 64) owner[s0 + k] = (uint16_t)b;
      }
      __syncthreads();
      uint2 v[kSP];
#pragma unroll
      for (int u = 0; u < kSP; ++u) {
        const uint32_t i = tid + NT * u;
        if (i < M) {
          const int b = owner[i];
          v[u] = L.get_in(b, i - sm.start[b]);
        }
      }
#pragma unroll
      for (int u = 0; u < kSP; ++u) {
        const uint32_t i = tid + NT * u;
        if (i < M) sm.stage[i] = v[u];
      }
      __syncthreads();
    }
    auto src = [&](uint32_t i) -> uint2 { return staged ? st[i] : L.get(i); };
    select_first_level<NT, true>(src, M, keff, sm);
    const uint32_t beta = sm.misc[0], above = sm.misc[1];
    if (pass == 0) {
      // the check: an incomplete block whose cut is not below beta may hold unlisted winners
      if (tid == 0) sm.misc[10] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kRP; ++j) {
        const int rg = tid + NT * j;
        if (rg < nreg && rvv[j] > rcv[j] && (beta >= (uint32_t)kHistBins || rcutv[j] >= (int32_t)beta)) {
          atomicOr(&sm.raw[rg >> 5], 1u << (rg & 31));
          sm.misc[10] = 1;
        }
      }
      __syncthreads();
      if (sm.misc[10]) {
        rescore_raw_regions<NT>(in, r, sm);
        M = prefix(true);
        __syncthreads();
        continue;
      }
    }
    select_winners<NT, SORTED>(src, M, keff, beta, above, sm, out_pos, out_key);
    break;
  }
  __syncthreads();
  return keff;
}

}  // namespace csa2
