// Indexer scoring.  "Compressed Sparse Attention 2 Or CSA2 In Simple Terms" (paper notes):
// each layer's indexer (32 query heads, "Model Setup Numbers Without Jargon") scores every
// visible past entry; the score is the head-weighted sum of per-head dot products.
//
// fp8 path (decode): per 32-key tile one v_mfma_f32_32x32x64_f8f6f4 computes all
// 32 heads x 32 keys x 64 dims (A = the E4M3-quantised query, kept in registers for the
// whole kernel; B = 32 keys streamed from HBM).  Lane l of the result holds key l%32 and
// 16 of the 32 heads, so the head-weighted sum is 16 in-lane FMAs plus one exchange
// with lane l^32.  The kernel is HBM-bound (68 B per key against 8 kFLOP of fp8 MFMA):
// each block streams one contiguous chunk of keys with nontemporal loads (they are read
// once; keeping them out of L2 measured ~15 % faster than cached loads on MI355X) and
// each wave keeps 16 KB in flight.  Optionally it also builds a per-row histogram of the
// scores' top bits for the Top-K select that follows.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "score_dev.hpp"
#include "topk_dev.hpp"

namespace csa2 {

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
constexpr int kPrefetch = 4;  // 32-key tiles in flight per wave (16 x 16 B nontemporal loads per lane)


// The block's candidate list for k_topk_select (LOCAL score kernels; 256 threads, kCols
// columns whose order keys are in s_key, 0 where not visible, and whose first-level
// histogram is in lhist).  Listed: the visible keys in bins above `cut`, where cut is the
// lowest bin such that the bins above it hold at most `cap` keys (-1: every visible key
// fits, the block is complete).  They are written in column order (ballot counts per
// (pass, wave), one exclusive scan), so a full scan's list is sorted by position.
template <int kCols>
__device__ __forceinline__ void list_block_candidates(const uint32_t* lhist, const uint32_t* s_key,
                                                      const int32_t* s_pos, bool cand, int64_t c0, int64_t lim,
                                                      int64_t ncols, const LocalCand& lc, int r, int blk, int nblk,
                                                      uint32_t* s_sh4, uint32_t* s_misc, uint32_t* s_off) {
  constexpr int kPer = kCols / 256;  // column passes
  static_assert(kPer * 4 <= 32, "one wave scans the (pass, wave) counts");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // cap: four times the winners a block of this row holds on average (K spread over the
  // visible columns), plus 32
  const int64_t nvis = cand ? ncols : (lim + 1 < ncols ? lim + 1 : ncols);
  const int64_t cap = list_cap(lc.K, kCols, nvis, kListMargin, lc.stride);
  uint32_t hb[8], local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hb[i] = lhist[8 * tid + i];
    local += hb[i];
  }
  const uint32_t suf = block_suffix<256, 256>(local, s_sh4);  // visible keys in bins >= 8 tid
  if (tid == 0) {
    s_misc[0] = suf;                 // the block's visible keys
    s_misc[1] = 0xFFFFFFFFu;         // cut (none)
    s_misc[2] = suf;                 // listed
  }
  __syncthreads();
  const uint32_t total = s_misc[0];
  if (total > (uint32_t)cap && suf > (uint32_t)cap && suf - local <= (uint32_t)cap) {
    uint32_t acc = suf - local;      // keys in bins above this thread's
    for (int i = 7; i >= 0; --i) {
      if (acc + hb[i] > (uint32_t)cap) {
        s_misc[1] = 8 * tid + i;
        s_misc[2] = acc;
        break;
      }
      acc += hb[i];
    }
  }
  __syncthreads();
  const uint32_t cut = s_misc[1];
  uint64_t bal[kPer];
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const uint32_t key = s_key[p * 256 + tid];
    bal[p] = __ballot(key != 0u && (cut == 0xFFFFFFFFu || hist_bin(key) > cut));
  }
  if (lane < kPer) {
    uint32_t n = 0;
#pragma unroll
    for (int p = 0; p < kPer; ++p)
      if (p == lane) n = (uint32_t)__builtin_popcountll(bal[p]);
    s_off[lane * 4 + wave] = n;
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t v = (lane < kPer * 4) ? s_off[lane] : 0u;
    const uint32_t sfx = wave_suffix(v);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
    if (lane < kPer * 4) s_off[lane] = tot - sfx;
  }
  __syncthreads();
  uint2* creg = lc.cand + ((int64_t)r * nblk + blk) * lc.stride;
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    if ((bal[p] >> lane) & 1ull) {
      const int j = p * 256 + tid;
      const uint32_t slot = s_off[p * 4 + wave] + lanes_below(bal[p]);
      creg[slot] = make_uint2(s_key[j], (uint32_t)(cand ? s_pos[j] : (int32_t)(c0 + j)));
    }
  }
  if (tid == 0) {
    const int64_t o = (int64_t)r * nblk + blk;
    lc.cnt[o] = s_misc[2];
    lc.cut[o] = (int32_t)cut;
    lc.vis[o] = total;
  }
}

// One block streams a contiguous chunk of 4 * TPW 32-key tiles; wave w takes tiles
// w, w+4, ... so that the block's loads sweep the chunk in order.  Order of issue matters
// because the vector-memory counter retires loads in order: the query row and head
// weights are loaded first (one 16-byte load per thread, staged in LDS), then kPrefetch
// key tiles per wave, so the query quantisation overlaps the first key loads.  The tile
// loop is fully unrolled so that every wait names exactly the tile it needs.
// F4: the 4-bit indexer (E2M1 keys, 32 B per key plus the fp32 scale; the query quantised
// to E2M1 per head); the same MFMA takes FP4 operands.
// LOCAL: the block also lists its Top-K candidates for k_topk_select (LocalCand): it keeps
// its scores' order keys in LDS, finds the lowest first-level bin `cut` such that the bins
// above it hold at most `cap` visible scores (cap from K and the row's visible count, about
// four times the winners a block holds on average, plus a margin), and writes those scores'
// (key, position) pairs in column order, their count, the cut and its visible count.  The
// scores themselves are written only when a later step reads them all (lc.store: a Full
// layer's candidate pool takes the block maxima); a selection that cannot trust a block's
// list re-scores that block's columns itself (k_topk_select, with this kernel's arithmetic).
// Launch bound: four waves per SIMD for the full scans (at most 128 VGPRs, so that all four
// blocks a CU gets at 16 x 131072 are resident at once: at 129 VGPRs a quarter of the
// blocks ran as a second wave after the first had streamed); the candidate scans keep two.
template <typename QT, bool CAND, int TPW, bool F4 = false, bool KEEP = false, bool LOCAL = false>
__global__ __launch_bounds__(256, CAND ? 2 : 4) void k_score_fp8(int T, int64_t ncols, const QT* __restrict__ q,
                                                   const float* __restrict__ w, const uint8_t* __restrict__ k8,
                                                   const float* __restrict__ ks, int64_t n_max,
                                                   const int32_t* __restrict__ n_keys,
                                                   const int32_t* __restrict__ q_limit,
                                                   const int32_t* __restrict__ cand, float* __restrict__ scores,
                                                   uint32_t* __restrict__ hist, int key_div, LocalCand lc) {
  constexpr int P = (kPrefetch < TPW) ? kPrefetch : TPW;
  constexpr int kQBytes = 32 * 64 * (int)sizeof(QT);           // 4 KB (bf16) or 8 KB (fp32)
  constexpr int kQLoads = kQBytes / (16 * 256);                 // 16-byte loads per thread
  constexpr int kCols = kScoreWaves * TPW * 32;                 // columns of one block
  __shared__ uint32_t lhist[kHistBins];
  __shared__ __align__(16) QT s_q[32 * 64];
  __shared__ float s_c[32];
  __shared__ uint32_t s_key[LOCAL ? kCols : 1];                // order keys, 0 = not visible
  __shared__ int32_t s_pos[LOCAL && CAND ? kCols : 1];         // candidate positions
  __shared__ uint32_t s_sh4[4];
  __shared__ uint32_t s_misc[4];
  __shared__ uint32_t s_off[32];
  const int r = blockIdx.y, b = r / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5;

  // 1. query row and head weights (issued first)
  v4i qraw[kQLoads];
  const v4i* qsrc = reinterpret_cast<const v4i*>(q + (int64_t)r * 32 * 64);
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) qraw[i] = qsrc[tid + 256 * i];
  const float wv = (tid < 32) ? w[(int64_t)r * 32 + tid] : 0.0f;

  // 2. first key tiles
  const int64_t lim = visible_limit(b, r, n_max, n_keys, q_limit, key_div);
  const int64_t c0 = (int64_t)blockIdx.x * (kScoreWaves * TPW * 32);
  const int64_t c1 = (c0 + kScoreWaves * TPW * 32 < ncols) ? c0 + kScoreWaves * TPW * 32 : ncols;
  constexpr int kKeyBytes = F4 ? 32 : 64;      // bytes per key row
  // fp8 keys: a tile's two 16-byte loads per lane each cover 16 whole keys (one kilobyte,
  // every cache line fully used): load 0 gives lane l chunk l / 16 of key l % 16, load 1 the
  // same chunk of key 16 + l % 16.  One row swap (v_permlane16_swap) then leaves lane
  // (n, half) with bytes 32 half .. 32 half + 31 of key n, the MFMA operand layout.  FP4
  // keys (32 bytes) are read in operand layout directly: lane (n, half) loads 16 bytes at
  // 16 half, and the 64 lanes cover the tile's kilobyte whole.
  const uint8_t* kb = k8 + (int64_t)b * n_max * kKeyBytes + (F4 ? half * 16 : 16 * (lane >> 4));
  const float* ksb = ks + (int64_t)b * n_max;
  const int32_t* crow = CAND ? cand + (int64_t)r * ncols : nullptr;
  // candidate positions of all this wave's tiles, loaded together up front: a position
  // loaded just before the key load that needs it would make every tile wait for all the
  // loads issued before it (the vector-memory counter retires in order)
  // (unconditional loads from a clamped column, masked afterwards: a load behind a branch
  // is waited for before the branch joins)
  // (fp8 keys also need the positions of the two keys this lane loads: cpos of key
  // lane % 16 and 16 + lane % 16; the lane's own key lane % 32 is one of them)
  int32_t cpos[CAND ? TPW : 1], cpos_lo[CAND && !F4 ? TPW : 1], cpos_hi[CAND && !F4 ? TPW : 1];
  if (CAND) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t t0 = c0 + (int64_t)(wave + kScoreWaves * i) * 32;
      if constexpr (F4) {
        const int64_t col = t0 + (lane & 31);
        cpos[i] = crow[col < c1 ? col : c1 - 1];
      } else {
        const int64_t cl = t0 + (lane & 15), ch = cl + 16;
        cpos_lo[i] = crow[cl < c1 ? cl : c1 - 1];
        cpos_hi[i] = crow[ch < c1 ? ch : c1 - 1];
      }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t t0 = c0 + (int64_t)(wave + kScoreWaves * i) * 32;
      if constexpr (F4) {
        if (t0 + (lane & 31) >= c1) cpos[i] = -1;
      } else {
        if (t0 + (lane & 15) >= c1) cpos_lo[i] = -1;
        if (t0 + (lane & 15) + 16 >= c1) cpos_hi[i] = -1;
        cpos[i] = (lane & 16) ? cpos_hi[i] : cpos_lo[i];
      }
    }
  }
  v4i ka[P], kc[P];
  float skv[P];
  bool vis[P];
  // the row of column `col` when it is visible, else row 0 (always valid; masked later):
  // branch-free loads
  auto row_of = [&](int64_t col, int32_t cp, bool& v) -> int64_t {
    int64_t row = -1;
    if (col < c1) row = CAND ? (int64_t)cp : col;
    v = row >= 0 && row <= lim;
    return v ? row : 0;
  };
  auto issue = [&](int i, int slot) {
    const int64_t t0 = c0 + (int64_t)(wave + kScoreWaves * i) * 32;
    const int64_t rr = row_of(t0 + (lane & 31), CAND ? cpos[i] : 0, vis[slot]);
    const v4i* src;
    const v4i* src2 = nullptr;
    if constexpr (F4) {
      src = reinterpret_cast<const v4i*>(kb + rr * kKeyBytes);
    } else {
      bool vl, vh;
      const int64_t rl = row_of(t0 + (lane & 15), CAND ? cpos_lo[i] : 0, vl);
      const int64_t rh = row_of(t0 + (lane & 15) + 16, CAND ? cpos_hi[i] : 0, vh);
      src = reinterpret_cast<const v4i*>(kb + rl * kKeyBytes);
      src2 = reinterpret_cast<const v4i*>(kb + rh * kKeyBytes);
    }
    if (KEEP) {  // a later layer rescans these keys: ordinary loads, which leave them in the MALL
      ka[slot] = *src;
      kc[slot] = F4 ? (v4i){0, 0, 0, 0} : *src2;
      skv[slot] = ksb[rr];
    } else {
      ka[slot] = __builtin_nontemporal_load(src);
      if (F4) kc[slot] = (v4i){0, 0, 0, 0};
      else kc[slot] = __builtin_nontemporal_load(src2);
      skv[slot] = __builtin_nontemporal_load(ksb + rr);
    }
  };
#pragma unroll
  for (int i = 0; i < P; ++i) issue(i, i);

  // 3. quantise the query from LDS while the key tiles are in flight
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) reinterpret_cast<v4i*>(s_q)[tid + 256 * i] = qraw[i];
  if (hist || LOCAL)
    for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0;
  __syncthreads();
  float sq;
  const v8i A = F4 ? quantize_query_operand_fp4(s_q, lane, sq) : quantize_query_operand<QT, CAND>(s_q, lane, sq);
  if (wave == 0 && lane < 32) s_c[lane] = sq;
  __syncthreads();
  if (tid < 32) s_c[tid] = wv * s_c[tid];
  __syncthreads();
  float cvec[16];
  tile_head_factors(s_c, half, cvec);
  float* srow = scores + (int64_t)r * ncols;

  // 4. stream the tiles
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int u = i % P;
    const int64_t col = c0 + (int64_t)(wave + kScoreWaves * i) * 32 + (lane & 31);
    v8i B;
    if constexpr (F4) {
      B[0] = ka[u][0]; B[1] = ka[u][1]; B[2] = ka[u][2]; B[3] = ka[u][3];
      B[4] = 0; B[5] = 0; B[6] = 0; B[7] = 0;
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const auto sw = __builtin_amdgcn_permlane16_swap((uint32_t)ka[u][d], (uint32_t)kc[u][d], false, false);
        B[d] = (int)sw[0];
        B[4 + d] = (int)sw[1];
      }
    }
    const bool v = vis[u];
    const float skl = skv[u];
    if (i + P < TPW) issue(i + P, u);
    const float sc = tile_score<F4>(A, B, cvec, v, skl);
    if (LOCAL) {
      const int j = (wave + kScoreWaves * i) * 32 + (lane & 31);  // column within the block
      if (half == 0) {
        const bool vv = col < c1 && visible(sc);
        if (lc.store && col < c1) __builtin_nontemporal_store(sc, srow + col);
        s_key[j] = vv ? order_key(sc) : 0u;
        if (CAND) s_pos[j] = cpos[i];
        if (vv) atomicAdd(&lhist[hist_bin(order_key(sc))], 1u);
      }
    } else if (half == 0 && col < c1) {
      srow[col] = sc;
      if (hist && visible(sc)) atomicAdd(&lhist[hist_bin(order_key(sc))], 1u);
    }
  }
  if (LOCAL) {
    __syncthreads();
    list_block_candidates<kCols>(lhist, s_key, s_pos, CAND, c0, lim, ncols, lc, r, (int)blockIdx.x, (int)gridDim.x,
                                 s_sh4, s_misc, s_off);
  } else if (hist) {
    __syncthreads();
    for (int i = tid; i < kHistBins; i += 256) {
      const uint32_t vv = lhist[i];
      if (vv) atomicAdd(&hist[(int64_t)r * kHistBins + i], vv);
    }
  }
}

// ------------------------------------------------------------------ fp8 path, many rows
// Chunked prefill scores many query rows of one sequence against the same keys: a dense
// fp8 contraction (rows x heads) x (keys), where re-streaming the keys once per row (as
// the decode kernel does) would move ~T times the key bytes.  Here a block takes a tile
// of kRowTile rows x (4 waves x NKT x 32) keys: the rows' E4M3 operands (quantised once
// per row by k_quant_query) sit in LDS, each wave keeps 4 key tiles in registers and
// runs all rows of the tile against them, so every key tile is read once per row tile.
// The per-row first-level Top-K histogram is kept in LDS with 16-bit counters packed in
// pairs (a block adds at most 128 x NKT <= 4096 to one bin of one row).
constexpr int kRowTile = 8;  // rows per tile of the many-row path (minimum T)

// q [R][32][64] -> E4M3 codes q8 [R][32][64] and c [R][32] = w * sq, with sq = absmax/448
// over the head's 64 values: the same arithmetic as quantize_query_operand.
template <typename QT>
__global__ __launch_bounds__(256) void k_quant_query(const QT* __restrict__ q, const float* __restrict__ w,
                                                     uint8_t* __restrict__ q8, float* __restrict__ c) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int h = tid >> 3, d0 = (tid & 7) * 8;  // 8 lanes per head, 8 dims per lane
  const QT* p = q + ((int64_t)r * 32 + h) * 64 + d0;
  float v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = load_as_f32(p + i);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  const float sq = amax / 448.0f;
  const ExactQuotient div(sq);
  const uint32_t keep = sq != 0.0f ? ~0u : 0u;
  uint32_t wd[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) wd[i >> 2] |= e4m3_encode(div(v[i])) << (8 * (i & 3));
  wd[0] &= keep;
  wd[1] &= keep;
  *reinterpret_cast<uint2*>(q8 + ((int64_t)r * 32 + h) * 64 + d0) = make_uint2(wd[0], wd[1]);
  if ((tid & 7) == 0) c[(int64_t)r * 32 + h] = w[(int64_t)r * 32 + h] * sq;
}

// TT rows per tile, NW waves per block, NKT key tiles of 32 per wave (groups of 4 tiles;
// with DB the next group's keys are loaded while the current one runs).
template <int TT, int NW, int NKT, bool DB>
__global__ __launch_bounds__(64 * NW) void k_score_fp8_rows(int T, int64_t ncols, const uint8_t* __restrict__ q8,
                                                            const float* __restrict__ cst,
                                                            const uint8_t* __restrict__ k8,
                                                            const float* __restrict__ ks, int64_t n_max,
                                                            const int32_t* __restrict__ n_keys,
                                                            const int32_t* __restrict__ q_limit,
                                                            float* __restrict__ scores, uint32_t* __restrict__ hist) {
  static_assert(NKT % 4 == 0 && (!DB || (NKT / 4) % 2 == 0), "key tiles come in (pairs of) groups of 4");
  constexpr int NT = 64 * NW;
  constexpr int kQRow = 80;  // bytes per head row in LDS: 64 + 16 padding, so that the 16-byte
                             // operand reads of 16 lanes fall on distinct banks
  __shared__ __align__(16) uint8_t s_q8[TT * 32 * kQRow];
  __shared__ __align__(16) float s_c[TT * 32];
  __shared__ int64_t s_lim[TT];
  __shared__ uint32_t s_h[TT * kHistBins / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  // grid x = row tiles (fastest), y = key ranges: the blocks in flight at once share a few
  // key ranges, which stay in L2 while every row tile reads them
  const int tiles_per_seq = (T + TT - 1) / TT;
  const int b = blockIdx.x / tiles_per_seq;
  const int t0 = (blockIdx.x % tiles_per_seq) * TT;
  const int nrows = (T - t0 < TT) ? T - t0 : TT;  // uniform per block
  const int64_t r0 = (int64_t)b * T + t0;
  const int64_t c0 = (int64_t)blockIdx.y * (NW * NKT * 32);

  // rows' operands and limits into LDS (rows past T: zero operands, never stored)
  {
    const uint4* src = reinterpret_cast<const uint4*>(q8 + r0 * 32 * 64);
    for (int i = tid; i < TT * 32 * 64 / 16; i += NT) {
      const int hr = i >> 2, part = i & 3;  // head row (t * 32 + h), 16-byte piece
      reinterpret_cast<uint4*>(s_q8 + hr * kQRow)[part] =
          (i < nrows * 32 * 64 / 16) ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int i = tid; i < TT * 32; i += NT) s_c[i] = (i < nrows * 32) ? cst[r0 * 32 + i] : 0.0f;
    if (tid < TT && tid >= nrows) s_lim[tid] = -1;
    if (tid < nrows) {
      int64_t nk = n_keys[b];
      int64_t lim = (nk < n_max ? nk : n_max) - 1;
      if (q_limit && q_limit[r0 + tid] < lim) lim = q_limit[r0 + tid];
      s_lim[tid] = lim;
    }
    if (hist)
      for (int i = tid; i < TT * kHistBins / 2; i += NT) s_h[i] = 0;
  }
  __syncthreads();

  const uint8_t* kb = k8 + (int64_t)b * n_max * 64 + half * 32;
  const float* ksb = ks + (int64_t)b * n_max;
  struct KeyGroup {
    v8i B[4];
    float sk[4];
    int64_t col[4];
  };
  auto load_group = [&](int g, KeyGroup& kg) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kg.col[u] = c0 + (int64_t)(wave + NW * (4 * g + u)) * 32 + (lane & 31);
      const int64_t rr = kg.col[u] < ncols ? kg.col[u] : 0;  // clamped, masked below
      const v4i* src = reinterpret_cast<const v4i*>(kb + rr * 64);
      const v4i x0 = src[0], x1 = src[1];
      kg.B[u][0] = x0[0]; kg.B[u][1] = x0[1]; kg.B[u][2] = x0[2]; kg.B[u][3] = x0[3];
      kg.B[u][4] = x1[0]; kg.B[u][5] = x1[1]; kg.B[u][6] = x1[2]; kg.B[u][7] = x1[3];
      kg.sk[u] = ksb[rr];
    }
  };
  auto run_group = [&](const KeyGroup& kg) {
    for (int t = 0; t < nrows; ++t) {
      const uint4* qa = reinterpret_cast<const uint4*>(s_q8 + (t * 32 + (lane & 31)) * kQRow + half * 32);
      const uint4 a0 = qa[0], a1 = qa[1];
      v8i A;
      A[0] = a0.x; A[1] = a0.y; A[2] = a0.z; A[3] = a0.w; A[4] = a1.x; A[5] = a1.y; A[6] = a1.z; A[7] = a1.w;
      float cvec[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 cc = *reinterpret_cast<const float4*>(&s_c[t * 32 + 8 * j + 4 * half]);
        cvec[4 * j] = cc.x; cvec[4 * j + 1] = cc.y; cvec[4 * j + 2] = cc.z; cvec[4 * j + 3] = cc.w;
      }
      const int64_t lim = s_lim[t];
      float* srow = scores + (r0 + t) * ncols;
      // the four contractions first (independent accumulators, so they issue back to
      // back), then their epilogues
      v16f acc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u] = (v16f){};
        acc[u] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, kg.B[u], acc[u], 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) part = fmaf(cvec[j], acc[u][j], part);
        const float total = part + swap_halves(part);
        const float sc = (kg.col[u] <= lim) ? total * kg.sk[u] : kNegInf;
        if (half == 0 && kg.col[u] < ncols) {
          srow[kg.col[u]] = sc;
          if (hist && visible(sc)) {
            const uint32_t bin = hist_bin(order_key(sc));
            atomicAdd(&s_h[t * (kHistBins / 2) + (bin >> 1)], 1u << (16 * (bin & 1)));
          }
        }
      }
    }
  };
  if (DB) {
    KeyGroup g0, g1;
    load_group(0, g0);
    for (int g = 0; g < NKT / 4; g += 2) {
      load_group(g + 1, g1);
      run_group(g0);
      if (g + 2 < NKT / 4) load_group(g + 2, g0);
      run_group(g1);
    }
  } else {
    for (int g = 0; g < NKT / 4; ++g) {
      KeyGroup kg;
      load_group(g, kg);
      run_group(kg);
    }
  }
  if (hist) {
    __syncthreads();
    for (int i = tid; i < nrows * (kHistBins / 2); i += NT) {
      const uint32_t v = s_h[i];
      if (v) {
        const int t = i / (kHistBins / 2), bp = i % (kHistBins / 2);
        uint32_t* hrow = hist + (r0 + t) * kHistBins;
        if (v & 0xFFFFu) atomicAdd(&hrow[2 * bp], v & 0xFFFFu);
        if (v >> 16) atomicAdd(&hrow[2 * bp + 1], v >> 16);
      }
    }
  }
}

// The many-row kernel with candidate lists instead of stored scores (chunked prefill's
// Top-K): a block takes TT rows and RPB consecutive regions of NW x NKT x 32 columns, one
// region at a time.  Per region it scores the TT rows, keeping each score in a register
// (lane half h keeps tiles u with u % 2 == h: both halves hold a tile's totals after the
// half exchange), and counts the rows' first-level histograms in LDS; then per row (rows
// dealt to the waves) the cut, the lowest bin such that the bins above hold at most `cap`
// visible scores (cap as for the decode lists with a smaller margin, at most lc.stride slots), and the listing of
// those scores' (key, position) pairs in column order (per-tile ballot counts, one wave scan
// per row) into the row's region of lc, with its count, cut and visible count.  Launch
// bound: four waves per SIMD (at most 128 VGPRs; the two region variants would take 130).
template <int TT, int NW, int NKT, int RPB>
__global__ __launch_bounds__(64 * NW, 4) void k_score_fp8_rows_list(int T, int64_t ncols, int nblk,
                                                                 const uint8_t* __restrict__ q8,
                                                                 const float* __restrict__ cst,
                                                                 const uint8_t* __restrict__ k8,
                                                                 const float* __restrict__ ks, int64_t n_max,
                                                                 const int32_t* __restrict__ n_keys,
                                                                 const int32_t* __restrict__ q_limit, LocalCand lc) {
  static_assert(NKT % 4 == 0, "key tiles come in groups of 4");
  static_assert(TT % NW == 0, "whole rows per wave in the cut search");
  constexpr int kRPW = TT / NW;          // rows per wave in the cut search
  constexpr int NT = 64 * NW;
  constexpr int kCols = NW * NKT * 32;   // columns of a region
  constexpr int kTiles = NW * NKT;       // 32-column tiles of a region
  static_assert(kCols < 65536, "16-bit histogram halves");
  static_assert(kTiles <= 64, "one wave scans a row's tile counts");
  constexpr int kKept = NKT / 2;         // scores kept per lane and row
  constexpr int kQRow = 80;
  __shared__ __align__(16) uint8_t s_q8[TT * 32 * kQRow];
  __shared__ __align__(16) float s_c[TT * 32];
  __shared__ int64_t s_lim[TT];
  __shared__ uint32_t s_cap[TT];           // the rows' list caps (once per block: a 64-bit division)
  __shared__ __align__(16) uint32_t s_h[TT * kHistBins / 2];
  __shared__ uint32_t s_cnt[TT * kTiles];  // listed per (row, tile), then their exclusive offsets
  __shared__ uint32_t s_cut[TT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int tiles_per_seq = (T + TT - 1) / TT;
  const int b = blockIdx.x / tiles_per_seq;
  const int t0 = (blockIdx.x % tiles_per_seq) * TT;
  const int nrows = (T - t0 < TT) ? T - t0 : TT;
  const int64_t r0 = (int64_t)b * T + t0;
  {
    const uint4* src = reinterpret_cast<const uint4*>(q8 + r0 * 32 * 64);
    for (int i = tid; i < TT * 32 * 64 / 16; i += NT) {
      const int hr = i >> 2, part = i & 3;
      reinterpret_cast<uint4*>(s_q8 + hr * kQRow)[part] =
          (i < nrows * 32 * 64 / 16) ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int i = tid; i < TT * 32; i += NT) s_c[i] = (i < nrows * 32) ? cst[r0 * 32 + i] : 0.0f;
    if (tid < TT && tid >= nrows) {
      s_lim[tid] = -1;
      s_cap[tid] = 0;
    }
    if (tid < nrows) {
      int64_t nk = n_keys[b];
      int64_t lim = (nk < n_max ? nk : n_max) - 1;
      if (q_limit && q_limit[r0 + tid] < lim) lim = q_limit[r0 + tid];
      s_lim[tid] = lim;
      const int64_t nvis = lim + 1 < ncols ? lim + 1 : ncols;
      s_cap[tid] = (uint32_t)list_cap(lc.K, kCols, nvis, kRowsListMargin, lc.stride);
    }
  }
  // whole-line key loads (as in k_score_fp8): load 0 gives lane l chunk l / 16 of key l % 16,
  // load 1 the same chunk of key 16 + l % 16; one row swap makes the MFMA operand
  const uint8_t* kb = k8 + (int64_t)b * n_max * 64 + 16 * (lane >> 4);
  const float* ksb = ks + (int64_t)b * n_max;

  for (int rg = 0; rg < RPB; ++rg) {
    const int blk = blockIdx.y * RPB + rg;
    if (blk >= nblk) break;  // uniform
    const int64_t c0 = (int64_t)blk * kCols;
    for (int i = tid; i < TT * kHistBins / 2; i += NT) s_h[i] = 0;
    __syncthreads();

    // every column of the region visible to every row of the block (all regions but the
    // causal tail and the last): no clamped addresses, no visibility tests
    bool full = c0 + kCols <= ncols;
#pragma unroll
    for (int t = 0; t < TT; ++t) full = full && c0 + kCols - 1 <= s_lim[t];
    // kept order keys (0: not visible, never the key of a visible score): slot k of lane
    // (half h, key l) is tile wave + NW (4 (k / 2) + 2 (k % 2) + h), column l of it
    uint32_t keep[TT][kKept];
    auto scan = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      const uint8_t* kw = kb + (c0 + wave * 32 + (lane & 15)) * 64;  // FULL: this lane's first key
      const float* skw = ksb + c0 + wave * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < NKT / 4; ++g) {
        v8i B[4];
        float sk[4];
        int64_t col[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t tbase = c0 + (int64_t)(wave + NW * (4 * g + u)) * 32;
          col[u] = tbase + (lane & 31);
          v4i x0, x1;
          if (FULL) {
            const uint8_t* p = kw + NW * (4 * g + u) * 32 * 64;
            x0 = *reinterpret_cast<const v4i*>(p);
            x1 = *reinterpret_cast<const v4i*>(p + 16 * 64);
            sk[u] = skw[NW * (4 * g + u) * 32];
          } else {
            const int64_t rr = col[u] < ncols ? col[u] : 0;  // clamped, masked below
            const int64_t rl = tbase + (lane & 15) < ncols ? tbase + (lane & 15) : 0;
            const int64_t rh = tbase + (lane & 15) + 16 < ncols ? tbase + (lane & 15) + 16 : 0;
            x0 = *reinterpret_cast<const v4i*>(kb + rl * 64);
            x1 = *reinterpret_cast<const v4i*>(kb + rh * 64);
            sk[u] = ksb[rr];
          }
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const auto sw = __builtin_amdgcn_permlane16_swap((uint32_t)x0[d], (uint32_t)x1[d], false, false);
            B[u][d] = (int)sw[0];
            B[u][4 + d] = (int)sw[1];
          }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const uint4* qa = reinterpret_cast<const uint4*>(s_q8 + (t * 32 + (lane & 31)) * kQRow + half * 32);
          const uint4 a0 = qa[0], a1 = qa[1];
          const v8i A = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          float cvec[16];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 cc = *reinterpret_cast<const float4*>(&s_c[t * 32 + 8 * j + 4 * half]);
            cvec[4 * j] = cc.x; cvec[4 * j + 1] = cc.y; cvec[4 * j + 2] = cc.z; cvec[4 * j + 3] = cc.w;
          }
          const int64_t lim = s_lim[t];
          float sc[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)  // columns past lim (incl. past ncols): -inf
            sc[u] = tile_score<false>(A, B[u], cvec, FULL || (col[u] <= lim && col[u] < ncols), sk[u]);
          // each half keeps (and counts in the row's histogram) its own two of the 4 tiles:
          // one atomic per lane and kept score, no lane idle
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float kv = half ? sc[2 * p + 1] : sc[2 * p];
            const uint32_t key = visible(kv) ? order_key(kv) : 0u;
            keep[t][2 * g + p] = key;
            const uint32_t bin = hist_bin(key);
            atomicAdd(&s_h[t * (kHistBins / 2) + (bin >> 1)], key ? 1u << (16 * (bin & 1)) : 0u);
          }
        }
      }
    };
    if (full)  // uniform
      scan(std::true_type{});
    else
      scan(std::false_type{});
    __syncthreads();

    // the cut of rows wave + NW rr: lane l holds bins 32 l .. 32 l + 31
#pragma unroll
    for (int rr = 0; rr < kRPW; ++rr) {
      const int t = wave + NW * rr;
      const uint32_t cap = s_cap[t];
      // the 32 bins as 16 packed pairs: a row has at most kCols (< 2^16) visible scores, so
      // the pairs add as whole words without a carry between the halves
      uint32_t pairs = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(&s_h[t * (kHistBins / 2) + 16 * lane + 4 * q]);
        pairs += w4.x + w4.y + w4.z + w4.w;
      }
      const uint32_t local = (pairs & 0xFFFFu) + (pairs >> 16);
      const uint32_t suf = wave_suffix(local);  // visible scores in bins >= 32 lane
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)suf, 0);
      uint32_t cut = 0xFFFFFFFFu, listed = total;
      const uint32_t need = (uint32_t)cap + 1;
      if (total >= need) {  // uniform: the cut bin holds the (cap + 1)-th largest
        const uint64_t grp = __ballot(suf >= need && suf - local < need);
        const int gl = __builtin_ctzll(grp);
        const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)(suf - local), gl);
        const uint32_t w2 = s_h[t * (kHistBins / 2) + 16 * gl + ((lane & 31) >> 1)];
        const uint32_t hvv = lane < 32 ? ((lane & 1) ? w2 >> 16 : w2 & 0xFFFFu) : 0u;
        const uint32_t s2 = base + wave_suffix(hvv);
        const uint64_t hit = __ballot(lane < 32 && s2 >= need && s2 - hvv < need);
        const int hl = __builtin_ctzll(hit);
        cut = (uint32_t)(32 * gl + hl);
        listed = (uint32_t)__builtin_amdgcn_readlane((int)(s2 - hvv), hl);
      }
      if (lane == 0) {
        s_cut[t] = cut;
        if (t < nrows) {
          const int64_t o = (r0 + t) * nblk + blk;
          lc.cnt[o] = listed;
          lc.cut[o] = (int32_t)cut;
          lc.vis[o] = total;
        }
      }
    }
    __syncthreads();
    // per (row, tile) counts of the listed scores: kept slot k of lane (h, key) is tile
    // wave + NW (4 (k / 2) + 2 (k % 2) + h); one ballot covers both halves' tiles, and the
    // ballots (wave-uniform) are kept for the listing
    uint64_t bals[TT][kKept];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint32_t cut = s_cut[t];
#pragma unroll
      for (int k = 0; k < kKept; ++k) {
        const uint32_t key = keep[t][k];
        bals[t][k] = __ballot(key != 0u && (cut == 0xFFFFFFFFu || hist_bin(key) > cut));
        if (lane == 0) {
          const int tile0 = wave + NW * (4 * (k >> 1) + 2 * (k & 1));
          s_cnt[t * kTiles + tile0] = (uint32_t)__builtin_popcountll(bals[t][k] & 0xFFFFFFFFull);
          s_cnt[t * kTiles + tile0 + NW] = (uint32_t)__builtin_popcountll(bals[t][k] >> 32);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < kRPW; ++rr) {  // exclusive offsets in tile (= column) order
      const int t = wave + NW * rr;
      const uint32_t v = lane < kTiles ? s_cnt[t * kTiles + lane] : 0u;
      const uint32_t sfx = wave_suffix(v);
      const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)sfx, 0);
      if (lane < kTiles) s_cnt[t * kTiles + lane] = tot - sfx;
    }
    __syncthreads();
    // the listing: a listed score's slot is its tile's offset plus the listed lanes of its
    // half below it (columns < 2^31, so positions are 32-bit)
    const uint32_t col0 = (uint32_t)c0 + (uint32_t)(wave * 32 + (lane & 31));
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= nrows) break;  // uniform
      uint2* creg = lc.cand + ((r0 + t) * nblk + blk) * lc.stride;
#pragma unroll
      for (int k = 0; k < kKept; ++k) {
        const uint64_t bal = bals[t][k];
        if (bal == 0) continue;  // uniform
        if ((bal >> lane) & 1ull) {
          const int tile = NW * (4 * (k >> 1) + 2 * (k & 1) + half);  // past this wave's first
          const uint32_t below = half ? __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), 0u)
                                      : __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u);
          const uint32_t slot = s_cnt[t * kTiles + wave + tile] + below;
          creg[slot] = make_uint2(keep[t][k], col0 + (uint32_t)tile * 32);
        }
      }
    }
  }
}

template <int TT, int NW, int NKT, bool DB>
static void launch_rows(const ScoreArgs& a, const uint8_t* q8, const float* cst, hipStream_t st) {
  const int64_t cpb = NW * NKT * 32;
  dim3 g((unsigned)(a.B * ((a.T + TT - 1) / TT)), (unsigned)((a.ncols + cpb - 1) / cpb));
  hipLaunchKernelGGL((k_score_fp8_rows<TT, NW, NKT, DB>), g, dim3(64 * NW), 0, st, a.T, a.ncols, q8, cst,
                     (const uint8_t*)a.k, a.k_scale, a.n_max, a.n_keys, a.q_limit, a.scores, a.hist);
}

// chunked prefill with candidate lists: 8 rows x one region of 1024 columns per block (measured
// fastest: more regions per block, or wider regions, ran slower)
constexpr int kRowsListWaves = 8, kRowsListTiles = 4, kRowsListRegions = 1;
int rows_list_cols() { return kRowsListWaves * kRowsListTiles * 32; }

int score_rows_tiled(const ScoreArgs& a) {
  return a.prec == 1 && a.cand == nullptr && a.key_div == 1 && a.T >= kRowTile && a.qstage != nullptr;
}

int score_cols_per_block(int64_t rows, int64_t ncols) {
  // tiles per wave: the largest of 16 / 8 / 4 / 2 that still gives >= 512 blocks (two per
  // CU), so that long scans stream 2048 keys per block and short ones (few rows, small N)
  // spread over the chip
  for (int tpw = 16; tpw > 2; tpw >>= 1) {
    const int64_t cpb = kScoreWaves * tpw * 32;
    if (rows * ((ncols + cpb - 1) / cpb) >= 512) return (int)cpb;
  }
  return kScoreWaves * 2 * 32;
}

template <typename QT, bool CAND, int TPW, bool F4>
static void launch_fp8(const ScoreArgs& a, hipStream_t st) {
  const int cpb = kScoreWaves * TPW * 32;
  dim3 g((unsigned)((a.ncols + cpb - 1) / cpb), a.B * a.T);
#define CSA2_SCORE(KEEP, LOC)                                                                                     \
  hipLaunchKernelGGL((k_score_fp8<QT, CAND, TPW, F4, KEEP, LOC>), g, dim3(256), 0, st, a.T, a.ncols, (const QT*)a.q, \
                     a.w, (const uint8_t*)a.k, a.k_scale, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist,   \
                     a.key_div, a.lc)
  if (a.local) {
    if constexpr (!CAND) {
      if (a.keep) {
        CSA2_SCORE(true, true);
        return;
      }
    }
    CSA2_SCORE(false, true);
    return;
  }
  if constexpr (!CAND) {
    if (a.keep) {
      CSA2_SCORE(true, false);
      return;
    }
  }
  CSA2_SCORE(false, false);
#undef CSA2_SCORE
}

template <typename QT, bool CAND, bool F4>
static void launch_fp8_tpw(const ScoreArgs& a, hipStream_t st) {
  const int cpb = score_cols_per_block((int64_t)a.B * a.T, a.ncols);
  if (cpb == kScoreWaves * 16 * 32) launch_fp8<QT, CAND, 16, F4>(a, st);
  else if (cpb == kScoreWaves * 8 * 32) launch_fp8<QT, CAND, 8, F4>(a, st);
  else if (cpb == kScoreWaves * 4 * 32) launch_fp8<QT, CAND, 4, F4>(a, st);
  else launch_fp8<QT, CAND, 2, F4>(a, st);
}

template <typename QT>
static void launch_lowbit(const ScoreArgs& a, hipStream_t st) {
  if (a.prec == 2) {
    if (a.cand) launch_fp8_tpw<QT, true, true>(a, st); else launch_fp8_tpw<QT, false, true>(a, st);
  } else {
    if (a.cand) launch_fp8_tpw<QT, true, false>(a, st); else launch_fp8_tpw<QT, false, false>(a, st);
  }
}

int launch_score(const ScoreArgs& a, hipStream_t st) {
  const int R = a.B * a.T;
  if (score_rows_tiled(a)) {
    uint8_t* q8 = a.qstage;
    float* cst = reinterpret_cast<float*>(a.qstage + (size_t)R * 32 * 64);
    if (a.q_bf16)
      hipLaunchKernelGGL(k_quant_query<uint16_t>, dim3(R), dim3(256), 0, st, (const uint16_t*)a.q, a.w, q8, cst);
    else
      hipLaunchKernelGGL(k_quant_query<float>, dim3(R), dim3(256), 0, st, (const float*)a.q, a.w, q8, cst);
    if (a.local) {
      const int nblk = (int)((a.ncols + rows_list_cols() - 1) / rows_list_cols());
      const dim3 g((unsigned)(a.B * ((a.T + kRowTile - 1) / kRowTile)),
                   (unsigned)((nblk + kRowsListRegions - 1) / kRowsListRegions));
      hipLaunchKernelGGL((k_score_fp8_rows_list<kRowTile, kRowsListWaves, kRowsListTiles, kRowsListRegions>), g,
                         dim3(64 * kRowsListWaves), 0, st, a.T, a.ncols, nblk, q8, cst, (const uint8_t*)a.k,
                         a.k_scale, a.n_max, a.n_keys, a.q_limit, a.lc);
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    // 8 rows x 4096 keys per block, single-buffered key groups: the variant measured
    // fastest (double buffering or 16-row tiles cost occupancy and ran slower)
    launch_rows<kRowTile, 4, 32, false>(a, q8, cst, st);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (a.prec == 0) {
    dim3 g((unsigned)((a.ncols + 255) / 256), R);
    const size_t sh = sizeof(float) * ((size_t)a.H * a.dk + a.H);
    if (a.cand)
      hipLaunchKernelGGL(k_score_f32<true>, g, dim3(256), sh, st, a.T, a.H, a.dk, a.ncols, (const float*)a.q, a.w,
                         (const float*)a.k, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist, a.key_div);
    else
      hipLaunchKernelGGL(k_score_f32<false>, g, dim3(256), sh, st, a.T, a.H, a.dk, a.ncols, (const float*)a.q, a.w,
                         (const float*)a.k, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist, a.key_div);
  } else if (a.q_bf16) {
    launch_lowbit<uint16_t>(a, st);
  } else {
    launch_lowbit<float>(a, st);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
