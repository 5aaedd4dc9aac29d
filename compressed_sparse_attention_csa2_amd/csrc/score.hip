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
constexpr int kPrefetch = 4;  // 32-key tiles in flight per wave (16 x 16 B nontemporal loads per lane)

typedef int v4i __attribute__((ext_vector_type(4)));

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

// One block streams a contiguous chunk of 4 * TPW 32-key tiles; wave w takes tiles
// w, w+4, ... so that the block's loads sweep the chunk in order.  Order of issue matters
// because the vector-memory counter retires loads in order: the query row and head
// weights are loaded first (one 16-byte load per thread, staged in LDS), then kPrefetch
// key tiles per wave, so the query quantisation overlaps the first key loads.  The tile
// loop is fully unrolled so that every wait names exactly the tile it needs.
// F4: the 4-bit indexer (E2M1 keys, 32 B per key plus the fp32 scale; the query quantised
// to E2M1 per head); the same MFMA takes FP4 operands.
template <typename QT, bool CAND, int TPW, bool F4 = false, bool KEEP = false>
__global__ __launch_bounds__(256) void k_score_fp8(int T, int64_t ncols, const QT* __restrict__ q,
                                                   const float* __restrict__ w, const uint8_t* __restrict__ k8,
                                                   const float* __restrict__ ks, int64_t n_max,
                                                   const int32_t* __restrict__ n_keys,
                                                   const int32_t* __restrict__ q_limit,
                                                   const int32_t* __restrict__ cand, float* __restrict__ scores,
                                                   uint32_t* __restrict__ hist, int key_div) {
  constexpr int P = (kPrefetch < TPW) ? kPrefetch : TPW;
  constexpr int kQBytes = 32 * 64 * (int)sizeof(QT);           // 4 KB (bf16) or 8 KB (fp32)
  constexpr int kQLoads = kQBytes / (16 * 256);                 // 16-byte loads per thread
  __shared__ uint32_t lhist[kHistBins];
  __shared__ __align__(16) QT s_q[32 * 64];
  __shared__ float s_c[32];
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
  const uint8_t* kb = k8 + (int64_t)b * n_max * kKeyBytes + half * (kKeyBytes / 2);
  const float* ksb = ks + (int64_t)b * n_max;
  const int32_t* crow = CAND ? cand + (int64_t)r * ncols : nullptr;
  // candidate positions of all this wave's tiles, loaded together up front: a position
  // loaded just before the key load that needs it would make every tile wait for all the
  // loads issued before it (the vector-memory counter retires in order)
  // (unconditional loads from a clamped column, masked afterwards: a load behind a branch
  // is waited for before the branch joins)
  int32_t cpos[CAND ? TPW : 1];
  if (CAND) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t col = c0 + (int64_t)(wave + kScoreWaves * i) * 32 + (lane & 31);
      cpos[i] = crow[col < c1 ? col : c1 - 1];
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int64_t col = c0 + (int64_t)(wave + kScoreWaves * i) * 32 + (lane & 31);
      if (col >= c1) cpos[i] = -1;
    }
  }
  v4i ka[P], kc[P];
  float skv[P];
  bool vis[P];
  auto issue = [&](int i, int slot) {
    const int64_t col = c0 + (int64_t)(wave + kScoreWaves * i) * 32 + (lane & 31);
    int64_t row = -1;
    if (col < c1) row = CAND ? (int64_t)cpos[i] : col;
    vis[slot] = row >= 0 && row <= lim;
    // branch-free: invisible columns read row 0 (always valid) and are masked later
    const int64_t rr = vis[slot] ? row : 0;
    const v4i* src = reinterpret_cast<const v4i*>(kb + rr * kKeyBytes);
    if (KEEP) {  // a later layer rescans these keys: ordinary loads, which leave them in the MALL
      ka[slot] = *src;
      kc[slot] = F4 ? (v4i){0, 0, 0, 0} : *(src + 1);
      skv[slot] = ksb[rr];
    } else {
      ka[slot] = __builtin_nontemporal_load(src);
      if (F4) kc[slot] = (v4i){0, 0, 0, 0};
      else kc[slot] = __builtin_nontemporal_load(src + 1);
      skv[slot] = __builtin_nontemporal_load(ksb + rr);
    }
  };
#pragma unroll
  for (int i = 0; i < P; ++i) issue(i, i);

  // 3. quantise the query from LDS while the key tiles are in flight
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) reinterpret_cast<v4i*>(s_q)[tid + 256 * i] = qraw[i];
  if (hist)
    for (int i = tid; i < kHistBins; i += 256) lhist[i] = 0;
  __syncthreads();
  float sq;
  const v8i A = F4 ? quantize_query_operand_fp4(s_q, lane, sq) : quantize_query_operand<QT, CAND>(s_q, lane, sq);
  if (wave == 0 && lane < 32) s_c[lane] = sq;
  __syncthreads();
  if (tid < 32) s_c[tid] = wv * s_c[tid];
  __syncthreads();
  float cvec[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) cvec[i] = s_c[8 * (i >> 2) + 4 * half + (i & 3)];
  float* srow = scores + (int64_t)r * ncols;

  // 4. stream the tiles
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int u = i % P;
    const int64_t col = c0 + (int64_t)(wave + kScoreWaves * i) * 32 + (lane & 31);
    v8i B;
    B[0] = ka[u][0]; B[1] = ka[u][1]; B[2] = ka[u][2]; B[3] = ka[u][3];
    B[4] = kc[u][0]; B[5] = kc[u][1]; B[6] = kc[u][2]; B[7] = kc[u][3];
    const bool v = vis[u];
    const float skl = skv[u];
    if (i + P < TPW) issue(i + P, u);
    v16f acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, F4 ? 4 : 0, F4 ? 4 : 0, 0, 0, 0, 0);
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) part = fmaf(cvec[j], acc[j], part);
    const float total = part + __shfl_xor(part, 32);
    const float sc = v ? total * skl : kNegInf;
    if (half == 0 && col < c1) {
      srow[col] = sc;
      if (hist && visible(sc)) atomicAdd(&lhist[hist_bin(order_key(sc))], 1u);
    }
  }
  if (hist) {
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

template <int TT, int NW, int NKT, bool DB>
static void launch_rows(const ScoreArgs& a, const uint8_t* q8, const float* cst, hipStream_t st) {
  const int64_t cpb = NW * NKT * 32;
  dim3 g((unsigned)(a.B * ((a.T + TT - 1) / TT)), (unsigned)((a.ncols + cpb - 1) / cpb));
  hipLaunchKernelGGL((k_score_fp8_rows<TT, NW, NKT, DB>), g, dim3(64 * NW), 0, st, a.T, a.ncols, q8, cst,
                     (const uint8_t*)a.k, a.k_scale, a.n_max, a.n_keys, a.q_limit, a.scores, a.hist);
}

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
  if constexpr (!CAND) {
    if (a.keep) {
      hipLaunchKernelGGL((k_score_fp8<QT, CAND, TPW, F4, true>), g, dim3(256), 0, st, a.T, a.ncols, (const QT*)a.q,
                         a.w, (const uint8_t*)a.k, a.k_scale, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist,
                         a.key_div);
      return;
    }
  }
  hipLaunchKernelGGL((k_score_fp8<QT, CAND, TPW, F4>), g, dim3(256), 0, st, a.T, a.ncols, (const QT*)a.q, a.w,
                     (const uint8_t*)a.k, a.k_scale, a.n_max, a.n_keys, a.q_limit, a.cand, a.scores, a.hist,
                     a.key_div);
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
