// Sparse softmax attention over the selected FP4 entries (gather + dequant + attention).
// "Compressed Sparse Attention 2 Or CSA2 In Simple Terms": only the selected entries are
// attended; "FP4 Main KV Cache To Halve Storage Again": the stored FP4 codes are expanded
// to real values only when attention needs them; "Model Setup Numbers Without Jargon": 64 heads of dim 512.  The whole
// dequantised entry is both key and value.
//
// Two main-KV layouts: one fp32 scale per (sequence, channel), and the pages' own one E4M3
// scale per 16 channels of each entry (G16, see k_attend_part).
//
// MFMA path (bf16 queries, Hq % 16 == 0, D in {128, 256, 512}).  A unit = one query row x 16
// heads (the MFMA M dimension) x one split of up to 512 selected entries, so the pages'
// Top-512 needs no merge; larger K runs several splits and a second kernel merges their
// partial softmaxes by log-sum-exp (a kernel boundary: merging inside the kernel would need a
// device-scope release fence).  The per-channel scale s_c factors out of both contractions:
// logits use q'' = q * s * 2^k_h in fp16 (2^k_h an exact per-head prescale keeping |q''| below
// 2^15, undone in that head's logits; ~2^-12 relative error) against the exact E2M1 values e in
// fp16; the output is s_c * sum_j p_j e_jc / l with p in fp16.  The split's FP4 rows are
// gathered whole into LDS (one wave instruction loads complete rows, 16 bytes per lane,
// straight into LDS) and both contractions read their operands from there.
//
// Channel split (grids of at most one block per CU: the decode shapes; G16 without a window):
// each unit runs as D / 128 blocks of 16 waves that all compute the logits, each then taking
// PV and the output of one 128-channel tile.  The logits come out transposed (lane: one head,
// 16 entries), each of the 8 logit waves takes its softmax statistics over its own 64 entries
// and feeds p from registers to PV over them; one barrier merges the waves' (m, l), and the
// waves' rescaled partial sums are added in LDS in a fixed order (deterministic).  With a
// sliding window, 4 otherwise idle waves attend its 128 rows in the same softmax.
//
// Undivided grid (many rows, or G16 with a window): one block per unit, 16 waves, PV split
// over waves by (channel tile, entry group), the groups summed in LDS in a fixed order; a
// sliding window is one more block column merged by the second kernel.  G16 layout: on the
// channel split its rows are gathered into LDS too (16 logit waves of 32 entries) and each
// lane loads its scale bytes from global memory; on the undivided grid the row operands are
// loaded from global memory directly and the group scales staged in LDS.
//
// fp32 path (fp32 queries): plain VALU, one block per (row, head), fp32 throughout.
#include "common.hpp"
#include "launch.hpp"

namespace csa2 {

constexpr int kAttHeads = 16;      // heads per block (MFMA M)
constexpr int kAttWaves = 16;      // four waves per SIMD
constexpr int kAttThreads = 64 * kAttWaves;
constexpr int kAttSplit = 512;     // entries per block: the pages' Top-512 in one block, no merge
constexpr int kCSBlocks = 4;       // channel split: blocks per (row, split, head group), at most D / 128
// The channel split repeats QK in each of its blocks, so it pays only while its whole grid runs
// in one round of blocks (one per CU: each holds about 150 KB of LDS); MI355X has 256 CUs.
constexpr long kCSMaxBlocks = 256;

// partials: part_o [R][P][Hq][D] normalised outputs, part_ml [R][P][Hq][2] (max, sum); P
// = the splits of the selected entries, plus one slot for the sliding window

// Two E4M3 codes (bytes 0 and 1 of w) -> two fp16 values (exact), low byte in the low half:
// gfx950's scaled conversion with scale 1.  Every E4M3 value, subnormals included, is an
// fp16 value; for all 65536 code pairs the result equals placing the code's exponent and
// mantissa bits at the top of an fp16 (the value times 2^-8: the biases are 7 and 15) and
// multiplying by 256, NaN payloads aside.  The _hi form converts bytes 2 and 3.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t e4m3x2_hi_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xFFFFu) | (hi16 << 16); }

// E2M1 pair in byte BS of `word` -> two fp16 values (exact; scale 1), low nibble first.
template <int BS>
__device__ __forceinline__ uint32_t cvt_pair_f16(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, BS));
}

// 8 E2M1 codes of one 32-bit word -> 8 fp16 values (exact), in nibble order.
__device__ __forceinline__ v8h decode8_f16(uint32_t word) {
  const uint4 u = make_uint4(cvt_pair_f16<0>(word), cvt_pair_f16<1>(word), cvt_pair_f16<2>(word),
                             cvt_pair_f16<3>(word));
  return __builtin_bit_cast(v8h, u);
}

// Sliding window of a layer: one block = one query row x 16 heads (8 working waves), up to
// kWinMax entries (the window rows [max(0, end - window), end) of the layer's own E4M3
// cache with one fp32 scale per row), written as partial slot `slot` for the merge with
// the selected entries ("CSA2 In Simple Terms": every layer also attends to recent tokens;
// the window cache stays 8-bit in "FP4 Main KV Cache To Halve Storage Again").
//   QK: wave w takes entries 16 w .. 16 w + 15; lane (entry n16, group g) reads 32 bytes
//       per 128-channel tile, converted exactly to fp16; the row scale multiplies the logit.
//   PV: wave w takes channels [w D / 8, (w + 1) D / 8) over all entries, so no cross-wave
//       sum is needed; lane (n16, g) reads D / 128 bytes of each of 8 entries and byte-
//       transposes them into the (entry 2p, entry 2p + 1) fp16 pairs the MFMA k-order
//       wants.  The row scales go into p (with one power-of-two normalisation 2^k so that
//       p * s * 2^k stays in fp16's normal range), undone after the sum.
constexpr int kWinMax = 128;
constexpr int kWinWaves = 8;

// two E4M3 codes (low 16 bits of w, first code in the low byte) -> two fp16 (exact)
__device__ __forceinline__ uint32_t e4m3x2_f16(uint32_t w) { return e4m3x2_to_f16x2(w); }

// LDS of the window path (carved from the attention block's shared union)
template <int D>
struct WinLds {
  static constexpr int kApad = D + 8;
  static constexpr int kPpad = kWinMax + 8;
  static constexpr size_t kA = (size_t)kAttHeads * kApad * 2;
  static constexpr size_t kP = (size_t)kAttHeads * kPpad * 2;
  static constexpr size_t kRed = (size_t)kWinWaves * kAttHeads * 4;
  static constexpr size_t kBytes = kA + kP + kRed + 2 * kAttHeads * 4 + (kAttWaves + kWinWaves) * 4;
};

// Runs on a whole attention block (kAttThreads threads): waves 0..kWinWaves-1 do the work,
// every wave takes part in the barriers.  `lds` holds WinLds<D>::kBytes (16-B aligned).
template <int D>
__device__ __forceinline__ void attend_window_block(
    int hg, int r, int T, int Hq, const uint16_t* __restrict__ q, const uint8_t* __restrict__ wcodes,
    const float* __restrict__ wscales, int64_t wn_max, const int32_t* __restrict__ wend, int window,
    float softmax_scale, int P, int slot, float* __restrict__ part, float* __restrict__ part_ml,
    unsigned char* lds) {
  constexpr int kCT = D / 128;
  constexpr int kApad = D + 8;
  constexpr int kPpad = kWinMax + 8;
  constexpr int kCPL = D / 128;                 // PV: channels per lane (bytes per entry)
  using WL = WinLds<D>;
  uint16_t* sA = reinterpret_cast<uint16_t*>(lds);
  uint16_t* sP = reinterpret_cast<uint16_t*>(lds + WL::kA);
  float (*s_red)[kAttHeads] = reinterpret_cast<float (*)[kAttHeads]>(lds + WL::kA + WL::kP);
  float* s_m = reinterpret_cast<float*>(lds + WL::kA + WL::kP + WL::kRed);
  float* s_l = s_m + kAttHeads;
  float* s_qmax = s_l + kAttHeads;
  float* s_smax = s_qmax + kAttWaves;
  const int b = r / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool act = wave < kWinWaves;           // waves past kWinWaves only join the barriers
  const int n16 = lane & 15, g = lane >> 4;
  int64_t e_end = wend[r];
  if (e_end > wn_max) e_end = wn_max;
  const int64_t e_start = e_end - window > 0 ? e_end - window : 0;
  const int nw = e_end > e_start ? (int)(e_end - e_start) : 0;  // entries in the window
  float* ml = part_ml + (((int64_t)r * P + slot) * Hq + hg * kAttHeads) * 2;
  float* po = part + (((int64_t)r * P + slot) * Hq + hg * kAttHeads) * (int64_t)D;
  if (nw == 0) {  // empty window: an empty partial (l = 0 drops it from the merge)
    for (int i = tid; i < kAttHeads * D; i += kAttThreads) po[i] = 0.0f;
    if (tid < kAttHeads) {
      ml[2 * tid] = kNegInf;
      ml[2 * tid + 1] = 0.0f;
    }
    return;
  }
  const uint8_t* wb = wcodes + ((int64_t)b * wn_max + e_start) * D;
  const float* wsb = wscales + (int64_t)b * wn_max + e_start;

  // ---- query loads, then this wave's QK rows (entries past the window read row 0 of it)
  const uint16_t* qb = q + ((int64_t)r * Hq + hg * kAttHeads) * D;
  constexpr int kQItems = kAttHeads * D / 8;
  constexpr int kQPer = (kQItems + kAttThreads - 1) / kAttThreads;
  uint4 qraw[kQPer];
#pragma unroll
  for (int it = 0; it < kQPer; ++it) {
    const int i = tid + it * kAttThreads;
    const int ic = i < kQItems ? i : kQItems - 1;
    qraw[it] = *reinterpret_cast<const uint4*>(qb + (int64_t)(ic / (D / 8)) * D + (ic % (D / 8)) * 8);
  }
  const int eq = wave * 16 + n16;                // this lane's QK entry (active waves)
  const bool q_ok = act && eq < nw;
  const uint8_t* rowq = wb + (int64_t)(q_ok ? eq : 0) * D + 32 * g;
  uint4 kw[kCT][2];
  if (act) {
#pragma unroll
    for (int i = 0; i < kCT; ++i) {
      kw[i][0] = *reinterpret_cast<const uint4*>(rowq + 128 * i);
      kw[i][1] = *reinterpret_cast<const uint4*>(rowq + 128 * i + 16);
    }
  }
  const float sq = q_ok ? wsb[eq] : 0.0f;

  // ---- q'' = q * 2^k in fp16 (exact power-of-two prescale, undone in the logits)
  float qmax = 0.0f;
  float qv[kQPer][8];
#pragma unroll
  for (int it = 0; it < kQPer; ++it) {
    const uint32_t wds[4] = {qraw[it].x, qraw[it].y, qraw[it].z, qraw[it].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[it][e] = bf16_to_f32((uint16_t)(wds[e >> 1] >> (16 * (e & 1))));
      qmax = fmaxf(qmax, fabsf(qv[it][e]));
    }
  }
  qmax = wave_max(qmax);
  if (lane == 0) s_qmax[wave] = qmax;
  __syncthreads();
  qmax = s_qmax[0];
#pragma unroll
  for (int w2 = 1; w2 < kAttWaves; ++w2) qmax = fmaxf(qmax, s_qmax[w2]);
  int qexp = 0;
  if (qmax > 0.0f) qexp = (int)((__float_as_uint(qmax) >> 23) & 255u) - 126;
  const float up = __uint_as_float((uint32_t)(127 + 15 - qexp) << 23);
  const float down = __uint_as_float((uint32_t)(127 - 15 + qexp) << 23);
#pragma unroll
  for (int it = 0; it < kQPer; ++it) {
    const int i = tid + it * kAttThreads;
    if (i >= kQItems) break;
    const int h = i / (D / 8), c = (i % (D / 8)) * 8;
    uint32_t wv[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const _Float16 a0 = (_Float16)(qv[it][2 * k2] * up), a1 = (_Float16)(qv[it][2 * k2 + 1] * up);
      wv[k2] = pack2(__builtin_bit_cast(uint16_t, a0), __builtin_bit_cast(uint16_t, a1));
    }
    *reinterpret_cast<uint4*>(&sA[h * kApad + c]) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  __syncthreads();

  // ---- logits of this wave's 16 entries (lane: entry n16, heads 4 g + rr)
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (act ? kCT : 0); ++i) {
    const uint32_t wd[8] = {kw[i][0].x, kw[i][0].y, kw[i][0].z, kw[i][0].w,
                            kw[i][1].x, kw[i][1].y, kw[i][1].z, kw[i][1].w};
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {  // channels 128 i + 32 g + 8 sub + [0, 8)
      const uint4 bw = make_uint4(e4m3x2_f16(wd[2 * sub]), e4m3x2_f16(wd[2 * sub] >> 16),
                                  e4m3x2_f16(wd[2 * sub + 1]), e4m3x2_f16(wd[2 * sub + 1] >> 16));
      const v8h av = *reinterpret_cast<const v8h*>(&sA[n16 * kApad + 128 * i + 32 * g + 8 * sub]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(v8h, bw), acc, 0, 0, 0);
    }
  }
  const float lscale = softmax_scale * down * sq;
  float logit[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) logit[rr] = q_ok ? acc[rr] * lscale : kNegInf;

  // ---- PV code loads now (their latency overlaps the softmax): lane (n16, g) takes
  //      channels cw0 + kCPL n16 + [0, kCPL) of entries 32 ks + 8 g + [0, 8)
  const int cw0 = wave * (D / kWinWaves);
  constexpr int kKS = kWinMax / 32;
  uint32_t pw[kKS][8];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (!act) {
        pw[ks][jj] = 0u;
        continue;
      }
      const int e = 32 * ks + 8 * g + jj;
      const uint8_t* src = wb + (int64_t)(e < nw ? e : 0) * D + cw0 + kCPL * n16;
      uint32_t v;
      if (kCPL == 4) v = *reinterpret_cast<const uint32_t*>(src);
      else if (kCPL == 2) v = *reinterpret_cast<const uint16_t*>(src);
      else v = *src;
      pw[ks][jj] = e < nw ? v : 0u;
    }
  }

  // ---- softmax statistics; the row scales' largest power of two
  if (act) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float v = row16_max(logit[rr]);
      if (n16 == 0) s_red[wave][4 * g + rr] = v;
    }
    const float smx = wave_max(sq);
    if (lane == 0) s_smax[wave] = smx;
  }
  __syncthreads();
  if (tid < kAttHeads) {
    float m = s_red[0][tid];
#pragma unroll
    for (int w2 = 1; w2 < kWinWaves; ++w2) m = fmaxf(m, s_red[w2][tid]);
    s_m[tid] = m;
  }
  float smax = s_smax[0];
#pragma unroll
  for (int w2 = 1; w2 < kWinWaves; ++w2) smax = fmaxf(smax, s_smax[w2]);
  // 2^pk with smax * 2^pk in [1, 2): p * s * 2^pk <= 2 (p <= 1)
  const int sexp = smax > 0.0f ? (int)((__float_as_uint(smax) >> 23) & 255u) - 127 : 0;
  const float pup = __uint_as_float((uint32_t)(127 - sexp) << 23);
  const float pdown = __uint_as_float((uint32_t)(127 + sexp) << 23);
  __syncthreads();
  if (act) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = 4 * g + rr;
      const float m = s_m[h];
      const float p = (m == kNegInf || !q_ok) ? 0.0f : __expf(logit[rr] - m);
      sP[h * kPpad + eq] = __builtin_bit_cast(uint16_t, (_Float16)(p * sq * pup));
      const float v = row16_sum(p);
      if (n16 == 0) s_red[wave][h] = v;
    }
  }
  __syncthreads();
  if (tid < kAttHeads) {
    float l = s_red[0][tid];
#pragma unroll
    for (int w2 = 1; w2 < kWinWaves; ++w2) l += s_red[w2][tid];
    s_l[tid] = l;
  }

  // ---- PV: o[h][c] = sum_e p'[h][e] E4M3(code[e][c]) over this wave's channels
  v4f o[kCPL];
#pragma unroll
  for (int m = 0; m < kCPL; ++m) o[m] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    if (!act || 32 * ks >= nw) break;
    const v8h pa = *reinterpret_cast<const v8h*>(&sP[n16 * kPpad + 32 * ks + 8 * g]);
#pragma unroll
    for (int m = 0; m < kCPL; m += 2) {
      // bytes m, m + 1 of entries (2 p2, 2 p2 + 1): (e0[m], e1[m], e0[m+1], e1[m+1])
      uint32_t bx[4], by[4];
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) {
        const uint32_t t = __builtin_amdgcn_perm(pw[ks][2 * p2 + 1], pw[ks][2 * p2],
                                                 (uint32_t)m | (uint32_t)(m + 4) << 8 | (uint32_t)(m + 1) << 16 |
                                                     (uint32_t)(m + 5) << 24);
        bx[p2] = e4m3x2_f16(t);          // channel m
        by[p2] = e4m3x2_f16(t >> 16);    // channel m + 1
      }
      o[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(v8h, make_uint4(bx[0], bx[1], bx[2], bx[3])),
                                                    o[m], 0, 0, 0);
      if (m + 1 < kCPL)
        o[m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            pa, __builtin_bit_cast(v8h, make_uint4(by[0], by[1], by[2], by[3])), o[m + 1], 0, 0, 0);
    }
  }
  __syncthreads();  // s_l
  // lane (n16, g) holds o[h = 4 g + rr][channel cw0 + kCPL n16 + m]
#pragma unroll
  for (int rr = 0; rr < (act ? 4 : 0); ++rr) {
    const int h = 4 * g + rr;
    const float l = s_l[h];
    const float sc = (l > 0.0f) ? pdown / l : 0.0f;
    float* dst = po + (int64_t)h * D + cw0 + kCPL * n16;
#pragma unroll
    for (int m = 0; m < kCPL; ++m) dst[m] = o[m][rr] * sc;
  }
  if (tid < kAttHeads) {
    ml[2 * tid] = s_m[tid];
    ml[2 * tid + 1] = s_l[tid];
  }
}

template <int D, int WPT, bool G16, int OW = D>
struct AttLds {
  static constexpr int kApad = D + 8;           // fp16 per A row (padding against bank conflicts)
  static constexpr int kPpad = kAttSplit + 8;
  static constexpr int kSpad = kAttSplit + 8;   // fp16 per group row of the entry scales (G16)
  static constexpr size_t kA = (size_t)kAttHeads * kApad * 2;
  static constexpr size_t kP = (size_t)kAttHeads * kPpad * 2;
  static constexpr size_t kS = G16 ? (size_t)(D / 16) * kSpad * 2 : 0;  // [group][entry] fp16 scales
  static constexpr size_t kO = (size_t)WPT * kAttHeads * OW * 4;  // per entry group, after sA/sP/sS are dead
  // per-channel layout: the split's FP4 rows are staged in LDS ([entry][D/2 bytes], 16-byte
  // chunks XOR-swizzled), followed by sA; sP takes sA's place once QK is done.  G16: sA,
  // sP, sS side by side (its rows are read from global memory).
  static constexpr size_t kRows = G16 ? 0 : (size_t)kAttSplit * (D / 2);
  static constexpr size_t kOffA = kRows;
  static constexpr size_t kOffP = G16 ? kA : kRows;
  static constexpr size_t kOffS = kA + kP;
  static constexpr size_t kAP = G16 ? kA + kP + kS : kRows + (kA > kP ? kA : kP);
  static constexpr size_t kWork = kAP > kO ? kAP : kO;
  static constexpr size_t kUnion = kWork > WinLds<D>::kBytes ? kWork : WinLds<D>::kBytes;
};

// One block = one query row x 16 heads x one split of up to kAttSplit selected entries.
// With one partial in all (P == 1) the block writes the final output; otherwise it writes
// its partial (normalised output, running max, sum) for k_attend_combine.
// G16: the cache holds one E4M3 scale per 16 channels of each entry (the pages' layout).
// The scale no longer factors out of the contractions; instead the split's scales are
// staged in LDS as fp16, [group][entry], and multiply the fp16 key / value operands after
// the E2M1 conversion (E2M1 * E4M3 is exact in fp16, so the operands stay exact).
template <int D, bool G16, bool CS, bool WIN>
__global__ __launch_bounds__(kAttThreads) void k_attend_part(
    int R, int T, int Hq, int K, int S, int P, const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const void* __restrict__ scales_v, int64_t n_max, const int32_t* __restrict__ idx, float softmax_scale, void* __restrict__ out, int out_bf16, float* __restrict__ lse,
    float* __restrict__ part, float* __restrict__ part_ml, const uint8_t* __restrict__ wcodes,
    const float* __restrict__ wscales, int64_t wn_max, const int32_t* __restrict__ wend, int window) {
  constexpr int kRowBytes = D / 2;
  constexpr int kCT = D / 128;                 // 128-channel tiles
  // waves that compute logits: per-channel, 8 waves of 4 tiles (each QK wave reads the whole
  // query operand from LDS once, so fewer, longer waves read less); G16, all 16 waves (its
  // operands come from global memory, and more waves issue those loads faster)
  // G16 on the channel split gathers its rows into LDS like the per-channel layout and loads
  // each lane's scale bytes from global memory; the undivided G16 kernel keeps operand-layout
  // row loads and stages the scales
  constexpr bool kOpG16 = G16 && !CS;
  constexpr int kQKW = G16 ? kAttWaves : 8;
  constexpr int kAttTPW = kAttSplit / 16 / kQKW;  // 16-entry QK tiles per QK wave
  static_assert(kAttTPW * 16 * kQKW == kAttSplit, "QK tiles cover the split");
  // CS (channel split): the block computes every logit and the softmax of its (row, split, head
  // group) but PV and the output only for channel tile `cb`; the kCT blocks of a head group
  // repeat QK and each takes one tile, so the chip runs kCT times as many blocks with a
  // quarter of the PV each (D = 512) and no merge
  constexpr int kNCB = CS ? (kCT < kCSBlocks ? kCT : kCSBlocks) : 1;  // channel blocks per head group
  constexpr int kPVT = kCT / kNCB;             // channel tiles per block in PV
  constexpr int kOW = 128 * kPVT;              // channels per head row of the partial sums
  // waves per tile in PV (CS: each logit wave takes PV over its own entries)
  // CS with a sliding window (WIN): kCSWinW more waves attend the window's rows (32 each) in
  // the same softmax
  constexpr int kCSWinW = kWinMax / 32;
  static_assert(!WIN || kQKW + kCSWinW <= kAttWaves, "window waves past the logit waves");
  constexpr int kWPT = CS ? kQKW + (WIN ? kCSWinW : 0)
                          : ((kAttWaves / kPVT < kAttSplit / 32) ? kAttWaves / kPVT : kAttSplit / 32);
  // per-channel layout: the split's rows are gathered whole (a wave instruction reads
  // kRPI complete rows, 16 bytes per lane) and staged in LDS; chunk c of entry e sits in
  // chunk slot c ^ swz(e), so that the 16 entries of an MFMA operand read spread over
  // all banks.  (Gathering 64-byte row pieces of 16 entries per instruction straight into
  // operand layout measured about 3x slower per byte when the rows are cached.)
  constexpr int kNC = kRowBytes / 16;          // 16-byte chunks per row: 4, 8 or 16
  constexpr int kRPI = 64 / kNC;               // rows per gather instruction
  constexpr int kGI = kAttSplit / (kRPI * kAttWaves);  // gather instructions per wave
  static_assert(kGI * kRPI * kAttWaves == kAttSplit, "the gather covers the split");
  auto swz = [](int e) { return (e / (16 / kNC)) & (kNC - 1); };
  constexpr int kEPW = kAttSplit / kWPT;       // entries per wave in PV (a multiple of 32)
  using L = AttLds<D, kWPT, kOpG16, kOW>;
  constexpr int kNG = D / 16;                  // scale groups per entry (G16)
  __shared__ float s_scale[G16 ? 1 : D];
  __shared__ __align__(16) int32_t s_idx[kAttSplit];
  __shared__ float s_red[2 * kAttWaves][kAttHeads];
  __shared__ float s_m[kAttHeads], s_l[kAttHeads];
  __shared__ float s_down[kAttHeads];          // per head: softmax scale / the query prescale
  __shared__ float s_wmax[WIN ? kAttHeads : 1];  // WIN: per head, the largest |q| (no channel scales)
  __shared__ __align__(16) unsigned char s_u[L::kUnion];
  uint16_t* sA = reinterpret_cast<uint16_t*>(s_u + L::kOffA);
  uint16_t* sP = reinterpret_cast<uint16_t*>(s_u + L::kOffP);
  uint16_t* sS = reinterpret_cast<uint16_t*>(s_u + L::kOffS);  // G16: [kNG][kSpad] fp16
  unsigned char* s_rows = s_u;                 // per-channel: the split's rows (see AttLds)
  float* sO = reinterpret_cast<float*>(s_u);  // [kWPT][16][kOW], used once the rows, sA, sP, sS are dead
  const float* scales = static_cast<const float*>(scales_v);

  // XCD-aware order: workgroups are dealt to the 8 XCDs in turn (L2 per XCD), so a unit
  // (row, split) takes workgroups wg with the same wg % 8 for all its head groups, which then
  // gather the same rows through one L2.  Units past the last (grid rounded up) exit.
  const int X = S + ((wcodes && !CS) ? 1 : 0);   // splits, plus the window's block (not CS)
  const int G = Hq / kAttHeads;                  // head groups
  const int wg = blockIdx.x, slot = wg >> 3;
  const int unit = (slot / (G * kNCB)) * 8 + (wg & 7), hg = (slot % (G * kNCB)) / kNCB;
  const int ctb = CS ? slot % kNCB : 0;        // CS: this block's channel tiles ctb kPVT + [0, kPVT)
  if (unit >= X * R) return;
  const int split = unit % X, r = unit / X;
  if (!CS && split == S) {  // the sliding window's block (grid.x = S + 1 with a window)
    attend_window_block<D>(hg, r, T, Hq, q, wcodes, wscales, wn_max, wend, window, softmax_scale, P, S, part, part_ml,
                           s_u);
    return;
  }
  const int b = r / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int e0 = split * kAttSplit;            // first entry of this split

  // ---- phase 0: scales, the split's entries, q'' = q * s * 2^k in fp16.  The query
  //      loads are issued first so that their latency overlaps the entry selection.
  const uint16_t* qb = q + ((int64_t)r * Hq + hg * kAttHeads) * D;
  constexpr int kQItems = kAttHeads * D / 8;       // 8 channels per item
  constexpr int kQPer = (kQItems + kAttThreads - 1) / kAttThreads;
  uint4 qraw[kQPer];
#pragma unroll
  for (int it = 0; it < kQPer; ++it) {
    const int i = tid + it * kAttThreads;
    const int ic = i < kQItems ? i : kQItems - 1;
    qraw[it] = *reinterpret_cast<const uint4*>(qb + (int64_t)(ic / (D / 8)) * D + (ic % (D / 8)) * 8);
  }
  // the channel scales: loaded now, stored to LDS once the entry selection is done (a store
  // now would wait for them, and with them for the query loads, before the selection starts)
  static_assert(CSA2_MAX_D_DEV <= kAttThreads, "one channel scale per thread");
  const float sc_reg = (!G16 && tid < D) ? scales[(int64_t)b * D + tid] : 0.0f;
  for (int i = tid; i < kAttSplit; i += kAttThreads) {
    const int e = e0 + i;
    const int32_t j = (e < K) ? idx[(int64_t)r * K + e] : -1;
    s_idx[i] = (j >= 0 && j < n_max) ? j : -1;
  }
  const int32_t* sel = s_idx;                    // the split's entries (LDS)
  if (!G16 && tid < D) s_scale[tid] = sc_reg;
  __syncthreads();  // s_scale, s_idx

  // ---- phase 1a: issue this wave's QK row loads now, so that their latency overlaps the
  //      query preparation.  Unconditional loads from a valid row (row 0 for skipped
  //      entries) keep them branch-free; skipped entries are masked in the logits.
  const uint8_t* cb = codes + (int64_t)b * n_max * kRowBytes;
  // G16: the split's entry scales in chunks of 16 (8 when D = 128) groups of one entry,
  // issued before the rows so that waiting for them (to stage them in LDS) does not wait
  // for the rows; the lanes of a wave take consecutive entries of one chunk column.
  // Skipped entries get scale 0 (their logits are masked and their p is 0 anyway).
  constexpr int kCB = kNG < 16 ? kNG : 16;     // scale bytes per chunk
  constexpr int kGC = kNG / kCB;               // chunks per entry
  constexpr int kScChunks = kAttSplit * kGC;
  constexpr int kScPer = G16 ? (kScChunks + kAttThreads - 1) / kAttThreads : 1;
  uint4 gsw[kScPer];
  const uint8_t* gsb = G16 ? static_cast<const uint8_t*>(scales_v) + (int64_t)b * n_max * kNG : nullptr;
  if (kOpG16) {
#pragma unroll
    for (int it = 0; it < kScPer; ++it) {
      const int i = tid + it * kAttThreads;
      const int ic = i < kScChunks ? i : kScChunks - 1;
      const int32_t j = sel[ic % kAttSplit];
      const uint8_t* src = gsb + (int64_t)(j >= 0 ? j : 0) * kNG + kCB * (ic / kAttSplit);
      if (kCB == 16) {
        gsw[it] = *reinterpret_cast<const uint4*>(src);
      } else {
        const uint2 h = *reinterpret_cast<const uint2*>(src);
        gsw[it] = make_uint4(h.x, h.y, 0u, 0u);
      }
      if (j < 0) gsw[it] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const bool qk_wave = wave < kQKW;            // wave-uniform
  const int qw = wave % kQKW;
  uint4 kw[kAttTPW][kCT];
  int32_t jt[kAttTPW];
#pragma unroll
  for (int t = 0; t < kAttTPW; ++t) {
    const int e = (qw * kAttTPW + t) * 16 + n16;
    jt[t] = sel[e];  // -1 past K
    if constexpr (kOpG16) {
      const uint8_t* rowp = cb + (int64_t)(jt[t] >= 0 ? jt[t] : 0) * kRowBytes + 16 * g;
#pragma unroll
      for (int i = 0; i < kCT; ++i) kw[t][i] = *reinterpret_cast<const uint4*>(rowp + 64 * i);
    }
  }

  // ---- phase 0b: q'' = q * s * 2^k_h in fp16 into LDS (A operand of QK), with one exact
  //      power-of-two prescale per head (|q''| < 2^15, the fp16 range), undone in that head's
  //      logits.  A head's D/8 items sit in one wave, so its maximum needs no block barrier.
  static_assert(kQPer == 1, "one query item per thread");
  constexpr int kLPH = D / 8;                  // lanes per head
  const bool q_act = tid < kQItems;
  const int qh = tid / kLPH, qc = (tid % kLPH) * 8;
  float qv[8];
  float qmax = 0.0f, qrmax = 0.0f;  // qrmax (WIN): without the channel scales
  {
    const uint32_t wds[4] = {qraw[0].x, qraw[0].y, qraw[0].z, qraw[0].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qe = bf16_to_f32((uint16_t)(wds[e >> 1] >> (16 * (e & 1))));
      qrmax = fmaxf(qrmax, fabsf(qe));
      qv[e] = qe * (G16 || !q_act ? 1.0f : s_scale[qc + e]);
      qmax = fmaxf(qmax, fabsf(qv[e]));
    }
  }
  // keep the query reads above the row loads (a wait for the query after them would also
  // wait for the rows)
  __builtin_amdgcn_sched_barrier(0);
  // per-channel: gather instruction j of a wave loads rows r0 .. r0 + kRPI - 1 (r0 =
  // (wave kGI + j) kRPI) straight into LDS, lane l's 16 bytes landing in chunk slot l % kNC of
  // row r0 + l / kNC; the lane reads logical chunk (l % kNC) ^ swz(row), which swizzles the
  // staged row.  Issued after the last LDS read of the query preparation: the loads stay in
  // flight through the query's conversion and stores (an LDS read while they are in flight
  // would wait for them).
  if constexpr (!kOpG16) {
#pragma unroll
    for (int j = 0; j < kGI; ++j) {
      const int r0 = (wave * kGI + j) * kRPI;
      const int row = r0 + lane / kNC;
      const int32_t jr = sel[row];
      const uint8_t* src = cb + (int64_t)(jr >= 0 ? jr : 0) * kRowBytes + 16 * ((lane % kNC) ^ swz(row));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(s_rows + r0 * kRowBytes), 16, 0, 0);
    }
  }
  // G16 on the channel split: this lane's scale bytes, loaded with the gather.  QK: the whole
  // 32-byte scale row of each of its entries (qw kAttTPW + t) 16 + n16 (it uses groups 8 i + 2 g
  // and 8 i + 2 g + 1); PV: group 8 ctb + n16 / 2 of the entries of its K slots.  Skipped
  // entries take scale 0 (their p is 0, and the row standing in for them may hold any byte).
  uint4 gqk[G16 && CS ? kAttTPW : 1][2];
  uint32_t gpv[2] = {0u, 0u};
  if constexpr (G16 && CS) {
    static_assert(kNG == 32 || kNG == 16 || kNG == 8, "scale row of D / 16 bytes");
#pragma unroll
    for (int t = 0; t < kAttTPW; ++t) {
      const int32_t j = sel[(qw * kAttTPW + t) * 16 + n16];
      const uint8_t* gp = gsb + (int64_t)(j >= 0 ? j : 0) * kNG;
      uint4 a0 = make_uint4(0u, 0u, 0u, 0u), a1 = a0;
      if constexpr (kNG >= 16) a0 = *reinterpret_cast<const uint4*>(gp);
      else a0 = make_uint4(reinterpret_cast<const uint2*>(gp)->x, reinterpret_cast<const uint2*>(gp)->y, 0u, 0u);
      if constexpr (kNG == 32) a1 = *reinterpret_cast<const uint4*>(gp + 16);
      gqk[t][0] = j >= 0 ? a0 : make_uint4(0u, 0u, 0u, 0u);
      gqk[t][1] = j >= 0 ? a1 : make_uint4(0u, 0u, 0u, 0u);
    }
    static_assert(kAttTPW == 2, "one PV step of two tiles per logit wave");
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int32_t j = sel[(qw * kAttTPW + (jj >> 2)) * 16 + 4 * g + (jj & 3)];
      const uint32_t v = gsb[(int64_t)(j >= 0 ? j : 0) * kNG + 8 * ctb + (n16 >> 1)];
      gpv[jj >> 2] |= (j >= 0 ? v : 0u) << (8 * (jj & 3));
    }
  }
  // WIN: the window waves' row scales and PV bytes (lane (channel block n16, g): channels
  // 128 ctb + 8 n16 + [0, 8) of the entries in its K slots, see the window waves below),
  // loaded now so that they arrive with the gathered rows
  int wnw = 0;
  const uint8_t* wbp = wcodes;
  float wsq[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  uint2 wvw[8];
  if constexpr (WIN) {
    if (wave >= kQKW && wave < kQKW + kCSWinW) {  // wave-uniform
      int64_t w_end = wend[r];
      if (w_end > wn_max) w_end = wn_max;
      const int64_t w_start = w_end - window > 0 ? w_end - window : 0;
      wnw = (split == 0 && w_end > w_start) ? (int)(w_end - w_start) : 0;
      if (wnw > 0) {
        const int ww = wave - kQKW;
        wbp = wcodes + ((int64_t)b * wn_max + w_start) * D;
        const float* wsb = wscales + (int64_t)b * wn_max + w_start;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int e = 32 * ww + 16 * t + 4 * g + rr;
            const float v = wsb[e < wnw ? e : 0];  // (unconditional loads from a valid row)
            wsq[t][rr] = e < wnw ? v : 0.0f;
          }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = 32 * ww + 16 * (j >> 2) + 4 * g + (j & 3);
          const uint2 v = *reinterpret_cast<const uint2*>(wbp + (int64_t)(e < wnw ? e : 0) * D + 128 * ctb + 8 * n16);
          wvw[j] = e < wnw ? v : make_uint2(0u, 0u);
        }
      }
    }
  }
  {  // the head's maximum over its kLPH lanes (16-lane rows, then rows of one head)
    float hm = row16_max(qmax);
    const float m0 = lane_read(hm, 0), m1 = lane_read(hm, 16), m2 = lane_read(hm, 32), m3 = lane_read(hm, 48);
    if (kLPH == 64) hm = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
    else if (kLPH == 32) hm = (lane < 32) ? fmaxf(m0, m1) : fmaxf(m2, m3);
    qmax = hm;
    if constexpr (WIN) {
      float hr = row16_max(qrmax);
      const float r0 = lane_read(hr, 0), r1 = lane_read(hr, 16), r2 = lane_read(hr, 32), r3 = lane_read(hr, 48);
      if (kLPH == 64) hr = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
      else if (kLPH == 32) hr = (lane < 32) ? fmaxf(r0, r1) : fmaxf(r2, r3);
      if (q_act && qc == 0) s_wmax[qh] = hr;
    }
  }
  int qexp = 0;
  if (qmax > 0.0f) qexp = (int)((__float_as_uint(qmax) >> 23) & 255u) - 126;
  const float up = __uint_as_float((uint32_t)(127 + 15 - qexp) << 23);
  if (q_act) {
    uint32_t wv[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      const _Float16 a0 = (_Float16)(qv[2 * k2] * up), a1 = (_Float16)(qv[2 * k2 + 1] * up);
      wv[k2] = pack2(__builtin_bit_cast(uint16_t, a0), __builtin_bit_cast(uint16_t, a1));
    }
    *reinterpret_cast<uint4*>(&sA[qh * L::kApad + qc]) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    if (qc == 0) s_down[qh] = softmax_scale * __uint_as_float((uint32_t)(127 - 15 + qexp) << 23);
  }
  if (kOpG16) {  // the scales as fp16, [group][entry]
#pragma unroll
    for (int it = 0; it < kScPer; ++it) {
      const int i = tid + it * kAttThreads;
      if (i >= kScChunks) break;
      const int e = i % kAttSplit, grp0 = kCB * (i / kAttSplit);
      const uint32_t wd[4] = {gsw[it].x, gsw[it].y, gsw[it].z, gsw[it].w};
#pragma unroll
      for (int k2 = 0; k2 < kCB / 2; ++k2) {
        const uint32_t s2 = e4m3x2_to_f16x2(wd[k2 >> 1] >> (16 * (k2 & 1)));
        sS[(grp0 + 2 * k2) * L::kSpad + e] = (uint16_t)(s2 & 0xFFFFu);
        sS[(grp0 + 2 * k2 + 1) * L::kSpad + e] = (uint16_t)(s2 >> 16);
      }
    }
  }
  if constexpr (!kOpG16) __builtin_amdgcn_s_waitcnt(0);  // this wave's row loads have landed in LDS
  __syncthreads();

  if constexpr (CS) {
    float m = kNegInf, lsum = 0.0f;
    float xdown = 1.0f;  // window waves: the power of two taken out of p, put back at the rescale
    v4f acc[kPVT][8];
    const bool win_wave = WIN && wave >= kQKW && wave < kQKW + kCSWinW;  // wave-uniform
    // ---- CS window waves (WIN, split 0): the row's sliding window, rows [max(0, end -
    //      window), end) of the layer's E4M3 cache with one fp32 scale per row, 32 entries per
    //      wave (kWinMax / 32 waves past the logit waves, idle until now).  The logits need the
    //      query without the main cache's channel scales: each lane loads its B operand (head
    //      n16, channels 128 ct + 32 g + 8 sub + [0, 8)) straight from global memory and takes
    //      the head's own power of two.  The row scale multiplies the logit and, with the
    //      wave's largest row scale 2^sx taken out (undone at the rescale), p in PV.
    if (win_wave) {
      if constexpr (WIN) {
        static_assert(kPVT == 1, "the window's PV takes one channel tile");
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) acc[0][mm] = (v4f){0.f, 0.f, 0.f, 0.f};
        const int ww = wave - kQKW;
        const int nw = wnw;
        if (nw > 0) {  // (an empty window leaves m = -inf, l = 0 and zero sums)
        const uint8_t* wb = wbp;
        const uint16_t* qrow = q + ((int64_t)r * Hq + hg * kAttHeads + n16) * D + 32 * g;
        const float (&sqv)[2][4] = wsq;  // row scales of this lane's logit entries 32 ww + 16 t + 4 g + rr
        const float qm = s_wmax[n16];    // the head's largest |q|
        int wexp = 0;
        if (qm > 0.0f) wexp = (int)((__float_as_uint(qm) >> 23) & 255u) - 126;
        wexp = wexp < -100 ? -100 : wexp;
        const float wup = __uint_as_float((uint32_t)(127 + 15 - wexp) << 23);
        const float wdn = softmax_scale * __uint_as_float((uint32_t)(127 - 15 + wexp) << 23);
        v4f a2[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
#pragma unroll 2
        for (int i = 0; i < kCT; ++i) {  // (two tiles in flight: the loads of all four spill)
          v8h qh8[4];  // B operand: the tile's query in fp16 with the head's power of two
#pragma unroll
          for (int sub = 0; sub < 4; ++sub) {
            const uint4 qv4 = *reinterpret_cast<const uint4*>(qrow + 128 * i + 8 * sub);
            const uint32_t wds[4] = {qv4.x, qv4.y, qv4.z, qv4.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) qh8[sub][e] = (_Float16)(bf16_to_f32((uint16_t)(wds[e >> 1] >> (16 * (e & 1)))) * wup);
          }
          uint4 kr[2][2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int e = 32 * ww + 16 * t + n16;
            const uint8_t* src = wb + (int64_t)(e < nw ? e : 0) * D + 128 * i + 32 * g;
            kr[t][0] = *reinterpret_cast<const uint4*>(src);
            kr[t][1] = *reinterpret_cast<const uint4*>(src + 16);
          }
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const uint4 hw = kr[t][sub >> 1];
              const uint32_t w0 = (sub & 1) ? hw.z : hw.x, w1 = (sub & 1) ? hw.w : hw.y;
              const uint4 bw = make_uint4(e4m3x2_f16(w0), e4m3x2_hi_to_f16x2(w0), e4m3x2_f16(w1), e4m3x2_hi_to_f16x2(w1));
              a2[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, bw), qh8[sub], a2[t], 0, 0, 0);
            }
        }
        float p2v[2][4];
        float wm = kNegInf, smx = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int e = 32 * ww + 16 * t + 4 * g + rr;
            p2v[t][rr] = e < nw ? a2[t][rr] * wdn * sqv[t][rr] : kNegInf;
            wm = fmaxf(wm, p2v[t][rr]);
            smx = fmaxf(smx, sqv[t][rr]);
          }
        wm = fmaxf(wm, __shfl_xor(wm, 16));
        wm = fmaxf(wm, __shfl_xor(wm, 32));
        smx = fmaxf(smx, __shfl_xor(smx, 16));
        smx = fmaxf(smx, __shfl_xor(smx, 32));
        float wl = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            p2v[t][rr] = (wm == kNegInf) ? 0.0f : __expf(p2v[t][rr] - wm);
            wl += p2v[t][rr];
          }
        wl += __shfl_xor(wl, 16);
        wl += __shfl_xor(wl, 32);
        // 2^sx with smx 2^-sx in [1, 2): p s 2^-sx <= 2
        const int sx = smx > 0.0f ? (int)((__float_as_uint(smx) >> 23) & 255u) - 127 : 0;
        const float sdn = __uint_as_float((uint32_t)(127 - sx) << 23);
        xdown = __uint_as_float((uint32_t)(127 + sx) << 23);
        v8h pa;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pa[rr] = (_Float16)(p2v[0][rr] * sqv[0][rr] * sdn);
          pa[4 + rr] = (_Float16)(p2v[1][rr] * sqv[1][rr] * sdn);
        }
        // PV: lane (channel block n16, g) takes channels 128 ctb + 8 n16 + [0, 8) (8 bytes) of
        // the entries in K slots 8 g + j (entry 32 ww + 16 (j >> 2) + 4 g + (j & 3)); pairs of
        // entries are byte-transposed so that one word holds (e0[c], e1[c], e0[c + 1], e1[c + 1])
        const uint2 (&vw)[8] = wvw;
#pragma unroll
        for (int hw = 0; hw < 2; ++hw)
#pragma unroll
          for (int mm = 0; mm < 4; mm += 2) {
            uint32_t bx[4], by[4];
#pragma unroll
            for (int p2 = 0; p2 < 4; ++p2) {
              const uint32_t lo = hw ? vw[2 * p2].y : vw[2 * p2].x, hi = hw ? vw[2 * p2 + 1].y : vw[2 * p2 + 1].x;
              const uint32_t tw = __builtin_amdgcn_perm(hi, lo, (uint32_t)mm | (uint32_t)(mm + 4) << 8 |
                                                                    (uint32_t)(mm + 1) << 16 | (uint32_t)(mm + 5) << 24);
              bx[p2] = e4m3x2_f16(tw);           // channel 4 hw + mm
              by[p2] = e4m3x2_hi_to_f16x2(tw);   // channel 4 hw + mm + 1
            }
            acc[0][4 * hw + mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                pa, __builtin_bit_cast(v8h, make_uint4(bx[0], bx[1], bx[2], bx[3])), acc[0][4 * hw + mm], 0, 0, 0);
            acc[0][4 * hw + mm + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                pa, __builtin_bit_cast(v8h, make_uint4(by[0], by[1], by[2], by[3])), acc[0][4 * hw + mm + 1], 0, 0, 0);
          }
        m = wm;
        lsum = wl;
        }
      }
    } else {
      // ---- CS phase 1: the logits transposed (rows x q''^T, the row chunk as the MFMA's A
      //      operand and q'' as B): lane (head n16, g) holds head n16's logits of the entries
      //      16 t' + 4 g + rr (t' = qw kAttTPW + t) of this wave's tiles
      v4f a[kAttTPW];
  #pragma unroll
      for (int t = 0; t < kAttTPW; ++t) a[t] = (v4f){0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int i = 0; i < (qk_wave ? kCT : 0); ++i) {
        uint32_t wd[kAttTPW][4];
        _Float16 gs[kAttTPW][2];  // G16: groups 8 i + 2 g and 8 i + 2 g + 1 of the lane's entry
  #pragma unroll
        for (int t = 0; t < kAttTPW; ++t) {
          const int el = (qw * kAttTPW + t) * 16 + n16;
          uint4 kv;
          kv = *reinterpret_cast<const uint4*>(s_rows + el * kRowBytes + 16 * ((4 * i + g) ^ swz(el)));
          if constexpr (G16) {  // bytes 8 i + 2 g, 8 i + 2 g + 1 of the entry's scale row
            const uint4 hv = gqk[t][(8 * i) >> 4];
            const int bo = (8 * i + 2 * g) & 15;
            const uint32_t wsel = (bo >> 2) == 0 ? hv.x : (bo >> 2) == 1 ? hv.y : (bo >> 2) == 2 ? hv.z : hv.w;
            const uint32_t s2 = e4m3x2_to_f16x2(wsel >> (8 * (bo & 3)));
            gs[t][0] = __builtin_bit_cast(_Float16, (uint16_t)(s2 & 0xFFFFu));
            gs[t][1] = __builtin_bit_cast(_Float16, (uint16_t)(s2 >> 16));
          }
          wd[t][0] = kv.x; wd[t][1] = kv.y; wd[t][2] = kv.z; wd[t][3] = kv.w;
        }
  #pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          const v8h qv8 = *reinterpret_cast<const v8h*>(&sA[n16 * L::kApad + 128 * i + 32 * g + 8 * sub]);
  #pragma unroll
          for (int t = 0; t < kAttTPW; ++t) {
            v8h kvh = decode8_f16(wd[t][sub]);
            if constexpr (G16) kvh = kvh * gs[t][sub >> 1];  // E2M1 x E4M3 is exact in fp16
            a[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kvh, qv8, a[t], 0, 0, 0);
          }
        }
      }
      // ---- CS phase 2: this wave's softmax statistics per head (no block barrier): the
      //      maximum and the sum over the lane's 4 kAttTPW logits, then over the 4 lanes of the
      //      head (g); p = exp(logit - m) stays in registers as PV's A operand
      const float dn = s_down[n16];
      float pr[kAttTPW][4];
      m = kNegInf;
  #pragma unroll
      for (int t = 0; t < kAttTPW; ++t) {
        const int4 sv = *reinterpret_cast<const int4*>(&s_idx[(qw * kAttTPW + t) * 16 + 4 * g]);
        const int32_t svv[4] = {sv.x, sv.y, sv.z, sv.w};
  #pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pr[t][rr] = (qk_wave && svv[rr] >= 0) ? a[t][rr] * dn : kNegInf;
          m = fmaxf(m, pr[t][rr]);
        }
      }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      lsum = 0.0f;
  #pragma unroll
      for (int t = 0; t < kAttTPW; ++t)
  #pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pr[t][rr] = (m == kNegInf) ? 0.0f : __expf(pr[t][rr] - m);
          lsum += pr[t][rr];
        }
      lsum += __shfl_xor(lsum, 16);  // the four lanes of a head add the same pairs: equal sums
      lsum += __shfl_xor(lsum, 32);
      // ---- CS phase 3: PV over this wave's entries for the block's channel tiles.  K step ks takes the
      //      wave's tiles 2 ks and 2 ks + 1; its K slot 8 g + j is entry 16 t0' + 4 g + j (j < 4)
      //      or 16 t1' + 4 g + j - 4 (j >= 4), which is where lane (head, g) holds p already;
      //      lane (channel block n16, g) reads word 16 ct + n16 (8 channels) of those 8 entries
      //      and nibble-interleaves pairs of them as in the other path.
  #pragma unroll
      for (int ci = 0; ci < kPVT; ++ci)
  #pragma unroll
        for (int mm = 0; mm < 8; ++mm) acc[ci][mm] = (v4f){0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int ks = 0; ks < (qk_wave ? kAttTPW / 2 : 0); ++ks) {
        v8h pa;
  #pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          pa[rr] = (_Float16)pr[2 * ks][rr];
          pa[4 + rr] = (_Float16)pr[2 * ks + 1][rr];
        }
  #pragma unroll
        for (int ci = 0; ci < kPVT; ++ci) {
        const int ct = ctb * kPVT + ci;
        uint32_t pw[8];
        v8h sc = {};  // G16: the scales of the 8 K-slot entries, group 8 ct + n16 / 2
        if constexpr (G16)
          sc = __builtin_bit_cast(v8h, make_uint4(e4m3x2_to_f16x2(gpv[0]), e4m3x2_hi_to_f16x2(gpv[0]),
                                                  e4m3x2_to_f16x2(gpv[1]), e4m3x2_hi_to_f16x2(gpv[1])));
  #pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int e = (qw * kAttTPW + 2 * ks + (jj >> 2)) * 16 + 4 * g + (jj & 3);
          pw[jj] = *reinterpret_cast<const uint32_t*>(s_rows + e * kRowBytes + 16 * ((4 * ct + (n16 >> 2)) ^ swz(e)) +
                                                      4 * (n16 & 3));
        }
        uint32_t xe[4], xo[4];
  #pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const uint32_t w0 = pw[2 * p2], w1 = pw[2 * p2 + 1];
          xe[p2] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);  // channels 0,2,4,6
          xo[p2] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);  // channels 1,3,5,7
        }
  #define CSA2_CS_MFMA(M, X, BS)                                                                                 \
    {                                                                                                          \
      const uint4 bw = make_uint4(cvt_pair_f16<BS>(X[0]), cvt_pair_f16<BS>(X[1]), cvt_pair_f16<BS>(X[2]),      \
                                  cvt_pair_f16<BS>(X[3]));                                                     \
      v8h bv = __builtin_bit_cast(v8h, bw);                                                                  \
      if constexpr (G16) bv = bv * sc;                                                                       \
      acc[ci][M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bv, acc[ci][M], 0, 0, 0);                      \
    }
        CSA2_CS_MFMA(0, xe, 0) CSA2_CS_MFMA(1, xo, 0) CSA2_CS_MFMA(2, xe, 1) CSA2_CS_MFMA(3, xo, 1)
        CSA2_CS_MFMA(4, xe, 2) CSA2_CS_MFMA(5, xo, 2) CSA2_CS_MFMA(6, xe, 3) CSA2_CS_MFMA(7, xo, 3)
  #undef CSA2_CS_MFMA
        }
      }
    }
    // ---- CS phase 4: every wave's (m, l) meets in LDS (s_red rows w and kAttWaves + w; the
    //      waves without entries hold (-inf, 0)); after one barrier every wave with a slice
    //      rescales its partial sums by exp(m_w - M) (window waves also by 2^sx; the logit
    //      waves by the main cache's channel scales) into its slice (the rows are dead then),
    //      and 16 threads form the block's (M, sum of exp(m_w - M) l_w) in a fixed order; the
    //      output stage adds the slices.
    if (g == 0) {
      s_red[wave][n16] = m;
      s_red[kAttWaves + wave][n16] = lsum;
    }
    __syncthreads();
    if (tid < kAttHeads) {
      float mx = kNegInf;
#pragma unroll
      for (int w2 = 0; w2 < kWPT; ++w2) mx = fmaxf(mx, s_red[w2][tid]);
      float ls = 0.0f;
#pragma unroll
      for (int w2 = 0; w2 < kWPT; ++w2) {
        const float mw = s_red[w2][tid];
        ls += (mw == kNegInf) ? 0.0f : __expf(mw - mx) * s_red[kAttWaves + w2][tid];
      }
      s_m[tid] = mx;
      s_l[tid] = ls;
    }
    if (qk_wave || win_wave) {
      float csc[kPVT][8];  // logit waves: the channel scales of this lane's output channels
#pragma unroll
      for (int ci = 0; ci < kPVT; ++ci)
#pragma unroll
        for (int mm = 0; mm < 8; ++mm)
          csc[ci][mm] = win_wave ? xdown : (G16 ? 1.0f : s_scale[G16 ? 0 : 128 * (ctb * kPVT + ci) + 8 * n16 + mm]);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int h = 4 * g + rr;
        float mx = kNegInf;
#pragma unroll
        for (int w2 = 0; w2 < kWPT; ++w2) mx = fmaxf(mx, s_red[w2][h]);
        const float mw = s_red[wave][h];
        const float f = (mw == kNegInf) ? 0.0f : __expf(mw - mx);
#pragma unroll
        for (int ci = 0; ci < kPVT; ++ci) {
          float4* o = reinterpret_cast<float4*>(&sO[((size_t)wave * kAttHeads + h) * kOW + 128 * ci]);
          const float* c8 = csc[ci];
          o[n16] = make_float4(acc[ci][0][rr] * f * c8[0], acc[ci][1][rr] * f * c8[1], acc[ci][2][rr] * f * c8[2],
                               acc[ci][3][rr] * f * c8[3]);
          o[16 + n16] = make_float4(acc[ci][4][rr] * f * c8[4], acc[ci][5][rr] * f * c8[5],
                                    acc[ci][6][rr] * f * c8[6], acc[ci][7][rr] * f * c8[7]);
        }
      }
    }
    __syncthreads();
  } else {
  // ---- phase 1b: logits of this wave's kAttTPW tiles of 16 entries.  The channel loop is
    //      outside the tile loop, so each A operand (16 B of q'' per lane) is read from LDS once
    //      for all of the wave's tiles.
    float logit[kAttTPW][4];
    v4f a[kAttTPW];
  #pragma unroll
    for (int t = 0; t < kAttTPW; ++t) a[t] = (v4f){0.f, 0.f, 0.f, 0.f};
  #pragma unroll
    for (int i = 0; i < (qk_wave ? kCT : 0); ++i) {
      uint32_t wd[kAttTPW][4];
      _Float16 gs[kAttTPW][2];
  #pragma unroll
      for (int t = 0; t < kAttTPW; ++t) {
        const int el = (qw * kAttTPW + t) * 16 + n16;  // this lane's entry in the split
        uint4 kv;
        if constexpr (G16) kv = kw[t][i];
        else kv = *reinterpret_cast<const uint4*>(s_rows + el * kRowBytes + 16 * ((4 * i + g) ^ swz(el)));
        wd[t][0] = kv.x; wd[t][1] = kv.y; wd[t][2] = kv.z; wd[t][3] = kv.w;
        gs[t][0] = gs[t][1] = (_Float16)1.0f;
        if (G16) {  // channels 128 i + 32 g + [0, 32): groups 8 i + 2 g and 8 i + 2 g + 1
          gs[t][0] = __builtin_bit_cast(_Float16, sS[(8 * i + 2 * g) * L::kSpad + el]);
          gs[t][1] = __builtin_bit_cast(_Float16, sS[(8 * i + 2 * g + 1) * L::kSpad + el]);
        }
      }
  #pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const v8h av = *reinterpret_cast<const v8h*>(&sA[n16 * L::kApad + 128 * i + 32 * g + 8 * sub]);
  #pragma unroll
        for (int t = 0; t < kAttTPW; ++t) {
          v8h bv = decode8_f16(wd[t][sub]);
          if (G16) bv = bv * gs[t][sub >> 1];
          a[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, a[t], 0, 0, 0);
        }
      }
    }
  #pragma unroll
    for (int t = 0; t < kAttTPW; ++t)
  #pragma unroll
      for (int rr = 0; rr < 4; ++rr) logit[t][rr] = (qk_wave && jt[t] >= 0) ? a[t][rr] * s_down[4 * g + rr] : kNegInf;
  
    // ---- phase 3a: read the PV code words now (staged rows in LDS; G16 on the undivided
    //      grid: global loads, cache hits since the rows were just read) so that they arrive
    //      during the softmax.  Wave
    //      (channel tile ct, entry group eq); lane (channel block n16, group g) takes one
    //      32-bit word (8 channels) of each of the 8 entries el..el+7 of every 32-entry k-step.
    const int ct = CS ? ctb : wave % kCT, eq = CS ? wave : wave / kCT;
    const bool pv_active = eq < kWPT;
    uint32_t pw[kEPW / 32][8];
  #pragma unroll
    for (int ks = 0; ks < kEPW / 32; ++ks) {
      const int el = eq * kEPW + 32 * ks + 8 * g;
  #pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int e = el + jj;
        if constexpr (G16) {
          const int32_t j = sel[e];  // -1 past K (read unconditionally: no branch per load)
          // p is 0 for skipped entries, so any valid row may stand in for them
          pw[ks][jj] = *reinterpret_cast<const uint32_t*>(cb + (int64_t)(j >= 0 ? j : 0) * kRowBytes + 64 * ct + 4 * n16);
        } else {  // word 16 ct + n16 of the staged row
          pw[ks][jj] = *reinterpret_cast<const uint32_t*>(s_rows + e * kRowBytes +
                                                           16 * ((4 * ct + (n16 >> 2)) ^ swz(e)) + 4 * (n16 & 3));
        }
      }
    }
  
    // ---- phase 2: softmax statistics of the split (heads 4g + rr of this lane).  Per-wave
    //      partials go to LDS; 256 threads (one 16-lane row per head) reduce them by DPP.
  #pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      float v = logit[0][rr];
  #pragma unroll
      for (int t = 1; t < kAttTPW; ++t) v = fmaxf(v, logit[t][rr]);
      v = row16_max(v);
      if (n16 == 0) s_red[wave][4 * g + rr] = v;
    }
    __syncthreads();
    static_assert(kAttWaves == 16 && kAttHeads == 16, "one 16-lane row per head reduces the 16 waves");
    if (tid < 256) {
      const float v = row16_max(s_red[tid & 15][tid >> 4]);
      if ((tid & 15) == 0) s_m[tid >> 4] = v;
    }
    __syncthreads();
  #pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = 4 * g + rr;
      const float m = s_m[h];
      float v = 0.0f;
  #pragma unroll
      for (int t = 0; t < (qk_wave ? kAttTPW : 0); ++t) {
        const float p = (m == kNegInf) ? 0.0f : __expf(logit[t][rr] - m);
        const _Float16 ph = (_Float16)p;
        sP[h * L::kPpad + (qw * kAttTPW + t) * 16 + n16] = __builtin_bit_cast(uint16_t, ph);
        v += p;
      }
      v = row16_sum(v);
      if (n16 == 0) s_red[wave][h] = v;
    }
    __syncthreads();
    if (tid < 256) {
      const float v = row16_sum(s_red[tid & 15][tid >> 4]);
      if ((tid & 15) == 0) s_l[tid >> 4] = v;
    }
  
    // ---- phase 3b: o[h][c] = sum_j p[h][j] e[j][c] over this wave's entries and channel
    //      tile.  For each pair of entries the two code words are nibble-interleaved so that
    //      one byte holds the same channel of both entries; one fp4->fp16 pair conversion
    //      then yields the (entry 2p, entry 2p+1) dword the MFMA k-order wants.
    v4f acc[8];
  #pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (pv_active) {
  #pragma unroll
      for (int ks = 0; ks < kEPW / 32; ++ks) {
        const int el = eq * kEPW + 32 * ks + 8 * g;  // first of this lane's 8 entries
        const v8h pa = *reinterpret_cast<const v8h*>(&sP[n16 * L::kPpad + el]);
        // G16: the scales of entries el..el+7 in this lane's group (channels 128 ct + 8 n16 ..)
        v8h sc = {};
        if (G16) sc = *reinterpret_cast<const v8h*>(&sS[(8 * ct + (n16 >> 1)) * L::kSpad + el]);
        uint32_t xe[4], xo[4];
  #pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const uint32_t w0 = pw[ks][2 * p2], w1 = pw[ks][2 * p2 + 1];
          xe[p2] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);  // channels 0,2,4,6
          xo[p2] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);  // channels 1,3,5,7
        }
  #define CSA2_PV_MFMA(M, X, BS)                                                                                  \
    {                                                                                                          \
      const uint4 bw = make_uint4(cvt_pair_f16<BS>(X[0]), cvt_pair_f16<BS>(X[1]), cvt_pair_f16<BS>(X[2]),      \
                                  cvt_pair_f16<BS>(X[3]));                                                     \
      v8h bv = __builtin_bit_cast(v8h, bw);                                                                    \
      if (G16) bv = bv * sc;                                                                                   \
      acc[M] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bv, acc[M], 0, 0, 0);                                \
    }
        CSA2_PV_MFMA(0, xe, 0) CSA2_PV_MFMA(1, xo, 0) CSA2_PV_MFMA(2, xe, 1) CSA2_PV_MFMA(3, xo, 1)
        CSA2_PV_MFMA(4, xe, 2) CSA2_PV_MFMA(5, xo, 2) CSA2_PV_MFMA(6, xe, 3) CSA2_PV_MFMA(7, xo, 3)
  #undef CSA2_PV_MFMA
      }
    }
  
    // ---- phase 4: every entry group writes its partial sums to its own LDS slice (sA and
    //      sP are dead once all waves are past PV); then each thread sums the kWPT slices of
    //      8 channels of one head in a fixed order (deterministic), normalises and stores.
    //      Within a head's 128-channel tile, channels 8 n .. 8 n + 3 sit at float4 n and
    //      8 n + 4 .. 8 n + 7 at float4 16 + n, so that the 16 lanes of a row write (and the
    //      summing threads read) 256 contiguous bytes: with the channels in order the head
    //      rows' writes hit the same banks (four-way conflicts, 1.3 us per wave).
    __syncthreads();
    if (pv_active) {
  #pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float4* o = reinterpret_cast<float4*>(&sO[((size_t)eq * kAttHeads + 4 * g + rr) * kOW + 128 * (CS ? 0 : ct)]);
        o[n16] = make_float4(acc[0][rr], acc[1][rr], acc[2][rr], acc[3][rr]);
        o[16 + n16] = make_float4(acc[4][rr], acc[5][rr], acc[6][rr], acc[7][rr]);
      }
    }
    __syncthreads();
    // items of 4 channels: 128 c0 + 8 n + 4 hf + [0, 4) of head hl sit at float4 16 hf + n of the
    // head's tile in every slice
  }
  constexpr int kOItems = kAttHeads * kOW / 4;
  for (int i = tid; i < kOItems; i += kAttThreads) {
    const int hl = i / (kOW / 4), ci = i % (kOW / 4);
    const int tile = ci >> 5, n = ci & 15, hf = (ci >> 4) & 1;
    const int c = 128 * (ctb * kPVT + tile) + 8 * n + 4 * hf;
    float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int gq = 0; gq < kWPT; ++gq) {
      const float4 a4 = reinterpret_cast<const float4*>(&sO[((size_t)gq * kAttHeads + hl) * kOW + 128 * tile])[16 * hf + n];
      o4.x += a4.x; o4.y += a4.y; o4.z += a4.z; o4.w += a4.w;
    }
    const float l = s_l[hl];
    const float inv_l = (l > 0.0f) ? 1.0f / l : 0.0f;
    float o[4] = {o4.x * inv_l, o4.y * inv_l, o4.z * inv_l, o4.w * inv_l};
    const int h = hg * kAttHeads + hl;
    if (!G16 && !CS) {  // (CS: already in the slices)
#pragma unroll
      for (int m = 0; m < 4; ++m) o[m] *= s_scale[c + m];
    }
    if (P == 1) {
      const int64_t oi = ((int64_t)r * Hq + h) * D + c;
      if (out_bf16) {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + oi) =
            make_uint2(pack2(bf16_rne(o[0]), bf16_rne(o[1])), pack2(bf16_rne(o[2]), bf16_rne(o[3])));
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
      }
    } else {
      *reinterpret_cast<float4*>(part + (((int64_t)r * P + split) * Hq + h) * D + c) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  if (tid < kAttHeads && ctb == 0) {
    const float l = s_l[tid];
    if (P == 1) {
      if (lse) lse[(int64_t)r * Hq + hg * kAttHeads + tid] = (l > 0.0f) ? s_m[tid] + __logf(l) : kNegInf;
    } else {
      float* ml = part_ml + (((int64_t)r * P + split) * Hq + hg * kAttHeads + tid) * 2;
      ml[0] = s_m[tid];
      ml[1] = l;
    }
  }
}

// Merge the P partials of (row, head group, channel tile) by log-sum-exp.  Thread t: head
// t / 16 of the group, channels 128 ct + 8 (t % 16) + [0, 8); all partial loads are issued
// before any is used.
template <int D>
__global__ __launch_bounds__(256) void k_attend_combine(int T, int Hq, int P, const float* __restrict__ part,
                                                        const float* __restrict__ part_ml, void* __restrict__ out,
                                                        int out_bf16, float* __restrict__ lse) {
  constexpr int kCT = D / 128;
  constexpr int kMaxP = CSA2_MAX_K_DEV / kAttSplit + 1;
  __shared__ float s_w[kMaxP][kAttHeads];
  const int hg = blockIdx.x / kCT, ct = blockIdx.x % kCT, r = blockIdx.y;
  const int tid = threadIdx.x;
  const int hl = tid >> 4, c = 128 * ct + 8 * (tid & 15);
  const int h = hg * kAttHeads + hl;
  float4 pv[kMaxP][2];
#pragma unroll
  for (int s = 0; s < kMaxP; ++s) {
    if (s < P) {
      const float4* src = reinterpret_cast<const float4*>(part + (((int64_t)r * P + s) * Hq + h) * D + c);
      pv[s][0] = src[0];
      pv[s][1] = src[1];
    }
  }
  if (tid < kAttHeads) {
    const float* ml = part_ml + ((int64_t)r * P) * Hq * 2;
    const int hh = hg * kAttHeads + tid;
    float mv[kMaxP], lv[kMaxP];
    float M = kNegInf;
#pragma unroll
    for (int s = 0; s < kMaxP; ++s) {
      mv[s] = (s < P) ? ml[((int64_t)s * Hq + hh) * 2] : kNegInf;
      lv[s] = (s < P) ? ml[((int64_t)s * Hq + hh) * 2 + 1] : 0.0f;
      if (lv[s] > 0.0f) M = fmaxf(M, mv[s]);
    }
    float Z = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxP; ++s) {
      const float wgt = (lv[s] > 0.0f) ? lv[s] * __expf(mv[s] - M) : 0.0f;
      s_w[s][tid] = wgt;
      Z += wgt;
    }
    const float inv = (Z > 0.0f) ? 1.0f / Z : 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxP; ++s) s_w[s][tid] *= inv;
    if (lse && ct == 0) lse[(int64_t)r * Hq + hh] = (Z > 0.0f) ? M + __logf(Z) : kNegInf;
  }
  __syncthreads();
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxP; ++s) {
    if (s < P) {
      const float wgt = s_w[s][hl];
      o[0] = fmaf(wgt, pv[s][0].x, o[0]); o[1] = fmaf(wgt, pv[s][0].y, o[1]);
      o[2] = fmaf(wgt, pv[s][0].z, o[2]); o[3] = fmaf(wgt, pv[s][0].w, o[3]);
      o[4] = fmaf(wgt, pv[s][1].x, o[4]); o[5] = fmaf(wgt, pv[s][1].y, o[5]);
      o[6] = fmaf(wgt, pv[s][1].z, o[6]); o[7] = fmaf(wgt, pv[s][1].w, o[7]);
    }
  }
  const int64_t oi = ((int64_t)r * Hq + h) * D + c;
  if (out_bf16) {
    uint32_t w4[4];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) w4[k2] = pack2(bf16_rne(o[2 * k2]), bf16_rne(o[2 * k2 + 1]));
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + oi) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  } else {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + oi);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  }
}

// fp32 path: one block per (row, head).  Dequantised value of channel c of cache row j of
// sequence b: E2M1 * s_c (per channel) or E2M1 * E4M3 group scale (G16).
template <bool G16>
__device__ __forceinline__ float deq_f32(const uint8_t* cb, const uint8_t* gsb, const float* s_scale, int D,
                                         int32_t j, int c) {
  const uint32_t byte = cb[(int64_t)j * (D / 2) + c / 2];
  const float e = e2m1_value((c & 1) ? (byte >> 4) : (byte & 15u));
  return G16 ? e * e4m3_value(gsb[(int64_t)j * (D / 16) + c / 16]) : e * s_scale[c];
}

// Entries 0 .. K-1 come from the selection (FP4 cache), entries K .. K+nw-1 from the
// sliding window (E4M3 rows with one fp32 scale each: E4M3 * s_row).
template <bool G16>
__global__ __launch_bounds__(256) void k_attend_f32(int T, int Hq, int D, int K, const float* __restrict__ q,
                                                    const uint8_t* __restrict__ codes,
                                                    const void* __restrict__ scales_v, int64_t n_max,
                                                    const int32_t* __restrict__ idx, const uint8_t* __restrict__ wcodes,
                                                    const float* __restrict__ wscales, int64_t wn_max,
                                                    const int32_t* __restrict__ wend, int window, float softmax_scale,
                                                    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float s_q[CSA2_MAX_D_DEV];
  __shared__ float s_scale[CSA2_MAX_D_DEV];
  __shared__ float s_logit[CSA2_MAX_K_DEV + CSA2_MAX_WINDOW_DEV];
  __shared__ int32_t s_idx[CSA2_MAX_K_DEV];
  __shared__ float s_red[8];
  const int h = blockIdx.x, r = blockIdx.y, b = r / T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* qh = q + ((int64_t)r * Hq + h) * D;
  int64_t w_end = 0, w_start = 0;
  if (wcodes) {
    w_end = wend[r] < wn_max ? wend[r] : wn_max;
    w_start = w_end - window > 0 ? w_end - window : 0;
  }
  const int nw = w_end > w_start ? (int)(w_end - w_start) : 0;
  const int E = K + nw;
  const uint8_t* wrow = wcodes ? wcodes + ((int64_t)b * wn_max + w_start) * D : nullptr;
  const float* wsc = wcodes ? wscales + (int64_t)b * wn_max + w_start : nullptr;
  for (int c = tid; c < D; c += 256) {
    s_q[c] = qh[c];
    if (!G16) s_scale[c] = static_cast<const float*>(scales_v)[(int64_t)b * D + c];
  }
  for (int e = tid; e < K; e += 256) {
    const int32_t j = idx[(int64_t)r * K + e];
    s_idx[e] = (j >= 0 && j < n_max) ? j : -1;
  }
  __syncthreads();
  const uint8_t* cb = codes + (int64_t)b * n_max * (D / 2);
  const uint8_t* gsb = G16 ? static_cast<const uint8_t*>(scales_v) + (int64_t)b * n_max * (D / 16) : nullptr;
  for (int e = wave; e < E; e += 4) {
    float dot = 0.0f;
    bool ok;
    if (e < K) {
      const int32_t j = s_idx[e];
      ok = j >= 0;
      if (ok)
        for (int c = lane; c < D; c += 64) dot = fmaf(s_q[c], deq_f32<G16>(cb, gsb, s_scale, D, j, c), dot);
    } else {
      ok = true;
      const uint8_t* row = wrow + (int64_t)(e - K) * D;
      for (int c = lane; c < D; c += 64) dot = fmaf(s_q[c], e4m3_value(row[c]), dot);
      dot *= wsc[e - K];
    }
    dot = wave_sum(dot);
    if (lane == 0) s_logit[e] = ok ? dot * softmax_scale : kNegInf;
  }
  __syncthreads();
  float m = kNegInf;
  for (int e = tid; e < E; e += 256) m = fmaxf(m, s_logit[e]);
  m = wave_max(m);
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float z = 0.0f;
  for (int e = tid; e < E; e += 256) {
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
      o = fmaf(s_logit[e], deq_f32<G16>(cb, gsb, s_scale, D, j, c), o);
    }
    for (int e = 0; e < nw; ++e) o = fmaf(s_logit[K + e], e4m3_value(wrow[(int64_t)e * D + c]) * wsc[e], o);
    out[((int64_t)r * Hq + h) * D + c] = o * inv;
  }
  if (lse && tid == 0) lse[(int64_t)r * Hq + h] = (z > 0.0f) ? m + logf(z) : kNegInf;
}

int attend_splits(int K) { return (K + kAttSplit - 1) / kAttSplit; }

// partial slots: the selection's splits, plus one for the sliding window
static int attend_parts(int K, bool window) { return attend_splits(K) + (window ? 1 : 0); }

size_t attend_ws_floats(int R, int Hq, int D, int K, int window) {
  const int P = attend_parts(K, window > 0);
  if (P <= 1) return 0;
  return (size_t)R * P * Hq * D + (size_t)R * P * Hq * 2;
}

template <int D, bool G16, bool CS, bool WIN>
static void launch_mfma(const AttendArgs& a, int S, int P, hipStream_t st) {
  // the window (if any) is one more block column, run beside the selection's splits
  // one block per (unit = (row, split or window), head group[, channel tile]), dealt in
  // XCD-aware order
  const int units = (S + ((a.swa_codes && !CS) ? 1 : 0)) * a.B * a.T;
  const int ncb = CS ? (D / 128 < kCSBlocks ? D / 128 : kCSBlocks) : 1;
  const dim3 g((unsigned)(8 * (a.Hq / kAttHeads) * ncb * ((units + 7) / 8)));
  float* part_ml = a.part ? a.part + (size_t)a.B * a.T * P * a.Hq * D : nullptr;
  hipLaunchKernelGGL((k_attend_part<D, G16, CS, WIN>), g, dim3(kAttThreads), 0, st, a.B * a.T, a.T, a.Hq, a.K, S, P,
                     (const uint16_t*)a.q, a.codes, a.scales, a.n_max, a.idx, a.softmax_scale, a.out, (int)a.out_bf16, a.lse, a.part, part_ml, a.swa_codes,
                     a.swa_scales, a.swa_n_max, a.swa_end, a.window);
  if (P > 1)
    hipLaunchKernelGGL(k_attend_combine<D>, dim3(a.Hq / kAttHeads * (D / 128), a.B * a.T), dim3(256), 0, st, a.T,
                       a.Hq, P, (const float*)a.part, (const float*)part_ml, a.out, (int)a.out_bf16, a.lse);
}

template <int D>
static void launch_mfma_d(const AttendArgs& a, int S, int P, bool cs, hipStream_t st) {
  if (a.g16 && cs)
    launch_mfma<D, true, true, false>(a, S, P, st);
  else if (a.g16)  // with a window: one more block column and partial slot, merged by k_attend_combine
    launch_mfma<D, true, false, false>(a, S, P, st);
  else if (!cs)  // likewise
    launch_mfma<D, false, false, false>(a, S, P, st);
  else if (a.swa_codes)  // the window in the selection's blocks and softmax
    launch_mfma<D, false, true, true>(a, S, P, st);
  else
    launch_mfma<D, false, true, false>(a, S, P, st);
}

// the channel-split kernel when its grid fits one round of blocks (G16: without a window)
static bool attend_channel_split(const AttendArgs& a, int S) {
  const long ncb = a.D / 128 < kCSBlocks ? a.D / 128 : kCSBlocks;
  return (!a.g16 || !a.swa_codes) && (long)a.B * a.T * S * (a.Hq / kAttHeads) * ncb <= kCSMaxBlocks;
}

int launch_attend(const AttendArgs& a, hipStream_t st) {
  const int R = a.B * a.T;
  if (a.swa_codes && (a.window < 1 || a.window > kWinMax)) return -1;
  if (!a.q_bf16) {
    if (a.g16)
      hipLaunchKernelGGL(k_attend_f32<true>, dim3(a.Hq, R), dim3(256), 0, st, a.T, a.Hq, a.D, a.K,
                         (const float*)a.q, a.codes, a.scales, a.n_max, a.idx, a.swa_codes, a.swa_scales,
                         a.swa_n_max, a.swa_end, a.window, a.softmax_scale, (float*)a.out, a.lse);
    else
      hipLaunchKernelGGL(k_attend_f32<false>, dim3(a.Hq, R), dim3(256), 0, st, a.T, a.Hq, a.D, a.K,
                         (const float*)a.q, a.codes, a.scales, a.n_max, a.idx, a.swa_codes, a.swa_scales,
                         a.swa_n_max, a.swa_end, a.window, a.softmax_scale, (float*)a.out, a.lse);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int S = attend_splits(a.K);
  // with the channel split the window is attended inside the selection's blocks; otherwise
  // it takes one more partial slot
  const bool cs = attend_channel_split(a, S);
  const int P = attend_parts(a.K, a.swa_codes != nullptr && !cs);
  if (P > 1 && !a.part) return -1;
  switch (a.D) {
    case 128: launch_mfma_d<128>(a, S, P, cs, st); break;
    case 256: launch_mfma_d<256>(a, S, P, cs, st); break;
    case 512: launch_mfma_d<512>(a, S, P, cs, st); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
