// Internal host-side launchers (one per kernel family).  Arguments are validated by the
// C ABI layer before these are called; launchers return 0 or -1 (launch error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// per-row state of the distributed Top-K select (zeroed before each use)
struct RowCtl {
  uint32_t pad;
  uint32_t beta;   // first-level bin holding the K-th largest score (written by the filter)
  uint32_t above;  // visible scores in first-level bins above beta
  uint32_t keff;   // min(K, visible scores)
};

int launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);

int launch_quantize_fp4(bool compute, bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                        const int32_t* n0, int64_t n_max, uint8_t* codes, float* scales, hipStream_t st);
// the pages' layout: codes [B][n_max][D/2], gscales [B][n_max][D/16] E4M3 bytes (D % 16 == 0)
int launch_quantize_fp4_g16(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                            const int32_t* n0, int64_t n_max, uint8_t* codes, uint8_t* gscales, hipStream_t st);
// E2M1 with one absmax/6 scale per row (4-bit indexer keys): codes [B][n_max][D/2]
int launch_quantize_fp4_rows(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                             const int32_t* n0, int64_t n_max, uint8_t* codes, float* scales, hipStream_t st);
int launch_quantize_fp8(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst, const int32_t* n0,
                        int64_t n_max, uint8_t* codes, float* scales, hipStream_t st);

// Candidate lists a LOCAL score kernel writes for k_topk_select: per row and score block
// (nreg blocks of `stride` columns), the visible scores above the block's cut as (order
// key, position) pairs in column order, their count, the cut (-1: every visible score
// listed) and the block's visible count.
struct LocalCand {
  uint2* cand;      // [R][nreg][stride]
  uint32_t* cnt;    // [R][nreg]
  int32_t* cut;     // [R][nreg]
  uint32_t* vis;    // [R][nreg]
  int stride;       // candidate slots per region (a block lists at most this many)
  int rcols;        // columns per score block (region)
  int K;            // the Top-K the lists serve (sizes the per-block cap)
  int store;        // also write every score (a later step reads them all)
};

struct ScoreArgs {
  int prec;           // 0 fp32, 1 fp8, 2 fp4
  bool q_bf16;
  int B, T, H, dk;
  const void* q;
  const float* w;
  const void* k;
  const float* k_scale;
  int64_t n_max;
  const int32_t* n_keys;
  const int32_t* q_limit;
  const int32_t* cand;
  int64_t ncols;
  float* scores;
  uint32_t* hist;     // nullable: [R][kHistBins], must be zero on entry
  int key_div;        // 1, or the coarse block size when columns are blocks
  uint8_t* qstage;    // nullable: score_stage_bytes(R) of scratch for the many-row fp8 path
  bool keep;          // decode scan whose keys a later layer reads again: cached loads
  bool local;         // decode fp8/fp4 scan that also writes candidate lists (lc)
  LocalCand lc;
};
int launch_score(const ScoreArgs& a, hipStream_t st);
// Many-row fp8 scoring (chunked prefill) stages the quantised query rows: E4M3 codes and
// head factors, R * (2048 + 128) bytes; used when T >= score_tiled_min_rows().
inline size_t score_stage_bytes(int64_t R) { return (size_t)R * (32 * 64 + 32 * 4); }
inline int score_tiled_min_rows() { return 8; }
int score_cols_per_block(int64_t rows, int64_t ncols);
int rows_list_cols();  // columns per region of the many-row kernel's candidate lists
// score blocks per row of a decode scan (= candidate regions of a LOCAL scan)
inline int score_blocks(int64_t rows, int64_t ncols) {
  const int cpb = score_cols_per_block(rows, ncols);
  return (int)((ncols + cpb - 1) / cpb);
}
// The exact Top-K from a LOCAL scan's candidate lists (a = the scan's arguments: rows, its
// lc, nreg = score_blocks regions per row; sorted: the candidate positions ascend with the
// column, so the winners come out ascending).  A block whose list may miss winners is
// re-scored by the select workgroup with the scan's arithmetic into a.scores ([R][ncols],
// written only there) and re-read whole.
// The candidate-list cap of one score block of kcols columns in a row of nvis visible
// columns: four times the Top-K winners such a block holds on average plus a margin, in
// multiples of 32, at most the block's columns and its slots.  The cut falls on a whole
// first-level bin (a quarter octave of the score), and the bin holding the K-th score can
// hold a few times the winners above it, all of which must be listed.
// margins: 32 for the decode scans' lists; 16 for the many-row prefill kernel, whose rows of
// hundreds of regions must still fit the selection's staging
constexpr int64_t kListMargin = 32, kRowsListMargin = 16;
__host__ __device__ inline int64_t list_cap(int64_t K, int64_t kcols, int64_t nvis, int64_t margin, int64_t slots) {
  const int64_t mu2 = nvis > 0 ? (4 * K * kcols + nvis - 1) / nvis : kcols;
  int64_t cap = ((mu2 + margin + 31) / 32) * 32;
  if (cap > kcols) cap = kcols;
  return cap < slots ? cap : slots;
}
// expand_out (nullable): the winners are blocks of expand_block positions; their positions
// ([R][K * expand_block], -1 past n_keys or for padding) are written there as well.
int launch_topk_select(const ScoreArgs& a, int K, bool sorted, int nreg, int32_t* idx_out, float* val_out,
                       hipStream_t st, uint32_t* clear = nullptr, int64_t clear_words = 0, int expand_block = 0,
                       int32_t* expand_out = nullptr);

// Top-K: histogram (zeroed on entry) -> filter into candidates (ctl zeroed on entry)
// -> finalize (here, or fused into the attention kernel).
int launch_topk_hist(int R, int64_t ncols, const float* scores, const int32_t* cand, uint32_t* hist, hipStream_t st);
// bmax [R][ceil(ncols / block)]: block maxima of the scores; hist (zeroed on entry): their
// first-level histogram
int launch_block_max(int R, int64_t ncols, int block, const float* scores, float* bmax, uint32_t* hist,
                     hipStream_t st);
// hist2 [R][kHistBins]: second-level histogram of the threshold bin (zeroed on entry).
// candbuf [R][regions][topk_region_cols(R)] and cnt [R][regions], regions = topk_regions.
int topk_region_cols(int R);
int topk_regions(int R, int64_t ncols);
// clear (nullable, 16-byte aligned, clear_words a multiple of 4): words the filter blocks
// zero on the side (the next selection's histograms and control words)
int launch_topk_filter(int R, int64_t ncols, const float* scores, const int32_t* cand, int K, const uint32_t* hist,
                       uint32_t* hist2, RowCtl* ctl, uint2* candbuf, uint32_t* cnt, hipStream_t st,
                       uint32_t* clear = nullptr, int64_t clear_words = 0);
// sorted: the candidates were filtered without a candidate map (list in position order)
// expand_out (nullable, needs sorted): also write the selected blocks' positions (block
// positions per selected column, -1 past n_keys[r] or for padding), [R][K * block]
int launch_topk_finalize(int R, int64_t ncols, int K, bool sorted, const RowCtl* ctl, const uint32_t* hist2,
                         const uint2* candbuf, const uint32_t* cnt, int32_t* idx_out, float* val_out, hipStream_t st,
                         int block = 0, const int32_t* n_keys = nullptr, int32_t* expand_out = nullptr,
                         int rps = 1);

struct AttendArgs {
  int B, T, Hq, D, K;
  const void* q;
  bool q_bf16;
  const uint8_t* codes;
  const void* scales;     // fp32 [B][D] (per channel) or E4M3 bytes [B][n_max][D/16] (g16)
  bool g16;
  int64_t n_max;
  const int32_t* idx;
  float softmax_scale;
  void* out;
  bool out_bf16;
  float* lse;
  float* part;        // MFMA path with more than one partial: partial results (attend_ws_floats)
  // sliding window (swa_codes null: none): E4M3 rows [B][swa_n_max][D], scales [B][swa_n_max]
  const uint8_t* swa_codes;
  const float* swa_scales;
  int64_t swa_n_max;
  const int32_t* swa_end;  // [B][T]
  int window;
};
int launch_attend(const AttendArgs& a, hipStream_t st);
int attend_splits(int K);
size_t attend_ws_floats(int R, int Hq, int D, int K, int window);

int launch_gather_dequant(bool g16, int B, int T, int K, int D, const uint8_t* codes, const void* scales,
                          int64_t n_max, const int32_t* idx, float* out, hipStream_t st);
// q_limit[b * T + t] = n_keys[b] - T + t: the causal limit of T decode tokens whose own
// entries are the cache's last T
int launch_causal_limits(int B, int T, const int32_t* n_keys, int32_t* q_limit, hipStream_t st);
int launch_coarse_keys(int B, int64_t n_max, const int32_t* n_keys, int dk, int block, const uint8_t* k8,
                       const float* k_scale, uint8_t* kb8, float* kb_scale, hipStream_t st);
// read-stream probe: `bytes` (a multiple of 16, 16-byte aligned) read once by `blocks` blocks
int launch_stream_read(const void* p, int64_t bytes, int blocks, uint32_t* sink, hipStream_t st);
}  // namespace csa2
