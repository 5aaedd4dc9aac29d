// Internal host-side launchers (one per kernel family).  Arguments are validated by the
// C ABI layer before these are called; launchers return 0 or -1 (launch error).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// per-row state of the distributed Top-K select (zeroed before each use)
struct RowCtl {
  uint32_t ncand;  // candidates appended so far
  uint32_t done;   // blocks of the select kernel finished
  uint32_t pad[2];
};

int launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);

int launch_quantize_fp4(bool compute, bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst,
                        const int32_t* n0, int64_t n_max, uint8_t* codes, float* scales, hipStream_t st);
int launch_quantize_fp8(bool bf16, int B, int T, int D, const void* x, int64_t xsb, int64_t xst, const int32_t* n0,
                        int64_t n_max, uint8_t* codes, float* scales, hipStream_t st);

struct ScoreArgs {
  int prec;           // 0 fp32, 1 fp8
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
};
int launch_score(const ScoreArgs& a, hipStream_t st);
int score_cols_per_block(int64_t ncols);

// Top-K select from scores whose histogram is in `hist`; ctl zeroed on entry.
int launch_topk_hist(int R, int64_t ncols, const float* scores, const int32_t* cand, uint32_t* hist, hipStream_t st);
int launch_topk_select(int R, int64_t ncols, const float* scores, const int32_t* cand, int K, const uint32_t* hist,
                       RowCtl* ctl, uint2* candbuf, int32_t* idx_out, float* val_out, hipStream_t st);

struct AttendArgs {
  int B, T, Hq, D, K;
  const void* q;
  bool q_bf16;
  const uint8_t* codes;
  const float* scales;
  int64_t n_max;
  const int32_t* idx;
  float softmax_scale;
  void* out;
  bool out_bf16;
  float* lse;
  int splits;         // MFMA path: number of entry groups
  float* part_o;      // [R][splits][Hq][D]
  float* part_ml;     // [R][splits][Hq][2]
  uint32_t* counters; // [R][Hq/16], zeroed on entry
};
int launch_attend(const AttendArgs& a, hipStream_t st);
int attend_entries_per_split();

int launch_gather_dequant(int B, int T, int K, int D, const uint8_t* codes, const float* scales, int64_t n_max,
                          const int32_t* idx, float* out, hipStream_t st);
int launch_coarse_keys(int B, int64_t n_max, const int32_t* n_keys, int dk, int block, const uint8_t* k8,
                       const float* k_scale, uint8_t* kb8, float* kb_scale, hipStream_t st);
int launch_expand_blocks(int B, int KB, int block, const int32_t* blocks, const int32_t* n_keys, int32_t* cand,
                         hipStream_t st);

}  // namespace csa2
