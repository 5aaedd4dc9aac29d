// C ABI of the CSA2 library: host-side validation, workspace layout and launch order.
// Every entry point validates all arguments before launching anything; nothing here
// synchronises with the device, allocates device memory or keeps state beyond the cached
// device check.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/csa2.h"
#include "common.hpp"
#include "launch.hpp"
#include "topk_dev.hpp"

using namespace csa2;

namespace {

constexpr int kMaxDevices = 64;
int g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::mutex g_dev_mu;

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CSA2_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return CSA2_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return CSA2_ERR_DEVICE;
    g_dev_ok[dev] = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return g_dev_ok[dev] == 1 ? CSA2_OK : CSA2_ERR_UNSUPPORTED;
}

inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int dev_status(int rc) { return rc ? CSA2_ERR_DEVICE : CSA2_OK; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// Top-K columns per row this build handles (the finaliser keeps per-region counts in LDS)
constexpr int64_t kMaxTopkCols = (int64_t)kFinMaxRegions * kFilterColsNarrow;

// Bump allocator over the caller's workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
    off += align256(count * sizeof(T));
    return p;
  }
};

// ---- Top-K workspace: hist [R][bins] | hist2 [R][bins] | ctl [R] (zeroed per use) |
//      candidate regions [R][regions][kFilterColsPerBlock] | counts [R][regions]
size_t topk_zero_bytes(int64_t R) {
  return 2 * align256((size_t)R * kHistBins * 4) + align256((size_t)R * sizeof(RowCtl));
}
size_t cand_bytes(int64_t R, int64_t ncols) {
  const int64_t nreg = topk_regions((int)R, ncols);
  return align256((size_t)R * nreg * topk_region_cols((int)R) * sizeof(uint2)) + align256((size_t)R * nreg * 4);
}
size_t topk_ws(int64_t R, int64_t ncols) { return topk_zero_bytes(R) + cand_bytes(R, ncols); }
struct TopkWs {
  uint32_t* hist;
  uint32_t* hist2;
  RowCtl* ctl;
  uint2* cand;
  uint32_t* cnt;
};
struct CandWs {
  uint2* cand;
  uint32_t* cnt;
};
CandWs carve_cand(Carve& c, int64_t R, int64_t ncols) {
  const int64_t nreg = topk_regions((int)R, ncols);
  CandWs w;
  w.cand = c.take<uint2>((size_t)R * nreg * topk_region_cols((int)R));
  w.cnt = c.take<uint32_t>((size_t)R * nreg);
  return w;
}
TopkWs carve_topk_zero(Carve& c, int64_t R) {
  TopkWs t;
  t.hist = c.take<uint32_t>((size_t)R * kHistBins);
  t.hist2 = c.take<uint32_t>((size_t)R * kHistBins);
  t.ctl = c.take<RowCtl>((size_t)R);
  t.cand = nullptr;
  t.cnt = nullptr;
  return t;
}
TopkWs carve_topk(Carve& c, int64_t R, int64_t ncols) {
  TopkWs t = carve_topk_zero(c, R);
  CandWs w = carve_cand(c, R, ncols);
  t.cand = w.cand;
  t.cnt = w.cnt;
  return t;
}
// zero the histograms and control words (contiguous at the start of the Top-K workspace)
int zero_topk(const TopkWs& t, int64_t R, hipStream_t st) {
  return launch_fill_u32(t.hist, (int64_t)(topk_zero_bytes(R) / 4), 0u, st);
}

// ---- candidate lists of LOCAL decode scans: pairs [R][nreg][stride] | cnt, cut, vis [R][nreg]
size_t local_pairs(int64_t R, int64_t ncols) {
  return (size_t)R * score_blocks(R, ncols) * score_cols_per_block(R, ncols);
}
size_t local_regions(int64_t R, int64_t ncols) { return (size_t)R * score_blocks(R, ncols); }
size_t local_ws(size_t pairs, size_t regions) {
  return align256(pairs * sizeof(uint2)) + 3 * align256(regions * 4);
}
size_t local_ws(int64_t R, int64_t ncols) { return local_ws(local_pairs(R, ncols), local_regions(R, ncols)); }
LocalCand carve_local(Carve& c, size_t pairs, size_t regions) {
  LocalCand l;
  l.cand = c.take<uint2>(pairs);
  l.cnt = c.take<uint32_t>(regions);
  l.cut = c.take<int32_t>(regions);
  l.vis = c.take<uint32_t>(regions);
  l.stride = 0;
  l.rcols = 0;
  l.K = 0;
  l.store = 0;
  return l;
}
// the same storage set up for a scan of ncols columns
LocalCand local_for(LocalCand l, int64_t R, int64_t ncols, int K) {
  l.stride = score_cols_per_block(R, ncols);
  l.rcols = l.stride;
  l.K = K;
  return l;
}
// the many-row fp8 kernel of chunked prefill (no candidate map, T >= 8 rows per sequence)
bool rows_scan(int prec, int T, const int32_t* cand) {
  return prec == CSA2_PREC_FP8 && !cand && T >= score_tiled_min_rows();
}
// decode scans (the fp8 / fp4 indexer's k_score_fp8) list their candidates for k_topk_select
// rows whose candidate lists fit the selection's staging: at most kLocalMaxRegions score
// blocks per row (262144 columns at 2048 per block); longer rows (a flat scan of a million
// entries) take the histogram filter, whose candidates do fit
constexpr int kLocalMaxRegions = 128;
bool local_fits(int64_t R, int64_t ncols) { return score_blocks(R, ncols) <= kLocalMaxRegions; }
bool local_scan(int prec, int T, const int32_t* cand, int64_t R, int64_t ncols) {
  return prec != CSA2_PREC_FP32 && !rows_scan(prec, T, cand) && local_fits(R, ncols);
}
// candidate lists of the many-row kernel: regions of rows_list_cols() columns, each listing
// at most kRowsSlots candidates (its cap: four times a region's expected winners plus 32,
// about 40 at 4096 x 262144; a region needing more is re-scored by the selection)
constexpr int kRowsSlots = 128;
int rows_regions(int64_t ncols) { return (int)((ncols + rows_list_cols() - 1) / rows_list_cols()); }
size_t rows_local_ws(int64_t R, int64_t ncols) {
  const size_t regions = (size_t)R * rows_regions(ncols);
  return local_ws(regions * kRowsSlots, regions);
}

bool valid_dtype(int d) { return d == CSA2_F32 || d == CSA2_BF16; }

// main-KV layouts the attention reads
int check_kv_fmt(int kv_fmt, int D) {
  if (kv_fmt != CSA2_FMT_FP4_PER_CHANNEL && kv_fmt != CSA2_FMT_FP4_G16) return CSA2_ERR_DTYPE;
  if (kv_fmt == CSA2_FMT_FP4_G16 && D % 16) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

int check_attend_shape(int B, int T, int Hq, int D, int K, int q_dtype, int out_dtype) {
  if (B < 1 || T < 1 || Hq < 1 || Hq > CSA2_MAX_HQ || D < 2 || D > CSA2_MAX_D || K < 1 || K > CSA2_MAX_K)
    return CSA2_ERR_SHAPE;
  if (!valid_dtype(q_dtype) || !valid_dtype(out_dtype)) return CSA2_ERR_DTYPE;
  if (D % 2) return CSA2_ERR_SHAPE;
  if (q_dtype == CSA2_F32) {
    if (out_dtype != CSA2_F32) return CSA2_ERR_DTYPE;
  } else {
    if (Hq % 16 || (D != 128 && D != 256 && D != 512)) return CSA2_ERR_UNSUPPORTED;
  }
  if ((int64_t)B * T > 65535) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

AttendArgs attend_args(int B, int T, int Hq, int D, int K, const void* q, int q_dtype, int kv_fmt,
                       const uint8_t* codes, const void* scales, int64_t n_max, const int32_t* idx,
                       float softmax_scale, void* out, int out_dtype, float* lse) {
  AttendArgs a;
  a.B = B; a.T = T; a.Hq = Hq; a.D = D; a.K = K;
  a.q = q; a.q_bf16 = (q_dtype == CSA2_BF16);
  a.codes = codes; a.scales = scales; a.g16 = (kv_fmt == CSA2_FMT_FP4_G16); a.n_max = n_max; a.idx = idx;
  a.softmax_scale = softmax_scale; a.out = out; a.out_bf16 = (out_dtype == CSA2_BF16); a.lse = lse;
  a.part = nullptr;
  a.swa_codes = nullptr; a.swa_scales = nullptr; a.swa_n_max = 0; a.swa_end = nullptr; a.window = 0;
  return a;
}

// a layer's sliding-window cache
int check_swa(const csa2_swa* w, int max_window) {
  if (!w) return CSA2_OK;
  if (!w->codes || !w->scales || !w->end) return CSA2_ERR_NULL;
  if (w->window < 1 || w->window > CSA2_MAX_WINDOW || w->window > max_window || w->n_max < 1) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

void set_swa(AttendArgs& a, const csa2_swa* w) {
  a.swa_codes = w ? w->codes : nullptr;
  a.swa_scales = w ? w->scales : nullptr;
  a.swa_n_max = w ? w->n_max : 0;
  a.swa_end = w ? w->end : nullptr;
  a.window = w ? w->window : 0;
}

int check_index_shape(int prec, int B, int T, int H, int dk, int q_dtype, const void* k_scale, int64_t ncols) {
  if (B < 1 || T < 1 || ncols < 1) return CSA2_ERR_SHAPE;
  if ((int64_t)B * T > 65535) return CSA2_ERR_SHAPE;
  if (!valid_dtype(q_dtype)) return CSA2_ERR_DTYPE;
  if (prec == CSA2_PREC_FP32) {
    if (q_dtype != CSA2_F32) return CSA2_ERR_DTYPE;
    if (H < 1 || H > CSA2_MAX_H || dk < 1 || dk > CSA2_MAX_DK || (int64_t)H * dk > 8192) return CSA2_ERR_SHAPE;
  } else if (prec == CSA2_PREC_FP8 || prec == CSA2_PREC_FP4) {
    if (H != 32 || dk != 64) return CSA2_ERR_UNSUPPORTED;
    if (!k_scale) return CSA2_ERR_NULL;
  } else {
    return CSA2_ERR_DTYPE;
  }
  return CSA2_OK;
}

ScoreArgs score_args(int prec, int B, int T, int H, int dk, const void* q, int q_dtype, const float* w, const void* k,
                     const float* k_scale, int64_t n_max, const int32_t* n_keys, const int32_t* q_limit,
                     const int32_t* cand, int64_t ncols, float* scores, uint32_t* hist, int key_div) {
  ScoreArgs a;
  a.prec = prec;
  a.q_bf16 = (q_dtype == CSA2_BF16);
  a.B = B; a.T = T; a.H = H; a.dk = dk;
  a.q = q; a.w = w; a.k = k; a.k_scale = k_scale;
  a.n_max = n_max; a.n_keys = n_keys; a.q_limit = q_limit; a.cand = cand;
  a.ncols = ncols; a.scores = scores; a.hist = hist; a.key_div = key_div;
  a.qstage = nullptr;
  a.keep = false;
  a.local = false;
  a.lc = LocalCand{nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0};
  return a;
}

// filter + finalize
int select_topk(int R, int64_t ncols, const float* scores, const int32_t* cand, int K, const TopkWs& t,
                int32_t* idx_out, float* val_out, hipStream_t st) {
  if (launch_topk_filter(R, ncols, scores, cand, K, t.hist, t.hist2, t.ctl, t.cand, t.cnt, st)) return -1;
  return launch_topk_finalize(R, ncols, K, cand == nullptr, t.ctl, t.hist2, t.cand, t.cnt, idx_out, val_out, st);
}

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_ERR_NULL: return "CSA2_ERR_NULL: a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "CSA2_ERR_SHAPE: a size is out of range or inconsistent";
    case CSA2_ERR_DTYPE: return "CSA2_ERR_DTYPE: unsupported dtype, format or precision";
    case CSA2_ERR_MODE: return "CSA2_ERR_MODE: invalid layer-mode schedule";
    case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE: workspace missing or too small";
    case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED: device or shape not supported";
    case CSA2_ERR_DEVICE: return "CSA2_ERR_DEVICE: HIP runtime or launch failure";
    default: return "unknown csa2 status";
  }
}

int csa2_device_check(void) { return check_device(); }

int csa2_quantize_kv(int fmt, int scale_policy, int B, int T, int D, const void* x, int x_dtype, int64_t x_stride_b,
                     int64_t x_stride_t, const int32_t* n0, int64_t n_max, uint8_t* codes, void* scales_v,
                     void* stream) {
  float* scales = static_cast<float*>(scales_v);
  if (!x || !codes || !scales) return CSA2_ERR_NULL;
  if (!valid_dtype(x_dtype)) return CSA2_ERR_DTYPE;
  if (B < 1 || T < 1 || D < 1 || n_max < 1 || x_stride_t < D || x_stride_b < 0 || B > 65535) return CSA2_ERR_SHAPE;
  const bool bf16 = (x_dtype == CSA2_BF16);
  if (fmt == CSA2_FMT_FP4_PER_CHANNEL) {
    if (D % 2) return CSA2_ERR_SHAPE;
    if (scale_policy != CSA2_SCALE_COMPUTE && scale_policy != CSA2_SCALE_GIVEN) return CSA2_ERR_DTYPE;
    int rc = check_device();
    if (rc) return rc;
    return dev_status(launch_quantize_fp4(scale_policy == CSA2_SCALE_COMPUTE, bf16, B, T, D, x, x_stride_b,
                                          x_stride_t, n0, n_max, codes, scales, S(stream)));
  }
  if (fmt == CSA2_FMT_FP8_PER_TOKEN) {
    if (scale_policy != CSA2_SCALE_COMPUTE) return CSA2_ERR_DTYPE;
    if (D > 4096) return CSA2_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return dev_status(launch_quantize_fp8(bf16, B, T, D, x, x_stride_b, x_stride_t, n0, n_max, codes, scales,
                                          S(stream)));
  }
  if (fmt == CSA2_FMT_FP4_PER_TOKEN) {
    if (scale_policy != CSA2_SCALE_COMPUTE) return CSA2_ERR_DTYPE;
    if (D % 2 || D > 4096) return CSA2_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return dev_status(launch_quantize_fp4_rows(bf16, B, T, D, x, x_stride_b, x_stride_t, n0, n_max, codes, scales,
                                               S(stream)));
  }
  if (fmt == CSA2_FMT_FP4_G16) {
    if (D % 16) return CSA2_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return dev_status(launch_quantize_fp4_g16(bf16, B, T, D, x, x_stride_b, x_stride_t, n0, n_max, codes,
                                              static_cast<uint8_t*>(scales_v), S(stream)));
  }
  return CSA2_ERR_DTYPE;
}

int csa2_gather_dequant(int kv_fmt, int B, int T, int K, int D, const uint8_t* codes, const void* scales,
                        int64_t n_max, const int32_t* idx, float* out, void* stream) {
  if (!codes || !scales || !idx || !out) return CSA2_ERR_NULL;
  if (kv_fmt != CSA2_FMT_FP4_PER_CHANNEL && kv_fmt != CSA2_FMT_FP4_G16) return CSA2_ERR_DTYPE;
  if (B < 1 || T < 1 || K < 1 || D < 8 || D % 8 || n_max < 1) return CSA2_ERR_SHAPE;
  if (kv_fmt == CSA2_FMT_FP4_G16 && D % 16) return CSA2_ERR_SHAPE;
  int rc = check_device();
  if (rc) return rc;
  return dev_status(
      launch_gather_dequant(kv_fmt == CSA2_FMT_FP4_G16, B, T, K, D, codes, scales, n_max, idx, out, S(stream)));
}

size_t csa2_index_score_workspace_size(int B, int T, int64_t) {
  return T >= score_tiled_min_rows() ? align256(score_stage_bytes((int64_t)B * T)) : 0;
}

int csa2_index_score(int prec, int B, int T, int H, int dk, const void* q, int q_dtype, const float* w, const void* k,
                     const float* k_scale, int64_t n_max, const int32_t* n_keys, const int32_t* q_limit,
                     const int32_t* cand, int C, float* scores, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !w || !k || !n_keys || !scores) return CSA2_ERR_NULL;
  if (n_max < 1 || (cand && C < 1)) return CSA2_ERR_SHAPE;
  const int64_t ncols = cand ? C : n_max;
  int rc = check_index_shape(prec, B, T, H, dk, q_dtype, k_scale, ncols);
  if (rc) return rc;
  const size_t need = csa2_index_score_workspace_size(B, T, ncols);
  if (need && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  rc = check_device();
  if (rc) return rc;
  ScoreArgs a = score_args(prec, B, T, H, dk, q, q_dtype, w, k, k_scale, n_max, n_keys, q_limit, cand, ncols, scores,
                           nullptr, 1);
  if (need) a.qstage = static_cast<uint8_t*>(ws);
  return dev_status(launch_score(a, S(stream)));
}

size_t csa2_topk_workspace_size(int B, int T, int64_t ncols, int) { return topk_ws((int64_t)B * T, ncols); }

int csa2_topk(int B, int T, int64_t ncols, const float* scores, const int32_t* cand, int K, int32_t* idx_out,
              float* val_out, void* ws, size_t ws_bytes, void* stream) {
  if (!scores || !idx_out) return CSA2_ERR_NULL;
  if (B < 1 || T < 1 || ncols < 1 || ncols > kMaxTopkCols || K < 1 || K > CSA2_MAX_K || (int64_t)B * T > 65535)
    return CSA2_ERR_SHAPE;
  const int64_t R = (int64_t)B * T;
  if (!ws || ws_bytes < topk_ws(R, ncols)) return CSA2_ERR_WORKSPACE;
  int rc = check_device();
  if (rc) return rc;
  Carve c(ws);
  TopkWs t = carve_topk(c, R, ncols);
  hipStream_t st = S(stream);
  if (zero_topk(t, R, st)) return CSA2_ERR_DEVICE;
  if (launch_topk_hist((int)R, ncols, scores, cand, t.hist, st)) return CSA2_ERR_DEVICE;
  return dev_status(select_topk((int)R, ncols, scores, cand, K, t, idx_out, val_out, st));
}

size_t csa2_index_topk_workspace_size(int B, int T, int64_t ncols, int) {
  const int64_t R = (int64_t)B * T;
  // the candidate lists of a decode scan (fp8 / fp4) or of the many-row scan, or the
  // histogram filter's regions; the scores (written by the fp32 scan, or where the selection
  // re-scores a region); the many-row scan's staged query
  size_t sel = local_ws(R, ncols) > topk_ws(R, ncols) ? local_ws(R, ncols) : topk_ws(R, ncols);
  if (T >= score_tiled_min_rows() && rows_local_ws(R, ncols) > sel) sel = rows_local_ws(R, ncols);
  return align256((size_t)R * ncols * 4) + sel + csa2_index_score_workspace_size(B, T, ncols);
}

int csa2_index_topk(int prec, int B, int T, int H, int dk, const void* q, int q_dtype, const float* w, const void* k,
                    const float* k_scale, int64_t n_max, const int32_t* n_keys, const int32_t* q_limit,
                    const int32_t* cand, int C, int K, int32_t* idx_out, float* val_out, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!q || !w || !k || !n_keys || !idx_out) return CSA2_ERR_NULL;
  if (n_max < 1 || (cand && C < 1) || K < 1 || K > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  const int64_t ncols = cand ? C : n_max;
  if (ncols > kMaxTopkCols) return CSA2_ERR_SHAPE;
  int rc = check_index_shape(prec, B, T, H, dk, q_dtype, k_scale, ncols);
  if (rc) return rc;
  const int64_t R = (int64_t)B * T;
  if (!ws || ws_bytes < csa2_index_topk_workspace_size(B, T, ncols, K)) return CSA2_ERR_WORKSPACE;
  rc = check_device();
  if (rc) return rc;
  Carve c(ws);
  float* scores = c.take<float>((size_t)R * ncols);
  hipStream_t st = S(stream);
  if (local_scan(prec, T, cand, R, ncols)) {
    // decode rows: the score blocks list their candidates, one select workgroup per row
    // finishes the exact Top-K (a candidate map in arbitrary order needs the ranked output)
    const LocalCand lc = local_for(carve_local(c, local_pairs(R, ncols), local_regions(R, ncols)), R, ncols, K);
    ScoreArgs a = score_args(prec, B, T, H, dk, q, q_dtype, w, k, k_scale, n_max, n_keys, q_limit, cand, ncols,
                             scores, nullptr, 1);
    a.local = true;
    a.lc = lc;
    if (launch_score(a, st)) return CSA2_ERR_DEVICE;
    return dev_status(launch_topk_select(a, K, cand == nullptr, score_blocks(R, ncols), idx_out, val_out, st));
  }
  if (rows_scan(prec, T, cand)) {
    // chunked prefill: the many-row blocks list their candidates per (row, region), one
    // select workgroup per row finishes the exact Top-K
    const int nreg = rows_regions(ncols);
    LocalCand lc = carve_local(c, (size_t)R * nreg * kRowsSlots, (size_t)R * nreg);
    lc.stride = kRowsSlots;
    lc.rcols = rows_list_cols();
    lc.K = K;
    uint8_t* qstage = c.take<uint8_t>(csa2_index_score_workspace_size(B, T, ncols));
    ScoreArgs a = score_args(prec, B, T, H, dk, q, q_dtype, w, k, k_scale, n_max, n_keys, q_limit, cand, ncols,
                             scores, nullptr, 1);
    a.qstage = qstage;
    a.local = true;
    a.lc = lc;
    if (launch_score(a, st)) return CSA2_ERR_DEVICE;
    return dev_status(launch_topk_select(a, K, true, nreg, idx_out, val_out, st));
  }
  TopkWs t = carve_topk(c, R, ncols);
  const size_t stage = csa2_index_score_workspace_size(B, T, ncols);
  uint8_t* qstage = stage ? c.take<uint8_t>(stage) : nullptr;
  if (zero_topk(t, R, st)) return CSA2_ERR_DEVICE;
  ScoreArgs a = score_args(prec, B, T, H, dk, q, q_dtype, w, k, k_scale, n_max, n_keys, q_limit, cand, ncols, scores,
                           t.hist, 1);
  a.qstage = qstage;
  if (launch_score(a, st)) return CSA2_ERR_DEVICE;
  return dev_status(select_topk((int)R, ncols, scores, cand, K, t, idx_out, val_out, st));
}

size_t csa2_sparse_attend_workspace_size(int B, int T, int Hq, int D, int K, int q_dtype, int window) {
  if (q_dtype != CSA2_BF16) return 0;
  return align256(attend_ws_floats(B * T, Hq, D, K, window) * 4);
}

int csa2_sparse_attend(int B, int T, int Hq, int D, const void* q, int q_dtype, int kv_fmt, const uint8_t* kv_codes,
                       const void* kv_scales, int64_t n_max, const int32_t* idx, int K, const csa2_swa* swa,
                       float softmax_scale, void* out, int out_dtype, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!q || !kv_codes || !kv_scales || !idx || !out) return CSA2_ERR_NULL;
  if (n_max < 1) return CSA2_ERR_SHAPE;
  int rc = check_kv_fmt(kv_fmt, D);
  if (rc) return rc;
  rc = check_attend_shape(B, T, Hq, D, K, q_dtype, out_dtype);
  if (rc) return rc;
  rc = check_swa(swa, CSA2_MAX_WINDOW);
  if (rc) return rc;
  const size_t need = csa2_sparse_attend_workspace_size(B, T, Hq, D, K, q_dtype, swa ? swa->window : 0);
  if (need && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  rc = check_device();
  if (rc) return rc;
  AttendArgs a = attend_args(B, T, Hq, D, K, q, q_dtype, kv_fmt, kv_codes, kv_scales, n_max, idx, softmax_scale,
                             out, out_dtype, lse);
  a.part = need ? static_cast<float*>(ws) : nullptr;
  set_swa(a, swa);
  return dev_status(launch_attend(a, S(stream)));
}

// ---------------------------------------------------------------------------- layer group
static int check_schedule(const csa2_layer* layers, int n) {
  bool seen_full = false, seen_index = false;
  for (int i = 0; i < n; ++i) {
    switch (layers[i].mode) {
      case CSA2_FULL: seen_full = seen_index = true; break;
      case CSA2_REINDEX:
        if (!seen_full) return CSA2_ERR_MODE;
        seen_index = true;
        break;
      case CSA2_REUSE:
        if (!seen_index) return CSA2_ERR_MODE;
        break;
      default: return CSA2_ERR_MODE;
    }
  }
  return n > 0 ? CSA2_OK : CSA2_ERR_MODE;
}

// true when a Reindex layer follows layer i before the next Full layer
static bool reindex_after(const csa2_layer* layers, int n, int i) {
  for (int j = i + 1; j < n; ++j) {
    if (layers[j].mode == CSA2_FULL) return false;
    if (layers[j].mode == CSA2_REINDEX) return true;
  }
  return false;
}

static int count_index_layers(const csa2_layer* layers, int n) {
  int c = 0;
  for (int i = 0; i < n; ++i) c += (layers[i].mode != CSA2_REUSE);
  return c;
}

static bool pool_on(const csa2_group_cache* c) { return c->pool_blocks > 0; }
static int64_t pool_cols(const csa2_group_cache* c) { return pool_on(c) ? (int64_t)c->pool_blocks * c->pool_block : 0; }
static int64_t pool_nb(const csa2_group_cache* c) {
  return pool_on(c) ? (c->n_max + c->pool_block - 1) / c->pool_block : 0;
}
// query tokens per sequence (multi-token decode)
static int group_T(const csa2_group_cache* c) { return c->T > 1 ? c->T : 1; }

// columns the scores and candidate regions are sized for (the full scan or the pool)
static int64_t group_cols(const csa2_group_cache* c) {
  const int64_t pc = pool_cols(c);
  return pc > c->n_max ? pc : c->n_max;
}

// Selections that use a histogram slot (hist, hist2, ctl; zeroed before use): with the fp8 /
// fp4 indexer only the candidate pools' block selections, with the fp32 indexer every one.
static bool group_local(const csa2_group_cache* c) {
  return c->prec != CSA2_PREC_FP32 && local_fits((int64_t)c->B * c->T, c->n_max);
}
static int group_slot_selections(const csa2_group_cache* c, int n_index, int n_full) {
  const int pool_sel = pool_on(c) ? n_full : 0;
  return group_local(c) ? pool_sel : n_index + pool_sel;
}
// storage of the decode scans' candidate lists: the larger of the full scan's and the pool's
static void group_local_sizes(const csa2_group_cache* c, int64_t R, size_t& pairs, size_t& regions) {
  pairs = local_pairs(R, c->n_max);
  regions = local_regions(R, c->n_max);
  if (pool_on(c)) {
    const size_t p2 = local_pairs(R, pool_cols(c)), r2 = local_regions(R, pool_cols(c));
    if (p2 > pairs) pairs = p2;
    if (r2 > regions) regions = r2;
  }
}
// candidate regions of the histogram filter (fp32 indexer: every selection; else the pools')
static int64_t group_filter_cols(const csa2_group_cache* c) {
  if (!group_local(c)) return group_cols(c);
  return pool_on(c) ? pool_nb(c) : 0;
}

// workspace: [hist, hist2, ctl per slot selection (the first zeroed per call, each later one
//            by the filter before it)] [scores] [filter regions] [candidate lists]
//            [attention partials] [pool positions, block maxima] [causal limits]
size_t csa2_layer_group_workspace_size(const csa2_group_cache* c, int n_layers) {
  if (!c || n_layers < 1) return 0;
  const int64_t R = (int64_t)c->B * group_T(c);
  const int sel = group_slot_selections(c, n_layers, n_layers);
  const int slots = sel < 64 ? sel : 64;
  const size_t att =
      (c->q_dtype == CSA2_BF16) ? align256(attend_ws_floats((int)R, c->Hq, c->D, c->K, c->window) * 4) : 0;
  const size_t pool = pool_on(c) ? align256((size_t)R * pool_cols(c) * 4) + align256((size_t)R * pool_nb(c) * 4) : 0;
  const size_t lim = group_T(c) > 1 ? align256((size_t)R * 4) : 0;
  size_t lp = 0, lr = 0;
  if (group_local(c)) group_local_sizes(c, R, lp, lr);
  const int64_t fc = group_filter_cols(c);
  return topk_zero_bytes(R) * (size_t)slots + align256((size_t)R * group_cols(c) * 4) + (fc ? cand_bytes(R, fc) : 0) +
         (group_local(c) ? local_ws(lp, lr) : 0) + att + pool + lim;
}

int csa2_layer_group(const csa2_layer* layers, int n_layers, const csa2_group_cache* c, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!layers || !c) return CSA2_ERR_NULL;
  if (n_layers < 1) return CSA2_ERR_MODE;
  int rc = check_schedule(layers, n_layers);
  if (rc) return rc;
  if (!c->n_keys || !c->kv_codes || !c->kv_scales || !c->k) return CSA2_ERR_NULL;
  if (c->n_max < 1 || c->n_max > kMaxTopkCols || c->K < 1 || c->K > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (c->pool_blocks < 0 || c->pool_blocks > CSA2_MAX_K || (pool_on(c) && c->pool_block < 1)) return CSA2_ERR_SHAPE;
  if (c->window < 0 || c->window > CSA2_MAX_WINDOW) return CSA2_ERR_SHAPE;
  if (c->T < 0 || c->T > CSA2_MAX_GROUP_T) return CSA2_ERR_SHAPE;
  if (pool_cols(c) > kMaxTopkCols || c->n_max > INT32_MAX) return CSA2_ERR_SHAPE;
  const int T = group_T(c);
  rc = check_index_shape(c->prec, c->B, T, c->H, c->dk, c->q_dtype, c->k_scale, c->n_max);
  if (rc) return rc;
  rc = check_kv_fmt(c->kv_fmt, c->D);
  if (rc) return rc;
  rc = check_attend_shape(c->B, T, c->Hq, c->D, c->K, c->q_dtype, c->out_dtype);
  if (rc) return rc;
  for (int i = 0; i < n_layers; ++i) {
    const csa2_layer& L = layers[i];
    if (!L.q_attn || !L.out) return CSA2_ERR_NULL;
    if (L.mode != CSA2_REUSE && (!L.q_idx || !L.w || !L.idx)) return CSA2_ERR_NULL;
    rc = check_swa(L.swa, c->window);
    if (rc) return rc;
  }
  if (!ws || ws_bytes < csa2_layer_group_workspace_size(c, n_layers)) return CSA2_ERR_WORKSPACE;
  rc = check_device();
  if (rc) return rc;

  const int64_t R = (int64_t)c->B * T;
  const bool pooled = pool_on(c);
  const bool local = group_local(c);
  int n_full = 0;
  for (int i = 0; i < n_layers; ++i) n_full += (layers[i].mode == CSA2_FULL);
  const int n_sel = group_slot_selections(c, count_index_layers(layers, n_layers), n_full);
  const int slots = n_sel < 64 ? n_sel : 64;
  Carve cv(ws);
  TopkWs tz[64];
  for (int i = 0; i < slots; ++i) tz[i] = carve_topk_zero(cv, R);
  float* scores = cv.take<float>((size_t)R * group_cols(c));
  const int64_t fc = group_filter_cols(c);
  CandWs cw = fc ? carve_cand(cv, R, fc) : CandWs{nullptr, nullptr};
  LocalCand lbase{nullptr, nullptr, nullptr, nullptr, 0, 0};
  if (local) {
    size_t lp = 0, lr = 0;
    group_local_sizes(c, R, lp, lr);
    lbase = carve_local(cv, lp, lr);
  }
  float* part =
      (c->q_dtype == CSA2_BF16) ? cv.take<float>(attend_ws_floats((int)R, c->Hq, c->D, c->K, c->window)) : nullptr;
  const int64_t pc = pool_cols(c), nb = pool_nb(c);
  int32_t* pool = pooled ? cv.take<int32_t>((size_t)R * pc) : nullptr;
  float* bmax = pooled ? cv.take<float>((size_t)R * nb) : nullptr;
  int32_t* q_limit = T > 1 ? cv.take<int32_t>((size_t)R) : nullptr;
  hipStream_t st = S(stream);
  if (q_limit && launch_causal_limits(c->B, T, c->n_keys, q_limit, st)) return CSA2_ERR_DEVICE;
  // the first slot selection's histograms and control words are cleared here; the filter of
  // each slot selection clears the slot the next one takes (more than 64 selections reuse
  // the last slot, cleared again before each reuse)
  const int64_t slot_words = (int64_t)(topk_zero_bytes(R) / 4);
  if (slots > 0 && launch_fill_u32(tz[0].hist, slot_words, 0u, st)) return CSA2_ERR_DEVICE;
  int si = 0;
  uint32_t* next_clear = nullptr;  // the slot after the one handed out last (nullptr: none)
  auto next_slot = [&](TopkWs& t) -> int {
    t = tz[si < slots ? si : slots - 1];
    const bool reuse = si >= slots;
    next_clear = (si + 1 < slots) ? tz[si + 1].hist : nullptr;
    ++si;
    return reuse ? zero_topk(t, R, st) : 0;
  };
  const int32_t* cur_pool = nullptr;  // the pool of the most recent Full layer

  AttendArgs a = attend_args(c->B, T, c->Hq, c->D, c->K, nullptr, c->q_dtype, c->kv_fmt, c->kv_codes, c->kv_scales,
                             c->n_max, nullptr, c->softmax_scale, nullptr, c->out_dtype, nullptr);
  a.part = part;
  const int32_t* last_idx = nullptr;
  for (int i = 0; i < n_layers; ++i) {
    const csa2_layer& L = layers[i];
    a.q = L.q_attn;
    a.out = L.out;
    a.lse = L.lse;
    set_swa(a, L.swa);
    if (L.mode != CSA2_REUSE) {
      // a Reindex layer after a pooled Full layer scores only the pool's positions; the pool
      // ascends, so its candidates are in position order like a full scan's
      const bool use_pool = (L.mode == CSA2_REINDEX) && cur_pool;
      const int64_t ncols = use_pool ? pc : c->n_max;
      const int32_t* cand = use_pool ? cur_pool : nullptr;
      ScoreArgs sa = score_args(c->prec, c->B, T, c->H, c->dk, L.q_idx, c->q_dtype, L.w, c->k, c->k_scale, c->n_max,
                                c->n_keys, q_limit, cand, ncols, scores, nullptr, 1);
      // a Full layer whose keys a later Reindex layer of this call rescans in full reads
      // them with cached loads, so that the rescan finds them in the Infinity Cache
      // (measured: the rescan 23.6 us instead of 29 us at 16 x 131072).  With a pool the
      // Reindex layers read only the pool's positions and the cached scan measured slower.
      sa.keep = (L.mode == CSA2_FULL) && !pooled && reindex_after(layers, n_layers, i);
      if (local) {
        // the score blocks list their candidates; one select workgroup per row finishes the
        // exact Top-K straight into the layer's idx
        sa.local = true;
        sa.lc = local_for(lbase, R, ncols, c->K);
        sa.lc.store = pooled && L.mode == CSA2_FULL;  // the pool's block maxima read every score
        if (launch_score(sa, st)) return CSA2_ERR_DEVICE;
        if (launch_topk_select(sa, c->K, true, score_blocks(R, ncols), L.idx, nullptr, st))
          return CSA2_ERR_DEVICE;
      } else {
        TopkWs t;
        if (next_slot(t)) return CSA2_ERR_DEVICE;
        sa.hist = t.hist;
        if (launch_score(sa, st)) return CSA2_ERR_DEVICE;
        if (launch_topk_filter((int)R, ncols, scores, cand, c->K, t.hist, t.hist2, t.ctl, cw.cand, cw.cnt, st,
                               next_clear, next_clear ? slot_words : 0))
          return CSA2_ERR_DEVICE;
        if (launch_topk_finalize((int)R, ncols, c->K, true, t.ctl, t.hist2, cw.cand, cw.cnt, L.idx, nullptr, st))
          return CSA2_ERR_DEVICE;
      }
      last_idx = L.idx;
    }
    a.idx = last_idx;
    if (launch_attend(a, st)) return CSA2_ERR_DEVICE;
    if (pooled && L.mode == CSA2_FULL) {
      // the pool: block maxima of this layer's scores, their best pool_blocks blocks (lowest
      // block on ties), expanded to positions (-1 past n_keys)
      TopkWs t;
      if (next_slot(t)) return CSA2_ERR_DEVICE;
      int32_t* dst = L.pool ? L.pool : pool;
      if (launch_block_max((int)R, c->n_max, c->pool_block, scores, bmax, t.hist, st)) return CSA2_ERR_DEVICE;
      if (launch_topk_filter((int)R, nb, bmax, nullptr, c->pool_blocks, t.hist, t.hist2, t.ctl, cw.cand, cw.cnt, st,
                             next_clear, next_clear ? slot_words : 0))
        return CSA2_ERR_DEVICE;
      if (launch_topk_finalize((int)R, nb, c->pool_blocks, true, t.ctl, t.hist2, cw.cand, cw.cnt, nullptr, nullptr, st,
                               c->pool_block, c->n_keys, dst, T))
        return CSA2_ERR_DEVICE;
      cur_pool = dst;
    }
  }
  return CSA2_OK;
}

int csa2_stream_probe(const void* src, int64_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (!src || !sink) return CSA2_ERR_NULL;
  if (bytes < 16 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) || blocks < 1 || blocks > (1 << 20))
    return CSA2_ERR_SHAPE;
  int rc = check_device();
  if (rc) return rc;
  return dev_status(launch_stream_read(src, bytes, blocks, sink, S(stream)));
}

// ---------------------------------------------------------------------------- two-level indexer
int csa2_coarse_keys(int B, int64_t n_max, const int32_t* n_keys, int dk, int block, const uint8_t* k8,
                     const float* k_scale, uint8_t* kb8, float* kb_scale, void* stream) {
  if (!n_keys || !k8 || !k_scale || !kb8 || !kb_scale) return CSA2_ERR_NULL;
  if (B < 1 || B > 65535 || n_max < 1 || dk < 1 || dk > CSA2_MAX_DK || block < 1) return CSA2_ERR_SHAPE;
  int rc = check_device();
  if (rc) return rc;
  return dev_status(launch_coarse_keys(B, n_max, n_keys, dk, block, k8, k_scale, kb8, kb_scale, S(stream)));
}

// Two-level select.  Rows whose coarse and fine stages both fit the candidate lists (at most
// kLocalMaxRegions score blocks each): [coarse and fine lists] [coarse and fine scores
// (written only where the selection re-scores a block)] [selected blocks] [their positions].
// Larger ones take the histogram selection: [both selections' zeroed state] [their candidate
// lists] [coarse scores] [selected blocks] [their positions] [fine scores].
static bool hier_lists(int B, int64_t nb, int64_t C) { return local_fits(B, nb) && local_fits(B, C); }
size_t csa2_hier_select_workspace_size(int B, int64_t n_max, int block, int block_topk, int) {
  const int64_t nb = (n_max + block - 1) / block;
  const int64_t C = (int64_t)block_topk * block;
  if (hier_lists(B, nb, C))
    return local_ws(B, nb) + local_ws(B, C) + align256((size_t)B * nb * 4) + align256((size_t)B * C * 4) +
           align256((size_t)B * block_topk * 4) + align256((size_t)B * C * 4);
  return align256((size_t)B * nb * 4) + topk_ws(B, nb) + align256((size_t)B * block_topk * 4) +
         align256((size_t)B * C * 4) + align256((size_t)B * C * 4) + topk_ws(B, C);
}
int csa2_hier_select(int B, int H, int dk, const void* q, int q_dtype, const float* w, const uint8_t* k8,
                     const float* k_scale, const uint8_t* kb8, const float* kb_scale, int64_t n_max,
                     const int32_t* n_keys, int block, int block_topk, int K, int32_t* idx_out, int32_t* block_out,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!q || !w || !k8 || !k_scale || !kb8 || !kb_scale || !n_keys || !idx_out) return CSA2_ERR_NULL;
  if (block < 1 || block_topk < 1 || block_topk > CSA2_MAX_K || K < 1 || K > CSA2_MAX_K || n_max < 1)
    return CSA2_ERR_SHAPE;
  const int64_t nb = (n_max + block - 1) / block;
  const int64_t C = (int64_t)block_topk * block;
  if (C > kMaxTopkCols || nb > kMaxTopkCols || n_max > INT32_MAX) return CSA2_ERR_SHAPE;
  int rc = check_index_shape(CSA2_PREC_FP8, B, 1, H, dk, q_dtype, k_scale, nb);
  if (rc) return rc;
  if (!ws || ws_bytes < csa2_hier_select_workspace_size(B, n_max, block, block_topk, K)) return CSA2_ERR_WORKSPACE;
  rc = check_device();
  if (rc) return rc;
  Carve cv(ws);
  hipStream_t st = S(stream);
  int32_t* bout = block_out;
  if (hier_lists(B, nb, C)) {
    const LocalCand l1 = local_for(carve_local(cv, local_pairs(B, nb), local_regions(B, nb)), B, nb, block_topk);
    const LocalCand l2 = local_for(carve_local(cv, local_pairs(B, C), local_regions(B, C)), B, C, K);
    float* cscores = cv.take<float>((size_t)B * nb);
    float* fscores = cv.take<float>((size_t)B * C);
    int32_t* blocks = cv.take<int32_t>((size_t)B * block_topk);
    int32_t* cand = cv.take<int32_t>((size_t)B * C);
    if (!bout) bout = blocks;
    // coarse: the block keys' scan lists its candidates; the block selection also writes the
    // selected blocks' positions (the fine candidates, ascending, -1 past n_keys)
    ScoreArgs a1 = score_args(CSA2_PREC_FP8, B, 1, H, dk, q, q_dtype, w, kb8, kb_scale, nb, n_keys, nullptr, nullptr,
                              nb, cscores, nullptr, block);
    a1.local = true;
    a1.lc = l1;
    if (launch_score(a1, st)) return CSA2_ERR_DEVICE;
    if (launch_topk_select(a1, block_topk, true, score_blocks(B, nb), bout, nullptr, st, nullptr, 0, block, cand))
      return CSA2_ERR_DEVICE;
    // fine: the exact score of every candidate position, listed, then the Top-K (the
    // candidates ascend, so the winners come out in position order)
    ScoreArgs a2 = score_args(CSA2_PREC_FP8, B, 1, H, dk, q, q_dtype, w, k8, k_scale, n_max, n_keys, nullptr, cand,
                              C, fscores, nullptr, 1);
    a2.local = true;
    a2.lc = l2;
    if (launch_score(a2, st)) return CSA2_ERR_DEVICE;
    return dev_status(launch_topk_select(a2, K, true, score_blocks(B, C), idx_out, nullptr, st));
  }
  // the histogram selection: both selections' zeroed state first (one fill), then their lists
  TopkWs t1 = carve_topk_zero(cv, B);
  TopkWs t2 = carve_topk_zero(cv, B);
  const CandWs w1 = carve_cand(cv, B, nb);
  const CandWs w2 = carve_cand(cv, B, C);
  t1.cand = w1.cand; t1.cnt = w1.cnt;
  t2.cand = w2.cand; t2.cnt = w2.cnt;
  float* cscores = cv.take<float>((size_t)B * nb);
  int32_t* blocks = cv.take<int32_t>((size_t)B * block_topk);
  int32_t* cand = cv.take<int32_t>((size_t)B * C);
  float* fscores = cv.take<float>((size_t)B * C);
  if (!bout) bout = blocks;
  if (launch_fill_u32(t1.hist, (int64_t)(2 * topk_zero_bytes(B) / 4), 0u, st)) return CSA2_ERR_DEVICE;
  ScoreArgs a1 = score_args(CSA2_PREC_FP8, B, 1, H, dk, q, q_dtype, w, kb8, kb_scale, nb, n_keys, nullptr, nullptr,
                            nb, cscores, t1.hist, block);
  if (launch_score(a1, st)) return CSA2_ERR_DEVICE;
  if (launch_topk_filter(B, nb, cscores, nullptr, block_topk, t1.hist, t1.hist2, t1.ctl, t1.cand, t1.cnt, st))
    return CSA2_ERR_DEVICE;
  if (launch_topk_finalize(B, nb, block_topk, true, t1.ctl, t1.hist2, t1.cand, t1.cnt, bout, nullptr, st, block,
                           n_keys, cand))
    return CSA2_ERR_DEVICE;
  ScoreArgs a2 = score_args(CSA2_PREC_FP8, B, 1, H, dk, q, q_dtype, w, k8, k_scale, n_max, n_keys, nullptr, cand, C,
                            fscores, t2.hist, 1);
  if (launch_score(a2, st)) return CSA2_ERR_DEVICE;
  // the expanded candidates ascend (blocks ascending, positions within a block ascending,
  // -1 for none), so the filtered list is in position order
  if (launch_topk_filter(B, C, fscores, cand, K, t2.hist, t2.hist2, t2.ctl, t2.cand, t2.cnt, st))
    return CSA2_ERR_DEVICE;
  return dev_status(launch_topk_finalize(B, C, K, true, t2.ctl, t2.hist2, t2.cand, t2.cnt, idx_out, nullptr, st));
}

}  // extern "C"
