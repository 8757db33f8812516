// Internal launch interface of the head kernels (host side).  Every launcher
// enqueues on `st` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbp {

// Per-token cross-entropy weight rule used by the label scan.
enum WeightMode : int {
  kWeightMean = 0,   // 1/len over the whole call (SFT)
  kWeightAdv = 1,    // adv[s]/len_s (GRPO)
  kWeightNone = 2,   // 0 (forward-only pass)
  kWeightCoef = 3,   // coef[s] (DPO backward)
};

// Tiles of the bf16 GEMMs.
constexpr int kLogitsBM = 256;  // vocab rows per logits tile = width of one LSE partial
constexpr int kLogitsBN = 256;  // tokens per logits tile
constexpr int kDhBM = 256, kDhBN = 256;
constexpr int kDwBM = 256, kDwBN = 256;
constexpr int kF32TileW = 64;   // fp32 tiles (all three GEMMs)
constexpr int kTiledRows = 256, kTiledCols = 32;  // storage tiles of the tiled logits operands
constexpr int kDwMinStages = 16;  // k-stages of 32 rows the accumulating dW loop runs at least

// ---- measurement aid -------------------------------------------------------
// `blocks` blocks of 4 waves, each issuing iters x 8 independent
// v_mfma_f32_32x32x16_bf16 (on operands that change per instruction when
// `changing`); mfma_probe_flops() gives the flops of one launch.
hipError_t launch_mfma_probe(int64_t blocks, int iters, bool changing, hipStream_t st);
double mfma_probe_flops(int64_t blocks, int iters);

// ---- bf16 MFMA GEMMs -------------------------------------------------------
// Gradient mode of the logits GEMM: with every token's log-sum-exp known, the
// epilogue writes G = w (softmax - onehot(y)) instead of Z and partials.
// Per-token arrays are indexed by tok0 + the chunk row, or through
// rowmap[tok0 + row] for the live rows under masked-row compaction.
struct LogitsGrad {
  const float* lse;
  const float* w;
  const int32_t* y;
  int64_t tok0;
  const int32_t* rowmap;  // NULL without compaction
  const int32_t* live;    // live row count (with live_base), NULL without compaction
  int64_t live_base;
};
// Logits from row-major W and a tiled copy of the chunk's rows of H (see
// launch_tile32).
hipError_t launch_logits_bf16(const uint16_t* W, const uint16_t* Ht, int64_t V, int64_t D, int64_t rows,
                              uint16_t* Z, int64_t ldz, float2* part, int64_t nvb, int tile_begin, int tile_end,
                              const int32_t* live_rows, int64_t live_base, const LogitsGrad* grad, hipStream_t st);
// Logits from tiled copies of W and H_c, bitwise equal to launch_logits_bf16.
hipError_t launch_logits_bf16_tiled(const uint16_t* Wt, const uint16_t* Ht, int64_t V, int64_t D, int64_t rows,
                                    uint16_t* Z, int64_t ldz, float2* part, int64_t nvb, int tile_begin, int tile_end,
                                    const int32_t* live_rows, int64_t live_base, const LogitsGrad* grad,
                                    hipStream_t st);
// X [rows][ld] bf16 (first `cols` columns) into 256 x 32 storage tiles,
// tile_rows x ceil(cols / 32) of them, zero-padded.
// X [rows][ld] bf16 (first `cols` columns) transposed into 256 x 32 storage
// tiles, ceil(cols / 256) x nrt of them (nrt * 32 >= rows), zero-padded.
hipError_t launch_tile32_t(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld, uint16_t* T, int64_t nrt,
                           const int32_t* live, int64_t live_base, hipStream_t st);
hipError_t launch_tile32(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld, uint16_t* T, int64_t tile_rows,
                         hipStream_t st);
hipError_t launch_dh_bf16(const uint16_t* G, int64_t ldz, const uint16_t* W, int64_t V, int64_t D,
                          int64_t rows, float* out, int splits, int64_t split_stride, const int32_t* live_rows,
                          int64_t live_base, hipStream_t st);
// dW (+)= G^T H_c from HcT, the chunk's rows of H transposed into 256 x 32
// tiles by launch_tile32_t (nrt tile columns, at least 16 when accumulating);
// with device-side live rows the tiles must be zero past the live rows
// (launch_tile32_t with the same live count).
hipError_t launch_dw_bf16(const uint16_t* G, int64_t ldz, const uint16_t* HcT, int64_t nrt, int64_t V, int64_t D,
                          int64_t rows, float* dW, int accumulate, const int32_t* live_rows, int64_t live_base,
                          hipStream_t st);

// ---- fp32 GEMMs --------------------------------------------------------------
hipError_t launch_logits_f32(const float* W, const float* Hc, int64_t V, int64_t D, int64_t rows, float* Z,
                             int64_t ldz, const int32_t* y, float2* part, int64_t nvb, float* zy,
                             hipStream_t st);
hipError_t launch_dh_f32(const float* G, int64_t ldz, const float* W, int64_t V, int64_t D, int64_t rows,
                         float* out, int splits, int64_t split_stride, hipStream_t st);
hipError_t launch_dw_f32(const float* G, int64_t ldz, const float* Hc, int64_t V, int64_t D, int64_t rows,
                         float* dW, int accumulate, hipStream_t st);

// ---- row-wise and small kernels ------------------------------------------
// Outputs of masked-row compaction (see launch_scan_labels): the valid token
// indices in order, their count, and the per-token logp / loss terms that the
// scan zeroes on the other rows.
struct CompactRows {
  int32_t* rowmap;
  int32_t* count;
  float* logp;
  double* loss_rows;
};

// `inv_len` (may be NULL) receives 1/len_s on the valid tokens of sequence s.
// With `cr` the scan also lists the valid rows for masked-row compaction.
hipError_t launch_scan_labels(const int32_t* y, int64_t T, int64_t V, const int32_t* offsets, int n_seq,
                              int mode, const float* adv, const double* coef, float* w, float* inv_len,
                              int32_t* seq_len, int64_t* n_valid, int32_t* status, const CompactRows* cr,
                              hipStream_t st);
// Masked-row compaction: dense copy of a chunk's live rows of H (bf16), and
// zeroing of the dH rows no chunk writes.
hipError_t launch_gather_rows(const uint16_t* H, int64_t D, const int32_t* rowmap, const int32_t* count, int64_t base,
                              int64_t cap, uint16_t* out, hipStream_t st);
hipError_t launch_zero_dead_rows(float* dH, int64_t T, int64_t D, const int32_t* y, int64_t V, const int32_t* status,
                                 hipStream_t st);
// Per-token inputs of the off-policy clipped-surrogate weight rule (rows of
// the current chunk): old and reference log-probs, 1/len_s, the clip range
// half-width and the KL coefficient.  `ref` may be NULL when beta == 0.
struct PpoArgs {
  const float* old;
  const float* ref;
  const float* inv_len;
  float eps;
  float beta;
};

// Combine LSE partials of each row, write logp and the row's loss term; with
// `backward`, overwrite the row of Z in place with G = w (softmax - onehot).
// The target logit comes from `zy` (fp32) or from the rows of Hc and W (bf16).
// With `ppo` non-NULL, w and the loss term come from the clipped surrogate
// (w holds A_s/len_s on entry); otherwise w is the cross-entropy weight.
hipError_t launch_rows(bool bf16, bool backward, void* Z, int64_t ldz, int64_t V, int64_t rows,
                       const float2* part, int64_t nvb, const float* zy, const void* Hc, const void* W, int64_t D,
                       const int32_t* y, const float* w, const PpoArgs* ppo, float* logp, double* loss_rows,
                       float* lse_out, const int32_t* rowmap, const int32_t* live, int64_t live_base, hipStream_t st);
// Fixed-order sum of the dH split-K slabs (rows x D); with `rowmap`, slab row
// r goes to out row rowmap[r] for the live rows only.
hipError_t launch_splitk_reduce(const float* part, int splits, int64_t split_stride, int64_t rows, int64_t D,
                                float* out, const int32_t* rowmap, const int32_t* live, int64_t live_base,
                                hipStream_t st);
hipError_t launch_sum_f64(const double* x, int64_t n, double* out, hipStream_t st);
hipError_t launch_seq_sums(const float* logp, const int32_t* offsets, int n_seq, int64_t T, double* out,
                           hipStream_t st);
hipError_t launch_dpo_pairs(const double* seq_logp, const double* ref_logp, int n_seq, double beta,
                            double* coef, double* loss, hipStream_t st);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
hipError_t launch_finish_empty(double* loss, int64_t* n_valid, int32_t* status, hipStream_t st);

}  // namespace sbp
