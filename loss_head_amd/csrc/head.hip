// Host side of the chunked LM-head library: argument checks, workspace
// layout, and the per-chunk launch sequence.  All device work is enqueued on
// the caller's stream; nothing is allocated here.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/streambp_head.h"
#include "kernels.h"

// Kernel kinds reported by the timing facility.
enum KernelKind : int {
  kKindScan = 0, kKindLogits, kKindRows, kKindDh, kKindDhReduce, kKindDw, kKindDpoPairs, kKindLossSum,
  kKindSeqSums, kKindFill, kKindGather, kKindZeroRows, kKindTileW, kKindTileH, kKindTileHT, kNumKinds
};
static const char* const kKindNames[kNumKinds] = {"scan_labels", "logits_lse", "rows_lse_dlogits", "dh_gemm",
                                                  "dh_splitk_reduce", "dw_gemm", "dpo_pairs", "loss_sum",
                                                  "seq_sums", "fill", "gather_rows", "zero_dead_rows",
                                                  "tile_w", "tile_h", "tile_ht"};

struct TimedLaunch {
  int kind;
  hipEvent_t ev[2];
};

struct streambp_head_s {
  int64_t D, V, C;
  streambp_dtype dtype;
  int device;
  int64_t ldz;     // row stride of the chunk logits buffer (V rounded up to 8)
  int64_t nvb;     // vocab tiles per row in the logits GEMM (= LSE partials per row)
  int dh_splits;   // split-K factor of the dH GEMM
  bool debug;      // synchronise and check after every launch
  bool compact = false;  // masked-row compaction (bf16 only)
  bool tiled = false;    // logits GEMM from tiled copies of W and H_c (bf16 only)
  std::string err;
  // timing facility
  bool timing = false;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> spare;
  double total_ms[kNumKinds] = {};
  int64_t launches[kNumKinds] = {};
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kNumCUs = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

streambp_status fail(streambp_head h, streambp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (h) h->err = buf;
  return s;
}

// Split of the dH GEMM's long K (the vocabulary) so that tiles x splits fills
// the 256 CUs in whole waves of blocks.
int choose_dh_splits(int64_t C, int64_t D, int64_t ldz, bool bf16) {
  const int64_t bm = bf16 ? sbp::kDhBM : sbp::kF32TileW, bn = bf16 ? sbp::kDhBN : sbp::kF32TileW;
  const int64_t bk = bf16 ? 64 : 16;
  const int64_t tiles = cdiv(C, bm) * cdiv(D, bn);
  int best = 1;
  double best_eff = 0.0;
  for (int s = 1; s <= 16; ++s) {
    if (s > 1 && cdiv(ldz, s) < 8 * bk) break;  // keep at least 8 k-stages per split
    const int64_t blocks = tiles * s;
    const double eff = (double)blocks / (double)(cdiv(blocks, kNumCUs) * kNumCUs);
    if (eff > best_eff + 0.02) {
      best_eff = eff;
      best = s;
    }
  }
  return best;
}

struct Layout {
  size_t z, part, zy, split, w, w2, logp, loss_rows, seq_len, coef, seqsum, rowmap, hdense, wt, ht, htt, scratch, total;
};

// Tile columns (of 32 rows) of the transposed copy of a chunk's rows of H.
int64_t dw_tile_cols(int64_t rows) {
  const int64_t n = cdiv(rows, sbp::kTiledCols);
  return n < sbp::kDwMinStages ? sbp::kDwMinStages : n;
}

Layout layout(const streambp_head_s* h, int64_t T, int64_t n_seq) {
  const size_t esize = h->dtype == STREAMBP_BF16 ? 2 : 4;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  L.z = take((size_t)h->C * h->ldz * esize);
  L.part = take((size_t)h->C * h->nvb * 8);
  L.zy = take((size_t)h->C * 4);
  // dH split-K slabs; masked-row compaction always reduces through them
  L.split = take((h->dh_splits > 1 || h->compact) ? (size_t)h->dh_splits * h->C * h->D * 4 : 0);
  L.w = take((size_t)T * 4);
  L.w2 = take((size_t)T * 4);
  L.logp = take((size_t)T * 4);
  L.loss_rows = take((size_t)T * 8);
  L.seq_len = take((size_t)n_seq * 4);
  L.coef = take((size_t)n_seq * 8);
  L.seqsum = take((size_t)n_seq * 8);
  L.rowmap = take(h->compact ? (size_t)T * 4 : 0);            // valid token indices
  L.hdense = take(h->compact ? (size_t)h->C * h->D * esize : 0);  // one chunk's live rows of H
  // tiled copies of the chunk's rows of H (bf16, per chunk) and, with the
  // tiled-logits option, of W (per call)
  const size_t tile_cols = (size_t)cdiv(h->D, sbp::kTiledCols) * sbp::kTiledCols;
  L.wt = take(h->tiled ? (size_t)cdiv(h->V, sbp::kTiledRows) * sbp::kTiledRows * tile_cols * 2 : 0);
  L.ht = take(h->dtype == STREAMBP_BF16 ? (size_t)cdiv(h->C, sbp::kTiledRows) * sbp::kTiledRows * tile_cols * 2 : 0);
  // the chunk's rows of H transposed into tiles for the dW GEMM (bf16), at
  // least 16 tile columns: the accumulating dW loop runs at least 16 k-stages
  L.htt = take(h->dtype == STREAMBP_BF16
                   ? (size_t)cdiv(h->D, sbp::kTiledRows) * sbp::kTiledRows * dw_tile_cols(h->C) * sbp::kTiledCols * 2
                   : 0);
  L.scratch = take(64);                                         // [0]: number of valid rows
  L.total = off;
  return L;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// The no-allocation entry point's workspace: one fixed array per device,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address that hipGetSymbolAddress returns for the current device,
// looked up once per device when a handle is created there.
static __device__ __align__(256) unsigned char scratch[STREAMBP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};
bool g_scratch_done[kMaxDevices] = {};

// Called with `device` current.
void lookup_static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_done[device]) return;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  g_scratch_err[device] = e;
  g_scratch_ptr[device] = e == hipSuccess ? p : nullptr;
  g_scratch_done[device] = true;
}

// The device address of the array on `device`, or NULL (then *err says why).
void* static_scratch(int device, hipError_t* err) {
  if (device < 0 || device >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  *err = g_scratch_done[device] ? g_scratch_err[device] : hipErrorNotInitialized;
  return g_scratch_ptr[device];
}

enum class Kind { Sft, Grpo, DpoLogp, DpoBwd, Ppo };

struct Call {
  Kind kind;
  int64_t T;
  const void* H;
  const void* W;
  const int32_t* labels;
  const int32_t* offsets;  // NULL for SFT
  int n_seq;
  const float* adv;
  float* logp_out;
  const double* seq_logp_in;
  const double* ref_logp;
  double beta;
  const float* logp_old;   // PPO: per-token behaviour log-probs
  const float* logp_ref;   // PPO: per-token reference log-probs (NULL when beta_kl = 0)
  double eps;              // PPO: clip range half-width
  double beta_kl;          // PPO: KL coefficient
  float* dH;
  float* dW;
  int accumulate;
  double* loss;
  int64_t* n_valid;
  double* seq_logp_out;
  float* token_lse_out;       // DPO pass 1: per-token log-sum-exp (optional)
  const float* token_lse_in;  // DPO pass 2: the same, from pass 1 (optional)
  int32_t* status;
  void* ws;
  size_t ws_bytes;
  hipStream_t st;
  bool static_scratch;     // workspace = the library's static device array (no events either)
  bool timing;             // bracket launches with the handle's timing events (set by run)
};

hipEvent_t take_event(streambp_head h) {
  if (!h->spare.empty()) {
    hipEvent_t e = h->spare.back();
    h->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Fold finished timed launches into the per-kind totals.
hipError_t drain_timing(streambp_head h) {
  hipError_t err = hipSuccess;
  for (TimedLaunch& t : h->pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(t.ev[1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.ev[0], t.ev[1]);
    if (e == hipSuccess) {
      h->total_ms[t.kind] += ms;
      h->launches[t.kind] += 1;
    } else {
      err = e;
    }
    h->spare.push_back(t.ev[0]);
    h->spare.push_back(t.ev[1]);
  }
  h->pending.clear();
  return err;
}

// Launch through SBP_LAUNCH_ON(kind, stream, expr): optional event pair around
// the launch on that stream, optional debug sync.  SBP_LAUNCH uses the call's stream.
#define SBP_LAUNCH_ON(kind, stream, expr)                                                      \
  do {                                                                                         \
    TimedLaunch tl_{kind, {nullptr, nullptr}};                                                 \
    if (c.timing) {                                                                            \
      tl_.ev[0] = take_event(h);                                                               \
      tl_.ev[1] = take_event(h);                                                               \
      if (!tl_.ev[0] || !tl_.ev[1]) return fail(h, STREAMBP_ERR_HIP, "hipEventCreate failed");  \
      (void)hipEventRecord(tl_.ev[0], stream);                                                 \
    }                                                                                          \
    hipError_t e_ = (expr);                                                                    \
    if (c.timing) {                                                                            \
      (void)hipEventRecord(tl_.ev[1], stream);                                                 \
      h->pending.push_back(tl_);                                                               \
    }                                                                                          \
    if (e_ == hipSuccess && h->debug) e_ = hipStreamSynchronize(stream);                       \
    if (e_ != hipSuccess) return fail(h, STREAMBP_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)
#define SBP_LAUNCH(kind, expr) SBP_LAUNCH_ON(kind, c.st, expr)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

streambp_status check_common(streambp_head h, const Call& c) {
  if (c.T < 0 || c.T > INT32_MAX) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "T=%lld out of range", (long long)c.T);
  if (!c.status) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "status pointer is NULL");
  const bool bwd = c.kind != Kind::DpoLogp;
  if (bwd && !c.dW) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "dW is NULL");
  if (bwd && !c.loss) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "loss is NULL");
  if (c.kind == Kind::DpoLogp && !c.seq_logp_out) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "seq_logp is NULL");
  if (c.kind != Kind::Sft) {
    if (c.n_seq < 1) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "n_seq=%d must be >= 1", c.n_seq);
    if (!c.offsets) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "seq_offsets is NULL");
  }
  if ((c.kind == Kind::Grpo || c.kind == Kind::Ppo) && !c.adv) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "adv is NULL");
  if (c.kind == Kind::Ppo) {
    if (!std::isfinite(c.eps) || c.eps < 0.0) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "clip eps must be finite and >= 0");
    if (!std::isfinite(c.beta_kl)) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "beta_kl is not finite");
    if (c.T > 0 && !c.logp_old) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "logp_old is NULL");
    if (c.T > 0 && c.beta_kl != 0.0 && !c.logp_ref)
      return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "logp_ref is NULL with beta_kl != 0");
  }
  if (c.kind == Kind::DpoBwd) {
    if (c.n_seq % 2) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "DPO needs an even n_seq (got %d)", c.n_seq);
    if (!c.seq_logp_in || !c.ref_logp) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "seq_logp/ref_logp is NULL");
    if (!std::isfinite(c.beta)) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "beta is not finite");
  }
  if (c.T > 0) {
    if (!c.H || !c.W || !c.labels) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "H, W or labels is NULL");
    if (bwd && !c.dH) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "dH is NULL");
    if (!aligned16(c.H) || !aligned16(c.W)) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "H and W must be 16-byte aligned");
    if (bwd && !aligned16(c.dH)) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "dH must be 16-byte aligned");
  }
  if (bwd && !aligned16(c.dW)) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "dW must be 16-byte aligned");
  const int n_seq = c.kind == Kind::Sft ? 1 : c.n_seq;
  const size_t need = layout(h, c.T, n_seq).total;
  if (!c.ws || ((uintptr_t)c.ws % kAlign) != 0)
    return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (c.ws_bytes < need)
    return fail(h, STREAMBP_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", c.ws_bytes, need);
  return STREAMBP_OK;
}

// The chunk loop: for each chunk of C rows, logits + LSE partials, the
// row-wise combine (and in-place logits gradient when `backward`), then the
// dH and dW GEMMs, all on the call's stream.  With masked-row compaction the
// chunks run over the valid rows only (token indices from the label scan):
// each chunk first copies its live rows of H into a dense buffer, and the
// number of live rows, known only on the device, bounds every kernel; dH rows
// are scattered back to their tokens by the split-K reduce.  The host still
// walks all ceil(T/C) chunks; chunks past the valid rows exit at once.
streambp_status run_chunks(streambp_head h, const Call& c, const Layout& L, bool backward) {
  char* ws = static_cast<char*>(c.ws);
  const bool bf16 = h->dtype == STREAMBP_BF16;
  const bool compact = h->compact;
  const size_t esize = bf16 ? 2 : 4;
  void* Z = ws + L.z;
  float2* part = reinterpret_cast<float2*>(ws + L.part);
  float* zy = reinterpret_cast<float*>(ws + L.zy);
  float* split = reinterpret_cast<float*>(ws + L.split);
  const float* w = reinterpret_cast<const float*>(ws + L.w);
  const float* inv_len = reinterpret_cast<const float*>(ws + L.w2);
  float* logp = c.logp_out ? c.logp_out : reinterpret_cast<float*>(ws + L.logp);
  double* loss_rows = reinterpret_cast<double*>(ws + L.loss_rows);
  const int32_t* rowmap = compact ? reinterpret_cast<const int32_t*>(ws + L.rowmap) : nullptr;
  const int32_t* live = compact ? reinterpret_cast<const int32_t*>(ws + L.scratch) : nullptr;
  uint16_t* Hdense = compact ? reinterpret_cast<uint16_t*>(ws + L.hdense) : nullptr;
  const bool tiled = bf16 && h->tiled;
  uint16_t* Wt = tiled ? reinterpret_cast<uint16_t*>(ws + L.wt) : nullptr;
  uint16_t* Ht = bf16 ? reinterpret_cast<uint16_t*>(ws + L.ht) : nullptr;
  uint16_t* HtT = bf16 ? reinterpret_cast<uint16_t*>(ws + L.htt) : nullptr;
  const int64_t D = h->D, V = h->V, C = h->C;
  const int vt_logits = (int)cdiv(V, sbp::kLogitsBM);

  auto chunk_rows = [&](int64_t row0) { return (c.T - row0 < C) ? c.T - row0 : C; };
  // rows of H the chunk's GEMMs read: the dense copy under compaction
  auto H_at = [&](int64_t row0) -> const char* {
    return compact ? reinterpret_cast<const char*>(Hdense) : static_cast<const char*>(c.H) + (size_t)row0 * D * esize;
  };
  // With every token's log-sum-exp known from the first DPO pass, the second
  // pass's logits epilogue writes G directly and the row pass is skipped (bf16).
  const bool fused = bf16 && backward && c.token_lse_in != nullptr;
  auto logits = [&](int64_t row0, int t0, int t1, hipStream_t st) -> streambp_status {
    const int64_t rows = chunk_rows(row0);
    const sbp::LogitsGrad lg{c.token_lse_in, w, c.labels, row0, rowmap, live, row0};
    const sbp::LogitsGrad* grad = fused ? &lg : nullptr;
    if (tiled)
      SBP_LAUNCH_ON(kKindLogits, st,
                    sbp::launch_logits_bf16_tiled(Wt, Ht, V, D, rows, backward ? static_cast<uint16_t*>(Z) : nullptr,
                                                  h->ldz, part, h->nvb, t0, t1, live, row0, grad, st));
    else if (bf16)
      SBP_LAUNCH_ON(kKindLogits, st,
                    sbp::launch_logits_bf16(static_cast<const uint16_t*>(c.W), Ht, V, D, rows,
                                            backward ? static_cast<uint16_t*>(Z) : nullptr, h->ldz, part, h->nvb, t0,
                                            t1, live, row0, grad, st));
    else
      SBP_LAUNCH_ON(kKindLogits, st,
                    sbp::launch_logits_f32(static_cast<const float*>(c.W), reinterpret_cast<const float*>(H_at(row0)), V,
                                           D, rows, static_cast<float*>(Z), h->ldz, c.labels + row0, part, h->nvb, zy, st));
    return STREAMBP_OK;
  };
  auto dw = [&](int64_t row0) -> streambp_status {
    const int64_t rows = chunk_rows(row0);
    const int acc = (c.accumulate || row0 > 0) ? 1 : 0;
    if (bf16)
      SBP_LAUNCH(kKindDw, sbp::launch_dw_bf16(static_cast<const uint16_t*>(Z), h->ldz, HtT, dw_tile_cols(rows), V, D,
                                              rows, c.dW, acc, live, row0, c.st));
    else
      SBP_LAUNCH(kKindDw, sbp::launch_dw_f32(static_cast<const float*>(Z), h->ldz,
                                             reinterpret_cast<const float*>(H_at(row0)), V, D, rows, c.dW, acc, c.st));
    return STREAMBP_OK;
  };
  streambp_status s;

  if (tiled && c.T > 0)
    SBP_LAUNCH(kKindTileW, sbp::launch_tile32(static_cast<const uint16_t*>(c.W), V, D, D, Wt,
                                              cdiv(V, sbp::kTiledRows), c.st));
  for (int64_t row0 = 0; row0 < c.T; row0 += C) {
    const int64_t rows = chunk_rows(row0);
    // per-token arrays: offset to the chunk, or indexed through the row map
    const int64_t tok0 = compact ? 0 : row0;
    const int32_t* cmap = compact ? rowmap + row0 : nullptr;
    if (compact)
      SBP_LAUNCH(kKindGather, sbp::launch_gather_rows(static_cast<const uint16_t*>(c.H), D, cmap, live, row0, rows,
                                                      Hdense, c.st));
    if (bf16)
      SBP_LAUNCH(kKindTileH, sbp::launch_tile32(reinterpret_cast<const uint16_t*>(H_at(row0)), rows, D, D, Ht,
                                                cdiv(rows, sbp::kTiledRows), c.st));
    if (bf16 && backward)
      SBP_LAUNCH(kKindTileHT, sbp::launch_tile32_t(reinterpret_cast<const uint16_t*>(H_at(row0)), rows, D, D, HtT,
                                                   dw_tile_cols(rows), live, row0, c.st));
    if ((s = logits(row0, 0, vt_logits, c.st)) != STREAMBP_OK) return s;
    sbp::PpoArgs pa{};
    if (c.kind == Kind::Ppo)
      pa = sbp::PpoArgs{c.logp_old + tok0, c.logp_ref ? c.logp_ref + tok0 : nullptr, inv_len + tok0, (float)c.eps,
                        (float)c.beta_kl};
    if (!fused)
      SBP_LAUNCH(kKindRows, sbp::launch_rows(bf16, backward, Z, h->ldz, V, rows, part, h->nvb, zy, H_at(row0), c.W, D,
                                             c.labels + tok0, w + tok0, c.kind == Kind::Ppo ? &pa : nullptr,
                                             logp + tok0, loss_rows + tok0,
                                             c.token_lse_out ? c.token_lse_out + tok0 : nullptr, cmap, live, row0,
                                             c.st));
    if (!backward) continue;
    float* dHc = c.dH + row0 * D;
    const int splits = h->dh_splits;
    // compaction always goes through the slabs: the reduce scatters the rows
    const bool slabs = splits > 1 || compact;
    float* dh_out = slabs ? split : dHc;
    const int64_t stride = C * D;
    if (bf16)
      SBP_LAUNCH(kKindDh, sbp::launch_dh_bf16(static_cast<const uint16_t*>(Z), h->ldz, static_cast<const uint16_t*>(c.W),
                                              V, D, rows, dh_out, splits, stride, live, row0, c.st));
    else
      SBP_LAUNCH(kKindDh, sbp::launch_dh_f32(static_cast<const float*>(Z), h->ldz, static_cast<const float*>(c.W), V, D,
                                             rows, dh_out, splits, stride, c.st));
    if (slabs)
      SBP_LAUNCH(kKindDhReduce, sbp::launch_splitk_reduce(split, splits, stride, rows, D, compact ? c.dH : dHc, cmap, live,
                                                          row0, c.st));

    if ((s = dw(row0)) != STREAMBP_OK) return s;
  }
  return STREAMBP_OK;
}

streambp_status run(streambp_head h, Call c) {
  if (!h) return STREAMBP_ERR_INVALID_ARGUMENT;
  h->err.clear();
  c.timing = h->timing && !c.static_scratch;  // the no-allocation entry creates no events
  const streambp_status chk = check_common(h, c);
  if (chk != STREAMBP_OK) return chk;
  DeviceGuard guard(h->device);
  if (!guard.ok) return fail(h, STREAMBP_ERR_HIP, "hipSetDevice(%d) failed", h->device);

  const int n_seq = c.kind == Kind::Sft ? 1 : c.n_seq;
  const Layout L = layout(h, c.T, n_seq);
  char* ws = static_cast<char*>(c.ws);
  float* w = reinterpret_cast<float*>(ws + L.w);
  int32_t* seq_len = reinterpret_cast<int32_t*>(ws + L.seq_len);
  double* coef = reinterpret_cast<double*>(ws + L.coef);
  double* loss_rows = reinterpret_cast<double*>(ws + L.loss_rows);
  float* logp = c.logp_out ? c.logp_out : reinterpret_cast<float*>(ws + L.logp);

  // dW is overwritten unless accumulating; with no rows nothing else writes it.
  if (c.kind != Kind::DpoLogp && c.T == 0 && !c.accumulate)
    SBP_LAUNCH(kKindFill, sbp::launch_fill_f32(c.dW, h->V * h->D, 0.f, c.st));

  // masked-row compaction: the scan lists the valid rows and zeroes the
  // per-token outputs of the others
  sbp::CompactRows cr{};
  if (h->compact)
    cr = sbp::CompactRows{reinterpret_cast<int32_t*>(ws + L.rowmap), reinterpret_cast<int32_t*>(ws + L.scratch), logp,
                          loss_rows};
  const sbp::CompactRows* crp = h->compact ? &cr : nullptr;

  switch (c.kind) {
    case Kind::Sft:
      SBP_LAUNCH(kKindScan, sbp::launch_scan_labels(c.labels, c.T, h->V, nullptr, 1, sbp::kWeightMean, nullptr, nullptr, w,
                                         nullptr, seq_len, c.n_valid, c.status, crp, c.st));
      break;
    case Kind::Grpo:
      SBP_LAUNCH(kKindScan, sbp::launch_scan_labels(c.labels, c.T, h->V, c.offsets, c.n_seq, sbp::kWeightAdv, c.adv, nullptr, w,
                                         nullptr, seq_len, nullptr, c.status, crp, c.st));
      break;
    case Kind::DpoLogp:
      SBP_LAUNCH(kKindScan, sbp::launch_scan_labels(c.labels, c.T, h->V, c.offsets, c.n_seq, sbp::kWeightNone, nullptr, nullptr,
                                         w, nullptr, seq_len, nullptr, c.status, crp, c.st));
      break;
    case Kind::Ppo:
      SBP_LAUNCH(kKindScan, sbp::launch_scan_labels(c.labels, c.T, h->V, c.offsets, c.n_seq, sbp::kWeightAdv, c.adv, nullptr, w,
                                         reinterpret_cast<float*>(ws + L.w2), seq_len, nullptr, c.status, crp, c.st));
      break;
    case Kind::DpoBwd:
      SBP_LAUNCH(kKindDpoPairs, sbp::launch_dpo_pairs(c.seq_logp_in, c.ref_logp, c.n_seq, c.beta, coef, c.loss, c.st));
      SBP_LAUNCH(kKindScan, sbp::launch_scan_labels(c.labels, c.T, h->V, c.offsets, c.n_seq, sbp::kWeightCoef, nullptr, coef, w,
                                         nullptr, seq_len, nullptr, c.status, crp, c.st));
      break;
  }

  if (h->compact && c.kind != Kind::DpoLogp && c.T > 0)
    SBP_LAUNCH(kKindZeroRows, sbp::launch_zero_dead_rows(c.dH, c.T, h->D, c.labels, h->V, c.status, c.st));

  const streambp_status s = run_chunks(h, c, L, c.kind != Kind::DpoLogp);
  if (s != STREAMBP_OK) return s;

  if (c.kind == Kind::Sft || c.kind == Kind::Grpo || c.kind == Kind::Ppo) SBP_LAUNCH(kKindLossSum, sbp::launch_sum_f64(loss_rows, c.T, c.loss, c.st));
  if (c.kind == Kind::DpoLogp) SBP_LAUNCH(kKindSeqSums, sbp::launch_seq_sums(logp, c.offsets, c.n_seq, c.T, c.seq_logp_out, c.st));
  return STREAMBP_OK;
}

}  // namespace

extern "C" {

STREAMBP_API const char* streambp_head_version(void) { return "streambp_head 0.1 (gfx950)"; }

STREAMBP_API streambp_status streambp_head_create(streambp_head* out, int64_t D, int64_t V, int64_t chunk, streambp_dtype dtype,
                                     int device) {
  if (!out) return STREAMBP_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (D <= 0 || V <= 0 || chunk <= 0) return STREAMBP_ERR_INVALID_ARGUMENT;
  if (D % 8 != 0) return STREAMBP_ERR_UNSUPPORTED;
  if (dtype != STREAMBP_F32 && dtype != STREAMBP_BF16) return STREAMBP_ERR_INVALID_ARGUMENT;
  if (V > INT32_MAX || D > INT32_MAX || chunk > INT32_MAX) return STREAMBP_ERR_UNSUPPORTED;
  if (device < 0) return STREAMBP_ERR_INVALID_ARGUMENT;
  // With no usable HIP runtime the handle is still created (argument checks
  // work without a device); calls then fail at hipSetDevice.
  int n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && device >= n) return STREAMBP_ERR_INVALID_ARGUMENT;
  streambp_head h = new (std::nothrow) streambp_head_s();
  if (!h) return STREAMBP_ERR_HIP;
  h->D = D;
  h->V = V;
  h->C = chunk;
  h->dtype = dtype;
  h->device = device;
  h->ldz = (V + 7) / 8 * 8;
  const bool bf16 = dtype == STREAMBP_BF16;
  h->nvb = cdiv(V, bf16 ? sbp::kLogitsBM : sbp::kF32TileW);
  h->dh_splits = choose_dh_splits(chunk, D, h->ldz, bf16);
  const char* dbg = getenv("STREAMBP_DEBUG");
  h->debug = dbg && dbg[0] && dbg[0] != '0';
  if (n > 0) {  // set-up of the no-allocation entry point on this device
    DeviceGuard guard(device);
    if (guard.ok) lookup_static_scratch(device);
  }
  *out = h;
  return STREAMBP_OK;
}

STREAMBP_API streambp_status streambp_head_destroy(streambp_head h) {
  if (!h) return STREAMBP_OK;
  {
    DeviceGuard guard(h->device);
    (void)drain_timing(h);
    for (hipEvent_t e : h->spare) (void)hipEventDestroy(e);
  }
  delete h;
  return STREAMBP_OK;
}

STREAMBP_API streambp_status streambp_head_set_timing(streambp_head h, int enable) {
  if (!h) return STREAMBP_ERR_INVALID_ARGUMENT;
  DeviceGuard guard(h->device);
  const hipError_t e = drain_timing(h);
  h->timing = enable != 0;
  for (int k = 0; k < kNumKinds; ++k) {
    h->total_ms[k] = 0.0;
    h->launches[k] = 0;
  }
  return e == hipSuccess ? STREAMBP_OK : fail(h, STREAMBP_ERR_HIP, "timing events: %s", hipGetErrorString(e));
}

STREAMBP_API streambp_status streambp_head_set_row_compaction(streambp_head h, int enable) {
  if (!h) return STREAMBP_ERR_INVALID_ARGUMENT;
  if (enable && h->dtype != STREAMBP_BF16)
    return fail(h, STREAMBP_ERR_UNSUPPORTED, "masked-row compaction needs a bf16 handle");
  h->compact = enable != 0;
  return STREAMBP_OK;
}

STREAMBP_API streambp_status streambp_head_set_tiled_logits(streambp_head h, int enable) {
  if (!h) return STREAMBP_ERR_INVALID_ARGUMENT;
  if (enable && h->dtype != STREAMBP_BF16)
    return fail(h, STREAMBP_ERR_UNSUPPORTED, "tiled logits operands need a bf16 handle");
  h->tiled = enable != 0;
  return STREAMBP_OK;
}

STREAMBP_API streambp_status streambp_head_mfma_probe(int64_t blocks, int32_t iters, int changing_operands,
                                                      double* flops, void* stream) {
  if (blocks < 1 || blocks > INT32_MAX || iters < 1) return STREAMBP_ERR_INVALID_ARGUMENT;
  if (sbp::launch_mfma_probe(blocks, iters, changing_operands != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
    return STREAMBP_ERR_HIP;
  if (flops) *flops = sbp::mfma_probe_flops(blocks, iters);
  return STREAMBP_OK;
}

STREAMBP_API int streambp_head_kernel_kinds(void) { return kNumKinds; }

STREAMBP_API const char* streambp_head_kernel_name(int kind) {
  return (kind >= 0 && kind < kNumKinds) ? kKindNames[kind] : "";
}

STREAMBP_API streambp_status streambp_head_kernel_times(streambp_head h, int kind, double* total_ms,
                                                        int64_t* launches) {
  if (!h || kind < 0 || kind >= kNumKinds) return STREAMBP_ERR_INVALID_ARGUMENT;
  DeviceGuard guard(h->device);
  const hipError_t e = drain_timing(h);
  if (total_ms) *total_ms = h->total_ms[kind];
  if (launches) *launches = h->launches[kind];
  return e == hipSuccess ? STREAMBP_OK : fail(h, STREAMBP_ERR_HIP, "timing events: %s", hipGetErrorString(e));
}

STREAMBP_API size_t streambp_head_workspace_bytes(streambp_head h, int64_t T, int32_t n_seq) {
  if (!h || T < 0) return 0;
  return layout(h, T, n_seq < 1 ? 1 : n_seq).total;
}

STREAMBP_API streambp_status streambp_head_suggest_chunk(int64_t D, int64_t V, int64_t T, int32_t n_seq,
                                            streambp_dtype dtype, size_t budget_bytes, int64_t* chunk_out) {
  if (!chunk_out) return STREAMBP_ERR_INVALID_ARGUMENT;
  *chunk_out = 0;
  if (D <= 0 || V <= 0 || T < 0 || n_seq < 1 || (dtype != STREAMBP_F32 && dtype != STREAMBP_BF16))
    return STREAMBP_ERR_INVALID_ARGUMENT;
  if (D % 8 != 0 || V > INT32_MAX || D > INT32_MAX) return STREAMBP_ERR_UNSUPPORTED;
  const int64_t top = T > 0 ? (T + 255) / 256 * 256 : 256;
  const bool bf16 = dtype == STREAMBP_BF16;
  // a host-only handle stand-in for the layout arithmetic
  streambp_head_s s;
  s.D = D;
  s.V = V;
  s.dtype = dtype;
  s.device = 0;
  s.ldz = (V + 7) / 8 * 8;
  s.nvb = cdiv(V, bf16 ? sbp::kLogitsBM : sbp::kF32TileW);
  s.debug = false;
  for (int64_t C = 256; C <= 16384 && C <= top; C *= 2) {
    s.C = C;
    s.dh_splits = choose_dh_splits(C, D, s.ldz, bf16);
    if (layout(&s, T, n_seq).total > budget_bytes) break;
    *chunk_out = C;
  }
  return *chunk_out ? STREAMBP_OK : STREAMBP_ERR_WORKSPACE_TOO_SMALL;
}

STREAMBP_API const char* streambp_head_last_error(streambp_head h) { return h ? h->err.c_str() : "null handle"; }

STREAMBP_API streambp_status streambp_head_sft(streambp_head h, int64_t T, const void* H, const void* W, const int32_t* labels,
                                  float* dH, float* dW, int accumulate_dW, double* loss, int64_t* n_valid,
                                  int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  Call c{};
  c.kind = Kind::Sft;
  c.T = T;
  c.H = H;
  c.W = W;
  c.labels = labels;
  c.n_seq = 1;
  c.dH = dH;
  c.dW = dW;
  c.accumulate = accumulate_dW;
  c.loss = loss;
  c.n_valid = n_valid;
  c.status = status;
  c.ws = workspace;
  c.ws_bytes = workspace_bytes;
  c.st = static_cast<hipStream_t>(stream);
  return run(h, c);
}

STREAMBP_API streambp_status streambp_head_sft_noalloc(streambp_head h, int64_t T, const void* H, const void* W,
                                                        const int32_t* labels, float* dH, float* dW, int accumulate_dW,
                                                        double* loss, int64_t* n_valid, int32_t* status, void* stream) {
  if (!h) return STREAMBP_ERR_INVALID_ARGUMENT;
  if (T < 0) return fail(h, STREAMBP_ERR_INVALID_ARGUMENT, "T=%lld out of range", (long long)T);
  const size_t need = layout(h, T, 1).total;
  if (need > STREAMBP_STATIC_SCRATCH_BYTES)
    return fail(h, STREAMBP_ERR_WORKSPACE_TOO_SMALL,
                "sft_noalloc: this call needs %zu bytes of workspace; the static scratch holds %zu "
                "(use streambp_head_sft with a caller workspace, or a smaller chunk)",
                need, (size_t)STREAMBP_STATIC_SCRATCH_BYTES);
  hipError_t e = hipSuccess;
  void* ws = static_scratch(h->device, &e);
  if (!ws) return fail(h, STREAMBP_ERR_HIP, "sft_noalloc: static scratch of device %d: %s", h->device, hipGetErrorString(e));
  Call c{};
  c.kind = Kind::Sft;
  c.T = T;
  c.H = H;
  c.W = W;
  c.labels = labels;
  c.n_seq = 1;
  c.dH = dH;
  c.dW = dW;
  c.accumulate = accumulate_dW;
  c.loss = loss;
  c.n_valid = n_valid;
  c.status = status;
  c.ws = ws;
  c.ws_bytes = STREAMBP_STATIC_SCRATCH_BYTES;
  c.st = static_cast<hipStream_t>(stream);
  c.static_scratch = true;
  return run(h, c);
}

STREAMBP_API streambp_status streambp_head_grpo(streambp_head h, int64_t T, const void* H, const void* W, const int32_t* labels,
                                   const int32_t* seq_offsets, int32_t n_seq, const float* adv, float* logp, float* dH,
                                   float* dW, int accumulate_dW, double* loss, int32_t* status, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  Call c{};
  c.kind = Kind::Grpo;
  c.T = T;
  c.H = H;
  c.W = W;
  c.labels = labels;
  c.offsets = seq_offsets;
  c.n_seq = n_seq;
  c.adv = adv;
  c.logp_out = logp;
  c.dH = dH;
  c.dW = dW;
  c.accumulate = accumulate_dW;
  c.loss = loss;
  c.status = status;
  c.ws = workspace;
  c.ws_bytes = workspace_bytes;
  c.st = static_cast<hipStream_t>(stream);
  return run(h, c);
}

STREAMBP_API streambp_status streambp_head_ppo(streambp_head h, int64_t T, const void* H, const void* W, const int32_t* labels,
                                  const int32_t* seq_offsets, int32_t n_seq, const float* adv, const float* logp_old,
                                  const float* logp_ref, double clip_eps, double beta_kl, float* logp, float* dH,
                                  float* dW, int accumulate_dW, double* loss, int32_t* status, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Call c{};
  c.kind = Kind::Ppo;
  c.T = T;
  c.H = H;
  c.W = W;
  c.labels = labels;
  c.offsets = seq_offsets;
  c.n_seq = n_seq;
  c.adv = adv;
  c.logp_old = logp_old;
  c.logp_ref = logp_ref;
  c.eps = clip_eps;
  c.beta_kl = beta_kl;
  c.logp_out = logp;
  c.dH = dH;
  c.dW = dW;
  c.accumulate = accumulate_dW;
  c.loss = loss;
  c.status = status;
  c.ws = workspace;
  c.ws_bytes = workspace_bytes;
  c.st = static_cast<hipStream_t>(stream);
  return run(h, c);
}

STREAMBP_API streambp_status streambp_head_dpo_logp(streambp_head h, int64_t T, const void* H, const void* W,
                                       const int32_t* labels, const int32_t* seq_offsets, int32_t n_seq,
                                       double* seq_logp, float* token_lse, int32_t* status, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  Call c{};
  c.kind = Kind::DpoLogp;
  c.T = T;
  c.H = H;
  c.W = W;
  c.labels = labels;
  c.offsets = seq_offsets;
  c.n_seq = n_seq;
  c.seq_logp_out = seq_logp;
  c.token_lse_out = token_lse;
  c.status = status;
  c.ws = workspace;
  c.ws_bytes = workspace_bytes;
  c.st = static_cast<hipStream_t>(stream);
  return run(h, c);
}

STREAMBP_API streambp_status streambp_head_dpo_bwd(streambp_head h, int64_t T, const void* H, const void* W,
                                      const int32_t* labels, const int32_t* seq_offsets, int32_t n_seq,
                                      const double* seq_logp, const double* ref_logp, double beta,
                                      const float* token_lse, float* dH, float* dW, int accumulate_dW, double* loss,
                                      int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  Call c{};
  c.kind = Kind::DpoBwd;
  c.T = T;
  c.H = H;
  c.W = W;
  c.labels = labels;
  c.offsets = seq_offsets;
  c.n_seq = n_seq;
  c.seq_logp_in = seq_logp;
  c.ref_logp = ref_logp;
  c.beta = beta;
  c.token_lse_in = token_lse;
  c.dH = dH;
  c.dW = dW;
  c.accumulate = accumulate_dW;
  c.loss = loss;
  c.status = status;
  c.ws = workspace;
  c.ws_bytes = workspace_bytes;
  c.st = static_cast<hipStream_t>(stream);
  return run(h, c);
}

}  // extern "C"
