// Launchers of the three bf16 MFMA GEMMs of one chunk.
#include "gemm_bf16.h"
#include "kernels.h"

#include <cstdlib>

namespace sbp {

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Tile-order bit: M is the fast tile index.  The dH GEMM uses it, so that
// the 4 token tiles sharing a W tile of one K slab run side by side on one
// XCD (its G tiles, 3x smaller in total, are the ones shared across XCDs).
constexpr int kOrderMFast = 2;

// The dW GEMM runs persistent (one block per CU walking the tiles) and
// pipelined (the next tile's first stages load while a tile stores) where it
// has more tiles than CUs.  STREAMBP_PERSISTENT_DW (read at every launch, for
// comparisons): 0 one tile per block, 1 persistent without the pipelining,
// 2 (default) pipelined where the shape allows it.
constexpr int kPersistentBlocks = 256;
static int persistent_dw() {
  const char* e = getenv("STREAMBP_PERSISTENT_DW");
  return (e && (e[0] == '0' || e[0] == '1')) ? e[0] - '0' : 2;
}

// Block-to-XCD tile mapping (on unless STREAMBP_XCD_REMAP=0).
static int xcd_remap() {
  static const int v = [] {
    const char* e = getenv("STREAMBP_XCD_REMAP");
    return (e && e[0] == '0') ? 0 : 1;
  }();
  return v;
}

// Z^T = W H_c^T: rows = vocab (K-major W), columns = tokens (K-major H_c), K = D.
// Only vocab tiles [tile_begin, tile_end) (of kLogitsBM rows) are computed.
// Z = NULL writes the LSE partials only (passes without a backward); `grad`
// (may be NULL) selects the gradient mode: G into Z, no partials.
template <class Epi>
static Epi logits_epilogue(uint16_t* Z, int64_t ldz, int64_t V, int64_t rows, float2* part, int64_t nvb,
                           const LogitsGrad* grad) {
  Epi e{Z, ldz, V, rows, part, nvb};
  if (grad != nullptr) {
    e.lse_in = grad->lse;
    e.w = grad->w;
    e.y = grad->y;
    e.tok0 = grad->tok0;
    e.rowmap = grad->rowmap;
    e.live = grad->live;
    e.live_base = grad->live_base;
  }
  return e;
}

// Z^T = W H_c^T from tiled copies of W and H_c (256 x 32 storage tiles, as
// written by launch_tile32), through the k = 32 ring.  Same results as
// launch_logits_bf16, bit for bit (same k order into the same accumulators).
hipError_t launch_logits_bf16_tiled(const uint16_t* Wt, const uint16_t* Ht, int64_t V, int64_t D, int64_t rows,
                                    uint16_t* Z, int64_t ldz, float2* part, int64_t nvb, int tile_begin, int tile_end,
                                    const int32_t* live_rows, int64_t live_base, const LogitsGrad* grad,
                                    hipStream_t st) {
  if (rows <= 0 || tile_end <= tile_begin) return hipSuccess;
  if (grad != nullptr && (Z == nullptr || grad->lse == nullptr || grad->w == nullptr || grad->y == nullptr))
    return hipErrorInvalidValue;
  const int64_t ntc = cdiv(D, kBK32);
  const OperandView A{Wt, ntc * kTile32, V, ntc * kBK32};
  const OperandView B{Ht, ntc * kTile32, rows, ntc * kBK32};
  const int tm = tile_end - tile_begin, tn = cdiv(rows, kLogitsBN);
  const LiveRows live{live_rows, live_base, rows, kLiveN, 0};
  if (grad != nullptr)
    gemm_bf16_pp_kernel<EpiLogitsGrad, kPPTiled, kPPTiled><<<tm * tn, kThreadsPP, 0, st>>>(
        A, B, tm, tn, tile_begin, ntc * kBK32, ntc * kBK32, xcd_remap(), live,
        logits_epilogue<EpiLogitsGrad>(Z, ldz, V, rows, part, nvb, grad));
  else
    gemm_bf16_pp_kernel<EpiLogits, kPPTiled, kPPTiled><<<tm * tn, kThreadsPP, 0, st>>>(
        A, B, tm, tn, tile_begin, ntc * kBK32, ntc * kBK32, xcd_remap(), live,
        logits_epilogue<EpiLogits>(Z, ldz, V, rows, part, nvb, nullptr));
  return hipGetLastError();
}

// Z^T = W H_c^T from row-major W and a tiled copy of H_c (the chunk's rows, as
// written by launch_tile32): H_c is small and read by every block, and its
// tiles turn each of its stages into one contiguous 16 KiB run.
hipError_t launch_logits_bf16(const uint16_t* W, const uint16_t* Ht, int64_t V, int64_t D, int64_t rows,
                              uint16_t* Z, int64_t ldz, float2* part, int64_t nvb, int tile_begin, int tile_end,
                              const int32_t* live_rows, int64_t live_base, const LogitsGrad* grad, hipStream_t st) {
  if (rows <= 0 || tile_end <= tile_begin) return hipSuccess;
  if (grad != nullptr && (Z == nullptr || grad->lse == nullptr || grad->w == nullptr || grad->y == nullptr))
    return hipErrorInvalidValue;
  const int64_t ntc = cdiv(D, kBK32);
  const OperandView A{W, D, V, D};
  const OperandView B{Ht, ntc * kTile32, rows, ntc * kBK32};
  const int tm = tile_end - tile_begin, tn = cdiv(rows, kLogitsBN);
  const LiveRows live{live_rows, live_base, rows, kLiveN, 0};
  if (grad != nullptr)
    gemm_bf16_pp_kernel<EpiLogitsGrad, kPPRowK, kPPTiled><<<tm * tn, kThreadsPP, 0, st>>>(
        A, B, tm, tn, tile_begin, ntc * kBK32, ntc * kBK32, xcd_remap(), live,
        logits_epilogue<EpiLogitsGrad>(Z, ldz, V, rows, part, nvb, grad));
  else
    gemm_bf16_pp_kernel<EpiLogits, kPPRowK, kPPTiled><<<tm * tn, kThreadsPP, 0, st>>>(
        A, B, tm, tn, tile_begin, ntc * kBK32, ntc * kBK32, xcd_remap(), live,
        logits_epilogue<EpiLogits>(Z, ldz, V, rows, part, nvb, nullptr));
  return hipGetLastError();
}

// X [rows][ld] (bf16 bits, the first `cols` columns, cols % 8 == 0) into 256 x 32
// storage tiles, tile-row tr holding rows 256 tr .. 256 tr + 255, ntc =
// ceil(cols / 32) tiles per tile-row, zero-padded.  A block converts 16 rows
// of 16 horizontally adjacent tiles (512 columns); each wave reads 4 of the
// rows as 1 KiB contiguous pieces (a lane's 16 bytes land in one tile row
// piece; the L2 merges the 64-byte pieces of a tile into whole lines).
constexpr int kTileGroup = 16;      // tiles per block of tile32_kernel
constexpr int kTileBlockRows = 16;  // rows per block (4 per wave: a chunk's copy runs 320 blocks at C = 1024, D = 2560)
constexpr int kTileThreads = 256;   // threads per block
__global__ __launch_bounds__(kTileThreads) void tile32_kernel(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld,
                                                          uint16_t* T, int64_t ntc) {
  const int64_t ngrp = (ntc + kTileGroup - 1) / kTileGroup;
  constexpr int kParts = 256 / kTileBlockRows;
  const int64_t tr = blockIdx.x / (ngrp * kParts), grp = (blockIdx.x / kParts) % ngrp;
  const int part = blockIdx.x % kParts;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t col = grp * kTileGroup * kBK32 + 8 * lane;  // this lane's 8 columns
  const int64_t tc = col / kBK32;
  if (tc >= ntc) return;
  const bool in_cols = col < cols;
  uint16_t* dst = T + (tr * ntc + tc) * kTile32 + (col % kBK32);
  constexpr int kWaveRows = kTileBlockRows * kWave / kTileThreads;
  constexpr int kBatch = kWaveRows < 8 ? kWaveRows : 8;  // rows in flight per lane
  static_assert(kWaveRows % kBatch == 0, "whole batches per wave");
  const int r_first = part * kTileBlockRows + wave * kWaveRows;
  for (int rr0 = r_first; rr0 < r_first + kWaveRows; rr0 += kBatch) {
    u32x4_t v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t r = tr * 256 + rr0 + b;
      v[b] = (in_cols && r < rows) ? *reinterpret_cast<const u32x4_t*>(X + r * ld + col) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) *reinterpret_cast<u32x4_t*>(dst + (rr0 + b) * kBK32) = v[b];
  }
}

hipError_t launch_tile32(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld, uint16_t* T, int64_t tile_rows,
                         hipStream_t st) {
  const int64_t ntc = cdiv(cols, kBK32);
  const int64_t blocks = tile_rows * ((ntc + kTileGroup - 1) / kTileGroup) * (256 / kTileBlockRows);
  if (blocks <= 0) return hipSuccess;
  tile32_kernel<<<(unsigned)blocks, kTileThreads, 0, st>>>(X, rows, cols, ld, T, ntc);
  return hipGetLastError();
}

// X [rows][ld] (bf16 bits, the first `cols` columns, cols % 8 == 0, X and ld
// 16-byte aligned) transposed into 256 x 32 storage tiles: tile (ct, rt), at
// T + (ct * nrt + rt) * kTile32, holds X[32 rt + k][256 ct + i] at [i][k],
// zero past rows and cols; nrt >= ceil(rows / 32) tile columns are written
// (the extra ones all zero).  One block per tile: the tile's 32 rows x 256
// columns come into LDS as 16-byte pieces (a wave reads two 512-byte row
// segments per instruction), then thread i writes the tile's row i, column
// 256 ct + i of those rows, as 64 contiguous bytes.
constexpr int kTpPad = 8;  // LDS row padding (bf16): rows stay 16-byte aligned
__global__ __launch_bounds__(kTileThreads) void tile32_t_kernel(const uint16_t* X, int64_t rows, int64_t cols,
                                                               int64_t ld, uint16_t* T, int64_t nrt,
                                                               const int32_t* live, int64_t live_base) {
  __shared__ __align__(16) uint16_t s[kBK32][256 + kTpPad];
  const int64_t ct = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  if (live != nullptr) {  // rows at or past the device-side live count are written as zero
    int64_t rc = (int64_t)__builtin_amdgcn_readfirstlane(*live) - live_base;
    rc = rc < 0 ? 0 : rc;
    rows = rc < rows ? rc : rows;
  }
  const int i = threadIdx.x;
  constexpr int kPieces = kBK32 * 256 / 8;  // 16-byte pieces of the block
  static_assert(kPieces % kTileThreads == 0, "whole pieces per thread");
#pragma unroll
  for (int q = 0; q < kPieces / kTileThreads; ++q) {
    const int idx = q * kTileThreads + i;
    const int r = idx >> 5, ch = idx & 31;  // row of the block, 16-byte piece of the row
    const int64_t gr = rt * kBK32 + r, gc = ct * 256 + 8 * ch;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (gr < rows && gc < cols) v = *reinterpret_cast<const u32x4_t*>(X + gr * ld + gc);
    *reinterpret_cast<u32x4_t*>(&s[r][8 * ch]) = v;
  }
  __syncthreads();
  uint32_t w[kBK32 / 2];
#pragma unroll
  for (int k2 = 0; k2 < kBK32 / 2; ++k2) w[k2] = (uint32_t)s[2 * k2][i] | ((uint32_t)s[2 * k2 + 1][i] << 16);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(T + (ct * nrt + rt) * kTile32 + (int64_t)i * kBK32);
#pragma unroll
  for (int q = 0; q < kBK32 / 8; ++q) dst[q] = u32x4_t{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
}

hipError_t launch_tile32_t(const uint16_t* X, int64_t rows, int64_t cols, int64_t ld, uint16_t* T, int64_t nrt,
                           const int32_t* live, int64_t live_base, hipStream_t st) {
  if (rows > nrt * kBK32) return hipErrorInvalidValue;
  const int64_t blocks = cdiv(cols, 256) * nrt;
  if (blocks <= 0) return hipSuccess;
  tile32_t_kernel<<<(unsigned)blocks, kTileThreads, 0, st>>>(X, rows, cols, ld, T, nrt, live, live_base);
  return hipGetLastError();
}

// dH_c = G W: rows = tokens (K-major G, K = padded vocab), columns = D (W is
// MN-major for this product).  `splits` slabs of K, each written to its own
// fp32 slab `split_stride` elements apart (or straight to dH when splits = 1).
hipError_t launch_dh_bf16(const uint16_t* G, int64_t ldz, const uint16_t* W, int64_t V, int64_t D, int64_t rows,
                          float* out, int splits, int64_t split_stride, const int32_t* live_rows, int64_t live_base,
                          hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const OperandView A{G, ldz, rows, ldz};
  const OperandView B{W, D, D, V};
  const EpiStore e{out, D, split_stride, rows, D};
  const int64_t ks = (int64_t)cdiv(cdiv(ldz, splits), kBK32) * kBK32;
  const int tm = cdiv(rows, kDhBM), tn = cdiv(D, kDhBN);
  gemm_bf16_pp_kernel<EpiStore, kPPRowK, kPPRowMN><<<tm * tn * splits, kThreadsPP, 0, st>>>(
      A, B, tm, tn, 0, ks, ldz, xcd_remap() | kOrderMFast, LiveRows{live_rows, live_base, rows, kLiveM, 0}, e);
  return hipGetLastError();
}

// dW (+)= G^T H_c, computed transposed: rows = D (H_c^T read from its 256 x
// 32 tiles, K-major: one ds_read_b128 per fragment), columns = vocab (G read
// MN-major), K = chunk rows; M is the fast tile index, so the D tiles that
// share a G tile run side by side on one XCD.  The tiles cover every k-stage
// the loop runs, padding included.  With device-side live rows (masked-row
// compaction) G reads zero past them, the tiles must be zero there too, and
// every tile is its own block; otherwise the launch is persistent where it
// has more tiles than CUs.
hipError_t launch_dw_bf16(const uint16_t* G, int64_t ldz, const uint16_t* HcT, int64_t nrt, int64_t V, int64_t D,
                          int64_t rows, float* dW, int accumulate, const int32_t* live_rows, int64_t live_base,
                          hipStream_t st) {
  const LiveRows live{live_rows, live_base, rows, kLiveK, accumulate};
  if (rows <= 0) return hipSuccess;
  static_assert(kDwMinStages == 2 * EpiAccum<kAccStream>::kPieces, "padded loop length of the streamed update");
  if (HcT == nullptr || nrt * kBK32 < rows || (accumulate && nrt < kDwMinStages)) return hipErrorInvalidValue;
  const OperandView A{HcT, nrt * kTile32, D, nrt * kBK32};
  const OperandView B{G, ldz, ldz, rows};
  const int tm = cdiv(D, kDwBM), tn = cdiv(V, kDwBN);
  const int order = xcd_remap() | kOrderMFast;
  const int ntiles = tm * tn;
  const int pmode = live_rows == nullptr ? persistent_dw() : 0;
  if (pmode == 2 && ntiles > kPersistentBlocks && D % kDwBM == 0 && rows > 4 * kBK32) {
    // pipelined: the next tile's first stages load while this one stores
    if (!accumulate)
      gemm_bf16_pp_persistent_kernel<EpiAccum<kAccStore, true>, kPPTiled, kPPRowMN, true>
          <<<kPersistentBlocks, kThreadsPP, 0, st>>>(A, B, tm, tn, 0, rows, rows, order, ntiles, live,
                                                    EpiAccum<kAccStore, true>{dW, D, D, V});
    else
      gemm_bf16_pp_persistent_kernel<EpiAccum<kAccStream, true>, kPPTiled, kPPRowMN, true>
          <<<kPersistentBlocks, kThreadsPP, 0, st>>>(A, B, tm, tn, 0, rows, rows, order, ntiles, live,
                                                    EpiAccum<kAccStream, true>{dW, D, D, V});
    return hipGetLastError();
  }
  if (pmode >= 1 && ntiles > kPersistentBlocks) {
    if (!accumulate)
      gemm_bf16_pp_persistent_kernel<EpiAccum<kAccStore>, kPPTiled, kPPRowMN, false>
          <<<kPersistentBlocks, kThreadsPP, 0, st>>>(A, B, tm, tn, 0, rows, rows, order, ntiles, live,
                                                    EpiAccum<kAccStore>{dW, D, D, V});
    else
      gemm_bf16_pp_persistent_kernel<EpiAccum<kAccStream>, kPPTiled, kPPRowMN, false>
          <<<kPersistentBlocks, kThreadsPP, 0, st>>>(A, B, tm, tn, 0, rows, rows, order, ntiles, live,
                                                    EpiAccum<kAccStream>{dW, D, D, V});
    return hipGetLastError();
  }
  // The first chunk of a call without accumulation only stores; the others
  // stream the old tile in during the loop.
  if (!accumulate)
    gemm_bf16_pp_kernel<EpiAccum<kAccStore>, kPPTiled, kPPRowMN><<<ntiles, kThreadsPP, 0, st>>>(
        A, B, tm, tn, 0, rows, rows, order, live, EpiAccum<kAccStore>{dW, D, D, V});
  else
    gemm_bf16_pp_kernel<EpiAccum<kAccStream>, kPPTiled, kPPRowMN><<<ntiles, kThreadsPP, 0, st>>>(
        A, B, tm, tn, 0, rows, rows, order, live, EpiAccum<kAccStream>{dW, D, D, V});
  return hipGetLastError();
}

}  // namespace sbp
