// bf16 MFMA GEMM core for gfx950 and the three head epilogues.
//
// C[m][n] = sum_k A[m][k] * B[n][k], bf16 operands, fp32 accumulation with
// v_mfma_f32_32x32x16_bf16.  A block of 256 threads (4 waves) owns a BM x BN
// output tile; waves form a WM x WN grid and each wave owns FM x FN MFMA
// tiles of 32 x 32.  k advances in stages of 64 through double-buffered LDS.
//
// Operands come in two storage orders.  K-major: element (i, k) at
// ptr[i*ld + k] (16-byte global loads, stored straight to LDS).  MN-major:
// element (i, k) at ptr[k*ld + i]; a thread loads an 8 (k) x 8 (i) block as
// eight 16-byte rows and transposes it in registers, so LDS always holds the
// operand as [i][k] with k contiguous and every MFMA fragment is one 16-byte
// LDS read.  16-byte chunks of an LDS row are XOR-swizzled to spread banks
// for both the transposing writes and the fragment reads.
//
// MFMA 32x32 output layout (checked on gfx950): lane l, accumulator r holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32 x 32 tile.
#pragma once
#include <type_traits>

#include "common.h"

namespace sbp {

constexpr int kBK = 64;         // k per LDS stage
constexpr int kThreads = 256;   // threads per GEMM block

struct OperandView {
  const uint16_t* ptr;
  int64_t ld;       // elements between consecutive storage rows
  int64_t mn_ext;   // rows (i) at or beyond this read as zero; multiple of 8 for MN-major
  int64_t k_ext;    // k at or beyond this reads as zero; multiple of 8 for K-major
};

__device__ __forceinline__ int lds_slot(int row, int kc) {
  return row * (kBK / 8) + (kc ^ ((row ^ (row >> 3)) & 7));
}

template <int R>
struct LoadKMajor {
  static constexpr int kPer = R * (kBK / 8) / kThreads;
  static_assert(kPer >= 1 && (R * (kBK / 8)) % kThreads == 0, "tile too small");
  u32x4_t v[kPer];
  __device__ __forceinline__ void load(const OperandView& op, int64_t i0, int64_t k0, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + kThreads * u;
      const int64_t i = i0 + (c >> 3), k = k0 + (c & 7) * 8;
      if (i < op.mn_ext && k < op.k_ext)
        v[u] = *reinterpret_cast<const u32x4_t*>(op.ptr + i * op.ld + k);
      else
        v[u] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(u32x4_t* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = tid + kThreads * u;
      lds[lds_slot(c >> 3, c & 7)] = v[u];
    }
  }
};

template <int R>
struct LoadMNMajor {
  static constexpr int kGroups = R / 8;               // 8-wide groups along i
  static constexpr int kUnits = kGroups * (kBK / 8);  // 8x8 blocks per tile
  static constexpr int kPer = (kUnits + kThreads - 1) / kThreads;
  u32x4_t v[kPer][8];
  __device__ __forceinline__ void load(const OperandView& op, int64_t i0, int64_t k0, int tid) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int unit = tid + kThreads * u;
      if (kUnits % kThreads != 0 && unit >= kUnits) continue;
      const int64_t i = i0 + (unit % kGroups) * 8;
      const int64_t kb = k0 + (unit / kGroups) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t k = kb + j;
        if (i < op.mn_ext && k < op.k_ext)
          v[u][j] = *reinterpret_cast<const u32x4_t*>(op.ptr + k * op.ld + i);
        else
          v[u][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(u32x4_t* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int unit = tid + kThreads * u;
      if (kUnits % kThreads != 0 && unit >= kUnits) continue;
      const int row0 = (unit % kGroups) * 8, kc = unit / kGroups;
      // v[u][j] holds k-row j (8 consecutive i).  Output row q needs element q
      // of each k-row: dword q/2, low half for even q, high half for odd q.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4_t lo, hi;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t a = v[u][2 * p][e], b = v[u][2 * p + 1][e];
          lo[p] = (a & 0xffffu) | (b << 16);
          hi[p] = (a >> 16) | (b & 0xffff0000u);
        }
        lds[lds_slot(row0 + 2 * e, kc)] = lo;
        lds[lds_slot(row0 + 2 * e + 1, kc)] = hi;
      }
    }
  }
};

// What an epilogue learns about its place in the output.
struct TileCtx {
  int64_t m_wave, n_wave;   // first row / column owned by this wave
  int64_t m_block, n_block; // first row / column of the block tile
  int lane, wm, wn, tm, tn, split;
  void* lds;                // free LDS (>= 64 KiB) once the main loop is done
};

__device__ __forceinline__ int64_t acc_row(const TileCtx& c, int i, int r) {
  return c.m_wave + 32 * i + 8 * (r >> 2) + 4 * (c.lane >> 5) + (r & 3);
}
__device__ __forceinline__ int64_t acc_col(const TileCtx& c, int j) { return c.n_wave + 32 * j + (c.lane & 31); }

template <int BM, int BN, int WM, int WN, bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(OperandView A, OperandView B, int tiles_m,
                                                             int tiles_n, int64_t k_split, int64_t K,
                                                             Epi epi) {
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  static_assert(WM * WN == kThreads / kWave, "4 waves");
  using LA = typename std::conditional<A_KMAJOR, LoadKMajor<BM>, LoadMNMajor<BM>>::type;
  using LB = typename std::conditional<B_KMAJOR, LoadKMajor<BN>, LoadMNMajor<BN>>::type;
  constexpr int kStage = (BM + BN) * (kBK / 8);  // 16-byte slots per stage
  __shared__ u32x4_t lds[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int per_split = tiles_m * tiles_n;
  const int split = blockIdx.x / per_split;
  const int t = blockIdx.x - split * per_split;
  const int tn = t % tiles_n, tm = t / tiles_n;  // consecutive blocks share an A tile
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = (int64_t)split * k_split;
  const int64_t ke = (kb + k_split < K) ? kb + k_split : K;
  const int nk = ke > kb ? (int)((ke - kb + kBK - 1) / kBK) : 0;

  LA la;
  LB lb;
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  if (nk > 0) {
    la.load(A, m0, kb, tid);
    lb.load(B, n0, kb, tid);
    la.store(lds, tid);
    lb.store(lds + BM * (kBK / 8), tid);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(A, m0, kb + (int64_t)(kt + 1) * kBK, tid);
      lb.load(B, n0, kb + (int64_t)(kt + 1) * kBK, tid);
    }
    const u32x4_t* as = lds + cur * kStage;
    const u32x4_t* bs = as + BM * (kBK / 8);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kc = 2 * ks + (lane >> 5);
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, as[lds_slot(wm * (BM / WM) + 32 * i + (lane & 31), kc)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t, bs[lds_slot(wn * (BN / WN) + 32 * j + (lane & 31), kc)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(lds + (cur ^ 1) * kStage, tid);
      lb.store(lds + (cur ^ 1) * kStage + BM * (kBK / 8), tid);
    }
    __syncthreads();
  }

  TileCtx c;
  c.m_block = m0;
  c.n_block = n0;
  c.m_wave = m0 + wm * (BM / WM);
  c.n_wave = n0 + wn * (BN / WN);
  c.lane = lane;
  c.wm = wm;
  c.wn = wn;
  c.tm = tm;
  c.tn = tn;
  c.split = split;
  c.lds = lds;
  epi.template run<FM, FN, WM, BN / WN>(acc, c);
}

// ---------------------------------------------------------------------------
// Epilogue of the chunk logits GEMM, computed as Z^T = W H_c^T (rows m = vocab
// v, columns n = token t of the chunk).  Per (token, vocab tile of BM) it
// writes the partial (max, sum exp(z - max)) of the fp32 logits, captures the
// fp32 logit of the label, and stores the tile of Z[t][v] rounded to bf16.
// ---------------------------------------------------------------------------
struct EpiLogits {
  uint16_t* Z;          // [rows][ldz] chunk logits (bf16 bits)
  int64_t ldz;
  int64_t V;
  int64_t rows;         // tokens in this chunk
  const int32_t* y;     // labels of the chunk
  float2* part;         // [rows][nvb] (max, sumexp) per vocab tile
  int64_t nvb;
  float* zy;            // [rows] fp32 logit of the label

  template <int FM, int FN, int WM, int WNCOLS>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    float2* red = reinterpret_cast<float2*>(c.lds);  // [WM][block columns]
    constexpr int kCols = WNCOLS * (kThreads / kWave / WM);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t t = acc_col(c, j);
      const int yt = t < rows ? y[t] : -1;
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(c, i, r) < V) m = fmaxf(m, acc[i][j][r]);
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (acc_row(c, i, r) < V) s += exp_fast(acc[i][j][r] - m);
      }
      s += __shfl_xor(s, 32, kWave);
      if (c.lane < 32) red[c.wm * kCols + (t - c.n_block)] = make_float2(m, s);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(c, i, r) == (int64_t)yt) zy[t] = acc[i][j][r];
      if (t < rows) {
        uint16_t* zrow = Z + t * ldz;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t v0 = acc_row(c, i, 4 * q);
            if (v0 < ldz) {
              u32x2_t pk;
              pk[0] = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
              pk[1] = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              *reinterpret_cast<u32x2_t*>(zrow + v0) = pk;
            }
          }
      }
    }
    __syncthreads();
    if (c.wm == 0 && c.lane < 32) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t t = acc_col(c, j);
        if (t >= rows) continue;
        const int col = (int)(t - c.n_block);
        float m = red[col].x, s = red[col].y;
#pragma unroll
        for (int w = 1; w < WM; ++w) lse_merge(m, s, red[w * kCols + col].x, red[w * kCols + col].y);
        part[t * nvb + c.tm] = make_float2(m, s);
      }
    }
  }
};

// Plain fp32 store of the tile (dH, or one split-K slab of it).
struct EpiStore {
  float* out;            // base of split 0
  int64_t ldo;
  int64_t split_stride;  // elements between split slabs
  int64_t m_ext, n_ext;

  template <int FM, int FN, int WM, int WNCOLS>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    float* o = out + (int64_t)c.split * split_stride;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = acc_col(c, j);
      if (n >= n_ext) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = acc_row(c, i, r);
          if (m < m_ext) o[m * ldo + n] = acc[i][j][r];
        }
    }
  }
};

// dW tile update: dW = (accumulate ? dW : 0) + tile.
struct EpiAccum {
  float* out;
  int64_t ldo;
  int64_t m_ext, n_ext;
  int accumulate;

  template <int FM, int FN, int WM, int WNCOLS>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = acc_col(c, j);
      if (n >= n_ext) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = acc_row(c, i, r);
          if (m < m_ext) {
            float* p = out + m * ldo + n;
            *p = accumulate ? *p + acc[i][j][r] : acc[i][j][r];
          }
        }
    }
  }
};

}  // namespace sbp
