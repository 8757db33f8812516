// fp32 GEMM core (VALU FMA) for float32 heads, and its three head epilogues.
//
// C[m][n] = sum_k A[m][k] * B[n][k] in fp32.  A 256-thread block owns a
// 64 x 64 tile; each thread owns 4 consecutive rows x 4 consecutive columns.
// LDS holds both operands as [k][i] (i contiguous) so the inner loop reads
// float4 rows.  Operands are K-major (element (i,k) at ptr[i*ld + k]) or
// MN-major (at ptr[k*ld + i]); K-major needs k_ext % 4 == 0, MN-major needs
// mn_ext % 4 == 0, so every float4 is wholly inside or outside.
#pragma once
#include "common.h"

namespace sbp {

constexpr int kF32Tile = 64;
constexpr int kF32BK = 16;

struct OperandViewF32 {
  const float* ptr;
  int64_t ld, mn_ext, k_ext;
};

template <bool KMAJOR>
__device__ __forceinline__ void f32_load_tile(const OperandViewF32& op, int64_t i0, int64_t k0, int tid,
                                              float (*s)[kF32Tile + 4]) {
  if (KMAJOR) {
    const int i = tid >> 2, kq = (tid & 3) * 4;  // 64 rows x 4 float4 along k
    const int64_t gi = i0 + i, gk = k0 + kq;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (gi < op.mn_ext && gk < op.k_ext) v = *reinterpret_cast<const f32x4_t*>(op.ptr + gi * op.ld + gk);
    s[kq + 0][i] = v[0];
    s[kq + 1][i] = v[1];
    s[kq + 2][i] = v[2];
    s[kq + 3][i] = v[3];
  } else {
    const int k = tid >> 4, iq = (tid & 15) * 4;  // 16 k-rows x 16 float4 along i
    const int64_t gi = i0 + iq, gk = k0 + k;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (gi < op.mn_ext && gk < op.k_ext) v = *reinterpret_cast<const f32x4_t*>(op.ptr + gk * op.ld + gi);
    *reinterpret_cast<f32x4_t*>(&s[k][iq]) = v;
  }
}

struct TileCtxF32 {
  int64_t m0, n0;   // first row / column of this thread's 4 x 4 block
  int64_t mb, nb;   // first row / column of the block tile
  int tid, tm, tn, split;
  float* lds;       // >= 64 x 65 floats of free LDS
};

template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(OperandViewF32 A, OperandViewF32 B, int tiles_m,
                                                       int tiles_n, int64_t k_split, int64_t K, Epi epi) {
  __shared__ float sa[kF32BK][kF32Tile + 4];
  __shared__ float sb[kF32BK][kF32Tile + 4];
  __shared__ float scratch[kF32Tile * (kF32Tile + 1)];
  const int tid = threadIdx.x;
  const int per_split = tiles_m * tiles_n;
  const int split = blockIdx.x / per_split;
  const int t = blockIdx.x - split * per_split;
  const int tn = t % tiles_n, tm = t / tiles_n;
  const int64_t mb = (int64_t)tm * kF32Tile, nb = (int64_t)tn * kF32Tile;
  const int64_t kb = (int64_t)split * k_split;
  const int64_t ke = (kb + k_split < K) ? kb + k_split : K;
  const int ty = tid >> 4, tx = tid & 15;

  float acc[4][4] = {};
  for (int64_t k0 = kb; k0 < ke; k0 += kF32BK) {
    f32_load_tile<A_KMAJOR>(A, mb, k0, tid, sa);
    f32_load_tile<B_KMAJOR>(B, nb, k0, tid, sb);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kF32BK; ++k) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&sa[k][ty * 4]);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&sb[k][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  TileCtxF32 c;
  c.m0 = mb + ty * 4;
  c.n0 = nb + tx * 4;
  c.mb = mb;
  c.nb = nb;
  c.tid = tid;
  c.tm = tm;
  c.tn = tn;
  c.split = split;
  c.lds = scratch;
  epi.run_f32(acc, c);
}

// Logits epilogue for Z^T = W H_c^T (rows = vocab, columns = tokens): tile
// partial (m, r) per token (see lse_merge), the label's logit, and Z[t][v] in
// fp32.
struct EpiLogitsF32 {
  float* Z;
  int64_t ldz, V, rows;
  const int32_t* y;
  float2* part;
  int64_t nvb;
  float* zy;

  __device__ __forceinline__ void run_f32(float (&acc)[4][4], const TileCtxF32& c) const {
    float* s = c.lds;  // [64 tokens][65]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = c.n0 + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[(c.n0 - c.nb + j) * (kF32Tile + 1) + (c.m0 - c.mb + i)] = acc[i][j];
      if (t < rows && c.m0 < ldz) {
        f32x4_t v = {acc[0][j], acc[1][j], acc[2][j], acc[3][j]};
        *reinterpret_cast<f32x4_t*>(Z + t * ldz + c.m0) = v;
      }
    }
    __syncthreads();
    if (c.tid < kF32Tile) {
      const int64_t t = c.nb + c.tid;
      if (t < rows) {
        const float* row = s + c.tid * (kF32Tile + 1);
        const int yt = y[t];
        float m = -INFINITY;
        for (int i = 0; i < kF32Tile; ++i)
          if (c.mb + i < V) m = fmaxf(m, row[i]);
        // (m, r) partial: the maximum's own term (1) is left out of the sum
        float r = 0.f, ties = 0.f;
        if (m != -INFINITY)
          for (int i = 0; i < kF32Tile; ++i)
            if (c.mb + i < V) {
              if (row[i] < m) r += expf(row[i] - m);
              else ties += 1.f;
            }
        if (yt >= c.mb && yt < c.mb + kF32Tile && yt < V) zy[t] = row[yt - c.mb];
        part[t * nvb + c.tm] = make_float2(m, r + (ties - 1.f));
      }
    }
  }
};

struct EpiStoreF32 {
  float* out;
  int64_t ldo, split_stride, m_ext, n_ext;
  __device__ __forceinline__ void run_f32(float (&acc)[4][4], const TileCtxF32& c) const {
    float* o = out + (int64_t)c.split * split_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = c.m0 + i;
      if (m >= m_ext) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c.n0 + j < n_ext) o[m * ldo + c.n0 + j] = acc[i][j];
    }
  }
};

struct EpiAccumF32 {
  float* out;
  int64_t ldo, m_ext, n_ext;
  int accumulate;
  __device__ __forceinline__ void run_f32(float (&acc)[4][4], const TileCtxF32& c) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = c.m0 + i;
      if (m >= m_ext) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c.n0 + j < n_ext) {
          float* p = out + m * ldo + c.n0 + j;
          *p = accumulate ? *p + acc[i][j] : acc[i][j];
        }
    }
  }
};

}  // namespace sbp
