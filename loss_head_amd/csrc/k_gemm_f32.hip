// Launchers of the three fp32 GEMMs of one chunk (float32 heads).
#include "gemm_f32.h"
#include "kernels.h"

namespace sbp {

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

hipError_t launch_logits_f32(const float* W, const float* Hc, int64_t V, int64_t D, int64_t rows, float* Z,
                             int64_t ldz, const int32_t* y, float2* part, int64_t nvb, float* zy, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const OperandViewF32 A{W, D, V, D};
  const OperandViewF32 B{Hc, D, rows, D};
  const EpiLogitsF32 e{Z, ldz, V, rows, y, part, nvb, zy};
  const int tm = cdiv(V, kF32Tile), tn = cdiv(rows, kF32Tile);
  gemm_f32_kernel<true, true, EpiLogitsF32><<<tm * tn, 256, 0, st>>>(A, B, tm, tn, D, D, e);
  return hipGetLastError();
}

hipError_t launch_dh_f32(const float* G, int64_t ldz, const float* W, int64_t V, int64_t D, int64_t rows,
                         float* out, int splits, int64_t split_stride, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const OperandViewF32 A{G, ldz, rows, ldz};
  const OperandViewF32 B{W, D, D, V};
  const EpiStoreF32 e{out, D, split_stride, rows, D};
  const int64_t ks = (int64_t)cdiv(cdiv(ldz, splits), kF32BK) * kF32BK;
  const int tm = cdiv(rows, kF32Tile), tn = cdiv(D, kF32Tile);
  gemm_f32_kernel<true, false, EpiStoreF32><<<tm * tn * splits, 256, 0, st>>>(A, B, tm, tn, ks, ldz, e);
  return hipGetLastError();
}

hipError_t launch_dw_f32(const float* G, int64_t ldz, const float* Hc, int64_t V, int64_t D, int64_t rows,
                         float* dW, int accumulate, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const OperandViewF32 A{G, ldz, ldz, rows};
  const OperandViewF32 B{Hc, D, D, rows};
  const EpiAccumF32 e{dW, D, V, D, accumulate};
  const int tm = cdiv(V, kF32Tile), tn = cdiv(D, kF32Tile);
  gemm_f32_kernel<false, false, EpiAccumF32><<<tm * tn, 256, 0, st>>>(A, B, tm, tn, rows, rows, e);
  return hipGetLastError();
}

}  // namespace sbp
