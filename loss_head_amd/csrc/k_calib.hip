// Measurement aid: a loop of nothing but bf16 MFMAs, the dense rate this chip
// sustains for the instruction the GEMMs use (v_mfma_f32_32x32x16_bf16), as
// opposed to the data-sheet peak: with the same operands in every
// instruction, and with operands that change from one instruction to the
// next as in a GEMM (the chip's power limit lowers the clock more then).
// Not part of the head computation.
#include "common.h"
#include "kernels.h"

namespace sbp {

// Written only if a sum takes one exact value that the operands below never
// produce; an externally visible variable, so that the MFMAs feeding the
// condition are not optimised away.
__device__ float g_probe_sink[1];

namespace {

constexpr int kProbeThreads = 256;  // 4 waves: one per SIMD for each block on a CU
constexpr int kProbeChains = 8;     // independent accumulators per wave (128 registers)

// kChanging: consecutive MFMAs read different operand pairs (as in a GEMM);
// else every MFMA reads the same pair, the least switching activity.
template <bool kChanging>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters) {
  const uint32_t lane = threadIdx.x & 63;
  // 8 operand pairs of pseudo-random bf16 values of both signs in (-1/16,
  // 1/16), fixed over the loop (no VALU work inside it)
  bf16x8_t a[kProbeChains], b[kProbeChains];
#pragma unroll
  for (int q = 0; q < kProbeChains; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t x = (lane * 8 + e) * 0x9E3779B1u + q * 0x85EBCA77u + blockIdx.x;
      x ^= x >> 15;
      x *= 0x2C1B3C6Du;
      x ^= x >> 12;
      const float u = (float)(x & 0xFFFF) * (1.f / 65536.f) - 0.5f;  // [-0.5, 0.5)
      a[q][e] = (__bf16)(u * 0.125f);
      b[q][e] = (__bf16)(((float)((x >> 16) & 0xFFFF) * (1.f / 65536.f) - 0.5f) * 0.125f);
    }
  f32x16_t acc[kProbeChains];
#pragma unroll
  for (int q = 0; q < kProbeChains; ++q) acc[q] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < kProbeChains; ++q)
      acc[q] = kChanging ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q], b[(q + 3) % kProbeChains], acc[q], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[q], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kProbeChains; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += fabsf(acc[q][r]);
  if (s == -1.f) g_probe_sink[0] = s;  // a sum of magnitudes is never -1
}

}  // namespace

double mfma_probe_flops(int64_t blocks, int iters) {
  return (double)blocks * (kProbeThreads / 64) * (double)iters * kProbeChains * (2.0 * 32 * 32 * 16);
}

hipError_t launch_mfma_probe(int64_t blocks, int iters, bool changing, hipStream_t st) {
  if (blocks <= 0 || blocks > INT32_MAX || iters <= 0) return hipErrorInvalidValue;
  if (changing)
    mfma_probe_kernel<true><<<(unsigned)blocks, kProbeThreads, 0, st>>>(iters);
  else
    mfma_probe_kernel<false><<<(unsigned)blocks, kProbeThreads, 0, st>>>(iters);
  return hipGetLastError();
}

}  // namespace sbp
