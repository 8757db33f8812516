// Row-wise and small kernels of the chunked head: label scan and per-token
// weights, log-sum-exp combine + in-place logits gradient, deterministic
// reductions, and the DPO pair factors.
#include "common.h"
#include "kernels.h"

namespace sbp {

namespace {

constexpr int kScanThreads = 1024;

template <typename Tv>
__device__ Tv block_sum(Tv v, Tv* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  Tv r = 0;
  for (int i = 0; i < nw; ++i) r += red[i];  // fixed order
  return r;
}

// Label scan (integer work; a single block).  Validates sequence offsets,
// flags labels outside [0, V) that are not -100, counts the valid labels of
// every sequence and writes the per-token cross-entropy weight.
__global__ __launch_bounds__(kScanThreads) void scan_labels_kernel(const int32_t* y, int64_t T, int64_t V,
                                                                   const int32_t* offsets, int n_seq, int mode,
                                                                   const float* adv, const double* coef,
                                                                   float* w, float* inv_len, int32_t* seq_len,
                                                                   int64_t* n_valid, int32_t* status,
                                                                   int32_t* rowmap, int32_t* n_rows, float* logp,
                                                                   double* loss_rows) {
  __shared__ int red[kScanThreads / 64];
  __shared__ int wsum[kScanThreads / 64];
  const int tid = threadIdx.x;
  int bad = 0;
  if (offsets != nullptr) {
    for (int s = tid; s <= n_seq; s += blockDim.x) {
      const int64_t o = offsets[s];
      if (o < 0 || o > T) bad = 1;
      if (s == 0 && o != 0) bad = 1;
      if (s == n_seq && o != T) bad = 1;
      if (s < n_seq && offsets[s + 1] < o) bad = 1;
    }
  }
  bad = block_sum(bad, red);
  int lbad = 0;
  for (int64_t t = tid; t < T; t += blockDim.x) {
    const int32_t v = y[t];
    if (v != -100 && !label_ok(v, V)) lbad = 1;
  }
  lbad = block_sum(lbad, red);

  int64_t total = 0;
  for (int s = 0; s < n_seq; ++s) {
    int64_t lo = offsets ? offsets[s] : 0, hi = offsets ? offsets[s + 1] : T;
    if (bad) lo = hi = 0;
    int cnt = 0;
    for (int64_t t = lo + tid; t < hi; t += blockDim.x) cnt += label_ok(y[t], V) ? 1 : 0;
    cnt = block_sum(cnt, red);
    double cf = 0.0;
    bool per_len = false;
    if (mode == kWeightMean) { cf = 1.0; per_len = true; }
    if (mode == kWeightAdv) { cf = (double)adv[s]; per_len = true; }
    if (mode == kWeightCoef) cf = coef[s];
    const double ws = cnt == 0 ? 0.0 : (per_len ? cf / (double)cnt : cf);
    const float wsf = (float)ws;
    const float ilf = cnt == 0 ? 0.f : (float)(1.0 / (double)cnt);
    for (int64_t t = lo + tid; t < hi; t += blockDim.x) {
      const bool ok = label_ok(y[t], V);
      w[t] = ok ? wsf : 0.f;
      if (inv_len != nullptr) inv_len[t] = ok ? ilf : 0.f;
    }
    if (tid == 0 && seq_len != nullptr) seq_len[s] = cnt;
    total += cnt;
  }
  if (bad)
    for (int64_t t = tid; t < T; t += blockDim.x) {
      w[t] = 0.f;
      if (inv_len != nullptr) inv_len[t] = 0.f;
    }
  if (tid == 0) {
    if (n_valid != nullptr) *n_valid = total;
    *status = bad ? 1 : (lbad ? 5 : 0);
  }
  if (rowmap == nullptr) return;
  // Masked-row compaction: the valid positions in order (none when the
  // offsets are malformed), and zero logp and loss terms for the others,
  // which no row pass will visit.
  const int lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int64_t t0 = 0; t0 < T; t0 += blockDim.x) {
    const int64_t t = t0 + tid;
    const bool ok = t < T && !bad && label_ok(y[t], V);
    if (t < T && !ok) {
      logp[t] = 0.f;
      loss_rows[t] = 0.0;
    }
    // inclusive prefix count inside the wave, then across waves
    int v = ok ? 1 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o, kWave);
      if (lane >= o) v += u;
    }
    __syncthreads();
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int before = 0, tile = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
      if (i < wave) before += wsum[i];
      tile += wsum[i];
    }
    if (ok) rowmap[base + before + v - 1] = (int32_t)t;
    base += tile;
  }
  if (tid == 0) *n_rows = base;
}

// Masked-row compaction: copy the live rows of one chunk (token indices
// rowmap[0 .. live)) into a dense [cap x D] buffer, one block per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* H, int64_t D, const int32_t* rowmap,
                                                          const int32_t* count, int64_t base, int64_t cap,
                                                          uint16_t* out) {
  const int64_t r = blockIdx.x;
  int64_t rc = (int64_t)*count - base;
  rc = rc < 0 ? 0 : (rc > cap ? cap : rc);
  if (r >= rc) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(H + (int64_t)rowmap[r] * D);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + r * D);
  for (int64_t c = threadIdx.x; c < D / 8; c += blockDim.x) dst[c] = src[c];
}

// Masked-row compaction: zero the dH rows that no chunk writes (labels that
// are ignored or out of range, or every row when the offsets are malformed).
__global__ __launch_bounds__(256) void zero_dead_rows_kernel(float* dH, int64_t D, const int32_t* y, int64_t V,
                                                             const int32_t* status) {
  const int64_t t = blockIdx.x;
  if (*status != 1 && label_ok(y[t], V)) return;
  f32x4_t* row = reinterpret_cast<f32x4_t*>(dH + t * D);
  for (int64_t c = threadIdx.x; c < D / 4; c += blockDim.x) row[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Target logit z_y = H_t . W_y of a valid bf16 row, fp32 products summed in
// fp32 (both factors are exact in fp32); the block's threads share the dot.
__device__ __forceinline__ float target_logit_bf16(const uint16_t* Hrow, const uint16_t* Wrow, int64_t D,
                                                   float* red4) {
  const u32x4_t* h = reinterpret_cast<const u32x4_t*>(Hrow);
  const u32x4_t* wv = reinterpret_cast<const u32x4_t*>(Wrow);
  float a = 0.f;
  for (int64_t c = threadIdx.x; c < D / 8; c += blockDim.x) {
    const u32x4_t x = h[c], y = wv[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a = fmaf(bf16_bits_to_f32(x[e] & 0xffffu), bf16_bits_to_f32(y[e] & 0xffffu), a);
      a = fmaf(bf16_bits_to_f32(x[e] >> 16), bf16_bits_to_f32(y[e] >> 16), a);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, kWave);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = a;
  __syncthreads();
  return (red4[0] + red4[1]) + (red4[2] + red4[3]);
}

// Off-policy clipped-surrogate terms of one valid token (news article: PPO is
// among the objectives; the reading is the standard clipped surrogate with a
// per-sequence length normaliser and a k3 KL penalty):
//   r = exp(logp - old), L = -min(r a, clip(r, 1-eps, 1+eps) a) + k (e^d - d - 1),
//   d = ref - logp, a = A_s/len_s, k = beta/len_s.
// Returns the cross-entropy weight -dL/dlogp; the min's slope is that of the
// unclipped product when it is the minimum (ties included), else 0.
__device__ __forceinline__ float ppo_weight(float ell, float a, float il, float old, const float* ref, int64_t t,
                                            float eps, float beta, double* loss) {
  const float r = expf(ell - old);
  const float un = r * a;
  const float cl = fminf(fmaxf(r, 1.f - eps), 1.f + eps) * a;
  const bool take_un = un <= cl;
  double L = -(double)(take_un ? un : cl);
  float dL = take_un ? -a * r : 0.f;
  if (beta != 0.f) {
    const float k = beta * il;
    const float d = ref[t] - ell;
    const float em1 = expm1f(d);
    L += (double)k * ((double)em1 - (double)d);
    dL += k * (-em1);
  }
  *loss = L;
  return -dL;
}

// One block per row of the chunk.  bf16 rows compute their target logit from
// H and W here; fp32 rows take it from `zy`, captured by the logits epilogue.
// PPO rows form their weight from their own log-prob (see ppo_weight).
// A bf16 row of Z holds bf16(z - m_j), m_j the maximum of vocabulary tile j
// (the first member of partial j), so the softmax is exp((z - m_j) + (m_j - lse)):
// the stored values carry no error proportional to the logits' size.
// The log-sum-exp is kept as M + l (M the row maximum, l = log sum exp(z - M)
// = log1p of the merged partials' r)
// and every exponent is formed as (z - M) - l, (z - m_j) + ((m_j - M) - l) for
// bf16: differences of nearby floats are exact, so no rounding of the full
// lse (of the logits' size) enters.  The label's entry p_y - 1 is expm1 of
// its exponent: for a confident row it is a small number that exp(x) - 1
// would lose to cancellation.
constexpr int kRowTilesLds = 1024;  // tile maxima kept in LDS (V <= 262144); beyond, read from the partials
static_assert(kLogitsBM == 256, "a 16-byte chunk c of a bf16 row lies in vocabulary tile c >> 5");
template <bool BF16, bool BACKWARD, bool PPO>
__global__ __launch_bounds__(256) void rows_kernel(void* Zv, int64_t ldz, int64_t V, const float2* part,
                                                   int64_t nvb, const float* zy, const uint16_t* Hc,
                                                   const uint16_t* Wm, int64_t D, const int32_t* y,
                                                   const float* w, PpoArgs ppo, float* logp, double* loss_rows,
                                                   float* lse_out, const int32_t* rowmap, const int32_t* live,
                                                   int64_t live_base) {
  __shared__ float2 red[4];
  __shared__ float dot[4];
  __shared__ float M_s, l_s, w_s, gy_s;
  __shared__ float tile_max[BF16 && BACKWARD ? kRowTilesLds : 1];
  // r: row of the chunk buffers; t: token (per-token arrays are indexed by t,
  // which is r itself unless masked-row compaction maps the chunk's rows)
  const int64_t r = blockIdx.x;
  int64_t t = r;
  if (rowmap != nullptr) {
    int64_t rc = (int64_t)*live - live_base;
    if (r >= rc) return;
    t = rowmap[r];
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t yt = y[t];
  const bool valid = label_ok(yt, V);
  // the label's stored logit, fetched early (the row pass of every chunk row
  // runs at once, so this block's serial latency is the kernel's)
  float z_label = 0.f;
  if (BACKWARD && valid && tid == 0) {
    if constexpr (BF16)
      z_label = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(Zv)[r * ldz + yt]);
    else
      z_label = reinterpret_cast<const float*>(Zv)[r * ldz + yt];
  }
  float zt = 0.f;
  if constexpr (BF16) {
    if (valid) zt = target_logit_bf16(Hc + r * D, Wm + (int64_t)yt * D, D, dot);
  } else {
    if (valid) zt = zy[r];
  }

  float m = -INFINITY, s = -1.f;  // the empty set's partial
  const float2* p = part + r * nvb;
  const bool max_in_lds = BF16 && BACKWARD && nvb <= kRowTilesLds;
  for (int64_t b = tid; b < nvb; b += 256) {
    const float2 q = p[b];
    if (max_in_lds) tile_max[b] = q.x;
    lse_merge(m, s, q.x, q.y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) red[wave] = make_float2(m, s);
  __syncthreads();
  if (tid == 0) {
    float M = red[0].x, S = red[0].y;
    for (int i = 1; i < 4; ++i) lse_merge(M, S, red[i].x, red[i].y);
    const float l = log1pf(S);  // log of the row's sum of exp(z - M)
    M_s = M;
    l_s = l;
    if (lse_out != nullptr) lse_out[t] = M + l;
    const float ell = valid ? (zt - M) - l : 0.f;
    logp[t] = ell;
    float wt;
    if constexpr (PPO) {
      double L = 0.0;
      wt = valid ? ppo_weight(ell, w[t], ppo.inv_len[t], ppo.old[t], ppo.ref, t, ppo.eps, ppo.beta, &L) : 0.f;
      loss_rows[t] = valid ? L : 0.0;
    } else {
      wt = valid ? w[t] : 0.f;
      loss_rows[t] = -(double)w[t] * (double)ell;
    }
    w_s = wt;
    if (BACKWARD && valid) {
      // the label's entry w (p_y - 1), from the same stored logit as the rest
      // of the row (read before the row is overwritten: a barrier follows)
      float x;
      if constexpr (BF16)
        x = z_label + (((max_in_lds ? tile_max[yt >> 8] : p[yt >> 8].x) - M) - l);
      else
        x = (z_label - M) - l;
      gy_s = wt * expm1f(x);
    }
  }
  if (!BACKWARD) return;
  __syncthreads();
  const float M = M_s, l = l_s;
  const float wt = w_s, gy = gy_s;
  if (BF16) {
    u32x4_t* row = reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(Zv) + r * ldz);
    const int64_t nc = ldz / 8;
    if (wt == 0.f) {
      for (int64_t c = tid; c < nc; c += 256) row[c] = u32x4_t{0u, 0u, 0u, 0u};
      return;
    }
    // chunks that hold the label or padding columns (v >= V) take a rare branch
    const int64_t c_label = yt / 8, c_pad = V / 8;
#pragma unroll 4
    for (int64_t c = tid; c < nc; c += 256) {
      const u32x4_t z = row[c];
      // the 8 values of chunk c lie in vocabulary tile (8 c) / 256
      const float off = ((max_in_lds ? tile_max[c >> 5] : p[c >> 5].x) - M) - l;
      float g[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[2 * e] = wt * exp_fast(bf16_bits_to_f32(z[e] & 0xffffu) + off);
        g[2 * e + 1] = wt * exp_fast(bf16_bits_to_f32(z[e] >> 16) + off);
      }
      if (c == c_label || c >= c_pad) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t v = 8 * c + e;
          if (v == yt) g[e] = gy;
          if (v >= V) g[e] = 0.f;
        }
      }
      row[c] = u32x4_t{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                       pack_bf16x2(g[6], g[7])};
    }
  } else {
    f32x4_t* row = reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(Zv) + r * ldz);
    const int64_t nc = ldz / 4;
    if (wt == 0.f) {
      for (int64_t c = tid; c < nc; c += 256) row[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      return;
    }
#pragma unroll 4
    for (int64_t c = tid; c < nc; c += 256) {
      f32x4_t z = row[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t v = 4 * c + e;
        const float g = v == yt ? gy : wt * expf((z[e] - M) - l);
        z[e] = v < V ? g : 0.f;
      }
      row[c] = z;
    }
  }
}

// Sum of the split-K slabs in a fixed order.  With `rowmap` (masked-row
// compaction) row r of the slabs goes to row rowmap[r] of `out`, for the
// live rows only.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int splits, int64_t stride,
                                                            int64_t n4, float* out, int64_t d4,
                                                            const int32_t* rowmap, const int32_t* live,
                                                            int64_t live_base) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  int64_t o = i;
  if (rowmap != nullptr) {
    const int64_t r = i / d4;
    if (r >= (int64_t)*live - live_base) return;
    o = (int64_t)rowmap[r] * d4 + (i - r * d4);
  }
  const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part);
  f32x4_t a = p[i];
  for (int s = 1; s < splits; ++s) a += p[i + s * (stride / 4)];
  reinterpret_cast<f32x4_t*>(out)[o] = a;
}

// Deterministic sum of n doubles (one block, fixed assignment and order).
__global__ __launch_bounds__(1024) void sum_f64_kernel(const double* x, int64_t n, double* out) {
  __shared__ double red[16];
  double a = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) a += x[i];
  a = block_sum(a, red);
  if (threadIdx.x == 0) *out = a;
}

// Per-sequence sum of logp in float64, one block per sequence.  Offsets are
// clamped to [0, T] (the label scan reports malformed offsets).
__global__ __launch_bounds__(256) void seq_sums_kernel(const float* logp, const int32_t* offsets, int64_t T,
                                                       double* out) {
  __shared__ double red[4];
  const int s = blockIdx.x;
  int64_t lo = offsets[s], hi = offsets[s + 1];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  double a = 0.0;
  for (int64_t t = lo + threadIdx.x; t < hi; t += blockDim.x) a += (double)logp[t];
  a = block_sum(a, red);
  if (threadIdx.x == 0) out[s] = a;
}

// DPO pair factors: Delta_i = (S_i - R_i) - (S_{P+i} - R_{P+i});
// loss = mean softplus(-beta Delta); coef = +-(beta/P) sigmoid(-beta Delta).
__global__ __launch_bounds__(256) void dpo_pairs_kernel(const double* S, const double* R, int n_seq, double beta,
                                                        double* coef, double* loss) {
  __shared__ double red[4];
  const int P = n_seq / 2;
  double a = 0.0;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const double delta = (S[i] - R[i]) - (S[P + i] - R[P + i]);
    const double x = -beta * delta;
    const double e = exp(-fabs(x));
    const double sp = fmax(x, 0.0) + log1p(e);
    const double sg = x >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
    const double f = beta / (double)P * sg;
    coef[i] = f;
    coef[P + i] = -f;
    a += sp;
  }
  a = block_sum(a, red);
  if (threadIdx.x == 0) *loss = P > 0 ? a / (double)P : 0.0;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void finish_empty_kernel(double* loss, int64_t* n_valid, int32_t* status) {
  if (loss) *loss = 0.0;
  if (n_valid) *n_valid = 0;
  if (status) *status = 0;
}

}  // namespace

hipError_t launch_scan_labels(const int32_t* y, int64_t T, int64_t V, const int32_t* offsets, int n_seq, int mode,
                              const float* adv, const double* coef, float* w, float* inv_len, int32_t* seq_len,
                              int64_t* n_valid, int32_t* status, const CompactRows* cr, hipStream_t st) {
  scan_labels_kernel<<<1, kScanThreads, 0, st>>>(y, T, V, offsets, n_seq, mode, adv, coef, w, inv_len, seq_len,
                                                 n_valid, status, cr ? cr->rowmap : nullptr,
                                                 cr ? cr->count : nullptr, cr ? cr->logp : nullptr,
                                                 cr ? cr->loss_rows : nullptr);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* H, int64_t D, const int32_t* rowmap, const int32_t* count, int64_t base,
                              int64_t cap, uint16_t* out, hipStream_t st) {
  if (cap <= 0) return hipSuccess;
  gather_rows_kernel<<<(unsigned)cap, 256, 0, st>>>(H, D, rowmap, count, base, cap, out);
  return hipGetLastError();
}

hipError_t launch_zero_dead_rows(float* dH, int64_t T, int64_t D, const int32_t* y, int64_t V, const int32_t* status,
                                 hipStream_t st) {
  if (T <= 0) return hipSuccess;
  zero_dead_rows_kernel<<<(unsigned)T, 256, 0, st>>>(dH, D, y, V, status);
  return hipGetLastError();
}

hipError_t launch_rows(bool bf16, bool backward, void* Z, int64_t ldz, int64_t V, int64_t rows, const float2* part,
                       int64_t nvb, const float* zy, const void* Hc, const void* W, int64_t D, const int32_t* y,
                       const float* w, const PpoArgs* ppo, float* logp, double* loss_rows, float* lse_out,
                       const int32_t* rowmap, const int32_t* live, int64_t live_base, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const dim3 g((unsigned)rows), b(256);
  const uint16_t* h16 = static_cast<const uint16_t*>(Hc);
  const uint16_t* w16 = static_cast<const uint16_t*>(W);
  const PpoArgs pa = ppo ? *ppo : PpoArgs{nullptr, nullptr, nullptr, 0.f, 0.f};
#define SBP_ROWS(B, K, P)                                                                                   \
  rows_kernel<B, K, P><<<g, b, 0, st>>>(Z, ldz, V, part, nvb, zy, h16, w16, D, y, w, pa, logp, loss_rows, lse_out, \
                                        rowmap, live, live_base)
  if (ppo) {
    if (!backward) return hipErrorInvalidValue;
    if (bf16)
      SBP_ROWS(true, true, true);
    else
      SBP_ROWS(false, true, true);
  } else if (bf16 && backward) {
    SBP_ROWS(true, true, false);
  } else if (bf16) {
    SBP_ROWS(true, false, false);
  } else if (backward) {
    SBP_ROWS(false, true, false);
  } else {
    SBP_ROWS(false, false, false);
  }
#undef SBP_ROWS
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int splits, int64_t split_stride, int64_t rows, int64_t D,
                                float* out, const int32_t* rowmap, const int32_t* live, int64_t live_base,
                                hipStream_t st) {
  const int64_t n4 = rows * D / 4;
  if (n4 <= 0) return hipSuccess;
  splitk_reduce_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(part, splits, split_stride, n4, out, D / 4,
                                                                    rowmap, live, live_base);
  return hipGetLastError();
}

hipError_t launch_sum_f64(const double* x, int64_t n, double* out, hipStream_t st) {
  sum_f64_kernel<<<1, 1024, 0, st>>>(x, n, out);
  return hipGetLastError();
}

hipError_t launch_seq_sums(const float* logp, const int32_t* offsets, int n_seq, int64_t T, double* out,
                           hipStream_t st) {
  seq_sums_kernel<<<n_seq, 256, 0, st>>>(logp, offsets, T, out);
  return hipGetLastError();
}

hipError_t launch_dpo_pairs(const double* seq_logp, const double* ref_logp, int n_seq, double beta, double* coef,
                            double* loss, hipStream_t st) {
  dpo_pairs_kernel<<<1, 256, 0, st>>>(seq_logp, ref_logp, n_seq, beta, coef, loss);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_finish_empty(double* loss, int64_t* n_valid, int32_t* status, hipStream_t st) {
  finish_empty_kernel<<<1, 1, 0, st>>>(loss, n_valid, status);
  return hipGetLastError();
}

}  // namespace sbp
