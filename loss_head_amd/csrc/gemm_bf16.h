// bf16 MFMA GEMM core for gfx950 and the three head epilogues.
//
// C[m][n] = sum_k A[m][k] * B[n][k], bf16 operands, fp32 accumulation with
// v_mfma_f32_32x32x16_bf16.  A block of 256 threads (4 waves) owns a BM x BN
// output tile; waves form a WM x WN grid and each wave owns FM x FN MFMA
// tiles of 32 x 32.
//
// Operand tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (lane l of a wave writes the 16 bytes it fetched to
// LDS base + 16*l), into two LDS stages of kBK = 64 k each, so no registers
// hold data in flight; a stage is refilled while the other is consumed.
// Which global chunk a lane fetches is chosen so that the LDS image is
// XOR-swizzled.  Lanes outside the operand fetch a 16-byte zero block.
//
//  K-major operand (element (i,k) at ptr[i*ld + k]): LDS [i][k], 128-byte rows
//    of eight 16-byte chunks; an MFMA fragment (8 consecutive k of one row) is
//    one ds_read_b128.
//  MN-major operand (element (i,k) at ptr[k*ld + i]): LDS [k][i], 512-byte
//    k-rows; a fragment is built from two ds_read_b64_tr_b16.  That
//    instruction works on groups of 16 lanes: lane q of a group receives
//    element q%4 of the 4-element rows addressed by lanes 4e + q/4, e = 0..3
//    (checked on gfx950).  Addressing lane j of a group at (k = kb + j/4,
//    i = ib + 4*(j%4)) therefore hands lane q the four k-values kb..kb+3 of
//    column ib + q.
//
// MFMA 32x32 output layout (checked on gfx950): lane l, accumulator r holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32 x 32 tile.
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"

namespace sbp {

constexpr int kBK = 64;         // k per LDS stage
constexpr int kStages = 2;      // LDS stages (double buffer)
constexpr int kSub = kBK / 16;  // MFMA k16 sub-steps per stage
constexpr int kThreads = 256;   // threads per GEMM block

struct OperandView {
  const uint16_t* ptr;
  int64_t ld;       // elements between consecutive storage rows
  int64_t mn_ext;   // rows (i) at or beyond this read as zero; multiple of 8 for MN-major
  int64_t k_ext;    // k at or beyond this reads as zero; multiple of 8 for K-major
};

// Cache-policy operand of the LDS-DMA builtin: the non-temporal bit (gfx950).
constexpr int kCachePolicyNT = 2;

// Rows that exist only on the device: with masked-row compaction the number
// of valid rows in a chunk (live = clamp(*count - base, 0, cap)) is known to
// the GPU alone.  `dim` says which GEMM dimension runs over those rows:
// tiles past them along M or N exit at once; along K the loop stops there,
// and a launch with no live rows exits without storing when `skip_empty`.
struct LiveRows {
  const int32_t* count;  // NULL: every row is live
  int64_t base;
  int64_t cap;
  int dim;               // kLiveM, kLiveN or kLiveK
  int skip_empty;
};
constexpr int kLiveM = 0, kLiveN = 1, kLiveK = 2;

// A 16-byte block of zeros in device memory: the source of out-of-range lanes.
__device__ u32x4_t g_zero16;

// Buffer-resource form of the LDS DMA (buffer_load_dwordx4 ... lds): the
// address is a uniform 48-bit base in the resource plus a per-lane 32-bit byte
// offset, and lanes at or past the resource's byte range read zero, so an
// in-range tile needs no per-lane address arithmetic or selects.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
extern "C" __device__ void sbp_raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) void* lds,
                                                   int size, int voffset, int soffset, int offset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// Raw (stride 0) resource over [base, base + bytes); the last word is the
// gfx9 data-format field for untyped dword access.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

// The same resource as the opaque type of the buffer load/store builtins.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_brsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0,
                                           __builtin_amdgcn_readfirstlane((int32_t)bytes), 0x00020000);
}

// K-major LDS: 16-byte slot of (row, k-chunk) in a [rows][64] bf16 stage
// (128-byte rows: one cache line of global memory per row and stage).
__device__ __forceinline__ int kmaj_slot(int row, int kc) { return row * 8 + (kc ^ ((row ^ (row >> 3)) & 7)); }
// MN-major LDS: chunk swizzle of a 512-byte k-row.
__device__ __forceinline__ int mn_swz(int k) { return 4 * ((k & 3) | (((k >> 3) & 1) << 2)); }

// Operand storage layouts (template argument of the GEMM kernel).
constexpr int kPlainK = 0;   // element (i,k) at ptr[i*ld + k]
constexpr int kPlainMN = 1;  // element (i,k) at ptr[k*ld + i]
__host__ __device__ constexpr bool layout_kmajor(int L) { return L == kPlainK; }

template <int R, int L>
struct TileDma {
  static constexpr bool KMAJOR = layout_kmajor(L);
  static constexpr int kSlots = R * kBK / 8;               // 16-byte slots per stage
  static constexpr int kInstr = kSlots / 64 / 4;           // DMA instructions per wave per stage
  static_assert(kInstr >= 1 && kSlots % 256 == 0, "tile too small");
  static_assert(KMAJOR || R == 256, "MN-major tiles are 256 wide");
  uint32_t off[kInstr];  // byte offset of this lane's chunk from the stage origin
  int kk[kInstr];        // k of this lane's chunk inside the stage; huge if outside along i
  int wave;              // wave-uniform

  __device__ __forceinline__ void plan(const OperandView& op, int64_t i0, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int s = (wave * kInstr + q) * 64 + lane;
      int i, k;
      if (KMAJOR) {
        i = s >> 3;
        k = ((s & 7) ^ ((i ^ (i >> 3)) & 7)) * 8;
        off[q] = (uint32_t)((i * op.ld + k) * 2);
      } else {
        k = s >> 5;
        i = ((s & 31) ^ mn_swz(k)) * 8;
        off[q] = (uint32_t)((k * op.ld + i) * 2);
      }
      kk[q] = (i0 + i < op.mn_ext) ? k : (1 << 30);
    }
  }
  // Stage with origin (i0, k0) through a buffer resource that ends where the
  // operand's last valid storage row ends, so rows past the operand read zero.
  // Exact for MN-major tiles: k-rows past k_ext are past the end, and columns
  // past mn_ext only feed output rows or columns that are never stored.  For
  // K-major tiles it is exact only when the whole stage lies below k_ext (the
  // caller checks; a partial last stage goes through issue()).
  __device__ __forceinline__ void issue_rsrc(const OperandView& op, int64_t i0, int64_t k0, u32x4_t* dst) const {
    const uint16_t* base = KMAJOR ? op.ptr + i0 * op.ld + k0 : op.ptr + k0 * op.ld + i0;
    const int64_t end = (KMAJOR ? op.mn_ext : op.k_ext) * op.ld;  // elements from op.ptr
    const int64_t left = end - (base - op.ptr);
    const int64_t bytes = left > 0 ? 2 * left : 0;
    const uint32_t range = bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
    const i32x4_t rsrc = make_rsrc(base, range);
#pragma unroll
    for (int q = 0; q < kInstr; ++q)
      sbp_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + (wave * kInstr + q) * 64), 16,
                              (int)off[q], 0, 0, 0);
  }
  // Stage with origin (i0, k0) into LDS stage `dst` (this operand's part).
  // `kleft` = number of k in range from k0 on (clamped to int).
  __device__ __forceinline__ void issue(const OperandView& op, int64_t i0, int64_t k0, int kleft, u32x4_t* dst,
                                        const char* zero) const {
    const char* base = reinterpret_cast<const char*>(KMAJOR ? op.ptr + i0 * op.ld + k0 : op.ptr + k0 * op.ld + i0);
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const char* src = kk[q] < kleft ? base + off[q] : zero;
      __builtin_amdgcn_global_load_lds(src, dst + (wave * kInstr + q) * 64, 16, 0, 0);
    }
  }
};

// LDS fragment reads are issued as inline asm: the compiler would otherwise
// treat the transpose read as possibly overlapping the in-flight LDS DMA and
// drain the whole ring before it.  Completion is then awaited explicitly with
// frag_wait(), which is tied to the fragment registers.
__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
  u32x4_t r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ u32x2_t lds_read_tr_b64(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
template <int N>
__device__ __forceinline__ void frag_wait(u32x4_t (&f)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}

// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)(p));
}

// Issue the reads of one MFMA operand fragment: 8 consecutive k (k16 substep
// `ks`, lane half lane/32) of tile row row0 + lane%32.  `st` is the LDS byte
// address of this operand's part of the stage.
template <bool KMAJOR, int R>
__device__ __forceinline__ u32x4_t issue_frag(uint32_t st, int row0, int ks, int lane) {
  if (KMAJOR) {
    const int row = row0 + (lane & 31);
    return lds_read_b128(st + 16u * kmaj_slot(row, 2 * ks + (lane >> 5)));
  } else {
    const int g = lane >> 4, j = lane & 15;
    const int i = row0 + 16 * (g & 1) + 4 * (j & 3);
    const int kb = 16 * ks + 8 * (g >> 1) + (j >> 2);
    const uint32_t a0 = st + 16u * (kb * (R / 8) + ((i >> 3) ^ mn_swz(kb))) + (i & 7) * 2;
    const uint32_t a1 = st + 16u * ((kb + 4) * (R / 8) + ((i >> 3) ^ mn_swz(kb + 4))) + (i & 7) * 2;
    const u32x2_t lo = lds_read_tr_b64(a0), hi = lds_read_tr_b64(a1);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
}

// Copy of an accumulator that must stay in an AGPR: VALU use of the
// accumulators otherwise lets the register allocator move them to VGPRs.
__device__ __forceinline__ float agpr_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// s_waitcnt with only the vector-memory counter bounded (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// What an epilogue learns about its place in the output.
struct TileCtx {
  int64_t m_wave, n_wave;   // first row / column owned by this wave
  int64_t m_block, n_block; // first row / column of the block tile
  int lane, wave, wm, wn, tm, tn, split;
  int nk;                   // k-stages of the main loop
  void* lds;                // free LDS (>= 64 KiB) once the main loop is done
  u32x4_t* extra;           // the epilogue's own LDS (Epi::kLdsExtra bytes), usable during the loop
};

__device__ __forceinline__ int64_t acc_row(const TileCtx& c, int i, int r) {
  return c.m_wave + 32 * i + 8 * (r >> 2) + 4 * (c.lane >> 5) + (r & 3);
}
__device__ __forceinline__ int64_t acc_col(const TileCtx& c, int j) { return c.n_wave + 32 * j + (c.lane & 31); }

// Block id -> logical tile.  The hardware deals consecutive blocks round-robin
// to the 8 XCDs (each with its own L2); give every XCD a contiguous range of
// logical tiles so that blocks sharing an operand tile share an L2.
__device__ __forceinline__ int xcd_logical_block(int b, int nb) {
  constexpr int kXcds = 8;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int per = nb / kXcds, rem = nb % kXcds;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Main loop.  Fragment reads always run one k16 sub-step ahead of the MFMAs,
// across stage boundaries.  At the last sub-step of stage kt a first barrier
// (all waves have read stage kt) lets the buffer of stage kt refill with
// stage kt+2; each wave then waits for its own loads of stage kt+1 and a
// second barrier publishes them, after which the reads of stage kt+1 start.
template <int BM, int BN, int WM, int WN, int LA, int LB, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(OperandView A, OperandView B, int tiles_m,
                                                             int tiles_n, int tm_base, int64_t k_split, int64_t K,
                                                             int order, LiveRows live, Epi epi) {
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  static_assert(WM * WN == kThreads / kWave, "4 waves");
  static_assert(kStages == 2, "double-buffered stages");
  constexpr bool A_KMAJOR = layout_kmajor(LA), B_KMAJOR = layout_kmajor(LB);
  using DA = TileDma<BM, LA>;
  using DB = TileDma<BN, LB>;
  constexpr int kStageSlots = DA::kSlots + DB::kSlots;
  constexpr int kPerStage = DA::kInstr + DB::kInstr;  // vector-memory ops per wave per stage
  __shared__ u32x4_t lds[kStages * kStageSlots + Epi::kLdsExtra / 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int per_split = tiles_m * tiles_n;
  // order: bit 0 of `order` maps blocks to XCDs in contiguous ranges of
  // logical tiles; bit 1 makes M the fast tile index (consecutive tiles share
  // a B tile) instead of N (consecutive tiles share an A tile)
  const int lb_id = (order & 1) ? xcd_logical_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int split = lb_id / per_split;
  const int t = lb_id - split * per_split;
  const bool m_fast = (order & 2) != 0;
  const int tn = m_fast ? t / tiles_m : t % tiles_n;
  const int tm = tm_base + (m_fast ? t % tiles_m : t / tiles_n);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = (int64_t)split * k_split;
  int64_t ke = (kb + k_split < K) ? kb + k_split : K;
  if (live.count != nullptr) {
    int64_t rc = (int64_t)__builtin_amdgcn_readfirstlane(*live.count) - live.base;
    rc = rc < 0 ? 0 : (rc > live.cap ? live.cap : rc);
    if (live.dim == kLiveM && m0 >= rc) return;
    if (live.dim == kLiveN && n0 >= rc) return;
    if (live.dim == kLiveK) {
      if (rc == 0 && live.skip_empty) return;
      // rows past the live ones read as zero in both operands
      if (A.k_ext > rc) A.k_ext = rc;
      if (B.k_ext > rc) B.k_ext = rc;
      if (ke > rc) ke = rc;
    }
  }
  int nk = ke > kb ? (int)((ke - kb + kBK - 1) / kBK) : 0;
  // an epilogue may need a minimum number of stages; those past ke read zeros
  if (nk > 0 && nk < Epi::kMinStages) nk = Epi::kMinStages;

  DA da;
  DB db;
  da.plan(A, m0, tid);
  db.plan(B, n0, tid);
  const char* zero = reinterpret_cast<const char*>(&g_zero16);
  const uint32_t lds_base = lds_addr(lds);
  auto issue = [&](int st) {
    u32x4_t* dst = lds + (st % kStages) * kStageSlots;
    const int64_t k0 = kb + (int64_t)st * kBK;
    const int64_t la = A.k_ext - k0, lbk = B.k_ext - k0;
    if (!A_KMAJOR || la >= kBK)
      da.issue_rsrc(A, m0, k0, dst);
    else
      da.issue(A, m0, k0, (int)la, dst, zero);
    if (!B_KMAJOR || lbk >= kBK)
      db.issue_rsrc(B, n0, k0, dst + DA::kSlots);
    else
      db.issue(B, n0, k0, (int)lbk, dst + DA::kSlots, zero);
  };
  auto read_frags = [&](u32x4_t (&f)[FM + FN], int st, int ks) {
    const uint32_t as = lds_base + 16u * (uint32_t)((st % kStages) * kStageSlots);
    const uint32_t bs = as + 16u * DA::kSlots;
#pragma unroll
    for (int i = 0; i < FM; ++i) f[i] = issue_frag<A_KMAJOR, BM>(as, wm * (BM / WM) + 32 * i, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) f[FM + j] = issue_frag<B_KMAJOR, BN>(bs, wn * (BN / WN) + 32 * j, ks, lane);
  };

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
  c.wave = __builtin_amdgcn_readfirstlane(wave);
  c.nk = nk;
  c.lds = lds;
  c.extra = lds + kStages * kStageSlots;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};
  epi.template pre_loop<FM, FN>(acc, c);

  u32x4_t fa[FM + FN], fb[FM + FN];
  if (nk > 0) {
    issue(0);
    if (nk > 1) {
      issue(1);
      wait_vmcnt<kPerStage>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    read_frags(fa, 0, 0);
    frag_wait(fa);
  }

  // MFMAs lo .. hi-1 of the FM x FN products of one sub-step (row-major).
  auto mfmas = [&](u32x4_t (&f)[FM + FN], auto lo, auto hi) {
    constexpr int kLo = decltype(lo)::value, kHi = decltype(hi)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (i * FN + j >= kLo && i * FN + j < kHi)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f[i]),
                                                              __builtin_bit_cast(bf16x8_t, f[FM + j]), acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using IH = std::integral_constant<int, FM * FN / 2>;
  using IN = std::integral_constant<int, FM * FN>;
  // One sub-step: read ahead into `nx`, multiply `cu`, wait for `nx`.  The
  // last sub-step of stage kt also turns the ring over:
  //  * every wave read its last fragments of stage kt in the previous
  //    sub-step, so after a first barrier that buffer is refilled with stage
  //    kt+2;
  //  * each wave then waits for its own loads of stage kt+1 only (loads
  //    complete in order, so kt+2 stays in flight), and a second barrier
  //    makes all of stage kt+1 visible before its first reads.
  // The epilogue's hook for compile-time stage number Q (>= 0 only in the
  // unrolled head of the loop) runs right after that wait.  The MFMAs stay
  // outside every run-time branch (accumulators merged across branches end up
  // in scratch).  Epi::kGrouped selects the instruction order: false leaves
  // the interleaving of reads and MFMAs to the compiler; true pins the reads
  // ahead of the MFMAs with scheduling barriers and, at the ring turn, runs
  // half of the MFMAs between the barriers (faster for the dW GEMM, whose
  // hook adds LDS traffic at the turn; slower for the other two).
  auto substep = [&](int kt, int ks, u32x4_t (&cu)[FM + FN], u32x4_t (&nx)[FM + FN], auto qc) {
    constexpr int Q = decltype(qc)::value;
    constexpr bool kG = Epi::kGrouped;
    if (ks + 1 < kSub) {
      read_frags(nx, kt, ks + 1);
      if constexpr (kG) __builtin_amdgcn_sched_barrier(0);
      mfmas(cu, I0{}, IN{});
    } else {
      __builtin_amdgcn_s_barrier();
      if constexpr (kG) {
        mfmas(cu, I0{}, IH{});
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kt + 2 < nk) {
        issue(kt + 2);
        wait_vmcnt<kPerStage>();
      } else {
        wait_vmcnt<0>();
      }
      if constexpr (Q >= 0) epi.template stage_hook<Q, FM, FN>(acc, c);
      __builtin_amdgcn_s_barrier();
      if (kt + 1 < nk) read_frags(nx, kt + 1, 0);
      if constexpr (kG) {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(cu, IH{}, IN{});
      } else {
        mfmas(cu, I0{}, IN{});
      }
    }
    if constexpr (kG) __builtin_amdgcn_sched_barrier(0);
    frag_wait(nx);
  };
  auto stage = [&](int kt, auto qc) {
    using NoHook = std::integral_constant<int, -1>;
    __builtin_amdgcn_sched_barrier(0);  // keep stages from being interleaved (register pressure)
    substep(kt, 0, fa, fb, NoHook{});
    substep(kt, 1, fb, fa, NoHook{});
    substep(kt, 2, fa, fb, NoHook{});
    substep(kt, 3, fb, fa, qc);
  };
  int kt = 0;
  if (epi.streams(c)) {
    // stages 0 .. kHookStages-1 with the hook's stage number as a constant
    [&]<int... Qs>(std::integer_sequence<int, Qs...>) {
      ((kt < nk ? (stage(kt, std::integral_constant<int, Qs>{}), ++kt) : 0), ...);
    }(std::make_integer_sequence<int, Epi::kHookStages>{});
  }
  for (; kt < nk; ++kt) stage(kt, std::integral_constant<int, -1>{});
  __syncthreads();
  epi.template run<FM, FN, WM, BN / WN>(acc, c);
}

// ---------------------------------------------------------------------------
// Main loop for two K-major operands kept in 256 x 32 storage tiles (16 KiB,
// row-major [256][32]; tile (i/256, k/32) at ptr + (i/256)*ld + (k/32)*8192),
// zero-padded to whole tiles.  A k-stage is then one contiguous tile per
// operand: full cache lines in a single run, where a stage of a row-major
// operand is 256 pieces of 64 bytes.  Stages of k = 32 (32 KiB for both
// operands) make a ring of 4 in the LDS a 256 x 256 tile leaves.
//
// The block has 8 waves, two per SIMD (waves w and w+4 share one), each
// owning a 128 x 64 piece of the tile (128 accumulator registers, so two
// waves fit a SIMD's register file).  Waves 0-3 and 4-7 run the same loop
// one phase apart ("ping-pong"): per stage a memory phase (issue this wave's
// part of the DMA of stage st+3, read the stage's 12 fragments, wait for them
// and for this wave's loads of stage st+1) and a compute phase (16 MFMAs),
// each ended by a block barrier.  Group 1 enters the loop one barrier late,
// so between any two barriers one wave of every SIMD issues MFMAs while the
// other issues memory operations: a wave stalled on a DMA or LDS issue no
// longer leaves its SIMD's matrix core idle.
//
// Barrier b is the b-th s_barrier after the prologue's.  Group 0 ends the
// memory phase of stage st at barrier 2st+1 and its compute phase at 2st+2;
// group 1 one later.  Stage st is read by group 0 between barriers 2st and
// 2st+1 and by group 1 between 2st+1 and 2st+2; every wave waited for its own
// loads of stage st at the end of its memory phase of stage st-1, i.e. by
// barrier 2st, so the stage is whole before either group reads it.  The DMA
// of stage st+3 refills the buffer of stage st-1, whose last reads (group 1,
// completed before barrier 2st) precede both groups' memory phase of stage st.
// Each accumulator still takes its k16 products in ascending k, so results
// are bitwise those of the plain loop.
constexpr int kBK32 = 32;
constexpr int kTile32 = 256 * kBK32;  // elements per storage tile
constexpr int kRing32 = 4;            // stages in the ring
constexpr int kThreadsPP = 512;       // threads of the ping-pong GEMM block

// LDS slot of 16-byte chunk kc (0..3) of row `row` of a k = 32 stage: 64-byte
// rows, chunks XOR-swizzled by bits 2-3 of the row, so that the 16 lanes of a
// ds_read_b128 phase (16 consecutive rows, one chunk) hit 16 distinct 4-bank
// groups.
__device__ __forceinline__ int t32_slot(int row, int kc) { return row * 4 + (kc ^ ((row >> 2) & 3)); }

struct TileDma32 {
  static constexpr int kSlots = 256 * kBK32 / 8;      // 16-byte slots per operand and stage
  static constexpr int kInstr = kSlots / kThreadsPP;  // DMA instructions per wave, operand and stage
  uint32_t off[kInstr];  // byte offset of this lane's chunk inside the tile
  int wave;
  __device__ __forceinline__ void plan(int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int sl = (wave * kInstr + q) * 64 + lane;
      const int i = sl >> 2, kc = (sl & 3) ^ ((i >> 2) & 3);
      off[q] = (uint32_t)((i * kBK32 + kc * 8) * 2);
    }
  }
  // resource over the tile of stage origin (i0, k0): i0 a multiple of 256, k0 of 32
  __device__ __forceinline__ i32x4_t rsrc(const OperandView& op, int64_t i0, int64_t k0) const {
    return make_rsrc(op.ptr + (i0 >> 8) * op.ld + (k0 >> 5) * kTile32, 2 * kTile32);
  }
  __device__ __forceinline__ void issue(i32x4_t r, u32x4_t* dst, int q) const {
    sbp_raw_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (wave * kInstr + q) * 64), 16,
                            (int)off[q], 0, 0, 0);
  }
};

// A K-major operand stored row-major (element (i,k) at ptr[i*ld + k]), staged
// into the same [256][32] LDS image as a storage tile: lane chunk (i, kc)
// comes from 16 bytes of row i, so a stage is 256 pieces of 64 bytes.
struct RowDma32 {
  static constexpr int kInstr = TileDma32::kInstr;
  uint32_t off[kInstr];  // byte offset of this lane's chunk from the stage origin (i0, k0)
  int kk[kInstr];        // k of the chunk inside the stage; huge if its row is past mn_ext
  int wave;
  __device__ __forceinline__ void plan(const OperandView& op, int64_t i0, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const int sl = (wave * kInstr + q) * 64 + lane;
      const int i = sl >> 2, kc = (sl & 3) ^ ((i >> 2) & 3);
      off[q] = (uint32_t)((i * op.ld + kc * 8) * 2);
      kk[q] = (i0 + i < op.mn_ext) ? kc * 8 : (1 << 30);
    }
  }
  // A stage wholly below k_ext, through a resource that ends with the
  // operand's last valid row: rows past it read zero.
  __device__ __forceinline__ void issue_rsrc(const OperandView& op, int64_t i0, int64_t k0, u32x4_t* dst) const {
    const uint16_t* base = op.ptr + i0 * op.ld + k0;
    const int64_t left = op.mn_ext * op.ld - (base - op.ptr);
    const int64_t bytes = left > 0 ? 2 * left : 0;
    const i32x4_t r = make_rsrc(base, bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes);
#pragma unroll
    for (int q = 0; q < kInstr; ++q)
      sbp_raw_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (wave * kInstr + q) * 64), 16,
                              (int)off[q], 0, 0, 0);
  }
  // The stage that crosses k_ext (`kleft` k in range): chunks past it, and
  // rows past mn_ext, copy the 16-byte zero block instead.
  __device__ __forceinline__ void issue(const OperandView& op, int64_t i0, int64_t k0, int kleft, u32x4_t* dst,
                                        const char* zero) const {
    const char* base = reinterpret_cast<const char*>(op.ptr + i0 * op.ld + k0);
#pragma unroll
    for (int q = 0; q < kInstr; ++q) {
      const char* src = kk[q] < kleft ? base + off[q] : zero;
      __builtin_amdgcn_global_load_lds(src, dst + (wave * kInstr + q) * 64, 16, 0, 0);
    }
  }
};

// TILED: both operands in 256 x 32 storage tiles (ld = elements between tile
// rows; K a multiple of 32); else both row-major K-major (k_ext a multiple of
// 8).  Device-side live rows (LiveRows) may bound M or N only.
template <class Epi, bool TILED>
__global__ __launch_bounds__(kThreadsPP) void gemm_bf16_pp_kernel(OperandView A, OperandView B, int tiles_m,
                                                                  int tiles_n, int tm_base, int64_t K, int order,
                                                                  LiveRows live, Epi epi) {
  static_assert(Epi::kHookStages == 0 && Epi::kMinStages == 0, "no stage hooks in this loop");
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, FM = 4, FN = 2;
  static_assert(WM * WN * kWave == kThreadsPP && FM * 32 * WM == BM && FN * 32 * WN == BN, "8 waves of 128 x 64");
  constexpr int kStage = 2 * TileDma32::kSlots;  // slots per stage (both operands)
  constexpr int kPer = 2 * TileDma32::kInstr;    // vector-memory ops per wave and stage
  __shared__ u32x4_t lds[kRing32 * kStage + Epi::kLdsExtra / 16];
  static_assert(kRing32 * kStage * 16 >= 128 * 1024, "epilogues use 128 KiB of the freed ring");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);  // waves w and w + 4 share a SIMD
  const int wm = wave % WM, wn = wave / WM;
  const int lb_id = (order & 1) ? xcd_logical_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const bool m_fast = (order & 2) != 0;
  const int tn = m_fast ? lb_id / tiles_m : lb_id % tiles_n;
  const int tm = tm_base + (m_fast ? lb_id % tiles_m : lb_id / tiles_n);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  if (live.count != nullptr) {
    int64_t rc = (int64_t)__builtin_amdgcn_readfirstlane(*live.count) - live.base;
    rc = rc < 0 ? 0 : (rc > live.cap ? live.cap : rc);
    if (live.dim == kLiveM && m0 >= rc) return;
    if (live.dim == kLiveN && n0 >= rc) return;
  }
  const int nk = (int)((K + kBK32 - 1) / kBK32);

  using Dma = std::conditional_t<TILED, TileDma32, RowDma32>;
  Dma da, db;
  if constexpr (TILED) {
    da.plan(tid);
    db.plan(tid);
  } else {
    da.plan(A, m0, tid);
    db.plan(B, n0, tid);
  }
  const char* zero = reinterpret_cast<const char*>(&g_zero16);
  const uint32_t lds_base = lds_addr(lds);
  auto issue_stage = [&](int st) {
    u32x4_t* dst = lds + (st % kRing32) * kStage;
    const int64_t k0 = (int64_t)st * kBK32;
    if constexpr (TILED) {
      const i32x4_t ra = da.rsrc(A, m0, k0), rb = db.rsrc(B, n0, k0);
#pragma unroll
      for (int q = 0; q < TileDma32::kInstr; ++q) da.issue(ra, dst, q);
#pragma unroll
      for (int q = 0; q < TileDma32::kInstr; ++q) db.issue(rb, dst + TileDma32::kSlots, q);
    } else {
      const int64_t la = A.k_ext - k0, lbk = B.k_ext - k0;
      if (la >= kBK32)
        da.issue_rsrc(A, m0, k0, dst);
      else
        da.issue(A, m0, k0, (int)la, dst, zero);
      if (lbk >= kBK32)
        db.issue_rsrc(B, n0, k0, dst + TileDma32::kSlots);
      else
        db.issue(B, n0, k0, (int)lbk, dst + TileDma32::kSlots, zero);
    }
  };
  // fragments of both k16 sub-steps of stage st
  u32x4_t fa[2][FM], fb[2][FN];
  auto read_stage = [&](int st) {
    const uint32_t as = lds_base + 16u * (uint32_t)((st % kRing32) * kStage);
    const uint32_t bs = as + 16u * TileDma32::kSlots;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = 2 * ks + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[ks][i] = lds_read_b128(as + 16u * t32_slot(wm * (BM / WM) + 32 * i + (lane & 31), kc));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[ks][j] = lds_read_b128(bs + 16u * t32_slot(wn * (BN / WN) + 32 * j + (lane & 31), kc));
    }
  };
  // wait until at most n stages of this wave's loads are outstanding
  auto wait_stages = [&](int n) {
    if (n <= 0)
      wait_vmcnt<0>();
    else if (n == 1)
      wait_vmcnt<kPer>();
    else
      wait_vmcnt<2 * kPer>();
  };
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  const int pre = nk < kRing32 - 1 ? nk : kRing32 - 1;
  for (int st = 0; st < pre; ++st) issue_stage(st);
  wait_stages(pre - 1);
  __builtin_amdgcn_s_barrier();                 // stage 0 is whole
  if (grp == 1) __builtin_amdgcn_s_barrier();  // group 1 runs one phase behind
  for (int st = 0; st < nk; ++st) {
    __builtin_amdgcn_sched_barrier(0);
    // memory phase
    if (st + kRing32 - 1 < nk) issue_stage(st + kRing32 - 1);
    read_stage(st);
    wait_stages((st + kRing32 - 1 < nk ? st + kRing32 - 1 : nk - 1) - (st + 1));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(fa[ks][i]));
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[ks][j]));
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // compute phase
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[ks][i]),
                                                              __builtin_bit_cast(bf16x8_t, fb[ks][j]), acc[i][j], 0,
                                                              0, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();  // both groups have passed the same number of barriers
  __syncthreads();
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
  c.split = 0;
  c.wave = __builtin_amdgcn_readfirstlane(wave);
  c.nk = nk;
  c.lds = lds;
  c.extra = lds + kRing32 * kStage;
  epi.template run<FM, FN, WM, BN / WN, kThreadsPP>(acc, c);
}

// ---------------------------------------------------------------------------
// Epilogue of the chunk logits GEMM, computed as Z^T = W H_c^T (rows m = vocab
// v, columns n = token t of the chunk).  Per (token, vocab tile of BM) it
// writes the partial (max, sum exp(z - max)) of the fp32 logits, and stores
// the tile of Z[t][v] rounded to bf16.  The tile goes through LDS (free after
// the main loop: 256 x 256 bf16 = 128 KiB) so that global stores are 16-byte,
// row-contiguous; 16-byte chunks of an LDS row are XOR-swizzled by the row.
struct EpiLogits {
  uint16_t* Z;          // [rows][ldz] chunk logits (bf16 bits); NULL: partials only (forward-only passes)
  int64_t ldz;
  int64_t V;
  int64_t rows;         // tokens in this chunk
  float2* part;         // [rows][nvb] (max, sumexp) per vocab tile
  int64_t nvb;
  // Gradient mode (lse_in != NULL): the log-sum-exp of every token is known
  // already, so the tile is written as G = w (softmax - onehot(y)) in bf16
  // straight from the fp32 logits, with no partials; padding columns
  // (v >= V) and rows past `rows` hold 0.  Per-token arrays are indexed by the
  // token of each chunk row r: rowmap[tok0 + r] under masked-row compaction
  // (rows at or past the device-side live count, *live - live_base, are left
  // alone), else tok0 + r.
  const float* lse_in = nullptr;
  const float* w = nullptr;
  const int32_t* y = nullptr;
  int64_t tok0 = 0;
  const int32_t* rowmap = nullptr;
  const int32_t* live = nullptr;
  int64_t live_base = 0;

  static constexpr int kLdsExtra = 4096;  // (max, sum) exchange between the two M-waves
  static constexpr int kHookStages = 0;
  static constexpr int kMinStages = 0;
  static constexpr bool kGrouped = false;
  __device__ __forceinline__ bool streams(const TileCtx&) const { return false; }
  template <int FM, int FN>
  __device__ __forceinline__ void pre_loop(f32x16_t (&)[FM][FN], const TileCtx&) const {}
  template <int Q, int FM, int FN>
  __device__ __forceinline__ void stage_hook(f32x16_t (&)[FM][FN], const TileCtx&) const {}

  // 4 consecutive vocab rows vl .. vl+3 (vl a multiple of 4) of token tl into
  // the LDS image of the bf16 tile
  static __device__ __forceinline__ void stage4(uint32_t* zt, int tl, int vl, float a, float b, float c2, float d) {
    const int chunk = (vl >> 3) ^ (tl & 31);
    const u32x2_t pk = {pack_bf16x2(a, b), pack_bf16x2(c2, d)};
    *reinterpret_cast<u32x2_t*>(zt + tl * 128 + chunk * 4 + ((vl >> 2) & 1) * 2) = pk;
  }
  // coalesced rows of the staged tile into Z: thread -> (token row, 16-byte chunk)
  template <int NT>
  __device__ __forceinline__ void store_tile(const uint32_t* zt, const TileCtx& c) const {
    const int tid = c.wave * kWave + c.lane;
#pragma unroll 4
    for (int u = 0; u < 256 * 32 / NT; ++u) {
      const int idx = u * NT + tid;
      const int tl = idx >> 5, ch = idx & 31;
      const int64_t t = c.n_block + tl, v = c.m_block + 8 * ch;
      if (t < rows && v < ldz) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(zt + tl * 128 + ((ch ^ (tl & 31)) * 4));
        *reinterpret_cast<u32x4_t*>(Z + t * ldz + v) = val;
      }
    }
  }

  template <int FM, int FN, int WM, int WNCOLS, int NT = kThreads>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    constexpr int kCols = WNCOLS * (NT / kWave / WM);        // block tile width (tokens)
    constexpr int kRows = FM * 32 * WM;                      // block tile height (vocab)
    static_assert(kCols == 256 && kRows == 256, "LDS staging assumes a 256 x 256 tile");
    uint32_t* zt = reinterpret_cast<uint32_t*>(c.lds);        // [256 tokens][128 dwords]
    const int vl0 = (int)(c.m_wave - c.m_block);              // this wave's first vocab row in the tile
    if (lse_in != nullptr) {
      int64_t rc = rows;  // rows with a token
      if (live != nullptr) {
        rc = (int64_t)__builtin_amdgcn_readfirstlane(*live) - live_base;
        rc = rc < 0 ? 0 : (rc > rows ? rows : rc);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int tl = (int)(c.n_wave - c.n_block) + 32 * j + (c.lane & 31);
        const int64_t r = c.n_block + tl;
        const bool ok = r < rc;
        const int64_t t = !ok ? 0 : (rowmap != nullptr ? (int64_t)rowmap[tok0 + r] : tok0 + r);
        const float l2 = ok ? lse_in[t] * kLog2e : 0.f;
        const float wt = ok ? w[t] : 0.f;
        const int64_t yt = ok ? (int64_t)y[t] : -1;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int vl = vl0 + 32 * i + 8 * q + 4 * (c.lane >> 5);
            const int64_t v = c.m_block + vl;
            float g[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // softmax from the fp32 logit: exp(z - lse) <= 1
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][4 * q + e], kLog2e, -l2));
              const float x = wt * (p - (v + e == yt ? 1.f : 0.f));
              // rows of zero weight are 0 whatever their log-sum-exp entry holds
              g[e] = (ok && wt != 0.f && v + e < V) ? x : 0.f;
            }
            stage4(zt, tl, vl, g[0], g[1], g[2], g[3]);
          }
      }
      __syncthreads();
      store_tile<NT>(zt, c);
      return;
    }
    float2* red = reinterpret_cast<float2*>(c.extra);        // [WM][kCols]
    const bool full_v = c.m_block + kRows <= V;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int tl = (int)(c.n_wave - c.n_block) + 32 * j + (c.lane & 31);  // token in the tile
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (full_v || acc_row(c, i, r) < V) m = fmaxf(m, acc[i][j][r]);
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (full_v || acc_row(c, i, r) < V) s += exp_fast(acc[i][j][r] - m);
      }
      s += __shfl_xor(s, 32, kWave);
      if (c.lane < 32) red[c.wm * kCols + tl] = make_float2(m, s);
      if (Z == nullptr) continue;
      // bf16 tile into LDS: 4 consecutive vocab rows (8 bytes) per store
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          stage4(zt, tl, vl0 + 32 * i + 8 * q + 4 * (c.lane >> 5), acc[i][j][4 * q], acc[i][j][4 * q + 1],
                 acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    }
    __syncthreads();
    // (max, sum) of the two waves that share a token column -> partial of the tile
    if (c.wm == 0 && c.lane < 32) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t t = acc_col(c, j);
        if (t >= rows) continue;
        const int col = (int)(t - c.n_block);
        float m = red[col].x, s = red[col].y;
#pragma unroll
        for (int w2 = 1; w2 < WM; ++w2) lse_merge(m, s, red[w2 * kCols + col].x, red[w2 * kCols + col].y);
        part[t * nvb + c.tm] = make_float2(m, s);
      }
    }
    if (Z == nullptr) return;
    store_tile<NT>(zt, c);
  }
};

// Plain fp32 store of the tile (dH, or one split-K slab of it).
struct EpiStore {
  float* out;            // base of split 0
  int64_t ldo;
  int64_t split_stride;  // elements between split slabs
  int64_t m_ext, n_ext;

  static constexpr int kLdsExtra = 0;
  static constexpr int kHookStages = 0;
  static constexpr int kMinStages = 0;
  static constexpr bool kGrouped = false;
  __device__ __forceinline__ bool streams(const TileCtx&) const { return false; }
  template <int FM, int FN>
  __device__ __forceinline__ void pre_loop(f32x16_t (&)[FM][FN], const TileCtx&) const {}
  template <int Q, int FM, int FN>
  __device__ __forceinline__ void stage_hook(f32x16_t (&)[FM][FN], const TileCtx&) const {}

  template <int FM, int FN, int WM, int WNCOLS>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    float* o = out + (int64_t)c.split * split_stride;
    if (c.m_wave + 32 * FM <= m_ext && c.n_wave + 32 * FN <= n_ext) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[acc_row(c, i, r) * ldo + acc_col(c, j)] = acc[i][j][r];
      return;
    }
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

// dW tile update, dW = (accumulate ? dW : 0) + tile, with the product taken
// transposed: rows m = feature d, columns n = vocabulary row v, so that the
// 4 consecutive accumulator rows a lane holds (r = 4q .. 4q+3) are 4
// consecutive floats of one row of dW [V][D].  The tile is then stored
// straight from the accumulators with 16-byte stores (each store instruction
// writes 32 B of each of 32 rows; the 4 of one MFMA tile complete 128-byte
// lines), and old values are read the same way.
//
// MODE (a compile-time choice, so that no run-time branch merges the
// accumulators):
//  kAccStore   write only (the first chunk of a call without accumulation);
//  kAccLoad    the old tile is added after the loop (launches too short to
//              stream): its pieces are copied into the LDS ring the loop has
//              freed, 8 per wave, two rows of 4 MFMA tiles ahead of the row
//              being added and stored;
//  kAccStream  the old tile is streamed in during the main loop: each wave
//              owns FM x FN MFMA tiles of 32 x 32 fp32 ("pieces", 4 KiB);
//              piece q is copied from HBM into one of the wave's two LDS
//              buffers during k-stage q-1 and added into its accumulators at
//              the end of stage q, right after the stage's wait for loads.
//              A piece sits in LDS as [v][d] rows of 128 bytes whose 16-byte
//              chunks are XOR-swizzled by bits 1-3 of v, so that the 16 lanes
//              of each ds_read_b128 phase (rows v .. v+15, one chunk) hit 16
//              distinct 4-bank groups;
//  kAccStreamPad  as kAccStream, for loops that may be shorter than the 16
//              hooked stages (fewer rows, or a length known only on the
//              device): the loop runs at least 16 stages; stages past the
//              rows read zeros, so every piece of the old tile is still added.
// Stores are plain (write-back): a store instruction covers 32 bytes of each
// of 32 rows, and the L2 merges the 4 of an MFMA tile into whole lines
// (non-temporal stores wrote the partial lines through to HBM and were about
// 1.7x slower).
constexpr int kAccStore = 0, kAccLoad = 1, kAccStream = 2, kAccStreamPad = 3;
template <int MODE>
struct EpiAccum {
  float* out;       // dW [V][ldo]
  int64_t ldo;      // D
  int64_t d_ext;    // D (rows m of the product)
  int64_t v_ext;    // V (columns n of the product)
  static constexpr bool kStream = MODE == kAccStream || MODE == kAccStreamPad;
  static constexpr int kPieceBytes = 32 * 32 * 4;
  static constexpr int kPieceSlots = kPieceBytes / 16;
  static constexpr int kLdsExtra = kStream ? 4 * 2 * kPieceBytes : 0;  // 4 waves x 2 buffers
  static constexpr int kHookStages = kStream ? 16 : 0;                   // = FM * FN of the dW tile
  static constexpr int kMinStages = MODE == kAccStreamPad ? kHookStages : 0;
  static constexpr bool kGrouped = kStream;

  __device__ __forceinline__ bool streams(const TileCtx&) const { return kStream; }

  // All accesses go through a buffer resource over this wave's tile: it starts
  // at (d = m_wave, v = n_wave) and ends with row V-1 of dW, so rows v >= V
  // read zero and are not written.  Features d >= D of a row reach into the
  // next row: they only feed accumulator rows that are never stored, and
  // stores skip them.  A lane's offsets are one 32-bit VGPR; the rest is
  // scalar.
  __device__ __forceinline__ const float* wave_base(const TileCtx& c) const { return out + c.n_wave * ldo + c.m_wave; }
  __device__ __forceinline__ uint32_t wave_bytes(const TileCtx& c) const {
    const int64_t left = (v_ext - c.n_wave) * ldo - c.m_wave;  // floats from the tile origin to the end
    const int64_t bytes = left > 0 ? 4 * left : 0;
    return bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
  }
  // lane's byte offset to its accumulators r = 4q .. 4q+3 of MFMA tile (0, 0), q = 0:
  // column n = lane % 32, rows m = 4 (lane / 32) .. +3
  __device__ __forceinline__ int acc_voff(const TileCtx& c) const {
    return (int)(((c.lane & 31) * ldo + 4 * (c.lane >> 5)) * 4);
  }
  // uniform byte offset of MFMA tile (i, j), sub-block q
  __device__ __forceinline__ int acc_soff(int i, int j, int q) const { return (int)((32 * j * ldo + 32 * i + 8 * q) * 4); }
  __device__ __forceinline__ bool row_stored(const TileCtx& c, int i, int q) const {
    return c.m_wave + 32 * i + 8 * q + 4 * (c.lane >> 5) < d_ext;
  }

  // LDS slot of 16-byte chunk ch of row v of a piece
  static __device__ __forceinline__ int piece_slot(int v, int ch) { return v * 8 + (ch ^ ((v >> 1) & 7)); }

  // Issue the copy of piece q into buffer q % 2 of this wave (4 x 1 KiB DMA):
  // LDS slot part*64 + lane holds row v = 8 part + lane/8 of the piece; its
  // chunk follows piece_slot, whose swizzle depends on the parity of `part`.
  template <int FN>
  __device__ __forceinline__ void issue_piece(const TileCtx& c, int q) const {
    issue_piece_to<FN>(c, q, c.extra + (c.wave * 2 + (q & 1)) * kPieceSlots);
  }
  template <int FN>
  __device__ __forceinline__ void issue_piece_to(const TileCtx& c, int q, u32x4_t* buf) const {
    const int i = q / FN, j = q % FN;
    const i32x4_t r = make_rsrc(wave_base(c), wave_bytes(c));
    const int v0 = c.lane >> 3;
    const int ch0 = (c.lane & 7) ^ ((v0 >> 1) & 3), ch1 = ch0 ^ 4;  // even / odd part
    const int vo0 = (int)((v0 * ldo + 4 * ch0) * 4), vo1 = (int)((v0 * ldo + 4 * ch1) * 4);
#pragma unroll
    for (int part = 0; part < 4; ++part)
      // non-temporal: the old tile is read once and should not push the
      // operand tiles shared by the blocks of this vocabulary tile out of L2
      sbp_raw_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(buf + part * 64), 16,
                              (part & 1) ? vo1 : vo0, (int)(((32 * j + 8 * part) * ldo + 32 * i) * 4), 0,
                              kCachePolicyNT);
  }

  template <int FM, int FN>
  __device__ __forceinline__ void pre_loop(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    static_assert(!kStream || FM * FN == kHookStages, "one piece per hooked stage");
    if constexpr (kStream) issue_piece<FN>(c, 0);
  }

  // End of stage Q: piece Q is in LDS (the caller waited for it); add it and
  // start the copy of piece Q+1.
  template <int Q, int FM, int FN>
  __device__ __forceinline__ void stage_hook(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    if constexpr (!kStream) return;
    add_piece(acc, c, Q / FN, Q % FN, c.extra + (c.wave * 2 + (Q & 1)) * kPieceSlots);
    if constexpr (Q + 1 < FM * FN) issue_piece<FN>(c, Q + 1);
  }
  // acc[i][j] += the piece in `buf`
  template <int FM, int FN>
  __device__ __forceinline__ void add_piece(f32x16_t (&acc)[FM][FN], const TileCtx& c, int i, int j,
                                            const u32x4_t* buf) const {
    const int v = c.lane & 31;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = 2 * q + (c.lane >> 5);
      const f32x4_t o = __builtin_bit_cast(f32x4_t, buf[piece_slot(v, ch)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += o[e];
    }
  }

  template <int FM, int FN, int WM, int WNCOLS>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    static_assert(FM == 4 && FN == 4 && WM == 2 && WNCOLS == 128, "256 x 256 tile of 2 x 2 waves");
    const __amdgpu_buffer_rsrc_t r = make_brsrc(wave_base(c), wave_bytes(c));
    const int vo = acc_voff(c);
    const bool full = c.m_wave + 32 * FM <= d_ext;
    // store the row of MFMA tiles (i, 0..FN-1)
    auto store_row = [&](int i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (full || row_stored(c, i, q))
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                    acc[i][j][4 * q + 3]}),
                r, vo, acc_soff(i, j, q), 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (MODE == kAccLoad) {
      static_assert(FM == 4 && 4 * 8 * kPieceBytes <= 2 * kStages * 32768, "8 piece slots per wave in the ring");
      // 8 slots of this wave in the freed ring: row i of pieces uses slots 4 (i % 2) ..
      u32x4_t* slots = reinterpret_cast<u32x4_t*>(c.lds) + c.wave * 8 * kPieceSlots;
      auto issue_row = [&](int i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) issue_piece_to<FN>(c, i * FN + j, slots + (4 * (i & 1) + j) * kPieceSlots);
      };
      // store row i of MFMA tiles plus its old values, piece by piece
      auto add_store_row = [&](int i) {
        const int v = c.lane & 31;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const u32x4_t* buf = slots + (4 * (i & 1) + j) * kPieceSlots;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t o = __builtin_bit_cast(f32x4_t, buf[piece_slot(v, 2 * q + (c.lane >> 5))]);
            const f32x4_t x = {agpr_read(acc[i][j][4 * q]) + o[0], agpr_read(acc[i][j][4 * q + 1]) + o[1],
                               agpr_read(acc[i][j][4 * q + 2]) + o[2], agpr_read(acc[i][j][4 * q + 3]) + o[3]};
            if (full || row_stored(c, i, q))
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, vo, acc_soff(i, j, q), 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slots read before they are refilled
      };
      // Vector-memory ops in issue order: rows 0 and 1 of pieces (16 each),
      // then per row i its stores (16) and the pieces of row i + 2 (16); each
      // wait below lets the ops after the row it needs stay in flight.
      // Stores skipped by row_stored (rows past D; all or none of an
      // instruction's lanes, as D and the row offsets are multiples of 8) are
      // not issued and loosen the waits after them.  Rows grow with i, so a
      // row with a skipped store is followed only by rows that are not stored
      // at all: every row that is stored was waited for exactly.
      issue_row(0);
      issue_row(1);
      wait_vmcnt<16>();  // row 0 in LDS
      add_store_row(0);
      issue_row(2);
      wait_vmcnt<32>();  // row 1 (stores of row 0 and pieces of row 2 may be in flight)
      add_store_row(1);
      issue_row(3);
      wait_vmcnt<32>();  // row 2
      add_store_row(2);
      wait_vmcnt<16>();  // row 3
      add_store_row(3);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) store_row(i);
    }
  }
};

}  // namespace sbp
