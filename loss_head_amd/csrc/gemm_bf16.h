// bf16 MFMA GEMM core for gfx950 and the three head epilogues.
//
// C[m][n] = sum_k A[m][k] * B[n][k], bf16 operands, fp32 accumulation with
// v_mfma_f32_32x32x16_bf16.  A block of 512 threads (8 waves, two per SIMD)
// owns a 256 x 256 output tile; each wave owns a 128 x 64 piece of it (4 x 2
// MFMA tiles of 32 x 32), and the two waves of a SIMD run the main loop one
// phase apart (see gemm_bf16_pp_kernel).
//
// Operand tiles go from global memory straight into LDS with the LDS-DMA
// form of buffer_load_dwordx4 (lane l of a wave writes the 16 bytes it
// fetched to LDS base + 16*l), into a ring of four stages of k = 32, so no
// registers hold data in flight.  Which global chunk a lane fetches is chosen
// so that the LDS image is XOR-swizzled.  Reads past an operand's end come
// back as zero from the buffer resource's range check, or copy a 16-byte
// zero block.
//
//  K-major operand (element (i,k) at ptr[i*ld + k], or in 256 x 32 storage
//    tiles): LDS [i][k], 64-byte rows of four 16-byte chunks; an MFMA
//    fragment (8 consecutive k of one row) is one ds_read_b128.
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

// A non-temporal 16-byte buffer store between wait states.  The compiler does
// not look inside inline asm for hazards, so the block carries its own:
//  - before: a VALU write of an SGPR (v_readlane restoring a spilled SGPR,
//    v_readfirstlane) needs 5 wait states before a vector-memory instruction
//    reads that SGPR as resource or offset; without them the store can use
//    the SGPR's previous value and write to the wrong place;
//  - after: on gfx950 a VALU write to a data register of a store wider than 8
//    bytes, issued right behind the store, has reached memory in place of the
//    stored value for some lanes.
// `rsrc` and `soff` are wave-uniform.
__device__ __forceinline__ void store_b128_nt_guarded(u32x4_t v, i32x4_t rsrc, int voff, int soff) {
  asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %0, %1, %2, %3 offen nt\n\ts_nop 3" ::"v"(v), "v"(voff), "s"(rsrc),
               "s"(soff)
               : "memory");
}

// MN-major LDS: chunk swizzle of a 512-byte k-row.
__device__ __forceinline__ int mn_swz(int k) { return 4 * ((k & 3) | (((k >> 3) & 1) << 2)); }

// LDS fragment reads are issued as inline asm: the compiler would otherwise
// treat the transpose read as possibly overlapping the in-flight LDS DMA and
// drain the whole ring before it.  Completion is then awaited explicitly
// (s_waitcnt lgkmcnt, with the fragment registers tied to it).
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
// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)(p));
}

// The reads of one MFMA operand fragment of an MN-major operand: 8
// consecutive k (k16 sub-step `ks`, lane half lane/32) of tile column
// row0 + lane%32.  `st` is the LDS byte address of this operand's part of the
// stage ([k][R] bf16, chunks swizzled by mn_swz).
template <int R>
__device__ __forceinline__ u32x4_t mn_frag(uint32_t st, int row0, int ks, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int i = row0 + 16 * (g & 1) + 4 * (j & 3);
  const int kb = 16 * ks + 8 * (g >> 1) + (j >> 2);
  const uint32_t a0 = st + 16u * (kb * (R / 8) + ((i >> 3) ^ mn_swz(kb))) + (i & 7) * 2;
  const uint32_t a1 = st + 16u * ((kb + 4) * (R / 8) + ((i >> 3) ^ mn_swz(kb + 4))) + (i & 7) * 2;
  const u32x2_t lo = lds_read_tr_b64(a0), hi = lds_read_tr_b64(a1);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
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
  void* lds;                // free LDS (128 KiB) once the main loop is done
  u32x4_t* extra;           // the epilogue's own LDS (Epi::kLdsExtra bytes)
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

// Operand loaders of the ping-pong loop.  Each stages its 256 x 32 part of a
// k = 32 stage (1024 16-byte slots, 16 KiB) into LDS; all share
//   plan(op, i0, tid)                 once per block,
//   stage(op, i0, k0, dst, zero)      per stage (k0 relative to op.ptr),
// and the fragment reads of pp_frag below.
constexpr int kPPTiled = 0;  // K-major, in 256 x 32 storage tiles
constexpr int kPPRowK = 1;   // K-major, row-major storage: element (i,k) at ptr[i*ld + k]
constexpr int kPPRowMN = 2;  // MN-major: element (i,k) at ptr[k*ld + i]
constexpr int kSlots32 = 256 * kBK32 / 8;        // 16-byte slots per operand and stage
constexpr int kInstr32 = kSlots32 / kThreadsPP;  // DMA instructions per wave, operand and stage

// Tiled operand: the stage is one contiguous tile.
struct TileDma32 {
  uint32_t off[kInstr32];  // byte offset of this lane's chunk inside the tile
  int wave;
  __device__ __forceinline__ void plan(const OperandView&, int64_t, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < kInstr32; ++q) {
      const int sl = (wave * kInstr32 + q) * 64 + lane;
      const int i = sl >> 2, kc = (sl & 3) ^ ((i >> 2) & 3);
      off[q] = (uint32_t)((i * kBK32 + kc * 8) * 2);
    }
  }
  // tile of stage origin (i0, k0): i0 a multiple of 256, k0 of 32
  __device__ __forceinline__ void stage(const OperandView& op, int64_t i0, int64_t k0, u32x4_t* dst,
                                        const char*) const {
    const i32x4_t r = make_rsrc(op.ptr + (i0 >> 8) * op.ld + (k0 >> 5) * kTile32, 2 * kTile32);
#pragma unroll
    for (int q = 0; q < kInstr32; ++q)
      sbp_raw_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (wave * kInstr32 + q) * 64), 16,
                              (int)off[q], 0, 0, 0);
  }
};

// A K-major operand stored row-major, staged into the same [256][32] LDS
// image as a storage tile: lane chunk (i, kc) comes from 16 bytes of row i,
// so a stage is 256 pieces of 64 bytes.
struct RowDma32 {
  uint32_t off[kInstr32];  // byte offset of this lane's chunk from the stage origin (i0, k0)
  int kk[kInstr32];        // k of the chunk inside the stage; huge if its row is past mn_ext
  int wave;
  __device__ __forceinline__ void plan(const OperandView& op, int64_t i0, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < kInstr32; ++q) {
      const int sl = (wave * kInstr32 + q) * 64 + lane;
      const int i = sl >> 2, kc = (sl & 3) ^ ((i >> 2) & 3);
      off[q] = (uint32_t)((i * op.ld + kc * 8) * 2);
      kk[q] = (i0 + i < op.mn_ext) ? kc * 8 : (1 << 30);
    }
  }
  // A stage wholly below k_ext goes through a resource that ends with the
  // operand's last valid row (rows past it read zero); the stage that
  // crosses k_ext copies the 16-byte zero block for chunks past it (and for
  // rows past mn_ext) instead.
  __device__ __forceinline__ void stage(const OperandView& op, int64_t i0, int64_t k0, u32x4_t* dst,
                                        const char* zero) const {
    const uint16_t* base = op.ptr + i0 * op.ld + k0;
    const int64_t kleft = op.k_ext - k0;
    if (kleft >= kBK32) {
      const int64_t left = op.mn_ext * op.ld - (base - op.ptr);
      const int64_t bytes = left > 0 ? 2 * left : 0;
      const i32x4_t r = make_rsrc(base, bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes);
#pragma unroll
      for (int q = 0; q < kInstr32; ++q)
        sbp_raw_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (wave * kInstr32 + q) * 64), 16,
                                (int)off[q], 0, 0, 0);
    } else {
      const char* b = reinterpret_cast<const char*>(base);
#pragma unroll
      for (int q = 0; q < kInstr32; ++q) {
        const char* src = kk[q] < kleft ? b + off[q] : zero;
        __builtin_amdgcn_global_load_lds(src, dst + (wave * kInstr32 + q) * 64, 16, 0, 0);
      }
    }
  }
};

// An MN-major operand, staged as [k][i] 512-byte rows with the chunk swizzle
// mn_swz(k) (the layout mn_frag<256> reads with transpose reads):
// a stage is 32 pieces of 512 bytes.  The resource ends with storage row
// k_ext - 1, so k-rows past it read zero; columns past mn_ext only feed
// output rows or columns that are never stored.
struct MnDma32 {
  uint32_t off[kInstr32];
  int wave;
  __device__ __forceinline__ void plan(const OperandView& op, int64_t, int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int q = 0; q < kInstr32; ++q) {
      const int sl = (wave * kInstr32 + q) * 64 + lane;
      const int k = sl >> 5, i = ((sl & 31) ^ mn_swz(k)) * 8;
      off[q] = (uint32_t)((k * op.ld + i) * 2);
    }
  }
  __device__ __forceinline__ void stage(const OperandView& op, int64_t i0, int64_t k0, u32x4_t* dst,
                                        const char*) const {
    const uint16_t* base = op.ptr + k0 * op.ld + i0;
    const int64_t left = op.k_ext * op.ld - (base - op.ptr);
    const int64_t bytes = left > 0 ? 2 * left : 0;
    const i32x4_t r = make_rsrc(base, bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes);
#pragma unroll
    for (int q = 0; q < kInstr32; ++q)
      sbp_raw_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (wave * kInstr32 + q) * 64), 16,
                              (int)off[q], 0, 0, 0);
  }
};

template <int L>
using PPDma = std::conditional_t<L == kPPTiled, TileDma32, std::conditional_t<L == kPPRowK, RowDma32, MnDma32>>;

// One MFMA operand fragment (8 consecutive k of k16 sub-step ks, tile row
// row0 + lane % 32) from the operand's part of a k = 32 stage at LDS byte
// address st.
template <int L>
__device__ __forceinline__ u32x4_t pp_frag(uint32_t st, int row0, int ks, int lane) {
  if constexpr (L == kPPRowMN)
    return mn_frag<256>(st, row0, ks, lane);
  else
    return lds_read_b128(st + 16u * t32_slot(row0 + (lane & 31), 2 * ks + (lane >> 5)));
}

// LA, LB: the loaders of A and B (kPPTiled: K a multiple of 32; kPPRowK:
// k_ext a multiple of 8).  Split-K: the blocks of split s work on k in
// [s * k_split, +k_split) of their tiles (k_split a multiple of 32).
// Device-side live rows (LiveRows) may bound any dimension; along K, rows
// past the live ones read zero (the RowMN loader's resource ends there).
constexpr int kStagePP = 2 * kSlots32;  // 16-byte slots per stage (both operands)

// LDS of the ping-pong kernels: the ring, then the epilogue's own part.
template <class Epi>
constexpr int pp_lds_slots() {
  return kRing32 * kStagePP + Epi::kLdsExtra / 16;
}

// Place of logical tile lb_id: split-K slab, tile row and column.
struct PPGeom {
  int split, tm, tn;
  int64_t m0, n0;
};
__device__ __forceinline__ PPGeom pp_geom(int lb_id, int tiles_m, int tiles_n, int tm_base, int order) {
  PPGeom g;
  const int per_split = tiles_m * tiles_n;
  g.split = lb_id / per_split;
  const int t = lb_id - g.split * per_split;
  const bool m_fast = (order & 2) != 0;
  g.tn = m_fast ? t / tiles_m : t % tiles_n;
  g.tm = tm_base + (m_fast ? t % tiles_m : t / tiles_n);
  g.m0 = (int64_t)g.tm * 256;
  g.n0 = (int64_t)g.tn * 256;
  return g;
}

// The first k-stage index and the number of stages of a tile's main loop.
template <class Epi>
__device__ __forceinline__ int pp_stages(int split, int64_t k_split, int64_t K, int64_t* kb_out) {
  const int64_t kb = (int64_t)split * k_split;
  const int64_t ke = kb + k_split < K ? kb + k_split : K;
  int nk = ke > kb ? (int)((ke - kb + kBK32 - 1) / kBK32) : 0;
  // an epilogue that streams pieces in during the loop needs segments of at
  // least 2 stages (stages past ke read zeros)
  if constexpr (Epi::kPieces > 0) {
    if (nk < 2 * Epi::kPieces) nk = 2 * Epi::kPieces;
  }
  *kb_out = kb;
  return nk;
}

// What an epilogue needs to know of this wave's place in tile g.
__device__ __forceinline__ TileCtx pp_ctx(const PPGeom& g, int nk, u32x4_t* lds, int extra_slot) {
  constexpr int WM = 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  TileCtx c;
  c.m_block = g.m0;
  c.n_block = g.n0;
  c.m_wave = g.m0 + wm * 128;
  c.n_wave = g.n0 + wn * 64;
  c.lane = lane;
  c.wm = wm;
  c.wn = wn;
  c.tm = g.tm;
  c.tn = g.tn;
  c.split = g.split;
  c.wave = __builtin_amdgcn_readfirstlane(wave);
  c.nk = nk;
  c.lds = lds;
  c.extra = lds + extra_slot;
  return c;
}

// Issue a tile's prologue: the epilogue's first streamed piece, then the DMA
// of stages 0 .. pre-1 into ring slots 0 .. pre-1.  Used by the persistent
// pipelined kernel to start the next tile while the current one stores.
template <class Epi, int LA, int LB>
__device__ __forceinline__ void pp_issue_prologue(const OperandView& A, const OperandView& B, const PPGeom& g,
                                                  int64_t kb, int pre, const Epi& epi, const TileCtx& c,
                                                  u32x4_t* lds) {
  const int tid = threadIdx.x;
  PPDma<LA> da;
  PPDma<LB> db;
  da.plan(A, g.m0, tid);
  db.plan(B, g.n0, tid);
  const char* zero = reinterpret_cast<const char*>(&g_zero16);
  if constexpr (Epi::kPieces > 0) epi.first_piece(c);
  for (int st = 0; st < pre; ++st) {
    u32x4_t* dst = lds + st * kStagePP;
    const int64_t k0 = kb + (int64_t)st * kBK32;
    da.stage(A, g.m0, k0, dst, zero);
    db.stage(B, g.n0, k0, dst + kSlots32, zero);
  }
}

struct NoTransition {
  __device__ __forceinline__ void operator()() const {}
};

// One 256 x 256 output tile (logical tile lb_id) of the ping-pong GEMM, from
// the prologue to the epilogue's last store.  `lds` is the kernel's LDS
// (pp_lds_slots<Epi>() slots).
// Pipelining across tiles (persistent kernel):
//  - kPreissued: the tile's prologue (piece 0, stages 0-2) was issued already,
//    by the previous tile's transition;
//  - kPending: that many vector-memory stores of the previous tile were issued
//    after those stages and may still be in flight; the waits of the
//    prologue and of stages 0 and 1 allow for them (stage 2's wait, for stage
//    3's DMA, which is younger than the stores, drains them);
//  - `transition` runs once every wave has finished reading the ring, before
//    the epilogue: it issues the next tile's prologue into ring slots 0-2.
template <class Epi, int LA, int LB, bool kPreissued = false, int kPending = 0, class Transition = NoTransition>
__device__ __forceinline__ void pp_tile(OperandView A, OperandView B, int lb_id, int tiles_m, int tiles_n,
                                        int tm_base, int64_t k_split, int64_t K, int order, const LiveRows& live,
                                        const Epi& epi, u32x4_t* lds, const Transition& transition = {}) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, FM = 4, FN = 2;
  static_assert(WM * WN * kWave == kThreadsPP && FM * 32 * WM == BM && FN * 32 * WN == BN, "8 waves of 128 x 64");
  constexpr int kStage = kStagePP;
  constexpr int kPer = 2 * kInstr32;    // vector-memory ops per wave and stage
  static_assert(kRing32 * kStage * 16 >= 128 * 1024, "epilogues use 128 KiB of the freed ring");
  static_assert(2 * kPer + kPending < 64, "vmcnt holds 6 bits");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);  // waves w and w + 4 share a SIMD
  const int wm = wave % WM, wn = wave / WM;
  const PPGeom geom = pp_geom(lb_id, tiles_m, tiles_n, tm_base, order);
  const int split = geom.split;
  const int64_t m0 = geom.m0, n0 = geom.n0;
  if (live.count != nullptr) {
    int64_t rc = (int64_t)__builtin_amdgcn_readfirstlane(*live.count) - live.base;
    rc = rc < 0 ? 0 : (rc > live.cap ? live.cap : rc);
    if (live.dim == kLiveM && m0 >= rc) return;
    if (live.dim == kLiveN && n0 >= rc) return;
    // (only the MN-major loaders bound their reads by k_ext alone, and a
    // tiled operand is read in whole zero-padded tiles: the launchers pass
    // kLiveK with an MN-major B only, and a tiled A must be zero past the
    // live rows)
    if constexpr (LB == kPPRowMN && (LA == kPPRowMN || LA == kPPTiled)) {
      if (live.dim == kLiveK) {
        if (rc == 0 && live.skip_empty) return;
        if (A.k_ext > rc) A.k_ext = rc;
        if (B.k_ext > rc) B.k_ext = rc;
        if (K > rc) K = rc;
      }
    }
  }
  int64_t kb;
  const int nk = pp_stages<Epi>(split, k_split, K, &kb);

  PPDma<LA> da;
  PPDma<LB> db;
  da.plan(A, m0, tid);
  db.plan(B, n0, tid);
  const char* zero = reinterpret_cast<const char*>(&g_zero16);
  const uint32_t lds_base = lds_addr(lds);
  auto issue_stage = [&](int st) {
    u32x4_t* dst = lds + (st % kRing32) * kStage;
    const int64_t k0 = kb + (int64_t)st * kBK32;
    da.stage(A, m0, k0, dst, zero);
    db.stage(B, n0, k0, dst + kSlots32, zero);
  };
  // fragments of both k16 sub-steps of stage st
  u32x4_t fa[2][FM], fb[2][FN];
  auto read_stage = [&](int st) {
    const uint32_t as = lds_base + 16u * (uint32_t)((st % kRing32) * kStage);
    const uint32_t bs = as + 16u * kSlots32;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[ks][i] = pp_frag<LA>(as, wm * (BM / WM) + 32 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[ks][j] = pp_frag<LB>(bs, wn * (BN / WN) + 32 * j, ks, lane);
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

  const TileCtx c = pp_ctx(geom, nk, lds, kRing32 * kStage);

  const int pre = nk < kRing32 - 1 ? nk : kRing32 - 1;
  if constexpr (kPreissued) {
    // piece 0 and stages 0-2 came from the previous tile's transition, with
    // kPending stores behind them
    wait_vmcnt<2 * kPer + kPending>();
  } else {
    if constexpr (Epi::kPieces > 0) epi.first_piece(c);
    for (int st = 0; st < pre; ++st) issue_stage(st);
    wait_stages(pre - 1);
  }
  __builtin_amdgcn_s_barrier();                 // stage 0 is whole
  if (grp == 1) __builtin_amdgcn_s_barrier();  // group 1 runs one phase behind
  // One stage; `hook` runs at the end of the memory phase, after its waits.
  auto stage = [&](int st, auto hook) {
    __builtin_amdgcn_sched_barrier(0);
    // memory phase
    if (st + kRing32 - 1 < nk) issue_stage(st + kRing32 - 1);
    read_stage(st);
    if (kPending > 0 && st < 2)
      wait_vmcnt<2 * kPer + kPending>();  // (the stores sit between stages 2 and 3)
    else
      wait_stages((st + kRing32 - 1 < nk ? st + kRing32 - 1 : nk - 1) - (st + 1));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(fa[ks][i]));
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[ks][j]));
    }
    hook();
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
  };
  if constexpr (Epi::kPieces > 0) {
    // Segment P of the loop ends with the hook for piece P (a compile-time
    // index into the accumulators).  Vector-memory operations of a wave
    // complete in order, and the wait in the memory phase of stage st leaves
    // only the DMA of stages st+2 and st+3 in flight (issued in the memory
    // phases of stages st-1 and st).  A piece issued in the memory phase of
    // stage h <= st-2 is older than both, so segments of 2 or more stages
    // find their piece whole.  The pieces sit in this wave's own LDS buffer:
    // no barrier.
    constexpr int kP = Epi::kPieces;
    [&]<int... Ps>(std::integer_sequence<int, Ps...>) {
      (
          [&] {
            const int b0 = Ps * nk / kP, b1 = (Ps + 1) * nk / kP;
            for (int st = b0; st < b1 - 1; ++st) stage(st, [] {});
            stage(b1 - 1, [&] { epi.template piece<Ps, FM, FN>(acc, c); });
          }(),
          ...);
    }(std::make_integer_sequence<int, kP>{});
  } else {
    for (int st = 0; st < nk; ++st) stage(st, [] {});
  }
  if (grp == 0) __builtin_amdgcn_s_barrier();  // both groups have passed the same number of barriers
  __syncthreads();
  transition();
  epi.template run<FM, FN, WM, BN / WN, kThreadsPP>(acc, c);
}

template <class Epi, int LA, int LB>
__global__ __launch_bounds__(kThreadsPP) void gemm_bf16_pp_kernel(OperandView A, OperandView B, int tiles_m,
                                                                  int tiles_n, int tm_base, int64_t k_split,
                                                                  int64_t K, int order, LiveRows live, Epi epi) {
  __shared__ u32x4_t lds[pp_lds_slots<Epi>()];
  const int lb_id = (order & 1) ? xcd_logical_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  pp_tile<Epi, LA, LB>(A, B, lb_id, tiles_m, tiles_n, tm_base, k_split, K, order, live, epi, lds);
}

// Persistent form: gridDim.x blocks (a multiple of 8, one per CU) walk the
// `ntiles` logical tiles, block b taking virtual block ids b, b + grid, ...
// Virtual id v runs on the XCD of block b (v % 8 == b % 8), so the XCD
// mapping of the one-tile-per-block launch is kept.
//
// Without kPipelined the block's LDS is free again only after every wave has
// finished a tile's epilogue, hence the barrier between tiles.  With
// kPipelined (an epilogue with kStage3Stores, no device-side live rows, at
// least 5 k-stages per tile) the next tile's prologue is issued as soon as
// every wave has read the ring for the last time, into ring slots 0-2, and the
// epilogue stages its stores through ring slot 3 meanwhile: the next tile's
// first stages load while this one's stores drain.
template <class Epi, int LA, int LB, bool kPipelined>
__global__ __launch_bounds__(kThreadsPP) void gemm_bf16_pp_persistent_kernel(OperandView A, OperandView B,
                                                                             int tiles_m, int tiles_n, int tm_base,
                                                                             int64_t k_split, int64_t K, int order,
                                                                             int ntiles, LiveRows live, Epi epi) {
  __shared__ u32x4_t lds[pp_lds_slots<Epi>()];
  auto logical = [&](int v) { return (order & 1) ? xcd_logical_block(v, ntiles) : v; };
  if constexpr (!kPipelined) {
    for (int v = blockIdx.x; v < ntiles; v += gridDim.x) {
      pp_tile<Epi, LA, LB>(A, B, logical(v), tiles_m, tiles_n, tm_base, k_split, K, order, live, epi, lds);
      __syncthreads();
    }
  } else {
    static_assert(Epi::kStage3Stores > 0, "pipelined tiles need an epilogue that stages through ring slot 3");
    // issues the prologue of virtual tile vn, if there is one
    auto transition_to = [&](int vn) {
      return [&, vn] {
        if (vn >= ntiles) return;
        const PPGeom g = pp_geom(logical(vn), tiles_m, tiles_n, tm_base, order);
        int64_t kb;
        const int nk = pp_stages<Epi>(g.split, k_split, K, &kb);
        pp_issue_prologue<Epi, LA, LB>(A, B, g, kb, kRing32 - 1, epi, pp_ctx(g, nk, lds, kRing32 * kStagePP), lds);
      };
    };
    int v = blockIdx.x;
    if (v >= ntiles) return;
    pp_tile<Epi, LA, LB>(A, B, logical(v), tiles_m, tiles_n, tm_base, k_split, K, order, live, epi, lds,
                         transition_to(v + (int)gridDim.x));
    for (v += gridDim.x; v < ntiles; v += gridDim.x)
      pp_tile<Epi, LA, LB, true, Epi::kStage3Stores>(A, B, logical(v), tiles_m, tiles_n, tm_base, k_split, K, order,
                                                      live, epi, lds, transition_to(v + (int)gridDim.x));
  }
}

// ---------------------------------------------------------------------------
// Epilogue of the chunk logits GEMM, computed as Z^T = W H_c^T (rows m = vocab
// v, columns n = token t of the chunk).  Per (token, vocab tile of BM) it
// writes the log-sum-exp partial (m, r) of the fp32 logits (m the tile's
// maximum, r the sum of exp(z - m) without the maximum's own term; see
// lse_merge), and stores the tile as bf16(Z[t][v] - m): the stored values are
// shifted by their own tile's maximum before rounding, so the rounding error
// of a logit near the top of its row is relative to its distance from m, not
// to the logit's size (a row pass later forms exp((z - m) + (m - lse))).  The
// tile goes through LDS (free after
// the main loop: 256 x 256 bf16 = 128 KiB) so that global stores are 16-byte,
// row-contiguous; 16-byte chunks of an LDS row are XOR-swizzled by the row.
// kGrad selects the gradient mode below at compile time, so that each kernel
// carries the registers of one mode only.
template <bool kGrad>
struct EpiLogitsT {
  uint16_t* Z;          // [rows][ldz] chunk logits (bf16 bits); NULL: partials only (forward-only passes)
  int64_t ldz;
  int64_t V;
  int64_t rows;         // tokens in this chunk
  float2* part;         // [rows][nvb] (max, sumexp) per vocab tile
  int64_t nvb;
  // Gradient mode (kGrad; lse_in, w, y non-NULL): the log-sum-exp of every
  // token is known already, so the tile is written as G = w (softmax - onehot(y)) in bf16
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
  static constexpr int kPieces = 0;       // no pieces streamed in during the loop
  static constexpr int kStage3Stores = 0;

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

  template <int FM, int FN, int WM, int WNCOLS, int NT>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    constexpr int kCols = WNCOLS * (NT / kWave / WM);        // block tile width (tokens)
    constexpr int kRows = FM * 32 * WM;                      // block tile height (vocab)
    static_assert(kCols == 256 && kRows == 256, "LDS staging assumes a 256 x 256 tile");
    uint32_t* zt = reinterpret_cast<uint32_t*>(c.lds);        // [256 tokens][128 dwords]
    const int vl0 = (int)(c.m_wave - c.m_block);              // this wave's first vocab row in the tile
    if constexpr (kGrad) {
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
        // vocabulary indices fit 32 bits (V <= INT32_MAX); relative to the tile
        // they keep fewer registers live than 64-bit ones
        const int64_t yd = ok ? (int64_t)y[t] - c.m_block : -1;
        const int yl = (yd >= 0 && yd < kRows) ? (int)yd : -1;  // label's row in the tile, -1 if outside
        const int vlim = (int)(V - c.m_block);             // rows of the tile inside the vocabulary
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int vl = vl0 + 32 * i + 8 * q + 4 * (c.lane >> 5);
            float g[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // softmax from the fp32 logit: exp(z - lse) <= 1
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i][j][4 * q + e], kLog2e, -l2));
              const float x = wt * (p - (vl + e == yl ? 1.f : 0.f));
              // rows of zero weight are 0 whatever their log-sum-exp entry holds
              g[e] = (ok && wt != 0.f && vl + e < vlim) ? x : 0.f;
            }
            stage4(zt, tl, vl, g[0], g[1], g[2], g[3]);
          }
      }
      __syncthreads();
      store_tile<NT>(zt, c);
    } else {
      run_partials<FM, FN, WM, WNCOLS, NT>(acc, c, zt, vl0);
    }
  }

  // (max, sum) partials of the tile and, unless Z is NULL, its bf16 (z - m)
  template <int FM, int FN, int WM, int WNCOLS, int NT>
  __device__ __forceinline__ void run_partials(f32x16_t (&acc)[FM][FN], const TileCtx& c, uint32_t* zt,
                                               int vl0) const {
    constexpr int kCols = WNCOLS * (NT / kWave / WM);        // block tile width (tokens)
    constexpr int kRows = FM * 32 * WM;                      // block tile height (vocab)
    float2* red = reinterpret_cast<float2*>(c.extra);        // [WM][kCols]
    const bool full_v = c.m_block + kRows <= V;
    // (max, sum exp(z - max)) over this wave's rows of token column j; rows
    // at or past V (in the last vocabulary tile only) are left out
    auto partial = [&](int j, auto full) {
      constexpr bool kFull = decltype(full)::value;
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kFull || acc_row(c, i, r) < V) m = fmaxf(m, acc[i][j][r]);
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      // (m, r) partial (see lse_merge): elements equal to the maximum are
      // counted, not summed, so that the maximum's own 1 stays out of r
      float s = 0.f;
      int ties = 0;
      if (m != -INFINITY) {
        const float ml = m * kLog2e;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kFull || acc_row(c, i, r) < V) {
              const float x = acc[i][j][r];
              const bool top = x == m;
              s += top ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -ml));
              ties += top ? 1 : 0;
            }
      }
      s += __shfl_xor(s, 32, kWave);
      ties += __shfl_xor(ties, 32, kWave);
      return make_float2(m, s + (float)(ties - 1));
    };
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int tl = (int)(c.n_wave - c.n_block) + 32 * j + (c.lane & 31);  // token in the tile
      const float2 ms = full_v ? partial(j, std::true_type{}) : partial(j, std::false_type{});
      if (c.lane < 32) red[c.wm * kCols + tl] = ms;
    }
    __syncthreads();
    if (Z != nullptr) {
      // bf16(z - m) into LDS, m the maximum of the token's column over the
      // whole tile (both M-waves): 4 consecutive vocab rows (8 bytes) per store
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int tl = (int)(c.n_wave - c.n_block) + 32 * j + (c.lane & 31);
        float m = red[tl].x;
#pragma unroll
        for (int w2 = 1; w2 < WM; ++w2) m = fmaxf(m, red[w2 * kCols + tl].x);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            stage4(zt, tl, vl0 + 32 * i + 8 * q + 4 * (c.lane >> 5), acc[i][j][4 * q] - m,
                   acc[i][j][4 * q + 1] - m, acc[i][j][4 * q + 2] - m, acc[i][j][4 * q + 3] - m);
      }
    }
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
    __syncthreads();
    store_tile<NT>(zt, c);
  }
};
using EpiLogits = EpiLogitsT<false>;
using EpiLogitsGrad = EpiLogitsT<true>;

// Plain fp32 store of the tile (dH, or one split-K slab of it).
struct EpiStore {
  float* out;            // base of split 0
  int64_t ldo;
  int64_t split_stride;  // elements between split slabs
  int64_t m_ext, n_ext;

  static constexpr int kLdsExtra = 0;
  static constexpr int kPieces = 0;
  static constexpr int kStage3Stores = 0;

  template <int FM, int FN, int WM, int WNCOLS, int NT>
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
// consecutive floats of one row of dW [V][D].  Stores go through LDS so that
// each store instruction writes 8 whole 128-byte lines (run below); old values
// come in as whole-line pieces (kAccStream below).
//
// MODE (a compile-time choice, so that no run-time branch merges the
// accumulators):
//  kAccStore   write only (the first chunk of a call without accumulation);
//  kAccStream  the old tile is streamed in during the main loop: each wave
//              owns 4 x 2 MFMA tiles of 32 x 32 fp32 ("pieces", 4 KiB); the
//              loop runs in 8 segments, and the end of segment P adds piece P
//              from the wave's LDS buffer and copies piece P+1 into it (whole
//              128-byte lines, LDS DMA), so the old tile's 256 KiB per block
//              are read over the whole loop rather than in a burst.  A piece
//              sits in LDS as [v][d] rows of 128 bytes whose 16-byte chunks are
//              XOR-swizzled by bits 1-3 of v, so that the 16 lanes of each
//              ds_read_b128 phase (rows v .. v+15, one chunk) hit 16 distinct
//              4-bank groups.
// Stores are non-temporal and write whole lines: dW is read again only by the
// next chunk's launch, and kept out of the caches it leaves them to the
// operands (the next logits GEMM's reads of W among them).
//
// kStage3: the persistent pipelined form.  The tile passes through this
// wave's 4 KiB of ring slot 3, one 32 x 32 tile at a time, so that ring slots
// 0-2 can take the next tile's first stages meanwhile; every wave then issues
// exactly kStage3Stores stores (D a multiple of 256: no store is skipped; rows
// v >= V fall outside the buffer resource and are dropped), the count the
// next tile's waits allow for.
constexpr int kAccStore = 0, kAccStream = 1;
template <int MODE, bool kStage3 = false>
struct EpiAccum {
  float* out;       // dW [V][ldo]
  int64_t ldo;      // D
  int64_t d_ext;    // D (rows m of the product)
  int64_t v_ext;    // V (columns n of the product)
  static_assert(MODE == kAccStore || MODE == kAccStream, "update mode");
  static constexpr int kPieceBytes = 32 * 32 * 4;
  static constexpr int kPieceSlots = kPieceBytes / 16;
  static constexpr int kWaves = kThreadsPP / kWave;
  static constexpr int kPieces = MODE == kAccStream ? 8 : 0;  // 4 x 2 MFMA tiles per wave
  static constexpr int kLdsExtra = MODE == kAccStream ? kWaves * kPieceBytes : 0;  // one buffer per wave
  static constexpr int kStage3Stores = kStage3 ? 4 * 2 * 4 : 0;                    // 8 tiles x 4 stores

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
  // LDS slot of 16-byte chunk ch of row v of a piece
  static __device__ __forceinline__ int piece_slot(int v, int ch) { return v * 8 + (ch ^ ((v >> 1) & 7)); }

  // Issue the copy of piece q into `buf` (4 x 1 KiB DMA): LDS slot
  // part*64 + lane holds row v = 8 part + lane/8 of the piece; its chunk
  // follows piece_slot, whose swizzle depends on the parity of `part`.
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

  // kAccStream: piece 0 is copied before the loop; the hook of piece P adds
  // it and copies piece P+1 into the same buffer.
  __device__ __forceinline__ void first_piece(const TileCtx& c) const {
    issue_piece_to<2>(c, 0, c.extra + c.wave * kPieceSlots);
  }
  template <int P, int FM, int FN>
  __device__ __forceinline__ void piece(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    static_assert(FM * FN == kPieces && FN == 2, "one piece per MFMA tile of the wave");
    u32x4_t* buf = c.extra + c.wave * kPieceSlots;
    const uint32_t base = lds_addr(buf);
    const int v = c.lane & 31;
    u32x4_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = lds_read_b128(base + 16u * piece_slot(v, 2 * q + (c.lane >> 5)));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the buffer is refilled
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      asm volatile("" : "+v"(o[q]));
      const f32x4_t f = __builtin_bit_cast(f32x4_t, o[q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[P / FN][P % FN][4 * q + e] += f[e];
    }
    if constexpr (P + 1 < kPieces) issue_piece_to<FN>(c, P + 1, buf);
  }

  // LDS slot of 16-byte chunk ch of row v of a staged 32 x 32 tile: chunks
  // XOR-swizzled by bits 0-2 of v, and bit 3 of v, so that both the writes (16
  // rows, one chunk, per 16 lanes) and the reads (2 rows, 8 chunks) meet
  // distinct 4-bank groups whether a pass serves 8 or 16 lanes.
  static __device__ __forceinline__ int stage_slot(int v, int ch) {
    return v * 8 + (ch ^ (v & 7) ^ ((v >> 3) & 1));
  }

  // Stores write whole 128-byte lines.  A lane holds 16-byte chunks 2q and
  // 2q+1 (by lane half) of row v = lane % 32 of an MFMA tile, so a store from
  // the accumulators would cover 32 rows with 32 bytes each.  The tiles pass
  // through this wave's 16 KiB of the ring instead (free after the loop), four
  // at a time, and come back as 8 rows x 8 chunks per read: each store then
  // covers 8 whole lines.
  template <int FM, int FN, int WM, int WNCOLS, int NT>
  __device__ __forceinline__ void run(f32x16_t (&acc)[FM][FN], const TileCtx& c) const {
    static_assert(FM == 4 && FN == 2 && WM == 2 && WNCOLS == 64 && NT == kThreadsPP,
                  "256 x 256 tile of 2 x 4 waves of 4 x 2 MFMA tiles");
    constexpr int kTileSlots = 32 * 8;  // one 32 x 32 fp32 tile
    static_assert(kWaves * 4 * kTileSlots <= kRing32 * 2 * kSlots32, "four tiles per wave in the ring");
    const i32x4_t r = make_rsrc(wave_base(c), wave_bytes(c));
    const int v = c.lane & 31, h = c.lane >> 5;   // staging: row, chunk parity
    const int rr = c.lane >> 3, ch = c.lane & 7;  // store: row within 8, chunk
    const int vo = (int)((rr * ldo + 4 * ch) * 4);
    if constexpr (kStage3) {
      static_assert(kWaves * kTileSlots * 16 <= 32 * 1024, "one 32 x 32 tile per wave in ring slot 3");
      u32x4_t* wb = static_cast<u32x4_t*>(c.lds) + 3 * kStagePP + c.wave * kTileSlots;
#pragma unroll
      for (int t = 0; t < FM * FN; ++t) {
        const int i = t / FN, j = t % FN;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          wb[stage_slot(v, 2 * q + h)] = __builtin_bit_cast(
              u32x4_t, f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]});
        u32x4_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = wb[stage_slot(8 * p + rr, ch)];
#pragma unroll
        for (int p = 0; p < 4; ++p) store_b128_nt_guarded(o[p], r, vo, (int)(((32 * j + 8 * p) * ldo + 32 * i) * 4));
      }
      return;
    }
    u32x4_t* wb = static_cast<u32x4_t*>(c.lds) + c.wave * 4 * kTileSlots;
    const bool full = c.m_wave + 32 * FM <= d_ext;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = 2 * half + t / 2, j = t % 2;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          wb[t * kTileSlots + stage_slot(v, 2 * q + h)] = __builtin_bit_cast(
              u32x4_t, f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]});
      }
      // all 16 reads first: the guarded stores are ordered against every
      // memory operation
      u32x4_t o[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p) o[t][p] = wb[t * kTileSlots + stage_slot(8 * p + rr, ch)];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = 2 * half + t / 2, j = t % 2;
        const bool ok = full || c.m_wave + 32 * i + 4 * ch < d_ext;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (ok) store_b128_nt_guarded(o[t][p], r, vo, (int)(((32 * j + 8 * p) * ldo + 32 * i) * 4));
      }
    }
  }
};

}  // namespace sbp
