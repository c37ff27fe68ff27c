// One 256x256 output tile of C[m][n] = sum_k A(m, k) B(n, k) on gfx950 matrix
// cores, fp32 accumulation.
//
// Operands come in two orientations:
//  * NT ("K-contiguous"): the operand is stored with rows = M (or N) indices and K
//    contiguous in a row: the LM-head weight W [v][d] and the hidden states H [t][d]
//    in the logit product, and dz [t][v] in the dH product.
//  * MN ("MN-contiguous"): rows = K indices, M (or N) contiguous: W [v][d] and
//    H [t][d] as the d-side of the dH / dW products, and dz [t][v] as the v-side of
//    the dW product.  Fragments are read from LDS with the transposing
//    ds_read_b64_tr_b16 (bf16), so no operand is ever transposed in memory.
//
// Geometry and pipeline:
//  * 512 threads = 8 waves in a 2 (M) x 4 (N) grid; each wave owns a 128x64
//    sub-tile as 8x4 blocks of 16x16 MFMA accumulators (128 fp32 per lane), so
//    two waves share each SIMD and the hardware issues one wave's MFMAs while the
//    other waits on memory or a barrier.
//  * bf16: v_mfma_f32_16x16x32_bf16, one per fragment pair.  Under the chip's power
//    limit this form sustains a markedly higher clock than 32x32x16 on random
//    operands at the same MFMA occupancy.  fp32: v_mfma_f32_16x16x4_f32, four per
//    fragment pair (exact fp32 products).
//  * K advances 128 bytes per stage (64 bf16 or 32 fp32); a stage is 32 KB of A and
//    32 KB of B in LDS, double buffered (128 KB of the CU's 160 KB).
//  * Global -> LDS through direct-to-LDS raw buffer loads, 16 B per lane, every
//    wave-wide load filling 1 KB of LDS.  Bytes outside an operand's buffer range
//    load as zeros; the ranges are set so that no invalid row (padded vocabulary,
//    tokens past the batch) is ever read.
//  * NT stage layout: 256 rows x 128 B; chunk c of row r sits at chunk
//    c ^ ((r >> 1) & 7).  A fragment read (ds_read_b128) has each group of 16 lanes
//    on 16 consecutive rows at one logical chunk: 16 distinct bank groups of the
//    64-bank LDS.
//  * MN stage layout (bf16): 64 K-rows x 512 B; 32-byte segment s of K-row k sits
//    at segment s ^ sw(k), sw(k) = (k & 3) | ((k >> 1) & 4).  One pass of a
//    transposing read serves 32 lanes on 8 K-rows at one logical segment: 8
//    distinct bank groups.  (fp32 MN: 32 K-rows x 1 KB, unswizzled, read with
//    ds_read_b32; the fp32 path exists for exactness, not speed.)
//
// Accumulator layout (per wave, block (i, j), element e of the 4), relative to
// the wave's sub-tile at (wm * 128, wn * 64):
//   row (M) = i*16 + (lane >> 4)*4 + e
//   col (N) = j*16 + (lane & 15)
// so each lane holds 4 consecutive M indices for one N index per (i, j).
#pragma once

#include "device_common.hpp"

namespace gh {

constexpr int kTile = 256;
constexpr int kWM = 2, kWN = 4;                 // wave grid
constexpr int kWaves = kWM * kWN;
constexpr int kThreads = 64 * kWaves;
constexpr int kBI = kTile / kWM / 16;           // 16-row accumulator blocks per wave (M)
constexpr int kBJ = kTile / kWN / 16;           // 16-col accumulator blocks per wave (N)
constexpr int kStageBytes = 128;                // K bytes per stage
constexpr int kOpLds = kTile * kStageBytes;     // one operand's stage: 32 KB
constexpr int kStageLds = 2 * kOpLds;           // A + B
constexpr int kGemmLds = 2 * kStageLds;         // two stage buffers: 128 KB
constexpr int kLoads = kOpLds / 1024 / kWaves;  // wave-wide 1 KB loads per operand and stage

// Addressing of an operand.  For the tile holding M/N indices [256 t, 256 t + 256):
//   base_t = base + t * tile_bytes, valid for clamp(span - t * tile_bytes, 0, cap)
//   bytes from base_t; bytes beyond load as zeros.
// NT: byte (row r of the tile, K byte kb) = r * ld + stage_off(kb / 128) + kb % 128,
//     stage_off(s) = (s >> group_shift) * group_bytes + (s & (2^group_shift - 1)) * 128.
// MN: byte (K row k, element r of the tile) = k * ld + r * element size, or, with
//     group_bytes > 0 (blocked by 64 elements), k * ld + (r / 64) * group_bytes +
//     (r % 64) * element size.
struct Operand {
  const char* base;
  int64_t ld;           // bytes between rows (NT: M/N rows; MN: K rows)
  int64_t tile_bytes;   // bytes between 256-wide M/N tiles
  int64_t span;         // valid bytes from base (see above)
  int64_t cap;          // most bytes one tile's resource may cover
  int64_t group_bytes;  // NT: bytes between K-stage groups; MN: between 64-element blocks
  int32_t group_shift;  // NT: log2(stages per group)
  int32_t mn;           // 1: MN-contiguous
};

// Row-major [rows][K] with K contiguous (pitch bytes per row); rows >= `rows` load
// as zeros.
__host__ __device__ inline Operand nt_row_major(const void* base, int64_t pitch, int64_t rows) {
  return Operand{(const char*)base, pitch, 256 * pitch, rows * pitch, 256 * pitch, 0, 30, 0};
}
// The v-blocked layout [blocks][rows_pad][64 elements] (dz) read K-contiguous with
// rows = its rows and K = the 64-element blocks in order: a stage of 256 rows is
// one contiguous run (bf16: one block; fp32: half a block per row).
__host__ __device__ inline Operand nt_vblocked(const void* base, int64_t rows_pad, int64_t esz,
                                              int64_t total_bytes) {
  const int32_t shift = esz == 2 ? 0 : 1;   // 128-byte stages per 64-element block
  return Operand{(const char*)base, 64 * esz, 256 * 64 * esz, total_bytes, total_bytes,
                 rows_pad * 64 * esz, shift, 0};
}
// Row-major [k_rows][cols] (pitch bytes per row) read MN-contiguous, K = its rows:
// K rows >= k_rows and columns >= cols of the last valid row load as zeros.
__host__ __device__ inline Operand mn_row_major(const void* base, int64_t pitch, int64_t k_rows,
                                               int64_t cols, int64_t esz) {
  return Operand{(const char*)base, pitch, 256 * esz,
                 k_rows > 0 ? (k_rows - 1) * pitch + cols * esz : 0, (int64_t)1 << 62, 0, 30, 1};
}
// The v-blocked layout read MN-contiguous: K = its rows, M/N = the elements; a
// 256-element tile is 4 blocks, and a K row of it 4 runs of 64 elements.
__host__ __device__ inline Operand mn_vblocked(const void* base, int64_t rows_pad, int64_t esz,
                                              int64_t blocks) {
  const int64_t bb = rows_pad * 64 * esz;
  return Operand{(const char*)base, 64 * esz, 4 * bb, blocks * bb, 4 * bb, bb, 30, 1};
}
// Byte offset of (row, element v) in the v-blocked layout.
__host__ __device__ inline int64_t vblocked_offset(int64_t row, int64_t v, int64_t rows_pad,
                                                   int64_t esz) {
  return (v >> 6) * rows_pad * 64 * esz + row * 64 * esz + (v & 63) * esz;
}

// Base and valid byte count of one M/N tile of an operand.
struct TileRange {
  const char* base;
  int64_t limit;
};
__device__ __forceinline__ TileRange tile_range(const Operand& op, int64_t r0) {
  const int64_t t = r0 >> 8;
  int64_t n = op.span - t * op.tile_bytes;
  n = n < 0 ? 0 : (n > op.cap ? op.cap : n);
  return TileRange{op.base + t * op.tile_bytes, n};
}

// Byte offset of K stage s from the tile base (64-bit: operands may exceed 4 GB).
template <typename T>
__device__ __forceinline__ int64_t stage_off(const Operand& op, int s) {
  if (op.mn) return (int64_t)s * (kStageBytes / (int)sizeof(T)) * op.ld;
  return (int64_t)(s >> op.group_shift) * op.group_bytes +
         (int64_t)(s & ((1 << op.group_shift) - 1)) * kStageBytes;
}

// Buffer resource of one K stage of a tile: based at the stage, so per-lane
// offsets stay small; bytes past the tile's valid range load as zeros.  With in_k
// false (a stage past the end of K: the pipeline's two trailing loads, never used)
// the range is empty, so the loads return zeros without a memory access.  Only the
// single-tile path with both operands K-contiguous (the backward's dlogits) uses
// it: there it measured faster, while in the MN-operand products and the chained
// forward the extra select measured slower.  (The clamp is written on 32-bit halves
// so it stays in scalar registers.)
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(const Operand& op,
                                                             const TileRange& tr, int s,
                                                             bool in_k = true) {
  const int64_t o = stage_off<T>(op, s);
  const int64_t n = in_k ? tr.limit - o : 0;
  const int32_t hi = (int32_t)(n >> 32);
  const uint32_t lo = (uint32_t)n;
  const uint32_t rec = hi < 0 ? 0u : (hi > 0 ? 0xffffffffu : lo);
  // every field is wave-uniform; say so, so the resource lives in scalar registers
  const uint64_t b = (uint64_t)(uintptr_t)(tr.base + o);
  const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)bhi << 32) | blo),
                   __builtin_amdgcn_readfirstlane(rec));
}

// Byte stride between consecutive K stages of an operand whose stages are evenly
// spaced: an MN-contiguous operand, a K-contiguous one stored row-major (no
// grouping of stages), or a K-contiguous one with one stage per group (the
// v-blocked dz in bf16).  gemm_tile_chain_mn takes only such operands.
template <typename T>
__device__ __forceinline__ int64_t stage_stride(const Operand& op, bool mn) {
  if (mn) return (int64_t)(kStageBytes / (int)sizeof(T)) * op.ld;
  return op.group_shift == 0 ? op.group_bytes : (int64_t)kStageBytes;
}

// Buffer resource over `limit` bytes from `base` (none if limit <= 0; at most
// 4 GB - 1), with wave-uniform fields kept in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const char* base, int64_t limit) {
  const int32_t hi = (int32_t)(limit >> 32);
  const uint32_t lo = (uint32_t)limit;
  const uint32_t rec = hi < 0 ? 0u : (hi > 0 ? 0xffffffffu : lo);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)bhi << 32) | blo),
                   __builtin_amdgcn_readfirstlane(rec));
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes at voffset + soffset of
// the resource land at LDS byte lds_addr + 16 l.  Issued as inline assembly so
// that the compiler does not treat the in-flight LDS writes as aliasing every
// later LDS read (it would wait for all loads before each read); the pipeline
// waits for these loads explicitly.  M0 holds the LDS address; nothing else in
// these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                      uint32_t soffset, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                   :
                   : "v"(voffset), "s"(r), "s"(soffset), "s"(lds_addr)
                   : "memory", "m0");
}
// One wave's share of a stage of one operand in the chained cores: kLoads pairs of
// loads (lane offsets o0 and o1, the pair's K rows i * step further on), filling
// the 1 KB LDS blocks lds_addr, + 4 KB, + 8 KB, ... in turn.  One asm block that
// steps M0 and the scalar offset itself, so the eight destinations take no
// registers of their own.  (s_nop after each M0 write: the wait state an M0 write
// needs before an LDS-DMA load.)
__device__ __forceinline__ void dma16_split(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t o1,
                                            uint32_t step, uint32_t lds_addr) {
  static_assert(kLoads == 4, "four pairs of loads per wave and stage");
  uint32_t t;
  __asm__ volatile(
      "s_mov_b32 m0, %[l]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v0], %[r], 0 offen lds\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v1], %[r], 0 offen lds\n\t"
      "s_mov_b32 %[t], %[st]\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v0], %[r], %[t] offen lds\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v1], %[r], %[t] offen lds\n\t"
      "s_add_u32 %[t], %[t], %[st]\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v0], %[r], %[t] offen lds\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v1], %[r], %[t] offen lds\n\t"
      "s_add_u32 %[t], %[t], %[st]\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v0], %[r], %[t] offen lds\n\t"
      "s_add_u32 m0, m0, 0x1000\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v1], %[r], %[t] offen lds"
      : [t] "=&s"(t)
      : [v0] "v"(o0), [v1] "v"(o1), [r] "s"(r), [st] "s"(step), [l] "s"(lds_addr)
      : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  static __device__ __forceinline__ void run(f32x4& c, i32x4 a, i32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x4& c, i32x4 a, i32x4 b) {
    const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], c, 0, 0, 0);
  }
};

typedef __attribute__((address_space(3))) char lds_t;

__device__ __forceinline__ i32x4 lds_read16(const lds_t* p) {
  return *(const __attribute__((address_space(3))) i32x4*)p;
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
// Transposing LDS read (ds_read_b64_tr_b16): 8 bytes per lane, redistributed within
// each group of 16 lanes.
__device__ __forceinline__ i32x2 lds_read_tr16(const lds_t* p) {
  return __builtin_bit_cast(
      i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p));
}
__device__ __forceinline__ int lds_read4(const lds_t* p) {
  return *(const __attribute__((address_space(3))) int*)p;
}

template <int N> __device__ __forceinline__ void wait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until every LDS access of this wave has completed (s_waitcnt lgkmcnt(0)),
// written as the builtin so that the compiler's own wait tracking sees it.
__device__ __forceinline__ void lgkm_drain() {
  // gfx9 s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8];
  // vmcnt and expcnt at their maxima (no wait), lgkmcnt 0
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Workgroup barrier for the K pipeline.  __syncthreads() would also drain every
// in-flight direct-to-LDS load (its fence waits for vmcnt(0)); here the caller
// waits for exactly the stage it needs, and this wave's LDS reads are drained
// so no other wave's loads can overwrite a buffer still being read.
__device__ __forceinline__ void pipe_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// NT stage swizzle: physical 16-B chunk of logical chunk c in row r is c ^ swz_nt(r)
__device__ __forceinline__ int swz_nt(int r) { return (r >> 1) & 7; }
// MN (bf16) stage swizzle: physical 32-B segment of logical segment s in K-row k
// is s ^ swz_mn(k)
__device__ __forceinline__ int swz_mn(int k) { return (k & 3) | ((k >> 1) & 4); }

// Per-lane byte offset (relative to the stage base) of this wave's first
// wave-wide load of one operand stage, and the byte step between its kLoads
// loads.  Load i fills LDS bytes [(wave + 8 i) * 1024, + 1024) of the operand's
// stage region, lane l the 16 bytes at + 16 l; the lane fetches the logical bytes
// that belong at that physical place.  Load i covers rows (NT) or K-rows (MN)
// 64 i, 16 i or 8 i further on, which leaves every swizzle unchanged, so one
// offset serves all loads.
template <typename T, int kBlocked = -1>
__device__ __forceinline__ uint32_t load_offset(const Operand& op, int wave, int lane,
                                                uint32_t& step) {
  // kBlocked: 1 or 0 when the caller knows whether an MN operand is blocked, -1
  // to look at op.group_bytes
  const bool blocked = kBlocked < 0 ? op.group_bytes != 0 : kBlocked != 0;
  if (!op.mn) {
    const int r = wave * 8 + (lane >> 3);                          // 8 rows of 128 B
    const int c = (lane & 7) ^ swz_nt(r);
    step = (uint32_t)(kWaves * 8 * op.ld);
    return (uint32_t)(r * op.ld + c * 16);
  } else if (sizeof(T) == 2) {
    const int k = wave * 2 + (lane >> 5);                          // 2 K-rows of 512 B
    const int pc = lane & 31;                                      // physical chunk
    const int c = (((pc >> 1) ^ swz_mn(k)) << 1) | (pc & 1);
    step = (uint32_t)(kWaves * 2 * op.ld);
    // blocked: 16-byte chunk c is element 8 c of the tile, in block c / 8
    return blocked ? (uint32_t)(k * op.ld + (c >> 3) * op.group_bytes + (c & 7) * 16)
                   : (uint32_t)(k * op.ld + c * 16);
  } else {
    const int k = wave;                                            // 1 K-row of 1 KB
    step = (uint32_t)(kWaves * op.ld);
    return blocked ? (uint32_t)(k * op.ld + (lane >> 4) * op.group_bytes + (lane & 15) * 16)
                   : (uint32_t)(k * op.ld + lane * 16);
  }
}

// Fragment of 16 M/N indices (block origin r0 within the 256-wide tile) for K
// sub-step ks (32 bf16 or 16 fp32 of the stage) from an operand stage region.
// Lane l gets index r0 + (l & 15) and K elements 8 (l >> 4) .. + 7 of the
// sub-step (bf16; fp32: 4 (l >> 4) .. + 3).
template <typename T, bool kMN>
__device__ __forceinline__ i32x4 read_frag(const lds_t* region, int r0, int ks, int lane) {
  if (!kMN) {
    const int r = r0 + (lane & 15);
    const int c = (4 * ks + (lane >> 4)) ^ swz_nt(r);
    return lds_read16(region + r * kStageBytes + c * 16);
  } else if (sizeof(T) == 2) {
    // Two transposing reads of 4 K-rows each.  Lane s of a 16-lane group points at
    // K-row (base + s / 4), elements r0 + 4 (s % 4) .. + 3; the read hands lane j
    // the 4 K values of element r0 + j.
    const int g = lane >> 4, s = lane & 15;
    const int seg = r0 >> 4;
    const int k0 = 32 * ks + 8 * g + (s >> 2);
    const int k1 = k0 + 4;
    const i32x2 lo = lds_read_tr16(region + k0 * 512 + ((seg ^ swz_mn(k0)) << 5) + (s & 3) * 8);
    const i32x2 hi = lds_read_tr16(region + k1 * 512 + ((seg ^ swz_mn(k1)) << 5) + (s & 3) * 8);
    return i32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    const int g = lane >> 4, r = r0 + (lane & 15);
    const lds_t* p = region + (16 * ks + 4 * g) * 1024 + r * 4;
    return i32x4{lds_read4(p), lds_read4(p + 1024), lds_read4(p + 2048), lds_read4(p + 3072)};
  }
}

// Load-issue modes of the tile core (see gemm_tile).
constexpr int kIssueSolo = 1;    // waves 0-3 load both operands for all 8 waves
constexpr int kIssueSplit = 2;   // waves 0-3 load all of B, waves 4-7 all of A

// acc[i][j] += A(m0 + wave rows, :) . B(n0 + wave cols, :) over nk K stages.  An
// MN-contiguous B is row-major (not blocked).
//
// Stage s lives in LDS buffer s % 2, filled with direct-to-LDS buffer loads
// issued by a subset of the waves (kIssue; the reason is at the issue code).  A
// stage is two 32-element sub-steps of 32 MFMAs per wave.  Iteration s: read
// stage s's second fragments and multiply its first; then wait for stage s + 1's
// loads and barrier -- after which every wave holds all of stage s in registers,
// so stage s's buffer can take the loads of stage s + 2, a full stage ahead of
// their use -- read stage s + 1's first fragments and multiply stage s's second.
// The next fragments' LDS reads always run under the current MFMAs, one read
// between consecutive MFMAs.  The loop has no data-dependent branches: the stages
// past the end of K are loaded (zeros, or unused bytes inside the operand) and read
// like the others and never used, so every wait count is a constant.  All
// loads are drained before returning: none may write LDS after the workgroup
// releases it.
template <typename T, bool kMNA, bool kMNB,
          int kIssue = (!kMNA && !kMNB) ? kIssueSolo : kIssueSplit>
__device__ __forceinline__ void gemm_tile(const Operand& A, const Operand& B, int64_t m0,
                                          int64_t n0, int nk, lds_t* lds,
                                          f32x4 (&acc)[kBI][kBJ]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;

  const TileRange ta = tile_range(A, m0), tb = tile_range(B, n0);
  const int rA = wm * (kTile / kWM), rB = wn * (kTile / kWN);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Load issue is uneven on purpose.  Waves w and w + 4 share a SIMD.  With both
  // operands K-contiguous, waves 0-3 issue every load of a stage (their own and
  // their partners'), so the partner never stalls on a load burst and keeps the
  // SIMD's matrix core fed meanwhile.  With an MN-contiguous B that measured
  // slower than an even share; there waves 0-3 load all of B and waves 4-7 all
  // of A, which measured faster than both the even share and the opposite split.
  constexpr bool kSolo = kIssue == kIssueSolo;
  constexpr int kHalf = kWaves / 2;
  const int lw = wave & (kHalf - 1);
  uint32_t stepA, stepB;
  const uint32_t offA0 = load_offset<T>(A, lw, lane, stepA);
  const uint32_t offA1 = load_offset<T>(A, lw + kHalf, lane, stepA);
  const uint32_t offB0 = load_offset<T, 0>(B, lw, lane, stepB);
  const uint32_t offB1 = load_offset<T, 0>(B, lw + kHalf, lane, stepB);
  auto issue = [&](int stage) {
    const uint32_t s0 = lds_base + (stage & 1) * kStageLds + lw * 1024;
    const uint32_t s1 = s0 + kHalf * 1024;
    const bool first = wave < kHalf;
    if (kSolo) {
      if (!first) return;
      const __amdgpu_buffer_rsrc_t ra = stage_rsrc<T>(A, ta, stage, stage < nk);
      const __amdgpu_buffer_rsrc_t rb = stage_rsrc<T>(B, tb, stage, stage < nk);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const uint32_t ia = __builtin_amdgcn_readfirstlane(i * stepA);
        const uint32_t ib = __builtin_amdgcn_readfirstlane(i * stepB);
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(s0 + i * kWaves * 1024);
        const uint32_t l1 = __builtin_amdgcn_readfirstlane(s1 + i * kWaves * 1024);
        dma16(ra, offA0, ia, l0);
        dma16(rb, offB0, ib, l0 + kOpLds);
        dma16(ra, offA1, ia, l1);
        dma16(rb, offB1, ib, l1 + kOpLds);
      }
    } else {
      // waves 0-3 take B, waves 4-7 take A; each loads the shares of waves lw, lw + 4
      const __amdgpu_buffer_rsrc_t r = first ? stage_rsrc<T>(B, tb, stage)
                                             : stage_rsrc<T>(A, ta, stage);
      const uint32_t o0 = first ? offB0 : offA0, o1 = first ? offB1 : offA1;
      const uint32_t step = first ? stepB : stepA;
      const uint32_t region = first ? (uint32_t)kOpLds : 0u;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const uint32_t is = __builtin_amdgcn_readfirstlane(i * step);
        dma16(r, o0, is, __builtin_amdgcn_readfirstlane(s0 + region + i * kWaves * 1024));
        dma16(r, o1, is, __builtin_amdgcn_readfirstlane(s1 + region + i * kWaves * 1024));
      }
    }
  };
  auto read_frags = [&](i32x4 (&fa)[kBI], i32x4 (&fb)[kBJ], int stage, int ks) {
    const lds_t* s = lds + (stage & 1) * kStageLds;
#pragma unroll
    for (int i = 0; i < kBI; ++i) fa[i] = read_frag<T, kMNA>(s, rA + 16 * i, ks, lane);
#pragma unroll
    for (int j = 0; j < kBJ; ++j) fb[j] = read_frag<T, kMNB>(s + kOpLds, rB + 16 * j, ks, lane);
  };
  // A sub-step runs as four quarters of 8 MFMAs (A blocks 2c, 2c + 1 by
  // every B block); quarter 0 reads all of the next B blocks (every quarter of
  // the next sub-step needs them), quarter c the next A blocks 2c, 2c + 1.
  auto quarter = [&](const i32x4 (&ca)[kBI], const i32x4 (&cb)[kBJ], i32x4 (&na)[kBI],
                     i32x4 (&nb)[kBJ], int rstage, int rks, int c) {
    const lds_t* s = lds + (rstage & 1) * kStageLds;
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < kBJ; ++j) nb[j] = read_frag<T, kMNB>(s + kOpLds, rB + 16 * j, rks, lane);
    }
    na[2 * c] = read_frag<T, kMNA>(s, rA + 16 * (2 * c), rks, lane);
    na[2 * c + 1] = read_frag<T, kMNA>(s, rA + 16 * (2 * c + 1), rks, lane);
#pragma unroll
    for (int i = 2 * c; i < 2 * c + 2; ++i)
#pragma unroll
      for (int j = 0; j < kBJ; ++j) Mma<T>::run(acc[i][j], ca[i], cb[j]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  static_assert(kBI == 8 && kBJ == 4, "quarters take the 8 A blocks in pairs");

  if (nk <= 0) return;
  i32x4 fa0[kBI], fb0[kBJ], fa1[kBI], fb1[kBJ];
  issue(0);
  issue(1);
  wait_vm<(kSolo ? 4 : 2) * kLoads>();   // stage 0 landed; stage 1 may be in flight
  pipe_barrier();
  read_frags(fa0, fb0, 0, 0);
  // Let these reads land before the loop.  With an MN operand they are 16 LDS
  // reads, more than the 4-bit LDS counter the compiler's wait tracking follows;
  // entering the loop with them in flight made it wait for every LDS read
  // (lgkmcnt(0)) at the head of each K stage, while drained here it emits exact
  // counts there.  The cost is one LDS round trip per tile.
  lgkm_drain();
  __builtin_amdgcn_sched_barrier(0);

  for (int kt = 0; kt < nk; ++kt) {
    // sub-step 0: read stage kt's second fragments, multiply its first
#pragma unroll
    for (int c = 0; c < 4; ++c) quarter(fa0, fb0, fa1, fb1, kt, 1, c);
    // sub-step 1: once every wave holds all of stage kt (its reads are drained) and
    // stage kt + 1 has landed, stage kt's buffer takes the loads of stage kt + 2,
    // a full stage ahead of their use (issued as one burst after the first quarter:
    // spread over the quarters, or issued before them, measured slower)
    wait_vm<0>();
    pipe_barrier();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      quarter(fa1, fb1, fa0, fb0, kt + 1, 0, c);
      if (c == 0) {
        issue(kt + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  wait_vm<0>();
  pipe_barrier();
}

// gemm_tile for two K-contiguous row-major operands (nt_row_major: stage s sits
// s x kStageBytes into each tile's range), chained across the tiles one workgroup
// computes in turn (an even number of K stages, so stage s of every tile sits in
// LDS buffer s % 2).  The loads that gemm_tile spends on the two stages past the
// end of K fetch the next tile's stages 0 and 1 instead, and the last fragment
// read of the loop is the next tile's first: on return with has_next, fa0/fb0 hold
// those fragments and stage 1 is in flight, which is the state gemm_tile's prologue
// builds.  The caller's epilogue may then use LDS outside the pipeline buffers and
// wait on LDS only (pipe_barrier), and calls again with first = false.  Without a
// next tile the loads are drained before returning, as in gemm_tile.
template <typename T>
__device__ __forceinline__ void gemm_tile_chain(const Operand& A, const Operand& B, int64_t m0,
                                                int64_t n0, bool has_next, int64_t m0n,
                                                int64_t n0n, int nk, bool first, lds_t* lds,
                                                f32x4 (&acc)[kBI][kBJ], i32x4 (&fa0)[kBI],
                                                i32x4 (&fb0)[kBJ]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;

  const TileRange ta = tile_range(A, m0), tb = tile_range(B, n0);
  const TileRange tan = tile_range(A, has_next ? m0n : m0);
  const TileRange tbn = tile_range(B, has_next ? n0n : n0);
  const int rA = wm * (kTile / kWM), rB = wn * (kTile / kWN);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // waves 0-3 issue every load of a stage (as gemm_tile does for two K-contiguous
  // operands); stages nk and nk + 1 come from the next tile when there is one
  constexpr int kHalf = kWaves / 2;
  const int lw = wave & (kHalf - 1);
  uint32_t stepA, stepB;
  const uint32_t offA0 = load_offset<T>(A, lw, lane, stepA);
  const uint32_t offA1 = load_offset<T>(A, lw + kHalf, lane, stepA);
  const uint32_t offB0 = load_offset<T>(B, lw, lane, stepB);
  const uint32_t offB1 = load_offset<T>(B, lw + kHalf, lane, stepB);
  // (which: 1 = A's loads, 2 = B's, 3 = both)
  auto issue = [&](int stage, int which) {
    if (wave >= kHalf) return;
    const uint32_t s0 = lds_base + (stage & 1) * kStageLds + lw * 1024;
    const bool nxt = has_next && stage >= nk;
    const int ks = nxt ? stage - nk : stage;
    // both operands K-contiguous: a stage starts kStageBytes further along each tile's
    // range, and each operand's eight loads go out in one asm block
    const int64_t o = (int64_t)ks * kStageBytes;
    const TileRange xa = nxt ? tan : ta, xb = nxt ? tbn : tb;
    const __amdgpu_buffer_rsrc_t ra = range_rsrc(xa.base + o, xa.limit - o);
    const __amdgpu_buffer_rsrc_t rb = range_rsrc(xb.base + o, xb.limit - o);
    const uint32_t l = __builtin_amdgcn_readfirstlane(s0);
    if (which & 1) dma16_split(ra, offA0, offA1, __builtin_amdgcn_readfirstlane(stepA), l);
    if (which & 2) dma16_split(rb, offB0, offB1, __builtin_amdgcn_readfirstlane(stepB), l + kOpLds);
  };
  auto quarter = [&](const i32x4 (&ca)[kBI], const i32x4 (&cb)[kBJ], i32x4 (&na)[kBI],
                     i32x4 (&nb)[kBJ], int rstage, int rks, int c) {
    const lds_t* s = lds + (rstage & 1) * kStageLds;
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < kBJ; ++j) nb[j] = read_frag<T, false>(s + kOpLds, rB + 16 * j, rks, lane);
    }
    na[2 * c] = read_frag<T, false>(s, rA + 16 * (2 * c), rks, lane);
    na[2 * c + 1] = read_frag<T, false>(s, rA + 16 * (2 * c + 1), rks, lane);
#pragma unroll
    for (int i = 2 * c; i < 2 * c + 2; ++i)
#pragma unroll
      for (int j = 0; j < kBJ; ++j) Mma<T>::run(acc[i][j], ca[i], cb[j]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  i32x4 fa1[kBI], fb1[kBJ];
  if (first) {
    issue(0, 3);
    issue(1, 3);
    wait_vm<4 * kLoads>();   // stage 0 landed; stage 1 may be in flight
    pipe_barrier();
    const lds_t* s = lds;
#pragma unroll
    for (int i = 0; i < kBI; ++i) fa0[i] = read_frag<T, false>(s, rA + 16 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < kBJ; ++j) fb0[j] = read_frag<T, false>(s + kOpLds, rB + 16 * j, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) quarter(fa0, fb0, fa1, fb1, kt, 1, c);
    wait_vm<0>();
    pipe_barrier();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      quarter(fa1, fb1, fa0, fb0, kt + 1, 0, c);
      // stage kt + 2's loads: B's after quarter 0, A's after quarter 1 (one burst of
      // both after quarter 0 ran the dlogits tiles 1.5% slower, the forward's 0.5%)
      if (c == 0) {
        issue(kt + 2, 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (c == 1) {
        issue(kt + 2, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!has_next) {
    wait_vm<0>();
    pipe_barrier();
  }
}

// gemm_tile_chain for a K-contiguous A whose stages are evenly spaced and an
// MN-contiguous B, blocked by 64 elements (kBlockedB: the dW product) or row-major
// (the dH product, which calls it for single tiles: has_next false, first true).
// Each operand is a plain stream of stages at a fixed byte stride, and waves 0-3
// issue every load, each operand's eight loads of a stage as one asm block, as in
// gemm_tile_chain.  With gemm_tile's generic stage addressing the compiler
// spilled registers in this loop; with one asm block per stage the waves 0-3
// issue pays off for these operands too (the gradient launch 13.90 -> 13.72 ms
// against waves 0-3 loading B and waves 4-7 A, in alternating runs).  The first
// wait of a chained call also waits for the caller's epilogue stores, which were
// issued after the next tile's stage-1 loads: letting them stay in flight there,
// with a second wait count for the first stage, made the compiler spill.
template <typename T, bool kBlockedB = true>
__device__ __forceinline__ void gemm_tile_chain_mn(const Operand& A, const Operand& B,
                                                   int64_t m0, int64_t n0, bool has_next,
                                                   int64_t m0n, int64_t n0n, int nk,
                                                   bool first, lds_t* lds,
                                                   f32x4 (&acc)[kBI][kBJ],
                                                   i32x4 (&fa0)[kBI], i32x4 (&fb0)[kBJ]) {
  const int tid = threadIdx.x;
  // (the lane index made opaque: the per-lane offsets below are then formed on each
  // call rather than hoisted out of the caller's tile loop and kept across it)
  int lane = tid & 63;
  __asm__ volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;

  const TileRange ta = tile_range(A, m0), tb = tile_range(B, n0);
  const TileRange tan = tile_range(A, has_next ? m0n : m0);
  const TileRange tbn = tile_range(B, has_next ? n0n : n0);
  const int rA = wm * (kTile / kWM), rB = wn * (kTile / kWN);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // stages nk and nk + 1 come from the next tile when there is one; waves 0-3 load
  // both operands, each the shares of waves lw and lw + 4
  constexpr int kHalf = kWaves / 2;
  const int lw = wave & (kHalf - 1);
  uint32_t stepA, stepB;
  const uint32_t offA0 = load_offset<T>(A, lw, lane, stepA);
  const uint32_t offA1 = load_offset<T>(A, lw + kHalf, lane, stepA);
  const uint32_t offB0 = load_offset<T, kBlockedB ? 1 : 0>(B, lw, lane, stepB);
  const uint32_t offB1 = load_offset<T, kBlockedB ? 1 : 0>(B, lw + kHalf, lane, stepB);
  const int64_t strideA = stage_stride<T>(A, false), strideB = stage_stride<T>(B, true);
  // (which: 1 = A's loads, 2 = B's, 3 = both)
  auto issue = [&](int stage, int which) {
    if (wave >= kHalf) return;
    const uint32_t s0 = lds_base + (stage & 1) * kStageLds + lw * 1024;
    const bool nxt = has_next && stage >= nk;
    const int ks = nxt ? stage - nk : stage;
    const TileRange xa = nxt ? tan : ta, xb = nxt ? tbn : tb;
    const int64_t oa = (int64_t)ks * strideA, ob = (int64_t)ks * strideB;
    const __amdgpu_buffer_rsrc_t ra = range_rsrc(xa.base + oa, xa.limit - oa);
    const __amdgpu_buffer_rsrc_t rb = range_rsrc(xb.base + ob, xb.limit - ob);
    const uint32_t l = __builtin_amdgcn_readfirstlane(s0);
    if (which & 1) dma16_split(ra, offA0, offA1, __builtin_amdgcn_readfirstlane(stepA), l);
    if (which & 2) dma16_split(rb, offB0, offB1, __builtin_amdgcn_readfirstlane(stepB), l + kOpLds);
  };
  auto quarter = [&](const i32x4 (&ca)[kBI], const i32x4 (&cb)[kBJ], i32x4 (&na)[kBI],
                     i32x4 (&nb)[kBJ], int rstage, int rks, int c) {
    const lds_t* s = lds + (rstage & 1) * kStageLds;
    if (c == 0) {
#pragma unroll
      for (int j = 0; j < kBJ; ++j) nb[j] = read_frag<T, true>(s + kOpLds, rB + 16 * j, rks, lane);
    }
    na[2 * c] = read_frag<T, false>(s, rA + 16 * (2 * c), rks, lane);
    na[2 * c + 1] = read_frag<T, false>(s, rA + 16 * (2 * c + 1), rks, lane);
#pragma unroll
    for (int i = 2 * c; i < 2 * c + 2; ++i)
#pragma unroll
      for (int j = 0; j < kBJ; ++j) Mma<T>::run(acc[i][j], ca[i], cb[j]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  i32x4 fa1[kBI], fb1[kBJ];
  if (first) {
    issue(0, 3);
    issue(1, 3);
    wait_vm<4 * kLoads>();   // stage 0 landed; stage 1 may be in flight
    pipe_barrier();
    const lds_t* s = lds;
#pragma unroll
    for (int i = 0; i < kBI; ++i) fa0[i] = read_frag<T, false>(s, rA + 16 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < kBJ; ++j) fb0[j] = read_frag<T, true>(s + kOpLds, rB + 16 * j, 0, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  // The MN operand's fragment reads outnumber the compiler's LDS wait counter (see
  // gemm_tile): enter the loop with none in flight.
  lgkm_drain();
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) quarter(fa0, fb0, fa1, fb1, kt, 1, c);
    wait_vm<0>();
    pipe_barrier();
    // stage kt + 2's loads: B's right after the barrier, A's after quarter 1.  The
    // gradient launch ran 2.3% slower with one burst of both right after the
    // barrier, and that was 1.3% faster than one burst after quarter 0.  (The logit
    // products lose with loads issued before quarter 0.)
    issue(kt + 2, 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      quarter(fa1, fb1, fa0, fb0, kt + 1, 0, c);
      if (c == 1) {
        issue(kt + 2, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!has_next) {
    wait_vm<0>();
    pipe_barrier();
  }
}

// The thread that takes the next tile of a persistent launch whose loads only
// waves 0-3 issue (the logit products): lane 0 of wave 4.  Its wave has no load in
// flight, so waiting for the queue access never waits for the next tile's loads
// (memory operations complete in issue order per wave).
constexpr int kGrabThread = 4 * 64;

// The next tile of a persistent launch for a workgroup on XCD `xcd` (queue_next:
// its own XCD's run of logical ids first, then the other XCDs'), as (M tile,
// N tile), or tm = -1 once every run is handed out.  queue[x] counts the ids handed
// out of XCD x's run and starts each launch at zero.  Taking from another XCD's
// run balances XCDs that finish their own at different times (their clocks differ
// by a few percent).
// Called by one thread; the tile counts pass through an empty asm statement so
// that the divisions are not hoisted out of the caller's tile loop, where their
// precomputed reciprocals would stay live across the K loop.
__device__ __forceinline__ void grab_tile(int32_t* queue, int xcd, int tiles_m, int tiles_n,
                                          int group_m, int& tm, int& tn) {
  __asm__("" : "+s"(tiles_m), "+s"(tiles_n), "+s"(group_m));
  auto take = [queue](int x) {
    return __hip_atomic_fetch_add(queue + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const int id = queue_next(take, xcd, tiles_m * tiles_n);
  if (id < 0) {
    tm = -1;
    tn = 0;
  } else {
    logical_coords(id, tiles_m, tiles_n, group_m, tm, tn);
  }
}

// Set every accumulator whose wave-local M row (0..127) is >= vlim to -inf.
// Used once per tile, only on the tile holding the vocabulary's ragged end.
__device__ __forceinline__ void mask_rows(f32x4 (&acc)[kBI][kBJ], int vlim) {
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < kBI; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool pad = i * 16 + q * 4 + e >= vlim;
#pragma unroll
      for (int j = 0; j < kBJ; ++j) acc[i][j][e] = pad ? -INFINITY : acc[i][j][e];
    }
}

__device__ __forceinline__ void zero_acc(f32x4 (&acc)[kBI][kBJ]) {
#pragma unroll
  for (int i = 0; i < kBI; ++i)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace gh
