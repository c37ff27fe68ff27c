// One 256x256 output tile of C = A . B^T on gfx950 matrix cores.
//
// A [M][K] and B [N][K] are row-major with K contiguous ("NT"): the layout of
// the LM-head weight (vocab rows, hidden contiguous) and of the hidden states
// (token rows, hidden contiguous), and the layout the backward's staging buffers
// are written in.  Accumulation is fp32.
//
//  * 512 threads = 8 waves in a 2 (M) x 4 (N) grid; each wave owns a 128x64
//    sub-tile as 8x4 blocks of 16x16 MFMA accumulators (128 fp32 per lane), so
//    two waves share each SIMD and the hardware issues one wave's MFMAs while the
//    other waits on memory or a barrier.
//  * K advances 128 bytes per stage (64 bf16 or 32 fp32); one stage of A and B is
//    2 x 32 KB of LDS, double buffered (128 KB of the CU's 160 KB).
//  * Operands are either row-major (the caller's W and H: rows ld_bytes apart,
//    a stage 128 bytes further along the row) or K-panel (the backward's own
//    staging buffers: each 256-row tile stores its K stages one after another,
//    256 x 128 contiguous bytes per stage), which keeps every stage of a tile in
//    one small address range.
//  * Global -> LDS through direct-to-LDS raw buffer loads (no register staging).
//    Rows at or beyond the operand's valid row count fall outside the buffer
//    resource and load as zeros, which also keeps padded vocabulary rows from ever
//    being read.
//  * LDS rows are 128 B (8 chunks of 16 B); chunk c of row r is stored at chunk
//    c ^ ((r >> 1) & 7).  gfx950's LDS has 64 banks (256 B) and serves a 16-byte
//    read for 16 lanes per pass; a fragment read has each group of 16 lanes on 16
//    consecutive rows at one logical chunk, i.e. physical (r & 1, c ^ ((r >> 1) & 7)),
//    all distinct, so every pass touches each bank once.
//  * bf16: v_mfma_f32_16x16x32_bf16, one per 16-B fragment pair.  fp32:
//    v_mfma_f32_16x16x4_f32, four per fragment pair (exact fp32 products).  Under
//    the chip's power limit the 16x16x32 form sustains a markedly higher clock
//    than 32x32x16 on random operands at the same MFMA occupancy.
//  * A fragment (16 B per lane) is row (16-row block origin + lane % 16), K bytes
//    16 * (4 ks + lane / 16) of the stage: the 16x16x32 operand layout.
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
// K pipeline: 128-byte K stages, 2 LDS buffers (128 KB)
constexpr int kRowB = 128;
constexpr int kNst = 2;

// Addressing of an operand: byte (row r of tile t, stage s, chunk c) lives at
//   base + t * tile_bytes + (r % 256) * ld_bytes + s * stage_bytes + 16 c.
struct Operand {
  const char* base;     // element (0, 0)
  int64_t ld_bytes;     // bytes between rows of a tile (row-major: the row pitch)
  int64_t stage_bytes;  // bytes between K stages (row-major: 128)
  int64_t tile_bytes;   // bytes between 256-row tiles (row-major: 256 * pitch)
  int64_t rows;         // valid rows; row-major rows beyond load as zero
  bool panel;           // K-panel layout: every row of every tile is initialised
};

__host__ __device__ inline Operand row_major(const void* base, int64_t pitch, int64_t rows) {
  return Operand{(const char*)base, pitch, 128, 256 * pitch, rows, false};
}
// K-panel layout of a [rows_pad][k_bytes] matrix (rows_pad a multiple of 256)
__host__ __device__ inline Operand k_panel(const void* base, int64_t k_bytes, int64_t rows) {
  return Operand{(const char*)base, 128, 256 * 128, 256 * k_bytes, rows, true};
}
// Byte offset of (row, byte kb along K) in the K-panel layout of a matrix whose
// rows hold k_bytes.
__host__ __device__ inline int64_t k_panel_offset(int64_t row, int64_t kb, int64_t k_bytes) {
  return (row >> 8) * 256 * k_bytes + (kb >> 7) * (256 * 128) + (row & 255) * 128 + (kb & 127);
}

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Operand& op, int64_t r0) {
  const char* base = op.base + (r0 >> 8) * op.tile_bytes;
  if (op.panel) return make_rsrc(base, (uint32_t)op.tile_bytes);
  int64_t valid = op.rows - r0;
  valid = valid < 0 ? 0 : (valid > kTile ? kTile : valid);
  return make_rsrc(base, (uint32_t)(valid * op.ld_bytes));
}

typedef __attribute__((address_space(3))) char lds_t;

__device__ __forceinline__ i32x4 lds_read16(const lds_t* p) {
  return *(const __attribute__((address_space(3))) i32x4*)p;
}

template <int N> __device__ __forceinline__ void wait_vm() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the K pipeline.  __syncthreads() would also drain every
// in-flight direct-to-LDS load (its fence waits for vmcnt(0)); here the caller
// waits for exactly the stage it needs, and this wave's LDS reads are drained
// so no other wave's loads can overwrite a buffer still being read.
__device__ __forceinline__ void pipe_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Shape of the K pipeline: ROWB bytes of K per stage and row (64 or 128) and
// NST stage buffers in LDS (loads run NST - 1 stages ahead of the MFMAs).
template <int ROWB, int NST> struct Pipe {
  static_assert(ROWB == 64 || ROWB == 128, "stage row bytes");
  static_assert(NST >= 2 && NST <= 5, "stages");
  static constexpr int kChunks = ROWB / 16;             // 16-byte chunks per row
  static constexpr int kStage = 2 * kTile * ROWB;       // A + B bytes per stage
  static constexpr int kLds = NST * kStage;
  static constexpr int kRowsPerLoad = 1024 / ROWB;      // rows one wave-wide load covers
  static constexpr int kKs = ROWB / 64;                 // 32-element bf16 K sub-steps
  // physical chunk of logical chunk c in row r; 16 consecutive rows read at one
  // logical chunk land on 16 distinct 16-byte bank groups of the 64-bank LDS
  static __device__ __forceinline__ int swz(int r) {
    return ROWB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
  }
};

// LDS bytes of the default pipeline.
constexpr int kGemmLds = Pipe<kRowB, kNst>::kLds;

// acc[i][j] += A[m0 + wave rows] . B[n0 + wave cols]^T over k_bytes of K.
//
// Stage s (ROWB bytes of K) lives in LDS buffer s % NST.  Each wave fills its
// share of a stage with direct-to-LDS buffer loads (16 B per lane; lane l's
// bytes land at the block base + 16 l, so the lane fetches the logical chunk
// that belongs at that physical position of the swizzled row).  Iteration s:
//   issue the loads of stage s + NST - 1 (into the buffer stage s - 1 used);
//   for each 32-element sub-step: read the next fragments, run 32 MFMAs on the
//   current ones; before the last sub-step's MFMAs, wait for stage s + 1's loads,
//   barrier, and read stage s + 1's first fragments, so that LDS latency hides
//   under those MFMAs.
// The loop has no data-dependent branches: stages past the end of K are loaded
// and read like the others (their offsets stay inside the operand, or past the
// resource end where loads return zeros) and are never used, so every wait count
// is a constant.  All loads are drained before returning: none may write LDS
// after the workgroup releases it.
template <typename T, int ROWB = kRowB, int NST = kNst>
__device__ __forceinline__ void gemm_tile(const Operand& A, const Operand& B, int64_t m0,
                                          int64_t n0, int64_t k_bytes, lds_t* lds,
                                          f32x4 (&acc)[kBI][kBJ]) {
  typedef Pipe<ROWB, NST> P;
  static_assert(ROWB == 128, "operand stage strides assume 128-byte stages");
  constexpr int kLoads = kTile / P::kRowsPerLoad / kWaves;   // per wave per operand
  constexpr int kAhead = (NST - 2) * 2 * kLoads;              // loads allowed in flight
  static_assert(kAhead <= 63, "vmcnt range");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;

  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(A, m0);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc(B, n0);

  // direct loads: wave-wide load i covers tile rows (wave + kWaves i) * 8 + lane / 8
  const int lrow = wave * P::kRowsPerLoad + lane / P::kChunks;
  const uint32_t cswz = (uint32_t)(((lane % P::kChunks) ^ P::swz(lrow)) << 4);
  const uint32_t offA = (uint32_t)(lrow * A.ld_bytes) + cswz;
  const uint32_t offB = (uint32_t)(lrow * B.ld_bytes) + cswz;
  const uint32_t stepA = (uint32_t)(kWaves * P::kRowsPerLoad * A.ld_bytes);
  const uint32_t stepB = (uint32_t)(kWaves * P::kRowsPerLoad * B.ld_bytes);
  const uint32_t kstA = (uint32_t)A.stage_bytes, kstB = (uint32_t)B.stage_bytes;

  // fragment reads: row (wave origin + 16 i + (lane & 15)), logical chunk 4 ks + (lane >> 4)
  const int frow = lane & 15, fquad = lane >> 4;
  const int fA = (wm * (kTile / kWM) + frow) * ROWB;
  const int fB = kTile * ROWB + (wn * (kTile / kWN) + frow) * ROWB;
  int fswz[P::kKs];
#pragma unroll
  for (int ks = 0; ks < P::kKs; ++ks) fswz[ks] = (((4 * ks + fquad) ^ P::swz(frow)) << 4);

  const int nk = (int)(k_bytes / ROWB);

  auto issue = [&](int stage) {
    lds_t* sa = lds + (stage % NST) * P::kStage + wave * 1024;
    lds_t* sb = sa + kTile * ROWB;
    const uint32_t ka = (uint32_t)stage * kstA, kb = (uint32_t)stage * kstB;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, sa + i * kWaves * 1024, 16,
                                               offA + i * stepA + ka, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, sb + i * kWaves * 1024, 16,
                                               offB + i * stepB + kb, 0, 0, 0);
    }
  };
  auto read_frags = [&](i32x4 (&fa)[kBI], i32x4 (&fb)[kBJ], int stage, int ks) {
    const lds_t* s = lds + (stage % NST) * P::kStage;
#pragma unroll
    for (int i = 0; i < kBI; ++i) fa[i] = lds_read16(s + fA + i * 16 * ROWB + fswz[ks]);
#pragma unroll
    for (int j = 0; j < kBJ; ++j) fb[j] = lds_read16(s + fB + j * 16 * ROWB + fswz[ks]);
  };
  auto mma = [&](const i32x4 (&fa)[kBI], const i32x4 (&fb)[kBJ]) {
#pragma unroll
    for (int i = 0; i < kBI; ++i)
#pragma unroll
      for (int j = 0; j < kBJ; ++j) Mma<T>::run(acc[i][j], fa[i], fb[j]);
  };

  if (nk <= 0) return;
  i32x4 fa0[kBI], fb0[kBJ], fa1[kBI], fb1[kBJ];
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue(s);
  wait_vm<kAhead>();
  pipe_barrier();
  read_frags(fa0, fb0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);

  // sched_barrier(0) pins each phase: the next fragments' LDS reads are issued
  // before the MFMAs that consume the current ones.
  for (int kt = 0; kt < nk; ++kt) {
    issue(kt + NST - 1);
#pragma unroll
    for (int ks = 0; ks < P::kKs; ++ks) {
      i32x4(&cur_a)[kBI] = (ks & 1) ? fa1 : fa0;
      i32x4(&cur_b)[kBJ] = (ks & 1) ? fb1 : fb0;
      i32x4(&nxt_a)[kBI] = (ks & 1) ? fa0 : fa1;
      i32x4(&nxt_b)[kBJ] = (ks & 1) ? fb0 : fb1;
      if (ks + 1 < P::kKs) {
        read_frags(nxt_a, nxt_b, kt, ks + 1);
      } else {
        wait_vm<kAhead>();
        pipe_barrier();
        read_frags(nxt_a, nxt_b, kt + 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mma(cur_a, cur_b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vm<0>();
  pipe_barrier();
}

// Set every accumulator whose wave-local M row (0..127) is >= vlim to -inf.
// Used once per tile, only on the tile holding the vocabulary's ragged end;
// each row mask serves the four column blocks and dies.
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
