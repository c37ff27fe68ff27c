// One 256x256 output tile of C = A . B^T on gfx950 matrix cores.
//
// A [M][K] and B [N][K] are row-major with K contiguous ("NT"): the layout of
// the LM-head weight (vocab rows, hidden contiguous) and of the hidden states
// (token rows, hidden contiguous), and the layout the backward's staging buffers
// are written in.  Accumulation is fp32.
//
//  * 256 threads = 4 waves in a 2x2 grid; each wave owns a 128x128 sub-tile as
//    4x4 blocks of 32x32 MFMA accumulators (256 fp32 per lane).
//  * K advances 128 bytes per stage (64 bf16 or 32 fp32); one stage of A and B is
//    2 x 32 KB of LDS, double buffered (128 KB of the CU's 160 KB).
//  * Global -> LDS through raw buffer loads.  Rows at or beyond the operand's
//    valid row count fall outside the buffer resource and load as zeros, which
//    also keeps padded vocabulary rows from ever being read.
//  * LDS rows are 128 B (8 chunks of 16 B); chunk c of row r is stored at chunk
//    c ^ (r & 7), so both the 16-B writes and the 16-B MFMA fragment reads hit
//    all 32 banks once per 8 lanes.
//  * bf16: v_mfma_f32_32x32x16_bf16, one per 16-B fragment pair.  fp32:
//    v_mfma_f32_32x32x2_f32, four per fragment pair (exact fp32 products).
//
// Accumulator layout (per wave, block (i, j), element e of the 16):
//   row (M) = i*32 + (e >> 2)*8 + (lane >> 5)*4 + (e & 3)
//   col (N) = j*32 + (lane & 31)
// so each lane holds 4 consecutive M indices for one N index per (i, j, e>>2).
#pragma once

#include "device_common.hpp"

namespace gh {

constexpr int kTile = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                     // K bytes per stage per row
constexpr int kStageBytes = 2 * kTile * kRowBytes; // A + B
constexpr int kGemmLds = 2 * kStageBytes;          // double buffered

struct Operand {
  const char* base;   // element (0, 0)
  int64_t ld_bytes;   // bytes between rows (multiple of 16)
  int64_t rows;       // valid rows; rows beyond load as zero
};

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  static __device__ __forceinline__ void run(f32x16& c, i32x4 a, i32x4 b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16& c, i32x4 a, i32x4 b) {
    const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], c, 0, 0, 0);
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Operand& op, int64_t r0) {
  int64_t valid = op.rows - r0;
  valid = valid < 0 ? 0 : (valid > kTile ? kTile : valid);
  return make_rsrc(op.base + r0 * op.ld_bytes, (uint32_t)(valid * op.ld_bytes));
}

// acc[i][j] += A[m0 + wave rows] . B[n0 + wave cols]^T over k_bytes of K.
template <typename T>
__device__ __forceinline__ void gemm_tile(const Operand& A, const Operand& B, int64_t m0,
                                          int64_t n0, int64_t k_bytes, char* lds,
                                          f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(A, m0);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc(B, n0);

  // global loads: thread covers rows (tid >> 3) + 32 i, chunk (tid & 7)
  const int lrow = tid >> 3, lchunk = tid & 7;
  const uint32_t goffA = (uint32_t)(lrow * A.ld_bytes + lchunk * 16);
  const uint32_t goffB = (uint32_t)(lrow * B.ld_bytes + lchunk * 16);
  const uint32_t gstepA = (uint32_t)(32 * A.ld_bytes), gstepB = (uint32_t)(32 * B.ld_bytes);
  const int swz_w = ((lchunk ^ (lrow & 7)) << 4);
  const int lds_w = lrow * kRowBytes + swz_w;    // + i * 32 * kRowBytes

  // fragment reads: row (w*128 + i*32 + (lane & 31)), chunk 2s + (lane >> 5)
  const int frow = lane & 31, fhalf = lane >> 5;
  const int fA = (wm * 128 + frow) * kRowBytes;
  const int fB = kTile * kRowBytes + (wn * 128 + frow) * kRowBytes;
  int fswz[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fswz[s] = (((2 * s + fhalf) ^ (frow & 7)) << 4);

  const int nk = (int)(k_bytes / kRowBytes);
  i32x4 pa[8], pb[8];

  auto gload = [&](int kt) {
    const uint32_t soff = (uint32_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pa[i] = buffer_load16(ra, goffA + i * gstepA, soff);
      pb[i] = buffer_load16(rb, goffB + i * gstepB, soff);
    }
  };
  auto lstore = [&](int stage) {
    char* s = lds + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(i32x4*)(s + lds_w + i * 32 * kRowBytes) = pa[i];
      *(i32x4*)(s + kTile * kRowBytes + lds_w + i * 32 * kRowBytes) = pb[i];
    }
  };
  auto compute = [&](int stage) {
    const char* s = lds + stage * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      i32x4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = *(const i32x4*)(s + fA + i * 32 * kRowBytes + fswz[ks]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = *(const i32x4*)(s + fB + j * 32 * kRowBytes + fswz[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mma<T>::run(acc[i][j], fa[i], fb[j]);
    }
  };

  if (nk <= 0) return;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(cur);
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

}  // namespace gh
