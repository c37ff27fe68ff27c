// Backward: recompute each logit tile, form dlogits, then the two gradient
// products.
//
//   G[t, v] = grad_output * coef_t * (1[v == y_t] - exp(z[t, v] - lse_t)) / tau
// (softmax recovered from the logits and the LSE, RL-Kernel PR #291, review
// thread on the saved fp32 logits; here the logits are recomputed per tile rather
// than saved).  Inactive tokens give 0.
//
// A token whose scale g_t = grad_output * coef_t / tau is zero (an inactive token,
// or a clipped one with no KL term) has an all-zero dlogits row: it adds nothing to
// dW and its dH row is zero.  The backward therefore runs on the chunk's live rows
// only, compacted in token order.  Their count stays on the device: each launch
// reads it and sizes its tile walk or K loop from it, so nothing waits on the host.
//
// Per token chunk, in ascending chunk order:
//   1. live_count_kernel, compact_kernel: the live tokens in ascending order
//      (rows[r] = token, rowpos[t] = r or -1), their (g_t, lse_t log2 e), the count
//   2. gather_rows_kernel : the live H rows, as Hg[r][d] and transposed, HT[d][r]
//      zero_dead_rows_kernel: dH rows of the dead tokens = 0
//   3. dlogits_kernel     : g_t (1[v == y_t] - p_tv) tile on the matrix cores -> dz
//                           (bf16, nearest even, on the bf16 path; fp32 on the fp32
//                           path)
//   4. grad_products_kernel, one launch of two products:
//      dH[rows[r]][d] = sum_v dz[r][v] W[v][d]
//      (M = r: dz K-contiguous; N = d: W read MN-contiguous), and
//      dW[v][d] (+)= sum_r HT[d][r] dz[r][v]
//      (M = d: HT K-contiguous; N = v: dz read MN-contiguous)
// W and dz are read where they are; the tile core forms the transposed MFMA
// fragments of the MN-contiguous operand with the gfx950 transposing LDS read,
// which delivers about half the bandwidth of a plain read, so each product keeps
// exactly one such operand, on the side with the smaller per-wave fragment count.
// dz is stored "v-blocked": [vocabulary / 64][chunk rows][64], so a K stage of the
// dH product (256 rows x 64 vocabulary entries, bf16) is one contiguous 32 KB run,
// and a K stage of the dW product (64 rows x 256 entries) four runs of 8 KB.  (A
// layout blocked by 256, whose dH stages are 256 runs of 128 B, 512 B apart and
// whose dW stages are one 32 KB run, measured 0.07 ms slower in the gradient launch
// and 0.02 ms faster in dlogits.)
#include <type_traits>

#include "gemm_tile.hpp"
#include "launch.hpp"

namespace gh {

__device__ __forceinline__ bool token_is_active(const uint8_t* mask, const int64_t* y,
                                                int64_t ignore_index, int64_t t) {
  return mask ? (mask[t] != 0) : (y[t] != ignore_index);
}

// Output tiles are written with non-temporal stores: a round of tiles writes about
// as many bytes as an XCD's L2 holds, and ordinary stores would evict the operand
// panels that the resident tiles are sharing.
template <typename T> struct Store4;
template <> struct Store4<__bf16> {
  static __device__ __forceinline__ void run(void* p, float a, float b, float c, float d) {
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    __builtin_nontemporal_store(__builtin_bit_cast(i32x2, v), (i32x2*)p);
  }
};
template <> struct Store4<float> {
  static __device__ __forceinline__ void run(void* p, float a, float b, float c, float d) {
    __builtin_nontemporal_store(f32x4{a, b, c, d}, (f32x4*)p);
  }
};

struct DlogitsArgs {
  const void* W; const void* H;   // H: the chunk's live rows (Hg)
  const float2* gl;               // per row: (g_t, lse_t * log2 e); (0, 0) past the live rows
  int64_t chunk_tokens;           // rows of H and gl inside the chunk
  int64_t d_model, v_real;
  float inv_tau;
  void* dz;                       // v-blocked [4 n_vt][dz_rows][64]
  int64_t dz_rows;
  int group_m;
  const int32_t* live;            // live row count (device); token tiles past it are skipped
  const int32_t* ytg;             // [dz_rows] target id of each row, -1 where there is none
  int32_t* queue;                 // [8] tile queues of the chained launch (cleared by the
                                  // compaction)
};

// Row compaction of one chunk (blocks of kCompactBlock tokens, one per thread).
struct CompactArgs {
  const int64_t* y; const uint8_t* mask; int64_t ignore_index;
  const float* coef; const float* lse; const float* grad_output; float inv_tau;
  int64_t n;          // tokens of the chunk
  int64_t n_pad;      // rows of the compact buffers
  int32_t* bcnt;      // [blocks] live tokens per block
  int32_t* live;      // live tokens of the chunk
  int32_t* rows;      // [n_pad] token of compact row r (-1 past the live rows)
  int32_t* rowpos;    // [n] compact row of token t, -1 if dead
  float2* gl;         // [n_pad] (g_t, lse_t log2 e) of compact row r; (0, 0) past them
  int32_t* bbase;     // [blocks] live tokens before each block, or null: each block sums
                      // the counts before it itself (few blocks)
  int64_t v_real;
  int32_t* ytg;       // [n_pad] target id of compact row r if in [0, v_real), else -1
  int32_t* dwq;       // [16] the tile queues of the dlogits launch ([0, 8)) and of the
                      // gradient launch's dW tiles ([8, 16)), cleared here
};

// g_t = grad_output * coef_t / tau for an active token, 0 otherwise.  A token is
// live when g_t != 0 (a NaN scale stays live, so it reaches the gradients).
__device__ __forceinline__ float grad_scale(const CompactArgs& a, int64_t t) {
  const bool act = token_is_active(a.mask, a.y, a.ignore_index, t);
  const float gout = a.grad_output ? *a.grad_output : 1.0f;
  return act ? gout * a.coef[t] * a.inv_tau : 0.0f;
}

constexpr int kCompactWaves = (int)kCompactBlock / 64;

__global__ __launch_bounds__(kCompactBlock) void live_count_kernel(CompactArgs a) {
  __shared__ int wcnt[kCompactWaves];
  const int64_t t = (int64_t)blockIdx.x * kCompactBlock + threadIdx.x;
  const bool lv = t < a.n && grad_scale(a, t) != 0.0f;
  const uint64_t b = __ballot(lv);
  if ((threadIdx.x & 63) == 0) wcnt[threadIdx.x >> 6] = __popcll(b);
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    for (int w = 0; w < kCompactWaves; ++w) c += wcnt[w];
    a.bcnt[blockIdx.x] = c;
  }
}

// Exclusive prefix sums of the per-block live counts, one block: thread i sums
// a contiguous run of counts, then the runs' totals are scanned in LDS.  Used when
// there are many blocks, so compact_kernel's work stays linear in the tokens.
__global__ __launch_bounds__(kCompactBlock) void block_scan_kernel(const int32_t* bcnt, int nb,
                                                                   int32_t* bbase) {
  __shared__ int run[kCompactBlock];
  const int per = (nb + kCompactBlock - 1) / kCompactBlock;
  const int b0 = threadIdx.x * per, b1 = b0 + per < nb ? b0 + per : nb;
  int c = 0;
  for (int b = b0; b < b1; ++b) c += bcnt[b];
  run[threadIdx.x] = c;
  __syncthreads();
  // Hillis-Steele inclusive scan of the run totals
  for (int o = 1; o < kCompactBlock; o <<= 1) {
    const int v = threadIdx.x >= o ? run[threadIdx.x - o] : 0;
    __syncthreads();
    run[threadIdx.x] += v;
    __syncthreads();
  }
  int acc = threadIdx.x > 0 ? run[threadIdx.x - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    bbase[b] = acc;
    acc += bcnt[b];
  }
}

// Each block places its live tokens after those of the blocks before it, in token
// order; the last block also writes the count and clears the rows past it.
__global__ __launch_bounds__(kCompactBlock) void compact_kernel(CompactArgs a) {
  __shared__ int wcnt[kCompactWaves];
  __shared__ int base;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    int c = 0;
    if (a.bbase) {
      c = a.bbase[blockIdx.x];
    } else {
      for (int b = lane; b < (int)blockIdx.x; b += 64) c += a.bcnt[b];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    }
    if (lane == 0) base = c;
  }
  const int64_t t = (int64_t)blockIdx.x * kCompactBlock + threadIdx.x;
  const float g = t < a.n ? grad_scale(a, t) : 0.0f;
  const bool lv = t < a.n && g != 0.0f;
  const uint64_t b = __ballot(lv);
  if (lane == 0) wcnt[wave] = __popcll(b);
  __syncthreads();
  int pos = base;
  for (int w = 0; w < wave; ++w) pos += wcnt[w];
  pos += __popcll(b & ((uint64_t(1) << lane) - 1));
  if (t < a.n) {
    a.rowpos[t] = lv ? pos : -1;
    if (lv) {
      a.rows[pos] = (int32_t)t;
      a.gl[pos] = make_float2(g, a.lse[t] * kLog2e);
      const int64_t yy = a.y[t];   // a live token is active: its target is defined
      a.ytg[pos] = (yy >= 0 && yy < a.v_real) ? (int32_t)yy : -1;
    }
  }
  if (blockIdx.x == gridDim.x - 1) {
    int total = base;
    for (int w = 0; w < kCompactWaves; ++w) total += wcnt[w];
    if (threadIdx.x == 0) *a.live = total;
    if (threadIdx.x < 16) a.dwq[threadIdx.x] = 0;
    for (int64_t r = total + threadIdx.x; r < a.n_pad; r += kCompactBlock) {
      a.rows[r] = -1;
      a.gl[r] = make_float2(0.0f, 0.0f);
      a.ytg[r] = -1;
    }
  }
}

// dz[r][v] = g_r (1[v == y_r] - p_rv) over the tile, for live row r: the target
// element is formed by the one lane that holds it, behind a wave-wide test (a tile
// holds about 256 * 256 / V targets), so the common path is -g p.  On the tile holding the
// vocabulary's ragged end the padded columns v >= v_real are set to -inf before
// the exponential, so their dz is zero: their W rows load as zeros, and a zero
// logit there would otherwise give -g 2^(-lse2), which overflows for a very
// negative LSE and would turn dH into NaN through 0 * inf.  (The padded rows of dW
// are written as zeros whatever dz holds.)  Rows past the live count get g = 0 and
// zero H rows, so their dz is zero.
template <typename T>
__global__ __launch_bounds__(kThreads) void dlogits_kernel(DlogitsArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  // the launch covers every token tile of the chunk; only those holding live rows run
  const int live_n = (int)ceil_div((int64_t)*a.live, kTile);
  if (live_n < tiles_n) tiles_n = live_n;
  const int nwg = tiles_m * tiles_n;
  if ((int)blockIdx.x >= nwg) return;
  int tm, tn;
  tile_coords(blockIdx.x, nwg, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t v0 = (int64_t)tm * kTile, t0 = (int64_t)tn * kTile;
  const int64_t esz = Elem<T>::size;
  const Operand A = nt_row_major(a.W, a.d_model * esz, a.v_real);
  const Operand B = nt_row_major(a.H, a.d_model * esz, a.chunk_tokens);
  f32x4 acc[kBI][kBJ];
  zero_acc(acc);
  gemm_tile<T, false, false>(A, B, v0, t0, (int)(a.d_model * esz / kStageBytes), (lds_t*)lds,
                             acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  if (v0 + kTile > a.v_real) {   // uniform per workgroup: only the ragged vocabulary tile
    const int64_t left = a.v_real - (v0 + wm * (kTile / kWM));
    mask_rows(acc, (int)(left < 0 ? 0 : (left > 128 ? 128 : left)));
  }
  const int vl = wm * (kTile / kWM) + (lane >> 4) * 4;   // tile-local vocabulary row
  const float c2 = a.inv_tau * kLog2e;
  // (g, lse2) of the lane's token columns; tokens past the chunk read zeros
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gl, (uint32_t)(a.chunk_tokens * 8));
  // this tile's part of dz: rows t0 .. t0 + 255 of the 4 vocabulary blocks from
  // v0 / 64, each row's 64 elements of a block one contiguous run
  char* tile = (char*)a.dz + vblocked_offset(t0, v0, a.dz_rows, esz);
  const int64_t block_bytes = a.dz_rows * 64 * esz;   // between 64-element blocks
  // bf16: the block is staged in LDS (now free) and written out as whole rows;
  // 32-byte segment s of LDS row t sits at segment s ^ (t & 15)
  char* L = lds;

  // target id of the lane's row; -1 past the live rows (cleared by the compaction)
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(a.ytg, (uint32_t)(a.dz_rows * 4));
  const int qg = lane >> 4;
  // the tile's elements of column block j; kFix: one lane of the wave holds a
  // target element, rel its row within the wave's 128 rows
  auto column = [&](int j, int tl, float g, float lse2, int32_t rel, bool own, auto fix) {
    constexpr bool kFix = decltype(fix)::value;
    char* rowp = tile + (int64_t)tl * 64 * esz;
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(acc[i][j][e] * c2 - lse2);
        d[e] = -g * p;
        if (kFix) d[e] = (own && rel == i * 16 + qg * 4 + e) ? g * (1.0f - p) : d[e];
      }
      const int v = vl + i * 16;                                 // 4 consecutive v
      if (sizeof(T) == 2) {
        const bf16x4 q = {(__bf16)d[0], (__bf16)d[1], (__bf16)d[2], (__bf16)d[3]};
        const int byte = v * 2;                                  // within the 512-B row
        const int seg = (byte >> 5) ^ (tl & 15);
        *(i32x2*)(L + tl * 512 + seg * 32 + (byte & 31)) = __builtin_bit_cast(i32x2, q);
      } else {
        Store4<T>::run(rowp + (v >> 6) * block_bytes + (v & 63) * esz, d[0], d[1], d[2], d[3]);
      }
    }
  };

#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int tl = wn * (kTile / kWN) + j * 16 + (lane & 15);   // tile-local token
    // (cast the whole vector: clang miscompiles bit_cast of a single vector element)
    const f32x2 glv = __builtin_bit_cast(
        f32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, (uint32_t)((t0 + tl) * 8), 0, 0));
    const float g = glv[0];
    const float lse2 = glv[1];
    const int32_t yt = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ry, (uint32_t)((t0 + tl) * 4),
                                                                    0, 0);
    const int32_t rel = yt - (int32_t)(v0 + wm * (kTile / kWM));
    const bool own = yt >= 0 && (uint32_t)rel < (uint32_t)(kTile / kWM) && ((rel >> 2) & 3) == qg;
    if (__builtin_amdgcn_ballot_w64(own) != 0)
      column(j, tl, g, lse2, rel, own, std::true_type{});
    else
      column(j, tl, g, lse2, rel, own, std::false_type{});
  }
  if (sizeof(T) == 2) {
    __syncthreads();
    // 256 rows x 32 chunks of 16 B: one wave writes two whole rows, each as 4 runs
    // of 128 B (chunks 8 b .. 8 b + 7 go to block b)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = q * kThreads + threadIdx.x;
      const int t = idx >> 5, c = idx & 31;
      const int seg = (c >> 1) ^ (t & 15);
      const i32x4 v = *(const i32x4*)(L + t * 512 + seg * 32 + (c & 1) * 16);
      __builtin_nontemporal_store(
          v, (i32x4*)(tile + (c >> 3) * block_bytes + (int64_t)t * 128 + (c & 7) * 16));
    }
  }
}

// The chained dlogits launch: one workgroup per compute unit, each taking logit
// tiles (of the token tiles holding live rows) from per-XCD queues, with the K
// pipeline running on from one tile into the next (gemm_tile_chain), as the
// forward's tile launch does.  The epilogue runs while the next tile's first loads
// land in the pipeline buffers, so it keeps to the LDS past them:
//  - a tile's per-token values, (g, lse log2 e) then the target id (3 KB), arrive by
//    direct-to-LDS loads that wave 0 issues at the start of the tile before, in three
//    buffers in turn (a wave may still read the previous tile's while wave 0 loads
//    the next one's);
//  - bf16: each wave passes its 128 (vocabulary) x 64 (token) sub-tile through its own
//    2 KB slice, 8 passes of 16 token rows x 64 entries (one v-block), with no
//    workgroup barrier, and writes each row's 64 entries as one 128-byte run; fp32
//    stores straight from the accumulators.
// Each tile's values are those of dlogits_kernel, bit for bit.
constexpr int kDlSlice = 2048;
constexpr int kDlTok = kTile * 12;
constexpr int kDlChainLds = kGemmLds + kWaves * kDlSlice + 3 * kDlTok + 8 * (int)sizeof(int32_t);

template <typename T>
__device__ __forceinline__ void dlogits_epilogue_wave(f32x4 (&acc)[kBI][kBJ],
                                                      const DlogitsArgs& a, int64_t v0,
                                                      int64_t t0, const char* tok,
                                                      lds_t* slice) {
  // (the lane index made opaque, so that nothing derived from it is hoisted out of
  // the tile loop, where it would stay live across the K loop)
  int lane = threadIdx.x & 63;
  __asm__ volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  if (v0 + kTile > a.v_real) {   // uniform per workgroup: only the ragged vocabulary tile
    const int64_t left = a.v_real - (v0 + wm * (kTile / kWM));
    mask_rows(acc, (int)(left < 0 ? 0 : (left > 128 ? 128 : left)));
  }
  const int64_t esz = Elem<T>::size;
  const int64_t block_bytes = a.dz_rows * 64 * esz;   // between 64-element blocks
  const float c2 = a.inv_tau * kLog2e;
  const int qg = lane >> 4;
  const int vl = wm * (kTile / kWM) + qg * 4;         // tile-local vocabulary row
  // this tile's part of dz: rows t0 .. t0 + 255 of the 4 vocabulary blocks from v0 / 64
  char* dzt = (char*)a.dz + vblocked_offset(t0, v0, a.dz_rows, esz);
  const int wr = lane & 15;                           // token row written by this lane
  auto column = [&](int j, int tl, float g, float lse2, int32_t rel, bool own, auto fix) {
    constexpr bool kFix = decltype(fix)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < kBI / 2; ++ii) {
        const int i = h * (kBI / 2) + ii;
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = fast_exp2(acc[i][j][e] * c2 - lse2);
          d[e] = -g * p;
          if (kFix) d[e] = (own && rel == i * 16 + qg * 4 + e) ? g * (1.0f - p) : d[e];
        }
        if (sizeof(T) == 2) {
          // token row wr, entries ii * 16 + qg * 4 .. + 3 of the pass's 64
          const bf16x4 q = {(__bf16)d[0], (__bf16)d[1], (__bf16)d[2], (__bf16)d[3]};
          const int c = ii * 2 + (qg >> 1);
          *(__attribute__((address_space(3))) i32x2*)(
              slice + wr * 128 + ((c ^ ((wr >> 1) & 7)) << 4) + (qg & 1) * 8) =
              __builtin_bit_cast(i32x2, q);
        } else {
          const int v = vl + i * 16;                  // 4 consecutive v
          Store4<T>::run(dzt + (v >> 6) * block_bytes + (int64_t)tl * 64 * esz + (v & 63) * esz,
                         d[0], d[1], d[2], d[3]);
        }
      }
      if (sizeof(T) == 2) {
        lgkm_drain();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int rr = u * 8 + (lane >> 3), c = lane & 7;
          const i32x4 v = *(const __attribute__((address_space(3))) i32x4*)(
              slice + rr * 128 + ((c ^ ((rr >> 1) & 7)) << 4));
          const int64_t t = wn * (kTile / kWN) + j * 16 + rr;   // tile-local token row
          __builtin_nontemporal_store(
              v, (i32x4*)(dzt + (wm * 2 + h) * block_bytes + t * 128 + c * 16));
        }
        lgkm_drain();
      }
    }
  };
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int tl = wn * (kTile / kWN) + j * 16 + wr;      // tile-local token
    const f32x2 glv = *(const __attribute__((address_space(3))) f32x2*)(tok + tl * 8);
    const int32_t yt = *(const __attribute__((address_space(3))) int32_t*)(tok + 2048 + tl * 4);
    const float g = glv[0];
    const float lse2 = glv[1];
    const int32_t rel = yt - (int32_t)(v0 + wm * (kTile / kWM));
    const bool own = yt >= 0 && (uint32_t)rel < (uint32_t)(kTile / kWM) && ((rel >> 2) & 3) == qg;
    if (__builtin_amdgcn_ballot_w64(own) != 0)
      column(j, tl, g, lse2, rel, own, std::true_type{});
    else
      column(j, tl, g, lse2, rel, own, std::false_type{});
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dlogits_chain_kernel(DlogitsArgs a, int tiles_m,
                                                                 int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kDlChainLds];
  const int live_n = (int)ceil_div((int64_t)*a.live, kTile);
  if (live_n < tiles_n) tiles_n = live_n;
  if (tiles_n <= 0) return;
  const int xcd = (int)blockIdx.x & 7;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char* tokbuf = lds + kGemmLds + kWaves * kDlSlice;
  int32_t* ring_m = (int32_t*)(tokbuf + 3 * kDlTok);
  int32_t* ring_n = ring_m + 4;
  lds_t* slice = (lds_t*)(lds + kGemmLds + wave * kDlSlice);
  const int64_t esz = Elem<T>::size;
  const int nk = (int)(a.d_model * esz / kStageBytes);
  const Operand A = nt_row_major(a.W, a.d_model * esz, a.v_real);
  const Operand B = nt_row_major(a.H, a.d_model * esz, a.chunk_tokens);
  // wave 0 loads token tile tn's (g, lse2) (2 KB; rows past the chunk read zeros) and
  // target ids (1 KB) into buffer q
  auto load_tok = [&](int tn, int q) {
    if (wave != 0) return;
    uint32_t ln = threadIdx.x & 63;
    __asm__ volatile("" : "+v"(ln));
    const __amdgpu_buffer_rsrc_t rg = range_rsrc((const char*)a.gl, a.chunk_tokens * 8);
    const __amdgpu_buffer_rsrc_t ry = range_rsrc((const char*)a.ytg, a.dz_rows * 4);
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tokbuf + q * kDlTok));
    const uint32_t r0 = (uint32_t)tn * kTile;
    dma16(rg, r0 * 8 + ln * 16, 0u, dst);
    dma16(rg, r0 * 8 + 1024 + ln * 16, 0u, dst + 1024);
    dma16(ry, r0 * 4 + ln * 16, 0u, dst + 2048);
  };
  if (threadIdx.x == 0)
    for (int q = 0; q < 3; ++q)
      grab_tile(a.queue, xcd, tiles_m, tiles_n, a.group_m, ring_m[q], ring_n[q]);
  __syncthreads();
  int tm = ring_m[0], tn = ring_n[0];
  int tmn = ring_m[1], tnn = ring_n[1];
  if (tm < 0) return;
  load_tok(tn, 0);
  i32x4 fa0[kBI], fb0[kBJ];
  for (int k = 0;; ++k) {
    const bool has_next = tmn >= 0;
    if (has_next) load_tok(tnn, (k + 1) % 3);
    const int64_t v0 = (int64_t)tm * kTile, t0 = (int64_t)tn * kTile;
    f32x4 acc[kBI][kBJ];
    zero_acc(acc);
    gemm_tile_chain<T>(A, B, v0, t0, has_next, (int64_t)tmn * kTile, (int64_t)tnn * kTile, nk,
                       k == 0, (lds_t*)lds, acc, fa0, fb0);
    int am = -1, an = 0;
    if (threadIdx.x == kGrabThread) grab_tile(a.queue, xcd, tiles_m, tiles_n, a.group_m, am, an);
    dlogits_epilogue_wave<T>(acc, a, v0, t0, tokbuf + (k % 3) * kDlTok, slice);
    if (threadIdx.x == kGrabThread) {
      ring_m[(k + 3) & 3] = am;
      ring_n[(k + 3) & 3] = an;
    }
    if (!has_next) break;
    tm = tmn;
    tn = tnn;
    tmn = ring_m[(k + 2) & 3];
    tnn = ring_n[(k + 2) & 3];
  }
}

// Products with a K-contiguous A and an MN-contiguous B.
//   dH: C[m = live row r][n = d] stored row-major at the row's token:
//       out[out_rows[m] * ld_out + n];
//   dW: C[m = d][n = v] stored as out[n * ld_out + m .. + 3].
struct ProductArgs {
  Operand A, B;
  int nk;                         // K stages
  void* out; int64_t ld_out;      // elements (of O) between out rows
  int64_t m_limit;                // M extent written
  int64_t n_limit;                // N extent written
  int64_t zero_from;              // dW rows (N) >= this are written as 0 (padded vocab)
  int accumulate;                 // add to out
  int group_m;
  // live row count (device): dH runs the M tiles holding live rows and writes
  // compact row m to out row out_rows[m]; dW runs the K stages covering them
  const int32_t* live;
  const int32_t* out_rows;
};

// Output element stores: fp32, or bf16 rounded to nearest even.
__device__ __forceinline__ float load_out(const float* p) { return *p; }
__device__ __forceinline__ float load_out(const __bf16* p) { return (float)*p; }
__device__ __forceinline__ void store_out(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_out(__bf16* p, float v) {
  const __bf16 b = (__bf16)v;
  __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, b), (uint16_t*)p);
}
__device__ __forceinline__ f32x4 load_out4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load_out4(const __bf16* p) {
  const bf16x4 b = *(const bf16x4*)p;
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
__device__ __forceinline__ void store_out4(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, (f32x4*)p);
}
__device__ __forceinline__ void store_out4(__bf16* p, f32x4 v) {
  const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  __builtin_nontemporal_store(__builtin_bit_cast(i32x2, b), (i32x2*)p);
}

// LDS of the gradient launch: the K pipeline's buffers, then, for the dW tiles,
// one epilogue slice per wave and a ring of four queued tile ids.
constexpr int kDwSlice = 2048;                        // bytes per wave
constexpr int kDwEpiLds = kWaves * kDwSlice;
constexpr int kGradLds = kGemmLds + kDwEpiLds + 8 * (int)sizeof(int32_t);

__device__ __forceinline__ void lds_store16(lds_t* p, f32x4 v) {
  *(__attribute__((address_space(3))) f32x4*)p = v;
}
__device__ __forceinline__ f32x4 lds_load16(const lds_t* p) {
  return *(const __attribute__((address_space(3))) f32x4*)p;
}

// Four output elements at byte offset off of a buffer resource (fp32, or bf16
// rounded to nearest even); offsets past the resource's range load zeros and
// store nothing.
__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off, float*) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off, __bf16*) {
  const bf16x4 b = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}
// cache policy 2: non-temporal (see Store4)
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v,
                                           float*) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 2);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v,
                                           __bf16*) {
  const bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), r, off, 0, 2);
}

// One dW tile's output, rows n0 .. n0 + 255 of out (vocabulary), columns
// m0 .. m0 + 255 (hidden), written while the next tile's loads are in flight: each
// wave passes its 128 (hidden) x 64 (vocabulary) sub-tile through its own 2 KB
// slice of LDS past the pipeline buffers, 16 passes of 16 rows x 32 columns, with
// no workgroup barrier, and writes each row's 32 columns as one 128-byte run (fp32).
// Rows >= zero_from are written as zeros; with accumulate the tile is added to
// what out holds.  Rows >= n_limit and columns >= m_limit lie outside the stores'
// buffer range and are dropped, so every wave issues the same stores.  In a slice,
// 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7), so both the writes
// (16 rows at one chunk) and the reads (8 whole rows) are free of bank conflicts.
template <typename O>
__device__ __forceinline__ void store_dw_tile_wave(const f32x4 (&acc)[kBI][kBJ], lds_t* slice,
                                                   O* out, int64_t ld_out, int64_t n0,
                                                   int64_t m0, int64_t n_limit, int64_t m_limit,
                                                   int64_t zero_from, int accumulate) {
  // (the lane index made opaque, so that nothing derived from it is hoisted out of
  // the caller's tile loop, where it would stay live across the K loop)
  int lane = threadIdx.x & 63;
  __asm__ volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  int64_t rows = n_limit - n0;
  rows = rows < 0 ? 0 : (rows > kTile ? kTile : rows);
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(out + n0 * ld_out, (uint32_t)(rows * ld_out * (int64_t)sizeof(O)));
  const int wr = lane & 15;                 // row written by this lane
  const int rq = lane >> 4;                 // its 4-column group within a block
  const int rc = lane & 7;                  // chunk read by this lane
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
#pragma unroll
    for (int g = 0; g < kBI / 2; ++g) {     // hidden columns g * 32 .. + 31 of the wave's 128
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = u * 4 + rq;
        lds_store16(slice + wr * 128 + ((c ^ ((wr >> 1) & 7)) << 4), acc[2 * g + u][j]);
      }
      lgkm_drain();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rr = u * 8 + (lane >> 3);
        f32x4 v = lds_load16(slice + rr * 128 + ((rc ^ ((rr >> 1) & 7)) << 4));
        const int64_t nl = wn * (kTile / kWN) + j * 16 + rr;      // tile-local row
        const int64_t m = m0 + wm * (kTile / kWM) + g * 32 + rc * 4;
        const uint32_t off =
            m < m_limit ? (uint32_t)((nl * ld_out + m) * (int64_t)sizeof(O)) : 0xFFFFFFF0u;
        if (n0 + nl >= zero_from) v = f32x4{0.f, 0.f, 0.f, 0.f};
        else if (accumulate) v += buf_load4(r, off, (O*)nullptr);
        buf_store4(r, off, v, (O*)nullptr);
      }
    }
  }
}

// One dH tile: workgroup `bid` of the launch's first ones, over the M tiles that
// hold live rows (the rest let go).  C[m = live row r][n = d] goes to
// out[out_rows[m] * ld_out + n].
template <typename T, typename O>
__device__ __forceinline__ void dh_tile(const ProductArgs& a, int bid, int tiles_m, int tiles_n,
                                        char* lds) {
  const int64_t na = *a.live;
  int64_t m_limit = a.m_limit;
  const int live_m = (int)ceil_div(na, kTile);
  if (live_m < tiles_m) tiles_m = live_m;
  const int nwg = tiles_m * tiles_n;
  if (bid >= nwg) return;
  if (na < m_limit) m_limit = na;
  int tm, tn;
  tile_coords(bid, nwg, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
  f32x4 acc[kBI][kBJ];
  zero_acc(acc);
  if constexpr (sizeof(T) == 2) {
    // the chained core of the dW tiles (its stage streams and one asm block per
    // operand's stage loads) also runs dH faster than gemm_tile: 14.46 -> 14.36 ms
    // for the gradient launch (three alternating pairs).  The fp32 dz blocks hold two
    // stages each, which that core's fixed stage stride does not cover.
    i32x4 fa0[kBI], fb0[kBJ];
    gemm_tile_chain_mn<T, false>(a.A, a.B, m0, n0, false, m0, n0, a.nk, true, (lds_t*)lds,
                                 acc, fa0, fb0);
  } else {
    gemm_tile<T, false, true>(a.A, a.B, m0, n0, a.nk, (lds_t*)lds, acc);
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t mbase = m0 + wm * (kTile / kWM) + (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int64_t n = n0 + wn * (kTile / kWN) + j * 16 + (lane & 15);
    if (n >= a.n_limit) continue;
    // 4 consecutive rows m, one column n: a 64-byte run per row across 16 lanes
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      const int64_t m = mbase + i * 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (m + e >= m_limit) continue;
        const int64_t row = a.out_rows[m + e];
        if (row < 0) continue;
        O* p = (O*)a.out + row * a.ld_out + n;
        const float v = a.accumulate ? acc[i][j][e] + load_out(p) : acc[i][j][e];
        store_out(p, v);
      }
    }
  }
}

// The dW tiles, C[m = d][n = v] = sum over the live rows r of HT[d][r] dz[r][v],
// stored as out[n * ld_out + m]: each of a fixed number of workgroups takes tiles
// from the queues until none is left, with the K pipeline running on from one
// tile into the next (gemm_tile_chain_mn), so a tile's epilogue overlaps the next
// tile's first loads.
// The K loop runs over the stages covering the live rows, rounded up to an even
// count (the rows past the live count up to the next 256 are zero in both
// operands).
//
// Thread 0 takes each tile three tiles ahead, during the current tile's epilogue,
// and puts its coordinates in a ring of four LDS slots at the epilogue's end; the
// other waves read them after the next tile's K-loop barriers, so no tile waits
// on a queue access or on an extra barrier.  Every workgroup stops after the
// first empty slot, having issued the same barriers in every wave.
template <typename T, typename O>
__device__ __forceinline__ void dw_tiles(const ProductArgs& a, int32_t* queue, int tiles_m,
                                         int tiles_n, char* lds) {
  const int xcd = (int)blockIdx.x & 7;
  const int wave = threadIdx.x >> 6;
  int32_t* ring_m = (int32_t*)(lds + kGemmLds + kDwEpiLds);
  int32_t* ring_n = ring_m + 4;
  lds_t* slice = (lds_t*)(lds + kGemmLds + wave * kDwSlice);
  const int64_t na = *a.live;

  if (na == 0) {
    // no live row: every tile is zeros (added to out when accumulating)
    f32x4 acc[kBI][kBJ];
    zero_acc(acc);
    for (;;) {
      if (threadIdx.x == 0) grab_tile(queue, xcd, tiles_m, tiles_n, a.group_m, ring_m[0], ring_n[0]);
      __syncthreads();
      const int tm = ring_m[0], tn = ring_n[0];
      __syncthreads();
      if (tm < 0) return;
      store_dw_tile_wave<O>(acc, slice, (O*)a.out, a.ld_out, (int64_t)tn * kTile,
                            (int64_t)tm * kTile, a.n_limit, a.m_limit, a.zero_from,
                            a.accumulate);
    }
  }
  int nk = (int)ceil_div(na * (int64_t)sizeof(T), kStageBytes);
  if (nk > a.nk) nk = a.nk;
  nk += nk & 1;   // a.nk is even (the rows are padded to 256)

  if (threadIdx.x == 0)
    for (int q = 0; q < 3; ++q) grab_tile(queue, xcd, tiles_m, tiles_n, a.group_m, ring_m[q], ring_n[q]);
  __syncthreads();
  int tm = ring_m[0], tn = ring_n[0];
  int tmn = ring_m[1], tnn = ring_n[1];
  if (tm < 0) return;
  i32x4 fa0[kBI], fb0[kBJ];
  for (int k = 0;; ++k) {
    const bool has_next = tmn >= 0;
    const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
    f32x4 acc[kBI][kBJ];
    zero_acc(acc);
    gemm_tile_chain_mn<T>(a.A, a.B, m0, n0, has_next, (int64_t)tmn * kTile,
                          (int64_t)tnn * kTile, nk, k == 0, (lds_t*)lds, acc, fa0, fb0);
    // (taken before the epilogue's stores, so waiting for it waits for nothing that
    // the next tile's first K stage does not wait for anyway)
    int am = -1, an = 0;
    if (threadIdx.x == 0) grab_tile(queue, xcd, tiles_m, tiles_n, a.group_m, am, an);
    store_dw_tile_wave<O>(acc, slice, (O*)a.out, a.ld_out, n0, m0, a.n_limit, a.m_limit,
                          a.zero_from, a.accumulate);
    if (threadIdx.x == 0) {
      ring_m[(k + 3) & 3] = am;
      ring_n[(k + 3) & 3] = an;
    }
    if (!has_next) break;
    tm = tmn;
    tn = tnn;
    tmn = ring_m[(k + 2) & 3];
    tnn = ring_n[(k + 2) & 3];
  }
}

// dH and dW in one launch.  Workgroups [0, dh_slots) take dH tiles (long: K runs
// over the vocabulary), one each; the rest (one per compute unit) take the dW
// tiles (short: K runs over the live rows) from the queues.  The dH workgroups
// are dispatched first, and the dW workgroups start on the compute units that the
// last partial round of dH tiles leaves idle, the others as the dH tiles finish.
// dh_slots is a multiple of 8, so a dW workgroup's XCD is still its index modulo 8.
template <typename T, typename O>
__global__ __launch_bounds__(kThreads) void grad_products_kernel(ProductArgs dh, ProductArgs dw,
                                                                 int32_t* queue, int dh_slots,
                                                                 int dh_tiles_m, int dh_tiles_n,
                                                                 int dw_tiles_m, int dw_tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGradLds];
  const int bid = (int)blockIdx.x;
  if (bid < dh_slots)
    dh_tile<T, O>(dh, bid, dh_tiles_m, dh_tiles_n, lds);
  else
    dw_tiles<T, O>(dw, queue, dw_tiles_m, dw_tiles_n, lds);
}

// The chunk's live H rows, Hg[r][d] = H[rows[r]][d], and their transpose
// HT[d][r], row-major with ht_pitch elements per row (the dW operand, read
// K-contiguous: a K stage of 256 hidden rows is 256 runs of 128 bytes one row
// apart, which measured about 1% faster in the gradient launch than a layout
// blocked by 64 rows with each stage one contiguous 32 KB run); zero for rows[r]
// past the live count.  Only the rows the products read are written: those of
// token tiles holding live rows.  Tiles of 64 rows x 64 elements (d_model is a
// multiple of 64): 16-byte loads and stores, the transpose through LDS.
template <typename E>
__global__ __launch_bounds__(256) void gather_rows_kernel(const E* __restrict__ H,
                                                          int64_t d_model,
                                                          const int32_t* __restrict__ rows,
                                                          const int32_t* live, E* __restrict__ Hg,
                                                          E* __restrict__ HT, int64_t ht_pitch,
                                                          int tiles_d) {
  constexpr int kV = 16 / (int)sizeof(E);        // elements per 16-byte vector
  constexpr int kVecs = 64 / kV;                 // vectors per 64-element row
  constexpr int kPass = 256 / kVecs;             // rows (or columns) per pass
  struct Vec { E e[kV]; };
  __shared__ __attribute__((aligned(16))) E tile[64][64 + kV];   // 16-byte aligned rows
  const int64_t td = blockIdx.x % tiles_d, tr = blockIdx.x / tiles_d;
  const int64_t d0 = td * 64, r0 = tr * 64;
  const int64_t na = *live;
  if (r0 >= ceil_div(na, kTile) * kTile) return;
  const int c = threadIdx.x % kVecs, q = threadIdx.x / kVecs;
  for (int k = q; k < 64; k += kPass) {
    const int64_t r = r0 + k, d = d0 + c * kV;
    const int64_t src = r < na ? rows[r] : -1;
    i32x4 v = {0, 0, 0, 0};
    if (src >= 0) v = *(const i32x4*)(H + src * d_model + d);
    *(i32x4*)(Hg + r * d_model + d) = v;
    *(i32x4*)&tile[k][c * kV] = v;
  }
  __syncthreads();
  // column k of the tile: rows c kV .. c kV + kV - 1 as one vector of HT row d0 + k
  E* blk = HT + d0 * ht_pitch + r0;
  for (int k = q; k < 64; k += kPass) {
    Vec out;
#pragma unroll
    for (int u = 0; u < kV; ++u) out.e[u] = tile[c * kV + u][k];
    *(i32x4*)(blk + k * ht_pitch + c * kV) = __builtin_bit_cast(i32x4, out);
  }
}

// dH rows of the chunk's dead tokens are zero (no product tile reaches them).
// One wave per token.
template <typename O>
__global__ __launch_bounds__(256) void zero_dead_rows_kernel(const int32_t* __restrict__ rowpos,
                                                             int64_t n, int64_t d_model,
                                                             O* __restrict__ dH) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n || rowpos[t] >= 0) return;
  O* row = dH + t * d_model;
  for (int64_t d = threadIdx.x & 63; d < d_model; d += 64) row[d] = (O)0.0f;
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  int64_t blocks = ceil_div(words, 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p,
                     words);
  return hipGetLastError();
}

template <typename T, typename O>
static hipError_t run_bwd(const BwdArgs& a, hipStream_t s) {
  const WsLayout& L = *a.L;
  const int64_t esz = sizeof(T);
  const int64_t N = a.n_tokens, D = a.d_model, VK = L.v_k, R = L.chunk;
  char* dz = a.ws + L.dz;
  char* ht = a.ws + L.ht;
  float2* gl = (float2*)(a.ws + L.gl);

  O* dW = (O*)a.dW;
  O* dH = (O*)a.dH;
  // padded vocabulary rows of dW that no tile reaches (left alone when accumulating)
  if (a.v_rows > VK && !a.accumulate_dw) {
    hipError_t e = launch_fill_zero(dW + VK * D, (size_t)(a.v_rows - VK) * D * sizeof(O), s);
    if (e != hipSuccess) return e;
  }
  if (N == 0) {
    if (a.accumulate_dw) return hipSuccess;
    return launch_fill_zero(dW, (size_t)(a.v_rows < VK ? a.v_rows : VK) * D * sizeof(O), s);
  }
  const StageEvents& ev = *a.marks;

  const int tiles_v = (int)L.n_vt;
  const int tiles_d = (int)ceil_div(D, kTile);
  int32_t* bcnt = (int32_t*)(a.ws + L.bcnt);
  int32_t* live = (int32_t*)(a.ws + L.live);
  int32_t* rows = (int32_t*)(a.ws + L.rows);
  int32_t* rowpos = (int32_t*)(a.ws + L.rowpos);
  char* hg = a.ws + L.hg;
  typedef typename std::conditional<sizeof(T) == 2, uint16_t, float>::type E;
  for (int64_t c0 = 0; c0 < N; c0 += R) {
    const int64_t nc = (N - c0) < R ? (N - c0) : R;
    const int64_t ncp = ceil_div(nc, kTokenTile) * kTokenTile;
    const int tiles_t = (int)(ncp / kTokenTile);
    const char* Hc = (const char*)a.H + c0 * D * esz;
    const uint8_t* cmask = a.mask ? a.mask + c0 : nullptr;

    // live rows of the chunk, their H rows, and zero dH rows for the dead tokens
    const unsigned nb = (unsigned)ceil_div(nc, kCompactBlock);
    // up to 64 blocks each block sums the counts before it in one pass of a wave;
    // beyond that a scan kernel forms the block offsets first
    int32_t* bbase = nb > 64 ? bcnt + nb : nullptr;
    int32_t* ytg = (int32_t*)(a.ws + L.ytg);
    int32_t* dwq = (int32_t*)(a.ws + L.dwq);
    const CompactArgs ca{a.y + c0, cmask, a.ignore_index, a.coef + c0, a.lse + c0, a.grad_output,
                         a.inv_tau, nc, ncp, bcnt, live, rows, rowpos, gl, bbase, a.v_real, ytg,
                         dwq};
    hipLaunchKernelGGL(live_count_kernel, dim3(nb), dim3(kCompactBlock), 0, s, ca);
    if (bbase)
      hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(kCompactBlock), 0, s,
                         (const int32_t*)bcnt, (int)nb, bbase);
    hipLaunchKernelGGL(compact_kernel, dim3(nb), dim3(kCompactBlock), 0, s, ca);
    const int ttd = (int)ceil_div(D, 64);
    hipLaunchKernelGGL(gather_rows_kernel<E>, dim3((unsigned)(ttd * (ncp / 64))), dim3(256), 0, s,
                       (const E*)Hc, D, (const int32_t*)rows, (const int32_t*)live, (E*)hg,
                       (E*)ht, R, ttd);
    hipLaunchKernelGGL(zero_dead_rows_kernel<O>, dim3((unsigned)ceil_div(nc, 4)), dim3(256), 0, s,
                       (const int32_t*)rowpos, nc, D, dH + c0 * D);

    DlogitsArgs d{a.W, hg, gl, nc, D, a.v_real, a.inv_tau, dz, R, a.group_dlogits, live, ytg,
                  dwq};
    const int dl_nk = (int)(D * esz / kStageBytes);
    const int cus = chain_workgroups();
    ev.mark(5, s);
    if (dl_nk % 2 == 0 && cus >= 8) {
      const int tiles = tiles_v * tiles_t;
      const int dl_wgs = tiles < cus ? (int)ceil_div(tiles, 8) * 8 : cus;
      hipLaunchKernelGGL(dlogits_chain_kernel<T>, dim3(dl_wgs), dim3(kThreads), 0, s, d, tiles_v,
                         tiles_t);
    } else {
      hipLaunchKernelGGL(dlogits_kernel<T>, dim3(tiles_v * tiles_t), dim3(kThreads), 0, s, d,
                         tiles_v, tiles_t);
    }
    ev.mark(6, s);

    // dH rows of the chunk: M = live row r (dz rows), N = d (W read MN-contiguous),
    // K = v; row r goes to token rows[r].  W rows >= v_real are never read (they
    // load as zeros).
    ProductArgs ph{nt_vblocked(dz, R, esz, (int64_t)tiles_v * R * 256 * esz),
                   mn_row_major(a.W, D * esz, a.v_real, D, esz), (int)(VK * esz / kStageBytes),
                   dH + c0 * D, D, nc, D, INT64_MAX, 0, a.group_dh, live, rows};

    // dW: M = d (HT K-contiguous), N = v (dz read MN-contiguous), K = live row.
    // Rows [v_real, VK) of the last tile are written as zeros, or, when
    // accumulating into the caller's dW, not written at all.
    ProductArgs pw{nt_row_major(ht, R * esz, D), mn_vblocked(dz, R, esz, 4 * tiles_v),
                   (int)(ncp * esz / kStageBytes), dW, D, D,
                   a.accumulate_dw ? a.v_real : (a.v_rows < VK ? a.v_rows : VK), a.v_real,
                   (c0 > 0 || a.accumulate_dw) ? 1 : 0, a.group_dw, live, nullptr};
    const int dh_slots = (int)ceil_div((int64_t)tiles_t * tiles_d, 8) * 8;
    const int dw_tiles = tiles_d * tiles_v;
    int dw_wgs = chain_workgroups();
    if (dw_wgs < 8) dw_wgs = 8;
    if (dw_wgs > dw_tiles) dw_wgs = (int)ceil_div(dw_tiles, 8) * 8;
    hipLaunchKernelGGL((grad_products_kernel<T, O>), dim3(dh_slots + dw_wgs), dim3(kThreads), 0,
                       s, ph, pw, dwq + 8, dh_slots, tiles_t, tiles_d, tiles_d, tiles_v);
    ev.mark(7, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t s) {
  if (a.grad_bf16) return dtype == 0 ? run_bwd<__bf16, __bf16>(a, s) : run_bwd<float, __bf16>(a, s);
  return dtype == 0 ? run_bwd<__bf16, float>(a, s) : run_bwd<float, float>(a, s);
}

}  // namespace gh
