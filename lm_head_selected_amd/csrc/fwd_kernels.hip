// Forward: vocabulary-tile logits -> per-tile (max, sumexp) partials -> merge.
//
// Tile-streamed selected-token log-prob (Liger-Kernel PR #1160, Summary): each
// workgroup computes one 256-vocab x 256-token logit tile on the matrix cores
// and reduces it to one (max, sumexp) partial per token; the [N, V] logits never
// leave registers.  Padded columns (vocab >= v_real) are -inf before the partial
// is formed, and the merge folds the partials in ascending tile order starting
// from the identity (-inf, 0) (RL-Kernel PR #291, commit notes: ShardingSpec,
// ReductionSpec): ascending within 8 consecutive runs of tiles, then the runs in
// ascending order.  Partials are kept in base-2 units: m2 = max z*log2(e) and
// s = sum 2^(z*log2(e) - m2), so every exponential is one v_exp_f32.
//
// The target logit z[t, y_t] is gathered by target_logit_kernel, one wave per
// token (a length-D dot product), rather than picked out of the tile: keeping the
// tile epilogue free of per-lane selects and branches keeps the 256 accumulators
// in registers.  Only the tile that holds the vocabulary's ragged end runs the
// masking variant of the tile kernel.
#include "gemm_tile.hpp"
#include "launch.hpp"

namespace gh {

__device__ __forceinline__ bool token_active(const uint8_t* mask, const int64_t* y,
                                             int64_t ignore_index, int64_t t) {
  return mask ? (mask[t] != 0) : (y[t] != ignore_index);
}

// The (max, sumexp) partial of every token column of a finished logit tile
// (vocabulary rows v0 .. v0 + 255, tokens t0 .. t0 + 255) in base-2 units.  The
// tile holding the vocabulary's ragged end first masks its rows >= v_real
// (padding: their W rows loaded as zeros) to -inf; the branch is uniform per
// workgroup.  half_stats is 4 KB of LDS for the two 128-row halves.  kChained:
// the next tile's loads are in flight, so the barrier waits on LDS only.
template <bool kChained>
__device__ __forceinline__ void tile_partials(f32x4 (&acc)[kBI][kBJ], const FwdTileArgs& a,
                                              int tm, int64_t v0, int64_t t0,
                                              float2 (*half_stats)[kTile]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const float c2 = a.inv_tau * kLog2e;
  if (v0 + kTile > a.v_real) {
    const int64_t left = a.v_real - (v0 + wm * 128);
    mask_rows(acc, (int)(left < 0 ? 0 : (left > 128 ? 128 : left)));
  }

  // column block j: token tl; the four 16-lane groups hold different rows of it
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int tl = wn * (kTile / kWN) + j * 16 + (lane & 15);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kBI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, acc[i][j][e]);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    // the maximum of the raw logits, scaled once: scaling by c2 > 0 keeps the order,
    // so this is the maximum of the scaled logits, and each exponent argument is one
    // fma (z * c2 - m2) rather than a multiply and a subtraction
    const float m2 = m * c2;
    float s = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kBI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += fast_exp2(__builtin_fmaf(acc[i][j][e], c2, -m2));
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    // all four lane groups hold the same (m, s); all write it
    half_stats[wm][tl] = make_float2(m2, s);
  }
  if (kChained) pipe_barrier();
  else __syncthreads();

  // merge the two 128-row halves (wave rows 0 then 1) and write the tile partial
  const int tl = threadIdx.x;
  const int64_t t = t0 + tl;
  if (tl < kTile && t < a.n_tokens) {
    const float2 p0 = half_stats[0][tl], p1 = half_stats[1][tl];
    float M, S;
    if (p1.x == -INFINITY) { M = p0.x; S = p0.y; }
    else if (p0.x == -INFINITY) { M = p1.x; S = p1.y; }
    else {
      M = fmaxf(p0.x, p1.x);
      S = p0.y * fast_exp2(p0.x - M) + p1.y * fast_exp2(p1.x - M);
    }
    a.partials[(int64_t)tm * a.n_tokens + t] = make_float2(M, S);
  }
}

// One workgroup per logit tile.
template <typename T>
__global__ __launch_bounds__(kThreads) void fwd_tile_kernel(FwdTileArgs a, int tiles_m,
                                                            int tiles_n) {
  // One LDS object only: with a second __shared__ array the compiler can no longer
  // tell the direct-to-LDS loads from the fragment reads and waits for every load
  // right after issuing it.  The per-half row statistics reuse the pipeline's
  // buffers once the K loop has drained.
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  static_assert(sizeof(float2) * 2 * kTile <= kGemmLds, "row statistics fit in LDS");

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t v0 = (int64_t)tm * kTile;   // vocabulary rows of this tile
  const int64_t t0 = (int64_t)tn * kTile;   // tokens of this tile
  const int64_t esz = Elem<T>::size;

  const Operand A = nt_row_major(a.W, a.d_model * esz, a.v_real);
  const Operand B = nt_row_major(a.H, a.d_model * esz, a.n_tokens);
  f32x4 acc[kBI][kBJ];
  zero_acc(acc);
  gemm_tile<T, false, false>(A, B, v0, t0, (int)(a.d_model * esz / kStageBytes), (lds_t*)lds,
                             acc);
  tile_partials<false>(acc, a, tm, v0, t0, (float2(*)[kTile])lds);
}

// A fixed number of workgroups (one per compute unit, a multiple of 8), each
// computing a sequence of logit tiles with the K pipeline running on from one
// tile into the next (gemm_tile_chain), so a tile's epilogue overlaps the next
// tile's first loads.  Workgroup b sits on XCD b % 8 and works through that XCD's
// run of logical tile ids (the runs tile_coords gives the XCDs), so the tiles
// resident together on an XCD are the same as with one workgroup per tile.
// kQueue: the workgroups take the ids from per-XCD queues (grab_tile), and an XCD
// that empties its run takes ids from the others' runs, which balances XCDs that
// run at different clocks (a few percent apart); one thread takes each id three
// tiles ahead and passes it on through a ring of four LDS slots, as the dW tiles
// of the backward do (here the thread is in wave 4, which issues no loads, so
// waiting for the queue access does not wait for the next tile's loads).  Without kQueue (no queue memory: the vocabulary-shard
// entry) workgroup b takes every (per-XCD count)-th id of its run from b / 8 on.
// Needs an even number of K stages.
template <typename T, bool kQueue>
__global__ __launch_bounds__(kThreads) void fwd_tile_chain_kernel(FwdTileArgs a, int tiles_m,
                                                                  int tiles_n, int32_t* queue) {
  // pipeline buffers, then the per-half row statistics, then the ring of queued
  // tiles (one LDS object: see above)
  constexpr int kStats = 2 * kTile * (int)sizeof(float2);
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds + kStats + (kQueue ? 32 : 0)];
  const int64_t esz = Elem<T>::size;
  const int nk = (int)(a.d_model * esz / kStageBytes);
  const Operand A = nt_row_major(a.W, a.d_model * esz, a.v_real);
  const Operand B = nt_row_major(a.H, a.d_model * esz, a.n_tokens);
  float2(*half_stats)[kTile] = (float2(*)[kTile])(lds + kGemmLds);
  i32x4 fa0[kBI], fb0[kBJ];
  if constexpr (kQueue) {
    const int xcd = (int)blockIdx.x & 7;
    int32_t* ring_m = (int32_t*)(lds + kGemmLds + kStats);
    int32_t* ring_n = ring_m + 4;
    if (threadIdx.x == 0)
      for (int q = 0; q < 3; ++q)
        grab_tile(queue, xcd, tiles_m, tiles_n, a.group_m, ring_m[q], ring_n[q]);
    __syncthreads();
    int tm = ring_m[0], tn = ring_n[0];
    int tmn = ring_m[1], tnn = ring_n[1];
    if (tm < 0) return;
    for (int k = 0;; ++k) {
      const bool has_next = tmn >= 0;
      const int64_t v0 = (int64_t)tm * kTile, t0 = (int64_t)tn * kTile;
      f32x4 acc[kBI][kBJ];
      zero_acc(acc);
      gemm_tile_chain<T>(A, B, v0, t0, has_next, (int64_t)tmn * kTile, (int64_t)tnn * kTile,
                         nk, k == 0, (lds_t*)lds, acc, fa0, fb0);
      int am = -1, an = 0;
      if (threadIdx.x == kGrabThread) grab_tile(queue, xcd, tiles_m, tiles_n, a.group_m, am, an);
      tile_partials<true>(acc, a, tm, v0, t0, half_stats);
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
  } else {
    const int per_xcd = (int)gridDim.x >> 3;
    int start, len;
    xcd_run((int)blockIdx.x & 7, tiles_m * tiles_n, start, len);
    int id = (int)blockIdx.x >> 3;
    if (id >= len) return;
    int tm, tn;
    logical_coords(start + id, tiles_m, tiles_n, a.group_m, tm, tn);
    for (bool first = true; id < len; first = false) {
      const int nid = id + per_xcd;
      const bool has_next = nid < len;
      int tmn = tm, tnn = tn;
      if (has_next) logical_coords(start + nid, tiles_m, tiles_n, a.group_m, tmn, tnn);
      const int64_t v0 = (int64_t)tm * kTile, t0 = (int64_t)tn * kTile;
      f32x4 acc[kBI][kBJ];
      zero_acc(acc);
      gemm_tile_chain<T>(A, B, v0, t0, has_next, (int64_t)tmn * kTile, (int64_t)tnn * kTile,
                         nk, first, (lds_t*)lds, acc, fa0, fb0);
      tile_partials<true>(acc, a, tm, v0, t0, half_stats);
      id = nid;
      tm = tmn;
      tn = tnn;
    }
  }
}

// Clears the tile queues of a persistent launch (8 counters).
__global__ void clear_queue_kernel(int32_t* queue) {
  if (threadIdx.x < 8) queue[threadIdx.x] = 0;
}

// One wave per token: z[t, y_t] * inv_tau = inv_tau * sum_d H[t, d] W[y_t, d] for
// an active token with a target in [0, v_real) (fp32 products and sums; bf16
// products are exact in fp32), written to zy[t] (mode 0), or for a vocabulary
// shard (mode 2) zy[t] for every token, 0 when the target lies elsewhere.
template <typename T>
__global__ __launch_bounds__(256) void target_logit_kernel(TargetArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.n_tokens) return;
  const bool act = token_active(a.mask, a.y, a.ignore_index, t);
  const int64_t yy = act ? a.y[t] : -1;
  const int64_t yl = yy - a.v_begin;                 // row within this W
  if (!act || yl < 0 || yl >= a.v_real) {
    if (a.mode == 2 && lane == 0) a.zy[t] = 0.0f;    // not this shard's target
    return;
  }
  constexpr int kPer = 16 / (int)sizeof(T);          // elements per 16-byte chunk
  const T* h = (const T*)a.H + t * a.d_model;
  const T* w = (const T*)a.W + yl * a.d_model;
  float acc = 0.0f;
  for (int64_t d0 = (int64_t)lane * kPer; d0 < a.d_model; d0 += 64 * kPer) {
    const i32x4 hv = *(const i32x4*)(h + d0);
    const i32x4 wv = *(const i32x4*)(w + d0);
    if (sizeof(T) == 2) {
      const u32x4 hw = __builtin_bit_cast(u32x4, hv), ww = __builtin_bit_cast(u32x4, wv);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t hu = hw[k], wu = ww[k];
        acc = fmaf(__builtin_bit_cast(float, hu << 16), __builtin_bit_cast(float, wu << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, hu & 0xffff0000u),
                   __builtin_bit_cast(float, wu & 0xffff0000u), acc);
      }
    } else {
      // cast whole vectors: clang miscompiles bit_cast of a single vector element
      const f32x4 hf = __builtin_bit_cast(f32x4, hv), wf = __builtin_bit_cast(f32x4, wv);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc = fmaf(hf[k], wf[k], acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane != 0) return;
  a.zy[t] = acc * a.inv_tau;
}

// (M, S) <- (M, S) (+) (m, s): the merge of two (max, sumexp) partials in base-2
// units; (-inf, 0) is the identity.
__device__ __forceinline__ void fold(float& M, float& S, float m, float s) {
  if (m == -INFINITY) return;                 // identity partial
  if (m > M) {
    S = S * fast_exp2(M - m) + s;             // M = -inf on the first real partial: S * 0
    M = m;
  } else {
    S = S + s * fast_exp2(m - M);
  }
}

// Fixed-order merge of the n_vt partials of each token.  A block serves 32 tokens
// with 8 threads each: thread g folds the tiles of the g-th of 8 consecutive runs
// in ascending order, then one thread per token folds the 8 run results in
// ascending order.  The order is fixed, so results are bitwise repeatable.
constexpr int kMergeTokens = 32, kMergeRuns = 8;
__global__ __launch_bounds__(kMergeTokens * kMergeRuns) void merge_kernel(MergeArgs a) {
  __shared__ float2 run_ms[kMergeRuns][kMergeTokens];
  const int tl = threadIdx.x % kMergeTokens, g = threadIdx.x / kMergeTokens;
  const int64_t t = (int64_t)blockIdx.x * kMergeTokens + tl;
  const int64_t per = (a.n_vt + kMergeRuns - 1) / kMergeRuns;
  const int64_t k0 = g * per, k1 = (k0 + per < a.n_vt) ? k0 + per : a.n_vt;
  float M = -INFINITY, S = 0.0f;
  if (t < a.n_tokens) {
    // loads in batches of 8 (all in flight together), folded in ascending order
    const float2* p = a.partials + t;
    constexpr int kBatch = 8;
    int64_t k = k0;
    for (; k + kBatch <= k1; k += kBatch) {
      float2 q[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) q[u] = p[(k + u) * a.n_tokens];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) fold(M, S, q[u].x, q[u].y);
    }
    for (; k < k1; ++k) {
      const float2 q = p[k * a.n_tokens];
      fold(M, S, q.x, q.y);
    }
  }
  run_ms[g][tl] = make_float2(M, S);
  __syncthreads();
  if (g != 0 || t >= a.n_tokens) return;
  M = -INFINITY;
  S = 0.0f;
#pragma unroll
  for (int r = 0; r < kMergeRuns; ++r) fold(M, S, run_ms[r][tl].x, run_ms[r][tl].y);
  const float lse = (M + fast_log2(S)) * kLn2;
  a.lse[t] = lse;
  float lp = 0.0f;
  if (token_active(a.mask, a.y, a.ignore_index, t)) {
    const int64_t yy = a.y[t];
    lp = (yy >= 0 && yy < a.v_real) ? a.zy[t] - lse : __builtin_nanf("");
  }
  a.logp[t] = lp;
}

template <typename T>
static void launch_tiles(const FwdTileArgs& a, int tiles_m, int tiles_n, int32_t* queue,
                         const StageEvents& ev, hipStream_t s) {
  const int64_t nk = a.d_model * (int64_t)sizeof(T) / kStageBytes;
  const int g = chain_workgroups();
  if (nk % 2 == 0 && g >= 8) {
    const int total = tiles_m * tiles_n;
    const int used = total < g ? (total + 7) / 8 * 8 : g;
    if (queue) {
      hipLaunchKernelGGL((fwd_tile_chain_kernel<T, true>), dim3(used), dim3(kThreads), 0, s, a,
                         tiles_m, tiles_n, queue);
    } else {
      hipLaunchKernelGGL((fwd_tile_chain_kernel<T, false>), dim3(used), dim3(kThreads), 0, s, a,
                         tiles_m, tiles_n, queue);
    }
  } else {
    hipLaunchKernelGGL(fwd_tile_kernel<T>, dim3(tiles_m * tiles_n), dim3(kThreads), 0, s, a,
                       tiles_m, tiles_n);
  }
  ev.mark(1, s);
}

hipError_t launch_fwd_tiles(int dtype, const FwdTileArgs& a, int64_t n_vt, int32_t* queue,
                            const StageEvents& ev, hipStream_t s) {
  const int tiles_m = (int)n_vt;
  const int tiles_n = (int)ceil_div(a.n_tokens, kTokenTile);
  if (tiles_m * tiles_n == 0) return hipSuccess;
  if (dtype == 0) launch_tiles<__bf16>(a, tiles_m, tiles_n, queue, ev, s);
  else launch_tiles<float>(a, tiles_m, tiles_n, queue, ev, s);
  return hipGetLastError();
}

hipError_t launch_clear_queue(int32_t* queue, hipStream_t s) {
  hipLaunchKernelGGL(clear_queue_kernel, dim3(1), dim3(64), 0, s, queue);
  return hipGetLastError();
}

hipError_t launch_target_logit(int dtype, const TargetArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(a.n_tokens, 4));
  if (dtype == 0) hipLaunchKernelGGL(target_logit_kernel<__bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(target_logit_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)ceil_div(a.n_tokens, kMergeTokens)),
                     dim3(kMergeTokens * kMergeRuns), 0, s, a);
  return hipGetLastError();
}

}  // namespace gh
