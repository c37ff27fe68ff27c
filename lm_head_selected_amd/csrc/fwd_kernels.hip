// Forward: vocabulary-tile logits -> per-tile (max, sumexp) partials -> merge.
//
// Tile-streamed selected-token log-prob (Liger-Kernel PR #1160, Summary): each
// workgroup computes one 256-vocab x 256-token logit tile on the matrix cores,
// reduces it to one (max, sumexp) partial per token and captures the target
// logit when the target falls inside the tile; the [N, V] logits never leave
// registers.  Padded columns (vocab >= v_real) are -inf before the partial is
// formed, and the merge folds the partials in ascending tile order starting from
// the identity (-inf, 0) (RL-Kernel PR #291, commit notes: ShardingSpec,
// ReductionSpec).  Partials are kept in base-2 units: m2 = max z*log2(e) and
// s = sum 2^(z*log2(e) - m2), so every exponential is one v_exp_f32.
#include "gemm_tile.hpp"
#include "launch.hpp"

namespace gh {

__device__ __forceinline__ bool token_active(const uint8_t* mask, const int64_t* y,
                                             int64_t ignore_index, int64_t t) {
  return mask ? (mask[t] != 0) : (y[t] != ignore_index);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void fwd_tile_kernel(FwdTileArgs a, int tiles_m,
                                                            int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  __shared__ float2 half_stats[2][kTile];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t v0 = (int64_t)tm * kTile;   // vocabulary rows of this tile
  const int64_t t0 = (int64_t)tn * kTile;   // tokens of this tile
  const int64_t esz = Elem<T>::size;

  Operand A{(const char*)a.W, a.d_model * esz, a.v_real};
  Operand B{(const char*)a.H, a.d_model * esz, a.n_tokens};
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_tile<T>(A, B, v0, t0, a.d_model * esz, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t vbase = v0 + wm * 128;
  const float c2 = a.inv_tau * kLog2e;
  const int hi = lane >> 5;
  // real vocabulary rows of this wave: [0, vlim) relative to vbase
  const int vlim = (int)((a.v_real - vbase) < 128 ? (a.v_real - vbase) : 128);

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = wn * 128 + j * 32 + (lane & 31);
    const int64_t t = t0 + tl;
    int ty = -1;  // target row inside this wave's 128 vocabulary rows
    if (t < a.n_tokens && token_active(a.mask, a.y, a.ignore_index, t)) {
      const int64_t yy = a.y[t];
      if (yy >= vbase && yy < vbase + 128 && yy < a.v_real) ty = (int)(yy - vbase);
    }
    float m = -INFINITY, zt = 0.0f;
    bool has = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = i * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
        const float z = acc[i][j][e];
        if (row == ty) { zt = z * a.inv_tau; has = true; }
        const float z2 = (row < vlim) ? z * c2 : -INFINITY;
        acc[i][j][e] = z2;
        m = fmaxf(m, z2);
      }
    m = fmaxf(m, __shfl_xor(m, 32));
    float s = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += fast_exp2(acc[i][j][e] - m);
    }
    s += __shfl_xor(s, 32);
    if (has) a.zy[t] = zt;
    if (hi == 0) half_stats[wm][tl] = make_float2(m, s);
  }
  __syncthreads();

  // merge the two 128-row halves (wave rows 0 then 1) and write the tile partial
  const int tl = threadIdx.x;
  const int64_t t = t0 + tl;
  if (t < a.n_tokens) {
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

// One thread per token: fold the n_vt partials in ascending tile order.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.n_tokens) return;
  float M = -INFINITY, S = 0.0f;
  const float2* p = a.partials + t;
  for (int64_t k = 0; k < a.n_vt; ++k) {
    const float2 q = p[k * a.n_tokens];
    if (q.x == -INFINITY) continue;           // identity partial
    if (q.x > M) {
      S = S * fast_exp2(M - q.x) + q.y;       // M = -inf on the first real tile: S*0
      M = q.x;
    } else {
      S = S + q.y * fast_exp2(q.x - M);
    }
  }
  const float lse = (M + fast_log2(S)) * kLn2;
  a.lse[t] = lse;
  float lp = 0.0f;
  if (token_active(a.mask, a.y, a.ignore_index, t)) {
    const int64_t yy = a.y[t];
    lp = (yy >= 0 && yy < a.v_real) ? a.zy[t] - lse : __builtin_nanf("");
  }
  a.logp[t] = lp;
}

hipError_t launch_fwd_tiles(int dtype, const FwdTileArgs& a, int64_t n_vt, hipStream_t s) {
  const int tiles_m = (int)n_vt;
  const int tiles_n = (int)ceil_div(a.n_tokens, kTokenTile);
  const int nwg = tiles_m * tiles_n;
  if (nwg == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL(fwd_tile_kernel<__bf16>, dim3(nwg), dim3(kThreads), 0, s, a, tiles_m,
                       tiles_n);
  else
    hipLaunchKernelGGL(fwd_tile_kernel<float>, dim3(nwg), dim3(kThreads), 0, s, a, tiles_m,
                       tiles_n);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)ceil_div(a.n_tokens, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gh
