// Backward: recompute each logit tile, form dlogits, then the two gradient
// products.
//
//   G[t, v] = grad_output * coef_t * (1[v == y_t] - exp(z[t, v] - lse_t)) / tau
// (softmax recovered from the logits and the LSE, RL-Kernel PR #291, review
// thread on the saved fp32 logits; here the logits are recomputed per tile rather
// than saved).  Inactive tokens give 0.
//
// Per token chunk, in ascending chunk order:
//   1. dlogits_prep_kernel: (g_t, lse_t log2 e) per token
//   2. dlogits_kernel     : -g_t p_tv tile on the matrix cores -> dz (bf16, nearest
//                           even, on the bf16 path; fp32 on the fp32 path)
//      target_logit_kernel: rewrites dz[t][y_t] = g_t (1 - p_t,y_t)
//   3. product_kernel     : dH[t][:] = dz[t][:] . W      as (W^T)(dz)^T
//   4. transposes         : dzT[v][t] and HT[d][t]
//   5. product_kernel     : dW[v][:] (+)= dzT[v][:] . H  as (H^T)(dzT)^T
// Every product is an NT contraction (both operands contiguous along K) run by
// the same tile core.  The staging buffers WT, HT, dz and dzT use the core's
// K-panel layout (each 256-row tile's K stages stored back to back); WT is built
// once per call.
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
  const void* W; const void* H;   // H already offset to the chunk's first token
  const float2* gl;               // per chunk token: (g_t, lse_t * log2 e); g_t = 0 if inactive
  int64_t chunk_tokens;           // valid tokens in this chunk
  int64_t d_model, v_real, v_k;
  float inv_tau;
  void* dz;                       // K-panel [chunk_pad][v_k]
  int group_m;
};

// g_t = grad_output * coef_t / tau for active tokens (0 otherwise) and lse_t in
// base-2 units, for the chunk's tokens.
__global__ __launch_bounds__(256) void dlogits_prep_kernel(const int64_t* y, const uint8_t* mask,
                                                           int64_t ignore_index, const float* coef,
                                                           const float* lse,
                                                           const float* grad_output, float inv_tau,
                                                           int64_t n, float2* gl) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const bool act = token_is_active(mask, y, ignore_index, t);
  const float gout = grad_output ? *grad_output : 1.0f;
  gl[t] = make_float2(act ? gout * coef[t] * inv_tau : 0.0f, lse[t] * kLog2e);
}

// dz[t][v] = -g_t p_tv over the tile (the target element is rewritten afterwards
// by the target-logit kernel).  Columns of padded vocabulary rows hold finite
// values that the products never use: they meet zero rows of W^T in dH and the
// padded rows of dW are written as zeros.
template <typename T>
__global__ __launch_bounds__(kThreads) void dlogits_kernel(DlogitsArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t v0 = (int64_t)tm * kTile, t0 = (int64_t)tn * kTile;
  const int64_t esz = Elem<T>::size;
  const Operand A = row_major(a.W, a.d_model * esz, a.v_real);
  const Operand B = row_major(a.H, a.d_model * esz, a.chunk_tokens);
  f32x4 acc[kBI][kBJ];
  zero_acc(acc);
  gemm_tile<T>(A, B, v0, t0, a.d_model * esz, (lds_t*)lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t vbase = v0 + wm * (kTile / kWM) + (lane >> 4) * 4;
  const float c2 = a.inv_tau * kLog2e;
  const int64_t kb = a.v_k * esz;   // bytes of one dz row along K (vocabulary)
  // (g, lse2) of the lane's token columns; tokens past the chunk read zeros
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gl, (uint32_t)(a.chunk_tokens * 8));

#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int64_t t = t0 + wn * (kTile / kWN) + j * 16 + (lane & 15);
    // (cast the whole vector: clang miscompiles bit_cast of a single vector element)
    const f32x2 glv = __builtin_bit_cast(
        f32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, (uint32_t)(t * 8), 0, 0));
    const float g = glv[0];
    const float lse2 = glv[1];
    char* rowp = (char*)a.dz + (t >> 8) * 256 * kb + (t & 255) * 128;
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      const int64_t v = vbase + i * 16;   // 4 consecutive vocabulary rows
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = -g * fast_exp2(acc[i][j][e] * c2 - lse2);
      const int64_t vb = v * esz;
      Store4<T>::run(rowp + (vb >> 7) * (256 * 128) + (vb & 127), d[0], d[1], d[2], d[3]);
    }
  }
}

// C[m][n] tile of A . B^T stored transposed as out[n][m..m+3] (4 consecutive M per
// lane), the layout of dH[t][d] and dW[v][d].
struct ProductArgs {
  Operand A, B;
  int64_t k_bytes;
  float* out; int64_t ld_out;     // elements between out rows
  int64_t m_limit;                // M extent written (d_model)
  int64_t n_limit;                // N rows of out written
  int64_t n_zero_from;            // out rows >= this are written as 0 (padded vocab)
  int accumulate;                 // add to out
  int group_m;
};

// kRole only separates the dH (0) and dW (1) launches under a profiler.
template <typename T, int kRole>
__global__ __launch_bounds__(kThreads) void product_kernel(ProductArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
  f32x4 acc[kBI][kBJ];
  zero_acc(acc);
  gemm_tile<T>(a.A, a.B, m0, n0, a.k_bytes, (lds_t*)lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int64_t mbase = m0 + wm * (kTile / kWM) + (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int64_t n = n0 + wn * (kTile / kWN) + j * 16 + (lane & 15);
    if (n >= a.n_limit) continue;
    const bool zero = n >= a.n_zero_from;
    float* rowp = a.out + n * a.ld_out;
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      const int64_t m = mbase + i * 16;   // 4 consecutive M
      if (m >= a.m_limit) continue;
      f32x4 v = acc[i][j];
      if (zero) v = f32x4{0.f, 0.f, 0.f, 0.f};
      else if (a.accumulate) v += *(const f32x4*)(rowp + m);
      __builtin_nontemporal_store(v, (f32x4*)(rowp + m));
    }
  }
}

// dst = src^T in K-panel layout: dst row c, K element r  <-  src row r, column c,
// for r < rows_valid and c < cols_valid, else 0.  src is row-major (pitch src_ld
// elements) or K-panel (rows of src_kb bytes).  64 x 64 element tiles; dst rows
// are dst_kb bytes long.
template <typename E>
__global__ __launch_bounds__(256) void transpose_panel_kernel(const E* __restrict__ src,
                                                              int64_t src_ld, int src_panel,
                                                              int64_t src_kb, int64_t rows_valid,
                                                              int64_t cols_valid,
                                                              E* __restrict__ dst, int64_t dst_kb,
                                                              int tiles_c) {
  __shared__ E tile[64][65];
  const int64_t tc = blockIdx.x % tiles_c;   // tile along src columns (dst rows)
  const int64_t tr = blockIdx.x / tiles_c;   // tile along src rows (dst K)
  const int64_t r0 = tr * 64, c0 = tc * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t esz = sizeof(E);
  for (int k = ty; k < 64; k += 4) {
    const int64_t r = r0 + k, c = c0 + tx;
    E v = E(0);
    if (r < rows_valid && c < cols_valid) {
      v = src_panel ? *(const E*)((const char*)src + k_panel_offset(r, c * esz, src_kb))
                    : src[r * src_ld + c];
    }
    tile[k][tx] = v;
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int64_t c = c0 + k, r = r0 + tx;
    *(E*)((char*)dst + k_panel_offset(c, r * esz, dst_kb)) = tile[tx][k];
  }
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

// transpose of a [src rows][src cols] matrix into a K-panel [dst_rows][dst_k] one
template <typename E>
static void transpose_panel(const void* src, int64_t src_ld, bool src_panel, int64_t src_kb,
                            int64_t rows_valid, int64_t cols_valid, void* dst, int64_t dst_rows,
                            int64_t dst_k, hipStream_t s) {
  const int tiles_c = (int)(dst_rows / 64), tiles_r = (int)(dst_k / 64);
  hipLaunchKernelGGL(transpose_panel_kernel<E>, dim3((unsigned)(tiles_c * tiles_r)), dim3(256), 0,
                     s, (const E*)src, src_ld, src_panel ? 1 : 0, src_kb, rows_valid, cols_valid,
                     (E*)dst, dst_k * (int64_t)sizeof(E), tiles_c);
}

template <typename T>
static hipError_t run_bwd(const BwdArgs& a, hipStream_t s) {
  typedef typename std::conditional<sizeof(T) == 2, uint16_t, float>::type E;
  const WsLayout& L = *a.L;
  const int64_t esz = sizeof(T);
  const int64_t N = a.n_tokens, D = a.d_model, VK = L.v_k;
  const int64_t Dp = ceil_div(D, kTile) * kTile;   // panel rows of WT and HT
  char* wt = a.ws + L.wt;
  char* ht = a.ws + L.ht;
  char* dz = a.ws + L.dz;
  char* dzt = a.ws + L.dzt;
  float2* gl = (float2*)(a.ws + L.gl);

  // padded vocabulary rows of dW that no tile reaches
  if (a.v_rows > VK) {
    hipError_t e = launch_fill_zero(a.dW + VK * D, (size_t)(a.v_rows - VK) * D * 4, s);
    if (e != hipSuccess) return e;
  }
  if (N == 0) {
    return launch_fill_zero(a.dW, (size_t)(a.v_rows < VK ? a.v_rows : VK) * D * 4, s);
  }
  // WT: rows d (Dp, zero past D), K = vocabulary (zero past v_real)
  transpose_panel<E>(a.W, D, false, 0, a.v_real, D, wt, Dp, VK, s);
  const StageEvents& ev = *a.marks;

  const int tiles_v = (int)L.n_vt;
  const int tiles_d = (int)ceil_div(D, kTile);
  for (int64_t c0 = 0; c0 < N; c0 += L.chunk) {
    const int64_t nc = (N - c0) < L.chunk ? (N - c0) : L.chunk;
    const int64_t ncp = ceil_div(nc, kTokenTile) * kTokenTile;
    const int tiles_t = (int)(ncp / kTokenTile);

    const uint8_t* cmask = a.mask ? a.mask + c0 : nullptr;
    hipLaunchKernelGGL(dlogits_prep_kernel, dim3((unsigned)ceil_div(nc, 256)), dim3(256), 0, s,
                       a.y + c0, cmask, a.ignore_index, a.coef + c0, a.lse + c0, a.grad_output,
                       a.inv_tau, nc, gl);
    DlogitsArgs d{a.W, (const char*)a.H + c0 * D * esz, gl, nc, D, a.v_real, VK, a.inv_tau, dz,
                  a.group_fwd};
    ev.mark(5, s);
    hipLaunchKernelGGL(dlogits_kernel<T>, dim3(tiles_v * tiles_t), dim3(kThreads), 0, s, d,
                       tiles_v, tiles_t);
    ev.mark(6, s);
    TargetArgs fx{(const char*)a.H + c0 * D * esz, a.W, a.y + c0, cmask, nc, D, a.v_real,
                  a.ignore_index, a.inv_tau, 1, nullptr, a.lse + c0, a.coef + c0,
                  a.grad_output, dz, VK};
    hipError_t e0 = launch_target_logit(sizeof(T) == 2 ? 0 : 1, fx, s);
    if (e0 != hipSuccess) return e0;
    ev.mark(7, s);

    // dH rows of the chunk: M = d (WT rows), N = t (dz rows), K = v
    ProductArgs ph{k_panel(wt, VK * esz, D), k_panel(dz, VK * esz, nc), VK * esz,
                   a.dH + c0 * D, D, D, nc, INT64_MAX, 0, a.group_dh};
    hipLaunchKernelGGL((product_kernel<T, 0>), dim3(tiles_d * tiles_t), dim3(kThreads), 0, s, ph,
                       tiles_d, tiles_t);
    ev.mark(8, s);

    // dzT: rows v, K = t;  HT: rows d, K = t
    transpose_panel<E>(dz, 0, true, VK * esz, ncp, VK, dzt, VK, ncp, s);
    transpose_panel<E>((const char*)a.H + c0 * D * esz, D, false, 0, nc, D, ht, Dp, ncp, s);
    ev.mark(9, s);

    // dW: M = d (HT rows), N = v (dzT rows), K = t
    ProductArgs pw{k_panel(ht, ncp * esz, D), k_panel(dzt, ncp * esz, VK), ncp * esz,
                   a.dW, D, D, (a.v_rows < VK ? a.v_rows : VK), a.v_real, c0 > 0 ? 1 : 0,
                   a.group_dw};
    hipLaunchKernelGGL((product_kernel<T, 1>), dim3(tiles_d * tiles_v), dim3(kThreads), 0, s, pw,
                       tiles_d, tiles_v);
    ev.mark(10, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t s) {
  return dtype == 0 ? run_bwd<__bf16>(a, s) : run_bwd<float>(a, s);
}

}  // namespace gh
