// Backward: recompute each logit tile, form dlogits, then the two gradient
// products.
//
//   G[t, v] = grad_output * coef_t * (1[v == y_t] - exp(z[t, v] - lse_t)) / tau
// (softmax recovered from the logits and the LSE, RL-Kernel PR #291, review
// thread on the saved fp32 logits; here the logits are recomputed per tile rather
// than saved).  Padded columns and inactive tokens give 0.
//
// Per token chunk, in ascending chunk order:
//   1. dlogits_kernel : G tile on the matrix cores -> staging buffer dz[t][v]
//                       (bf16, nearest-even, on the bf16 path; fp32 on the fp32 path)
//   2. transpose      : dz -> dzT[v][t] and H chunk -> HT[d][t]
//   3. dh_kernel      : dH[t][:] = dz[t][:] . W      as (W^T)(dz)^T  on WT[d][v]
//   4. dw_kernel      : dW[v][:] (+)= dzT[v][:] . H  as (H^T)(dzT)^T on HT[d][t]
// Every product is an NT contraction (both operands contiguous along K) run by
// the same 256x256 tile core.  WT[d][v] is built once per call.
#include "gemm_tile.hpp"
#include "launch.hpp"

namespace gh {

__device__ __forceinline__ bool token_is_active(const uint8_t* mask, const int64_t* y,
                                                int64_t ignore_index, int64_t t) {
  return mask ? (mask[t] != 0) : (y[t] != ignore_index);
}

template <typename T> struct Store4;
template <> struct Store4<__bf16> {
  static __device__ __forceinline__ void run(void* p, float a, float b, float c, float d) {
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    *(bf16x4*)p = v;
  }
};
template <> struct Store4<float> {
  static __device__ __forceinline__ void run(void* p, float a, float b, float c, float d) {
    *(f32x4*)p = f32x4{a, b, c, d};
  }
};

struct DlogitsArgs {
  const void* W; const void* H;   // H already offset to the chunk's first token
  const int64_t* y; const uint8_t* mask; const float* lse; const float* coef;
  const float* grad_output;
  int64_t chunk_tokens;           // valid tokens in this chunk
  int64_t d_model, v_real, v_k, ignore_index;
  float inv_tau;
  void* dz;                       // [chunk_pad][v_k]
  int group_m;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void dlogits_kernel(DlogitsArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t v0 = (int64_t)tm * kTile, t0 = (int64_t)tn * kTile;
  const int64_t esz = Elem<T>::size;
  Operand A{(const char*)a.W, a.d_model * esz, a.v_real};
  Operand B{(const char*)a.H, a.d_model * esz, a.chunk_tokens};
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_tile<T>(A, B, v0, t0, a.d_model * esz, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t vbase = v0 + wm * 128;
  const float c2 = a.inv_tau * kLog2e;
  const float gout = a.grad_output ? *a.grad_output : 1.0f;
  const int hi = lane >> 5;
  const int vlim = (int)((a.v_real - vbase) < 128 ? (a.v_real - vbase) : 128);

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + wn * 128 + j * 32 + (lane & 31);
    float g = 0.0f, lse2 = 0.0f;
    int ty = -1;  // target row relative to vbase, if inside this wave's rows
    if (t < a.chunk_tokens && token_is_active(a.mask, a.y, a.ignore_index, t)) {
      g = gout * a.coef[t] * a.inv_tau;
      lse2 = a.lse[t] * kLog2e;
      const int64_t yy = a.y[t];
      if (yy >= vbase && yy < vbase + 128) ty = (int)(yy - vbase);
    }
    char* rowp = (char*)a.dz + (t * a.v_k) * esz;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rq = i * 32 + q * 8 + hi * 4;
        float d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rq + e;
          const float p = fast_exp2(acc[i][j][q * 4 + e] * c2 - lse2);
          const float x = g * ((r == ty ? 1.0f : 0.0f) - p);
          d[e] = r < vlim ? x : 0.0f;
        }
        Store4<T>::run(rowp + (vbase + rq) * esz, d[0], d[1], d[2], d[3]);
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

template <typename T>
__global__ __launch_bounds__(kThreads) void product_kernel(ProductArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_tile<T>(a.A, a.B, m0, n0, a.k_bytes, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int hi = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
    if (n >= a.n_limit) continue;
    const bool zero = n >= a.n_zero_from;
    float* rowp = a.out + n * a.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wm * 128 + i * 32 + q * 8 + hi * 4;
        if (m >= a.m_limit) continue;
        f32x4 v = {acc[i][j][q * 4], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                   acc[i][j][q * 4 + 3]};
        if (zero) v = f32x4{0.f, 0.f, 0.f, 0.f};
        else if (a.accumulate) v += *(const f32x4*)(rowp + m);
        *(f32x4*)(rowp + m) = v;
      }
  }
}

// dst[c][r] = src[r][c] for r < rows_valid and c < cols_valid, else 0; 64x64 tiles.
// dst is [dst_rows][dst_cols] with dst_rows, dst_cols multiples of 64.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ src,
                                                        int64_t src_ld, int64_t rows_valid,
                                                        int64_t cols_valid, E* __restrict__ dst,
                                                        int64_t dst_ld, int tiles_c) {
  __shared__ E tile[64][65];
  const int64_t tc = blockIdx.x % tiles_c;   // tile along src columns (dst rows)
  const int64_t tr = blockIdx.x / tiles_c;   // tile along src rows (dst columns)
  const int64_t r0 = tr * 64, c0 = tc * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < rows_valid && c < cols_valid) ? src[r * src_ld + c] : E(0);
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) dst[(c0 + k) * dst_ld + r0 + tx] = tile[tx][k];
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

template <typename E>
static void transpose(const void* src, int64_t src_ld, int64_t rows_valid, int64_t cols_valid,
                      void* dst, int64_t dst_rows, int64_t dst_cols, hipStream_t s) {
  const int tiles_c = (int)(dst_rows / 64), tiles_r = (int)(dst_cols / 64);
  hipLaunchKernelGGL(transpose_kernel<E>, dim3((unsigned)(tiles_c * tiles_r)), dim3(256), 0, s,
                     (const E*)src, src_ld, rows_valid, cols_valid, (E*)dst, dst_cols, tiles_c);
}

template <typename T>
static hipError_t run_bwd(const BwdArgs& a, hipStream_t s) {
  typedef typename std::conditional<sizeof(T) == 2, uint16_t, float>::type E;
  const WsLayout& L = *a.L;
  const int64_t esz = sizeof(T);
  const int64_t N = a.n_tokens, D = a.d_model, VK = L.v_k;
  char* wt = a.ws + L.wt;
  char* ht = a.ws + L.ht;
  char* dz = a.ws + L.dz;
  char* dzt = a.ws + L.dzt;

  // padded vocabulary rows of dW that no tile reaches
  if (a.v_rows > VK) {
    hipError_t e = launch_fill_zero(a.dW + VK * D, (size_t)(a.v_rows - VK) * D * 4, s);
    if (e != hipSuccess) return e;
  }
  if (N == 0) {
    return launch_fill_zero(a.dW, (size_t)(a.v_rows < VK ? a.v_rows : VK) * D * 4, s);
  }
  // WT[d][v] = W[v][d] for v < v_real, 0 up to v_k
  transpose<E>(a.W, D, a.v_real, D, wt, D, VK, s);
  const StageEvents& ev = *a.marks;

  const int tiles_v = (int)L.n_vt;
  const int tiles_d = (int)ceil_div(D, kTile);
  for (int64_t c0 = 0; c0 < N; c0 += L.chunk) {
    const int64_t nc = (N - c0) < L.chunk ? (N - c0) : L.chunk;
    const int64_t ncp = ceil_div(nc, kTokenTile) * kTokenTile;
    const int tiles_t = (int)(ncp / kTokenTile);
    ev.mark(5, s);

    DlogitsArgs d{a.W, (const char*)a.H + c0 * D * esz, a.y + c0,
                  a.mask ? a.mask + c0 : nullptr, a.lse + c0, a.coef + c0, a.grad_output,
                  nc, D, a.v_real, VK, a.ignore_index, a.inv_tau, dz, a.group_fwd};
    hipLaunchKernelGGL(dlogits_kernel<T>, dim3(tiles_v * tiles_t), dim3(kThreads), 0, s, d,
                       tiles_v, tiles_t);
    ev.mark(6, s);

    // dH rows of the chunk: M = d (WT rows), N = t (dz rows), K = v
    ProductArgs ph{Operand{wt, VK * esz, D}, Operand{dz, VK * esz, nc}, VK * esz,
                   a.dH + c0 * D, D, D, nc, INT64_MAX, 0, a.group_dh};
    hipLaunchKernelGGL(product_kernel<T>, dim3(tiles_d * tiles_t), dim3(kThreads), 0, s, ph,
                       tiles_d, tiles_t);
    ev.mark(7, s);

    // transposes for dW: dzT[v][t] and HT[d][t]
    transpose<E>(dz, VK, nc, VK, dzt, VK, ncp, s);
    transpose<E>((const char*)a.H + c0 * D * esz, D, nc, D, ht, D, ncp, s);
    ev.mark(8, s);

    // dW: M = d (HT rows), N = v (dzT rows), K = t
    ProductArgs pw{Operand{ht, ncp * esz, D}, Operand{dzt, ncp * esz, VK}, ncp * esz,
                   a.dW, D, D, (a.v_rows < VK ? a.v_rows : VK), a.v_real, c0 > 0 ? 1 : 0,
                   a.group_dw};
    hipLaunchKernelGGL(product_kernel<T>, dim3(tiles_d * tiles_v), dim3(kThreads), 0, s, pw,
                       tiles_d, tiles_v);
    ev.mark(9, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t s) {
  return dtype == 0 ? run_bwd<__bf16>(a, s) : run_bwd<float>(a, s);
}

}  // namespace gh
