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
//   3. product_kernel<0>  : dH[t][d] = sum_v dz[t][v] W[v][d]
//      (M = t: dz K-contiguous; N = d: W read MN-contiguous)
//   4. transpose_kernel   : HT[d][t] of the chunk (small: D x chunk)
//   5. product_kernel<1>  : dW[v][d] (+)= sum_t HT[d][t] dz[t][v]
//      (M = d: HT K-contiguous; N = v: dz read MN-contiguous)
// W and dz are read where they are; the tile core forms the transposed MFMA
// fragments of the MN-contiguous operand with the gfx950 transposing LDS read,
// which delivers about half the bandwidth of a plain read, so each product keeps
// exactly one such operand, on the side with the smaller per-wave fragment count.
// dz is stored "v-tiled": [vocabulary / 256][chunk rows][256], so a 256x256
// dlogits tile is one contiguous 128 KB block (bf16) and either product streams
// it in large contiguous runs.
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
  int64_t d_model, v_real;
  float inv_tau;
  void* dz;                       // v-tiled [n_vt][dz_rows][256]
  int64_t dz_rows;
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
// values that the products never use: they meet zero rows of W in dH, and the
// padded rows of dW are written as zeros.  Token rows past the chunk get g = 0.
template <typename T>
__global__ __launch_bounds__(kThreads) void dlogits_kernel(DlogitsArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
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
  const int vl = wm * (kTile / kWM) + (lane >> 4) * 4;   // tile-local vocabulary row
  const float c2 = a.inv_tau * kLog2e;
  // (g, lse2) of the lane's token columns; tokens past the chunk read zeros
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gl, (uint32_t)(a.chunk_tokens * 8));
  // this tile's block of dz: rows t0 .. t0 + 255 of vocabulary group tm, one
  // contiguous [256][256] block
  char* tile = (char*)a.dz + vtiled_offset(t0, v0, a.dz_rows, esz);
  // bf16: the block is staged in LDS (now free) and written out as whole rows;
  // 32-byte segment s of LDS row t sits at segment s ^ (t & 15)
  char* L = lds;

#pragma unroll
  for (int j = 0; j < kBJ; ++j) {
    const int tl = wn * (kTile / kWN) + j * 16 + (lane & 15);   // tile-local token
    // (cast the whole vector: clang miscompiles bit_cast of a single vector element)
    const f32x2 glv = __builtin_bit_cast(
        f32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, (uint32_t)((t0 + tl) * 8), 0, 0));
    const float g = glv[0];
    const float lse2 = glv[1];
    char* rowp = tile + (int64_t)tl * 256 * esz;
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      float d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = -g * fast_exp2(acc[i][j][e] * c2 - lse2);
      const int v = vl + i * 16;                                 // 4 consecutive v
      if (sizeof(T) == 2) {
        const bf16x4 q = {(__bf16)d[0], (__bf16)d[1], (__bf16)d[2], (__bf16)d[3]};
        const int byte = v * 2;                                  // within the 512-B row
        const int seg = (byte >> 5) ^ (tl & 15);
        *(i32x2*)(L + tl * 512 + seg * 32 + (byte & 31)) = __builtin_bit_cast(i32x2, q);
      } else {
        Store4<T>::run(rowp + v * esz, d[0], d[1], d[2], d[3]);
      }
    }
  }
  if (sizeof(T) == 2) {
    __syncthreads();
    // 256 rows x 32 chunks of 16 B, row-major: one wave writes two whole rows
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = q * kThreads + threadIdx.x;
      const int t = idx >> 5, c = idx & 31;
      const int seg = (c >> 1) ^ (t & 15);
      const i32x4 v = *(const i32x4*)(L + t * 512 + seg * 32 + (c & 1) * 16);
      __builtin_nontemporal_store(v, (i32x4*)(tile + (int64_t)t * 512 + c * 16));
    }
  }
}

// Products with a K-contiguous A and an MN-contiguous B.
//   kRole 0 (dH): C[m = t][n = d] stored row-major: out[m * ld_out + n];
//   kRole 1 (dW): C[m = d][n = v] stored as out[n * ld_out + m .. + 3].
struct ProductArgs {
  Operand A, B;
  int nk;                         // K stages
  void* out; int64_t ld_out;      // elements (of O) between out rows
  int64_t m_limit;                // M extent written
  int64_t n_limit;                // N extent written
  int64_t zero_from;              // dW rows (N) >= this are written as 0 (padded vocab)
  int accumulate;                 // add to out
  int group_m;
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

// The dW tile's epilogue: rows n0 .. n0 + 255 (vocabulary), columns m0 .. m0 + 255
// (hidden), staged through the (now free) pipeline LDS in two halves of 128 rows
// and written as whole 1 KB row segments.  16-byte chunk c of LDS row r sits at
// chunk c ^ (r & 15).  Rows >= zero_from are written as zeros; with accumulate
// the tile is added to what out holds.
template <typename O>
__device__ __forceinline__ void store_dw_tile(const f32x4 (&acc)[kBI][kBJ], char* lds, O* out,
                                              int64_t ld_out, int64_t n0, int64_t m0,
                                              int64_t n_limit, int64_t m_limit,
                                              int64_t zero_from, int accumulate) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  float* L = (float*)lds;   // [128][256]
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if ((wn >> 1) == p) {
#pragma unroll
      for (int j = 0; j < kBJ; ++j) {
        const int r = (wn & 1) * 64 + j * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < kBI; ++i) {
          const int c = (wm * 128 + i * 16 + (lane >> 4) * 4) >> 2;
          *(f32x4*)(L + r * 256 + ((c ^ (r & 15)) << 2)) = acc[i][j];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = (threadIdx.x >> 6) + 8 * q, c = threadIdx.x & 63;
      const int64_t n = n0 + p * 128 + r, m = m0 + c * 4;
      if (n < n_limit && m < m_limit) {
        f32x4 v = *(const f32x4*)(L + r * 256 + ((c ^ (r & 15)) << 2));
        O* o = out + n * ld_out + m;
        if (n >= zero_from) v = f32x4{0.f, 0.f, 0.f, 0.f};
        else if (accumulate) v += load_out4(o);
        store_out4(o, v);
      }
    }
    __syncthreads();
  }
}

template <typename T, int kRole, typename O>
__global__ __launch_bounds__(kThreads) void product_kernel(ProductArgs a, int tiles_m,
                                                           int tiles_n) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, a.group_m, tm, tn);
  const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
  f32x4 acc[kBI][kBJ];
  zero_acc(acc);
  gemm_tile<T, false, true>(a.A, a.B, m0, n0, a.nk, (lds_t*)lds, acc);

  if (kRole == 1) {
    store_dw_tile<O>(acc, lds, (O*)a.out, a.ld_out, n0, m0, a.n_limit, a.m_limit, a.zero_from,
                     a.accumulate);
    return;
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
        if (m + e >= a.m_limit) continue;
        O* p = (O*)a.out + (m + e) * a.ld_out + n;
        const float v = a.accumulate ? acc[i][j][e] + load_out(p) : acc[i][j][e];
        store_out(p, v);
      }
    }
  }
}

// HT[d][t] = H[t][d] for t < rows, 0 for rows <= t < rows_pad; HT rows are
// ld_out elements long.  64 x 64 element tiles through LDS.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ H, int64_t d_model,
                                                        int64_t rows, E* __restrict__ HT,
                                                        int64_t ld_out, int tiles_d) {
  __shared__ E tile[64][65];
  const int64_t td = blockIdx.x % tiles_d, tt = blockIdx.x / tiles_d;
  const int64_t d0 = td * 64, t0 = tt * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t t = t0 + k, d = d0 + tx;
    tile[k][tx] = (t < rows && d < d_model) ? H[t * d_model + d] : E(0);
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int64_t d = d0 + k, t = t0 + tx;
    if (d < d_model) HT[d * ld_out + t] = tile[tx][k];
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
  for (int64_t c0 = 0; c0 < N; c0 += R) {
    const int64_t nc = (N - c0) < R ? (N - c0) : R;
    const int64_t ncp = ceil_div(nc, kTokenTile) * kTokenTile;
    const int tiles_t = (int)(ncp / kTokenTile);
    const char* Hc = (const char*)a.H + c0 * D * esz;

    const uint8_t* cmask = a.mask ? a.mask + c0 : nullptr;
    hipLaunchKernelGGL(dlogits_prep_kernel, dim3((unsigned)ceil_div(nc, 256)), dim3(256), 0, s,
                       a.y + c0, cmask, a.ignore_index, a.coef + c0, a.lse + c0, a.grad_output,
                       a.inv_tau, nc, gl);
    DlogitsArgs d{a.W, Hc, gl, nc, D, a.v_real, a.inv_tau, dz, R, a.group_fwd};
    ev.mark(5, s);
    hipLaunchKernelGGL(dlogits_kernel<T>, dim3(tiles_v * tiles_t), dim3(kThreads), 0, s, d,
                       tiles_v, tiles_t);
    ev.mark(6, s);
    TargetArgs fx{Hc, a.W, a.y + c0, cmask, nc, D, a.v_real, a.ignore_index, a.inv_tau, 1,
                  nullptr, a.lse + c0, a.coef + c0, a.grad_output, dz, R};
    hipError_t e0 = launch_target_logit(sizeof(T) == 2 ? 0 : 1, fx, s);
    if (e0 != hipSuccess) return e0;
    ev.mark(7, s);

    // dH rows of the chunk: M = t (dz rows), N = d (W read MN-contiguous), K = v.
    // W rows >= v_real are never read (they load as zeros).
    ProductArgs ph{nt_vtiled(dz, R, esz, (int64_t)tiles_v * R * 256 * esz),
                   mn_row_major(a.W, D * esz, a.v_real, D, esz), (int)(VK * esz / kStageBytes),
                   dH + c0 * D, D, nc, D, INT64_MAX, 0, a.group_dh};
    hipLaunchKernelGGL((product_kernel<T, 0, O>), dim3(tiles_t * tiles_d), dim3(kThreads), 0, s,
                       ph, tiles_t, tiles_d);
    ev.mark(8, s);

    // HT of the chunk: D rows of ncp tokens (zero past nc)
    typedef typename std::conditional<sizeof(T) == 2, uint16_t, float>::type E;
    const int ttd = (int)ceil_div(D, 64);
    hipLaunchKernelGGL(transpose_kernel<E>, dim3((unsigned)(ttd * (ncp / 64))), dim3(256), 0, s,
                       (const E*)Hc, D, nc, (E*)ht, R, ttd);
    ev.mark(9, s);

    // dW: M = d (HT K-contiguous), N = v (dz read MN-contiguous), K = t.  Rows
    // [v_real, VK) of the last tile are written as zeros, or, when accumulating
    // into the caller's dW, not written at all.
    ProductArgs pw{nt_row_major(ht, R * esz, D), mn_vtiled(dz, R, esz, tiles_v),
                   (int)(ncp * esz / kStageBytes), dW, D, D,
                   a.accumulate_dw ? a.v_real : (a.v_rows < VK ? a.v_rows : VK), a.v_real,
                   (c0 > 0 || a.accumulate_dw) ? 1 : 0, a.group_dw};
    hipLaunchKernelGGL((product_kernel<T, 1, O>), dim3(tiles_d * tiles_v), dim3(kThreads), 0, s,
                       pw, tiles_d, tiles_v);
    ev.mark(10, s);
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
