// Objective stage: per-token ratio / clip / KL terms, fixed-order per-sequence
// totals, the scalar triple and the per-token coefficient.
//
// The objective acts per token (GRPO) or per segment (GSPO); only the final sums
// depend on the layout, so those sums are pinned to one order: tokens of a
// sequence in a fixed strided-then-tree order, then sequences in a fixed tree
// order (RL-Kernel PR #291, Overview / Key Changes).  Normalisers:
// token mean over active tokens (global_active_tokens), mean over sequences
// with at least one active token of each sequence's token mean
// (per_sequence_then_mean), or the active-token sum over a caller constant
// (fixed_constant, the Dr. GRPO normaliser; same page, Key Changes).  GSPO
// aggregates m_t (logp_t - old_t) per segment (the index_add of Fast-LLM PR #554,
// What), then forms the segment ratio, the loss, the new_logprobs metric and the
// unscaled per-token coefficient.
// An empty batch yields zeros, never a division by zero.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace gh {

constexpr int kSeqThreads = 256;
constexpr int kRedThreads = 1024;

__device__ __forceinline__ bool active_at(const uint8_t* mask, const int64_t* y,
                                          int64_t ignore_index, int64_t t) {
  return mask ? (mask[t] != 0) : (y[t] != ignore_index);
}

// first index in [0, n) with sid[i] >= key (sid non-decreasing)
__device__ int64_t lower_bound_sid(const int32_t* sid, int64_t n, int32_t key) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (sid[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int NT, int K>
__device__ __forceinline__ void block_sum(float (&v)[K], float (*sh)[NT]) {
#pragma unroll
  for (int k = 0; k < K; ++k) sh[k][threadIdx.x] = v[k];
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
#pragma unroll
      for (int k = 0; k < K; ++k) sh[k][threadIdx.x] += sh[k][threadIdx.x + w];
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = sh[k][0];
  __syncthreads();
}

__device__ __forceinline__ float k3(float lp, float ref) {
  const float d = ref - lp;
  return expf(d) - d - 1.0f;
}

// Per-sequence totals.  One workgroup per sequence s:
//   L_s (active count) and, over active tokens,
//   GRPO: F0 = sum pol_t, F1 = sum kl_t
//   GSPO: F0 = sum (logp_t - old_t), F1 = sum kl_t, F2 = sum logp_t
__global__ __launch_bounds__(kSeqThreads) void seq_totals_kernel(LossArgs a) {
  __shared__ float sh[4][kSeqThreads];
  const int32_t s = (int32_t)blockIdx.x;
  const int64_t lo = lower_bound_sid(a.sid, a.n_tokens, s);
  const int64_t hi = lower_bound_sid(a.sid, a.n_tokens, s + 1);
  const float adv = a.adv[s];
  const float clo = 1.0f - a.eps_low, chi = 1.0f + a.eps_high;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t t = lo + threadIdx.x; t < hi; t += kSeqThreads) {
    if (!active_at(a.mask, a.y, a.ignore_index, t)) continue;
    const float lp = a.logp[t];
    const float old = a.old_logp[t];
    v[3] += 1.0f;
    if (a.level == 0) {
      const float r = expf(lp - old);
      const float c = fminf(fmaxf(r, clo), chi);
      v[0] += -fminf(r * adv, c * adv);
    } else {
      v[0] += lp - old;
      v[2] += lp;
    }
    if (a.ref_logp) v[1] += k3(lp, a.ref_logp[t]);
  }
  block_sum<kSeqThreads, 4>(v, sh);
  if (threadIdx.x == 0) {
    a.seq_L[s] = (int32_t)v[3];
    a.seq_F[4 * s + 0] = v[0];
    a.seq_F[4 * s + 1] = v[1];
    a.seq_F[4 * s + 2] = v[2];
    a.seq_F[4 * s + 3] = 0.f;
  }
}

// Scalars.  One workgroup of 1024 threads over all sequences.
// scal[0] = 1/T_act (1/norm_const for fixed_constant), scal[1] = 1/S_live (0 for an
// empty batch).
__global__ __launch_bounds__(kRedThreads) void loss_scalars_kernel(LossArgs a) {
  __shared__ float sh[6][kRedThreads];
  const float clo = 1.0f - a.eps_low, chi = 1.0f + a.eps_high;
  // v: 0 T_act, 1 S_live, 2 sum F0 (token), 3 sum F1 (token),
  //    4 sum of per-sequence means of F0 (or GSPO pol_s), 5 of F1
  float v[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t s = threadIdx.x; s < a.n_seqs; s += kRedThreads) {
    const int32_t L = a.seq_L[s];
    const float F0 = a.seq_F[4 * s], F1 = a.seq_F[4 * s + 1], F2 = a.seq_F[4 * s + 2];
    if (a.counts) a.counts[s] = L;
    float g = 0.0f, segmean = 0.0f;
    if (L > 0) {
      const float fl = (float)L;
      v[0] += fl;
      v[1] += 1.0f;
      v[2] += F0;
      v[3] += F1;
      if (a.level == 0) {
        v[4] += F0 / fl;
      } else {
        const float A = a.adv[s];
        const float sigma = expf(F0 / fl);
        const float c = fminf(fmaxf(sigma, clo), chi);
        v[4] += -fminf(sigma * A, c * A);
        g = (sigma * A <= c * A) ? -A * sigma : 0.0f;
        segmean = F2 / fl;
      }
      v[5] += F1 / fl;
    }
    if (a.level == 1) {
      a.seq_G[s] = g;
      if (a.seg_mean) a.seg_mean[s] = segmean;
    }
  }
  block_sum<kRedThreads, 6>(v, sh);
  if (threadIdx.x == 0) {
    const float T = v[0], S = v[1];
    float pol = 0.f, kl = 0.f;
    const bool fixed = a.level == 0 && a.reduction == 2;
    if (fixed) {
      pol = v[2] / a.norm_const;
      kl = v[3] / a.norm_const;
    } else if (T > 0.f) {
      if (a.level == 0 && a.reduction == 0) {
        pol = v[2] / T;
        kl = v[3] / T;
      } else {
        pol = v[4] / S;
        kl = v[5] / S;
      }
    }
    if (a.ref_logp == nullptr) kl = 0.f;
    a.out3[0] = pol + a.beta * kl;
    a.out3[1] = pol;
    a.out3[2] = kl;
    a.scal[0] = fixed ? 1.0f / a.norm_const : (T > 0.f ? 1.0f / T : 0.f);
    a.scal[1] = S > 0.f ? 1.0f / S : 0.f;
  }
}

// Per-token coefficient d loss / d logp_t.
__global__ __launch_bounds__(256) void coef_kernel(LossArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.n_tokens) return;
  float cf = 0.0f;
  if (active_at(a.mask, a.y, a.ignore_index, t)) {
    int32_t s = a.sid[t];
    s = s < 0 ? 0 : (s >= a.n_seqs ? (int32_t)(a.n_seqs - 1) : s);
    const float invT = a.scal[0], invS = a.scal[1];
    const float L = (float)a.seq_L[s];
    const float lp = a.logp[t];
    const float wseq = L > 0.f ? invS / L : 0.f;
    const float dkl = a.ref_logp ? 1.0f - expf(a.ref_logp[t] - lp) : 0.0f;
    if (a.level == 0) {
      const float w = a.reduction == 1 ? wseq : invT;   // token mean or fixed constant
      const float adv = a.adv[s];
      const float r = expf(lp - a.old_logp[t]);
      const float c = fminf(fmaxf(r, 1.0f - a.eps_low), 1.0f + a.eps_high);
      const float dpol = (r * adv <= c * adv) ? -adv * r : 0.0f;
      cf = w * (dpol + a.beta * dkl);
    } else {
      cf = wseq * (a.seq_G[s] + a.beta * dkl);
    }
  }
  a.coef[t] = cf;
}

hipError_t launch_loss(const LossArgs& a, hipStream_t s) {
  if (a.n_seqs > 0 && a.n_tokens > 0)
    hipLaunchKernelGGL(seq_totals_kernel, dim3((unsigned)a.n_seqs), dim3(kSeqThreads), 0, s, a);
  else if (a.n_seqs > 0) {
    hipError_t e = launch_fill_zero(a.seq_L, a.n_seqs * sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    e = launch_fill_zero(a.seq_F, a.n_seqs * 4 * sizeof(float), s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(loss_scalars_kernel, dim3(1), dim3(kRedThreads), 0, s, a);
  if (a.n_tokens > 0)
    hipLaunchKernelGGL(coef_kernel, dim3((unsigned)ceil_div(a.n_tokens, 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Group-relative advantage of each sequence from its scalar reward: consecutive
// groups of G sequences; mean, then the variance of the deviations (two passes,
// the mean subtracted before squaring: RL-Kernel PR #291, review thread on the
// TWO_PASS enum), divided by G; A = (r - mean) / (std + eps), 0 when that divisor
// is 0, or A = r - mean without the std scaling.  One thread per group, each sum
// in index order, so the result is bitwise repeatable.  adv may be r itself (in
// place): a thread reads each reward of its group before writing that element,
// and no other thread touches the group, so r and adv are not restrict.
__global__ __launch_bounds__(256) void group_advantage_kernel(const float* r, int64_t n_groups,
                                                              int64_t G, float eps, int scale,
                                                              float* adv) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const float* rg = r + g * G;
  float* ag = adv + g * G;
  float sum = 0.0f;
  for (int64_t i = 0; i < G; ++i) sum += rg[i];
  const float mean = sum / (float)G;
  if (!scale) {
    for (int64_t i = 0; i < G; ++i) ag[i] = rg[i] - mean;
    return;
  }
  float ss = 0.0f;
  for (int64_t i = 0; i < G; ++i) {
    const float d = rg[i] - mean;
    ss += d * d;
  }
  const float den = sqrtf(ss / (float)G) + eps;
  for (int64_t i = 0; i < G; ++i) ag[i] = den > 0.0f ? (rg[i] - mean) / den : 0.0f;
}

hipError_t launch_group_advantage(const float* r, int64_t n_seqs, int64_t G, float eps,
                                  int scale, float* adv, hipStream_t s) {
  const int64_t n_groups = n_seqs / G;
  if (n_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(group_advantage_kernel, dim3((unsigned)ceil_div(n_groups, 256)), dim3(256),
                     0, s, r, n_groups, G, eps, scale, adv);
  return hipGetLastError();
}

// Validation (only with validate = 1): one workgroup scans every token.
__global__ __launch_bounds__(1024) void validate_kernel(ValidateArgs a) {
  __shared__ uint32_t sflag[1024];
  __shared__ uint32_t scount[1024];
  uint32_t f = 0, cnt = 0;
  for (int64_t t = threadIdx.x; t < a.n_tokens; t += 1024) {
    const bool act = a.mask ? a.mask[t] != 0 : a.y[t] != a.ignore_index;
    if (act) {
      ++cnt;
      if (a.check_targets && a.y && (a.y[t] < 0 || a.y[t] >= a.v_real)) f |= kFlagTarget;
      if (a.b && !isfinite(a.b[t])) f |= kFlagNonfinite;
      if (a.c && !isfinite(a.c[t])) f |= kFlagNonfinite;
      if (a.d && !isfinite(a.d[t])) f |= kFlagNonfinite;
    }
    if (a.a && !isfinite(a.a[t])) f |= kFlagNonfinite;
    if (a.sid) {
      const int32_t s = a.sid[t];
      if (s < 0 || s >= a.n_seqs || (t > 0 && a.sid[t - 1] > s)) f |= kFlagSid;
    }
  }
  sflag[threadIdx.x] = f;
  scount[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      sflag[threadIdx.x] |= sflag[threadIdx.x + w];
      scount[threadIdx.x] += scount[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    uint32_t ff = sflag[0];
    if (a.out3)
      for (int k = 0; k < 3; ++k)
        if (!isfinite(a.out3[k])) ff |= kFlagNonfinite;
    a.flags[0] = ff;
    a.flags[1] = scount[0];
  }
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace gh
