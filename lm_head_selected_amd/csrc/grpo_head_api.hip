// C ABI of the fused LM-head GRPO / GSPO loss (declared in include/grpo_head.h).
//
// Host side only: argument checks (before anything is enqueued), workspace
// layout, launch sequencing on the caller's stream, the optional validation
// sync and the thread-local error text.  Failing loudly instead of falling back
// follows RL-Kernel PR #291 (commit notes: incompatible backends are rejected
// with explicit reasons and never used as a silent fallback); the validation sync
// being opt-in follows the same page's review thread on per-call device syncs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/grpo_head.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;
gh::StageEvents g_marks;  // stage timing events (grpo_head_set_stage_events)

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return GRPO_HEAD_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(GRPO_HEAD_HIP_ERROR, "%s: %s", where, hipGetErrorString(e));
}

// Every tile-row block of an operand is addressed with 32-bit buffer offsets.
constexpr int64_t kMaxRowBytes = (int64_t(1) << 31) / 256 - 1;

int check_gemm(const grpo_head_params* p);

int check_common(const grpo_head_params* p, bool need_gemm) {
  if (!p) return fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
  if (p->n_tokens < 0) return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_tokens < 0");
  if (p->n_tokens > (int64_t(1) << 31) - 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_tokens above 2^31 - 1");
  if (p->n_seqs < 0 || (p->n_tokens > 0 && p->n_seqs < 1))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_seqs must be >= 1 when n_tokens > 0");
  if (p->n_seqs > (int64_t(1) << 31) - 1) return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_seqs too large");
  if (p->level != GRPO_HEAD_LEVEL_TOKEN && p->level != GRPO_HEAD_LEVEL_SEQUENCE_GSPO)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "unknown level %d", p->level);
  if (p->reduction != GRPO_HEAD_TOKEN_MEAN && p->reduction != GRPO_HEAD_SEQUENCE_MEAN &&
      p->reduction != GRPO_HEAD_FIXED_CONSTANT)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "unknown reduction %d", p->reduction);
  if (p->reduction == GRPO_HEAD_FIXED_CONSTANT) {
    if (p->level != GRPO_HEAD_LEVEL_TOKEN)
      return fail(GRPO_HEAD_INVALID_ARGUMENT, "fixed_constant applies to the token level only");
    if (!(p->norm_const > 0.0f) || !std::isfinite(p->norm_const))
      return fail(GRPO_HEAD_INVALID_ARGUMENT, "norm_const must be finite and > 0");
  }
  if (p->accumulate_dw != 0 && p->accumulate_dw != 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "accumulate_dw must be 0 or 1");
  if (p->grad_dtype != GRPO_HEAD_GRAD_F32 && p->grad_dtype != GRPO_HEAD_GRAD_BF16)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "unknown grad_dtype %d", p->grad_dtype);
  if (p->reserved != 0) return fail(GRPO_HEAD_INVALID_ARGUMENT, "reserved must be 0");
  if (!(p->eps_low >= 0.0f && p->eps_low < 1.0f))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "eps_low must be in [0, 1)");
  if (!(p->eps_high >= 0.0f) || !std::isfinite(p->eps_high))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "eps_high must be finite and >= 0");
  if (!(p->beta >= 0.0f) || !std::isfinite(p->beta))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "beta must be finite and >= 0");
  if (p->validate != 0 && p->validate != 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "validate must be 0 or 1");
  if (!need_gemm) return GRPO_HEAD_OK;
  return check_gemm(p);
}

// The fields the vocabulary-tile stage uses (grpo_head_logp checks only these).
int check_gemm(const grpo_head_params* p) {
  if (p->n_tokens < 0) return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_tokens < 0");
  if (p->n_tokens > (int64_t(1) << 31) - 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_tokens above 2^31 - 1");
  if (p->validate != 0 && p->validate != 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "validate must be 0 or 1");
  if (p->dtype != GRPO_HEAD_BF16 && p->dtype != GRPO_HEAD_F32)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "unknown dtype %d", p->dtype);
  if (p->d_model <= 0 || p->d_model % 64 != 0)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "d_model must be a positive multiple of 64 (got %lld)",
                (long long)p->d_model);
  if (p->v_real < 1) return fail(GRPO_HEAD_INVALID_ARGUMENT, "v_real must be >= 1");
  if (p->v_rows < p->v_real) return fail(GRPO_HEAD_INVALID_ARGUMENT, "v_rows < v_real");
  if (!(p->inv_tau > 0.0f) || !std::isfinite(p->inv_tau))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "inv_tau must be finite and > 0");
  if (p->chunk_tokens < 0) return fail(GRPO_HEAD_INVALID_ARGUMENT, "chunk_tokens < 0");
  const int64_t esz = p->dtype == GRPO_HEAD_BF16 ? 2 : 4;
  const int64_t vk = gh::ceil_div(p->v_real, gh::kVocabTile) * gh::kVocabTile;
  if (p->d_model * esz > kMaxRowBytes || vk * esz > kMaxRowBytes ||
      gh::ceil_div(p->n_tokens, gh::kTokenTile) * gh::kTokenTile * esz > kMaxRowBytes)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a row of an operand exceeds %lld bytes",
                (long long)kMaxRowBytes);
  if (gh::ceil_div(p->v_real, gh::kVocabTile) * gh::ceil_div(p->n_tokens, gh::kTokenTile) >
      (int64_t(1) << 31) - 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "problem too large for one launch");
  return GRPO_HEAD_OK;
}

gh::WsLayout layout(const grpo_head_params* p, bool with_gemm = true) {
  gh::WsLayout L;
  const int64_t N = p->n_tokens, S = p->n_seqs, D = p->d_model;
  const int64_t esz = p->dtype == GRPO_HEAD_F32 ? 4 : 2;
  L.n_vt = (with_gemm && p->v_real > 0) ? gh::ceil_div(p->v_real, gh::kVocabTile) : 0;
  L.v_k = L.n_vt * gh::kVocabTile;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = gh::align_up(off + bytes); return o; };
  L.partials = take((size_t)L.n_vt * N * 8);
  L.zy = take(with_gemm ? (size_t)N * 4 : 0);
  L.seq_L = take((size_t)S * 4);
  L.seq_F = take((size_t)S * 16);
  L.seq_G = take((size_t)S * 4);
  L.scal = take(64);
  L.flags = take(64);
  L.fq = take(with_gemm ? 8 * 4 : 0);
  L.fwd_bytes = off;
  if (!with_gemm) return L;

  int64_t chunk = p->chunk_tokens > 0 ? p->chunk_tokens : N;
  if (chunk > N) chunk = N;
  chunk = gh::ceil_div(chunk > 0 ? chunk : 1, gh::kTokenTile) * gh::kTokenTile;
  L.chunk = chunk;
  off = 0;
  L.bflags = take(64);
  L.gl = take((size_t)chunk * 8);
  L.dz = take((size_t)chunk * L.v_k * esz);   // dlogits of one chunk, v-blocked
  L.ht = take((size_t)D * chunk * esz);       // the chunk's live H rows transposed
  L.bcnt = take((size_t)gh::ceil_div(chunk, gh::kCompactBlock) * 8);   // counts, then offsets
  L.live = take(4);
  L.rows = take((size_t)chunk * 4);
  L.rowpos = take((size_t)chunk * 4);
  L.hg = take((size_t)chunk * D * esz);       // the chunk's live H rows
  L.ytg = take((size_t)chunk * 4);            // target id of each compact row
  L.dwq = take(16 * 4);                       // tile queues of dlogits and of the dW tiles
  L.bwd_bytes = off > L.fwd_bytes ? off : L.fwd_bytes;
  return L;
}

// Tile-order group sizes (M-tiles walked per N-tile), chosen by measurement.
// dH and dW: 4 (8 and 2 measured slower).  The backward's logit recompute
// (dlogits): 4, also where the forward takes 8 -- it streams 128 KB of dz out
// per tile besides its operands; on the Qwen3-8B head at 8192 tokens 4 ran 3-4%
// faster than 8, and 2, 3 and 6 in between.
constexpr int kGroupDh = 4, kGroupDw = 4, kGroupDlogits = 4;

// Group size of the forward's logit product (vocabulary tiles walked per token
// tile).  The W panels of the groups resident on the 8 XCDs, plus all of H, should
// fit in the 256 MB last-level cache; otherwise both are fetched from HBM again
// and again.  Measured on the Qwen3-8B head: 8 is best at 8192 tokens and 4 at
// 16384 (which runs 7% slower with 8); 16 is slower at both, 2 slower at 16384.
int logit_group(int64_t tokens, int64_t d_model, int64_t esz) {
  const int64_t budget = (int64_t)192 << 20;
  const int64_t panel = 256 * d_model * esz, h = tokens * d_model * esz;
  return 8 * 8 * panel + h <= budget ? 8 : 4;
}

int finish_validation(uint32_t* dflags, hipStream_t s, bool check_active) {
  uint32_t h[2] = {0, 0};
  hipError_t e = hipMemcpyAsync(h, dflags, sizeof h, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "validation copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "validation sync");
  if (h[0] & (gh::kFlagTarget | gh::kFlagSid))
    return fail(GRPO_HEAD_TARGET_OUT_OF_RANGE, "%s",
                (h[0] & gh::kFlagTarget) ? "an active target is outside [0, v_real)"
                                         : "sid is decreasing or outside [0, n_seqs)");
  if (check_active && h[1] == 0) return fail(GRPO_HEAD_NO_ACTIVE_TOKENS, "no active token");
  if (h[0] & gh::kFlagNonfinite) return fail(GRPO_HEAD_NONFINITE, "non-finite value");
  return ok();
}

// The vocabulary-tile stage, the target-logit gather and the ordered merge:
// logp and lse of every token (nothing is enqueued for an empty batch).
int run_logp(const grpo_head_params* p, const gh::WsLayout& L, char* w, const void* H,
             const void* W, const int64_t* y, const uint8_t* mask, float* logp, float* lse,
             hipStream_t s) {
  if (p->n_tokens == 0) return GRPO_HEAD_OK;
  int32_t* fq = (int32_t*)(w + L.fq);
  hipError_t e = gh::launch_clear_queue(fq, s);
  if (e != hipSuccess) return hip_fail(e, "queue clear kernel");
  g_marks.mark(0, s);
  gh::FwdTileArgs fa{W, H, p->n_tokens, p->d_model, p->v_real, p->inv_tau,
                     (float2*)(w + L.partials),
                     logit_group(p->n_tokens, p->d_model, p->dtype == GRPO_HEAD_F32 ? 4 : 2)};
  e = gh::launch_fwd_tiles(p->dtype, fa, L.n_vt, fq, g_marks, s);
  if (e != hipSuccess) return hip_fail(e, "forward tile kernel");
  gh::TargetArgs ta{H, W, y, mask, p->n_tokens, p->d_model, p->v_real, p->ignore_index,
                    p->inv_tau, 0, (float*)(w + L.zy)};
  e = gh::launch_target_logit(p->dtype, ta, s);
  if (e != hipSuccess) return hip_fail(e, "target logit kernel");
  gh::MergeArgs ma{(const float2*)(w + L.partials), (const float*)(w + L.zy), y, mask,
                   p->n_tokens, L.n_vt, p->v_real, p->ignore_index, logp, lse};
  e = gh::launch_merge(ma, s);
  if (e != hipSuccess) return hip_fail(e, "merge kernel");
  g_marks.mark(2, s);
  return GRPO_HEAD_OK;
}

// Workspace layout of grpo_head_logp: the sequence fields play no part.
gh::WsLayout logp_layout(const grpo_head_params* p) {
  grpo_head_params q = *p;
  q.n_seqs = 0;
  return layout(&q);
}

int run_loss(const grpo_head_params* p, const gh::WsLayout& L, char* ws, const float* logp,
             const float* old_logp, const float* ref_logp, const uint8_t* mask,
             const int64_t* y, const int32_t* sid, const float* adv, float* out3, float* coef,
             int32_t* counts, float* seg_mean, hipStream_t s) {
  gh::LossArgs la{};
  la.n_tokens = p->n_tokens;
  la.n_seqs = p->n_seqs;
  la.level = p->level;
  la.reduction = p->reduction;
  la.eps_low = p->eps_low;
  la.eps_high = p->eps_high;
  la.beta = p->beta;
  la.norm_const = p->norm_const;
  la.logp = logp;
  la.old_logp = old_logp;
  la.ref_logp = ref_logp;
  la.adv = adv;
  la.sid = sid;
  la.mask = mask;
  la.y = y;
  la.ignore_index = p->ignore_index;
  la.seq_L = (int32_t*)(ws + L.seq_L);
  la.seq_F = (float*)(ws + L.seq_F);
  la.seq_G = (float*)(ws + L.seq_G);
  la.scal = (float*)(ws + L.scal);
  la.out3 = out3;
  la.coef = coef;
  la.counts = counts;
  la.seg_mean = seg_mean;
  hipError_t e = gh::launch_loss(la, s);
  if (e != hipSuccess) return hip_fail(e, "objective kernels");
  return GRPO_HEAD_OK;
}

// Shard bounds of grpo_head_shard_partials; returns the shard's real row count.
int check_shard(const grpo_head_params* p, int64_t v_begin, int64_t v_end, int64_t* real_rows) {
  if (!p) return fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
  int rc = check_gemm(p);
  if (rc) return rc;
  if (v_begin < 0 || v_end <= v_begin || v_end > p->v_rows)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "shard [%lld, %lld) outside [0, v_rows)",
                (long long)v_begin, (long long)v_end);
  if (v_begin % gh::kVocabTile != 0 || (v_end % gh::kVocabTile != 0 && v_end < p->v_real))
    return fail(GRPO_HEAD_INVALID_ARGUMENT,
                "shard bounds must lie on the %d-row tile grid (or the end at or past v_real)",
                (int)gh::kVocabTile);
  const int64_t hi = v_end < p->v_real ? v_end : p->v_real;
  *real_rows = hi > v_begin ? hi - v_begin : 0;
  return GRPO_HEAD_OK;
}

// Scratch of grpo_head_logp_noalloc: a file-scope device array, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels and copies get the address hipGetSymbolAddress
// returns for the current device, looked up once per device and kept.
constexpr size_t kNoAllocScratchBytes = GRPO_HEAD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (the symbol lookup allocates
// nothing: the array is part of the loaded code object).
int noalloc_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(GRPO_HEAD_HIP_ERROR, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return GRPO_HEAD_OK;
}

}  // namespace

extern "C" {

size_t grpo_head_fwd_workspace_size(const grpo_head_params* p) {
  if (check_common(p, true) != GRPO_HEAD_OK) return 0;
  return layout(p).fwd_bytes;
}

size_t grpo_head_workspace_size(const grpo_head_params* p) {
  if (check_common(p, true) != GRPO_HEAD_OK) return 0;
  return layout(p).bwd_bytes;
}

size_t gspo_segment_workspace_size(const grpo_head_params* p) {
  if (!p) {
    fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
    return 0;
  }
  grpo_head_params q = *p;
  q.level = GRPO_HEAD_LEVEL_SEQUENCE_GSPO;
  if (check_common(&q, false) != GRPO_HEAD_OK) return 0;
  return layout(&q, false).fwd_bytes;
}

const char* grpo_head_last_error(void) { return g_last_error.c_str(); }

size_t grpo_head_shard_partials_bytes(const grpo_head_params* p, int64_t v_begin,
                                      int64_t v_end) {
  int64_t rows = 0;
  if (check_shard(p, v_begin, v_end, &rows) != GRPO_HEAD_OK) return 0;
  return (size_t)gh::ceil_div(rows, gh::kVocabTile) * (size_t)p->n_tokens * 8;
}

int grpo_head_shard_partials(const grpo_head_params* p, int64_t v_begin, int64_t v_end,
                             const void* H, const void* W_shard, const int64_t* y,
                             const uint8_t* mask, void* partials, float* zy, void* stream) {
  int64_t rows = 0;
  int rc = check_shard(p, v_begin, v_end, &rows);
  if (rc) return rc;
  if (p->n_tokens == 0) return ok();
  if (!H || !W_shard || !y || !zy || (rows > 0 && !partials))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  hipStream_t s = (hipStream_t)stream;
  const int64_t n_st = gh::ceil_div(rows, gh::kVocabTile);
  if (n_st > 0) {
    gh::FwdTileArgs fa{W_shard, H, p->n_tokens, p->d_model, rows, p->inv_tau, (float2*)partials,
                       logit_group(p->n_tokens, p->d_model, p->dtype == GRPO_HEAD_F32 ? 4 : 2)};
    hipError_t e = gh::launch_fwd_tiles(p->dtype, fa, n_st, nullptr, gh::StageEvents{}, s);
    if (e != hipSuccess) return hip_fail(e, "forward tile kernel");
  }
  gh::TargetArgs ta{H, W_shard, y, mask, p->n_tokens, p->d_model, rows, p->ignore_index,
                    p->inv_tau, 2, zy, v_begin};
  hipError_t e = gh::launch_target_logit(p->dtype, ta, s);
  if (e != hipSuccess) return hip_fail(e, "target logit kernel");
  return ok();
}

int grpo_head_merge_partials(const grpo_head_params* p, const void* partials, const float* zy,
                             const int64_t* y, const uint8_t* mask, float* logp, float* lse,
                             void* stream) {
  if (!p) return fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
  int rc = check_gemm(p);
  if (rc) return rc;
  if (p->n_tokens == 0) return ok();
  if (!partials || !zy || !y || !logp || !lse)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  const int64_t n_vt = gh::ceil_div(p->v_real, gh::kVocabTile);
  gh::MergeArgs ma{(const float2*)partials, zy, y, mask, p->n_tokens, n_vt, p->v_real,
                   p->ignore_index, logp, lse};
  hipError_t e = gh::launch_merge(ma, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge kernel");
  return ok();
}

int grpo_group_advantage(const float* rewards, int64_t n_seqs, int64_t group_size, float eps,
                         int32_t scale_by_std, float* adv, void* stream) {
  if (n_seqs < 0) return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_seqs < 0");
  if (group_size < 1) return fail(GRPO_HEAD_INVALID_ARGUMENT, "group_size must be >= 1");
  if (n_seqs % group_size != 0)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "group_size %lld does not divide n_seqs %lld",
                (long long)group_size, (long long)n_seqs);
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (scale_by_std != 0 && scale_by_std != 1)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "scale_by_std must be 0 or 1");
  if (n_seqs > 0 && (!rewards || !adv))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "rewards and adv must not be NULL");
  hipError_t e = gh::launch_group_advantage(rewards, n_seqs, group_size, eps, scale_by_std, adv,
                                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "advantage kernel");
  return ok();
}

int grpo_head_set_stage_events(void* const* events, int n_events) {
  if (n_events < 0 || n_events > 16)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "n_events must be in [0, 16]");
  gh::StageEvents m;
  if (events) {
    for (int i = 0; i < n_events; ++i) m.ev[i] = events[i];
    m.n = n_events;
  }
  g_marks = m;
  return ok();
}

int grpo_head_fwd(const grpo_head_params* p, const void* H, const void* W, const int64_t* y,
                  const uint8_t* mask, const int32_t* sid, const float* adv,
                  const float* old_logp, const float* ref_logp, float* logp, float* lse,
                  float* out3, float* coef, int32_t* counts, void* ws, size_t ws_bytes,
                  void* stream) {
  int rc = check_common(p, true);
  if (rc) return rc;
  if (!out3) return fail(GRPO_HEAD_INVALID_ARGUMENT, "out3 is NULL");
  if (p->n_seqs > 0 && (!adv || !counts))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "adv and counts must not be NULL");
  if (p->n_tokens > 0 && (!H || !W || !y || !sid || !old_logp || !logp || !lse || !coef))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  if (p->beta > 0.0f && p->n_tokens > 0 && !ref_logp)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "beta > 0 needs ref_logp");
  const gh::WsLayout L = layout(p);
  if (!ws || ws_bytes < L.fwd_bytes)
    return fail(GRPO_HEAD_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes,
                L.fwd_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  hipError_t e;
  rc = run_logp(p, L, w, H, W, y, mask, logp, lse, s);
  if (rc) return rc;
  rc = run_loss(p, L, w, logp, old_logp, ref_logp, mask, y, sid, adv, out3, coef, counts,
                nullptr, s);
  if (rc) return rc;
  if (p->n_tokens > 0) g_marks.mark(3, s);
  if (p->validate) {
    gh::ValidateArgs va{p->n_tokens, p->n_seqs, p->v_real, p->ignore_index, y, mask, sid,
                        lse, logp, old_logp, ref_logp, out3, (uint32_t*)(w + L.flags)};
    e = gh::launch_validate(va, s);
    if (e != hipSuccess) return hip_fail(e, "validation kernel");
    return finish_validation((uint32_t*)(w + L.flags), s,
                             p->reduction != GRPO_HEAD_FIXED_CONSTANT);
  }
  return ok();
}

size_t grpo_head_logp_workspace_size(const grpo_head_params* p) {
  if (!p) {
    fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
    return 0;
  }
  if (check_gemm(p) != GRPO_HEAD_OK) return 0;
  return logp_layout(p).fwd_bytes;
}

int grpo_head_logp(const grpo_head_params* p, const void* H, const void* W, const int64_t* y,
                   const uint8_t* mask, float* logp, float* lse, void* ws, size_t ws_bytes,
                   void* stream) {
  if (!p) return fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
  int rc = check_gemm(p);
  if (rc) return rc;
  if (p->n_tokens > 0 && (!H || !W || !y || !logp || !lse))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  const gh::WsLayout L = logp_layout(p);
  if (!ws || ws_bytes < L.fwd_bytes)
    return fail(GRPO_HEAD_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes,
                L.fwd_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  rc = run_logp(p, L, w, H, W, y, mask, logp, lse, s);
  if (rc) return rc;
  if (p->validate) {
    gh::ValidateArgs va{p->n_tokens, 0, p->v_real, p->ignore_index, y, mask, nullptr,
                        lse, logp, nullptr, nullptr, nullptr, (uint32_t*)(w + L.flags)};
    hipError_t e = gh::launch_validate(va, s);
    if (e != hipSuccess) return hip_fail(e, "validation kernel");
    return finish_validation((uint32_t*)(w + L.flags), s, false);
  }
  return ok();
}

int grpo_head_logp_noalloc(const grpo_head_params* p, const void* H, const void* W,
                           const int64_t* y, const uint8_t* mask, float* logp, float* lse,
                           void* stream) {
  // every argument check runs before any HIP call, as in grpo_head_logp
  if (!p) return fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
  int rc = check_gemm(p);
  if (rc) return rc;
  if (p->n_tokens > 0 && (!H || !W || !y || !logp || !lse))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  const gh::WsLayout L = logp_layout(p);
  if (L.fwd_bytes > kNoAllocScratchBytes)
    return fail(GRPO_HEAD_INVALID_ARGUMENT,
                "this problem needs %zu bytes of scratch; the static scratch holds %zu "
                "(use grpo_head_logp with a workspace)",
                L.fwd_bytes, kNoAllocScratchBytes);
  if (p->n_tokens == 0) return ok();
  char* w = nullptr;
  rc = noalloc_scratch(&w);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  rc = run_logp(p, L, w, H, W, y, mask, logp, lse, s);
  if (rc) return rc;
  if (p->validate) {
    gh::ValidateArgs va{p->n_tokens, 0, p->v_real, p->ignore_index, y, mask, nullptr,
                        lse, logp, nullptr, nullptr, nullptr, (uint32_t*)(w + L.flags)};
    hipError_t e = gh::launch_validate(va, s);
    if (e != hipSuccess) return hip_fail(e, "validation kernel");
    return finish_validation((uint32_t*)(w + L.flags), s, false);
  }
  return ok();
}

int grpo_head_bwd(const grpo_head_params* p, const void* H, const void* W, const int64_t* y,
                  const uint8_t* mask, const float* lse, const float* coef,
                  const float* grad_output, void* dH, void* dW, void* ws, size_t ws_bytes,
                  void* stream) {
  int rc = check_common(p, true);
  if (rc) return rc;
  if (!W || !dW) return fail(GRPO_HEAD_INVALID_ARGUMENT, "W and dW must not be NULL");
  if (p->n_tokens > 0 && (!H || !y || !lse || !coef || !dH))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  if (p->n_tokens > 0 && !mask && !y)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "y is needed without a mask");
  const gh::WsLayout L = layout(p);
  if (!ws || ws_bytes < L.bwd_bytes)
    return fail(GRPO_HEAD_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes,
                L.bwd_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  g_marks.mark(4, s);
  gh::BwdArgs ba{H, W, y, mask, lse, coef, grad_output, dH, dW, p->n_tokens, p->d_model,
                 p->v_real, p->v_rows, p->ignore_index, p->inv_tau, w, &L,
                 kGroupDlogits, kGroupDh, kGroupDw, &g_marks, p->accumulate_dw,
                 p->grad_dtype == GRPO_HEAD_GRAD_BF16 ? 1 : 0};
  hipError_t e = gh::launch_bwd(p->dtype, ba, s);
  if (e != hipSuccess) return hip_fail(e, "backward kernels");
  if (p->validate) {
    gh::ValidateArgs va{p->n_tokens, p->n_seqs > 0 ? p->n_seqs : 1, p->v_real, p->ignore_index,
                        y, mask, nullptr, lse, coef, nullptr, nullptr, nullptr,
                        (uint32_t*)(w + L.bflags)};
    e = gh::launch_validate(va, s);
    if (e != hipSuccess) return hip_fail(e, "validation kernel");
    return finish_validation((uint32_t*)(w + L.bflags), s, false);
  }
  return ok();
}

int gspo_segment_reduce(const grpo_head_params* p, const float* logp, const float* old_logp,
                        const float* ref_logp, const uint8_t* mask, const int64_t* y,
                        const int32_t* sid, const float* adv, float* out3, float* coef,
                        float* seg_mean_logp, int32_t* counts, void* ws, size_t ws_bytes,
                        void* stream) {
  if (!p) return fail(GRPO_HEAD_INVALID_ARGUMENT, "params is NULL");
  // the segment level is implied: check the block as it will run (GSPO keeps its
  // segment mean, so a fixed_constant reduction is rejected like in grpo_head_fwd)
  grpo_head_params q = *p;
  q.level = GRPO_HEAD_LEVEL_SEQUENCE_GSPO;
  int rc = check_common(&q, false);
  if (rc) return rc;
  if (!out3) return fail(GRPO_HEAD_INVALID_ARGUMENT, "out3 is NULL");
  if (p->n_seqs > 0 && (!adv || !counts))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "adv and counts must not be NULL");
  if (p->n_tokens > 0 && (!logp || !old_logp || !sid || !coef))
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "a required buffer is NULL");
  if (p->n_tokens > 0 && !mask && !y)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "y is needed without a mask");
  if (p->beta > 0.0f && p->n_tokens > 0 && !ref_logp)
    return fail(GRPO_HEAD_INVALID_ARGUMENT, "beta > 0 needs ref_logp");
  const gh::WsLayout L = layout(&q, false);
  if (!ws || ws_bytes < L.fwd_bytes)
    return fail(GRPO_HEAD_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes,
                L.fwd_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  rc = run_loss(&q, L, w, logp, old_logp, ref_logp, mask, y, sid, adv, out3, coef, counts,
                seg_mean_logp, s);
  if (rc) return rc;
  if (p->validate) {
    gh::ValidateArgs va{p->n_tokens, p->n_seqs, p->v_real, p->ignore_index, y, mask, sid,
                        nullptr, logp, old_logp, ref_logp, out3, (uint32_t*)(w + L.flags)};
    va.check_targets = 0;
    hipError_t e = gh::launch_validate(va, s);
    if (e != hipSuccess) return hip_fail(e, "validation kernel");
    return finish_validation((uint32_t*)(w + L.flags), s, true);
  }
  return ok();
}

}  // extern "C"
