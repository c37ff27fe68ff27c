// Host-side launch interface between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gh {

constexpr int64_t kVocabTile = 256;   // vocabulary rows per forward/backward tile
constexpr int64_t kTokenTile = 256;   // tokens per tile
constexpr int64_t kCompactBlock = 1024;  // tokens per block of the backward row compaction
constexpr size_t kAlign = 256;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Byte offsets into the caller's workspace.
struct WsLayout {
  // forward / segment stage
  size_t partials = 0, zy = 0, seq_L = 0, seq_F = 0, seq_G = 0, scal = 0, flags = 0;
  size_t fq = 0;           // the forward tile launch's queues: one counter per XCD
  size_t fwd_bytes = 0;
  // backward (reuses the workspace from offset 0)
  size_t bflags = 0, gl = 0, dz = 0, ht = 0;
  // backward row compaction: per-block live counts, the live count, the live rows'
  // token indices, every token's compact row (-1 if dead), the gathered H rows and
  // each compact row's target id
  size_t bcnt = 0, live = 0, rows = 0, rowpos = 0, hg = 0, ytg = 0;
  // the tile queues of the dlogits launch and of the gradient launch's dW tiles:
  // one counter per XCD each
  size_t dwq = 0;
  size_t bwd_bytes = 0;
  int64_t n_vt = 0;        // vocabulary tiles covering [0, v_real)
  int64_t v_k = 0;         // n_vt * 256: vocabulary extent of the dlogits buffer
  int64_t chunk = 0;       // tokens per backward chunk (multiple of 256)
};

// Workgroups of the persistent matrix-core launches: one per compute unit of the
// current device (a multiple of 8), looked up once per device; 0 if unknown.
inline int chain_workgroups() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = cus / 8 * 8;
  }
  return cached[dev];
}

// Validation flags (bit set in the flags word)
enum : uint32_t { kFlagTarget = 1u, kFlagNonfinite = 2u, kFlagSid = 4u };

struct FwdTileArgs {
  const void* W; const void* H;
  int64_t n_tokens, d_model, v_real;
  float inv_tau;
  float2* partials;  // [n_vt][n_tokens]
  int group_m;
};
// Target-logit gather (mode 0: zy[t] for the active tokens with a target in
// [0, v_real)), or a vocabulary shard's gather (mode 2: W holds rows
// [v_begin, v_begin + v_real) and zy[t] is written for every token, 0 unless y_t
// lies in the shard).
struct TargetArgs {
  const void* H; const void* W; const int64_t* y; const uint8_t* mask;
  int64_t n_tokens, d_model, v_real, ignore_index;
  float inv_tau;
  int mode;
  float* zy;
  int64_t v_begin = 0;
};
struct MergeArgs {
  const float2* partials; const float* zy; const int64_t* y; const uint8_t* mask;
  int64_t n_tokens, n_vt, v_real, ignore_index;
  float* logp; float* lse;
};
struct LossArgs {
  int64_t n_tokens; int64_t n_seqs; int32_t level, reduction;
  float eps_low, eps_high, beta;
  float norm_const;  // fixed_constant divisor (reduction 2)
  const float* logp; const float* old_logp; const float* ref_logp; const float* adv;
  const int32_t* sid; const uint8_t* mask; const int64_t* y; int64_t ignore_index;
  int32_t* seq_L; float* seq_F; float* seq_G; float* scal;
  float* out3; float* coef; int32_t* counts; float* seg_mean;
};
struct ValidateArgs {
  int64_t n_tokens, n_seqs, v_real, ignore_index;
  const int64_t* y; const uint8_t* mask; const int32_t* sid;
  const float* a; const float* b; const float* c; const float* d;  // checked if non-null
  const float* out3;
  uint32_t* flags;  // [0] = flag bits, [1] = active-token count
  int check_targets = 1;  // check active targets against [0, v_real)
};
// Optional stage-boundary events (see grpo_head_set_stage_events).
struct StageEvents {
  void* ev[16] = {};
  int n = 0;
  void mark(int i, hipStream_t s) const {
    if (i < n && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], s);
  }
};

struct BwdArgs {
  const void* H; const void* W; const int64_t* y; const uint8_t* mask;
  const float* lse; const float* coef; const float* grad_output;
  void* dH; void* dW;
  int64_t n_tokens, d_model, v_real, v_rows, ignore_index;
  float inv_tau;
  char* ws; const WsLayout* L;
  int group_dlogits, group_dh, group_dw;
  const StageEvents* marks;
  int accumulate_dw;   // add the gradient to dW rows [0, v_real) instead of overwriting
  int grad_bf16;       // dH and dW are bf16 (else fp32)
};

// records stage event 1 after the tile launch; queue: the 8 tile-queue counters of
// the chained launch, cleared beforehand by launch_clear_queue (null: a fixed
// tile schedule)
hipError_t launch_fwd_tiles(int dtype, const FwdTileArgs& a, int64_t n_vt, int32_t* queue,
                            const StageEvents& ev, hipStream_t s);
hipError_t launch_clear_queue(int32_t* queue, hipStream_t s);
hipError_t launch_target_logit(int dtype, const TargetArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_loss(const LossArgs& a, hipStream_t s);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t s);
hipError_t launch_group_advantage(const float* r, int64_t n_seqs, int64_t G, float eps,
                                  int scale, float* adv, hipStream_t s);
hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace gh
