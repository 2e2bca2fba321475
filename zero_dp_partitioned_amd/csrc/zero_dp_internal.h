// Internal interface between the host API (api.cpp) and the gfx950 kernels
// (kernels.hip). Not installed; the public ABI is include/zero_dp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/zero_dp.h"

namespace zdp {

constexpr int kBlock = 256;          // threads per block in the streaming kernels
constexpr int kVec = 8;              // elements per thread per iteration (16 B of 16-bit, 32 B of fp32)
constexpr int kMaxBlocks = 4096;     // partial slots per group
constexpr int kInlineReplicas = 64;  // replica pointers carried in the kernel arguments
constexpr size_t kWorkspaceHeader = 256;

// One block's contribution to the norm and the overflow flag.
struct Partial {
  double sumsq;
  int32_t flag;
  int32_t pad;
};
static_assert(sizeof(Partial) == 16, "partial layout");

// Where the averaged gradient of a shard comes from.
struct GradSource {
  const void* rep[kInlineReplicas];  // replica r at rep[r] (table), or rep[0] + r*stride
  int64_t stride;                    // elements between replicas when strided != 0
  const float* avg;                  // fp32 average (pre-unscale) when non-null
  int32_t n_d;
  int32_t strided;
  float inv_nd;  // 1/n_d when n_d is a power of two (multiplying is then exact), else 0
  float nd;      // n_d as fp32, for the division otherwise
};

// Arguments of the per-group update kernel.
struct AdamArgs {
  GradSource src;
  int64_t n;
  float* master;
  float* m;
  float* v;
  void* param;          // flat_param + param_offset (already offset), or null
  int32_t param_dt;     // ZERO_DT_F16 / ZERO_DT_BF16 / 0
  int32_t param_align;  // 16, 8, 4 or 2: largest power-of-two alignment of param, capped
  double beta1_d, beta2_d;
  float lr, beta1, beta2, eps, c1, c2, decay;
  int32_t has_decay;
  int32_t group;
  const zero_step_state* state;
  Partial* partials;  // slot of this group: kMaxBlocks entries
  int32_t* count;     // number of blocks that wrote partials for this group
};

// Arguments of the average kernel (checked pipeline) and of the single-copy scan.
struct ReduceArgs {
  GradSource src;
  int64_t n;
  float* avg_out;  // null: scan only
  const zero_step_state* state;
  Partial* partials;
  int32_t* count;
};

struct FinalizeArgs {
  const Partial* partials;  // base: group g at partials + g * kMaxBlocks
  const int32_t* counts;
  zero_step_state* state;
  int32_t n_groups;
  int32_t mode;  // 0: norm + skip verdict only; 1: norm, then commit a static-scale step
  int32_t skip_on_overflow;
  int32_t pad;
  double beta1[ZERO_MAX_GROUPS];
  double beta2[ZERO_MAX_GROUPS];
};

struct CommitArgs {
  zero_step_state* state;
  int32_t n_groups;
  int32_t dynamic;
  int32_t growth_interval;
  int32_t pad;
  double backoff, growth, min_scale;
  double beta1[ZERO_MAX_GROUPS];
  double beta2[ZERO_MAX_GROUPS];
};

struct CastArgs {
  const float* master;
  int64_t n;
  void* param;  // already offset
  int32_t param_dt;
  int32_t param_align;
};

enum SrcKind { kSrcAvg = 0, kSrcF16 = 1, kSrcBF16 = 2 };

// Launchers (kernels.hip). Each returns the hipError_t of the launch.
// `grid` is chosen by the caller; `vec` selects the 16-byte vector path.
hipError_t launch_adam(const AdamArgs& a, int src_kind, bool vec, bool checked, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, int src_kind, bool vec, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_state_init(zero_step_state* st, float loss_scale, hipStream_t s);
hipError_t launch_cast(const CastArgs& a, bool vec, hipStream_t s);

}  // namespace zdp
