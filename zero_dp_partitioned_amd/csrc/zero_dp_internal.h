// Internal interface between the host API (api.cpp) and the gfx950 kernels
// (kernels.hip). Not installed; the public ABI is include/zero_dp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/zero_dp.h"

namespace zdp {

// Streaming layout: a block of 256 threads owns tiles of 4096 consecutive
// elements; in a tile, lane l of the block handles the 4-element quads
// l, l + 256, l + 512, l + 768, so each wavefront instruction touches one
// contiguous run (1 KiB of fp32, 512 B of 16-bit data).
constexpr int kBlock = 256;
constexpr int kQuadsPerThread = 4;
constexpr int kTile = kBlock * kQuadsPerThread * 4;  // elements per tile
// With many gradient copies the update kernel's lanes take 8 quads (tiles of
// 8192), so a block reads each copy in 16 KiB runs, and a wave keeps at most
// kWideInflight gradient loads in flight; with fewer copies, and in the
// averaging pass, 4 quads per lane and eight copies' loads at once. See
// source_tile.
constexpr int kQuadsWide = 8;
constexpr int kWideCopies = 32;
constexpr int kWideInflight = 3;
constexpr int tile_inflight(int quads) { return quads == kQuadsWide ? kWideInflight : 0; }
// The averaging pass (checked pipeline) keeps 4 quads per lane. With
// kCappedReduceCopies to kWideCopies copies it takes the batched read: every
// load of a tile in flight at once, at most kBatchBlocksPerCU blocks per CU
// (reduce_batched); with more copies its waves keep at most kWideInflight
// gradient loads in flight at full residency; with fewer, eight copies' loads
// at once at full residency.
constexpr int kCappedReduceCopies = 8;
// With 2 to kWideCopies - 1 copies the update kernel takes the batched
// schedule (see adam_kernel): every load of a tile in flight at once, then the
// arithmetic, then the stores array by array, with at most kBatchBlocksPerCU
// blocks resident per compute unit. Residency is capped by giving each block
// an otherwise unused share of the CU's LDS (batch_lds_bytes). The update from
// an fp32 average (checked pipeline) keeps the per-quad schedule but runs at
// the same residency.
constexpr int kBatchBlocksPerCU = 2;
constexpr int kMaxGrid = 1 << 21;                    // blocks per launch (tiles beyond: grid-stride)
constexpr int kInlineReplicas = 64;                  // replica pointers carried in the kernel arguments

// Workspace: [0, kHeaderBytes) per-group level-2 norm partials, then one fp64
// partial per block of the last launch (reused launch after launch: the
// fold that consumes it runs before the next launch in stream order).
constexpr int kFoldBlocks = 256;                     // level-2 partials per group
constexpr size_t kHeaderBytes = static_cast<size_t>(ZERO_MAX_GROUPS) * kFoldBlocks * sizeof(double);
constexpr size_t kScratchBytes = static_cast<size_t>(kMaxGrid) * sizeof(double);
constexpr size_t kWorkspaceBytes = kHeaderBytes + kScratchBytes;

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
  float* master_alt;    // optimistic pipeline: the second state set
  float* m_alt;
  float* v_alt;
  void* param;          // flat_param + param_offset (already offset), or null
  int32_t param_dt;     // ZERO_DT_F16 / ZERO_DT_BF16 / 0
  int32_t param_align;  // 8, 4 or 2: largest power-of-two alignment of param, capped at 8
  double beta1_d, beta2_d;
  float lr, beta1, beta2, eps, c1, c2, decay;
  int32_t has_decay;
  int32_t group;
  const zero_step_state* state;
  double* partials;  // one per block (fused and optimistic pipelines); null in the checked one
  int64_t head;      // leading elements (0-3) block 0 updates one by one, so that the quad
                     // path starts where every array is aligned (see aligned_head)
  double* level2 = nullptr;  // the group's level-2 partials: a launch of at most kFoldBlocks
                             // blocks writes them directly instead of `partials` (no fold)
  int32_t fill = 0;          // set by the launcher: partial slots [grid, fill) are written as 0
};

// Arguments of the average kernel (checked pipeline) and of the single-copy scan.
struct ReduceArgs {
  GradSource src;
  int64_t n;
  float* avg_out;  // null: scan only
  const zero_step_state* state;
  double* partials;
  int64_t head;    // as AdamArgs::head
  double* level2 = nullptr;  // as AdamArgs::level2
  int32_t fill = 0;          // as AdamArgs::fill
};

// Fold one launch's block partials into a group's level-2 partials, in a
// fixed order (block j of the fold sums a fixed contiguous range).
struct FoldArgs {
  const double* partials;
  int64_t count;
  double* level2;  // kFoldBlocks entries of the group
};

struct FinalizeArgs {
  const double* level2;  // ZERO_MAX_GROUPS x kFoldBlocks
  zero_step_state* state;
  int32_t n_groups;
  int32_t mode;  // 0: norm, skip verdict, clip multiplier; 1: norm, then commit a static-scale step;
                 // 2: norm, then commit or discard an optimistic step (dynamic scale), or, when
                 //    max_grad_norm asks for clipping, defer the commit to the second pass
  int32_t skip_on_overflow;
  int32_t growth_interval;  // mode 2
  double max_grad_norm;     // modes 0 and 2: clip threshold (0 = none)
  double backoff, growth, min_scale;  // mode 2
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

// Rewrite a group's parameter slice from its current master when the step was voided.
struct RestoreArgs {
  const float* master;
  const float* master_alt;
  int64_t n;
  void* param;  // already offset
  int32_t param_dt;
  int32_t param_align;
  const zero_step_state* state;
};

enum SrcKind { kSrcAvg = 0, kSrcF16 = 1, kSrcBF16 = 2 };
// kRedo: the second pass of a clipped optimistic step (runs only when the
// norm asked for clipping; small resident grid so that it costs little otherwise)
enum StepMode { kFused = 0, kChecked = 1, kOptimistic = 2, kRedo = 3 };
constexpr int kRedoGrid = 65536;
constexpr int kScanGrid = 65536;  // blocks of the single-copy scan (each loops over tiles)

// Quads per lane of an update launch: the wide tile for the aligned path over
// kWideCopies or more copies, else kQuadsPerThread.
inline int tile_quads(int src_kind, bool vec, int n_d) {
  return vec && src_kind != kSrcAvg && n_d >= kWideCopies ? kQuadsWide : kQuadsPerThread;
}

// Upper bound on the blocks of every streaming launch set by
// zero_set_grid_limit (0: none beyond each launch's own cap). Tests lower it
// so that small shards run the grid-stride loops of every kernel.
extern std::atomic<int32_t> g_grid_limit;

// `grid` blocks, or fewer if zero_set_grid_limit asked for fewer.
inline int limit_grid(int grid) {
  const int32_t lim = g_grid_limit.load(std::memory_order_relaxed);
  return lim > 0 && lim < grid ? lim : grid;
}

// Blocks of a streaming launch over n elements (tiles of kBlock * quads * 4).
inline int stream_grid(int64_t n, int quads = kQuadsPerThread) {
  const int64_t tile = static_cast<int64_t>(kBlock) * quads * 4;
  int64_t tiles = (n + tile - 1) / tile;
  if (tiles < 1) tiles = 1;
  return limit_grid(static_cast<int>(tiles < kMaxGrid ? tiles : kMaxGrid));
}

// Launchers (kernels.hip). Each returns the hipError_t of its launches.
// `vec` selects the aligned quad path; *blocks receives the number of block
// partials the launch leaves to fold: its grid size, or 0 when it wrote the
// group's level-2 partials itself (args.level2 set and a grid of at most
// kFoldBlocks blocks).
// batch_lds: dynamic LDS bytes per block of the batched schedule's launches,
// which caps them at kBatchBlocksPerCU blocks per CU on the current device.
hipError_t launch_adam(const AdamArgs& a, int src_kind, bool vec, int mode, size_t batch_lds, hipStream_t s,
                       int* blocks);
// Whether an update launch takes the batched schedule.
inline bool batched(int src_kind, bool vec, int n_d) {
  return vec && src_kind != kSrcAvg && n_d > 1 && n_d < kWideCopies;
}
// LDS per block that leaves room for exactly kBatchBlocksPerCU blocks on a CU
// with lds_per_cu bytes (each block also holds the kernels' few static bytes),
// at most 64 KiB.
inline size_t batch_lds_bytes(size_t lds_per_cu) {
  size_t b = lds_per_cu / kBatchBlocksPerCU;
  b = b > 1024 ? (b - 1024) / 256 * 256 : 0;
  return b < (64u << 10) ? b : (64u << 10);
}
// Whether an averaging launch takes the batched read (batch_lds as above).
inline bool reduce_batched(bool vec, int n_d) {
  return vec && n_d >= kCappedReduceCopies && n_d <= kWideCopies;
}
hipError_t launch_reduce(const ReduceArgs& a, int src_kind, bool vec, size_t batch_lds, hipStream_t s,
                         int* blocks);
// Single-copy scan (partials only) of a 16-byte-aligned copy; scan_grid(n) blocks, one partial each.
hipError_t launch_scan(const ReduceArgs& a, int src_kind, hipStream_t s, int* blocks);
int scan_grid(int64_t n);
hipError_t launch_fold(const FoldArgs& a, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_redo_commit(const CommitArgs& a, hipStream_t s);
hipError_t launch_state_init(zero_step_state* st, float loss_scale, hipStream_t s);
hipError_t launch_cast(const CastArgs& a, bool vec, hipStream_t s);
// Device address (on the current device) of the kWorkspaceBytes static
// scratch array that zero_adam_step_static uses instead of a workspace.
hipError_t static_scratch(void** ptr);
hipError_t launch_restore(const RestoreArgs& a, bool vec, hipStream_t s);

}  // namespace zdp
