// Host-side logic of the C ABI under the address and undefined-behaviour
// sanitizers: the partition index map at extreme sizes, tensor slices, the
// arena planner, and the argument checks of every device call (which must
// fail before any launch; the launchers here abort if reached).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "zero_dp.h"
#include "../../zero_dp_partitioned_amd/csrc/zero_dp_internal.h"

static int failures = 0;
#define EXPECT(cond)                                                 \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "line %d: %s failed (%s)\n", __LINE__, #cond, zero_last_error()); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static void partitions() {
  const int64_t numels[] = {0, 1, 7, 787971, 1557611200LL, 13000000000LL, INT64_MAX - 5, INT64_MAX};
  const int32_t nds[] = {1, 2, 3, 8, 64, 1023, 4096};
  const int64_t aligns[] = {1, 2, 64, 1LL << 40};
  for (int64_t numel : numels)
    for (int32_t nd : nds)
      for (int64_t al : aligns) {
        std::vector<zero_segment> segs(nd);
        int64_t padded = -1;
        const int rc = zero_partition(numel, nd, al, segs.data(), &padded);
        if (rc != ZERO_OK) {
          EXPECT(rc == ZERO_ERR_INVALID_ARG);  // only padding overflow may fail
          continue;
        }
        int64_t at = 0;
        for (int32_t r = 0; r < nd; ++r) {
          EXPECT(segs[r].offset == at);
          at += segs[r].size;
        }
        EXPECT(at == padded);
      }
  zero_segment one;
  EXPECT(zero_partition(-1, 1, 1, &one, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_partition(10, 0, 1, &one, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_partition(10, 1, 0, &one, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_partition(10, 1, 1, nullptr, nullptr) == ZERO_ERR_INVALID_ARG);
}

static void slices() {
  const int64_t numels[] = {512 * 768, 768, 768 * 513, 3};
  zero_tensor_slice out[4];
  int32_t n_out = -1;
  for (int32_t r = 0; r < 4; ++r) {
    EXPECT(zero_partition_tensors(numels, 4, 4, r, 1, out, 4, &n_out) == ZERO_OK);
    int64_t covered = 0;
    for (int32_t i = 0; i < n_out; ++i) covered += out[i].length;
    EXPECT(covered == 196993 - (r >= 3 ? 1 : 0) || covered == 196993);
  }
  EXPECT(zero_partition_tensors(numels, 4, 4, 1, 1, out, 1, &n_out) == ZERO_ERR_INVALID_ARG);
  const int64_t big[] = {INT64_MAX, 1};
  EXPECT(zero_partition_tensors(big, 2, 2, 0, 1, out, 4, &n_out) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_partition_tensors(numels, 4, 4, 4, 1, out, 4, &n_out) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_partition_tensors(nullptr, 4, 4, 0, 1, out, 4, &n_out) == ZERO_ERR_INVALID_ARG);
}

static void arenas() {
  std::vector<zero_arena_buffer> b(40);
  for (int i = 0; i < 40; ++i) {
    b[i].bytes = (int64_t)(i * 7919 % 1000 + 1) << 20;
    b[i].traffic = i * 31 % 17;
  }
  int64_t total = 0;
  EXPECT(zero_plan_arena(b.data(), 40, 1LL << 30, 0, 64LL << 30, &total) == ZERO_ERR_UNSUPPORTED);  // 16 x 1 GiB < 20 GiB
  EXPECT(zero_plan_arena(b.data(), 40, 4LL << 30, 0, 64LL << 30, &total) == ZERO_OK);
  EXPECT(total > 0);
  EXPECT(zero_plan_arena(b.data(), 40, 0, 3, 280LL << 30, &total) == ZERO_OK);
  b[3].bytes = INT64_MAX;
  EXPECT(zero_plan_arena(b.data(), 40, 0, 0, 280LL << 30, &total) == ZERO_ERR_INVALID_ARG);
  b[3].bytes = INT64_MAX - (4LL << 20);
  EXPECT(zero_plan_arena(b.data(), 40, 0, 0, INT64_MAX, &total) == ZERO_ERR_UNSUPPORTED);
  b[3].bytes = 1;
  EXPECT(zero_plan_arena(b.data(), 40, 0, 16, INT64_MAX, &total) == ZERO_OK);
  EXPECT(zero_plan_arena(b.data(), 40, 0, 17, INT64_MAX, &total) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_plan_arena(b.data(), 0, 0, 0, INT64_MAX, &total) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_plan_arena(b.data(), 40, 3, 0, INT64_MAX, &total) == ZERO_ERR_INVALID_ARG);
}

static void device_call_checks() {
  alignas(256) static char ws[64];
  const size_t wsb = zero_workspace_bytes(1);
  EXPECT(wsb > 0 && zero_workspace_bytes(0) == 0 && zero_workspace_bytes(9) == 0);
  void* fake = (void*)0x100000;
  zero_step_state* st = (zero_step_state*)0x100000;
  EXPECT(zero_state_init(nullptr, 1.0f, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_state_init((zero_step_state*)0x100001, 1.0f, nullptr) == ZERO_ERR_ALIGNMENT);
  EXPECT(zero_state_init(st, 0.0f, nullptr) == ZERO_ERR_INVALID_ARG);
  const void* reps[2] = {fake, fake};
  EXPECT(zero_reduce_grad_segment(reps, 2, 1, -1, (float*)fake, fake, wsb, 0, st, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_reduce_grad_segment(reps, 2, 1, 10, (float*)fake, ws, 64, 0, st, nullptr) == ZERO_ERR_WORKSPACE);
  EXPECT(zero_reduce_grad_segment(reps, 0, 1, 10, (float*)fake, fake, wsb, 0, st, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_reduce_grad_segment(reps, 5000, 1, 10, (float*)fake, fake, wsb, 0, st, nullptr) == ZERO_ERR_UNSUPPORTED);
  EXPECT(zero_reduce_grad_segment(reps, 2, 7, 10, (float*)fake, fake, wsb, 0, st, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_reduce_grad_segment(reps, 2, 1, 10, (float*)fake, fake, wsb, 8, st, nullptr) == ZERO_ERR_WORKSPACE);
  const int64_t counts[1] = {-3};
  EXPECT(zero_grad_norm_overflow(reps, counts, 1, 1, fake, wsb, nullptr, st, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_grad_norm_overflow(nullptr, nullptr, 1, 0, fake, wsb, nullptr, st, nullptr) == ZERO_ERR_INVALID_ARG);
  zero_policy bad;
  memset(&bad, 0, sizeof bad);
  bad.max_grad_norm = -1.0;
  EXPECT(zero_grad_norm_overflow(nullptr, nullptr, 1, 1, fake, wsb, &bad, st, nullptr) == ZERO_ERR_INVALID_ARG);
  zero_group g;
  memset(&g, 0, sizeof g);
  g.n = 10;
  g.replicas = reps;
  g.n_d = 2;
  g.grad_dt = 1;
  g.master = g.exp_avg = g.exp_avg_sq = (float*)fake;
  g.lr = 1e-3;
  g.beta1 = 0.9;
  g.beta2 = 0.999;
  g.eps = 1e-8;
  g.beta1 = 1.5;
  EXPECT(zero_adam_step(&g, 1, nullptr, fake, wsb, st, nullptr) == ZERO_ERR_INVALID_ARG);
  g.beta1 = 0.9;
  g.master = (float*)0x100002;
  EXPECT(zero_adam_step(&g, 1, nullptr, fake, wsb, st, nullptr) == ZERO_ERR_ALIGNMENT);
  g.master = (float*)fake;
  g.avg = (const float*)fake;  // both sources
  EXPECT(zero_adam_step(&g, 1, nullptr, fake, wsb, st, nullptr) == ZERO_ERR_INVALID_ARG);
  g.avg = nullptr;
  zero_policy opt;
  memset(&opt, 0, sizeof opt);
  opt.optimistic = 1;
  EXPECT(zero_adam_step(&g, 1, &opt, fake, wsb, st, nullptr) == ZERO_ERR_INVALID_ARG);
  opt.skip_on_overflow = 1;
  opt.backoff = 0.5;
  opt.growth = 2.0;
  opt.min_scale = 1.0;
  EXPECT(zero_adam_step(&g, 1, &opt, fake, wsb, st, nullptr) == ZERO_ERR_INVALID_ARG);  // no *_alt set
  EXPECT(zero_adam_step(&g, 9, nullptr, fake, wsb, st, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_cast_writeback((const float*)fake, 10, fake, -1, 1, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_cast_writeback((const float*)0x100001, 10, fake, 0, 1, nullptr) == ZERO_ERR_ALIGNMENT);
  EXPECT(zero_cast_writeback((const float*)fake, 0, fake, 0, 1, nullptr) == ZERO_OK);  // nothing to write
  // the test knob on the grid size: any cap >= 0 is taken, a negative one refused
  EXPECT(zero_set_grid_limit(-1) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_set_grid_limit(3) == ZERO_OK);
  EXPECT(zdp::stream_grid(int64_t(1) << 40) == 3 && zdp::stream_grid(10) == 1);
  EXPECT(zero_set_grid_limit(0) == ZERO_OK);
  EXPECT(zdp::stream_grid(int64_t(1) << 40) == zdp::kMaxGrid && zdp::stream_grid(4097) == 2);
  // the copy probe's argument checks
  EXPECT(zero_copy_probe(fake, fake, fake, fake, -16, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_copy_probe(fake, fake, fake, fake, 17, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_copy_probe(fake, fake, fake, nullptr, 32, nullptr) == ZERO_ERR_INVALID_ARG);
  EXPECT(zero_copy_probe(fake, (void*)0x100008, fake, fake, 32, nullptr) == ZERO_ERR_ALIGNMENT);
  EXPECT(zero_copy_probe(nullptr, nullptr, nullptr, nullptr, 0, nullptr) == ZERO_OK);  // nothing to copy
}

// Which launches take the batched schedule (update) and the batched read
// (averaging pass), and the LDS share that caps their residency.
static void launch_shapes() {
  using namespace zdp;
  EXPECT(!batched(kSrcF16, true, 1) && batched(kSrcF16, true, 2) && batched(kSrcBF16, true, 31));
  EXPECT(!batched(kSrcF16, true, 32) && !batched(kSrcAvg, true, 8) && !batched(kSrcF16, false, 8));
  EXPECT(!reduce_batched(true, 7) && reduce_batched(true, 8) && reduce_batched(true, 32));
  EXPECT(!reduce_batched(true, 33) && !reduce_batched(false, 16));
  const size_t b160 = batch_lds_bytes(160u << 10), b64 = batch_lds_bytes(64u << 10);
  EXPECT(b160 == (64u << 10) && 2 * (b160 + 1024) <= (160u << 10) && 3 * b160 > (160u << 10));
  EXPECT(b64 % 256 == 0 && 2 * (b64 + 1024) <= (64u << 10) && 3 * b64 > (64u << 10));
}

int main() {
  partitions();
  slices();
  arenas();
  device_call_checks();
  launch_shapes();
  if (failures) {
    fprintf(stderr, "host checks: %d failure(s)\n", failures);
    return 1;
  }
  printf("host checks: ok\n");
  return 0;
}
