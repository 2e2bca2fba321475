/*
 * A plain C consumer of the zero_dp C ABI: no torch, no Python.
 *
 * Lays out one rank's shard the way a training loop would (rank `rank` of
 * `n_d` over a flat fp16 vector of `psi` elements), places its buffers in one
 * hipMalloc'd arena at the offsets zero_plan_arena gives (64 MiB regions, so
 * the arena stays small), fills the inputs from a fixed integer recipe, runs
 * `steps` steps on the null stream, and writes the inputs and results to a
 * binary file for the test to check against the CPU oracle:
 *
 *   step_demo OUT PSI N_D RANK STEPS [checked]
 *
 * Default: the fused pipeline (zero_adam_step on the copies, static loss
 * scale 1). "checked": the verdict before the update, with a dynamic loss
 * scale starting at 1024 -- zero_reduce_grad_segment averages the copies into
 * an fp32 buffer, zero_grad_norm_overflow forms the norm and the skip verdict,
 * zero_adam_step updates from the average; the second step has +inf written
 * into the last copy at element size / 2, so it is voided and the scale
 * halves. Either way the program ends with zero_cast_writeback of the master
 * into a bf16 copy of the flat vector at the rank's offset.
 *
 * File layout (little endian): int64 psi, n_d, rank, offset, size, steps,
 * checked; uint16 replicas[steps][n_d][size] (as stepped, the inf included);
 * float master0[size]; float master[size], m[size], v[size]; uint16 flat[psi]
 * (after); uint16 flat0[psi] (before); uint16 cast[psi] (the bf16 vector
 * after the cast; before it, flat0's bits); double grad_norm_sq; int64 step;
 * float loss_scale; int32 overflow, skipped.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_dp.h"

#define HIP_OK(x)                                                             \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

#define ZERO_OK_OR_DIE(x)                                                     \
  do {                                                                        \
    int rc_ = (x);                                                            \
    if (rc_ != ZERO_OK) {                                                     \
      fprintf(stderr, "zero_dp error %d: %s (line %d)\n", rc_, zero_last_error(), __LINE__); \
      exit(3);                                                                \
    }                                                                         \
  } while (0)

/* a small deterministic integer mix, turned into fp16 bits of a modest value */
static uint32_t mix(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdULL;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ULL;
  x ^= x >> 33;
  return (uint32_t)x;
}

static uint16_t grad_bits(uint64_t key) {
  /* fp16 with exponent 5..14 (values about 3e-5 .. 0.5), random sign and mantissa */
  uint32_t h = mix(key);
  uint16_t sign = (uint16_t)((h >> 31) << 15);
  uint16_t expo = (uint16_t)(5 + (h >> 10) % 10);
  uint16_t frac = (uint16_t)(h & 0x3ff);
  return sign | (uint16_t)(expo << 10) | frac;
}

int main(int argc, char** argv) {
  if (argc != 6 && argc != 7) {
    fprintf(stderr, "usage: %s OUT PSI N_D RANK STEPS [checked]\n", argv[0]);
    return 1;
  }
  const int checked = argc == 7 && strcmp(argv[6], "checked") == 0;
  if (argc == 7 && !checked) {
    fprintf(stderr, "bad arguments\n");
    return 1;
  }
  const char* out_path = argv[1];
  const int64_t psi = atoll(argv[2]);
  const int32_t n_d = atoi(argv[3]);
  const int32_t rank = atoi(argv[4]);
  const int64_t steps = atoll(argv[5]);
  if (n_d < 1 || n_d > 64 || rank < 0 || rank >= n_d || psi < 1 || steps < 1) {
    fprintf(stderr, "bad arguments\n");
    return 1;
  }

  zero_segment* segs = malloc(sizeof(zero_segment) * (size_t)n_d);
  ZERO_OK_OR_DIE(zero_partition(psi, n_d, 1, segs, NULL));
  const int64_t off = segs[rank].offset, n = segs[rank].size;
  free(segs);

  /* host inputs */
  uint16_t* flat0 = malloc(sizeof(uint16_t) * (size_t)psi);
  for (int64_t i = 0; i < psi; ++i) flat0[i] = grad_bits(0x5eed0000ULL + (uint64_t)i);
  float* master0 = malloc(sizeof(float) * (size_t)n);
  for (int64_t j = 0; j < n; ++j) master0[j] = ((float)(mix(0xabcULL + (uint64_t)j) % 20001) - 10000.0f) * 2e-6f;
  uint16_t* reps = malloc(sizeof(uint16_t) * (size_t)(steps * n_d * n));
  for (int64_t k = 0; k < steps; ++k)
    for (int32_t r = 0; r < n_d; ++r)
      for (int64_t j = 0; j < n; ++j)
        reps[(k * n_d + r) * n + j] = grad_bits(((uint64_t)k << 48) ^ ((uint64_t)r << 40) ^ (uint64_t)(off + j));
  if (checked && steps >= 2) reps[(1 * n_d + (n_d - 1)) * n + n / 2] = 0x7C00; /* +inf: the second step overflows */

  /* device buffers, owned here: master, m, v, the n_d copies (one buffer),
   * the flat vector, the fp32 average (checked pipeline) and the bf16 copy of
   * the flat vector the final cast writes into, carved from one arena */
  enum { NB = 7 };
  zero_arena_buffer plan[NB];
  memset(plan, 0, sizeof plan);
  const int64_t sizes[NB] = {4 * n, 4 * n, 4 * n, 2 * n * n_d, 2 * psi, 4 * n, 2 * psi};
  const int64_t traffic[NB] = {8 * n, 8 * n, 8 * n, 2 * n * n_d, 2 * n, 8 * n, 2 * n};
  for (int i = 0; i < NB; ++i) {
    plan[i].bytes = sizes[i] > 0 ? sizes[i] : 1;
    plan[i].traffic = traffic[i];
  }
  int64_t arena_bytes = 0;
  ZERO_OK_OR_DIE(zero_plan_arena(plan, NB, 64LL << 20, 0, 1LL << 30, &arena_bytes));
  char* d_arena;
  HIP_OK(hipMalloc((void**)&d_arena, (size_t)arena_bytes));
  float* d_master = (float*)(d_arena + plan[0].offset);
  float* d_m = (float*)(d_arena + plan[1].offset);
  float* d_v = (float*)(d_arena + plan[2].offset);
  uint16_t* d_reps = (uint16_t*)(d_arena + plan[3].offset);
  uint16_t* d_flat = (uint16_t*)(d_arena + plan[4].offset);
  float* d_avg = (float*)(d_arena + plan[5].offset);
  uint16_t* d_cast = (uint16_t*)(d_arena + plan[6].offset);
  void *d_ws, *d_state;
  const size_t ws_bytes = zero_workspace_bytes(1);
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMalloc(&d_state, sizeof(zero_step_state)));
  HIP_OK(hipMemcpy(d_master, master0, sizeof(float) * (size_t)n, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(d_m, 0, sizeof(float) * (size_t)n));
  HIP_OK(hipMemset(d_v, 0, sizeof(float) * (size_t)n));
  HIP_OK(hipMemcpy(d_flat, flat0, sizeof(uint16_t) * (size_t)psi, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_cast, flat0, sizeof(uint16_t) * (size_t)psi, hipMemcpyHostToDevice));
  ZERO_OK_OR_DIE(zero_state_init((zero_step_state*)d_state, checked ? 1024.0f : 1.0f, NULL));
  zero_policy policy;
  memset(&policy, 0, sizeof policy);
  policy.skip_on_overflow = 1;
  policy.growth_interval = 1000;
  policy.backoff = 0.5;
  policy.growth = 2.0;
  policy.min_scale = 1.0;

  const void* rep_ptrs[64];
  for (int32_t r = 0; r < n_d; ++r) rep_ptrs[r] = d_reps + (size_t)r * (size_t)n;
  zero_group g;
  memset(&g, 0, sizeof g);
  g.n = n;
  g.replicas = rep_ptrs;
  g.n_d = n_d;
  g.grad_dt = ZERO_DT_F16;
  g.master = d_master;
  g.exp_avg = d_m;
  g.exp_avg_sq = d_v;
  g.flat_param = d_flat;
  g.param_offset = off;
  g.param_dt = ZERO_DT_F16;
  g.lr = 1e-3;
  g.beta1 = 0.9;
  g.beta2 = 0.999;
  g.eps = 1e-8;
  g.weight_decay = 0.01;
  zero_step_state* st_dev = (zero_step_state*)d_state;
  for (int64_t k = 0; k < steps; ++k) {
    HIP_OK(hipMemcpy(d_reps, reps + k * n_d * n, sizeof(uint16_t) * (size_t)(n_d * n), hipMemcpyHostToDevice));
    if (!checked) {
      ZERO_OK_OR_DIE(zero_adam_step(&g, 1, NULL, d_ws, ws_bytes, st_dev, NULL));
      continue;
    }
    /* the verdict first: average, norm and flag, then the update from the average */
    ZERO_OK_OR_DIE(zero_reduce_grad_segment(rep_ptrs, n_d, ZERO_DT_F16, n, d_avg, d_ws, ws_bytes, 0, st_dev, NULL));
    ZERO_OK_OR_DIE(zero_grad_norm_overflow(NULL, NULL, ZERO_DT_F16, 1, d_ws, ws_bytes, &policy, st_dev, NULL));
    g.replicas = NULL;
    g.n_d = 0;
    g.avg = d_avg;
    ZERO_OK_OR_DIE(zero_adam_step(&g, 1, &policy, d_ws, ws_bytes, st_dev, NULL));
    g.replicas = rep_ptrs;
    g.n_d = n_d;
    g.avg = NULL;
  }
  /* the master, rounded to bf16, into the other copy of the flat vector */
  ZERO_OK_OR_DIE(zero_cast_writeback(d_master, n, d_cast, off, ZERO_DT_BF16, NULL));
  HIP_OK(hipDeviceSynchronize());

  float* master = malloc(sizeof(float) * (size_t)n);
  float* m = malloc(sizeof(float) * (size_t)n);
  float* v = malloc(sizeof(float) * (size_t)n);
  uint16_t* flat = malloc(sizeof(uint16_t) * (size_t)psi);
  uint16_t* cast = malloc(sizeof(uint16_t) * (size_t)psi);
  zero_step_state st;
  HIP_OK(hipMemcpy(master, d_master, sizeof(float) * (size_t)n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(m, d_m, sizeof(float) * (size_t)n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(v, d_v, sizeof(float) * (size_t)n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(flat, d_flat, sizeof(uint16_t) * (size_t)psi, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(cast, d_cast, sizeof(uint16_t) * (size_t)psi, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&st, d_state, sizeof st, hipMemcpyDeviceToHost));

  FILE* f = fopen(out_path, "wb");
  if (!f) return 4;
  const int64_t hdr[7] = {psi, n_d, rank, off, n, steps, checked};
  fwrite(hdr, sizeof hdr, 1, f);
  fwrite(reps, sizeof(uint16_t), (size_t)(steps * n_d * n), f);
  fwrite(master0, sizeof(float), (size_t)n, f);
  fwrite(master, sizeof(float), (size_t)n, f);
  fwrite(m, sizeof(float), (size_t)n, f);
  fwrite(v, sizeof(float), (size_t)n, f);
  fwrite(flat, sizeof(uint16_t), (size_t)psi, f);
  fwrite(flat0, sizeof(uint16_t), (size_t)psi, f);
  fwrite(cast, sizeof(uint16_t), (size_t)psi, f);
  fwrite(&st.grad_norm_sq, sizeof(double), 1, f);
  fwrite(&st.step, sizeof(int64_t), 1, f);
  fwrite(&st.loss_scale, sizeof(float), 1, f);
  fwrite(&st.overflow, sizeof(int32_t), 1, f);
  fwrite(&st.skipped, sizeof(int32_t), 1, f);
  fclose(f);
  printf("step_demo: %s psi=%lld n_d=%d rank=%d offset=%lld n=%lld steps=%lld norm=%g scale=%g arena=%lld bytes, "
         "regions", checked ? "checked" : "fused", (long long)psi, n_d, rank, (long long)off, (long long)n,
         (long long)steps, (double)st.grad_norm, (double)st.loss_scale, (long long)arena_bytes);
  for (int i = 0; i < NB; ++i) printf(" %d", plan[i].region);
  printf("\n");

  hipFree(d_arena);
  hipFree(d_ws);
  hipFree(d_state);
  free(flat0);
  free(master0);
  free(reps);
  free(master);
  free(m);
  free(v);
  free(flat);
  free(cast);
  return 0;
}
