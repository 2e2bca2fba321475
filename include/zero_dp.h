/*
 * zero_dp.h -- C ABI of the ZeRO-DP partitioned optimizer step for AMD MI355X
 * (gfx950). One rank's shard, on one GPU.
 *
 * The step follows the pages on ZeRO:
 *   - "DeepSpeed ZeRO stage 1/2" walkthrough ("01 · ZeRO 的显存数学与 Stage 1/2"):
 *     §3 (flatten a parameter group into one vector, split it into N_d
 *     segments, each rank owns one), §4 ② (base = numel / N_d, remainder to the
 *     first ranks), §4 ④ / §7 (a tensor may straddle two segments; alignment
 *     padding), §6 (step: overflow check and skip, global norm, unscale, Adam on
 *     the shard, copy the fp32 shard back into the 16-bit flat vector).
 *   - "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
 *     reading notes, second part §3 (per-coordinate Adam update) and §4 (the
 *     averaged shard is (1/N_d) * sum over ranks of that shard).
 *   - ZeRO paper translation, §3.1 (fp16/bf16 params and grads, fp32 master,
 *     momentum and variance).
 *
 * Conventions for every call:
 *   - All device buffers are owned by the caller. The library never allocates
 *     or frees device memory and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *     is enqueued asynchronously, in stream order; no call synchronises the
 *     host. Scalar results (norm, overflow flag, loss scale, step count) stay in
 *     the device-resident zero_step_state.
 *   - Arguments are checked on the host before anything is enqueued: a
 *     non-zero return other than ZERO_ERR_HIP means nothing was launched, and
 *     zero_last_error() gives a thread-local message. ZERO_ERR_HIP reports a
 *     failed launch; launches of the same call before it stay enqueued.
 *     Numerical overflow is not an error; it is a flag. A device fault
 *     surfaces at the caller's next synchronisation.
 *   - Buffer extents are the caller's to get right: the library knows
 *     pointers, counts and offsets, not allocation sizes (for example
 *     flat_param must hold param_offset + n elements).
 *   - Calls on different streams with disjoint buffers may run concurrently.
 *     Calls that share a workspace or a state must be ordered by the caller.
 *   - Element counts and offsets are int64 (offsets above 2^32 are normal).
 */
#ifndef ZERO_DP_H
#define ZERO_DP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define ZERO_OK 0
#define ZERO_ERR_INVALID_ARG (-1) /* null pointer, bad count, dtype, rank ... */
#define ZERO_ERR_ALIGNMENT (-2)   /* fp32 pointer not 4-byte, 16-bit not 2-byte aligned */
#define ZERO_ERR_WORKSPACE (-3)   /* workspace missing or group index out of range */
#define ZERO_ERR_HIP (-4)         /* a HIP runtime call or launch failed */
#define ZERO_ERR_UNSUPPORTED (-5) /* device is not gfx950, or a size limit below */

/* ---- limits ------------------------------------------------------------ */
#define ZERO_MAX_GROUPS 8       /* parameter groups per step / per state */
#define ZERO_MAX_REPLICAS 4096  /* N_d */

/* ---- dtypes (values are part of the ABI) -------------------------------- */
#define ZERO_DT_F16 1  /* IEEE binary16 */
#define ZERO_DT_BF16 2 /* bfloat16 */

/* One rank's segment of a flat vector: elements [offset, offset + size). */
typedef struct {
  int64_t offset;
  int64_t size;
} zero_segment;

/* The part of tensor `tensor` that lies inside a rank's segment:
 * shard[shard_begin + i] is tensor[tensor_begin + i] for i < length. */
typedef struct {
  int32_t tensor;
  int32_t reserved;
  int64_t shard_begin;
  int64_t tensor_begin;
  int64_t length;
} zero_tensor_slice;

/* Optimizer and loss-scale state of one rank, resident in device memory.
 * Allocate sizeof(zero_step_state) bytes (8-byte aligned) and fill it with
 * zero_state_init(). The kernels read and write it; the host reads it after
 * synchronising (for example to log the norm or the loss scale). */
typedef struct {
  double beta1_pow[ZERO_MAX_GROUPS]; /* beta1^t per group (t = applied steps), by
                                        successive fp64 multiplication       */
  double beta2_pow[ZERO_MAX_GROUPS]; /* beta2^t per group                    */
  double grad_norm_sq;  /* last step: sum of squares of the unscaled averaged
                           gradient over all groups, in fp64                  */
  float grad_norm;      /* sqrt(grad_norm_sq) rounded to fp32                  */
  float loss_scale;     /* S: stored gradients are the true ones times S       */
  int64_t step;         /* applied steps t                                     */
  int32_t overflow;     /* last step: 1 if any averaged gradient was inf/NaN   */
  int32_t skipped;      /* last step: 1 if it was voided by the overflow check */
  int32_t good_steps;   /* applied steps since the last loss-scale change      */
  float clip_coef;      /* last step: gradient-clipping multiplier (1 = none)  */
  int32_t cur;          /* optimistic pipeline: 0 = master/exp_avg/exp_avg_sq
                           hold the current state, 1 = the *_alt arrays do    */
  int32_t redo;         /* optimistic pipeline with clipping: 1 between the
                           norm and the second pass of a clipped step (0 once
                           zero_adam_step's work has run)                    */
} zero_step_state;

/* Step policy: loss scaling and gradient clipping.
 * skip_on_overflow = 0: static scale, every step applies (an inf/NaN gradient
 *   then propagates into the state).
 * skip_on_overflow = 1: dynamic scale: a step whose averaged gradient holds
 *   inf/NaN changes nothing but the scale (S <- max(S * backoff, min_scale));
 *   after growth_interval applied steps in a row, S <- S * growth
 *   (growth_interval 0 = never).
 * max_grad_norm > 0: clip the unscaled gradient to this global norm
 *   [DeepSpeed walkthrough §6 step 3, unscaling and clipping]: multiplier
 *   c = min(1, max_norm / (norm + 1e-6)) formed in fp64 and rounded once to
 *   fp32, g <- (avg * (1/S)) * c; 0 = no clipping.
 * optimistic = 1 (with skip_on_overflow = 1): instead of waiting for the
 *   overflow verdict and the norm, update into a second state set and commit
 *   or discard it afterwards; a step the norm says to clip is recomputed from
 *   the current set by a second pass (see zero_adam_step).
 * Skipping or clipping without `optimistic` needs the norm before the update
 * and selects the checked pipeline. */
typedef struct {
  int32_t skip_on_overflow;
  int32_t growth_interval;
  int32_t optimistic;
  int32_t reserved;
  double backoff;
  double growth;
  double min_scale;
  double max_grad_norm;
} zero_policy;

/* One parameter group's shard for zero_adam_step().
 * Gradient source, exactly one of:
 *   replicas: host array of n_d device pointers, each to n elements of
 *             grad_dt: the N_d gradient copies of this rank's segment. Their
 *             average is formed in the kernel (fused mode), or
 *   avg:      device fp32 [n] average written by zero_reduce_grad_segment().
 * State: master, exp_avg (m), exp_avg_sq (v): device fp32 [n], updated in place.
 *   The optimistic pipeline also needs master_alt, exp_avg_alt, exp_avg_sq_alt
 *   (fp32 [n], contents ignored until first written); NULL otherwise.
 * Writeback: flat_param (device, param_dt elements) receives the updated master
 *   rounded to 16 bits at elements [param_offset, param_offset + n); NULL skips
 *   it. Any 2-byte alignment of flat_param + param_offset is accepted.
 * Speed: the fast path moves 4 elements per access; it needs master, exp_avg,
 *   exp_avg_sq (and the *_alt set, and avg or every replica) to start at the
 *   same offset modulo 4 elements, as views into flat buffers at one segment
 *   offset do (up to 3 leading elements are then updated one by one). Arrays
 *   at different offsets are still handled exactly, element by element, at
 *   well under half the bandwidth.
 * Hyperparameters: lr, beta1, beta2, eps; weight_decay != 0 applies decoupled
 *   (AdamW) decay master *= (1 - lr * weight_decay) before the Adam update. */
typedef struct {
  int64_t n;
  const void* const* replicas;
  int32_t n_d;
  int32_t grad_dt;
  const float* avg;
  float* master;
  float* exp_avg;
  float* exp_avg_sq;
  float* master_alt;
  float* exp_avg_alt;
  float* exp_avg_sq_alt;
  void* flat_param;
  int64_t param_offset;
  int32_t param_dt;
  int32_t reserved;
  double lr, beta1, beta2, eps, weight_decay;
} zero_group;

/* ---- host-only calls ---------------------------------------------------- */

/* Partition a flat vector of `numel` elements over n_d ranks [DeepSpeed
 * walkthrough §4 ②]: after optional padding of numel up to a multiple of
 * align_elems (1 = none) [§4 ①, §7], base = padded / n_d, rem = padded % n_d,
 * rank r gets base + (r < rem) elements starting at r * base + min(r, rem).
 * segs: host array of n_d entries (written). padded_numel: may be NULL.
 * Errors: INVALID_ARG for numel < 0, n_d < 1, align_elems < 1, NULL segs,
 * int64 overflow. */
int zero_partition(int64_t numel, int32_t n_d, int64_t align_elems,
                   zero_segment* segs, int64_t* padded_numel);

/* The tensor slices inside rank `rank`'s segment when n_tensors tensors of
 * numels[i] elements are laid end to end into one flat vector and partitioned
 * as zero_partition() does [DeepSpeed walkthrough §3 ①, §4 ④]. Writes up to
 * `cap` entries of `out` in tensor order and their count to *n_out.
 * Errors: INVALID_ARG (bad counts, rank out of range, cap too small). */
int zero_partition_tensors(const int64_t* numels, int32_t n_tensors, int32_t n_d,
                           int32_t rank, int64_t align_elems, zero_tensor_slice* out,
                           int32_t cap, int32_t* n_out);

/* Bytes of device workspace the step calls need for up to n_groups groups:
 * the gradient-norm partials (about 16 MiB, the same for any shard size and
 * any n_groups in range). 0 if n_groups is out of range. The workspace must
 * be 256-byte aligned; its contents need no initialisation. Every call that
 * takes a workspace also takes its size and returns ZERO_ERR_WORKSPACE if it
 * is smaller. */
size_t zero_workspace_bytes(int32_t n_groups);

/* ---- placement in HBM (host-only) ----------------------------------------
 * Not an operation of the pages: a layout helper for MI355X. Its 288 GiB of
 * HBM3E behave as three address regions of 96 GiB (which matches the three
 * stack-ID groups of its 12-high stacks; the cause is inferred, the effect
 * measured). Measured on gfx950 with this library's step kernels:
 * when every stream of a step lies in one region the step sustains about
 * 5.4 TB/s; with its traffic spread over two or more regions about 6.4 TB/s.
 * HIP exposes no physical addresses, so the helper plans byte offsets inside
 * one arena that the caller allocates in a single piece, first, taking all
 * free device memory but a small reserve: such an allocation is backed across
 * the whole of HBM in address order, so offset ranges of the arena fall into
 * the regions (to within the few MiB the runtime holds below it). A smaller
 * allocation is backed wherever the driver finds room and gives no such
 * guarantee. The rest of each region stays free for the caller's other data
 * (weights, activations). */
#define ZERO_HBM_REGION_BYTES (96LL << 30)
#define ZERO_ARENA_ALIGN (2LL << 20) /* offsets and sizes are rounded to 2 MiB */

typedef struct {
  int64_t bytes;   /* in: buffer size, > 0 */
  int64_t traffic; /* in: bytes a step moves through it (reads + writes), >= 0 */
  int64_t offset;  /* out: byte offset from the arena base, a multiple of ZERO_ARENA_ALIGN */
  int32_t region;  /* out: index of the region the buffer lies in */
  int32_t reserved;
} zero_arena_buffer;

/* Plan offsets for n_buffers buffers in one arena. Regions are
 * [r * region_bytes, (r + 1) * region_bytes), the last cut at max_bytes (the
 * largest arena the caller can allocate). Buffers are taken heaviest traffic
 * first (ties: larger first, then lower index); each goes to the region with
 * the least traffic so far among those with room for it (ties: lower region),
 * packed upward from that region's start. region_bytes: 0 means
 * ZERO_HBM_REGION_BYTES, else a multiple of ZERO_ARENA_ALIGN. n_regions: 0
 * means the fewest regions, at least two where max_bytes allows, that hold
 * every buffer (at most 16); else exactly that many. *arena_bytes receives the
 * end of the last buffer (the size to allocate). buffers is a host array; the
 * plan depends only on the arguments.
 * Errors: INVALID_ARG (bad counts or sizes), UNSUPPORTED (the buffers do not
 * fit below max_bytes). */
int zero_plan_arena(zero_arena_buffer* buffers, int32_t n_buffers, int64_t region_bytes,
                    int32_t n_regions, int64_t max_bytes, int64_t* arena_bytes);

/* Thread-local text of the last error returned on this thread. */
const char* zero_last_error(void);

/* ---- device calls -------------------------------------------------------- */

/* Initialise a device zero_step_state: beta powers 1, step 0, loss scale
 * `loss_scale` (> 0), flags and norm 0. */
int zero_state_init(zero_step_state* state, float loss_scale, void* stream);

/* Average this rank's segment over its N_d gradient copies [reading notes,
 * second part §4: avg = (1/N_d) * sum_r g_r]: for each j < n,
 *   acc = 0 (fp32); acc += float(replicas[r][j]) for r = 0 .. n_d-1 in order;
 *   avg_out[j] = acc / n_d.
 * avg_out keeps the loss scale (it is not unscaled). The same pass writes the
 * overflow flag and sum-of-squares partials of the unscaled gradient
 * avg_out[j] * (1 / state->loss_scale) into workspace slot `group`, for
 * zero_grad_norm_overflow(). replicas: host array of n_d device pointers.
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE, UNSUPPORTED (n_d too large). */
int zero_reduce_grad_segment(const void* const* replicas, int32_t n_d, int32_t grad_dt,
                             int64_t n, float* avg_out, void* workspace, size_t workspace_bytes,
                             int32_t group, const zero_step_state* state, void* stream);

/* Overflow check and gradient norm of one step [DeepSpeed walkthrough §6
 * steps 1-2]. If `grads` is not NULL, first scan grads[g] (device pointer to
 * counts[g] elements of grad_dt, a single gradient copy, N_d = 1) into
 * workspace slot g for each g < n_groups with grads[g] != NULL. Then combine
 * the partials of slots 0 .. n_groups-1 in a fixed order into
 * state->grad_norm_sq / grad_norm (the norm of the unscaled gradient over all
 * groups) and state->overflow, set state->skipped = overflow &&
 * policy->skip_on_overflow and state->clip_coef from policy->max_grad_norm
 * (policy may be NULL: no skip, no clip). When overflow is set the norm is
 * reported as NaN. Does not advance the step. `grads` and `counts` are host
 * arrays.
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE. */
int zero_grad_norm_overflow(const void* const* grads, const int64_t* counts, int32_t grad_dt,
                            int32_t n_groups, void* workspace, size_t workspace_bytes,
                            const zero_policy* policy, zero_step_state* state, void* stream);

/* One Adam/AdamW step over n_groups groups of this rank's shard [reading
 * notes, second part §3; DeepSpeed walkthrough §6 steps 3-5]. With applied
 * step t = state->step + 1, per group b1 = fp32(1 - beta1^t),
 * b2 = fp32(1 - beta2^t), and per element, every operation in fp32
 * round-to-nearest-even, no fused multiply-add:
 *   g = avg * fp32(1 / S);  theta = master;  if wd: theta *= fp32(1 - lr*wd)
 *   m = beta1*m + fp32(1-beta1)*g;   v = beta2*v + fp32(1-beta2)*(g*g)
 *   theta -= lr * ((m / b1) / (sqrt(v / b2) + eps))
 *   master = theta;  flat_param[param_offset + j] = RNE16(theta)
 * Pipelines, chosen by the policy:
 *   - "fused" (policy NULL, or no skip and no clipping): one pass per group
 *     reads the gradient source, averages, unscales, updates and writes back,
 *     and emits norm/overflow partials; a fold and a one-block kernel form the
 *     norm and the flag and advance the step. No zero_grad_norm_overflow()
 *     call is needed.
 *   - "checked" (skip_on_overflow 1 or max_grad_norm > 0, not optimistic):
 *     the caller has already run zero_grad_norm_overflow() on this step's
 *     gradients with the same policy; if it set state->skipped, nothing but
 *     the loss scale changes; otherwise the update is applied with g
 *     multiplied by state->clip_coef, and the step advances. Scale
 *     backoff/growth happen here.
 *   - "optimistic" (skip_on_overflow 1, optimistic 1): one pass per group
 *     reads the current set (state->cur), writes the updated values into the
 *     other set and into flat_param, and emits norm partials; then without
 *     overflow the other set becomes current (cur flips) and the step
 *     advances; with overflow the current set stays, the scale backs off, and
 *     flat_param's slice is rewritten from the current master. That restores
 *     it exactly when the slice held RNE16(current master) before the step,
 *     as it does after zero_cast_writeback() or any applied step. With
 *     max_grad_norm > 0, a step whose norm asks for clipping (multiplier < 1)
 *     is recomputed by a second pass from the current set with the
 *     multiplier, then committed: the result is the checked pipeline's, and
 *     steps that need no clipping stay one pass. Costs a second state set
 *     (12 B/param) instead of the checked pipeline's extra pass over an fp32
 *     average.
 * `groups` is a host array; group g uses workspace slot g and the beta powers
 * state->beta*_pow[g].
 * Errors: INVALID_ARG, ALIGNMENT, WORKSPACE, UNSUPPORTED. */
int zero_adam_step(const zero_group* groups, int32_t n_groups, const zero_policy* policy,
                   void* workspace, size_t workspace_bytes, zero_step_state* state, void* stream);

/* zero_adam_step without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels and results, with the norm
 * partials in a static device array of the library (16 MiB + 16 KiB,
 * ZERO_MAX_GROUPS groups, any shard size) instead of a caller's workspace.
 * Each GPU the library runs on holds one copy of that array until the process
 * ends; its address is looked up on the first call on a device (code that
 * captures the call into a graph makes one call on the device first). The call
 * allocates and frees nothing. Every call on a GPU shares that GPU's array,
 * so calls that overlap on one GPU (concurrent streams, threads) race; order
 * them. The contents need no initialisation (each call writes the partials it
 * reads). Works for every pipeline; in the checked one the preceding
 * zero_reduce_grad_segment / zero_grad_norm_overflow calls still take a
 * workspace, since zero_adam_step reads only the state in that pipeline.
 * Errors: as zero_adam_step; INVALID_ARG for n_groups beyond ZERO_MAX_GROUPS;
 * HIP if the array's address cannot be found. */
int zero_adam_step_static(const zero_group* groups, int32_t n_groups, const zero_policy* policy,
                          zero_step_state* state, void* stream);

/* Copy an fp32 master shard into the 16-bit flat vector [DeepSpeed
 * walkthrough §6 step 5]: flat_param[offset + j] = RNE16(master[j]) for j < n
 * (NaN becomes the canonical quiet NaN). Used at initialisation and to restore
 * parameters from the master. Errors: INVALID_ARG, ALIGNMENT. */
int zero_cast_writeback(const float* master, int64_t n, void* flat_param, int64_t offset,
                        int32_t param_dt, void* stream);

/* ---- testing --------------------------------------------------------------
 * Not an operation of the pages. Caps the blocks of every streaming launch
 * (update, second pass, averaging, scan, restore, cast) at max_blocks > 0, on
 * top of each launch's own cap (2^21 tiles per launch; 65,536 blocks for the
 * second pass and the scan; 1,024 for the restore). Every streaming kernel
 * loops over the tiles its grid does not cover, so a small shard under a low
 * cap runs the same grid-stride loops that otherwise only shards of billions
 * of elements reach; tests use it to check those loops element by element.
 * 0 removes the cap (the default). Elementwise results do not depend on it;
 * the norm is the same sum of squares grouped into other partials (equal to
 * within fp64 reassociation). Process-wide, for every device and thread; a
 * launch on another thread while it changes sees either value.
 * Errors: INVALID_ARG for max_blocks < 0. */
int zero_set_grid_limit(int32_t max_blocks);

/* ---- measurement ----------------------------------------------------------
 * Not an operation of the pages. Copies n_bytes from src0 to dst0 and from
 * src1 to dst1 (device buffers, 16-byte aligned, n_bytes a multiple of 16;
 * the ranges must not overlap) with the update kernel's access shape: one
 * block per 16 KiB tile of each stream, 16-byte non-temporal loads and
 * stores, each wavefront access one contiguous 1 KiB run. A step of half
 * reads, half writes over buffers in two HBM regions (N_d = 1) moves its bytes
 * the way this copy does with src0/dst1 in one region and src1/dst0 in the
 * other, so its bandwidth is the ceiling such a step meets on that placement;
 * bench.py reports it beside the step. Stream-ordered, allocates nothing.
 * Errors: INVALID_ARG (negative or unaligned size, NULL buffer), ALIGNMENT,
 * UNSUPPORTED (not gfx950), HIP. */
int zero_copy_probe(const void* src0, const void* src1, void* dst0, void* dst1, int64_t n_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_DP_H */
