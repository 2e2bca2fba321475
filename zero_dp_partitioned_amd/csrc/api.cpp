// Host side of the C ABI (include/zero_dp.h): argument checks, the partition
// index map, workspace layout, and the order in which kernels are enqueued.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>
#include <unordered_map>

#include "zero_dp_internal.h"

using namespace zdp;

namespace zdp {
std::atomic<int32_t> g_grid_limit{0};
// Two-stream copy of `words` 16-byte words, src0 -> dst0 and src1 -> dst1 (copy_probe.hip).
hipError_t launch_copy_probe(const void* src0, const void* src1, void* dst0, void* dst1, int64_t words,
                             hipStream_t s);
}  // namespace zdp

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ZERO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_dt(int32_t dt) { return dt == ZERO_DT_F16 || dt == ZERO_DT_BF16; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Largest of 8/4/2 dividing the address (the widest 16-bit store is 8 bytes).
int32_t align_class(const void* p) {
  const uintptr_t u = reinterpret_cast<uintptr_t>(p);
  if ((u & 7) == 0) return 8;
  if ((u & 3) == 0) return 4;
  return 2;
}

// The quad path loads fp32 arrays 16 bytes and 16-bit arrays 8 bytes at a
// time, 4 elements either way. Arrays that all sit at the same offset modulo
// 4 elements (views into flat buffers at one segment offset, say) reach that
// alignment after the same number h < 4 of leading elements: the kernels
// update those h elements one by one and the rest on the quad path. HeadCheck
// collects the arrays of one launch; head() is that h, or -1 if they disagree
// (then every element takes the element path).
class HeadCheck {
 public:
  void add(const void* p, int64_t elem_bytes) {
    const uintptr_t u = reinterpret_cast<uintptr_t>(p);
    const int64_t h = (4 - static_cast<int64_t>((u / elem_bytes) % 4)) % 4;
    if (h_ == kUnset) h_ = h;
    else if (h_ != h) h_ = kMixed;
  }
  int64_t head() const { return h_ == kUnset ? 0 : h_; }

 private:
  static constexpr int64_t kUnset = -2, kMixed = -1;
  int64_t h_ = kUnset;
};

// What the launches need to know of a device, found once per device.
struct DeviceInfo {
  bool gfx950;
  size_t batch_lds;  // dynamic LDS per block of the batched update schedule
};

// The current device must be gfx950. *info (optional) receives its DeviceInfo.
int check_device(DeviceInfo* info = nullptr) {
  static std::mutex mu;
  static std::unordered_map<int, DeviceInfo> known;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  auto it = known.find(dev);
  if (it == known.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    int lds = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(LDS per CU)");
    DeviceInfo d;
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.batch_lds = batch_lds_bytes(static_cast<size_t>(lds));
    it = known.emplace(dev, d).first;
  }
  if (!it->second.gfx950)
    return fail(ZERO_ERR_UNSUPPORTED, "device %d is not gfx950, the target this library is built for", dev);
  if (info) *info = it->second;
  return ZERO_OK;
}

// Workspace: per-group level-2 partials, then the block partials of the latest launch.
double* level2_of(void* ws, int32_t g) { return static_cast<double*>(ws) + static_cast<int64_t>(g) * kFoldBlocks; }
double* scratch_of(void* ws) { return reinterpret_cast<double*>(static_cast<char*>(ws) + kHeaderBytes); }

// Reduce the `blocks` partials a launch just wrote into the level-2 partials
// of group g (the launchers report their grid size, or 0 when a small launch
// wrote the level-2 partials itself: then there is nothing to fold).
hipError_t fold_into(void* ws, int32_t g, int64_t blocks, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  FoldArgs F;
  F.partials = scratch_of(ws);
  F.count = blocks;
  F.level2 = level2_of(ws, g);
  return launch_fold(F, s);
}

int check_workspace(const void* ws, size_t have) {
  if (!ws) return fail(ZERO_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(ZERO_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (have < kWorkspaceBytes)
    return fail(ZERO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", have, kWorkspaceBytes);
  return ZERO_OK;
}

int check_policy(const zero_policy* p) {
  if (!p) return ZERO_OK;
  if (!(p->max_grad_norm >= 0.0) || p->max_grad_norm == __builtin_inf())
    return fail(ZERO_ERR_INVALID_ARG, "max_grad_norm must be finite and >= 0");
  if (p->skip_on_overflow && (!(p->backoff > 0.0) || !(p->growth >= 1.0) || !(p->min_scale > 0.0) ||
                              p->growth_interval < 0))
    return fail(ZERO_ERR_INVALID_ARG, "bad loss-scale policy");
  return ZERO_OK;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Fill a GradSource from a host array of replica pointers (which path the
// kernels take is HeadCheck's business). An empty shard (n == 0) reads
// nothing, so its pointers may be NULL.
int make_source(const void* const* replicas, int32_t n_d, int32_t dt, int64_t n, GradSource* S) {
  memset(S, 0, sizeof *S);
  if (!replicas) return fail(ZERO_ERR_INVALID_ARG, "replica pointer array is NULL");
  if (n_d < 1) return fail(ZERO_ERR_INVALID_ARG, "n_d = %d < 1", n_d);
  if (n_d > ZERO_MAX_REPLICAS) return fail(ZERO_ERR_UNSUPPORTED, "n_d = %d > %d", n_d, ZERO_MAX_REPLICAS);
  if (!valid_dt(dt)) return fail(ZERO_ERR_INVALID_ARG, "gradient dtype %d is not f16/bf16", dt);
  if (n == 0) {
    S->n_d = n_d;
    S->nd = static_cast<float>(n_d);
    return ZERO_OK;
  }
  for (int32_t r = 0; r < n_d; ++r) {
    if (!replicas[r]) return fail(ZERO_ERR_INVALID_ARG, "replica %d is NULL", r);
    if (!aligned(replicas[r], 2)) return fail(ZERO_ERR_ALIGNMENT, "replica %d is not 2-byte aligned", r);
  }
  if (n_d <= kInlineReplicas) {
    for (int32_t r = 0; r < n_d; ++r) S->rep[r] = replicas[r];
    S->strided = 0;
  } else {
    // Beyond the inline table the copies must be equally spaced in one buffer.
    const char* base = static_cast<const char*>(replicas[0]);
    const ptrdiff_t d = static_cast<const char*>(replicas[1]) - base;
    if (d <= 0 || d % 2 != 0)
      return fail(ZERO_ERR_UNSUPPORTED, "n_d > %d needs equally spaced replicas in one buffer",
                  kInlineReplicas);
    for (int32_t r = 2; r < n_d; ++r)
      if (static_cast<const char*>(replicas[r]) - base != static_cast<ptrdiff_t>(r) * d)
        return fail(ZERO_ERR_UNSUPPORTED, "n_d > %d needs equally spaced replicas in one buffer",
                    kInlineReplicas);
    S->rep[0] = replicas[0];
    S->stride = d / 2;
    S->strided = 1;
  }
  S->n_d = n_d;
  S->nd = static_cast<float>(n_d);
  S->inv_nd = is_pow2(n_d) ? 1.0f / static_cast<float>(n_d) : 0.0f;
  return ZERO_OK;
}

}  // namespace

extern "C" {

const char* zero_last_error(void) { return g_err; }

int zero_partition(int64_t numel, int32_t n_d, int64_t align_elems, zero_segment* segs,
                   int64_t* padded_numel) {
  if (numel < 0) return fail(ZERO_ERR_INVALID_ARG, "numel = %lld < 0", (long long)numel);
  if (n_d < 1) return fail(ZERO_ERR_INVALID_ARG, "n_d = %d < 1", n_d);
  if (align_elems < 1) return fail(ZERO_ERR_INVALID_ARG, "align_elems < 1");
  if (!segs) return fail(ZERO_ERR_INVALID_ARG, "segs is NULL");
  int64_t padded = numel;
  const int64_t r = numel % align_elems;
  if (r) {
    if (numel > INT64_MAX - (align_elems - r)) return fail(ZERO_ERR_INVALID_ARG, "padded numel overflows int64");
    padded = numel + (align_elems - r);
  }
  const int64_t base = padded / n_d, rem = padded % n_d;
  for (int32_t k = 0; k < n_d; ++k) {
    segs[k].offset = k * base + (k < rem ? k : rem);
    segs[k].size = base + (k < rem ? 1 : 0);
  }
  if (padded_numel) *padded_numel = padded;
  return ZERO_OK;
}

int zero_partition_tensors(const int64_t* numels, int32_t n_tensors, int32_t n_d, int32_t rank,
                           int64_t align_elems, zero_tensor_slice* out, int32_t cap, int32_t* n_out) {
  if (!numels && n_tensors > 0) return fail(ZERO_ERR_INVALID_ARG, "numels is NULL");
  if (n_tensors < 0) return fail(ZERO_ERR_INVALID_ARG, "n_tensors < 0");
  if (n_d < 1 || rank < 0 || rank >= n_d) return fail(ZERO_ERR_INVALID_ARG, "rank %d out of [0, %d)", rank, n_d);
  if (!n_out) return fail(ZERO_ERR_INVALID_ARG, "n_out is NULL");
  int64_t total = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    if (numels[t] < 0) return fail(ZERO_ERR_INVALID_ARG, "numels[%d] < 0", t);
    if (total > INT64_MAX - numels[t]) return fail(ZERO_ERR_INVALID_ARG, "total numel overflows int64");
    total += numels[t];
  }
  // the rank's segment, by the same rule as zero_partition
  int64_t padded = total;
  if (align_elems < 1) return fail(ZERO_ERR_INVALID_ARG, "align_elems < 1");
  const int64_t r = total % align_elems;
  if (r) {
    if (total > INT64_MAX - (align_elems - r)) return fail(ZERO_ERR_INVALID_ARG, "padded numel overflows int64");
    padded = total + (align_elems - r);
  }
  const int64_t base = padded / n_d, rem = padded % n_d;
  const int64_t lo = rank * base + (rank < rem ? rank : rem);
  const int64_t hi = lo + base + (rank < rem ? 1 : 0);
  int32_t count = 0;
  int64_t start = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    const int64_t b = start, e = start + numels[t];
    start = e;
    const int64_t ob = b > lo ? b : lo, oe = e < hi ? e : hi;
    if (ob >= oe) continue;
    if (count >= cap || !out) return fail(ZERO_ERR_INVALID_ARG, "output capacity %d too small", cap);
    out[count].tensor = t;
    out[count].reserved = 0;
    out[count].shard_begin = ob - lo;
    out[count].tensor_begin = ob - b;
    out[count].length = oe - ob;
    ++count;
  }
  *n_out = count;
  return ZERO_OK;
}

int zero_plan_arena(zero_arena_buffer* buffers, int32_t n_buffers, int64_t region_bytes,
                    int32_t n_regions, int64_t max_bytes, int64_t* arena_bytes) {
  constexpr int32_t kMaxRegions = 16;
  const int64_t A = ZERO_ARENA_ALIGN;
  if (!buffers || n_buffers < 1) return fail(ZERO_ERR_INVALID_ARG, "no buffers");
  if (!arena_bytes) return fail(ZERO_ERR_INVALID_ARG, "arena_bytes is NULL");
  if (region_bytes == 0) region_bytes = ZERO_HBM_REGION_BYTES;
  if (region_bytes < A || region_bytes % A)
    return fail(ZERO_ERR_INVALID_ARG, "region_bytes must be a positive multiple of %lld", (long long)A);
  if (n_regions < 0 || n_regions > kMaxRegions)
    return fail(ZERO_ERR_INVALID_ARG, "n_regions = %d outside [0, %d]", n_regions, kMaxRegions);
  if (max_bytes < A) return fail(ZERO_ERR_INVALID_ARG, "max_bytes below one alignment unit");
  std::vector<int64_t> size(n_buffers);
  for (int32_t i = 0; i < n_buffers; ++i) {
    if (buffers[i].bytes < 1) return fail(ZERO_ERR_INVALID_ARG, "buffers[%d].bytes < 1", i);
    if (buffers[i].traffic < 0) return fail(ZERO_ERR_INVALID_ARG, "buffers[%d].traffic < 0", i);
    if (buffers[i].bytes > INT64_MAX - A) return fail(ZERO_ERR_INVALID_ARG, "buffers[%d].bytes too large", i);
    size[i] = (buffers[i].bytes + A - 1) / A * A;
  }
  // heaviest traffic first; ties: larger first, then lower index
  std::vector<int32_t> order(n_buffers);
  for (int32_t i = 0; i < n_buffers; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (buffers[a].traffic != buffers[b].traffic) return buffers[a].traffic > buffers[b].traffic;
    return size[a] > size[b];
  });
  std::vector<int64_t> off(n_buffers);
  std::vector<int32_t> reg(n_buffers);
  auto place = [&](int32_t regions) -> bool {
    std::vector<int64_t> cap(regions), used(regions, 0), load(regions, 0);
    for (int32_t r = 0; r < regions; ++r) {
      const int64_t start = static_cast<int64_t>(r) * region_bytes;
      const int64_t room = start < max_bytes ? (max_bytes - start) / A * A : 0;
      cap[r] = room < region_bytes ? room : region_bytes;
    }
    for (int32_t i : order) {
      int32_t best = -1;
      for (int32_t r = 0; r < regions; ++r)
        if (size[i] <= cap[r] - used[r] && (best < 0 || load[r] < load[best])) best = r;
      if (best < 0) return false;
      reg[i] = best;
      off[i] = static_cast<int64_t>(best) * region_bytes + used[best];
      used[best] += size[i];
      load[best] += buffers[i].traffic;
    }
    return true;
  };
  bool ok = false;
  if (n_regions > 0) {
    if (static_cast<int64_t>(n_regions - 1) > (max_bytes - 1) / region_bytes)
      return fail(ZERO_ERR_UNSUPPORTED, "%d regions of %lld bytes do not start below max_bytes = %lld",
                  n_regions, (long long)region_bytes, (long long)max_bytes);
    ok = place(n_regions);
  } else {
    // the fewest regions, at least two where max_bytes allows, that hold every buffer
    const int64_t avail = (max_bytes - 1) / region_bytes + 1;
    const int32_t most = static_cast<int32_t>(avail < kMaxRegions ? avail : kMaxRegions);
    for (int32_t r = most >= 2 ? 2 : 1; r <= most && !ok; ++r) ok = place(r);
  }
  if (!ok) return fail(ZERO_ERR_UNSUPPORTED, "the buffers do not fit in the regions below max_bytes");
  int64_t end = 0;
  for (int32_t i = 0; i < n_buffers; ++i) {
    buffers[i].offset = off[i];
    buffers[i].region = reg[i];
    buffers[i].reserved = 0;
    end = std::max(end, off[i] + size[i]);
  }
  *arena_bytes = end;
  return ZERO_OK;
}

size_t zero_workspace_bytes(int32_t n_groups) {
  if (n_groups < 1 || n_groups > ZERO_MAX_GROUPS) return 0;
  return kWorkspaceBytes;
}

int zero_state_init(zero_step_state* state, float loss_scale, void* stream) {
  if (!state) return fail(ZERO_ERR_INVALID_ARG, "state is NULL");
  if (!aligned(state, 8)) return fail(ZERO_ERR_ALIGNMENT, "state is not 8-byte aligned");
  if (!(loss_scale > 0.0f) || loss_scale == __builtin_inff())
    return fail(ZERO_ERR_INVALID_ARG, "loss_scale must be finite and > 0");
  if (int rc = check_device()) return rc;
  hipError_t e = launch_state_init(state, loss_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZERO_OK : hip_fail(e, "state init launch");
}

int zero_reduce_grad_segment(const void* const* replicas, int32_t n_d, int32_t grad_dt, int64_t n,
                             float* avg_out, void* workspace, size_t workspace_bytes, int32_t group,
                             const zero_step_state* state, void* stream) {
  if (n < 0) return fail(ZERO_ERR_INVALID_ARG, "n < 0");
  if (!avg_out && n > 0) return fail(ZERO_ERR_INVALID_ARG, "avg_out is NULL");
  if (!aligned(avg_out, 4)) return fail(ZERO_ERR_ALIGNMENT, "avg_out is not 4-byte aligned");
  if (!state) return fail(ZERO_ERR_INVALID_ARG, "state is NULL");
  if (int rc = check_workspace(workspace, workspace_bytes)) return rc;
  if (group < 0 || group >= ZERO_MAX_GROUPS) return fail(ZERO_ERR_WORKSPACE, "group %d out of range", group);
  ReduceArgs R;
  if (int rc = make_source(replicas, n_d, grad_dt, n, &R.src)) return rc;
  DeviceInfo dev;
  if (int rc = check_device(&dev)) return rc;
  HeadCheck hc;
  hc.add(avg_out, 4);
  for (int32_t r = 0; r < n_d && n > 0; ++r) hc.add(replicas[r], 2);
  const bool vec = hc.head() >= 0;
  R.head = vec ? std::min<int64_t>(hc.head(), n) : 0;
  R.n = n;
  R.avg_out = avg_out;
  R.state = state;
  R.partials = scratch_of(workspace);
  R.level2 = level2_of(workspace, group);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int blocks = 0;
  hipError_t e = launch_reduce(R, grad_dt == ZERO_DT_BF16 ? kSrcBF16 : kSrcF16, vec, dev.batch_lds, s, &blocks);
  if (e != hipSuccess) return hip_fail(e, "reduce launch");
  e = fold_into(workspace, group, blocks, s);
  return e == hipSuccess ? ZERO_OK : hip_fail(e, "fold launch");
}

int zero_grad_norm_overflow(const void* const* grads, const int64_t* counts, int32_t grad_dt,
                            int32_t n_groups, void* workspace, size_t workspace_bytes,
                            const zero_policy* policy, zero_step_state* state, void* stream) {
  if (n_groups < 1 || n_groups > ZERO_MAX_GROUPS)
    return fail(ZERO_ERR_INVALID_ARG, "n_groups = %d out of [1, %d]", n_groups, ZERO_MAX_GROUPS);
  if (!state) return fail(ZERO_ERR_INVALID_ARG, "state is NULL");
  if (int rc = check_workspace(workspace, workspace_bytes)) return rc;
  if (int rc = check_policy(policy)) return rc;
  ReduceArgs R[ZERO_MAX_GROUPS];
  bool vec[ZERO_MAX_GROUPS] = {};
  bool scan[ZERO_MAX_GROUPS] = {};
  if (grads) {
    if (!counts) return fail(ZERO_ERR_INVALID_ARG, "counts is NULL");
    if (!valid_dt(grad_dt)) return fail(ZERO_ERR_INVALID_ARG, "gradient dtype %d is not f16/bf16", grad_dt);
    for (int32_t g = 0; g < n_groups; ++g) {
      if (!grads[g]) continue;
      if (counts[g] < 0) return fail(ZERO_ERR_INVALID_ARG, "counts[%d] < 0", g);
      const void* one[1] = {grads[g]};
      if (int rc = make_source(one, 1, grad_dt, counts[g], &R[g].src)) return rc;
      R[g].n = counts[g];
      R[g].avg_out = nullptr;
      R[g].state = state;
      R[g].partials = scratch_of(workspace);
      R[g].level2 = level2_of(workspace, g);
      HeadCheck hc;
      hc.add(grads[g], 2);
      vec[g] = true;  // one array: a head of h < 4 elements always aligns it
      R[g].head = std::min<int64_t>(hc.head(), counts[g]);
      scan[g] = true;
    }
  }
  if (int rc = check_device()) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int src = grad_dt == ZERO_DT_BF16 ? kSrcBF16 : kSrcF16;
  for (int32_t g = 0; g < n_groups; ++g) {
    if (!scan[g]) continue;
    // 16-byte-aligned copies take the wide-load scan; others the streaming pass
    const bool wide = aligned(grads[g], 16);
    if (wide) R[g].head = 0;
    int blocks = 0;
    // (one copy: the averaging launch never takes the batched read, so it needs no LDS share)
    hipError_t e = wide ? launch_scan(R[g], src, s, &blocks) : launch_reduce(R[g], src, vec[g], 0, s, &blocks);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
    e = fold_into(workspace, g, blocks, s);
    if (e != hipSuccess) return hip_fail(e, "fold launch");
  }
  FinalizeArgs F;
  memset(&F, 0, sizeof F);
  F.level2 = level2_of(workspace, 0);
  F.state = state;
  F.n_groups = n_groups;
  F.mode = 0;
  F.skip_on_overflow = policy ? (policy->skip_on_overflow != 0) : 0;
  F.max_grad_norm = policy ? policy->max_grad_norm : 0.0;
  hipError_t e = launch_finalize(F, s);
  return e == hipSuccess ? ZERO_OK : hip_fail(e, "finalize launch");
}

int zero_adam_step(const zero_group* groups, int32_t n_groups, const zero_policy* policy,
                   void* workspace, size_t workspace_bytes, zero_step_state* state, void* stream) {
  if (!groups) return fail(ZERO_ERR_INVALID_ARG, "groups is NULL");
  if (n_groups < 1 || n_groups > ZERO_MAX_GROUPS)
    return fail(ZERO_ERR_INVALID_ARG, "n_groups = %d out of [1, %d]", n_groups, ZERO_MAX_GROUPS);
  if (!state) return fail(ZERO_ERR_INVALID_ARG, "state is NULL");
  if (!aligned(state, 8)) return fail(ZERO_ERR_ALIGNMENT, "state is not 8-byte aligned");
  if (int rc = check_workspace(workspace, workspace_bytes)) return rc;
  if (int rc = check_policy(policy)) return rc;
  const bool dynamic = policy && policy->skip_on_overflow;
  const bool optimistic = policy && policy->optimistic;
  if (optimistic && !dynamic) return fail(ZERO_ERR_INVALID_ARG, "the optimistic pipeline needs skip_on_overflow");
  const bool clip_redo = optimistic && policy->max_grad_norm > 0.0;
  const bool checked = !optimistic && policy && (policy->skip_on_overflow || policy->max_grad_norm > 0.0);
  const int mode = optimistic ? kOptimistic : (checked ? kChecked : kFused);
  AdamArgs A[ZERO_MAX_GROUPS];
  int src[ZERO_MAX_GROUPS];
  bool vec[ZERO_MAX_GROUPS];
  for (int32_t g = 0; g < n_groups; ++g) {
    const zero_group& G = groups[g];
    AdamArgs& a = A[g];
    memset(&a, 0, sizeof a);
    if (G.n < 0) return fail(ZERO_ERR_INVALID_ARG, "group %d: n < 0", g);
    if ((!G.master || !G.exp_avg || !G.exp_avg_sq) && G.n > 0)
      return fail(ZERO_ERR_INVALID_ARG, "group %d: master/exp_avg/exp_avg_sq is NULL", g);
    if (!aligned(G.master, 4) || !aligned(G.exp_avg, 4) || !aligned(G.exp_avg_sq, 4))
      return fail(ZERO_ERR_ALIGNMENT, "group %d: fp32 state not 4-byte aligned", g);
    HeadCheck hc;
    hc.add(G.master, 4);
    hc.add(G.exp_avg, 4);
    hc.add(G.exp_avg_sq, 4);
    if (optimistic) {
      if ((!G.master_alt || !G.exp_avg_alt || !G.exp_avg_sq_alt) && G.n > 0)
        return fail(ZERO_ERR_INVALID_ARG, "group %d: the optimistic pipeline needs the *_alt state set", g);
      if (!aligned(G.master_alt, 4) || !aligned(G.exp_avg_alt, 4) || !aligned(G.exp_avg_sq_alt, 4))
        return fail(ZERO_ERR_ALIGNMENT, "group %d: fp32 *_alt state not 4-byte aligned", g);
      hc.add(G.master_alt, 4);
      hc.add(G.exp_avg_alt, 4);
      hc.add(G.exp_avg_sq_alt, 4);
      a.master_alt = G.master_alt;
      a.m_alt = G.exp_avg_alt;
      a.v_alt = G.exp_avg_sq_alt;
    }
    if ((G.replicas != nullptr) == (G.avg != nullptr) && !(G.n == 0 && !G.replicas))
      return fail(ZERO_ERR_INVALID_ARG, "group %d: give exactly one of replicas and avg", g);
    if (G.avg || !G.replicas) {
      if (!aligned(G.avg, 4)) return fail(ZERO_ERR_ALIGNMENT, "group %d: avg not 4-byte aligned", g);
      a.src.avg = G.avg;
      a.src.n_d = 1;
      src[g] = kSrcAvg;
      hc.add(G.avg, 4);
    } else {
      if (int rc = make_source(G.replicas, G.n_d, G.grad_dt, G.n, &a.src)) return rc;
      src[g] = G.grad_dt == ZERO_DT_BF16 ? kSrcBF16 : kSrcF16;
      for (int32_t r = 0; r < G.n_d && G.n > 0; ++r) hc.add(G.replicas[r], 2);
    }
    const bool v = hc.head() >= 0;
    a.head = v ? std::min<int64_t>(hc.head(), G.n) : 0;
    if (G.flat_param && G.n > 0) {
      if (!valid_dt(G.param_dt)) return fail(ZERO_ERR_INVALID_ARG, "group %d: param dtype %d", g, G.param_dt);
      if (G.param_offset < 0) return fail(ZERO_ERR_INVALID_ARG, "group %d: param_offset < 0", g);
      if (!aligned(G.flat_param, 2)) return fail(ZERO_ERR_ALIGNMENT, "group %d: flat_param not 2-byte aligned", g);
      a.param = static_cast<uint16_t*>(G.flat_param) + G.param_offset;
      a.param_dt = G.param_dt;
      a.param_align = align_class(static_cast<uint16_t*>(a.param) + a.head);  // quads start at the head
    }
    if (!(G.lr >= 0.0) || !(G.beta1 >= 0.0 && G.beta1 < 1.0) || !(G.beta2 >= 0.0 && G.beta2 < 1.0) ||
        !(G.eps > 0.0) || !(G.weight_decay >= 0.0))
      return fail(ZERO_ERR_INVALID_ARG, "group %d: hyperparameters out of range", g);
    a.n = G.n;
    a.master = G.master;
    a.m = G.exp_avg;
    a.v = G.exp_avg_sq;
    a.beta1_d = G.beta1;
    a.beta2_d = G.beta2;
    a.lr = static_cast<float>(G.lr);
    a.beta1 = static_cast<float>(G.beta1);
    a.beta2 = static_cast<float>(G.beta2);
    a.eps = static_cast<float>(G.eps);
    a.c1 = static_cast<float>(1.0 - G.beta1);
    a.c2 = static_cast<float>(1.0 - G.beta2);
    a.decay = static_cast<float>(1.0 - G.lr * G.weight_decay);
    a.has_decay = G.weight_decay != 0.0;
    a.group = g;
    a.state = state;
    a.partials = checked ? nullptr : scratch_of(workspace);
    a.level2 = checked ? nullptr : level2_of(workspace, g);
    vec[g] = v;
  }
  DeviceInfo dev;
  if (int rc = check_device(&dev)) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t g = 0; g < n_groups; ++g) {
    int blocks = 0;
    hipError_t e = launch_adam(A[g], src[g], vec[g], mode, dev.batch_lds, s, &blocks);
    if (e != hipSuccess) return hip_fail(e, "update launch");
    if (!checked) {
      e = fold_into(workspace, g, blocks, s);
      if (e != hipSuccess) return hip_fail(e, "fold launch");
    }
  }
  if (!checked) {
    FinalizeArgs F;
    memset(&F, 0, sizeof F);
    F.level2 = level2_of(workspace, 0);
    F.state = state;
    F.n_groups = n_groups;
    F.mode = optimistic ? 2 : 1;
    if (optimistic) {
      F.skip_on_overflow = 1;
      F.growth_interval = policy->growth_interval;
      F.backoff = policy->backoff;
      F.growth = policy->growth;
      F.min_scale = policy->min_scale;
      F.max_grad_norm = policy->max_grad_norm;
    }
    for (int32_t g = 0; g < n_groups; ++g) {
      F.beta1[g] = groups[g].beta1;
      F.beta2[g] = groups[g].beta2;
    }
    hipError_t e = launch_finalize(F, s);
    if (e != hipSuccess) return hip_fail(e, "finalize launch");
    if (optimistic) {
      // a voided step already wrote its values into the parameter slices:
      // rewrite them from the current master (the launch exits at once otherwise)
      for (int32_t g = 0; g < n_groups; ++g) {
        if (!A[g].param || A[g].n == 0) continue;
        RestoreArgs R;
        R.master = A[g].master;
        R.master_alt = A[g].master_alt;
        R.n = A[g].n;
        R.param = A[g].param;
        R.param_dt = A[g].param_dt;
        R.param_align = align_class(A[g].param);  // the restore kernel starts its quads at element 0
        R.state = state;
        const bool rv = aligned(R.master, 16) && aligned(R.master_alt, 16);
        e = launch_restore(R, rv, s);
        if (e != hipSuccess) return hip_fail(e, "restore launch");
      }
    }
    if (clip_redo) {
      // a step the norm says to clip: recompute it from the current set with
      // the multiplier (the launches exit at once otherwise), then commit it
      for (int32_t g = 0; g < n_groups; ++g) {
        AdamArgs a = A[g];
        a.partials = nullptr;
        a.level2 = nullptr;
        int blocks = 0;
        e = launch_adam(a, src[g], vec[g], kRedo, dev.batch_lds, s, &blocks);
        if (e != hipSuccess) return hip_fail(e, "second-pass launch");
      }
      CommitArgs C;
      memset(&C, 0, sizeof C);
      C.state = state;
      C.n_groups = n_groups;
      C.dynamic = 1;
      C.growth_interval = policy->growth_interval;
      C.backoff = policy->backoff;
      C.growth = policy->growth;
      C.min_scale = policy->min_scale;
      for (int32_t g = 0; g < n_groups; ++g) {
        C.beta1[g] = groups[g].beta1;
        C.beta2[g] = groups[g].beta2;
      }
      e = launch_redo_commit(C, s);
      if (e != hipSuccess) return hip_fail(e, "second-pass commit launch");
    }
    return ZERO_OK;
  }
  CommitArgs C;
  memset(&C, 0, sizeof C);
  C.state = state;
  C.n_groups = n_groups;
  C.dynamic = dynamic ? 1 : 0;
  C.growth_interval = policy->growth_interval;
  C.backoff = policy->backoff;
  C.growth = policy->growth;
  C.min_scale = policy->min_scale;
  for (int32_t g = 0; g < n_groups; ++g) {
    C.beta1[g] = groups[g].beta1;
    C.beta2[g] = groups[g].beta2;
  }
  hipError_t e = launch_commit(C, s);
  return e == hipSuccess ? ZERO_OK : hip_fail(e, "commit launch");
}

int zero_adam_step_static(const zero_group* groups, int32_t n_groups, const zero_policy* policy,
                          zero_step_state* state, void* stream) {
  if (n_groups < 1 || n_groups > ZERO_MAX_GROUPS)
    return fail(ZERO_ERR_INVALID_ARG, "n_groups = %d out of [1, %d]: the static scratch holds the partials of at most %d "
                "groups", n_groups, ZERO_MAX_GROUPS, ZERO_MAX_GROUPS);
  if (int rc = check_device()) return rc;
  void* ws = nullptr;
  hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "address of the static scratch (hipGetSymbolAddress)");
  return zero_adam_step(groups, n_groups, policy, ws, kWorkspaceBytes, state, stream);
}

int zero_set_grid_limit(int32_t max_blocks) {
  if (max_blocks < 0) return fail(ZERO_ERR_INVALID_ARG, "max_blocks = %d < 0", max_blocks);
  g_grid_limit.store(max_blocks, std::memory_order_relaxed);
  return ZERO_OK;
}

int zero_copy_probe(const void* src0, const void* src1, void* dst0, void* dst1, int64_t n_bytes, void* stream) {
  if (n_bytes < 0) return fail(ZERO_ERR_INVALID_ARG, "n_bytes < 0");
  if (n_bytes % 16) return fail(ZERO_ERR_INVALID_ARG, "n_bytes = %lld is not a multiple of 16", (long long)n_bytes);
  if (n_bytes == 0) return ZERO_OK;
  if (!src0 || !src1 || !dst0 || !dst1) return fail(ZERO_ERR_INVALID_ARG, "a buffer is NULL");
  if (!aligned(src0, 16) || !aligned(src1, 16) || !aligned(dst0, 16) || !aligned(dst1, 16))
    return fail(ZERO_ERR_ALIGNMENT, "buffers must be 16-byte aligned");
  if (int rc = check_device()) return rc;
  hipError_t e = launch_copy_probe(src0, src1, dst0, dst1, n_bytes / 16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZERO_OK : hip_fail(e, "copy probe launch");
}

int zero_cast_writeback(const float* master, int64_t n, void* flat_param, int64_t offset, int32_t param_dt,
                        void* stream) {
  if (n < 0) return fail(ZERO_ERR_INVALID_ARG, "n < 0");
  if (offset < 0) return fail(ZERO_ERR_INVALID_ARG, "offset < 0");
  if (!valid_dt(param_dt)) return fail(ZERO_ERR_INVALID_ARG, "param dtype %d is not f16/bf16", param_dt);
  if (n == 0) return ZERO_OK;  // nothing to write
  if (!master || !flat_param) return fail(ZERO_ERR_INVALID_ARG, "master or flat_param is NULL");
  if (!aligned(master, 4)) return fail(ZERO_ERR_ALIGNMENT, "master is not 4-byte aligned");
  if (!aligned(flat_param, 2)) return fail(ZERO_ERR_ALIGNMENT, "flat_param is not 2-byte aligned");
  if (int rc = check_device()) return rc;
  CastArgs C;
  C.master = master;
  C.n = n;
  C.param = static_cast<uint16_t*>(flat_param) + offset;
  C.param_dt = param_dt;
  C.param_align = align_class(C.param);
  hipError_t e = launch_cast(C, aligned(master, 16), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ZERO_OK : hip_fail(e, "cast launch");
}

}  // extern "C"
