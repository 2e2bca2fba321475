// gfx950 (CDNA4) kernels of the ZeRO-DP partitioned optimizer step.
//
// The step is a bandwidth-bound elementwise pass plus two small reductions, so
// these are streaming kernels: 64-lane wavefronts, 256-thread blocks, a
// grid-stride loop over 8 elements per thread per iteration (one 16-byte load
// per 16-bit gradient copy, two 16-byte loads per fp32 state array), a grid
// sized to what stays resident on the 256 CUs, and no matrix cores.
//
// Numerics follow the per-coordinate Adam update of the ZeRO reading notes
// (second part, §3) in fp32 with one rounding per operation: fp-contract is off
// for this file, division and square root are the correctly rounded IEEE
// operations, and the fp32 -> 16-bit writeback rounds to nearest even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>

#include "zero_dp_internal.h"

#pragma clang fp contract(off)

namespace zdp {
namespace {

// ------------------------------------------------------------------------
// 16-bit encodings
// ------------------------------------------------------------------------

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h));
  return static_cast<float>(x);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

template <int DT>
__device__ __forceinline__ float decode16(uint32_t h) {
  if constexpr (DT == kSrcBF16)
    return bf16_to_f32(h);
  else
    return f16_to_f32(h);
}

// fp32 -> 16 bits, round to nearest even, NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t encode16(float x, int dt) {
  if (__builtin_isnan(x)) return dt == ZERO_DT_BF16 ? 0x7FC0u : 0x7E00u;
  if (dt == ZERO_DT_BF16) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
  }
  _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Write 8 consecutive 16-bit values at element pointer p (byte alignment `al`).
__device__ __forceinline__ void store8_16(void* p, const uint32_t h[8], int al) {
  const uint32_t w0 = h[0] | (h[1] << 16), w1 = h[2] | (h[3] << 16);
  const uint32_t w2 = h[4] | (h[5] << 16), w3 = h[6] | (h[7] << 16);
  if (al >= 16) {
    *reinterpret_cast<uint4*>(p) = make_uint4(w0, w1, w2, w3);
  } else if (al == 8) {
    uint2* q = reinterpret_cast<uint2*>(p);
    q[0] = make_uint2(w0, w1);
    q[1] = make_uint2(w2, w3);
  } else if (al == 4) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    q[0] = w0;
    q[1] = w1;
    q[2] = w2;
    q[3] = w3;
  } else {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = static_cast<uint16_t>(h[k]);
  }
}

// ------------------------------------------------------------------------
// Gradient source: the average of this rank's segment over its N_d copies,
//   acc = 0; acc += float(copy_r[j]) for r in order; a = acc / N_d
// ------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ const uint16_t* replica(const GradSource& S, int r) {
  if (S.strided)
    return static_cast<const uint16_t*>(S.rep[0]) + static_cast<int64_t>(r) * S.stride;
  return static_cast<const uint16_t*>(S.rep[r]);
}

template <int DT>
__device__ __forceinline__ void accumulate8(float acc[8], uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc[2 * k] = acc[2 * k] + decode16<DT>(w[k] & 0xFFFFu);
    acc[2 * k + 1] = acc[2 * k + 1] + decode16<DT>(w[k] >> 16);
  }
}

__device__ __forceinline__ float finish_average(float acc, const GradSource& S) {
  if (S.n_d == 1) return acc;
  if (S.inv_nd != 0.0f) return acc * S.inv_nd;  // exact for a power-of-two N_d
  return acc / S.nd;
}

// Averaged gradient of elements j .. j+7 (16-byte aligned vector path).
template <int SRC>
__device__ __forceinline__ void source8(const GradSource& S, int64_t j, float a[8]) {
  if constexpr (SRC == kSrcAvg) {
    const float4 x0 = *reinterpret_cast<const float4*>(S.avg + j);
    const float4 x1 = *reinterpret_cast<const float4*>(S.avg + j + 4);
    a[0] = x0.x; a[1] = x0.y; a[2] = x0.z; a[3] = x0.w;
    a[4] = x1.x; a[5] = x1.y; a[6] = x1.z; a[7] = x1.w;
  } else {
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    const int nd = S.n_d;
    int r = 0;
    // Four copies in flight per step; the additions stay in replica order.
    for (; r + 4 <= nd; r += 4) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(replica<SRC>(S, r) + j);
      const uint4 x1 = *reinterpret_cast<const uint4*>(replica<SRC>(S, r + 1) + j);
      const uint4 x2 = *reinterpret_cast<const uint4*>(replica<SRC>(S, r + 2) + j);
      const uint4 x3 = *reinterpret_cast<const uint4*>(replica<SRC>(S, r + 3) + j);
      accumulate8<SRC>(acc, x0);
      accumulate8<SRC>(acc, x1);
      accumulate8<SRC>(acc, x2);
      accumulate8<SRC>(acc, x3);
    }
    for (; r < nd; ++r) {
      const uint4 x = *reinterpret_cast<const uint4*>(replica<SRC>(S, r) + j);
      accumulate8<SRC>(acc, x);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = finish_average(acc[k], S);
  }
}

// Averaged gradient of one element (any alignment).
template <int SRC>
__device__ __forceinline__ float source1(const GradSource& S, int64_t j) {
  if constexpr (SRC == kSrcAvg) {
    return S.avg[j];
  } else {
    float acc = 0.0f;
    for (int r = 0; r < S.n_d; ++r) acc = acc + decode16<SRC>(replica<SRC>(S, r)[j]);
    return finish_average(acc, S);
  }
}

// ------------------------------------------------------------------------
// Adam / AdamW on one coordinate
// ------------------------------------------------------------------------

struct Scalars {
  float inv_scale, b1, b2, beta1, beta2, c1, c2, eps, lr, decay;
  bool has_decay;
};

__device__ __forceinline__ Scalars load_scalars(const AdamArgs& A) {
  const zero_step_state* st = A.state;
  Scalars s;
  s.inv_scale = static_cast<float>(1.0 / static_cast<double>(st->loss_scale));
  // beta^t for the step being applied: the stored beta^(t-1) times beta, in fp64
  s.b1 = static_cast<float>(1.0 - st->beta1_pow[A.group] * A.beta1_d);
  s.b2 = static_cast<float>(1.0 - st->beta2_pow[A.group] * A.beta2_d);
  s.beta1 = A.beta1;
  s.beta2 = A.beta2;
  s.c1 = A.c1;
  s.c2 = A.c2;
  s.eps = A.eps;
  s.lr = A.lr;
  s.decay = A.decay;
  s.has_decay = A.has_decay != 0;
  return s;
}

__device__ __forceinline__ void adam1(float g, float& th, float& m, float& v, const Scalars& s) {
  float t = th;
  if (s.has_decay) t = t * s.decay;
  const float mt = s.beta1 * m + s.c1 * g;
  const float vt = s.beta2 * v + s.c2 * (g * g);
  const float mh = mt / s.b1;
  const float vh = vt / s.b2;
  const float den = __builtin_sqrtf(vh) + s.eps;
  const float u = mh / den;
  th = t - s.lr * u;
  m = mt;
  v = vt;
}

// ------------------------------------------------------------------------
// Block reduction of the norm / overflow partials (wavefront butterfly, then
// the four wavefronts of the block through LDS), written to the group's slot.
// ------------------------------------------------------------------------

__device__ __forceinline__ void write_partial(double s, int bad, Partial* out, int32_t* count) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  const int any_bad = __any(bad);
  __shared__ double ws[kBlock / 64];
  __shared__ int wf[kBlock / 64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (lane == 0) {
    ws[w] = s;
    wf[w] = any_bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    int f = 0;
#pragma unroll
    for (int k = 0; k < kBlock / 64; ++k) {
      t += ws[k];
      f |= wf[k];
    }
    Partial p;
    p.sumsq = t;
    p.flag = f ? 1 : 0;
    p.pad = 0;
    out[blockIdx.x] = p;
    if (blockIdx.x == 0) *count = static_cast<int32_t>(gridDim.x);
  }
}

// ------------------------------------------------------------------------
// The fused / checked update kernel
//   CHECKED = false: average, overflow + norm partials, Adam, writeback.
//   CHECKED = true : exits if the step was voided; no partials.
// ------------------------------------------------------------------------

template <int SRC, bool VEC, bool CHECKED>
__global__ void __launch_bounds__(kBlock) adam_kernel(const AdamArgs A) {
  if constexpr (CHECKED) {
    if (A.state->skipped) return;
  }
  const Scalars s = load_scalars(A);
  double sumsq = 0.0;
  int bad = 0;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kBlock;
  const int pdt = A.param_dt;
  char* const param = static_cast<char*>(A.param);

  auto one = [&](int64_t j) {
    const float a = source1<SRC>(A.src, j);
    const float g = a * s.inv_scale;
    if constexpr (!CHECKED) {
      bad |= !__builtin_isfinite(a);
      const double gd = static_cast<double>(g);
      sumsq = __builtin_fma(gd, gd, sumsq);
    }
    float th = A.master[j], m = A.m[j], v = A.v[j];
    adam1(g, th, m, v, s);
    A.master[j] = th;
    A.m[j] = m;
    A.v[j] = v;
    if (pdt) reinterpret_cast<uint16_t*>(param)[j] = static_cast<uint16_t>(encode16(th, pdt));
  };

  if constexpr (VEC) {
    const int64_t nv = A.n / kVec;
    for (int64_t i = tid; i < nv; i += nthreads) {
      const int64_t j = i * kVec;
      float a[8];
      source8<SRC>(A.src, j, a);
      const float4 t0 = *reinterpret_cast<const float4*>(A.master + j);
      const float4 t1 = *reinterpret_cast<const float4*>(A.master + j + 4);
      const float4 m0 = *reinterpret_cast<const float4*>(A.m + j);
      const float4 m1 = *reinterpret_cast<const float4*>(A.m + j + 4);
      const float4 v0 = *reinterpret_cast<const float4*>(A.v + j);
      const float4 v1 = *reinterpret_cast<const float4*>(A.v + j + 4);
      float th[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
      float mm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float g = a[k] * s.inv_scale;
        if constexpr (!CHECKED) {
          bad |= !__builtin_isfinite(a[k]);
          const double gd = static_cast<double>(g);
          sumsq = __builtin_fma(gd, gd, sumsq);
        }
        adam1(g, th[k], mm[k], vv[k], s);
      }
      *reinterpret_cast<float4*>(A.master + j) = make_float4(th[0], th[1], th[2], th[3]);
      *reinterpret_cast<float4*>(A.master + j + 4) = make_float4(th[4], th[5], th[6], th[7]);
      *reinterpret_cast<float4*>(A.m + j) = make_float4(mm[0], mm[1], mm[2], mm[3]);
      *reinterpret_cast<float4*>(A.m + j + 4) = make_float4(mm[4], mm[5], mm[6], mm[7]);
      *reinterpret_cast<float4*>(A.v + j) = make_float4(vv[0], vv[1], vv[2], vv[3]);
      *reinterpret_cast<float4*>(A.v + j + 4) = make_float4(vv[4], vv[5], vv[6], vv[7]);
      if (pdt) {
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = encode16(th[k], pdt);
        store8_16(param + 2 * j, h, A.param_align);
      }
    }
    // ragged tail: fewer than 8 elements, one per thread
    const int64_t j = nv * kVec + tid;
    if (j < A.n) one(j);
  } else {
    for (int64_t j = tid; j < A.n; j += nthreads) one(j);
  }
  if constexpr (!CHECKED) write_partial(sumsq, bad, A.partials, A.count);
}

// ------------------------------------------------------------------------
// Average-only pass (checked pipeline) and single-copy scan: writes the fp32
// average (if avg_out) and the norm / overflow partials.
// ------------------------------------------------------------------------

template <int SRC, bool VEC>
__global__ void __launch_bounds__(kBlock) reduce_kernel(const ReduceArgs R) {
  const float inv_scale = static_cast<float>(1.0 / static_cast<double>(R.state->loss_scale));
  double sumsq = 0.0;
  int bad = 0;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kBlock;
  float* const out = R.avg_out;
  auto one = [&](int64_t j) {
    const float a = source1<SRC>(R.src, j);
    bad |= !__builtin_isfinite(a);
    const double gd = static_cast<double>(a * inv_scale);
    sumsq = __builtin_fma(gd, gd, sumsq);
    if (out) out[j] = a;
  };
  if constexpr (VEC) {
    const int64_t nv = R.n / kVec;
    for (int64_t i = tid; i < nv; i += nthreads) {
      const int64_t j = i * kVec;
      float a[8];
      source8<SRC>(R.src, j, a);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        bad |= !__builtin_isfinite(a[k]);
        const double gd = static_cast<double>(a[k] * inv_scale);
        sumsq = __builtin_fma(gd, gd, sumsq);
      }
      if (out) {
        *reinterpret_cast<float4*>(out + j) = make_float4(a[0], a[1], a[2], a[3]);
        *reinterpret_cast<float4*>(out + j + 4) = make_float4(a[4], a[5], a[6], a[7]);
      }
    }
    const int64_t j = nv * kVec + tid;
    if (j < R.n) one(j);
  } else {
    for (int64_t j = tid; j < R.n; j += nthreads) one(j);
  }
  write_partial(sumsq, bad, R.partials, R.count);
}

// ------------------------------------------------------------------------
// One-block kernels: combine partials, state bookkeeping
// ------------------------------------------------------------------------

constexpr int kFinalizeThreads = 1024;

__global__ void __launch_bounds__(kFinalizeThreads) finalize_kernel(const FinalizeArgs F) {
  double s = 0.0;
  int f = 0;
  for (int g = 0; g < F.n_groups; ++g) {
    const Partial* p = F.partials + static_cast<int64_t>(g) * kMaxBlocks;
    int cnt = F.counts[g];  // written by the pass that filled the slot
    cnt = cnt < 0 ? 0 : (cnt > kMaxBlocks ? kMaxBlocks : cnt);
    for (int i = threadIdx.x; i < cnt; i += kFinalizeThreads) {
      s += p[i].sumsq;
      f |= p[i].flag;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  const int any_bad = __any(f);
  __shared__ double ws[kFinalizeThreads / 64];
  __shared__ int wf[kFinalizeThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    ws[w] = s;
    wf[w] = any_bad;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double t = 0.0;
  int flag = 0;
  for (int k = 0; k < kFinalizeThreads / 64; ++k) {
    t += ws[k];
    flag |= wf[k];
  }
  zero_step_state* st = F.state;
  st->grad_norm_sq = t;
  st->grad_norm = static_cast<float>(__builtin_sqrt(t));
  st->overflow = flag ? 1 : 0;
  if (F.mode == 1) {
    // static loss scale: the update was applied whatever the flag says
    st->skipped = 0;
    st->step = st->step + 1;
    for (int g = 0; g < F.n_groups; ++g) {
      st->beta1_pow[g] = st->beta1_pow[g] * F.beta1[g];
      st->beta2_pow[g] = st->beta2_pow[g] * F.beta2[g];
    }
  } else {
    st->skipped = (flag && F.skip_on_overflow) ? 1 : 0;
  }
}

__global__ void commit_kernel(const CommitArgs C) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  zero_step_state* st = C.state;
  if (st->skipped) {
    double sc = static_cast<double>(st->loss_scale) * C.backoff;
    if (sc < C.min_scale) sc = C.min_scale;
    st->loss_scale = static_cast<float>(sc);
    st->good_steps = 0;
    return;
  }
  st->step = st->step + 1;
  for (int g = 0; g < C.n_groups; ++g) {
    st->beta1_pow[g] = st->beta1_pow[g] * C.beta1[g];
    st->beta2_pow[g] = st->beta2_pow[g] * C.beta2[g];
  }
  if (C.dynamic) {
    st->good_steps = st->good_steps + 1;
    if (C.growth_interval > 0 && st->good_steps == C.growth_interval) {
      st->loss_scale = static_cast<float>(static_cast<double>(st->loss_scale) * C.growth);
      st->good_steps = 0;
    }
  }
}

__global__ void state_init_kernel(zero_step_state* st, float loss_scale) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  for (int g = 0; g < ZERO_MAX_GROUPS; ++g) {
    st->beta1_pow[g] = 1.0;
    st->beta2_pow[g] = 1.0;
  }
  st->grad_norm_sq = 0.0;
  st->grad_norm = 0.0f;
  st->loss_scale = loss_scale;
  st->step = 0;
  st->overflow = 0;
  st->skipped = 0;
  st->good_steps = 0;
  st->reserved = 0;
}

// ------------------------------------------------------------------------
// fp32 master -> 16-bit flat vector
// ------------------------------------------------------------------------

template <bool VEC>
__global__ void __launch_bounds__(kBlock) cast_kernel(const CastArgs C) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kBlock;
  char* const param = static_cast<char*>(C.param);
  uint16_t* const p16 = static_cast<uint16_t*>(C.param);
  if constexpr (VEC) {
    const int64_t nv = C.n / kVec;
    for (int64_t i = tid; i < nv; i += nthreads) {
      const int64_t j = i * kVec;
      const float4 x0 = *reinterpret_cast<const float4*>(C.master + j);
      const float4 x1 = *reinterpret_cast<const float4*>(C.master + j + 4);
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t h[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) h[k] = encode16(x[k], C.param_dt);
      store8_16(param + 2 * j, h, C.param_align);
    }
    const int64_t j = nv * kVec + tid;
    if (j < C.n) p16[j] = static_cast<uint16_t>(encode16(C.master[j], C.param_dt));
  } else {
    for (int64_t j = tid; j < C.n; j += nthreads)
      p16[j] = static_cast<uint16_t>(encode16(C.master[j], C.param_dt));
  }
}

// ------------------------------------------------------------------------
// Grid sizing: as many blocks as stay resident on the device (occupancy times
// compute units), no more than the work needs, at most kMaxBlocks.
// ------------------------------------------------------------------------

int resident_blocks(const void* kernel) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  const uint64_t key = (reinterpret_cast<uint64_t>(kernel) << 8) ^ static_cast<uint64_t>(dev);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  int blocks = cus * per_cu;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = blocks;
  return blocks;
}

int grid_for(const void* kernel, int64_t n, bool vec) {
  // threads needed: one per 8-element vector (+ tail) on the vector path,
  // one per element otherwise
  const int64_t units = vec ? (n / kVec + ((n % kVec) ? 1 : 0)) : n;
  int64_t need = (units + kBlock - 1) / kBlock;
  if (need < 1) need = 1;
  const int cap = resident_blocks(kernel);
  return static_cast<int>(need < cap ? need : cap);
}

template <int SRC, bool VEC, bool CHECKED>
hipError_t adam_launch(const AdamArgs& a, hipStream_t s) {
  const void* k = reinterpret_cast<const void*>(&adam_kernel<SRC, VEC, CHECKED>);
  const int grid = grid_for(k, a.n, VEC);
  hipLaunchKernelGGL((adam_kernel<SRC, VEC, CHECKED>), dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int SRC, bool VEC>
hipError_t reduce_launch(const ReduceArgs& a, hipStream_t s) {
  const void* k = reinterpret_cast<const void*>(&reduce_kernel<SRC, VEC>);
  const int grid = grid_for(k, a.n, VEC);
  hipLaunchKernelGGL((reduce_kernel<SRC, VEC>), dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_adam(const AdamArgs& a, int src, bool vec, bool checked, hipStream_t s) {
#define ZDP_ADAM(SRC)                                                         \
  if (src == SRC) {                                                           \
    if (vec) return checked ? adam_launch<SRC, true, true>(a, s)              \
                            : adam_launch<SRC, true, false>(a, s);            \
    return checked ? adam_launch<SRC, false, true>(a, s)                      \
                   : adam_launch<SRC, false, false>(a, s);                    \
  }
  ZDP_ADAM(kSrcAvg)
  ZDP_ADAM(kSrcF16)
  ZDP_ADAM(kSrcBF16)
#undef ZDP_ADAM
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, int src, bool vec, hipStream_t s) {
  if (src == kSrcF16) return vec ? reduce_launch<kSrcF16, true>(a, s) : reduce_launch<kSrcF16, false>(a, s);
  if (src == kSrcBF16) return vec ? reduce_launch<kSrcBF16, true>(a, s) : reduce_launch<kSrcBF16, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kFinalizeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_state_init(zero_step_state* st, float loss_scale, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(64), 0, s, st, loss_scale);
  return hipGetLastError();
}

hipError_t launch_cast(const CastArgs& a, bool vec, hipStream_t s) {
  if (vec) {
    const void* k = reinterpret_cast<const void*>(&cast_kernel<true>);
    hipLaunchKernelGGL(cast_kernel<true>, dim3(grid_for(k, a.n, true)), dim3(kBlock), 0, s, a);
  } else {
    const void* k = reinterpret_cast<const void*>(&cast_kernel<false>);
    hipLaunchKernelGGL(cast_kernel<false>, dim3(grid_for(k, a.n, false)), dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace zdp
