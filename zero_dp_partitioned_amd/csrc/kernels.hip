// gfx950 (CDNA4) kernels of the ZeRO-DP partitioned optimizer step.
//
// The step is a bandwidth-bound elementwise pass plus a norm reduction, so
// these are streaming kernels without matrix cores. Layout (see
// zero_dp_internal.h): 256-thread blocks own 4096-element tiles and walk them
// as 4-element quads, lane l on quads l, l+256, l+512, l+768, so every
// wavefront load or store is one contiguous 1 KiB (fp32) or 512 B (16-bit)
// run. One block per tile: the hardware dispatcher hands out tiles in order,
// which keeps the resident blocks on one advancing window of HBM; on gfx950
// this sustains clearly more bandwidth for a read-modify-write stream than a
// resident grid looping over the vector (launches beyond 2^21 tiles do loop).
// With 32 or more gradient copies the update kernel's lanes take 8 quads
// (8192-element tiles) and read the copies one after another with a cap on
// the loads in flight (source_tile). With 2 to 31 copies it takes the batched
// schedule instead: a whole tile's loads in flight at once, then the
// arithmetic, then the stores array by array, at two blocks per CU (a dynamic
// LDS share the kernel never touches caps the residency); the averaging pass
// reads that way from 8 to 32 copies, and the update from an fp32 average runs
// at the same two blocks per CU. Arrays that all start at the same offset
// modulo 4 elements run the quad path after a head of up to 3 elements that
// block 0 updates one by one.
//
// Numerics follow the per-coordinate Adam update of the ZeRO reading notes
// (second part, §3) in fp32 with one rounding per operation: fp-contract is off
// for this file, division and square root are the correctly rounded IEEE
// operations, and the fp32 -> 16-bit writeback rounds to nearest even.
//
// Norm and overflow flag: every block writes one fp64 partial (sum of g^2 of
// its elements, or NaN if one of its averaged gradients was inf/NaN); a fold
// kernel reduces a launch's partials into 256 per-group values, and a one-block
// kernel combines those. Every reduction has a fixed shape, so the norm is the
// same bit pattern run after run.
//
// The exceptions to one block per tile are launches that either rarely do any
// work or are bound by per-block costs: the restore and second-pass launches
// of the optimistic pipeline (they exit at once unless a step was voided or
// clipped) and the single-copy scan (16-byte loads, a block reads many tiles).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_dp_internal.h"

#pragma clang fp contract(off)

namespace zdp {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------
// Streaming accesses. Every byte a step touches is read once and written
// once, so the vector loads and stores of the quad paths carry the
// non-temporal hint: on gfx950 the read-modify-write of the fp32 state then
// sustains a few per cent more HBM bandwidth than with the default policy.
// ------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, T x) {
  __builtin_nontemporal_store(x, p);
}

// ------------------------------------------------------------------------
// 16-bit encodings
// ------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ float decode16(uint32_t h) {
  if constexpr (DT == kSrcBF16) {
    return __uint_as_float(h << 16);
  } else {
    const _Float16 x = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h));
    return static_cast<float>(x);
  }
}

// fp32 -> 16 bits, round to nearest even, NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t encode16(float x, int dt) {
  if (__builtin_isnan(x)) return dt == ZERO_DT_BF16 ? 0x7FC0u : 0x7E00u;
  if (dt == ZERO_DT_BF16) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
  }
  const _Float16 h = static_cast<_Float16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Four consecutive 16-bit values at p, with p's byte alignment `al` (8, 4, 2).
__device__ __forceinline__ void store4_16(uint16_t* p, const uint32_t h[4], int al) {
  const uint32_t w0 = h[0] | (h[1] << 16), w1 = h[2] | (h[3] << 16);
  if (al >= 8) {
    u2 w;
    w.x = w0;
    w.y = w1;
    st_stream(reinterpret_cast<u2*>(p), w);
  } else if (al == 4) {
    st_stream(reinterpret_cast<uint32_t*>(p), w0);
    st_stream(reinterpret_cast<uint32_t*>(p) + 1, w1);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = static_cast<uint16_t>(h[k]);
  }
}

// ------------------------------------------------------------------------
// Gradient source: the average of this rank's segment over its N_d copies,
//   acc = 0; acc += float(copy_r[j]) for r in order; a = acc / N_d
// ------------------------------------------------------------------------

__device__ __forceinline__ const uint16_t* replica(const GradSource& S, int r) {
  if (S.strided) return static_cast<const uint16_t*>(S.rep[0]) + static_cast<int64_t>(r) * S.stride;
  return static_cast<const uint16_t*>(S.rep[r]);
}

template <int DT>
__device__ __forceinline__ void accumulate4(float acc[4], u2 x) {
  acc[0] = acc[0] + decode16<DT>(x.x & 0xFFFFu);
  acc[1] = acc[1] + decode16<DT>(x.x >> 16);
  acc[2] = acc[2] + decode16<DT>(x.y & 0xFFFFu);
  acc[3] = acc[3] + decode16<DT>(x.y >> 16);
}

__device__ __forceinline__ float finish_average(float acc, const GradSource& S) {
  if (S.n_d == 1) return acc;
  if (S.inv_nd != 0.0f) return acc * S.inv_nd;  // exact for a power-of-two N_d
  return acc / S.nd;
}

// Averaged gradient of elements e .. e+3 (aligned quad path).
template <int SRC>
__device__ __forceinline__ void source4(const GradSource& S, int64_t e, float a[4]) {
  if constexpr (SRC == kSrcAvg) {
    const f4 x = ld_stream(reinterpret_cast<const f4*>(S.avg + e));
    a[0] = x.x;
    a[1] = x.y;
    a[2] = x.z;
    a[3] = x.w;
  } else {
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int nd = S.n_d;
    int r = 0;
    // eight copies in flight at a time; the additions stay in replica order
    for (; r + 8 <= nd; r += 8) {
      u2 x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = ld_stream(reinterpret_cast<const u2*>(replica(S, r + q) + e));
#pragma unroll
      for (int q = 0; q < 8; ++q) accumulate4<SRC>(acc, x[q]);
    }
    for (; r < nd; ++r) accumulate4<SRC>(acc, ld_stream(reinterpret_cast<const u2*>(replica(S, r) + e)));
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = finish_average(acc[k], S);
  }
}

// Waits until at most N-1 of the wave's vector loads are outstanding.
template <int N>
__device__ __forceinline__ void bound_loads_in_flight() {
  static_assert(N >= 1 && N <= 8, "bound of 1-8 loads");
  if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else if constexpr (N == 7) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
}

// Averaged gradients of a lane's QL quads of a full tile (quads at t0 +
// (k*256 + lane)*4, k < QL), copy by copy: a block reads copy 0's QL * 2 KiB
// of the tile, then copy 1's, and so on. INFL > 0 caps the gradient loads a
// wave has in flight at INFL; INFL = 0 issues eight copies' loads at once.
// With many copies the capped order is faster: the requests HBM has queued
// then fall into few DRAM rows at a time. The additions per element stay in
// replica order either way.
template <int SRC, int QL, int INFL>
__device__ __forceinline__ void source_tile(const GradSource& S, int64_t t0, float a[QL][4]) {
  float acc[QL][4] = {};
  const int nd = S.n_d;
  const int64_t lane4 = static_cast<int64_t>(threadIdx.x) * 4;
  int r = 0;
  if constexpr (INFL == 0) {
    for (; r + 8 <= nd; r += 8) {
      u2 x[8][QL];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int k = 0; k < QL; ++k)
          x[q][k] = ld_stream(reinterpret_cast<const u2*>(replica(S, r + q) + t0 + k * kBlock * 4 + lane4));
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int k = 0; k < QL; ++k) accumulate4<SRC>(acc[k], x[q][k]);
    }
  }
  for (; r < nd; ++r) {
    const uint16_t* const c = replica(S, r) + t0 + lane4;
    u2 x[QL];
#pragma unroll
    for (int k = 0; k < QL; ++k) {
      x[k] = ld_stream(reinterpret_cast<const u2*>(c + k * kBlock * 4));
      if constexpr (INFL > 0) bound_loads_in_flight<INFL>();
    }
#pragma unroll
    for (int k = 0; k < QL; ++k) accumulate4<SRC>(acc[k], x[k]);
  }
#pragma unroll
  for (int k = 0; k < QL; ++k)
#pragma unroll
    for (int q = 0; q < 4; ++q) a[k][q] = finish_average(acc[k][q], S);
}

// Averaged gradient of one element (any alignment).
template <int SRC>
__device__ __forceinline__ float source1(const GradSource& S, int64_t j) {
  if constexpr (SRC == kSrcAvg) {
    return S.avg[j];
  } else {
    float acc = 0.0f;
    for (int r = 0; r < S.n_d; ++r) acc = acc + decode16<SRC>(replica(S, r)[j]);
    return finish_average(acc, S);
  }
}

// ------------------------------------------------------------------------
// Adam / AdamW on one coordinate
// ------------------------------------------------------------------------

struct Scalars {
  float inv_scale, clip, b1, b2, beta1, beta2, c1, c2, eps, lr, decay;
  bool has_decay;
};

__device__ __forceinline__ Scalars load_scalars(const AdamArgs& A) {
  const zero_step_state* st = A.state;
  Scalars s;
  s.inv_scale = static_cast<float>(1.0 / static_cast<double>(st->loss_scale));
  s.clip = st->clip_coef;  // set by the norm pass of the checked pipeline; 1 = none
  // beta^t of the step being applied: the stored beta^(t-1) times beta, in fp64
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

// Norm / overflow contribution of one averaged gradient.
__device__ __forceinline__ void account(float a, float g, double& sumsq, int& bad) {
  bad |= !__builtin_isfinite(a);
  const double gd = static_cast<double>(g);
  sumsq = __builtin_fma(gd, gd, sumsq);
}

// One fp64 partial per block: wavefront butterfly, then the block's four
// wavefronts through LDS in a fixed order. NaN marks a non-finite gradient.
// With fill > gridDim.x (a small launch writing a group's level-2 partials
// directly) the blocks also zero the slots [gridDim.x, fill), each once.
__device__ __forceinline__ void write_block_partial(double s, int bad, double* out, int fill) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  const int any_bad = __any(bad);
  __shared__ double ws[kBlock / 64];
  __shared__ int wf[kBlock / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
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
    out[blockIdx.x] = f ? __builtin_nan("") : t;
    for (int k = blockIdx.x + gridDim.x; k < fill; k += gridDim.x) out[k] = 0.0;
  }
}

// ------------------------------------------------------------------------
// The update kernel
//   kFused: average, norm partials, Adam, writeback.
//   kChecked: exits if the step was voided; clip multiplier; no partials.
//   kOptimistic: as kFused, but reads the current state set and writes the
//     other one (state->cur picks which is which).
//   kRedo: the second pass of a clipped optimistic step: exits unless
//     state->redo; as kOptimistic with the clip multiplier, no partials.
// VEC: fp32 arrays 16-byte and 16-bit copies 8-byte aligned (quad path).
// QL: quads per lane, so tiles of kBlock * QL * 4 elements (see tile_quads).
// BATCH (several copies, 4-quad tiles): a full tile is read in one batch --
//   the state of all four quads first, then every copy -- then updated, then
//   stored one array at a time (master, m, v, parameters), each store a 1 KiB
//   run per wave. Launched with at most two blocks per CU (see adam_launch).
//   On the 13B shard at N_d = 8 (optimistic) this moves the step from 79.2 %
//   to 80.0 % of 8 TB/s; either change alone, or the batch at three blocks per
//   CU (its register-bound residency), is slower than the plain schedule.
//   Results are the same bits: the same operations per element, and the norm
//   partials accumulate in the same order.
// ------------------------------------------------------------------------

template <int SRC, bool VEC, int MODE, int QL, bool BATCH>
__global__ void __launch_bounds__(kBlock) adam_kernel(const AdamArgs A) {
  constexpr bool CHECKED = MODE == kChecked;
  constexpr bool REDO = MODE == kRedo;
  constexpr bool CLIPPED = CHECKED || REDO;      // multiplier known before the update; no partials
  constexpr bool SWAP = MODE == kOptimistic || REDO;
  if constexpr (CHECKED) {
    if (A.state->skipped) return;
  }
  if constexpr (REDO) {
    if (!A.state->redo) return;
  }
  const Scalars s = load_scalars(A);
  const float* mst_in = A.master;
  const float* m_in = A.m;
  const float* v_in = A.v;
  float* mst_out = A.master;
  float* m_out = A.m;
  float* v_out = A.v;
  if constexpr (SWAP) {
    const bool alt_is_current = A.state->cur != 0;
    mst_in = alt_is_current ? A.master_alt : A.master;
    m_in = alt_is_current ? A.m_alt : A.m;
    v_in = alt_is_current ? A.v_alt : A.v;
    mst_out = alt_is_current ? A.master : A.master_alt;
    m_out = alt_is_current ? A.m : A.m_alt;
    v_out = alt_is_current ? A.v : A.v_alt;
  }
  double sumsq = 0.0;
  int bad = 0;
  const int pdt = A.param_dt;
  uint16_t* const param = static_cast<uint16_t*>(A.param);
  const int64_t n = A.n;
  constexpr int64_t T = static_cast<int64_t>(kBlock) * QL * 4;
  const int64_t h = A.head;  // tiles start at element h (aligned for the quad path)
  const int64_t ntiles = (n - h + T - 1) / T;

  auto one = [&](int64_t j) {
    const float a = source1<SRC>(A.src, j);
    float g = a * s.inv_scale;
    if constexpr (!CLIPPED) account(a, g, sumsq, bad);
    if constexpr (CLIPPED) g = g * s.clip;
    float th = mst_in[j], m = m_in[j], v = v_in[j];
    adam1(g, th, m, v, s);
    mst_out[j] = th;
    m_out[j] = m;
    v_out[j] = v;
    if (pdt) param[j] = static_cast<uint16_t>(encode16(th, pdt));
  };

  // one quad's update from its averaged gradient a[4] (quad path)
  auto quad = [&](int64_t e, const float a[4]) {
    const f4 t4 = ld_stream(reinterpret_cast<const f4*>(mst_in + e));
    const f4 m4 = ld_stream(reinterpret_cast<const f4*>(m_in + e));
    const f4 v4 = ld_stream(reinterpret_cast<const f4*>(v_in + e));
    float th[4] = {t4.x, t4.y, t4.z, t4.w};
    float mm[4] = {m4.x, m4.y, m4.z, m4.w};
    float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float g = a[q] * s.inv_scale;
      if constexpr (!CLIPPED) account(a[q], g, sumsq, bad);
      if constexpr (CLIPPED) g = g * s.clip;
      adam1(g, th[q], mm[q], vv[q], s);
    }
    st_stream(reinterpret_cast<f4*>(mst_out + e), (f4){th[0], th[1], th[2], th[3]});
    st_stream(reinterpret_cast<f4*>(m_out + e), (f4){mm[0], mm[1], mm[2], mm[3]});
    st_stream(reinterpret_cast<f4*>(v_out + e), (f4){vv[0], vv[1], vv[2], vv[3]});
    if (pdt) {
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = encode16(th[q], pdt);
      store4_16(param + e, h, A.param_align);
    }
  };

  if (blockIdx.x == 0 && threadIdx.x < h) one(threadIdx.x);
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t t0 = h + t * T;
    if constexpr (BATCH && VEC && SRC != kSrcAvg && QL == kQuadsPerThread) {
      if (A.src.n_d > 1 && t0 + T <= n) {
        const int64_t lane4 = static_cast<int64_t>(threadIdx.x) * 4;
        f4 T4[QL], M4[QL], V4[QL];
#pragma unroll
        for (int k = 0; k < QL; ++k) {
          const int64_t e = t0 + k * kBlock * 4 + lane4;
          T4[k] = ld_stream(reinterpret_cast<const f4*>(mst_in + e));
          M4[k] = ld_stream(reinterpret_cast<const f4*>(m_in + e));
          V4[k] = ld_stream(reinterpret_cast<const f4*>(v_in + e));
        }
        float at[QL][4];
        source_tile<SRC, QL, 0>(A.src, t0, at);
#pragma unroll
        for (int k = 0; k < QL; ++k) {
          float th[4] = {T4[k].x, T4[k].y, T4[k].z, T4[k].w};
          float mm[4] = {M4[k].x, M4[k].y, M4[k].z, M4[k].w};
          float vv[4] = {V4[k].x, V4[k].y, V4[k].z, V4[k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float g = at[k][q] * s.inv_scale;
            if constexpr (!CLIPPED) account(at[k][q], g, sumsq, bad);
            if constexpr (CLIPPED) g = g * s.clip;
            adam1(g, th[q], mm[q], vv[q], s);
          }
          T4[k] = (f4){th[0], th[1], th[2], th[3]};
          M4[k] = (f4){mm[0], mm[1], mm[2], mm[3]};
          V4[k] = (f4){vv[0], vv[1], vv[2], vv[3]};
        }
#pragma unroll
        for (int k = 0; k < QL; ++k) st_stream(reinterpret_cast<f4*>(mst_out + t0 + k * kBlock * 4 + lane4), T4[k]);
#pragma unroll
        for (int k = 0; k < QL; ++k) st_stream(reinterpret_cast<f4*>(m_out + t0 + k * kBlock * 4 + lane4), M4[k]);
#pragma unroll
        for (int k = 0; k < QL; ++k) st_stream(reinterpret_cast<f4*>(v_out + t0 + k * kBlock * 4 + lane4), V4[k]);
        if (pdt) {
#pragma unroll
          for (int k = 0; k < QL; ++k) {
            const uint32_t hq[4] = {encode16(T4[k].x, pdt), encode16(T4[k].y, pdt), encode16(T4[k].z, pdt),
                                    encode16(T4[k].w, pdt)};
            store4_16(param + t0 + k * kBlock * 4 + lane4, hq, A.param_align);
          }
        }
        continue;
      }
    }
    if constexpr (VEC && SRC != kSrcAvg) {
      // several copies, a full tile: read them copy by copy
      if (A.src.n_d > 1 && t0 + T <= n) {
        float at[QL][4];
        source_tile<SRC, QL, tile_inflight(QL)>(A.src, t0, at);
#pragma unroll
        for (int k = 0; k < QL; ++k) quad(t0 + static_cast<int64_t>(k * kBlock + threadIdx.x) * 4, at[k]);
        continue;
      }
    }
#pragma unroll
    for (int k = 0; k < QL; ++k) {
      const int64_t e = t0 + static_cast<int64_t>(k * kBlock + threadIdx.x) * 4;
      if (VEC && e + 4 <= n) {
        float a[4];
        source4<SRC>(A.src, e, a);
        quad(e, a);
      } else {
        for (int q = 0; q < 4; ++q)
          if (e + q < n) one(e + q);
      }
    }
  }
  if constexpr (!CLIPPED) write_block_partial(sumsq, bad, A.partials, A.fill);
}

// ------------------------------------------------------------------------
// Average-only pass (checked pipeline) and single-copy scan: the fp32 average
// (if avg_out) and the norm / overflow partials.
// ------------------------------------------------------------------------

template <int SRC, bool VEC, int QL, int INFL>
__global__ void __launch_bounds__(kBlock) reduce_kernel(const ReduceArgs R) {
  const float inv_scale = static_cast<float>(1.0 / static_cast<double>(R.state->loss_scale));
  double sumsq = 0.0;
  int bad = 0;
  float* const out = R.avg_out;
  const int64_t n = R.n;
  constexpr int64_t T = static_cast<int64_t>(kBlock) * QL * 4;
  const int64_t h = R.head;  // tiles start at element h (aligned for the quad path)
  const int64_t ntiles = (n - h + T - 1) / T;
  if (blockIdx.x == 0 && threadIdx.x < h) {
    const float a = source1<SRC>(R.src, threadIdx.x);
    account(a, a * inv_scale, sumsq, bad);
    if (out) out[threadIdx.x] = a;
  }
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t t0 = h + t * T;
    if constexpr (VEC) {
      // several copies, a full tile: read them copy by copy
      if (R.src.n_d > 1 && t0 + T <= n) {
        float at[QL][4];
        source_tile<SRC, QL, INFL>(R.src, t0, at);
#pragma unroll
        for (int k = 0; k < QL; ++k) {
          const int64_t e = t0 + static_cast<int64_t>(k * kBlock + threadIdx.x) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q) account(at[k][q], at[k][q] * inv_scale, sumsq, bad);
          if (out) st_stream(reinterpret_cast<f4*>(out + e), (f4){at[k][0], at[k][1], at[k][2], at[k][3]});
        }
        continue;
      }
    }
#pragma unroll
    for (int k = 0; k < QL; ++k) {
      const int64_t e = t0 + static_cast<int64_t>(k * kBlock + threadIdx.x) * 4;
      if (VEC && e + 4 <= n) {
        float a[4];
        source4<SRC>(R.src, e, a);
#pragma unroll
        for (int q = 0; q < 4; ++q) account(a[q], a[q] * inv_scale, sumsq, bad);
        if (out) st_stream(reinterpret_cast<f4*>(out + e), (f4){a[0], a[1], a[2], a[3]});
      } else {
        for (int q = 0; q < 4; ++q) {
          if (e + q >= n) break;
          const float a = source1<SRC>(R.src, e + q);
          account(a, a * inv_scale, sumsq, bad);
          if (out) out[e + q] = a;
        }
      }
    }
  }
  write_block_partial(sumsq, bad, R.partials, R.fill);
}

// ------------------------------------------------------------------------
// Scan of one 16-byte-aligned gradient copy (N_d = 1, no average written):
// the norm / overflow partials only. Lanes take 8 consecutive elements
// (16-byte loads), tiles of 4096 as elsewhere; a capped grid loops over the
// tiles, so each block reads many tiles and its fixed costs amortise.
// ------------------------------------------------------------------------

template <int SRC>
__global__ void __launch_bounds__(kBlock) scan_kernel(const ReduceArgs R) {
  const float inv_scale = static_cast<float>(1.0 / static_cast<double>(R.state->loss_scale));
  const uint16_t* const src = static_cast<const uint16_t*>(R.src.rep[0]);
  double sumsq = 0.0;
  int bad = 0;
  const int64_t n = R.n;
  const int64_t ntiles = (n + kTile - 1) / kTile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
#pragma unroll
    for (int k = 0; k < kTile / (kBlock * 8); ++k) {
      const int64_t e = t * kTile + static_cast<int64_t>(k * kBlock + threadIdx.x) * 8;
      if (e + 8 <= n) {
        const u4 x = ld_stream(reinterpret_cast<const u4*>(src + e));
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = decode16<SRC>(w[q] & 0xFFFFu), hi = decode16<SRC>(w[q] >> 16);
          account(lo, lo * inv_scale, sumsq, bad);
          account(hi, hi * inv_scale, sumsq, bad);
        }
      } else {
        for (int64_t j = e; j < n && j < e + 8; ++j) {
          const float a = decode16<SRC>(src[j]);
          account(a, a * inv_scale, sumsq, bad);
        }
      }
    }
  }
  write_block_partial(sumsq, bad, R.partials, R.fill);
}

// ------------------------------------------------------------------------
// Fold: block j of kFoldBlocks sums partials [j*C, min((j+1)*C, count)) with
// C = ceil(count / kFoldBlocks), thread i taking i, i+256, ... of the range.
// ------------------------------------------------------------------------

__device__ __forceinline__ double block_sum(double s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  __shared__ double ws[kBlock / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) ws[w] = s;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < kBlock / 64; ++k) t += ws[k];
  __syncthreads();
  return t;
}

__global__ void __launch_bounds__(kBlock) fold_kernel(const FoldArgs F) {
  const int64_t per = (F.count + kFoldBlocks - 1) / kFoldBlocks;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < F.count ? lo + per : F.count;
  double s = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) s += F.partials[i];
  const double t = block_sum(s);
  if (threadIdx.x == 0) F.level2[blockIdx.x] = t;
}

// ------------------------------------------------------------------------
// One-block kernels: combine the groups' level-2 partials, state bookkeeping
// ------------------------------------------------------------------------

// An applied step: t + 1, beta powers, and (dynamic scale) the growth window.
__device__ __forceinline__ void advance(zero_step_state* st, int n_groups, const double* beta1,
                                        const double* beta2, bool dynamic, int growth_interval,
                                        double growth) {
  st->step = st->step + 1;
  for (int g = 0; g < n_groups; ++g) {
    st->beta1_pow[g] = st->beta1_pow[g] * beta1[g];
    st->beta2_pow[g] = st->beta2_pow[g] * beta2[g];
  }
  if (dynamic) {
    st->good_steps = st->good_steps + 1;
    if (growth_interval > 0 && st->good_steps == growth_interval) {
      st->loss_scale = static_cast<float>(static_cast<double>(st->loss_scale) * growth);
      st->good_steps = 0;
    }
  }
}

// Clip multiplier min(1, max_norm / (norm + 1e-6)) from the fp64 norm², rounded once; 1 = none.
__device__ __forceinline__ float clip_multiplier(double max_grad_norm, double norm_sq) {
  if (!(max_grad_norm > 0.0) || !__builtin_isfinite(norm_sq)) return 1.0f;
  const double c = max_grad_norm / (__builtin_sqrt(norm_sq) + 1e-6);
  return static_cast<float>(c < 1.0 ? c : 1.0);
}

__global__ void __launch_bounds__(kBlock) finalize_kernel(const FinalizeArgs F) {
  double total = 0.0;
  for (int g = 0; g < F.n_groups; ++g) total += block_sum(F.level2[g * kFoldBlocks + threadIdx.x]);
  if (threadIdx.x != 0) return;
  zero_step_state* st = F.state;
  const int flag = __builtin_isnan(total) ? 1 : 0;  // a non-finite gradient poisons its partial
  st->grad_norm_sq = total;
  st->grad_norm = static_cast<float>(__builtin_sqrt(total));
  st->overflow = flag;
  if (F.mode == 1) {
    // static loss scale: the update was applied whatever the flag says
    st->clip_coef = 1.0f;
    st->skipped = 0;
    advance(st, F.n_groups, F.beta1, F.beta2, false, 0, 1.0);
  } else if (F.mode == 2) {
    // optimistic: the update went to the other state set; keep it, drop it, or
    // (clipping) have the second pass redo it from the current set
    st->clip_coef = 1.0f;
    st->redo = 0;
    if (flag) {
      st->skipped = 1;
      double sc = static_cast<double>(st->loss_scale) * F.backoff;
      if (sc < F.min_scale) sc = F.min_scale;
      st->loss_scale = static_cast<float>(sc);
      st->good_steps = 0;
    } else {
      st->skipped = 0;
      const float clip = clip_multiplier(F.max_grad_norm, total);
      if (clip < 1.0f) {
        st->clip_coef = clip;
        st->redo = 1;  // redo_commit_kernel flips and advances after the second pass
      } else {
        st->cur = st->cur ^ 1;
        advance(st, F.n_groups, F.beta1, F.beta2, true, F.growth_interval, F.growth);
      }
    }
  } else {
    st->skipped = (flag && F.skip_on_overflow) ? 1 : 0;
    st->clip_coef = clip_multiplier(F.max_grad_norm, total);
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
  advance(st, C.n_groups, C.beta1, C.beta2, C.dynamic != 0, C.growth_interval, C.growth);
}

// After the second pass of a clipped optimistic step: the other set now holds
// the clipped update; make it current and count the step.
__global__ void redo_commit_kernel(const CommitArgs C) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  zero_step_state* st = C.state;
  if (!st->redo) return;
  st->redo = 0;
  st->cur = st->cur ^ 1;
  advance(st, C.n_groups, C.beta1, C.beta2, true, C.growth_interval, C.growth);
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
  st->clip_coef = 1.0f;
  st->cur = 0;
  st->redo = 0;
}

// ------------------------------------------------------------------------
// fp32 master -> 16-bit flat vector
// ------------------------------------------------------------------------

template <bool VEC>
__global__ void __launch_bounds__(kBlock) cast_kernel(const CastArgs C) {
  uint16_t* const p16 = static_cast<uint16_t*>(C.param);
  const int64_t n = C.n;
  const int64_t ntiles = (n + kTile - 1) / kTile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
#pragma unroll
    for (int k = 0; k < kQuadsPerThread; ++k) {
      const int64_t e = t * kTile + static_cast<int64_t>(k * kBlock + threadIdx.x) * 4;
      if (VEC && e + 4 <= n) {
        const f4 x = ld_stream(reinterpret_cast<const f4*>(C.master + e));
        const uint32_t h[4] = {encode16(x.x, C.param_dt), encode16(x.y, C.param_dt),
                               encode16(x.z, C.param_dt), encode16(x.w, C.param_dt)};
        store4_16(p16 + e, h, C.param_align);
      } else {
        for (int q = 0; q < 4; ++q)
          if (e + q < n) p16[e + q] = static_cast<uint16_t>(encode16(C.master[e + q], C.param_dt));
      }
    }
  }
}

// Voided optimistic step: rewrite the parameter slice from the current master.
// A small resident grid, so that the launch costs little when there is
// nothing to do (the common case).
constexpr int kRestoreGrid = 1024;

template <bool VEC>
__global__ void __launch_bounds__(kBlock) restore_kernel(const RestoreArgs R) {
  const zero_step_state* st = R.state;
  if (!st->skipped) return;
  const float* master = st->cur ? R.master_alt : R.master;
  uint16_t* const p16 = static_cast<uint16_t*>(R.param);
  const int64_t n = R.n;
  const int64_t ntiles = (n + kTile - 1) / kTile;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
#pragma unroll
    for (int k = 0; k < kQuadsPerThread; ++k) {
      const int64_t e = t * kTile + static_cast<int64_t>(k * kBlock + threadIdx.x) * 4;
      if (VEC && e + 4 <= n) {
        const f4 x = ld_stream(reinterpret_cast<const f4*>(master + e));
        const uint32_t h[4] = {encode16(x.x, R.param_dt), encode16(x.y, R.param_dt),
                               encode16(x.z, R.param_dt), encode16(x.w, R.param_dt)};
        store4_16(p16 + e, h, R.param_align);
      } else {
        for (int q = 0; q < 4; ++q)
          if (e + q < n) p16[e + q] = static_cast<uint16_t>(encode16(master[e + q], R.param_dt));
      }
    }
  }
}

// A launch of at most kFoldBlocks blocks with the group's level-2 partials at
// hand writes them itself: block b's partial into slot b, zeros into the
// slots past its grid. That is what the fold would write: with one partial
// per slot, its sums only add zeros, which changes no bit (a partial, a sum
// of squares from +0, is never -0). *blocks = 0 then tells the caller that
// nothing is left to fold; otherwise it is the grid.
template <typename Args>
Args route_partials(const Args& a, int grid, int* blocks) {
  Args b = a;
  b.fill = 0;
  *blocks = grid;
  if (a.level2 && a.partials && grid <= kFoldBlocks) {
    b.partials = a.level2;
    b.fill = kFoldBlocks;
    *blocks = 0;
  }
  return b;
}

// The batched schedule (2 to 31 copies, 4-quad tiles) gets `batch_lds` bytes
// of dynamic LDS per block, which it never touches: it caps the blocks
// resident per CU at kBatchBlocksPerCU.
template <int SRC, bool VEC, int MODE, int QL>
hipError_t adam_launch(const AdamArgs& args, size_t batch_lds, hipStream_t s, int* blocks) {
  int grid = stream_grid(args.n - args.head, QL);
  if (MODE == kRedo && grid > kRedoGrid) grid = kRedoGrid;
  const AdamArgs a = route_partials(args, grid, blocks);
  if constexpr (QL == kQuadsPerThread && VEC && SRC != kSrcAvg) {
    if (batched(SRC, VEC, a.src.n_d)) {
      hipLaunchKernelGGL((adam_kernel<SRC, VEC, MODE, QL, true>), dim3(grid), dim3(kBlock), batch_lds, s, a);
      return hipGetLastError();
    }
  }
  // the update from an fp32 average (checked pipeline) is capped the same way:
  // at its register-bound eight blocks per CU it ran 0.3-0.5 % slower
  const size_t lds = (SRC == kSrcAvg && VEC) ? batch_lds : 0;
  hipLaunchKernelGGL((adam_kernel<SRC, VEC, MODE, QL, false>), dim3(grid), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

template <int SRC, bool VEC, int INFL>
hipError_t reduce_launch(const ReduceArgs& args, size_t lds, hipStream_t s, int* blocks) {
  const int grid = stream_grid(args.n - args.head, kQuadsPerThread);
  const ReduceArgs a = route_partials(args, grid, blocks);
  hipLaunchKernelGGL((reduce_kernel<SRC, VEC, kQuadsPerThread, INFL>), dim3(grid), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_adam(const AdamArgs& a, int src, bool vec, int mode, size_t batch_lds, hipStream_t s,
                       int* blocks) {
  const bool wide = tile_quads(src, vec, a.src.n_d) == kQuadsWide;
#define ZDP_ADAM_MODE(SRC, VEC, QL)                                                            \
  switch (mode) {                                                                              \
    case kFused: return adam_launch<SRC, VEC, kFused, QL>(a, batch_lds, s, blocks);            \
    case kChecked: return adam_launch<SRC, VEC, kChecked, QL>(a, batch_lds, s, blocks);        \
    case kOptimistic: return adam_launch<SRC, VEC, kOptimistic, QL>(a, batch_lds, s, blocks);  \
    case kRedo: return adam_launch<SRC, VEC, kRedo, QL>(a, batch_lds, s, blocks);              \
    default: return hipErrorInvalidValue;                                                      \
  }
#define ZDP_ADAM(SRC)                                                               \
  if (src == SRC) {                                                                 \
    if (vec) { ZDP_ADAM_MODE(SRC, true, kQuadsPerThread) }                          \
    ZDP_ADAM_MODE(SRC, false, kQuadsPerThread)                                      \
  }
#define ZDP_ADAM_WIDE(SRC)                                                          \
  if (src == SRC) { ZDP_ADAM_MODE(SRC, true, kQuadsWide) }
  if (wide) {
    ZDP_ADAM_WIDE(kSrcF16)
    ZDP_ADAM_WIDE(kSrcBF16)
    return hipErrorInvalidValue;
  }
  ZDP_ADAM(kSrcAvg)
  ZDP_ADAM(kSrcF16)
  ZDP_ADAM(kSrcBF16)
#undef ZDP_ADAM_WIDE
#undef ZDP_ADAM
#undef ZDP_ADAM_MODE
  return hipErrorInvalidValue;
}

hipError_t launch_restore(const RestoreArgs& a, bool vec, hipStream_t s) {
  int grid = stream_grid(a.n);  // already within the grid limit
  if (grid > kRestoreGrid) grid = kRestoreGrid;
  if (vec)
    hipLaunchKernelGGL(restore_kernel<true>, dim3(grid), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(restore_kernel<false>, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

// The averaging pass keeps 4 quads per lane at every N_d (it has no state
// streams, and the wide read measured slower there). From kCappedReduceCopies
// to kWideCopies copies it issues every load of a tile at once with residency
// capped at kBatchBlocksPerCU blocks per CU by batch_lds bytes of otherwise
// unused LDS; above that it caps the gradient loads in flight instead; below
// it, eight copies' loads at once at full residency.
hipError_t launch_reduce(const ReduceArgs& a, int src, bool vec, size_t batch_lds, hipStream_t s, int* blocks) {
  const bool batch = reduce_batched(vec, a.src.n_d);
  const bool capped = vec && !batch && a.src.n_d >= kCappedReduceCopies;
  const size_t lds = batch ? batch_lds : 0;
  if (src == kSrcF16) {
    if (capped) return reduce_launch<kSrcF16, true, kWideInflight>(a, 0, s, blocks);
    return vec ? reduce_launch<kSrcF16, true, 0>(a, lds, s, blocks) : reduce_launch<kSrcF16, false, 0>(a, 0, s, blocks);
  }
  if (src == kSrcBF16) {
    if (capped) return reduce_launch<kSrcBF16, true, kWideInflight>(a, 0, s, blocks);
    return vec ? reduce_launch<kSrcBF16, true, 0>(a, lds, s, blocks) : reduce_launch<kSrcBF16, false, 0>(a, 0, s, blocks);
  }
  return hipErrorInvalidValue;
}

int scan_grid(int64_t n) {
  const int g = stream_grid(n);
  return g < kScanGrid ? g : kScanGrid;
}

hipError_t launch_scan(const ReduceArgs& args, int src, hipStream_t s, int* blocks) {
  const int g = scan_grid(args.n);
  const ReduceArgs a = route_partials(args, g, blocks);
  const dim3 grid(g);
  if (src == kSrcF16) hipLaunchKernelGGL(scan_kernel<kSrcF16>, grid, dim3(kBlock), 0, s, a);
  else if (src == kSrcBF16) hipLaunchKernelGGL(scan_kernel<kSrcBF16>, grid, dim3(kBlock), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fold_kernel, dim3(kFoldBlocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_redo_commit(const CommitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(redo_commit_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_state_init(zero_step_state* st, float loss_scale, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(64), 0, s, st, loss_scale);
  return hipGetLastError();
}

hipError_t launch_cast(const CastArgs& a, bool vec, hipStream_t s) {
  if (vec)
    hipLaunchKernelGGL(cast_kernel<true>, dim3(stream_grid(a.n)), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(cast_kernel<false>, dim3(stream_grid(a.n)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace zdp
