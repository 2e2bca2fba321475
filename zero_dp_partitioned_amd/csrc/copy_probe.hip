// A two-stream device copy with the update kernel's access shape, for
// measuring the HBM bandwidth a kernel that reads and writes half its bytes
// each reaches on a given placement (zero_copy_probe). Not part of the step.
//
// One 256-thread block per 16 KiB tile of each stream; lane l moves the
// 16-byte words l, l + 256, l + 512, l + 768 of the tile, so every wavefront
// load or store is one contiguous 1 KiB run; loads and stores carry the
// non-temporal hint, as in the update kernel. Launches beyond the grid cap
// loop over tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_dp_internal.h"

namespace zdp {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWordsPerLane = 4;
constexpr int64_t kTileWords = static_cast<int64_t>(kBlock) * kWordsPerLane;  // 16 KiB

__global__ void __launch_bounds__(kBlock) copy2_kernel(const f4* a, const f4* b, f4* c, f4* d, int64_t words) {
  const int64_t tiles = (words + kTileWords - 1) / kTileWords;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t base = t * kTileWords + threadIdx.x;
    if (base + (kWordsPerLane - 1) * kBlock < words) {
      f4 x[kWordsPerLane], y[kWordsPerLane];
#pragma unroll
      for (int k = 0; k < kWordsPerLane; ++k) {
        x[k] = __builtin_nontemporal_load(a + base + k * kBlock);
        y[k] = __builtin_nontemporal_load(b + base + k * kBlock);
      }
#pragma unroll
      for (int k = 0; k < kWordsPerLane; ++k) {
        __builtin_nontemporal_store(x[k], c + base + k * kBlock);
        __builtin_nontemporal_store(y[k], d + base + k * kBlock);
      }
    } else {
      for (int k = 0; k < kWordsPerLane; ++k) {
        const int64_t w = base + k * kBlock;
        if (w < words) {
          c[w] = a[w];
          d[w] = b[w];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_probe(const void* src0, const void* src1, void* dst0, void* dst1, int64_t words,
                             hipStream_t s) {
  int64_t tiles = (words + kTileWords - 1) / kTileWords;
  if (tiles < 1) tiles = 1;
  const int grid = limit_grid(static_cast<int>(tiles < kMaxGrid ? tiles : kMaxGrid));
  hipLaunchKernelGGL(copy2_kernel, dim3(grid), dim3(kBlock), 0, s, static_cast<const f4*>(src0),
                     static_cast<const f4*>(src1), static_cast<f4*>(dst0), static_cast<f4*>(dst1), words);
  return hipGetLastError();
}

}  // namespace zdp
