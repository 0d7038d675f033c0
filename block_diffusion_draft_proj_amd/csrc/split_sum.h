// Reduction of split-K partial sums, shared by the projection and draft-layer
// epilogue kernels.
#pragma once

#include "common.h"

namespace dflash {

// Sum of the split partials at one float4 position, in split order.  The loads of
// up to kSumBatch splits are all issued before the first add (the address of a
// split past the last is clamped and its value dropped), so a reduce over 8 splits
// costs one memory round trip instead of eight.
constexpr int kSumBatch = 8;
__device__ __forceinline__ f32x4 sum_splits(const float* base, int64_t stride, int splits) {
  f32x4 s = *reinterpret_cast<const f32x4*>(base);
  for (int z0 = 1; z0 < splits; z0 += kSumBatch) {
    f32x4 v[kSumBatch];
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(base + (int64_t)min(z0 + u, splits - 1) * stride);
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u)
      if (z0 + u < splits) s += v[u];
  }
  return s;
}

}  // namespace dflash
