// RoPE tables: cos / sin of pos * base^(-2j/d), evaluated in double precision on
// the device and rounded to fp32 ("DFlash dual implementations: PyTorch vs MLX",
// §1: the draft reuses the Qwen3 rotary embedding; rotate-half pairs (j, j+d/2)).
// Angles reach ~3e4 rad at long context, where fp32 argument reduction would
// already be off by ~1e-3 rad; double keeps the table exact to fp32 rounding.
#include "common.h"
#include "launch.h"

namespace dflash {

namespace {
__global__ __launch_bounds__(256) void rope_tables_kernel(double base, int half, int max_pos,
                                                          float* cos_out, float* sin_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)max_pos * half) return;
  const int pos = (int)(i / half);
  const int j = (int)(i - (int64_t)pos * half);
  const double inv_freq = pow(base, -2.0 * (double)j / (double)(2 * half));
  const double th = (double)pos * inv_freq;
  double s, c;
  sincos(th, &s, &c);
  cos_out[i] = (float)c;
  sin_out[i] = (float)s;
}
}  // namespace

hipError_t launch_rope_tables(double base, int head_dim, int max_pos, float* cos_out, float* sin_out,
                              hipStream_t stream) {
  const int half = head_dim / 2;
  const int64_t n = (int64_t)max_pos * half;
  const int grid = (int)((n + 255) / 256);
  hipLaunchKernelGGL(rope_tables_kernel, dim3(grid), dim3(256), 0, stream, base, half, max_pos, cos_out,
                     sin_out);
  return hipGetLastError();
}

}  // namespace dflash
