// The rest of a draft layer around the block attention: RMSNorm, o_proj with the
// residual add, and the SwiGLU MLP with its residual add.
//
// Page "DFlash dual implementations: PyTorch vs MLX", §1 model definition: the
// draft model reuses Qwen3's RMSNorm, MLP and rotary embedding; §2: the
// attention between them.  A pre-norm residual layer over the M = 16 B block rows:
//   n1 = RMSNorm(x; w_in)                               (dflash_rmsnorm)
//   x1 = x + bf16(attn) W_o^T,  n2 = RMSNorm(x1; w_post)
//   x2 = x1 + bf16(silu(n2 W_gate^T) * (n2 W_up^T)) W_down^T
// RMSNorm(x; w) = x / sqrt(mean(x^2) + eps) * w.  Every stored tensor is bf16.
//
// gfx950 mapping: the three products are weight streams at M = 16 B rows (the
// weights, 335 MB at a Qwen3-8B-shaped layer, dominate the bytes), so they run on
// the split-K skinny MFMA GEMM of the projection; the small kernels here fold the
// split partial sums into the next step: residual add + RMSNorm in one row-wise
// pass, the SwiGLU product (inside the gate/up product itself when that takes one K
// split), the last residual add.  The RMSNorm factor is
// computed in fp64 (a row of D bf16 squares, then one rsqrt) and each output is
// rounded once from its fp64 value, so it agrees with an exact evaluation except
// within fp64 error of a bf16 rounding midpoint.
#include <math.h>

#include "common.h"
#include "launch.h"
#include "split_sum.h"

namespace dflash {

namespace {

constexpr int kRowThreads = 512;  // one workgroup per row: 8 waves (8 columns per thread per pass)

// A double moved across lanes by DPP (its two halves): a VALU move, no LDS round trip.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// v + (the same lane's value in the paired row): the row-swap permute returns the two
// values of each lane pair {l, l ^ 16} (or l ^ 32), one per result, and their sum does
// not depend on which is which.
__device__ __forceinline__ double add_pair(uint32_t lo0, uint32_t hi0, uint32_t lo1, uint32_t hi1) {
  return __longlong_as_double((long long)(((uint64_t)hi0 << 32) | lo0)) +
         __longlong_as_double((long long)(((uint64_t)hi1 << 32) | lo1));
}
__device__ __forceinline__ double sum_rows16(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  return add_pair(lo[0], hi[0], lo[1], hi[1]);
}
__device__ __forceinline__ double sum_rows32(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  return add_pair(lo[0], hi[0], lo[1], hi[1]);
}

// Sum over the workgroup in a fixed order: a balanced tree inside each wave (pairs, then
// quads, then the four quads of a 16-lane row, then rows 0 + 1 and 2 + 3, then the two
// halves), whose result lane 0 holds, then the wave totals in wave order.
__device__ __forceinline__ double block_sum(double v, double* red) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x124>(v);  // row_ror 4
  v += dpp_f64<0x128>(v);  // row_ror 8
  v = sum_rows16(v);
  v = sum_rows32(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red[] free (an earlier call's readers are done)
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int i = 1; i < kRowThreads / 64; ++i) t += red[i];
  return t;
}

__device__ __forceinline__ uint16_t bf16_of_f64(double v) { return bf16_of_exact_sum(v, 0.0); }

// 8 bf16 of a 16-byte load as doubles.
__device__ __forceinline__ void unpack8(const u32x4 v, double* o) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = (double)bf16_lo(v[e]);
    o[2 * e + 1] = (double)bf16_hi(v[e]);
  }
}

// n = bf16(x * r * w) for the 8 columns c..c+7 of one row (x as doubles).
__device__ __forceinline__ u32x4 norm8(const double* x, double r, const uint16_t* w, int c) {
  double wv[8];
  unpack8(ld16(w + c), wv);
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = (uint32_t)bf16_of_f64(x[2 * e] * r * wv[2 * e]) |
           ((uint32_t)bf16_of_f64(x[2 * e + 1] * r * wv[2 * e + 1]) << 16);
  return o;
}

// RMSNorm of bf16 rows: one workgroup per row, two passes over the row (the second
// is served by the cache).  cols % 8 == 0.
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(RmsNormParams p) {
  __shared__ double red[kRowThreads / 64];
  const int m = blockIdx.x;
  const uint16_t* xr = p.x + (int64_t)m * p.ld_x;
  double ss = 0.0;
  for (int c = threadIdx.x * 8; c < p.cols; c += kRowThreads * 8) {
    double x[8];
    unpack8(ld16(xr + c), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  }
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / p.cols + (double)p.eps);
  uint16_t* orow = p.out + (int64_t)m * p.ld_out;
  for (int c = threadIdx.x * 8; c < p.cols; c += kRowThreads * 8) {
    double x[8];
    unpack8(ld16(xr + c), x);
    st16(orow + c, norm8(x, r, p.w, c));
  }
}


// x1 = bf16(x + sum of the o_proj partials), then n2 = RMSNorm(x1; w_post): one
// workgroup per row.  The row's x1 chunks stay in registers between the passes
// (cols <= kRowThreads * 8 * kMaxChunks).
constexpr int kMaxChunks = 4;  // hidden <= 16384
__global__ __launch_bounds__(kRowThreads) void residual_norm_kernel(LayerPostParams p) {
  __shared__ double red[kRowThreads / 64];
  const int m = blockIdx.x;
  const int D = p.hidden;
  const int64_t zs = (int64_t)p.M * D;
  double x1[kMaxChunks][8];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    const int c = (k * kRowThreads + threadIdx.x) * 8;
    if (c >= D) break;
    double xr[8];
    unpack8(ld16(p.x + (int64_t)m * D + c), xr);
    const f32x4 s0 = sum_splits(p.part_o + (int64_t)m * D + c, zs, p.splits_o);
    const f32x4 s1 = sum_splits(p.part_o + (int64_t)m * D + c + 4, zs, p.splits_o);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t b = bf16_of_exact_sum(xr[e], (double)(e < 4 ? s0[e] : s1[e - 4]));
      x1[k][e] = (double)bf16_to_f32(b);
      ss += x1[k][e] * x1[k][e];
      if (e & 1) o[e >> 1] |= (uint32_t)b << 16;
      else o[e >> 1] = b;
    }
    st16(p.x1 + (int64_t)m * D + c, o);
  }
  ss = block_sum(ss, red);
  const double r = 1.0 / sqrt(ss / D + (double)p.eps);
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    const int c = (k * kRowThreads + threadIdx.x) * 8;
    if (c >= D) break;
    st16(p.n2 + (int64_t)m * D + c, norm8(x1[k], r, p.w_post, c));
  }
}

// act = bf16(silu(g) * u) from the gate / up partials (columns j and I + j of the
// [M][2I] product): 4 columns per thread.
__global__ __launch_bounds__(256) void swiglu_kernel(LayerPostParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index into [M][I]
  const int I = p.inter;
  if (i >= (int64_t)p.M * I / 4) return;
  const int64_t m = 4 * i / I;
  const int j = (int)(4 * i - m * I);
  const int64_t zs = (int64_t)p.M * 2 * I;
  const f32x4 g = sum_splits(p.part_gu + m * 2 * I + j, zs, p.splits_gu);
  const f32x4 u = sum_splits(p.part_gu + m * 2 * I + I + j, zs, p.splits_gu);
  float a[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = g[e] / (1.f + expf(-g[e])) * u[e];
  *reinterpret_cast<u32x2*>(p.act + m * I + j) = (u32x2){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
}

// x2 = bf16(x1 + sum of the down partials): 4 columns per thread.
__global__ __launch_bounds__(256) void residual_add_kernel(LayerPostParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int D = p.hidden;
  if (i >= (int64_t)p.M * D / 4) return;
  const f32x4 s = sum_splits(p.part_d + 4 * i, (int64_t)p.M * D, p.splits_d);
  const u32x2 x = *reinterpret_cast<const u32x2*>(p.x1 + 4 * i);
  const float v0 = bf16_lo(x[0]) + s[0], v1 = bf16_hi(x[0]) + s[1];
  const float v2 = bf16_lo(x[1]) + s[2], v3 = bf16_hi(x[1]) + s[3];
  *reinterpret_cast<u32x2*>(p.x_out + 4 * i) = (u32x2){pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

// The attention's fp32 output as bf16 rows (the o_proj's A operand): [B][16][Hq][d]
// is already row m = 16 b + i, column h d + j.  8 values per thread.
__global__ __launch_bounds__(256) void attn_to_bf16_kernel(LayerPostParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.M * p.attn_cols / 8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p.attn + 8 * i);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p.attn + 8 * i + 4);
  st16(p.a_bf16 + 8 * i, (u32x4){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                 pack_bf16x2(b[2], b[3])});
}

unsigned blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

LayerPlan plan_draft_layer_post(int rows, int hidden, int attn_cols, int inter, int num_cu) {
  LayerPlan pl{};
  pl.o = plan_block_qkv(rows, attn_cols, hidden, num_cu);
  pl.gu = plan_block_qkv(rows, hidden, 2 * inter, num_cu);
  pl.dn = plan_block_qkv(rows, inter, hidden, num_cu);
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // word 0: device error mask (unused here, kept for the common layout)
  pl.off_a = off;
  off = align(off + 2 * (size_t)rows * attn_cols);
  pl.off_po = off;
  off = align(off + sizeof(float) * (size_t)pl.o.splits * rows * hidden);
  pl.off_x1 = off;
  off = align(off + 2 * (size_t)rows * hidden);
  pl.off_n2 = off;
  off = align(off + 2 * (size_t)rows * hidden);
  pl.off_pgu = off;
  off = align(off + sizeof(float) * (size_t)pl.gu.splits * rows * 2 * inter);
  pl.off_act = off;
  off = align(off + 2 * (size_t)rows * inter);
  pl.off_pd = off;
  off = align(off + sizeof(float) * (size_t)pl.dn.splits * rows * hidden);
  pl.ws_bytes = off;
  return pl;
}

hipError_t launch_rmsnorm(const RmsNormParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(p.rows), dim3(kRowThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_draft_layer_post(const LayerPostParams& p, const LayerPlan& pl, hipStream_t stream) {
  const int64_t M = p.M;
  hipLaunchKernelGGL(attn_to_bf16_kernel, dim3(blocks(M * p.attn_cols / 8, 256)), dim3(256), 0, stream, p);
  GemmParams g{};
  g.a_seg[0] = p.a_bf16;
  g.lda = p.attn_cols;
  g.seg_k = p.attn_cols;
  g.b0 = g.b1 = p.w_o;
  g.n_b0 = p.hidden;
  g.M = p.M;
  g.N = p.hidden;
  g.K = p.attn_cols;
  g.k_per_split = pl.o.kps;
  g.out = p.part_o;
  hipError_t e = launch_gemm_nt(g, pl.o.splits, pl.o.small, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(residual_norm_kernel, dim3(p.M), dim3(kRowThreads), 0, stream, p);
  g = GemmParams{};
  g.a_seg[0] = p.n2;
  g.lda = p.hidden;
  g.seg_k = p.hidden;
  g.b0 = p.w_gate;
  g.b1 = p.w_up;
  g.n_b0 = p.inter;
  g.M = p.M;
  g.N = 2 * p.inter;
  g.K = p.hidden;
  g.k_per_split = pl.gu.kps;
  g.out = p.part_gu;
  if (pl.gu.small && pl.gu.splits == 1) {
    // One split: the product holds whole results, so it applies the SwiGLU itself
    // (no fp32 partials of [M][2I], no separate kernel).
    g.act = p.act;
    e = launch_gemm_swiglu(g, stream);
    if (e != hipSuccess) return e;
  } else {
    e = launch_gemm_nt(g, pl.gu.splits, pl.gu.small, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(swiglu_kernel, dim3(blocks(M * p.inter / 4, 256)), dim3(256), 0, stream, p);
  }
  g = GemmParams{};
  g.a_seg[0] = p.act;
  g.lda = p.inter;
  g.seg_k = p.inter;
  g.b0 = g.b1 = p.w_down;
  g.n_b0 = p.hidden;
  g.M = p.M;
  g.N = p.hidden;
  g.K = p.inter;
  g.k_per_split = pl.dn.kps;
  g.out = p.part_d;
  e = launch_gemm_nt(g, pl.dn.splits, pl.dn.small, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(residual_add_kernel, dim3(blocks(M * p.hidden / 4, 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dflash
