// Rollback of recurrent (GatedDeltaNet) state after a verify: replay of the
// accepted steps of an innovation tape onto the state saved before the block.
//
// Page "dflash-mlx: lossless speculative decoding", guarantee 3: verifying the
// block advances the recurrent state by all 16 candidate steps and, unlike an
// attention cache, it cannot be cropped; during the verify a tape of per-step
// k, g and increments is recorded and, once the accept length is known, only
// the accepted steps are replayed onto the saved state.  Page "DFlash dual
// implementations", §7: the state is rolled back along the accepted prefix.
// With the gated delta rule (per head, state S [d_v][d_k]; alpha = exp(g);
// innovation delta_t = beta_t (v_t - alpha_t S_{t-1} k_t) recorded on the tape),
//   S_t = alpha_t S_{t-1} + delta_t k_t^T,      t = 0 .. accept_len,
// so each state element is replayed on its own: no S k product, no reduction.
//
// gfx950 mapping: HBM-bound (the fp32 state is read and written once; the tape is
// small).  One workgroup per (sequence, head, 16 or 32 state rows): every thread
// first issues the loads of all its float4 chunks of the state (streamed past the
// caches, all in flight at once), then the accepted steps' keys (as fp32),
// innovations and decays go to LDS while those loads are outstanding; the steps
// are replayed on the chunks in registers and the chunks are streamed back.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dflash {

namespace {

constexpr int kReplayThreads = 256;
constexpr int kMaxDk = 256;

// ROWS state rows (value dims) per workgroup: 32, or 16 where 32 would give fewer
// than 8 workgroups per CU (a short grid then finishes sooner with twice the
// workgroups; with a full grid the larger share per workgroup is faster).
template <int ROWS>
__global__ __launch_bounds__(kReplayThreads) void gdn_replay_kernel(GdnReplayParams p) {
  constexpr int kReplayRows = ROWS;
  constexpr int kMaxChunksPerThread = kReplayRows * (kMaxDk / 4) / kReplayThreads;
  __shared__ float s_k[kBlock][kMaxDk];
  __shared__ float s_d[kBlock][kReplayRows];
  __shared__ float s_alpha[kBlock];
  const int parts = (p.dv + kReplayRows - 1) / kReplayRows;
  const int unit = blockIdx.x / parts, part = blockIdx.x - unit * parts;
  const int b = unit / p.n_heads, h = unit - b * p.n_heads;
  const int tid = threadIdx.x;
  int a = p.accept_len[b];
  if (a < 0 || a > kBlock - 1) {
    if (tid == 0 && part == 0 && h == 0 && p.err) set_dev_error(p.err, kDevErrAccept);
    a = a < 0 ? 0 : kBlock - 1;
  }
  const int n = a + 1;  // committed steps: the staged token and the accepted drafts
  const int row0 = part * kReplayRows;
  // The state loads go first (they do not depend on the tape), so their latency
  // overlaps the tape's staging in LDS.
  const int cpr = p.dk / 4;                       // float4 chunks per state row
  const int rows = min(kReplayRows, p.dv - row0);
  const int n_chunks = rows * cpr;
  const int64_t base = ((int64_t)unit * p.dv + row0) * p.dk;
  f32x4 s[kMaxChunksPerThread];
#pragma unroll
  for (int u = 0; u < kMaxChunksPerThread; ++u) {
    const int c = tid + u * kReplayThreads;
    if (c < n_chunks) s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.state_in + base + (int64_t)c * 4));
  }
  for (int i = tid; i < n * p.dk; i += kReplayThreads) {
    const int t = i / p.dk, j = i - t * p.dk;
    s_k[t][j] = bf16_to_f32(p.k_tape[(((int64_t)b * kBlock + t) * p.n_heads + h) * p.dk + j]);
  }
  for (int i = tid; i < n * kReplayRows; i += kReplayThreads) {
    const int t = i / kReplayRows, r = i - t * kReplayRows;
    const int row = row0 + r;
    s_d[t][r] = row < p.dv ? p.delta_tape[(((int64_t)b * kBlock + t) * p.n_heads + h) * p.dv + row] : 0.f;
  }
  if (tid < n) s_alpha[tid] = expf(p.g_tape[((int64_t)b * kBlock + tid) * p.n_heads + h]);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kMaxChunksPerThread; ++u) {
    const int c = tid + u * kReplayThreads;
    if (c >= n_chunks) break;
    const int r = c / cpr, j = (c - r * cpr) * 4;
    f32x4 v = s[u];
    for (int t = 0; t < n; ++t) {
      const float al = s_alpha[t], d = s_d[t][r];
      const f32x4 k = *reinterpret_cast<const f32x4*>(&s_k[t][j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = v[e] * al + d * k[e];
    }
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p.state_out + base + (int64_t)c * 4));
  }
}

}  // namespace

hipError_t launch_gdn_replay(const GdnReplayParams& p, hipStream_t stream) {
  const int64_t units = (int64_t)p.batch * p.n_heads;
  if (units * ((p.dv + 31) / 32) < 2048) {
    const int64_t grid = units * ((p.dv + 15) / 16);
    hipLaunchKernelGGL(gdn_replay_kernel<16>, dim3((unsigned)grid), dim3(kReplayThreads), 0, stream, p);
  } else {
    const int64_t grid = units * ((p.dv + 31) / 32);
    hipLaunchKernelGGL(gdn_replay_kernel<32>, dim3((unsigned)grid), dim3(kReplayThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dflash
