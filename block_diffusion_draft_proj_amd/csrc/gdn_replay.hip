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
// small).  One workgroup per (sequence, head, 16 or 32 state rows).  Every load is
// issued before the first wait, so the workgroup costs one memory round trip: first the
// tape (the accepted steps' keys in 8-byte pieces, this workgroup's innovations, the
// decays), then all float4 chunks of the state, streamed past the caches.  The tape goes
// to LDS (as fp32) while the state is still in flight -- waiting for the tape loads does
// not wait for the younger state loads -- and the steps are replayed on the chunks in
// registers, which are streamed back.  All loads are unconditional (indices clamped into
// their buffers; the extra values are never used), so the compiler's wait before the
// first use of the tape counts exactly the younger state loads.
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
  constexpr int kMaxChunksPerThread = ROWS * (kMaxDk / 4) / kReplayThreads;
  constexpr int kKeyPieces = kBlock * kMaxDk / 4 / kReplayThreads;  // 8-byte key pieces per thread
  constexpr int kDeltas = kBlock * ROWS / kReplayThreads;            // innovations per thread
  __shared__ float s_k[kBlock][kMaxDk];
  __shared__ float s_d[kBlock][ROWS];
  __shared__ float s_alpha[kBlock];
  const int parts = (p.dv + ROWS - 1) / ROWS;
  const int unit = blockIdx.x / parts, part = blockIdx.x - unit * parts;
  const int b = unit / p.n_heads, h = unit - b * p.n_heads;
  const int tid = threadIdx.x;
  int a = p.accept_len[b];
  if (a < 0 || a > kBlock - 1) {
    if (tid == 0 && part == 0 && h == 0 && p.err) set_dev_error(p.err, kDevErrAccept);
    a = a < 0 ? 0 : kBlock - 1;
  }
  const int n = a + 1;  // committed steps: the staged token and the accepted drafts
  const int row0 = part * ROWS;
  const int64_t step0 = (int64_t)b * kBlock * p.n_heads + h;  // (b, t = 0, h); step t adds t * n_heads

  // The tape: keys, innovations of rows row0.., decays.
  const int kq = p.dk / 4, nk = n * kq;  // 8-byte pieces per step (d_k % 4 == 0), in all
  u32x2 kr[kKeyPieces];
#pragma unroll
  for (int u = 0; u < kKeyPieces; ++u) {
    const int i = min(tid + u * kReplayThreads, nk - 1);
    const int t = i / kq, j = (i - t * kq) * 4;
    kr[u] = *reinterpret_cast<const u32x2*>(p.k_tape + (step0 + (int64_t)t * p.n_heads) * p.dk + j);
  }
  float dr[kDeltas];
#pragma unroll
  for (int u = 0; u < kDeltas; ++u) {
    const int i = tid + u * kReplayThreads;
    const int t = min(i / ROWS, n - 1), row = min(row0 + i % ROWS, p.dv - 1);
    dr[u] = p.delta_tape[(step0 + (int64_t)t * p.n_heads) * p.dv + row];
  }
  const float gr = p.g_tape[step0 + (int64_t)min(tid, n - 1) * p.n_heads];

  // The state: every float4 chunk of rows row0 .. row0 + ROWS - 1.
  const int cpr = p.dk / 4;  // float4 chunks per state row
  const int rows = min(ROWS, p.dv - row0);
  const int n_chunks = rows * cpr;
  const int64_t base = ((int64_t)unit * p.dv + row0) * p.dk;
  f32x4 sv[kMaxChunksPerThread];
#pragma unroll
  for (int u = 0; u < kMaxChunksPerThread; ++u) {
    const int c = min(tid + u * kReplayThreads, n_chunks - 1);
    sv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.state_in + base + (int64_t)c * 4));
  }

  // Stage the tape in LDS while the state loads are in flight.  The stores are as
  // unconditional as the loads (a guarded store would let the compiler sink its load
  // past the state loads): lanes past the end rewrite the last piece with the same value.
#pragma unroll
  for (int u = 0; u < kKeyPieces; ++u) {
    const int i = min(tid + u * kReplayThreads, nk - 1);
    const int t = i / kq, j = (i - t * kq) * 4;
    *reinterpret_cast<f32x4*>(&s_k[t][j]) =
        (f32x4){__uint_as_float(kr[u][0] << 16), __uint_as_float(kr[u][0] & 0xffff0000u),
                __uint_as_float(kr[u][1] << 16), __uint_as_float(kr[u][1] & 0xffff0000u)};
  }
#pragma unroll
  for (int u = 0; u < kDeltas; ++u) {
    const int i = tid + u * kReplayThreads;
    const int t = min(i / ROWS, n - 1), r = i % ROWS;
    s_d[t][r] = row0 + r < p.dv ? dr[u] : 0.f;
  }
  s_alpha[min(tid, n - 1)] = expf(gr);
  lds_barrier();  // LDS only: the state loads stay in flight

#pragma unroll
  for (int u = 0; u < kMaxChunksPerThread; ++u) {
    const int c = tid + u * kReplayThreads;
    if (c >= n_chunks) break;
    const int r = c / cpr, j = (c - r * cpr) * 4;
    f32x4 v = sv[u];
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
