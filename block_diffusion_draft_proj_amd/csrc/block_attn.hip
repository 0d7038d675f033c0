// Dual-source, non-causal GQA block attention of the DFlash draft.
//
// Page "DFlash dual implementations: PyTorch vs MLX", §2 attention: K/V are the
// concatenation of the context (projected target hidden states) and the block
// tokens, Q comes from the block tokens only, and attention inside the block is
// non-causal; §1: RoPE is the Qwen3 rotary embedding.  For one (sequence b,
// kv head g) "unit" the G query heads of the group each contribute 16 block
// rows, all of which see all L context keys and all 16 block keys.
//
// Mapping onto gfx950:
//  * workgroup = one (unit, split of the context) with G waves, wave w = query
//    head g*G+w and its 16 block rows; the K/V tile is staged once in LDS and
//    shared by the G heads (the context K/V stream is the HBM-bound part);
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: keys are the
//    MFMA row dimension, so the score tile comes out with one query row per lane
//    column, the online-softmax statistics stay per lane, and the score
//    registers are already the B operand of the PV product (the key order of the
//    two 16-key score tiles is interleaved so each lane owns 8 consecutive keys);
//  * V is transposed on its way into LDS (4 keys x 8 dims per thread through
//    byte permutes) so the V^T operand is one 16-byte LDS read per lane;
//  * K and V^T tiles use XOR-swizzled 16-byte chunks: every 16-lane read group
//    and every row-wide write touches distinct banks;
//  * the context is split over workgroups (flash-decoding); each split keeps
//    (max, sum, O) in the workspace and a small second kernel merges them
//    (log-sum-exp).  The kernel boundary is the handoff: merging inside the
//    kernel would cost an L2 writeback (agent-scope release) per workgroup,
//    measured at several times the merge itself.  All splits of a unit sit on
//    one XCD, so their partials are written and re-read through one L2;
//  * probabilities enter the PV product as a bf16 hi/lo pair (P = P_hi + P_lo),
//    so the only rounding of operands is the bf16 storage of Q, K and V.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dflash {

namespace {

constexpr int TK = 64;  // keys per tile

template <int D>
__device__ __forceinline__ int k_swz(int t) {
  if constexpr (D == 128) return (t & 3) | (((t >> 3) & 3) << 2);
  else return ((t >> 1) & 1) | (((t >> 3) & 3) << 1);
}
// K tile: row t = one key (D bf16); 16-byte chunk c of row t lives at chunk c ^ k_swz(t).
template <int D>
__device__ __forceinline__ int k_off(int t, int c) { return t * (D * 2) + ((c ^ k_swz<D>(t)) << 4); }
// V^T tile: row d = one head dimension (TK keys = 128 bytes); 8-key chunk lc at lc ^ ((d>>1)&7).
__device__ __forceinline__ int v_off(int d, int lc) { return d * (TK * 2) + ((lc ^ ((d >> 1) & 7)) << 4); }

template <bool PAGED>
__device__ __forceinline__ const uint16_t* key_row(const AttnParams& p, const uint16_t* cache, int b, int g,
                                                   int t, int D) {
  if constexpr (PAGED) {
    int page = p.page_table[(int64_t)b * p.capacity + (t >> 4)];
    if ((unsigned)page >= (unsigned)p.num_pages) {
      set_dev_error(p.err, 1u << 1);
      page = 0;
    }
    return cache + (((int64_t)page * p.n_kv_heads + g) * 16 + (t & 15)) * D;
  } else {
    return cache + (((int64_t)b * p.n_kv_heads + g) * p.capacity + t) * D;
  }
}

template <int D, int NT, bool PAGED>
struct TileRegs {
  static constexpr int NCH = D / 8;
  static constexpr int KCH = TK * NCH;
  static constexpr int KPER = (KCH + NT - 1) / NT;
  static constexpr int VIT = (TK / 4) * NCH;
  static constexpr int VPER = (VIT + NT - 1) / NT;
  u32x4 kr[KPER];
  u32x4 vr[VPER][4];

  // Context keys [t0, t0+TK) of unit (b, g); keys >= tend become zero rows.
  __device__ __forceinline__ void load(const AttnParams& p, int b, int g, int t0, int tend, int tid) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int cid = tid + NT * i;
      const int t = t0 + cid / NCH;
      kr[i] = z;
      if ((KCH % NT == 0 || cid < KCH) && t < tend)
        kr[i] = ld16(key_row<PAGED>(p, p.k_cache, b, g, t, D) + (cid % NCH) * 8);
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int id = tid + NT * i;
      const int t = t0 + (id / NCH) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) vr[i][k] = z;
      if ((VIT % NT == 0 || id < VIT) && t < tend) {
        // 4 consecutive keys never cross a 16-token page.
        const uint16_t* src = key_row<PAGED>(p, p.v_cache, b, g, t, D) + (id % NCH) * 8;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (t + k < tend) vr[i][k] = ld16(src + k * D);
      }
    }
  }

  __device__ __forceinline__ void store(char* lds_k, char* lds_v, int tid) const {
#pragma unroll
    for (int i = 0; i < KPER; ++i) {
      const int cid = tid + NT * i;
      if (KCH % NT == 0 || cid < KCH)
        *reinterpret_cast<u32x4*>(lds_k + k_off<D>(cid / NCH, cid % NCH)) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VPER; ++i) {
      const int id = tid + NT * i;
      if (VIT % NT == 0 || id < VIT) {
        const int dc = id % NCH, kq = id / NCH;
        const int half = (kq & 1) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x0 = vr[i][0][j], x1 = vr[i][1][j], x2 = vr[i][2][j], x3 = vr[i][3][j];
          const int d = dc * 8 + 2 * j;
          *reinterpret_cast<u32x2*>(lds_v + v_off(d, kq >> 1) + half) =
              (u32x2){pack_lo16(x0, x1), pack_lo16(x2, x3)};
          *reinterpret_cast<u32x2*>(lds_v + v_off(d + 1, kq >> 1) + half) =
              (u32x2){pack_hi16(x0, x1), pack_hi16(x2, x3)};
        }
      }
    }
  }
};

// One wave: 16 block rows of one query head against the TK-key tile in LDS.
// nvalid: keys [0, nvalid) of the tile are real, the rest are masked out.
template <int D, bool PLO>
__device__ __forceinline__ void attend_tile(const char* lds_k, const char* lds_v, const bf16x8* qB, f32x4* o,
                                            float& m, float& lsum, int lane, int nvalid, float scale_log2) {
  constexpr int KS = D / 32, DT = D / 16;
  const int r = lane & 15, q = lane >> 4;
  const int nkk = nvalid > 32 ? 2 : 1;
  float x[2][2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (kk < nkk) {
        const int t = 32 * kk + 8 * (r >> 2) + 4 * j + (r & 3);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + k_off<D>(t, ks * 4 + q));
          acc = mfma16x16x32(a, qB[ks], acc);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) x[kk][j][v] = acc[v] * scale_log2;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) x[kk][j][v] = -INFINITY;
      }
    }
  }
  if (nvalid < TK) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (32 * kk + 8 * q + 4 * j + v >= nvalid) x[kk][j][v] = -INFINITY;
  }
  float mt = x[0][0][0];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) mt = fmaxf(mt, x[kk][j][v]);
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float mnew = fmaxf(m, mt);
  const float mref = (mnew == -INFINITY) ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(m - mref);
  float psum = 0.f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = __builtin_amdgcn_exp2f(x[kk][j][v] - mref);
        x[kk][j][v] = e;
        psum += e;
      }
  lsum = lsum * alpha + psum;
  m = mnew;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

  bf16x8 ph[2], pl[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const __bf16 hi = static_cast<__bf16>(x[kk][j][v]);
        ph[kk][4 * j + v] = hi;
        if constexpr (PLO) pl[kk][4 * j + v] = static_cast<__bf16>(x[kk][j][v] - static_cast<float>(hi));
      }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (kk < nkk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_v + v_off(dt * 16 + r, 4 * kk + q));
        o[dt] = mfma16x16x32(a, ph[kk], o[dt]);
        if constexpr (PLO) o[dt] = mfma16x16x32(a, pl[kk], o[dt]);
      }
    }
  }
}

template <int D, int G, bool PAGED, bool PLO>
__global__ __launch_bounds__(64 * G) void block_attn_kernel(AttnParams p) {
  constexpr int NT = 64 * G;
  constexpr int KS = D / 32, DT = D / 16, HALF = D / 2;
  __shared__ __attribute__((aligned(16))) char lds_k[TK * D * 2];
  __shared__ __attribute__((aligned(16))) char lds_v[D * TK * 2];

  // XCD-aware decode: WG i runs on XCD i % 8; every split of a unit shares one XCD.
  const int i_wg = blockIdx.x;
  const int xcd = i_wg % kNumXcd;
  const int jj = i_wg / kNumXcd;
  const int s = jj % p.n_splits;
  const int u = (jj / p.n_splits) * kNumXcd + xcd;
  if (u >= p.n_units) return;
  const int b = u / p.n_kv_heads, g = u - b * p.n_kv_heads;

  int L = p.ctx_len[b];
  if (L < 0 || L > p.max_ctx) {
    if (threadIdx.x == 0 && s == 0) set_dev_error(p.err, 1u);
    L = L < 0 ? 0 : p.max_ctx;
  }
  const int ns = L > 0 ? (L + p.kps - 1) / p.kps : 1;
  if (s >= ns) return;
  const int kb = s * p.kps;
  const int ke = min(L, kb + p.kps);
  const bool last_split = (s == ns - 1);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int h = g * G + w;

  // Q of head h: rows at positions L + r, RoPE in fp32, rounded to bf16, as the
  // B operand of S^T = K Q^T (lane holds dims 32*ks + 8*q .. +8 of row r).
  bf16x8 qB[KS];
  {
    const uint16_t* qrow = p.q_blk + (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D;
    u32x4 raw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = ld16(qrow + 32 * ks + 8 * q);
    const float* cr = p.rope_cos + (int64_t)(L + r) * HALF;
    const float* sr = p.rope_sin + (int64_t)(L + r) * HALF;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
      const int j0 = 32 * ks + 8 * q;
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cr + j0), c1 = *reinterpret_cast<const f32x4*>(cr + j0 + 4);
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(sr + j0), s1 = *reinterpret_cast<const f32x4*>(sr + j0 + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wl = raw[ks][e >> 1], wh = raw[ks + KS / 2][e >> 1];
        const float lo = (e & 1) ? bf16_hi(wl) : bf16_lo(wl);
        const float hi = (e & 1) ? bf16_hi(wh) : bf16_lo(wh);
        const float c = e < 4 ? c0[e] : c1[e - 4];
        const float sn = e < 4 ? s0[e] : s1[e - 4];
        float ylo, yhi;
        rope_pair(lo, hi, c, sn, ylo, yhi);
        qB[ks][e] = static_cast<__bf16>(ylo);
        qB[ks + KS / 2][e] = static_cast<__bf16>(yhi);
      }
    }
  }

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // Context keys [kb, ke): register-prefetched tiles through LDS.
  const int n_tiles = (ke - kb + TK - 1) / TK;
  TileRegs<D, NT, PAGED> regs;
  if (n_tiles > 0) regs.load(p, b, g, kb, ke, tid);
  for (int it = 0; it < n_tiles; ++it) {
    const int t0 = kb + it * TK;
    if (it > 0) __syncthreads();
    regs.store(lds_k, lds_v, tid);
    __syncthreads();
    if (it + 1 < n_tiles) regs.load(p, b, g, t0 + TK, ke, tid);
    attend_tile<D, PLO>(lds_k, lds_v, qB, o, m, lsum, lane, min(TK, ke - t0), p.scale_log2);
  }

  // Block keys (positions L .. L+15), handled by the last split of the unit.
  if (last_split) {
    __syncthreads();
    for (int off = tid * 16; off < TK * D * 2; off += NT * 16) {
      *reinterpret_cast<u32x4*>(lds_k + off) = (u32x4){0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(lds_v + off) = (u32x4){0u, 0u, 0u, 0u};
    }
    __syncthreads();
    for (int id = tid; id < kBlock * HALF; id += NT) {
      const int t = id / HALF, j = id - t * HALF;
      const int64_t rowoff = (((int64_t)b * kBlock + t) * p.n_kv_heads + g) * D;
      const uint16_t* kr = p.k_blk + rowoff;
      const uint16_t* vr = p.v_blk + rowoff;
      const float c = p.rope_cos[(int64_t)(L + t) * HALF + j];
      const float sn = p.rope_sin[(int64_t)(L + t) * HALF + j];
      float y0, y1;
      rope_pair(bf16_to_f32(kr[j]), bf16_to_f32(kr[j + HALF]), c, sn, y0, y1);
      *reinterpret_cast<uint16_t*>(lds_k + k_off<D>(t, j >> 3) + 2 * (j & 7)) = f32_to_bf16(y0);
      *reinterpret_cast<uint16_t*>(lds_k + k_off<D>(t, (j + HALF) >> 3) + 2 * (j & 7)) = f32_to_bf16(y1);
      *reinterpret_cast<uint16_t*>(lds_v + v_off(j, t >> 3) + 2 * (t & 7)) = vr[j];
      *reinterpret_cast<uint16_t*>(lds_v + v_off(j + HALF, t >> 3) + 2 * (t & 7)) = vr[j + HALF];
    }
    __syncthreads();
    attend_tile<D, PLO>(lds_k, lds_v, qB, o, m, lsum, lane, kBlock, p.scale_log2);
  }

  float lt = lsum + __shfl_xor(lsum, 16);
  lt += __shfl_xor(lt, 32);

  float* outp = p.out + (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D + 4 * q;
  if (ns == 1) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(outp + dt * 16) = o[dt] * inv;
    return;
  }

  // Split partials; attn_merge_kernel combines them after this kernel.
  const int64_t slot = ((int64_t)u * p.n_splits + s) * G + w;
  float* po = p.ws_o + slot * (DT * 256);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(po + (dt * 64 + lane) * 4) = o[dt];
  if (q == 0) {
    p.ws_ml[(slot * 16 + r) * 2 + 0] = m;
    p.ws_ml[(slot * 16 + r) * 2 + 1] = lt;
  }
}

// Log-sum-exp merge of the split partials of one unit: wave w = query head
// g*G + w, lane = (row r, dims 4q..4q+3 of every 16-dim tile).
template <int D, int G>
__global__ __launch_bounds__(64 * G) void attn_merge_kernel(AttnParams p) {
  constexpr int DT = D / 16;
  const int u = blockIdx.x;
  const int b = u / p.n_kv_heads, g = u - b * p.n_kv_heads;
  int L = p.ctx_len[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int ns = L > 0 ? (L + p.kps - 1) / p.kps : 1;
  if (ns == 1) return;  // written directly by the split kernel
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int h = g * G + w;
  float mmax = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) {
    const int64_t sl = ((int64_t)u * p.n_splits + sp) * G + w;
    mmax = fmaxf(mmax, p.ws_ml[(sl * 16 + r) * 2]);
  }
  float den = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ns; ++sp) {
    const int64_t sl = ((int64_t)u * p.n_splits + sp) * G + w;
    const float wgt = __builtin_amdgcn_exp2f(p.ws_ml[(sl * 16 + r) * 2] - mmax);
    den += wgt * p.ws_ml[(sl * 16 + r) * 2 + 1];
    const float* ps = p.ws_o + sl * (DT * 256);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] += wgt * *reinterpret_cast<const f32x4*>(ps + (dt * 64 + lane) * 4);
  }
  const float inv = 1.f / den;
  float* outp = p.out + (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D + 4 * q;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(outp + dt * 16) = acc[dt] * inv;
}

template <int D, int G, bool PAGED>
hipError_t launch_t(const AttnParams& p, hipStream_t stream) {
  const int groups = (p.n_units + kNumXcd - 1) / kNumXcd;
  const int grid = kNumXcd * p.n_splits * groups;
  hipLaunchKernelGGL((block_attn_kernel<D, G, PAGED, true>), dim3(grid), dim3(64 * G), 0, stream, p);
  if (p.n_splits > 1) hipLaunchKernelGGL((attn_merge_kernel<D, G>), dim3(p.n_units), dim3(64 * G), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_g(const AttnParams& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<D, 1, PAGED>(p, stream);
    case 2: return launch_t<D, 2, PAGED>(p, stream);
    case 3: return launch_t<D, 3, PAGED>(p, stream);
    case 4: return launch_t<D, 4, PAGED>(p, stream);
    case 5: return launch_t<D, 5, PAGED>(p, stream);
    case 6: return launch_t<D, 6, PAGED>(p, stream);
    case 7: return launch_t<D, 7, PAGED>(p, stream);
    case 8: return launch_t<D, 8, PAGED>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

AttnPlan plan_block_attn(int batch, int n_q_heads, int n_kv_heads, int head_dim, int max_ctx, int num_cu) {
  AttnPlan pl{};
  const int64_t units = (int64_t)batch * n_kv_heads;
  const int group = n_q_heads / n_kv_heads;
  // Aim for ~2 workgroups per CU over the longest sequence, with at least 256 keys
  // per split so the per-split fixed cost (Q load, partial write) stays small.
  const int64_t target_wg = 2LL * (num_cu > 0 ? num_cu : 256);
  int64_t kps = (units * (int64_t)max_ctx + target_wg - 1) / target_wg;
  kps = ((kps + TK - 1) / TK) * TK;
  if (kps < 256) kps = 256;
  if (kps > 8192) kps = 8192;
  pl.kps = (int)kps;
  pl.n_splits = max_ctx > 0 ? (int)((max_ctx + kps - 1) / kps) : 1;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // word 0: device error mask
  pl.off_ml = off;
  off = align(off + sizeof(float) * 2 * 16 * (size_t)group * pl.n_splits * units);
  pl.off_o = off;
  off = align(off + sizeof(float) * 16 * (size_t)group * head_dim * pl.n_splits * units);
  pl.ws_bytes = off;
  return pl;
}

hipError_t launch_block_attn(const AttnParams& p, int head_dim, int group, bool paged, hipStream_t stream) {
  if (head_dim == 128) return paged ? launch_g<128, true>(p, group, stream) : launch_g<128, false>(p, group, stream);
  if (head_dim == 64) return paged ? launch_g<64, true>(p, group, stream) : launch_g<64, false>(p, group, stream);
  return hipErrorInvalidValue;
}

}  // namespace dflash
