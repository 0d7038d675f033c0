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
//    head g*G+w and its 16 block rows; each K/V tile is brought into LDS once
//    and shared by the G heads (the context K/V stream is the HBM-bound part);
//  * context K/V tiles go HBM -> LDS with global_load_lds (16 bytes per lane, no
//    register staging) through an NST-stage ring of TK-key stages, so NST-1
//    stages are always in flight while one is consumed;
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16: keys are the
//    MFMA row dimension, so the score tile comes out with one query row per lane
//    column, the online-softmax statistics stay per lane, and the score
//    registers are already the B operand of the PV product (the key order of the
//    two 16-key score tiles is interleaved so each lane owns 8 consecutive keys);
//  * V stays row-major in LDS; the V^T operand is read with ds_read_b64_tr_b16
//    (LDS transpose read): lane j of a 16-lane group points at 4 dims of key row
//    j/4 and lane i receives one dim of 4 consecutive keys;
//  * both tiles use XOR-swizzled 16-byte chunks, chosen on the global side of
//    the LDS load (the LDS side of global_load_lds is lane-contiguous), so the
//    16-lane K reads and the 8-row transpose reads hit distinct banks;
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

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int TK = 32;   // keys per pipeline stage
constexpr int NST = 4;   // stages in the LDS ring

template <int D>
struct Geo {
  static constexpr int NCH = D / 8;                  // 16-byte chunks per key row
  static constexpr int ROW = D * 2;                  // bytes per key row
  static constexpr int TILE = TK * ROW;              // one K or V tile
  static constexpr int STAGE = 2 * TILE;             // K tile, then V tile
  static constexpr int RPL = 64 / NCH;               // key rows per wave-wide 1 KB load
  static constexpr int LOADS = 2 * TK / RPL;         // wave-wide loads per stage (K + V)
};

// Chunk swizzles (row t of a tile, 16-byte chunk c stored at c ^ swz(t)).
// K: the 16 rows 8(r/4) + 4j + r%4 read by one 16-lane group map to 16 distinct
// bank quads (d=128: 16 chunks per 256-byte row) or (row parity, chunk) pairs (d=64).
template <int D>
__device__ __forceinline__ int kswz(int t) {
  if constexpr (D == 128) return (t & 3) | (((t >> 3) & 3) << 2);
  else return ((t >> 1) & 1) | (((t >> 3) & 3) << 1);
}
// V: a transpose read of one 16-dim tile touches 32 bytes of each of the rows
// {0..3, 8..11} (+4, +16, +24); those 32-byte pieces land in distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int t) {
  if constexpr (D == 128) return 2 * ((t & 3) | (((t >> 3) & 1) << 2));
  else return 2 * (((t >> 1) & 1) | (((t >> 3) & 1) << 1));
}

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

// Issue this wave's share of the global->LDS loads of one stage: keys [t0, t0+TK)
// of unit (b, g), clamped to tend-1 (rows past the range hold a real, finite key
// row whose scores are masked, so no stale LDS data can leak in).
template <int D, int G, bool PAGED>
__device__ __forceinline__ void issue_stage(const AttnParams& p, char* stage, int b, int g, int t0, int tend,
                                            int w, int lane) {
  using GE = Geo<D>;
  const int rsub = lane / GE::NCH, pch = lane % GE::NCH;
#pragma unroll
  for (int li = w; li < GE::LOADS; li += G) {
    const bool is_v = li >= GE::LOADS / 2;
    const int rb = is_v ? li - GE::LOADS / 2 : li;
    const int row = rb * GE::RPL + rsub;
    const int key = min(t0 + row, tend - 1);
    const int c = pch ^ (is_v ? vswz<D>(row) : kswz<D>(row));
    // a 1 KB load covers RPL (4 or 8) aligned rows: never crosses a 16-token page
    const uint16_t* src = key_row<PAGED>(p, is_v ? p.v_cache : p.k_cache, b, g, key, D) + c * 8;
    char* dst = stage + (is_v ? GE::TILE : 0) + rb * 1024;
    lds_dma16_nt(src, dst);
  }
}

// Wait until at most `after` stages of this wave's loads are still in flight.
// Waves issue at least LOADS/G loads per stage, so counting with that minimum
// can only wait for more completions than needed.
template <int D, int G>
__device__ __forceinline__ void wait_stages(int after) {
  constexpr int L = Geo<D>::LOADS / G;
  if (after >= 2) wait_vmcnt<(2 * L < 63 ? 2 * L : 63)>();
  else if (after == 1) wait_vmcnt<(L < 63 ? L : 63)>();
  else wait_vmcnt<0>();
}

// One wave: 16 block rows of one query head against one TK-key stage in LDS,
// in NKK = TK/32 sub-steps of 32 keys.  Keys [0, nvalid) of the stage are real,
// the rest are masked out (sub-steps past nvalid are skipped).
template <int D, bool PLO>
__device__ __forceinline__ void attend_stage(const char* stage, const bf16x8* qB, f32x4* o, float& m,
                                             float& lsum, int lane, int nvalid, float scale_log2) {
  using GE = Geo<D>;
  constexpr int KS = D / 32, DT = D / 16, NKK = TK / 32;
  const int r = lane & 15, q = lane >> 4;
  const char* kt = stage;
  const char* vt = stage + GE::TILE;
  const int nkk = (nvalid + 31) >> 5;
  float x[NKK][2][4];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (kk < nkk) {
        const int t = 32 * kk + 8 * (r >> 2) + 4 * j + (r & 3);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + t * GE::ROW + (((ks * 4 + q) ^ kswz<D>(t)) << 4));
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
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (32 * kk + 8 * q + 4 * j + v >= nvalid) x[kk][j][v] = -INFINITY;
  }
  float mt = x[0][0][0];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) mt = fmaxf(mt, x[kk][j][v]);
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  // Lazy rescaling: the reference max m moves only when a stage max exceeds it
  // by more than 8 (log2 units), so probabilities stay <= 2^8 and the O / sum
  // rescale (all accumulators) runs a handful of times per split instead of once
  // per stage.  O and the sum always share the reference, so the result is the
  // same softmax.  Every stage has a real key, so mt is finite.
  if (__builtin_amdgcn_ballot_w64(mt > m + 8.f)) {
    const float mnew = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // m = -inf on the first stage -> 0
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    m = mnew;
  }
  float psum = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float e = __builtin_amdgcn_exp2f(x[kk][j][v] - m);
        x[kk][j][v] = e;
        psum += e;
      }
  lsum += psum;

  // V^T operand via transpose reads: lane (group q, index i) points at key row
  // 32kk + 8q + 4h + i/4, dims 4(i%4)..+3 of the 16-dim tile; it receives dim
  // dt*16 + i of keys 32kk + 8q + 4h .. +3.
  const int trow0 = 8 * q + (r >> 2);
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (kk >= nkk) break;
    bf16x8 ph, pl;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const __bf16 hi = static_cast<__bf16>(x[kk][j][v]);
        ph[4 * j + v] = hi;
        if constexpr (PLO) pl[4 * j + v] = static_cast<__bf16>(x[kk][j][v] - static_cast<float>(hi));
      }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      i16x4 part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 32 * kk + trow0 + 4 * h;
        const int c = 2 * dt + ((r & 3) >> 1);
        const char* addr = vt + t * GE::ROW + ((c ^ vswz<D>(t)) << 4) + (r & 1) * 8;
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(addr));
      }
      const i16x8 cat = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
      o[dt] = mfma16x16x32(a, ph, o[dt]);
      if constexpr (PLO) o[dt] = mfma16x16x32(a, pl, o[dt]);
    }
  }
}

template <int D, int G, bool PAGED, bool PLO>
__global__ __launch_bounds__(64 * G) void block_attn_kernel(AttnParams p) {
  using GE = Geo<D>;
  constexpr int KS = D / 32, DT = D / 16, HALF = D / 2;
  __shared__ __attribute__((aligned(1024))) char lds[NST * GE::STAGE];

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

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int h = g * G + w;

  // Start the context stream before anything else.
  const int n_st = (ke - kb + TK - 1) / TK;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < n_st) issue_stage<D, G, PAGED>(p, lds + st * GE::STAGE, b, g, kb + st * TK, ke, w, lane);

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

  // Context keys [kb, ke) through the stage ring.
  for (int it = 0; it < n_st; ++it) {
    wait_stages<D, G>(min(NST - 2, n_st - 1 - it));
    __syncthreads();  // stage `it` landed for every wave; stage it-1 is free again
    if (it + NST - 1 < n_st)
      issue_stage<D, G, PAGED>(p, lds + ((it + NST - 1) % NST) * GE::STAGE, b, g, kb + (it + NST - 1) * TK, ke,
                               w, lane);
    attend_stage<D, PLO>(lds + (it % NST) * GE::STAGE, qB, o, m, lsum, lane, min(TK, ke - kb - it * TK),
                         p.scale_log2);
  }

  // Block keys (positions L .. L+15), handled by the last split of the unit:
  // rotated K rows and V rows written into stage 0, rows 16..31 zero.
  if (last_split) {
    __syncthreads();
    char* kt = lds;
    char* vt = lds + GE::TILE;
    for (int off = tid * 16; off < GE::STAGE; off += 64 * G * 16)
      *reinterpret_cast<u32x4*>(lds + off) = (u32x4){0u, 0u, 0u, 0u};
    __syncthreads();
    for (int id = tid; id < kBlock * HALF; id += 64 * G) {
      const int t = id / HALF, j = id - t * HALF;
      const int64_t rowoff = (((int64_t)b * kBlock + t) * p.n_kv_heads + g) * D;
      const uint16_t* kr = p.k_blk + rowoff;
      const uint16_t* vr = p.v_blk + rowoff;
      const float c = p.rope_cos[(int64_t)(L + t) * HALF + j];
      const float sn = p.rope_sin[(int64_t)(L + t) * HALF + j];
      float y0, y1;
      rope_pair(bf16_to_f32(kr[j]), bf16_to_f32(kr[j + HALF]), c, sn, y0, y1);
      const int j2 = j + HALF;
      *reinterpret_cast<uint16_t*>(kt + t * GE::ROW + (((j >> 3) ^ kswz<D>(t)) << 4) + 2 * (j & 7)) = f32_to_bf16(y0);
      *reinterpret_cast<uint16_t*>(kt + t * GE::ROW + (((j2 >> 3) ^ kswz<D>(t)) << 4) + 2 * (j2 & 7)) = f32_to_bf16(y1);
      *reinterpret_cast<uint16_t*>(vt + t * GE::ROW + (((j >> 3) ^ vswz<D>(t)) << 4) + 2 * (j & 7)) = vr[j];
      *reinterpret_cast<uint16_t*>(vt + t * GE::ROW + (((j2 >> 3) ^ vswz<D>(t)) << 4) + 2 * (j2 & 7)) = vr[j2];
    }
    __syncthreads();
    attend_stage<D, PLO>(lds, qB, o, m, lsum, lane, kBlock, p.scale_log2);
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

// Log-sum-exp merge of the split partials: one workgroup per (unit, query head),
// thread = (row r, 8 consecutive dims).  Partials are stored in the split
// kernel's lane order: dims 16*dt + 4*q + v of row r at lane r + 16*q.
template <int D>
__global__ __launch_bounds__(2 * D) void attn_merge_kernel(AttnParams p, int group) {
  constexpr int DT = D / 16, NCH = D / 8;
  const int u = blockIdx.x / group, w = blockIdx.x - u * group;
  const int b = u / p.n_kv_heads, g = u - b * p.n_kv_heads;
  int L = p.ctx_len[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int ns = L > 0 ? (L + p.kps - 1) / p.kps : 1;
  if (ns == 1) return;  // written directly by the split kernel
  const int r = threadIdx.x / NCH, c = threadIdx.x % NCH;
  const int dt = c >> 1, q0 = 2 * (c & 1);
  const int h = g * group + w;
  const int64_t slot0 = (int64_t)u * p.n_splits * group + w;  // slot of split sp: slot0 + sp * group
  float mmax = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) mmax = fmaxf(mmax, p.ws_ml[((slot0 + (int64_t)sp * group) * 16 + r) * 2]);
  float den = 0.f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int sp = 0; sp < ns; ++sp) {
    const int64_t sl = slot0 + (int64_t)sp * group;
    const float* ml = p.ws_ml + (sl * 16 + r) * 2;
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - mmax);
    den += wgt * ml[1];
    const float* ps = p.ws_o + sl * (DT * 256) + (dt * 64 + r + 16 * q0) * 4;
    a0 += wgt * *reinterpret_cast<const f32x4*>(ps);
    a1 += wgt * *reinterpret_cast<const f32x4*>(ps + 64);
  }
  const float inv = 1.f / den;
  float* outp = p.out + (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D + 8 * c;
  *reinterpret_cast<f32x4*>(outp) = a0 * inv;
  *reinterpret_cast<f32x4*>(outp + 4) = a1 * inv;
}

template <int D, int G, bool PAGED>
hipError_t launch_t(const AttnParams& p, hipStream_t stream) {
  const int groups = (p.n_units + kNumXcd - 1) / kNumXcd;
  const int grid = kNumXcd * p.n_splits * groups;
  hipLaunchKernelGGL((block_attn_kernel<D, G, PAGED, true>), dim3(grid), dim3(64 * G), 0, stream, p);
  if (p.n_splits > 1) hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(p.n_units * G), dim3(2 * D), 0, stream, p, G);
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
