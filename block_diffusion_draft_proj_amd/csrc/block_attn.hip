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
//    (max, sum, O) in the workspace and the last split of a unit to finish
//    merges them (log-sum-exp).  All splits of a unit sit on one XCD, so the
//    partials and the arrival counter are handed over inside one L2, without
//    the L2 writeback a device-scope release costs.  Above 8 splits a small
//    second kernel merges instead;
//  * probabilities enter the PV product as a bf16 hi/lo pair (P = P_hi + P_lo),
//    so the only rounding of operands is the bf16 storage of Q, K and V.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace dflash {

namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int TK = 32;        // keys per pipeline stage
constexpr int NST = 8;        // stages in the LDS ring
constexpr int kMaxFused = 8;  // up to this many splits per unit merge inside the split kernel
constexpr int kMaxSplitKeys = 8192;  // context keys per split at most
constexpr int kMaxPtEntries = kMaxSplitKeys / 16 + 1;  // page-table slice of a split (paged caches)

// Wave groups per workgroup: group k consumes stage NGRP*pack + k of every pack of
// NGRP consecutive stages.  Two groups while the workgroup stays within 10 waves
// (so a wave keeps >= 168 VGPRs), one for larger query groups.
template <int G>
constexpr int ngrp() { return G <= 5 ? 2 : 1; }

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

// Cache row of a key.  `t` is the key's row in the unit's storage order, unwrapped:
// without a window it is the key's position; with a sliding window of W rows it runs
// past W where the ring wraps (row t - W), and t < 2W.  Paged caches: the page ids
// of the split come from its page-table slice in LDS (`pt`, entry i = page of rows
// 16*(pt0 + i) .. in the same unwrapped order; W is a multiple of 16, so t & 15 is
// the row in the page), so no global load precedes a DMA: waiting for one would
// also wait for every stage load issued before it.
template <bool PAGED>
__device__ __forceinline__ const uint16_t* key_row(const AttnParams& p, const uint16_t* cache, int b, int g,
                                                   int t, int D, const int32_t LDS_AS* pt, int pt0) {
  if constexpr (PAGED) {
    int page = pt[(t >> 4) - pt0];
    if ((unsigned)page >= (unsigned)p.num_pages) {
      set_dev_error(p.err, kDevErrPageId);
      page = 0;
    }
    return cache + (((int64_t)page * p.n_kv_heads + g) * 16 + (t & 15)) * D;
  } else {
    if (p.window > 0 && t >= p.window) t -= p.window;
    return cache + (((int64_t)b * p.n_kv_heads + g) * p.capacity + t) * D;
  }
}

// One wave-wide 1 KB load (index li of the stage's LOADS) of the stage holding keys
// [t0, t0+TK) of unit (b, g), clamped to tend-1 (rows past the range hold a real,
// finite key row whose scores are masked, so no stale LDS data can leak in).  Key t
// sits in storage row t + roff (unwrapped, see key_row).
template <int D, bool PAGED>
__device__ __forceinline__ void issue_load(const AttnParams& p, uint32_t stage, int b, int g, int t0, int tend,
                                           int li, int lane, const int32_t LDS_AS* pt, int pt0, int roff) {
  using GE = Geo<D>;
  const int rsub = lane / GE::NCH, pch = lane % GE::NCH;
  const bool is_v = li >= GE::LOADS / 2;
  const int rb = is_v ? li - GE::LOADS / 2 : li;
  const int row = rb * GE::RPL + rsub;
  const int key = min(t0 + row, tend - 1);
  const int c = pch ^ (is_v ? vswz<D>(row) : kswz<D>(row));
  // a 1 KB load covers RPL (4 or 8) aligned rows: never crosses a 16-token page
  const uint16_t* src = key_row<PAGED>(p, is_v ? p.v_cache : p.k_cache, b, g, key + roff, D, pt, pt0) + c * 8;
  lds_dma16_nt_m0(src, stage + (is_v ? GE::TILE : 0) + rb * 1024);
}

// Max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with the
// gfx950 row-swap permutes (VALU, no LDS round trip).
__device__ __forceinline__ float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
// Sum over the same four lanes: each permute returns the two values of a lane pair,
// one per result, so the sum is the same whichever is which.
__device__ __forceinline__ float sum_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// bf16 hi/lo split of two probabilities: hi = RNE(x), lo = RNE(x - hi), packed.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, b16x2));
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0 - h0, x1 - h1}, b16x2));
}

// One wave: 16 block rows of one query head against one 32-key stage in LDS.
// Keys [0, nvalid) of the stage are real (nvalid >= 1), the rest are masked out.
// Scores stay unscaled until the exponent: p = exp2(s * scale_log2 - m), with the
// running max m kept in scaled units (scale > 0, so max and scaling commute).
// QHL: Q comes as a bf16 pair (qB = hi, qL = lo, Q = hi + lo), so S^T takes two MFMAs
// per K step.
template <int D, bool QHL = false>
__device__ __forceinline__ void attend_stage(const char* stage, const bf16x8* qB, const bf16x8* qL, f32x4* o,
                                             float& m, float& lsum, int lane, int nvalid, float scale_log2) {
  using GE = Geo<D>;
  static_assert(TK == 32, "one 32-key MFMA step per stage");
  constexpr int KS = D / 32, DT = D / 16;
  const int r = lane & 15, q = lane >> 4;
  const char* kt = stage;
  const char* vt = stage + GE::TILE;

  // S^T = K Q^T for the two 16-key tiles j: MFMA row r of tile j is key
  // 8(r/4) + 4j + r%4, so lane (r, q) ends up with keys 8q + 4j + v.  The two
  // accumulation chains are interleaved.
  bf16x8 ka[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = 8 * (r >> 2) + 4 * j + (r & 3);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[j][ks] = *reinterpret_cast<const bf16x8*>(kt + t * GE::ROW + (((ks * 4 + q) ^ kswz<D>(t)) << 4));
  }
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s0 = mfma16x16x32(ka[0][ks], qB[ks], s0);
    s1 = mfma16x16x32(ka[1][ks], qB[ks], s1);
    if constexpr (QHL) {
      s0 = mfma16x16x32(ka[0][ks], qL[ks], s0);
      s1 = mfma16x16x32(ka[1][ks], qL[ks], s1);
    }
  }
  float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};  // key 8q + e
  if (nvalid < TK) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * q + e >= nvalid) x[e] = -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  mt = max_across_rows(mt) * scale_log2;
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
  for (int e = 0; e < 8; ++e) {
    x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], scale_log2, -m));
    psum += x[e];
  }
  lsum += psum;

  // P as the B operand of O^T += V^T P^T, as a bf16 hi/lo pair (P = hi + lo).
  u32x4 hw, lw;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t hh, ll;
    split_bf16x2(x[2 * i], x[2 * i + 1], hh, ll);
    hw[i] = hh;
    lw[i] = ll;
  }
  const bf16x8 ph = __builtin_bit_cast(bf16x8, hw), pl = __builtin_bit_cast(bf16x8, lw);

  // V^T operand via transpose reads: lane (group q, index i) points at key row
  // 8q + 4h + i/4, dims 4(i%4)..+3 of the 16-dim tile; it receives dim dt*16 + i
  // of keys 8q + 4h .. +3.
  const int trow0 = 8 * q + (r >> 2);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    i16x4 part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = trow0 + 4 * h;
      const int c = 2 * dt + ((r & 3) >> 1);
      const char* addr = vt + t * GE::ROW + ((c ^ vswz<D>(t)) << 4) + (r & 1) * 8;
      part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(addr));
    }
    const i16x8 cat = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
    o[dt] = mfma16x16x32(a, ph, o[dt]);
    o[dt] = mfma16x16x32(a, pl, o[dt]);
  }
}

// Split hand-off inside one L2.  Workgroup i runs on XCD i % 8 (round-robin
// dispatch; any partition into 1, 2, 4 or 8 XCDs keeps equal i % 8 on one XCD), and
// the decode below gives every split of a unit the same i % 8, so all of them share
// one L2.  Counter updates are atomics performed in that L2 (no device-scope bit: a
// device-scope atomic or write-through goes past the L2 to memory and costs
// microseconds).  A split that stores a partial stores it write-through (the L2
// acknowledges each store once it holds the data, and keeps a valid copy) and
// waits for the acknowledgements before it counts the partial as stored.  The
// reader's loads are served by the L2: a unit's partial slots are read once, by
// the unit's last split, and never share a cache line with another unit's slots,
// so no CU can hold an older copy of them in its L1 (which every launch starts
// empty).  A workgroup-scope buffer_inv would not help here: it leaves the L1's
// lines in place.  Each counter has a 128-byte line of its own, so no two XCDs ever
// hold one counter line in a launch; across launches the kernel-boundary L2
// writeback and invalidate keep the counters coherent.
constexpr int kCntStride = 32;  // uint32 words per arrival counter (one 128-byte line)
constexpr int kMergeSpinLimit = 1 << 20;  // polls of the stored count (~0.5 s) before giving up

// Issue this wave's share of the loads of stage pack `pk` (stages NP*pk ..
// NP*pk + NP-1): NP * LOADS wave-wide loads dealt round-robin over the NW waves.
// Clamped per-row addressing (used for paged caches and for a pack that reaches
// past the split's last key).
template <int D, int NW, int NP, bool PAGED>
__device__ __forceinline__ void issue_pack(const AttnParams& p, uint32_t ring, int b, int g, int kb, int ke, int pk,
                                           int w, int lane, const int32_t LDS_AS* pt, int pt0, int roff) {
  using GE = Geo<D>;
#pragma unroll
  for (int li = w; li < NP * GE::LOADS; li += NW) {
    const int sub = li / GE::LOADS;
    const int st = NP * pk + sub;
    issue_load<D, PAGED>(p, ring + (st % NST) * GE::STAGE, b, g, kb + st * TK, ke, li - sub * GE::LOADS, lane, pt,
                         pt0, roff);
  }
}

// Per-wave load plan of a dense cache for packs that lie inside the split: load k
// of this wave (index li = w + k*NW of the pack) reads from the K or V base of
// the pack at a per-lane byte offset that is the same for every pack.
template <int D, int NW, int NP>
struct DensePlan {
  static constexpr int NL = (NP * Geo<D>::LOADS + NW - 1) / NW;  // loads per wave per pack (upper bound)
  uint32_t voff[NL];   // per-lane byte offset from the pack base
  uint32_t lds_off[NL];  // LDS byte offset of the load within the ring, for pack 0
  bool is_v[NL];
  bool live[NL];
};

template <int D, int NW, int NP>
__device__ __forceinline__ DensePlan<D, NW, NP> dense_plan(int w, int lane) {
  using GE = Geo<D>;
  DensePlan<D, NW, NP> pl;
  const int rsub = lane / GE::NCH, pch = lane % GE::NCH;
#pragma unroll
  for (int k = 0; k < pl.NL; ++k) {
    const int li = w + k * NW;
    pl.live[k] = li < NP * GE::LOADS;
    const int sub = li / GE::LOADS, lj = li - sub * GE::LOADS;
    const bool is_v = lj >= GE::LOADS / 2;
    const int rb = is_v ? lj - GE::LOADS / 2 : lj;
    const int row = rb * GE::RPL + rsub;
    const int c = pch ^ (is_v ? vswz<D>(row) : kswz<D>(row));
    pl.is_v[k] = is_v;
    pl.voff[k] = (uint32_t)((sub * TK + row) * GE::ROW + c * 16);
    pl.lds_off[k] = (uint32_t)(sub * GE::STAGE + (is_v ? GE::TILE : 0) + rb * 1024);
  }
  return pl;
}

// Fast issue of pack `pk` of a dense cache (every key of the pack < ke):
// k_pack / v_pack are the byte addresses of the pack's first key row.
template <int D, int NW, int NP>
__device__ __forceinline__ void issue_pack_dense(const DensePlan<D, NW, NP>& pl, const char* k_pack,
                                                 const char* v_pack, uint32_t lds_ring, int pk) {
  using GE = Geo<D>;
  const uint32_t slot = (uint32_t)((pk % (NST / NP)) * NP * GE::STAGE);
#pragma unroll
  for (int k = 0; k < pl.NL; ++k)
    if (pl.live[k]) lds_dma16_nt_sv(pl.is_v[k] ? v_pack : k_pack, pl.voff[k], lds_ring + slot + pl.lds_off[k]);
}

// Wait until this wave has at most `after` (<= A) packs of loads in flight.  Every
// wave issues at least L loads per pack; counting with that minimum (and capping
// at the counter's 63) can only wait for more completions than needed.
template <int L, int A>
__device__ __forceinline__ void wait_packs(int after) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= A) wait_vmcnt<(A * L < 63 ? A * L : 63)>();
    else wait_packs<L, A - 1>(after);
  }
}

// QHL: the q / k inputs come already rotated (dflash_block_qkv_attn's reduce kernel):
// Q as a bf16 hi/lo pair (q_blk = hi, q_lo = lo; no RoPE here), the block K rotated
// and rounded.
template <int D, int G, bool PAGED, bool QHL>
__global__ __launch_bounds__(64 * ngrp<G>() * G) void block_attn_kernel(AttnParams p) {
  using GE = Geo<D>;
  constexpr int NGRP = ngrp<G>();
  constexpr int NW = NGRP * G;    // waves per workgroup
  constexpr int NPK = NST / NGRP;  // packs in the ring
  constexpr int LPK = NGRP * GE::LOADS / NW;  // loads per wave per pack (minimum)
  constexpr int KS = D / 32, DT = D / 16, HALF = D / 2;
  static_assert(NST % NGRP == 0 && NPK >= 3, "ring of stage packs, two or more packs in flight");
  static_assert(LPK >= 1, "every wave issues loads in every pack");
  // The stage ring, then (two wave groups only) the Q rows [16][G*D] bf16 and the
  // cos and sin rows [16][D/2] fp32 of positions L..L+15, staged through LDS by the
  // same DMA as the context.
  constexpr int QST = NGRP > 1 ? 32 * D * (G + 2) : 0;
  __shared__ __attribute__((aligned(1024))) char lds[NST * GE::STAGE + QST];
  char* const qst = lds + NST * GE::STAGE;
  __shared__ uint32_t s_last, s_early;
  __shared__ int32_t s_pt[PAGED ? kMaxPtEntries : 1];

  // XCD-aware decode: WG i runs on XCD i % 8; every split of a unit shares one XCD.
  // The merge's hand-off through one XCD's L2 depends on it, so a workgroup that finds
  // itself elsewhere raises DEVERR_XCD (with 2 or 4 XCDs per partition, i % 8 still
  // fixes the die: checked modulo the partition's XCD count).
  const int i_wg = blockIdx.x;
  if (p.fused && threadIdx.x == 0 && ((xcc_id() ^ (uint32_t)i_wg) & p.xcc_mask) != 0)
    set_dev_error(p.err, kDevErrXcd);
  const int xcd = i_wg % kNumXcd;
  const int jj = i_wg / kNumXcd;
  const int s = jj % p.n_splits;
  const int u = (jj / p.n_splits) * kNumXcd + xcd;
  if (u >= p.n_units) return;
  const int b = u / p.n_kv_heads, g = u - b * p.n_kv_heads;

  int L = p.ctx_len[b];
  if (L < 0 || L > p.max_ctx) {
    if (threadIdx.x == 0 && s == 0) set_dev_error(p.err, kDevErrCtxLen);
    L = L < 0 ? 0 : p.max_ctx;
  }
  // Context keys: the last Lw = min(L, W) positions under a sliding window of W,
  // else all L.  Key j (0 <= j < Lw) is position L - Lw + j.
  const int Lw = p.window > 0 ? min(L, p.window) : L;
  const int ns = Lw > 0 ? (Lw + p.kps - 1) / p.kps : 1;
  if (s >= ns) return;
  const int kb = s * p.kps;
  const int ke = min(Lw, kb + p.kps);
  const bool last_split = (s == ns - 1);
  // Storage row of key kb: its position, or with a window the position mod W (the
  // cache is a ring of W rows).  Rows of the split run on from there, unwrapped
  // (key t in row t + roff, wrapping at W; see key_row).
  const int sr = p.window > 0 ? (L - Lw + kb) % p.window : kb;
  const int roff = sr - kb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w / G, hw = w - grp * G;  // wave group, head within the kv group
  const int r = lane & 15, q = lane >> 4;
  const int h = g * G + hw;

  // Paged caches: the split's page ids go to LDS first, with plain loads waited for
  // before any stage load is issued: entries of the pages holding rows sr ..
  // sr + (ke - kb) - 1 only.  Every index stays inside the sequence's page-table row:
  // without a window the rows are keys < L <= 16*capacity; with one, the column
  // wraps at W/16 <= capacity (W a multiple of 16, checked on the host).
  const int32_t LDS_AS* pt_lds = (const int32_t LDS_AS*)s_pt;
  if constexpr (PAGED) {
    const int n_pt = ke > kb ? ((sr + (ke - kb) - 1) >> 4) - (sr >> 4) + 1 : 0;
    const int32_t* src = p.page_table + (int64_t)b * p.capacity;
    const int wcols = p.window >> 4;
    for (int i = tid; i < n_pt; i += 64 * NW) {
      int col = (sr >> 4) + i;
      if (wcols > 0 && col >= wcols) col -= wcols;
      s_pt[i] = src[col];
    }
    __syncthreads();
  }

  // Start the context stream right after the Q loads: packs 0 .. NPK-2 (part of
  // them after the Q wait, see QF).  Dense packs inside the split take the
  // scalar-base path; the rest clamp per row.
  const int n_st = (ke - kb + TK - 1) / TK;
  const int n_pk = (n_st + NGRP - 1) / NGRP;
  // packs with every key < ke (and, in a ring, every row before the wrap)
  const int n_fast = PAGED ? 0 : (p.window > 0 ? min(ke - kb, p.window - sr) : ke - kb) / (NGRP * TK);
  const DensePlan<D, NW, NGRP> dpl = dense_plan<D, NW, NGRP>(w, lane);
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(LDS_AS char*)lds;
  const uint32_t qst_lds = lds_ring + NST * GE::STAGE;
  const int64_t unit_row0 = ((int64_t)b * p.n_kv_heads + g) * p.capacity + sr;  // dense: row of key kb
  const char* k_split = reinterpret_cast<const char*>(p.k_cache) + unit_row0 * GE::ROW;
  const char* v_split = reinterpret_cast<const char*>(p.v_cache) + unit_row0 * GE::ROW;
  auto issue = [&](int pk) {
    if (pk < n_fast) {
      const int64_t off = (int64_t)pk * NGRP * TK * GE::ROW;
      issue_pack_dense<D, NW, NGRP>(dpl, k_split + off, v_split + off, lds_ring, pk);
    } else {
      issue_pack<D, NW, NGRP, PAGED>(p, lds_ring, b, g, kb, ke, pk, w, lane, pt_lds, sr >> 4, roff);
    }
  };
  constexpr int QL = G * D / 32, CL = D / 32;  // wave loads: Q rows, cos rows (sin the same)
  if constexpr (NGRP > 1) {
    // Q / cos / sin go first, so that waiting for them leaves the context stream in flight.
    const int qrow_chunks = G * D / 8;
    const char* qsrc = reinterpret_cast<const char*>(p.q_blk + (((int64_t)b * kBlock) * p.n_q_heads + g * G) * D);
    const char* csrc = reinterpret_cast<const char*>(p.rope_cos + (int64_t)L * HALF);
    const char* ssrc = reinterpret_cast<const char*>(p.rope_sin + (int64_t)L * HALF);
    if constexpr (QHL) {
      // Q hi into the Q area; Q lo into the rest of it (the cos / sin part, 2*CL loads)
      // and then the ring slot of stage NST-2, which the context stream first fills
      // inside the loop (Q is in registers by then).
      const char* lsrc = reinterpret_cast<const char*>(p.q_lo + (((int64_t)b * kBlock) * p.n_q_heads + g * G) * D);
#pragma unroll
      for (int li = w; li < 2 * QL; li += NW) {
        const int lo = li >= QL, l = li - lo * QL;
        const int ci = l * 64 + lane, row = ci / qrow_chunks, col = ci - row * qrow_chunks;
        const uint32_t dst = !lo ? qst_lds + l * 1024
                                 : (l < 2 * CL ? qst_lds + (QL + l) * 1024
                                               : lds_ring + (NST - 2) * GE::STAGE + (l - 2 * CL) * 1024);
        lds_dma16_m0((lo ? lsrc : qsrc) + ((int64_t)row * p.n_q_heads * D + col * 8) * 2, dst);
      }
    }
#pragma unroll
    for (int li = w; li < (QHL ? 0 : QL + 2 * CL); li += NW) {
      if (li < QL) {
        const int ci = li * 64 + lane, row = ci / qrow_chunks, col = ci - row * qrow_chunks;
        lds_dma16_m0(qsrc + ((int64_t)row * p.n_q_heads * D + col * 8) * 2, qst_lds + li * 1024);
      } else if (li < QL + CL) {
        lds_dma16_m0(csrc + (int64_t)((li - QL) * 64 + lane) * 16, qst_lds + li * 1024);
      } else {
        lds_dma16_m0(ssrc + (int64_t)((li - QL - CL) * 64 + lane) * 16, qst_lds + li * 1024);
      }
    }
    if (last_split) {
      // Block keys (positions L .. L+15) of the last split go into the ring slot of
      // the last pack, which the context stream first fills inside the loop: V rows
      // straight into their swizzled places (rows 16..31 zero), raw K rows into
      // rows 16..31 of the K tile for the RoPE pass below.
      constexpr int BL = kBlock / GE::RPL;  // wave loads per block tile
      const uint32_t bslot = lds_ring + (NST - 1) * GE::STAGE;
      const int64_t brow0 = ((int64_t)b * kBlock * p.n_kv_heads + g) * D;  // element offset of row t = 0
      const int64_t bstride = (int64_t)p.n_kv_heads * D;                   // elements between rows t
#pragma unroll
      for (int li = w; li < 2 * BL; li += NW) {
        const int is_v = li >= BL;
        const int t = (li - is_v * BL) * GE::RPL + lane / GE::NCH, pch = lane % GE::NCH;
        const uint16_t* src = (is_v ? p.v_blk : p.k_blk) + brow0 + t * bstride;
        if (is_v)
          lds_dma16_m0(src + ((pch ^ vswz<D>(t)) << 3), bslot + GE::TILE + (li - BL) * 1024);
        else if (QHL)  // already rotated: straight into its swizzled place
          lds_dma16_m0(src + ((pch ^ kswz<D>(t)) << 3), bslot + li * 1024);
        else
          lds_dma16_m0(src + (pch << 3), bslot + kBlock * GE::ROW + li * 1024);
      }
      char* vz = lds + (NST - 1) * GE::STAGE + GE::TILE + kBlock * GE::ROW;
      for (int off = tid * 16; off < (TK - kBlock) * GE::ROW; off += 64 * NW * 16)
        *reinterpret_cast<u32x4*>(vz + off) = (u32x4){0u, 0u, 0u, 0u};
    }
  }
  // Packs issued before the Q wait: Q, cos and sin compete with every CU's ring fill
  // for HBM, so with the whole ring ahead of them they land ~4.4 us after the start,
  // well after the ring is full; with two packs ahead they land at ~3.1 us and the
  // rest of the ring goes out right after them (measured inside the bench step).
  constexpr int QF = NGRP > 1 ? 2 : NPK - 1;
#pragma unroll
  for (int pk = 0; pk < QF; ++pk)
    if (pk < n_pk) issue(pk);

  // Q of head h: rows at positions L + r, rotated exactly and rounded once to bf16, as the
  // B operand of S^T = K Q^T (lane holds dims 32*ks + 8*q .. +8 of row r).
  bf16x8 qB[KS], qL[QHL ? KS : 1];
  if constexpr (NGRP > 1 && QHL) {
    wait_packs<LPK, QF>(n_pk);  // this wave's Q loads landed
    __syncthreads();                 // ... and every other wave's
#pragma unroll
    for (int pk = QF; pk < NPK - 1; ++pk)
      if (pk < n_pk) issue(pk);
    const int off0 = (r * G * D + hw * D + 8 * q) * 2;  // byte offset of this lane's row chunk in a Q blob
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = off0 + 64 * ks, blk = off >> 10;
      qB[ks] = *reinterpret_cast<const bf16x8*>(qst + off);
      const char* lsrc = blk < 2 * CL ? qst + (QL + blk) * 1024
                                      : lds + (NST - 2) * GE::STAGE + (blk - 2 * CL) * 1024;
      qL[ks] = *reinterpret_cast<const bf16x8*>(lsrc + (off & 1023));
    }
  } else if constexpr (NGRP > 1) {
    wait_packs<LPK, QF>(n_pk);  // this wave's Q / cos / sin loads landed
    __syncthreads();                 // ... and every other wave's
#pragma unroll
    for (int pk = QF; pk < NPK - 1; ++pk)
      if (pk < n_pk) issue(pk);
    const char* qrow = qst + (r * G * D + hw * D) * 2;
    const float* cr = reinterpret_cast<const float*>(qst + 32 * G * D) + r * HALF;
    const float* sr = reinterpret_cast<const float*>(qst + 32 * G * D + 32 * D) + r * HALF;
    u32x4 raw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ks] = *reinterpret_cast<const u32x4*>(qrow + (32 * ks + 8 * q) * 2);
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
        uint16_t ylo, yhi;
        rope_pair_bf16(lo, hi, c, sn, ylo, yhi);
        qB[ks][e] = __builtin_bit_cast(__bf16, ylo);
        qB[ks + KS / 2][e] = __builtin_bit_cast(__bf16, yhi);
      }
    }
  } else if constexpr (QHL) {
    const int64_t qo = (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qB[ks] = __builtin_bit_cast(bf16x8, ld16(p.q_blk + qo + 32 * ks + 8 * q));
      qL[ks] = __builtin_bit_cast(bf16x8, ld16(p.q_lo + qo + 32 * ks + 8 * q));
    }
  } else {
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
        uint16_t ylo, yhi;
        rope_pair_bf16(lo, hi, c, sn, ylo, yhi);
        qB[ks][e] = __builtin_bit_cast(__bf16, ylo);
        qB[ks + KS / 2][e] = __builtin_bit_cast(__bf16, yhi);
      }
    }
  }

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  if constexpr (NGRP > 1) {
    if (last_split) {
      // The block tile first (its loads landed with Q): rotate the raw K rows with
      // the cos / sin rows of the same positions, one 8-dim chunk pair per thread,
      // then wave group 0 attends to the 16 block keys while the context streams in.
      // (QHL: the block K came rotated, straight into its place.)
      char* kt = lds + (NST - 1) * GE::STAGE;
      const float* cq = reinterpret_cast<const float*>(qst + 32 * G * D);
      const float* sq = reinterpret_cast<const float*>(qst + 32 * G * D + 32 * D);
      constexpr int HC = HALF / 8;  // chunks per half row
      for (int it = tid; it < (QHL ? 0 : kBlock * HC); it += 64 * NW) {
        const int t = it / HC, c = it - t * HC;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kt + (kBlock + t) * GE::ROW + c * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kt + (kBlock + t) * GE::ROW + (c + HC) * 16);
        u32x4 ylo, yhi;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint16_t y[2][2];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const int j = 8 * c + 2 * e2 + hb;
            const float xl = hb ? bf16_hi(lo[e2]) : bf16_lo(lo[e2]);
            const float xh = hb ? bf16_hi(hi[e2]) : bf16_lo(hi[e2]);
            rope_pair_bf16(xl, xh, cq[t * HALF + j], sq[t * HALF + j], y[0][hb], y[1][hb]);
          }
          ylo[e2] = (uint32_t)y[0][0] | ((uint32_t)y[0][1] << 16);
          yhi[e2] = (uint32_t)y[1][0] | ((uint32_t)y[1][1] << 16);
        }
        *reinterpret_cast<u32x4*>(kt + t * GE::ROW + ((c ^ kswz<D>(t)) << 4)) = ylo;
        *reinterpret_cast<u32x4*>(kt + t * GE::ROW + (((c + HC) ^ kswz<D>(t)) << 4)) = yhi;
      }
      __syncthreads();
      if (grp == 0) attend_stage<D, QHL>(kt, qB, qL, o, m, lsum, lane, kBlock, p.scale_log2);
    }
  }

  // Context keys [kb, ke): wave group grp consumes stage NGRP*pk + grp of each pack.
  for (int pk = 0; pk < n_pk; ++pk) {
    wait_packs<LPK, NPK - 2>(n_pk - 1 - pk);
    __syncthreads();  // pack pk landed for every wave; pack pk-1 is free again
    if (pk + NPK - 1 < n_pk) issue(pk + NPK - 1);
    const int st = NGRP * pk + grp;
    if (st < n_st)
      attend_stage<D, QHL>(lds + (st % NST) * GE::STAGE, qB, qL, o, m, lsum, lane, min(TK, ke - kb - st * TK),
                           p.scale_log2);
  }

  // One wave group: block keys (positions L .. L+15) after the context, in the
  // last split: rotated K rows and V rows written into stage 0, rows 16..31 zero.
  if (NGRP == 1 && last_split) {
    __syncthreads();
    char* kt = lds;
    char* vt = lds + GE::TILE;
    for (int off = tid * 16; off < GE::STAGE; off += 64 * NW * 16)
      *reinterpret_cast<u32x4*>(lds + off) = (u32x4){0u, 0u, 0u, 0u};
    __syncthreads();
    for (int id = tid; id < kBlock * HALF; id += 64 * NW) {
      const int t = id / HALF, j = id - t * HALF;
      const int64_t rowoff = (((int64_t)b * kBlock + t) * p.n_kv_heads + g) * D;
      const uint16_t* kr = p.k_blk + rowoff;
      const uint16_t* vr = p.v_blk + rowoff;
      uint16_t y0 = kr[j], y1 = kr[j + HALF];  // QHL: already rotated
      if (!QHL) {
        const float c = p.rope_cos[(int64_t)(L + t) * HALF + j];
        const float sn = p.rope_sin[(int64_t)(L + t) * HALF + j];
        rope_pair_bf16(bf16_to_f32(kr[j]), bf16_to_f32(kr[j + HALF]), c, sn, y0, y1);
      }
      const int j2 = j + HALF;
      *reinterpret_cast<uint16_t*>(kt + t * GE::ROW + (((j >> 3) ^ kswz<D>(t)) << 4) + 2 * (j & 7)) = y0;
      *reinterpret_cast<uint16_t*>(kt + t * GE::ROW + (((j2 >> 3) ^ kswz<D>(t)) << 4) + 2 * (j2 & 7)) = y1;
      *reinterpret_cast<uint16_t*>(vt + t * GE::ROW + (((j >> 3) ^ vswz<D>(t)) << 4) + 2 * (j & 7)) = vr[j];
      *reinterpret_cast<uint16_t*>(vt + t * GE::ROW + (((j2 >> 3) ^ vswz<D>(t)) << 4) + 2 * (j2 & 7)) = vr[j2];
    }
    __syncthreads();
    if (grp == 0) attend_stage<D, QHL>(lds, qB, qL, o, m, lsum, lane, kBlock, p.scale_log2);
  }

  // Combine the wave groups in LDS (stage slots 2.. are free: every wave passed
  // its last stage).  Each group keeps half of the dimension tiles (group k: tiles
  // k*DTG ..): it hands the other half of its O, with its (m, lsum), to the other
  // group and folds that group's share of its own half.  Both groups evaluate the
  // combined (m, lsum) with one expression (group 0's terms first), so they hold
  // identical values.  Lane layout of O: dims 16*dt + 4*q + v of row r.
  constexpr int DTG = DT / NGRP;
  const int dt0 = grp * DTG;
  f32x4 oh[DTG];

  // Fused merge, early hand-off.  The split that attends to the block keys (the last
  // one) usually ends its loop after the others.  It reads its unit's counter before
  // the wave-group fold, so the read's round trip overlaps the fold: if the other
  // ns - 1 splits have all stored their partials, it is the last arrival and goes
  // straight to the merge, with no arrival to count and no wait (its loads, issued
  // after that read, see every stored partial in the L2).  Otherwise it takes the
  // hand-off below.
  uint32_t* cnt = p.count + (int64_t)u * kCntStride;
  const bool try_early = p.fused && ns > 1 && last_split;
  uint32_t early_v = 0;
  if (try_early && tid == 0) {
    uint32_t zero;  // an opaque zero: see the poll below
    asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
    early_v = __hip_atomic_fetch_add(cnt, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  if constexpr (NGRP > 1) {
    static_assert(NGRP == 2, "two wave groups");
    __syncthreads();
    float* xo = reinterpret_cast<float*>(lds + 2 * GE::STAGE);  // [2][G][DTG][64][4]
    float* xml = xo + 2 * G * DTG * 256;                         // [2][G][64][2]
    float* give = xo + (grp * G + hw) * DTG * 256;
#pragma unroll
    for (int j = 0; j < DTG; ++j)
      *reinterpret_cast<f32x4*>(give + (j * 64 + lane) * 4) = grp ? o[j] : o[DTG + j];
    *reinterpret_cast<float2*>(xml + ((grp * G + hw) * 64 + lane) * 2) = make_float2(m, lsum);
    if (try_early && tid == 0) s_early = (early_v >> 16) == (uint32_t)(ns - 1) ? 1u : 0u;
    __syncthreads();
    const int oth = 1 - grp;
    const float* take = xo + (oth * G + hw) * DTG * 256;
    const float2 mlo = *reinterpret_cast<const float2*>(xml + ((oth * G + hw) * 64 + lane) * 2);
    // A group that saw no key has m = -inf; one of the two always saw one (the
    // split has a key), but guard the empty case anyway.
    const float mn = fmaxf(m, mlo.x);
    const bool none = mn == -INFINITY;
    const float a_own = none ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    const float a_oth = none ? 0.f : __builtin_amdgcn_exp2f(mlo.x - mn);
    const float l0 = grp ? mlo.y : lsum, w0 = grp ? a_oth : a_own;
    const float l1 = grp ? lsum : mlo.y, w1 = grp ? a_own : a_oth;
    lsum = l0 * w0 + l1 * w1;
    m = mn;
#pragma unroll
    for (int j = 0; j < DTG; ++j)
      oh[j] = (grp ? o[DTG + j] : o[j]) * a_own + *reinterpret_cast<const f32x4*>(take + (j * 64 + lane) * 4) * a_oth;
  } else {
#pragma unroll
    for (int j = 0; j < DTG; ++j) oh[j] = o[j];
    if (try_early) {
      if (tid == 0) s_early = (early_v >> 16) == (uint32_t)(ns - 1) ? 1u : 0u;
      __syncthreads();
    }
  }
  const bool early = try_early && __builtin_amdgcn_readfirstlane(s_early) != 0u;
  // Every wave now holds the split's (m, lsum) for query head hw and its O for
  // dimension tiles dt0 .. dt0 + DTG - 1.

  const float lt = sum_across_rows(lsum);

  float* outp = p.out + (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D + 4 * q;
  if (ns == 1) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int j = 0; j < DTG; ++j) *reinterpret_cast<f32x4*>(outp + (dt0 + j) * 16) = oh[j] * inv;
    return;
  }

  const int64_t slot = ((int64_t)u * p.n_splits + s) * G + hw;
  float* po = p.ws_o + slot * (DT * 256);
  // Partials are stored write-through (cache policy sc0 sc1, system scope): the L2
  // keeps the line for the merging split, and the lines are clean by the time the
  // kernel ends, so the end-of-kernel L2 writeback has ~6 MB less to write
  // (-0.3 to -0.6 us per call, interleaved A/B; plain and non-temporal stores both
  // measured slower).
  constexpr int kWriteThrough = 1 | 16;  // sc0 | sc1
  auto store_partial = [&]() {
    const __amdgpu_buffer_rsrc_t rs_po = __builtin_amdgcn_make_buffer_rsrc(po, 0, DT * 1024, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_pm = __builtin_amdgcn_make_buffer_rsrc(p.ws_ml + slot * 32, 0, 16 * 8, 0x00020000);
#pragma unroll
    for (int j = 0; j < DTG; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, oh[j]), rs_po, ((dt0 + j) * 64 + lane) * 16, 0, kWriteThrough);
    if (grp == 0 && q == 0)
      __builtin_amdgcn_raw_buffer_store_b64((u32x2){__float_as_uint(m), __float_as_uint(lt)}, rs_pm, r * 8, 0, kWriteThrough);
  };
  if (!p.fused) {  // attn_merge_kernel combines the splits after this kernel
    store_partial();
    return;
  }

  // Fused merge.  The unit's counter word holds arrivals (low 16 bits) and stored
  // partials (high 16 bits).  A split counts its arrival first: the split that
  // arrives last keeps its own state in registers and never stores it; every other
  // split stores its partial, waits for the L2 to acknowledge it, then counts it as
  // stored.  The last arrival waits until the other ns - 1 partials are stored
  // (those splits already arrived, so they are running and only storing), clears
  // the counter for the next call and combines all ns states (log-sum-exp, in
  // split order).
  if (early) {
    // every other split arrived and stored: clear the counter for the next call
    if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    uint32_t prev = 0;
    if (tid == 0) {
      prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      s_last = (prev & 0xffffu) == (uint32_t)(ns - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_last)) {
      store_partial();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      wait_vmcnt<0>();  // this wave's partial is in the L2
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __syncthreads();  // ... and every other wave's
      if (tid == 0) __hip_atomic_fetch_add(cnt, 1u << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return;
    }
    if (tid == 0) {
      uint32_t v = prev;
      for (int spin = 0; (v >> 16) != (uint32_t)(ns - 1); ++spin) {
        if (spin >= kMergeSpinLimit) {  // cannot happen while the stored splits run; never hang
          set_dev_error(p.err, kDevErrMerge);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        // Re-read the count with an atomic add of an opaque zero, performed in the L2.
        // A load would not do: the first one brings the line into this CU's L1 and the
        // next ones hit that stale copy (a workgroup-scope invalidate does not drop
        // it), and the compiler turns an atomic add of a literal zero into such a load.
        uint32_t zero;
        asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
        v = __hip_atomic_fetch_add(cnt, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
  }

  // The merge: every wave combines its DTG dimension tiles of its head over all
  // splits: its own split from registers, the others from the shared L2 (sc0
  // loads; see the hand-off notes above).  All loads of a chunk of CH splits, and every
  // split's (m, l), are issued before any is used (addresses clamped to a real
  // split), so up to CH splits cost one memory round trip.
  constexpr int CH = (DTG * 4 * kMaxFused <= 128 && NW <= 8) ? kMaxFused : (NW <= 8 ? 4 : 2);
  constexpr int kL2 = 1;  // cache policy sc0
  const int64_t slot0 = (int64_t)u * p.n_splits * G;  // first slot of the unit
  const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_o + slot0 * (DT * 256), 0, p.n_splits * G * DT * 1024, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_ml = __builtin_amdgcn_make_buffer_rsrc(
      p.ws_ml + slot0 * 32, 0, p.n_splits * G * 16 * 8, 0x00020000);
  u32x4 part[CH][DTG];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int sp = min(c0 + k, ns - 1);
      if (sp == s) continue;  // own state stays in registers
      const int sl = sp * G + hw;
#pragma unroll
      for (int j = 0; j < DTG; ++j)
        part[k][j] = __builtin_amdgcn_raw_buffer_load_b128(rs_o, (sl * DT * 64 + (dt0 + j) * 64 + lane) * 16, 0, kL2);
    }
  };
  load_chunk(0);
  float mv[kMaxFused], lv[kMaxFused];
#pragma unroll
  for (int sp = 0; sp < kMaxFused; ++sp) {
    const int sl = min(sp, ns - 1) * G + hw;
    const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(rs_ml, (sl * 16 + r) * 8, 0, kL2);
    mv[sp] = sp < ns ? (sp == s ? m : __uint_as_float(ml[0])) : -INFINITY;
    lv[sp] = sp < ns ? (sp == s ? lt : __uint_as_float(ml[1])) : 0.f;
  }
  float mmax = mv[0];
#pragma unroll
  for (int sp = 1; sp < kMaxFused; ++sp) mmax = fmaxf(mmax, mv[sp]);
  float den = 0.f;
  f32x4 acc[DTG];
#pragma unroll
  for (int j = 0; j < DTG; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c0 = 0; c0 < kMaxFused; c0 += CH) {
    if (c0 >= ns) break;
    if (c0 > 0) load_chunk(c0);
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int sp = c0 + k;
      if (sp >= ns) break;
      const float wgt = __builtin_amdgcn_exp2f(mv[sp] - mmax);
      den += wgt * lv[sp];
#pragma unroll
      for (int j = 0; j < DTG; ++j) acc[j] += wgt * (sp == s ? oh[j] : __builtin_bit_cast(f32x4, part[k][j]));
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int j = 0; j < DTG; ++j) *reinterpret_cast<f32x4*>(outp + (dt0 + j) * 16) = acc[j] * inv;
}

// Log-sum-exp merge of the split partials (more than kMaxFused splits per unit):
// one workgroup per (unit, query head, quarter of the dimensions: 32 dims).  Thread
// (split group sg, row r, 8-dim chunk c) combines splits sg, sg+4, ... of its row's
// 8 dims with all their loads issued before the first is used; the four split
// groups are summed through LDS, in a fixed order.  Partials are stored in the
// split kernel's lane order: dims 16*dt + 4*q + v of row r at lane r + 16*q.
constexpr int kMergeGroups = 4;
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p, int group) {
  constexpr int DT = D / 16, NQ = D / 32;
  __shared__ float s_acc[kMergeGroups][64][9];
  const int dq = blockIdx.x % NQ, uh = blockIdx.x / NQ;
  const int u = uh / group, w = uh - u * group;
  const int b = u / p.n_kv_heads, g = u - b * p.n_kv_heads;
  int L = p.ctx_len[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  const int Lw = p.window > 0 ? min(L, p.window) : L;
  const int ns = Lw > 0 ? (Lw + p.kps - 1) / p.kps : 1;
  if (ns == 1) return;  // written directly by the split kernel
  const int tid = threadIdx.x, sg = tid >> 6, rc = tid & 63;
  const int r = rc >> 2, c = rc & 3;  // row, 8-dim chunk of the quarter
  const int dt = 2 * dq + (c >> 1), q0 = 2 * (c & 1);
  const int h = g * group + w;
  const int64_t slot0 = (int64_t)u * p.n_splits * group + w;  // slot of split sp: slot0 + sp * group
  float mmax = -INFINITY;
#pragma unroll 8
  for (int sp = 0; sp < ns; ++sp) mmax = fmaxf(mmax, p.ws_ml[((slot0 + (int64_t)sp * group) * 16 + r) * 2]);
  float den = 0.f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int sp = sg; sp < ns; sp += kMergeGroups) {
    const int64_t sl = slot0 + (int64_t)sp * group;
    const float* ml = p.ws_ml + (sl * 16 + r) * 2;
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - mmax);
    den += wgt * ml[1];
    const float* ps = p.ws_o + sl * (DT * 256) + (dt * 64 + r + 16 * q0) * 4;
    a0 += wgt * *reinterpret_cast<const f32x4*>(ps);
    a1 += wgt * *reinterpret_cast<const f32x4*>(ps + 64);
  }
  float* sa = s_acc[sg][rc];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    sa[e] = a0[e];
    sa[4 + e] = a1[e];
  }
  sa[8] = den;
  __syncthreads();
  if (sg != 0) return;
#pragma unroll
  for (int k = 1; k < kMergeGroups; ++k) {
    const float* o = s_acc[k][rc];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a0[e] += o[e];
      a1[e] += o[4 + e];
    }
    den += o[8];
  }
  const float inv = 1.f / den;
  float* outp = p.out + (((int64_t)b * kBlock + r) * p.n_q_heads + h) * D + 32 * dq + 8 * c;
  *reinterpret_cast<f32x4*>(outp) = a0 * inv;
  *reinterpret_cast<f32x4*>(outp + 4) = a1 * inv;
}

template <int D, int G, bool PAGED>
hipError_t launch_t(const AttnParams& p, hipStream_t stream) {
  const int groups = (p.n_units + kNumXcd - 1) / kNumXcd;
  const int grid = kNumXcd * p.n_splits * groups;
  if (p.q_lo)
    hipLaunchKernelGGL((block_attn_kernel<D, G, PAGED, true>), dim3(grid), dim3(64 * ngrp<G>() * G), 0, stream, p);
  else
    hipLaunchKernelGGL((block_attn_kernel<D, G, PAGED, false>), dim3(grid), dim3(64 * ngrp<G>() * G), 0, stream, p);
  if (p.n_splits > 1 && !p.fused)
    hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(p.n_units * G * (D / 32)), dim3(256), 0, stream, p, G);
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
  // One workgroup per CU over the longest sequence, with at least 256 keys per
  // split so the per-split fixed cost (Q load, partial write) stays small.
  const int64_t target_wg = num_cu > 0 ? num_cu : 256;
  int64_t kps = (units * (int64_t)max_ctx + target_wg - 1) / target_wg;
  kps = ((kps + 2 * TK - 1) / (2 * TK)) * (2 * TK);
  // At most a quarter of the longest context per split, a sixteenth when there are at
  // least as many units as CUs (the GPU is full without splitting, so splits serve
  // balance only): the host does not know the lengths of a ragged batch, and its
  // longest sequences then come in 4 or 16 pieces that the dispatcher spreads over
  // the CUs.  A uniform batch that leaves CUs to fill is unaffected: there the bound
  // above is already <= max_ctx / 4.  (Ragged batch of 32 x 8 units: 715 us with
  // 8192-key splits, 352 us with a quarter, 291 us with an eighth; later, with an
  // eighth 308 us against 298 us with a sixteenth, whose 16 splits take the separate
  // merge kernel.)
  const int64_t div = units >= target_wg ? 16 : 4;
  const int64_t quarter = ((max_ctx / div + 2 * TK - 1) / (2 * TK)) * (2 * TK);
  if (kps > quarter) kps = quarter;
  if (kps < 256) kps = 256;
  if (kps > kMaxSplitKeys) kps = kMaxSplitKeys;
  pl.kps = (int)kps;
  pl.n_splits = max_ctx > 0 ? (int)((max_ctx + kps - 1) / kps) : 1;
  pl.fused = pl.n_splits <= kMaxFused;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // word 0: device error mask
  pl.off_cnt = off;  // per-unit arrival counters (fused merge), left at zero by every call
  static_assert(sizeof(uint32_t) * kCntStride * kMaxCountSlots == kCountRegionBytes, "counter region");
  off = align(off + kCountRegionBytes);
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
