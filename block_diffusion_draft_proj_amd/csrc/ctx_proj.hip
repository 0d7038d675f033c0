// Context projection of the DFlash draft: target-layer hidden states are
// concatenated, projected by the fc layer into the draft's context feature C,
// and C is projected by the layer's K/V weights into context K/V rows that
// are rotated (K only) and written into the context cache at their token
// positions.
//
// Pages: "DFlash dual implementations: PyTorch vs MLX" §4 (select target layers
// by id and concatenate their hidden states), §2 (context K/V come from the
// projected target hidden states), §1 (Qwen3 rotary embedding); "dflash-mlx:
// lossless speculative decoding", "block-diffusion draft" (the draft reads the
// target hidden states) and "single-forward verify" step 9 (only the committed
// prefix stays in the cache: rows with a negative position are not written).
//
// gfx950 mapping: both products are "A x W^T" with K contiguous in both
// operands, which is exactly the MFMA operand layout (each lane holds 8
// consecutive K elements of one row), so A and W tiles go global -> XOR-swizzled
// LDS (global_load_lds, no register staging) -> v_mfma_f32_16x16x32_bf16 with no
// transposes.  The concatenation is implicit: the K loop walks the layer
// pointers.  For the per-cycle case (M = B*16 rows) the product is a weight
// stream, so K is split over workgroups to put a workgroup on every CU; fp32
// partial sums are reduced by small epilogue kernels (bf16 rounding of C; RoPE,
// bf16 rounding and cache scatter of K/V).
#include "common.h"
#include "launch.h"
#include "split_sum.h"

namespace dflash {

namespace {

// Tiled product for many activation rows (more than 256: prefill chunks).  A
// workgroup owns a 256 (rows of A) x 256 (rows of B) output tile; eight waves each own
// 128 x 64 of it (per 32-wide K step 8 A and 4 B operand reads feed 32 MFMAs).  K goes
// in 64-element stages: 128-byte LDS rows, so a wave-wide load covers 8 rows in 8 cache
// lines (32-element stages, 64-byte rows, take 16 lines per load and measured ~5 % of
// the MFMA peak slower).  A stage is an A tile and a B tile of 32 KB each; LDS holds a ring of five such
// tiles (160 KB).  While the waves read the tiles of stage it, the B tile of stage
// it + 1 and the A tile of stage it + 2 stream in, so half of the data is asked for one
// and a half stages ahead.  Waves 0..3, one on each SIMD, issue all loads, sixteen
// per iteration spread over their 64 MFMAs (one before every fourth): a wave held at the
// address unit then leaves its SIMD to the other wave there, which never issues a load.
// (Issued together after the barrier, the loads of all waves queue at the address unit
// and hold every wave off its MFMAs.)
// The operand base addresses are wave-uniform register values, chosen with scalar
// selects: a base indexed at run time (a segment table, or a per-lane choice between
// the two weight pointers) compiles to a load inside the loop whose wait also waits
// for every stage load in flight, which empties the ring at each stage.
// Tile order (workgroup i runs on XCD i % 8): with at least 8 rows of tiles, XCD x takes
// tile rows x, x + 8, ... in bands of 4 rows, column-major within a band, so the 32
// workgroups resident on a die at a time cover 4 x 8 tiles and share their A and B
// panels in its L2; with fewer, each XCD takes a contiguous run of row-major tiles.
constexpr int BK = 64;  // K stage of both products (128-byte LDS rows)
constexpr int kThreads = 512;
constexpr int GBM = 256, GBN = 256;
constexpr int G_TILE = GBM * BK * 2;                   // one operand tile of a stage (32 KB)
constexpr int G_SLOTS = 5;                             // LDS ring of operand tiles (160 KB)
constexpr int kIssueWaves = 4;                        // waves 0..3 (one per SIMD) issue the loads
constexpr int G_LOADS_W = G_TILE / 1024 / kIssueWaves;  // wave-wide 1 KB loads per tile and issuing wave (8)
constexpr int kBand = 4;                               // tile rows per band of the tile order
static_assert(GBM == GBN, "A and B tiles share the slot size");
static_assert(G_TILE % (1024 * kIssueWaves) == 0, "tile loads split evenly over the issuing waves");

// 128-byte rows (64 bf16 of K); 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7):
// the 16 rows read by one 16-lane MFMA operand group hit distinct banks.
__device__ __forceinline__ int swz_off(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

// Tile (tm, tn) of workgroup index i in the order above; false if i has none.
__device__ __forceinline__ bool tile_of(int i, int ntm, int ntn, int& tm, int& tn) {
  const int x = i % kNumXcd, j = i / kNumXcd;
  if (ntm >= kNumXcd) {
    const int rows = (ntm - x + kNumXcd - 1) / kNumXcd;  // tile rows x, x + 8, ... of this XCD
    const int band = j / (kBand * ntn);
    if (band * kBand >= rows) return false;
    const int gh = min(kBand, rows - band * kBand);  // rows of this band
    const int k = j - band * kBand * ntn;
    if (k >= gh * ntn) return false;                  // past a short last band
    tm = x + kNumXcd * (band * kBand + k % gh);
    tn = k / gh;
    return true;
  }
  const int tiles = ntm * ntn, per = (tiles + kNumXcd - 1) / kNumXcd;
  const int t = x * per + j;
  if (j >= per || t >= tiles) return false;
  tm = t / ntn;
  tn = t % ntn;
  return true;
}

// A 64-bit pointer made a provably wave-uniform value (two readfirstlanes).
__device__ __forceinline__ uint64_t uniform_u64(const void* ptr) {
  const uint64_t a = (uint64_t)(uintptr_t)ptr;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[G_SLOTS * G_TILE];
  const int ntn = (p.N + GBN - 1) / GBN, ntm = (p.M + GBM - 1) / GBM;
  int tm, tn;
  if (!tile_of((int)blockIdx.x, ntm, ntn, tm, tn)) return;
  const int n0 = tn * GBN, m0 = tm * GBM, z = blockIdx.y;
  const int kbeg = z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int n_st = (kend - kbeg) / BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int lrow = lane >> 3, pch = lane & 7;  // one wave-wide load = 8 rows x 128 bytes
  const int wm = w >> 2, wn = w & 3;          // rows 128 wm .. of A, 64 wn .. of B
  const uint32_t ring = (uint32_t)(uintptr_t)(LDS_AS char*)lds;

  static_assert(kMaxLayers == 8, "one register value per segment below");
  const uint64_t sb0 = uniform_u64(p.a_seg[0]), sb1 = uniform_u64(p.a_seg[1]), sb2 = uniform_u64(p.a_seg[2]);
  const uint64_t sb3 = uniform_u64(p.a_seg[3]), sb4 = uniform_u64(p.a_seg[4]), sb5 = uniform_u64(p.a_seg[5]);
  const uint64_t sb6 = uniform_u64(p.a_seg[6]), sb7 = uniform_u64(p.a_seg[7]);
  const uint64_t bb0 = uniform_u64(p.b0), bb1 = uniform_u64(p.b1);
  // Loads of an issuing wave, fixed for the whole K loop: load i covers rows 8 (4 i + w)
  // .. + 7 of a tile; each lane brings 16 bytes of its row, global chunk pch ^ swizzle, so
  // LDS holds the row's chunk c at c ^ swizzle.  Rows past M or N are clamped to the
  // last real row: every load is in bounds and the extra results are never stored.
  uint64_t a_row[G_LOADS_W], b_row[G_LOADS_W];  // byte offset in a layer, byte address
#pragma unroll
  for (int i = 0; i < G_LOADS_W; ++i) {
    const int row = (i * kIssueWaves + w) * 8 + lrow;
    const int sw = (pch ^ ((row >> 1) & 7)) << 3;
    const int m = min(m0 + row, p.M - 1);
    const int n = min(n0 + row, p.N - 1);
    a_row[i] = 2 * ((uint64_t)m * p.lda + sw);
    b_row[i] = (n < p.n_b0 ? bb0 + 2 * ((uint64_t)n * p.K) : bb1 + 2 * ((uint64_t)(n - p.n_b0) * p.K)) + 2 * sw;
  }
  auto seg_base = [&](int seg) -> uint64_t {
    return seg == 0 ? sb0 : seg == 1 ? sb1 : seg == 2 ? sb2 : seg == 3 ? sb3
         : seg == 4 ? sb4 : seg == 5 ? sb5 : seg == 6 ? sb6 : sb7;
  };
  // Load i of an A tile whose K columns start at byte `a_k` of the layer rows (a
  // wave-uniform address: the layer base plus the column offset), and of the B tile
  // of the stage starting at column k0; into ring slot `slot`.
  auto issue_a = [&](uint64_t a_k, int slot, int i) {
    lds_dma16_m0(reinterpret_cast<const char*>((uintptr_t)(a_k + a_row[i])),
                 ring + (uint32_t)(slot * G_TILE) + (uint32_t)((i * kIssueWaves + w) * 1024));
  };
  auto issue_b = [&](int k0, int slot, int i) {
    lds_dma16_m0(reinterpret_cast<const char*>((uintptr_t)b_row[i]) + 2 * (int64_t)k0,
                 ring + (uint32_t)(slot * G_TILE) + (uint32_t)((i * kIssueWaves + w) * 1024));
  };
  // A stage's 64 columns lie in one layer (seg_k is a multiple of 64).  The layer and
  // column of the next A tile to issue are stepped once per stage, so the division
  // and the select chain run only when a layer boundary is crossed.
  auto a_addr = [&](int k0) -> uint64_t {
    const int seg = k0 / p.seg_k;
    return seg_base(seg) + 2 * (uint64_t)(k0 - seg * p.seg_k);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int ma = 0; ma < 8; ++ma)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[ma][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Operand tile h is the A tile of stage h / 2 for even h, its B tile for odd h, in
  // ring slot h % 5.  Tiles 0, 1 (stage 0) and 2 (A of stage 1) go before the loop;
  // iteration it then asks for tiles 2 it + 3 (B of stage it + 1) and 2 it + 4 (A of
  // stage it + 2), in that order, into the slots of stage it - 1.
  const bool issuer = w < kIssueWaves;
  if (issuer && n_st > 0) {
#pragma unroll
    for (int i = 0; i < G_LOADS_W; ++i) issue_a(a_addr(kbeg), 0, i);
#pragma unroll
    for (int i = 0; i < G_LOADS_W; ++i) issue_b(kbeg, 1, i);
  }
  if (issuer && n_st > 1) {
#pragma unroll
    for (int i = 0; i < G_LOADS_W; ++i) issue_a(a_addr(kbeg + BK), 2, i);
  }
  // the next A tile to issue: stage 2, in layer a_seg at column a_col
  int a_seg = (kbeg + 2 * BK) / p.seg_k, a_col = kbeg + 2 * BK - a_seg * p.seg_k;
  uint64_t a_next = seg_base(a_seg) + 2 * (uint64_t)a_col;
  // The issuing wave of each SIMD carries the loads besides the same MFMAs as its partner
  // and reaches the barrier last; with the higher priority the SIMD favours it when both
  // are ready (prefill chunk of 2048 / 8192 / 32768 rows 0.7-1.5 % faster, interleaved
  // A/B; the reverse order is 7-10 % slower).
  if (issuer) __builtin_amdgcn_s_setprio(1);
  for (int it = 0; it < n_st; ++it) {
    // the tiles of stage it landed for this wave: at most tile 2 it + 2 still flies
    if (!issuer) {
    } else if (it + 1 < n_st) {
      wait_vmcnt<G_LOADS_W>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();  // ... for every wave; the slots of stage it - 1 are free again
    const char* sa = lds + ((2 * it) % G_SLOTS) * G_TILE;
    const char* sb = lds + ((2 * it + 1) % G_SLOTS) * G_TILE;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 bw[4], ax[8];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bw[nb] = *reinterpret_cast<const bf16x8*>(sb + swz_off(wn * 64 + nb * 16 + r, kh * 4 + q));
#pragma unroll
      for (int ma = 0; ma < 8; ++ma) ax[ma] = *reinterpret_cast<const bf16x8*>(sa + swz_off(wm * 128 + ma * 16 + r, kh * 4 + q));
#pragma unroll
      for (int ma = 0; ma < 8; ++ma) {
        if (issuer) {  // load kh * 8 + ma of this iteration's sixteen
          const int g = kh * 8 + ma;
          if (g < G_LOADS_W) {
            if (it + 1 < n_st) issue_b(kbeg + (it + 1) * BK, (2 * it + 3) % G_SLOTS, g);
          } else {
            if (it + 2 < n_st) issue_a(a_next, (2 * it + 4) % G_SLOTS, g - G_LOADS_W);
          }
          __builtin_amdgcn_sched_barrier(0);  // keep the load between these MFMAs
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[ma][nb] = mfma16x16x32(bw[nb], ax[ma], acc[ma][nb]);
      }
    }
    a_col += BK;
    a_next += 2 * BK;
    if (a_col >= p.seg_k) {  // the next A tile starts the next layer
      a_col = 0;
      a_next = seg_base(++a_seg);
    }
  }

  // D layout: lane holds A row m0 + 128 wm + 16 ma + r and B rows 4q .. 4q+3 of its
  // 16-row group: 4 consecutive outputs of one row, one 16-byte store (N % 4 == 0).
  float* out = p.out + (int64_t)z * p.M * p.N;
#pragma unroll
  for (int ma = 0; ma < 8; ++ma) {
    const int m = m0 + wm * 128 + ma * 16 + r;
    if (m >= p.M) continue;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + wn * 64 + nb * 16 + 4 * q;
      if (n < p.N) *reinterpret_cast<f32x4*>(out + (int64_t)m * p.N + n) = acc[ma][nb];
    }
  }
}

// Skinny product (M <= 256 rows of activations, the per-cycle case): a weight
// stream.  Each workgroup owns 128 weight rows (4 row waves x 32; 64 rows, 4 x 16,
// when the grid would otherwise leave half of the CUs idle, see launch_skinny) and
// one K range, and sees all 16*MT activation rows (MT = 4, 8 or 16: two wave groups
// of 4, each on half of the activation tiles).  A 64-K stage holds the weight tile
// (128 rows, 16 KB) and the activation tile (16*MT rows, MT x 2 KB); stages go
// global -> swizzled LDS by global_load_lds through a 4-stage ring (128 KB at
// MT = 8), so three stages are in flight while one feeds the MFMAs.
// Per stage a wave reads its own 16 x RT weight rows and its activation tiles
// from LDS and does 2 x MTW x RT MFMAs; each weight byte crosses LDS 1 + TG times
// and each activation byte five times (vs. thirteen for a square-tile GEMM).
// The activations either come packed step by step ([K/64][16*MT rows][64]: the K/V
// product reads C packed by fc_reduce_kernel, or by pack_rows_kernel when the rows
// already are C), a step's tile then being one contiguous 16*MT x 128-byte block, or
// are read in place from their rows (the fc product walks the target layers' rows,
// the q/k/v and draft-layer products their activation rows), see PACKED below.
constexpr int SK_RW = 4;                     // weight-row wave groups (32 rows each)
// Up to kSkinnyMaxRows activation rows take the skinny kernel (MT = 16 at 129..256
// rows), one pass over the weights.  Above that the tiled kernel is faster: the
// qwen3_8b-shaped projection (5 x 4096 -> 4096 -> 2 x 1024) at 384 rows 169 against
// 151 us, at 512 rows (two skinny passes) 195 against 154 us; at 256 rows the skinny
// pass wins, 110 against 126 us.
constexpr int kSkinnyMaxRows = 256;
constexpr int SK_RT = 2;                     // 16-row weight tiles per wave (1 on small grids)
constexpr int SK_ROWS = SK_RW * SK_RT * 16;  // weight rows per workgroup (128; the planner's tile)

template <int MT, int RT = SK_RT>
struct SkGeo {
  static constexpr int ROWS = SK_RW * RT * 16;                // weight rows per workgroup
  static constexpr int W_TILE = ROWS * BK * 2;                // RT x 8 KB
  static constexpr int X_TILE = 16 * MT * BK * 2;             // MT x 2 KB
  static constexpr int STAGE = W_TILE + X_TILE;
  static constexpr int NS = (160 * 1024) / STAGE < 4 ? (160 * 1024) / STAGE : 4;  // ring stages
  static constexpr int LOADS = STAGE / 1024;                  // wave-wide 1 KB loads per stage
  // A second group of four waves takes half of the activation tiles whenever the
  // stage's loads split evenly over eight waves: two waves per SIMD hide the LDS
  // read and MFMA latency of one another (4% faster at 128 rows x 20480 x 4096).
  static constexpr int TG = MT % 4 == 0 ? 2 : 1;              // activation-tile wave groups
  static constexpr int WAVES = SK_RW * TG;
  static constexpr int MTW = MT / TG;                         // activation tiles per wave
  static constexpr int LW = LOADS / WAVES;                    // per wave (every wave the same)
  static_assert(LOADS % WAVES == 0, "stage loads split evenly over the waves");
  static_assert(NS >= 3, "two stages in flight");
};

// PACKED: activations come packed as [K/64][mp][64] steps (written by
// fc_reduce_kernel for the K/V product); else they are read in place from the
// segments a_seg[] ([M][lda] each, seg_k columns of K per segment).
// SWIGLU: one split, and each workgroup's 128 weight rows are 64 gate rows (B0 rows
// j0 .. j0 + 63, waves 0 and 1) over the same 64 up rows (B1, waves 2 and 3), so the
// epilogue has both results of its columns and writes bf16(silu(g) * u) instead of
// partial sums.
template <int MT, bool PACKED, int RT, bool SWIGLU = false>
__global__ __launch_bounds__((SkGeo<MT, RT>::WAVES * 64)) void gemm_skinny_kernel(GemmParams p) {
  using SG = SkGeo<MT, RT>;
  __shared__ __attribute__((aligned(1024))) char lds[SG::NS * SG::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int lrow = lane >> 3, pch = lane & 7;  // one wave-wide load = 8 rows x 128 bytes
  // XCD-aware decode (workgroup i runs on XCD i % 8): with a multiple of 8 splits every
  // XCD works on as few K ranges as possible, so the activation slice of its range
  // (16*MT rows x K/splits) stays in that XCD's L2 while all column tiles stream their
  // weights past it.  With 1, 2 or 4 splits the plain decode below does the same; with
  // 3, 5, 6 or 7 (at most 8 splits, small activation slices) an XCD reads several.
  const int splits = (p.K + p.k_per_split - 1) / p.k_per_split;
  const int id = blockIdx.x;
  int z, col;
  if (splits % kNumXcd == 0) {
    const int per = splits / kNumXcd, j = id / kNumXcd;
    z = id % kNumXcd + kNumXcd * (j % per);
    col = j / per;
  } else {
    z = id % splits;
    col = id / splits;
  }
  const int n0 = col * SG::ROWS;
  const int kbeg = z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int n_st = (kend - kbeg) / BK;
  const uint32_t ring = (uint32_t)(uintptr_t)(LDS_AS char*)lds;

  // Loads of stage st: li < 16 weight rows 8li..8li+7, then activation rows
  // 8(li-16).. (rows past N / M clamp to the last real row: every load stays in
  // bounds and the extra results are never stored).
  // Column tiles walk their K range from different starting steps, so the
  // activation steps read at one time are spread over the range.
  const int rot = n_st > 0 ? col % n_st : 0;
  // In-place reads: the segment bases, made wave-uniform register values once, so
  // the per-stage choice below is a chain of scalar selects.  (Indexing a_seg[] at
  // run time instead puts a scalar load in every stage, whose wait counter also
  // counts LDS reads.)
  static_assert(kMaxLayers == 8, "one register value per segment below");
  auto uniform_ptr = [&](int l) -> uint64_t { return PACKED ? 0 : uniform_u64(p.a_seg[l]); };
  const uint64_t sb0 = uniform_ptr(0), sb1 = uniform_ptr(1), sb2 = uniform_ptr(2), sb3 = uniform_ptr(3);
  const uint64_t sb4 = uniform_ptr(4), sb5 = uniform_ptr(5), sb6 = uniform_ptr(6), sb7 = uniform_ptr(7);
  // issue(st, i0, i1): this wave's loads i0 .. i1-1 of stage st.
  auto issue = [&](int st, int i0, int i1) {
    const int ks = st + rot < n_st ? st + rot : st + rot - n_st;
    const int k0 = kbeg + ks * BK;
    const uint16_t* xstep = PACKED ? p.xp + ((int64_t)(k0 / BK) * p.mp + p.m_off) * BK : nullptr;
    const uint32_t stage = ring + (uint32_t)((st % SG::NS) * SG::STAGE);
#pragma unroll
    for (int i = 0; i < SG::LW; ++i) {
      if (i < i0 || i >= i1) continue;
      const int li = i * SG::WAVES + w;  // wave-uniform
      if (li < SG::W_TILE / 1024) {
        const int row = li * 8 + lrow;
        int n;
        if constexpr (SWIGLU) {
          const int j = min(col * 64 + (row & 63), p.n_b0 - 1);
          n = row < 64 ? j : p.n_b0 + j;
        } else {
          n = min(n0 + row, p.N - 1);
        }
        const uint16_t* brow = n < p.n_b0 ? p.b0 + (int64_t)n * p.K : p.b1 + (int64_t)(n - p.n_b0) * p.K;
        lds_dma16_nt_m0(brow + k0 + ((pch ^ ((row >> 1) & 7)) << 3), stage + li * 1024);
      } else {
        const int row = (li - SG::W_TILE / 1024) * 8 + lrow;
        const int sw = (pch ^ ((row >> 1) & 7)) << 3;
        if (PACKED) {
          // packed activations: the 16*MT rows of step ks are one contiguous block
          lds_dma16_m0(xstep + row * BK + sw, stage + li * 1024);
        } else {
          // in place: 128 bytes of row m_off + row (clamped to the last real row, whose
          // extra results are never stored), columns k0 .. k0 + 63 of A, which lie in
          // one segment (seg_k is a multiple of 64)
          const int m = min(p.m_off + row, p.M - 1);
          const int seg = k0 / p.seg_k;  // wave-uniform
          const uint64_t base = seg == 0 ? sb0 : seg == 1 ? sb1 : seg == 2 ? sb2 : seg == 3 ? sb3
                              : seg == 4 ? sb4 : seg == 5 ? sb5 : seg == 6 ? sb6 : sb7;
          const uint16_t* src = reinterpret_cast<const uint16_t*>((uintptr_t)base);
          lds_dma16_m0(src + (int64_t)m * p.lda + (k0 - seg * p.seg_k) + sw, stage + li * 1024);
        }
      }
    }
  };

  constexpr int MTW = SG::MTW;
  const int wr = w % SK_RW, wt = w / SK_RW;  // weight rows 16*RT*wr.., activation tiles MTW*wt..
  f32x4 acc[RT][MTW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) acc[rt][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < SG::NS - 1; ++st)
    if (st < n_st) issue(st, 0, SG::LW);
  // The refill of stage it + NS - 1 is spread over the stage's two K halves, each part
  // issued once that half's LDS reads are in flight: right after the barrier all waves
  // would otherwise queue their loads at the CU's address unit at once and only then
  // start their MFMAs (per-stage timestamps: 844 of ~1880 cycles spent issuing).
  constexpr int LH = (SG::LW + 1) / 2;  // loads issued in the first half
  for (int it = 0; it < n_st; ++it) {
    // stage `it` landed for this wave: at most min(NS-2, n_st-1-it) younger stages in flight
    const int after = min(SG::NS - 2, n_st - 1 - it);
    if (after >= 4) wait_vmcnt<(4 * SG::LW < 63 ? 4 * SG::LW : 63)>();
    else if (after == 3) wait_vmcnt<3 * SG::LW>();
    else if (after == 2) wait_vmcnt<2 * SG::LW>();
    else if (after == 1) wait_vmcnt<SG::LW>();
    else wait_vmcnt<0>();
    __syncthreads();  // every wave's part of stage `it` landed; stage it-1 is free again
    const bool refill = it + SG::NS - 1 < n_st;
    const char* sw = lds + (it % SG::NS) * SG::STAGE;
    const char* sx = sw + SG::W_TILE;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      bf16x8 a[RT], xb[MTW];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        a[rt] = *reinterpret_cast<const bf16x8*>(sw + swz_off(wr * (16 * RT) + rt * 16 + r, kh * 4 + q));
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
        xb[mt] = *reinterpret_cast<const bf16x8*>(sx + swz_off((wt * MTW + mt) * 16 + r, kh * 4 + q));
      if (refill) issue(it + SG::NS - 1, kh == 0 ? 0 : LH, kh == 0 ? LH : SG::LW);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) acc[rt][mt] = mfma16x16x32(a[rt], xb[mt], acc[rt][mt]);
    }
  }

  // D layout: lane holds activation row 16*(MTW*wt + mt) + r and weight rows 4q .. 4q+3 of
  // the 16-row tile: 4 consecutive outputs of one row, one 16-byte store.
  if constexpr (SWIGLU) {
    static_assert(RT == 2 && SK_RW == 4, "gate rows in waves 0 and 1, the same up rows in waves 2 and 3");
    // Wave wr + 2 holds the up results of wave wr's gate columns, in the same lanes: it
    // hands them over through the ring, which every wave has finished reading.
    __syncthreads();
    f32x4* xch = reinterpret_cast<f32x4*>(lds) + ((wt * 2 + (wr & 1)) * RT * MTW) * 64 + lane;
    if (wr >= 2) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) xch[(rt * MTW + mt) * 64] = acc[rt][mt];
    }
    __syncthreads();
    if (wr >= 2) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int j = col * 64 + wr * 32 + rt * 16 + 4 * q;
      if (j >= p.n_b0) continue;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        const int m = (wt * MTW + mt) * 16 + r;
        if (m >= p.m_rows) continue;
        const f32x4 g = acc[rt][mt], u = xch[(rt * MTW + mt) * 64];
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = g[e] / (1.f + expf(-g[e])) * u[e];
        *reinterpret_cast<u32x2*>(p.act + (int64_t)(p.m_off + m) * p.n_b0 + j) =
            (u32x2){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
      }
    }
    return;
  }
  float* out = p.out + (int64_t)z * p.M * p.N;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = n0 + wr * (16 * RT) + rt * 16 + 4 * q;
    if (n >= p.N) continue;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
      const int m = (wt * MTW + mt) * 16 + r;
      if (m < p.m_rows) *reinterpret_cast<f32x4*>(out + (int64_t)(p.m_off + m) * p.N + n) = acc[rt][mt];
    }
  }
}

// Activation rows -> [K/64][mp][64] packed steps (rows >= M zero): one 16-byte
// chunk per thread, reads and writes both coalesced.
__global__ __launch_bounds__(256) void pack_rows_kernel(PackParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // chunk index
  const int64_t per_step = (int64_t)p.mp * 8;
  if (i >= (int64_t)(p.K / 64) * per_step) return;
  const int st = (int)(i / per_step);
  const int rem = (int)(i - st * per_step);
  const int row = rem >> 3, c = rem & 7;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < p.M) {
    const int k = st * 64 + c * 8;
    const int seg = k / p.seg_k;
    v = ld16(p.a_seg[seg] + (int64_t)row * p.lda + (k - seg * p.seg_k));
  }
  st16(p.xp + i * 8, v);
}

// C = bf16(sum over splits): 4 columns per thread; written row-major and/or packed.
__global__ __launch_bounds__(256) void fc_reduce_kernel(FcReduceParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int64_t total = (int64_t)p.M * p.N / 4;
  if (i >= total) return;
  const f32x4 s = sum_splits(p.part + 4 * i, (int64_t)p.M * p.N, p.splits);
  const u32x2 v = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  if (p.c_buf) *reinterpret_cast<u32x2*>(p.c_buf + 4 * i) = v;
  if (p.c_out) *reinterpret_cast<u32x2*>(p.c_out + 4 * i) = v;
  if (p.c_pack) {
    const int64_t m = 4 * i / p.N;
    const int n = (int)(4 * i - m * p.N);
    *reinterpret_cast<u32x2*>(p.c_pack + ((int64_t)(n >> 6) * p.mp + m) * 64 + (n & 63)) = v;
  }
}

// Block q / k / v = bf16(sum over splits), 4 columns per thread.  Columns [0, nq) go
// to q, [nq, nq + nk) to k, the rest to v, each token-major ([M][heads * d]).  nq and
// nk are multiples of 64, so a 4-column group never straddles two outputs.
__global__ __launch_bounds__(256) void qkv_reduce_kernel(QkvReduceParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int64_t total = (int64_t)p.M * p.N / 4;
  if (i >= total) return;
  const f32x4 s = sum_splits(p.part + 4 * i, (int64_t)p.M * p.N, p.splits);
  const u32x2 v = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  const int64_t m = 4 * i / p.N;
  const int n = (int)(4 * i - m * p.N);
  uint16_t* dst;
  if (n < p.nq) dst = p.q + m * p.nq + n;
  else if (n < p.nq + p.nk) dst = p.k + m * p.nk + (n - p.nq);
  else dst = p.v + m * p.nk + (n - p.nq - p.nk);
  *reinterpret_cast<u32x2*>(dst) = v;
}

// The block's q/k/v handed to the attention: thread = (row, head of q, k or v, 4
// consecutive j < d/2), i.e. columns j .. j+3 and j+d/2 .. j+d/2+3 of one head.  The
// split sums are issued before the row's position is known.
//   q: rotated at the position (fp64 products and sum, then fp32: within 2^-24
//      relative), kept as hi = bf16(y) and lo = bf16(y - hi) (y - hi is exact in fp32),
//      which carry y to about 2^-17 relative;
//   k: the exact rotation rounded once to bf16;  v: bf16.
__global__ __launch_bounds__(256) void qkv_rope_kernel(QkvRopeParams p) {
  const int half = p.head_dim / 2;
  const int per_row = p.N / 8;  // (Hq + 2 Hkv) heads x d/8 column groups
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.M * per_row) return;
  const int m = (int)(i / per_row);
  const int rem = (int)(i - (int64_t)m * per_row);
  const int head = rem / (half / 4);            // over q, k and v heads in column order
  const int j = (rem - head * (half / 4)) * 4;
  const int c0 = head * p.head_dim + j;         // columns c0 .. c0+3 and c0+half ..
  const float* base = p.part + (int64_t)m * p.N;
  const int64_t zs = (int64_t)p.M * p.N;
  const f32x4 x0 = sum_splits(base + c0, zs, p.splits);
  const f32x4 x1 = sum_splits(base + c0 + half, zs, p.splits);
  if (c0 >= p.nq + p.nk) {  // v
    uint16_t* dst = p.v_out + (int64_t)m * p.nk + (c0 - p.nq - p.nk);
    *reinterpret_cast<u32x2*>(dst) = (u32x2){pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3])};
    *reinterpret_cast<u32x2*>(dst + half) = (u32x2){pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
    return;
  }
  const int seq = m / kBlock;
  int L = p.ctx_len[seq];
  if (L < 0 || L > p.max_ctx) {
    if ((m & (kBlock - 1)) == 0 && rem == 0) set_dev_error(p.err, kDevErrCtxLen);
    L = L < 0 ? 0 : p.max_ctx;
  }
  const int pos = L + (m & (kBlock - 1));
  const f32x4 c = *reinterpret_cast<const f32x4*>(p.rope_cos + (int64_t)pos * half + j);
  const f32x4 s = *reinterpret_cast<const f32x4*>(p.rope_sin + (int64_t)pos * half + j);
  if (c0 >= p.nq) {  // k
    uint16_t y0[4], y1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_pair_bf16(x0[e], x1[e], c[e], s[e], y0[e], y1[e]);
    uint16_t* dst = p.k_out + (int64_t)m * p.nk + (c0 - p.nq);
    *reinterpret_cast<u32x2*>(dst) = (u32x2){y0[0] | (uint32_t)y0[1] << 16, y0[2] | (uint32_t)y0[3] << 16};
    *reinterpret_cast<u32x2*>(dst + half) = (u32x2){y1[0] | (uint32_t)y1[1] << 16, y1[2] | (uint32_t)y1[3] << 16};
    return;
  }
  uint16_t h0[4], h1[4], l0[4], l1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // products of fp32 values are exact in fp64: one rounding there, one to fp32
    const float y0 = (float)((double)x0[e] * c[e] - (double)x1[e] * s[e]);
    const float y1 = (float)((double)x1[e] * c[e] + (double)x0[e] * s[e]);
    h0[e] = f32_to_bf16(y0);
    h1[e] = f32_to_bf16(y1);
    l0[e] = f32_to_bf16(y0 - bf16_to_f32(h0[e]));
    l1[e] = f32_to_bf16(y1 - bf16_to_f32(h1[e]));
  }
  const int64_t o = (int64_t)m * p.nq + c0;
  auto pack4 = [](const uint16_t (&v)[4]) {
    return (u32x2){v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16};
  };
  *reinterpret_cast<u32x2*>(p.q_hi + o) = pack4(h0);
  *reinterpret_cast<u32x2*>(p.q_hi + o + half) = pack4(h1);
  *reinterpret_cast<u32x2*>(p.q_lo + o) = pack4(l0);
  *reinterpret_cast<u32x2*>(p.q_lo + o + half) = pack4(l1);
}

// K/V rows: sum splits, rotate K (pairs j, j+d/2) at the row's position (exactly,
// one rounding to bf16) and write into the cache.  Thread = (row, kv head, 4 consecutive j < d/2).
__global__ __launch_bounds__(256) void kv_epilogue_kernel(KvEpilogueParams p) {
  const int half = p.head_dim / 2;
  const int per_row = p.n_kv_heads * (half / 4);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.M * per_row) return;
  const int m = (int)(i / per_row);
  const int rem = (int)(i - (int64_t)m * per_row);
  const int hh = rem / (half / 4);
  const int j = (rem - hh * (half / 4)) * 4;
  // The split sums do not depend on the row's position: issue them with it.
  const int N = 2 * p.n_kv_heads * p.head_dim;
  const int ck = hh * p.head_dim + j;
  const int cv = p.n_kv_heads * p.head_dim + ck;
  const float* base = p.part + (int64_t)m * N;
  const int64_t zs = (int64_t)p.M * N;
  const int pos = p.row_pos[m];
  const f32x4 k0 = sum_splits(base + ck, zs, p.splits);
  const f32x4 k1 = sum_splits(base + ck + half, zs, p.splits);
  const f32x4 v0 = sum_splits(base + cv, zs, p.splits);
  const f32x4 v1 = sum_splits(base + cv + half, zs, p.splits);
  if (pos < 0) return;  // uncommitted block slot
  const int seq = p.row_seq[m];
  const bool paged = p.page_size > 0;
  // Storage row: the position, or with a sliding window of W rows the position mod W
  // (a ring; the host checked W against the capacity).
  const int row = p.window > 0 ? pos % p.window : pos;
  const bool bad = (unsigned)seq >= (unsigned)p.batch || pos >= p.max_pos ||
                   (paged ? (row >> 4) >= p.capacity : row >= p.capacity);
  if (bad) {
    set_dev_error(p.err, kDevErrRow);
    return;
  }
  int64_t row_off;
  if (paged) {
    const int page = p.page_table[(int64_t)seq * p.capacity + (row >> 4)];
    if ((unsigned)page >= (unsigned)p.num_pages) {
      set_dev_error(p.err, kDevErrPageId);
      return;
    }
    row_off = (((int64_t)page * p.n_kv_heads + hh) * 16 + (row & 15)) * p.head_dim;
  } else {
    row_off = (((int64_t)seq * p.n_kv_heads + hh) * p.capacity + row) * p.head_dim;
  }
  const f32x4 c = *reinterpret_cast<const f32x4*>(p.rope_cos + (int64_t)pos * half + j);
  const f32x4 s = *reinterpret_cast<const f32x4*>(p.rope_sin + (int64_t)pos * half + j);
  uint16_t y0[4], y1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) rope_pair_bf16(k0[e], k1[e], c[e], s[e], y0[e], y1[e]);
  uint16_t* kd = p.k_cache + row_off;
  uint16_t* vd = p.v_cache + row_off;
  *reinterpret_cast<u32x2*>(kd + j) = (u32x2){y0[0] | ((uint32_t)y0[1] << 16), y0[2] | ((uint32_t)y0[3] << 16)};
  *reinterpret_cast<u32x2*>(kd + j + half) = (u32x2){y1[0] | ((uint32_t)y1[1] << 16), y1[2] | ((uint32_t)y1[3] << 16)};
  *reinterpret_cast<u32x2*>(vd + j) = (u32x2){pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3])};
  *reinterpret_cast<u32x2*>(vd + j + half) = (u32x2){pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
}

// Tiled path: split K so that the tiles fill the CUs (one workgroup each), while
// the fp32 partial sums (splits x M x N x 4 bytes, written and read back once) stay
// within the operand bytes ((M + N) x K x 2) and every split keeps >= 4 stages.
int split_count(int tiles, int M, int N, int K, int num_cu) {
  if (tiles < 1) tiles = 1;
  int splits = (num_cu + tiles - 1) / tiles;
  const int64_t mn = (int64_t)(M > 0 ? M : 1) * (N > 0 ? N : 1);
  const int by_traffic = (int)(((int64_t)(M + N) * K) / (2 * mn));
  const int by_depth = K / (4 * BK);
  splits = min(splits, max(1, by_traffic));
  splits = min(splits, max(1, by_depth));
  return max(1, splits);
}

int k_per_split(int K, int splits) {
  int kps = (K + splits - 1) / splits;
  return ((kps + BK - 1) / BK) * BK;
}

}  // namespace

// Skinny plan: workgroups of 128 weight rows, one per CU at a time.  K is split to
// minimise the time of the rounds of workgroups: rounds (tiles x splits / CUs, rounded
// up) times a workgroup's steps (K / 64 / splits) plus a fixed cost of about eight
// steps (ring fill and partial store).  The draft layer's gate/up product (192 column
// tiles over 4096 of K) then takes one split, 192 workgroups of 64 steps: with two (a
// full round and a half-empty one) the layer's post-attention call took 122.3 us, with
// four 128.1, with one 115.7.  The fp32 partial sums (splits x M x N x 4 bytes, written
// and read back once) stay within half the weight bytes (N x K x 2; twice them above
// 128 rows) and every split keeps >= 2 steps.  Ties go to fewer splits.
int skinny_splits(int N, int M, int K, int num_cu) {
  const int tiles = (N + SK_ROWS - 1) / SK_ROWS;
  // fp32 partials within half the weight bytes at <= 128 rows; within twice them above,
  // where a half-weight budget left the K/V product 2 splits (32 workgroups) at 256
  // rows and more.
  const int cap = max(1, min((int)((int64_t)K / ((M > 128 ? 1 : 4) * (int64_t)(M > 0 ? M : 1))), K / (2 * BK)));
  constexpr int64_t kFixedSteps = 8;
  const int64_t steps = (K + BK - 1) / BK;
  auto cost = [&](int s) {  // in steps x splits, to compare without division
    const int64_t rounds = ((int64_t)tiles * s + num_cu - 1) / num_cu;
    return rounds * (steps + kFixedSteps * s);
  };
  // candidates: every count up to 8, then multiples of 8 (the XCD-aware decode needs
  // a multiple of 8; below that the activations of a K range are at most a few MB and
  // every XCD reads them whole).  Counts between the powers of two fill a round that
  // they would leave short: the block q/k/v product (48 tiles) takes 5 splits, 240
  // workgroups (26.0 -> 24.7 us per call), the long-context fc product (40 tiles) 6
  // instead of 24 splits in four rounds (its projection 65.1 -> 58.9 us, interleaved A/B).
  int best = 1;
  for (int s = 2; s <= cap; s = s < 8 ? s + 1 : s + 8)
    if (cost(s) * best < cost(best) * s) best = s;  // cost(s) / s < cost(best) / best
  return best;
}

ProjPlan plan_ctx_proj(int n_rows, int k_fc, int hidden, int kv_width, bool has_fc, int num_cu) {
  ProjPlan pl{};
  const int cus = num_cu > 0 ? num_cu : 256;
  const int mtiles = (n_rows + GBM - 1) / GBM;
  pl.fc_small = pl.kv_small = n_rows <= kSkinnyMaxRows;  // skinny weight-streaming kernel
  if (has_fc) {
    const int sp = pl.fc_small ? skinny_splits(hidden, n_rows, k_fc, cus)
                               : split_count(mtiles * ((hidden + GBN - 1) / GBN), n_rows, hidden, k_fc, cus);
    pl.fc_kps = k_per_split(k_fc, sp);
    pl.fc_splits = (k_fc + pl.fc_kps - 1) / pl.fc_kps;  // every split has a non-empty K range
  }
  const int sp = pl.kv_small ? skinny_splits(kv_width, n_rows, hidden, cus)
                             : split_count(mtiles * ((kv_width + GBN - 1) / GBN), n_rows, kv_width, hidden, cus);
  pl.kv_kps = k_per_split(hidden, sp);
  pl.kv_splits = (hidden + pl.kv_kps - 1) / pl.kv_kps;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // word 0: device error mask
  pl.off_fc = off;
  if (has_fc) off = align(off + sizeof(float) * (size_t)pl.fc_splits * n_rows * hidden);
  pl.off_c = off;
  if (has_fc) off = align(off + 2 * (size_t)n_rows * hidden);
  pl.off_kv = off;
  off = align(off + sizeof(float) * (size_t)pl.kv_splits * n_rows * kv_width);
  // Rows of a packed step (skinny path only): the skinny kernel reads 16*MT rows,
  // 32*ceil(rows / 32) up to 128 rows and 256 above.  Rows past n_rows hold whatever the
  // workspace held (zero from pack_rows_kernel); an MFMA output row depends on its own
  // activation row only, and the products of those rows are never stored.
  pl.mp = n_rows <= 128 ? 32 * ((n_rows + 31) / 32) : kSkinnyMaxRows;
  pl.off_cp = off;
  if (pl.kv_small) off = align(off + 2 * (size_t)hidden * pl.mp);
  pl.ws_bytes = off;
  return pl;
}

// The block q/k/v product is shaped like the fc product (many weight rows, few
// activation rows), so it takes the same split rule and tile choice.
QkvPlan plan_block_qkv(int n_rows, int hidden, int n_out, int num_cu) {
  QkvPlan pl{};
  const int cus = num_cu > 0 ? num_cu : 256;
  const int mtiles = (n_rows + GBM - 1) / GBM;
  pl.small = n_rows <= kSkinnyMaxRows;
  const int sp = pl.small ? skinny_splits(n_out, n_rows, hidden, cus)
                          : split_count(mtiles * ((n_out + GBN - 1) / GBN), n_rows, n_out, hidden, cus);
  pl.kps = k_per_split(hidden, sp);
  pl.splits = (hidden + pl.kps - 1) / pl.kps;
  pl.mp = n_rows <= 128 ? 32 * ((n_rows + 31) / 32) : kSkinnyMaxRows;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // word 0: device error mask
  pl.off_part = off;
  off = align(off + sizeof(float) * (size_t)pl.splits * n_rows * n_out);
  pl.ws_bytes = off;  // the product reads its activations in place: no packed copy
  return pl;
}

template <int MT, bool PACKED, int RT>
void launch_skinny_rt(const GemmParams& p, int splits, hipStream_t stream) {
  using SG = SkGeo<MT, RT>;
  dim3 grid(((p.N + SG::ROWS - 1) / SG::ROWS) * splits, 1, 1);
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, PACKED, RT>), grid, dim3(SG::WAVES * 64), 0, stream, p);
}

// The planner splits K for 128-row weight tiles.  Where its tiles times splits fill at
// most half of the CUs (the K/V product at 128 rows: 16 tiles x 8 splits), each
// workgroup takes 64 weight rows instead, so twice the workgroups stream the same
// weights with the same splits (and the same fp32 partials): the batched projection
// 57.6 -> 56.3 us per call (interleaved A/B inside the step, events).
template <int MT, bool PACKED>
void launch_skinny(const GemmParams& p, int splits, hipStream_t stream) {
  const int64_t tiles = (p.N + SK_ROWS - 1) / SK_ROWS;
  if (2 * tiles * splits <= kPlanCUs) launch_skinny_rt<MT, PACKED, 1>(p, splits, stream);
  else launch_skinny_rt<MT, PACKED, SK_RT>(p, splits, stream);
}

// Up to kSkinnyMaxRows rows; activation tiles in pairs of 16 rows.
template <bool PACKED>
void launch_skinny_rows(const GemmParams& c, int splits, hipStream_t stream) {
  switch ((c.m_rows + 31) / 32) {
    case 0:
    case 1: launch_skinny<2, PACKED>(c, splits, stream); break;
    case 2: launch_skinny<4, PACKED>(c, splits, stream); break;
    case 3: launch_skinny<6, PACKED>(c, splits, stream); break;
    case 4: launch_skinny<8, PACKED>(c, splits, stream); break;
    default: launch_skinny<16, PACKED>(c, splits, stream); break;
  }
}

hipError_t launch_gemm_swiglu(const GemmParams& p, hipStream_t stream) {
  if (p.M > kSkinnyMaxRows || p.k_per_split < p.K || p.N != 2 * p.n_b0) return hipErrorInvalidValue;
  GemmParams c = p;
  c.m_off = 0;
  c.m_rows = p.M;
  const dim3 grid((p.n_b0 + 63) / 64), block(SkGeo<8, 2>::WAVES * 64);
  switch ((c.m_rows + 31) / 32) {
    case 0:
    case 1: hipLaunchKernelGGL((gemm_skinny_kernel<2, false, 2, true>), grid, dim3(SkGeo<2, 2>::WAVES * 64), 0, stream, c); break;
    case 2: hipLaunchKernelGGL((gemm_skinny_kernel<4, false, 2, true>), grid, dim3(SkGeo<4, 2>::WAVES * 64), 0, stream, c); break;
    case 3: hipLaunchKernelGGL((gemm_skinny_kernel<6, false, 2, true>), grid, dim3(SkGeo<6, 2>::WAVES * 64), 0, stream, c); break;
    case 4: hipLaunchKernelGGL((gemm_skinny_kernel<8, false, 2, true>), grid, block, 0, stream, c); break;
    default: hipLaunchKernelGGL((gemm_skinny_kernel<16, false, 2, true>), grid, dim3(SkGeo<16, 2>::WAVES * 64), 0, stream, c); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const GemmParams& p, int splits, bool small_m, hipStream_t stream) {
  if (small_m) {
    // All rows in one pass over the weights; activation tiles in pairs of 16 rows
    // (stage loads split evenly over the waves).
    if (p.M > kSkinnyMaxRows) return hipErrorInvalidValue;
    GemmParams c = p;
    c.m_off = 0;
    c.m_rows = p.M;
    if (p.xp) launch_skinny_rows<true>(c, splits, stream);
    else launch_skinny_rows<false>(c, splits, stream);
    return hipGetLastError();
  }
  // Workgroups per XCD: all tiles of its rows of tiles (x, x + 8, ...), or a contiguous
  // run of tiles below 8 rows of tiles.
  const int ntm = (p.M + GBM - 1) / GBM, ntn = (p.N + GBN - 1) / GBN;
  int64_t per_xcd;
  if (ntm >= kNumXcd) {
    per_xcd = (int64_t)((ntm + kNumXcd - 1) / kNumXcd) * ntn;  // rows of the XCD with most
  } else {
    per_xcd = ((int64_t)ntm * ntn + kNumXcd - 1) / kNumXcd;
  }
  const dim3 grid((unsigned)(kNumXcd * per_xcd), (unsigned)splits, 1);
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_pack_rows(const PackParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)(p.K / 64) * p.mp * 8;
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fc_reduce(const FcReduceParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.M * p.N / 4;
  hipLaunchKernelGGL(fc_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_qkv_reduce(const QkvReduceParams& p, hipStream_t stream) {
  const int64_t n4 = (int64_t)p.M * p.N / 4;
  hipLaunchKernelGGL(qkv_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_qkv_rope(const QkvRopeParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.M * (p.N / 8);
  hipLaunchKernelGGL(qkv_rope_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_epilogue(const KvEpilogueParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.M * p.n_kv_heads * (p.head_dim / 8);
  hipLaunchKernelGGL(kv_epilogue_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dflash
