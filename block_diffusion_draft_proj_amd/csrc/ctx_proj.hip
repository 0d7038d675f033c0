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
// stream, so K is split over workgroups to put ~2 workgroups on every CU; fp32
// partial sums are reduced by small epilogue kernels (bf16 rounding of C; RoPE,
// bf16 rounding and cache scatter of K/V).
#include "common.h"
#include "launch.h"

namespace dflash {

namespace {

// Tile of one workgroup: 128 rows (A / activations) x 64 columns (B / weight
// rows), K consumed in 64-element stages.  Each stage lands in LDS through
// global_load_lds (A tile 16 KB, B tile 8 KB) in a 3-stage ring, so two stages
// are in flight while one feeds the MFMAs; two workgroups fit on a CU.
// Eight waves each own 16 rows x 64 columns of the tile.  The 24 wave-wide
// 1 KB loads of a stage are dealt round-robin (load i to wave i % 8), so the
// weight loads, which miss every cache, are spread over all waves instead of
// queueing behind one wave's memory counter (measured: 2.4x faster than giving
// each wave a contiguous run of loads).
// The weights are read exactly once (non-temporal); the activation tile is
// re-read by every column tile and is left cacheable.
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kGemmWaves = kThreads / kWave;
constexpr int GBM = 128, GBN = 64, GNST = 3;
constexpr int A_TILE = GBM * BK * 2;
constexpr int B_TILE = GBN * BK * 2;
constexpr int G_STAGE = A_TILE + B_TILE;
constexpr int G_LOADS_W = G_STAGE / 1024 / kGemmWaves;  // wave-wide 1 KB loads per wave per stage (3)
static_assert(GBM == 16 * kGemmWaves, "one 16-row MFMA strip per wave");
static_assert(G_STAGE % (1024 * kGemmWaves) == 0, "stage loads split evenly over the waves");

// 128-byte rows (64 bf16 of K); 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7):
// the 16 rows read by one 16-lane MFMA operand group hit distinct banks.
__device__ __forceinline__ int swz_off(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[GNST * G_STAGE];
  const int n0 = blockIdx.x * GBN, m0 = blockIdx.y * GBM, z = blockIdx.z;
  const int kbeg = z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int n_st = (kend - kbeg) / BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const int lrow = lane >> 3, pch = lane & 7;  // one wave-wide load = 8 rows x 128 bytes

  // Rows past M or N are clamped to the last real row: every load is in bounds
  // and the extra results are never stored.
  auto issue = [&](int st) {
    const int k0 = kbeg + st * BK;
    const int seg = k0 / p.seg_k;
    const uint16_t* abase = p.a_seg[seg] + (k0 - seg * p.seg_k);
    char* stage = lds + (st % GNST) * G_STAGE;
#pragma unroll
    for (int i = 0; i < G_LOADS_W; ++i) {
      const int li = i * kGemmWaves + w;  // 0..15: A tile, 16..23: B tile (wave-uniform)
      if (li < A_TILE / 1024) {
        const int row = li * 8 + lrow;
        const int m = min(m0 + row, p.M - 1);
        lds_dma16(abase + (int64_t)m * p.lda + ((pch ^ ((row >> 1) & 7)) << 3), stage + li * 1024);
      } else {
        const int row = (li - A_TILE / 1024) * 8 + lrow;
        const int n = min(n0 + row, p.N - 1);
        const uint16_t* brow = n < p.n_b0 ? p.b0 + (int64_t)n * p.K : p.b1 + (int64_t)(n - p.n_b0) * p.K;
        lds_dma16_nt(brow + k0 + ((pch ^ ((row >> 1) & 7)) << 3), stage + li * 1024);
      }
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < GNST - 1; ++st)
    if (st < n_st) issue(st);
  for (int it = 0; it < n_st; ++it) {
    if (it + 1 < n_st) wait_vmcnt<G_LOADS_W>();  // stage it landed, stage it+1 may still fly
    else wait_vmcnt<0>();
    __syncthreads();
    if (it + GNST - 1 < n_st) issue(it + GNST - 1);
    const char* sa = lds + (it % GNST) * G_STAGE;
    const char* sb = sa + A_TILE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 b[4];
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sa + swz_off(w * 16 + r, ks * 4 + q));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[nt] = *reinterpret_cast<const bf16x8*>(sb + swz_off(nt * 16 + r, ks * 4 + q));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = mfma16x16x32(a, b[nt], acc[nt]);
    }
  }

  // C tile: lane holds column n0 + 16nt + r, rows m0 + 16w + 4q + v.
  float* out = p.out + (int64_t)z * p.M * p.N;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int n = n0 + nt * 16 + r;
    if (n >= p.N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + w * 16 + 4 * q + v;
      if (m < p.M) out[(int64_t)m * p.N + n] = acc[nt][v];
    }
  }
}

// C = bf16(sum over splits): 4 columns per thread.
__global__ __launch_bounds__(256) void fc_reduce_kernel(FcReduceParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int64_t total = (int64_t)p.M * p.N / 4;
  if (i >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(p.part + 4 * i);
  for (int z = 1; z < p.splits; ++z) s += *reinterpret_cast<const f32x4*>(p.part + (int64_t)z * p.M * p.N + 4 * i);
  const u32x2 v = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  *reinterpret_cast<u32x2*>(p.c_buf + 4 * i) = v;
  if (p.c_out) *reinterpret_cast<u32x2*>(p.c_out + 4 * i) = v;
}

// K/V rows: sum splits, rotate K (pairs j, j+d/2) at the row's position, round to
// bf16 and write into the cache.  Thread = (row, kv head, 4 consecutive j < d/2).
__global__ __launch_bounds__(256) void kv_epilogue_kernel(KvEpilogueParams p) {
  const int half = p.head_dim / 2;
  const int per_row = p.n_kv_heads * (half / 4);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.M * per_row) return;
  const int m = (int)(i / per_row);
  const int rem = (int)(i - (int64_t)m * per_row);
  const int hh = rem / (half / 4);
  const int j = (rem - hh * (half / 4)) * 4;
  const int pos = p.row_pos[m];
  if (pos < 0) return;  // uncommitted block slot
  const int seq = p.row_seq[m];
  const bool paged = p.page_size > 0;
  const bool bad = (unsigned)seq >= (unsigned)p.batch || pos >= p.max_pos ||
                   (paged ? (pos >> 4) >= p.capacity : pos >= p.capacity);
  if (bad) {
    set_dev_error(p.err, 4u);
    return;
  }
  int64_t row_off;
  if (paged) {
    const int page = p.page_table[(int64_t)seq * p.capacity + (pos >> 4)];
    if ((unsigned)page >= (unsigned)p.num_pages) {
      set_dev_error(p.err, 2u);
      return;
    }
    row_off = (((int64_t)page * p.n_kv_heads + hh) * 16 + (pos & 15)) * p.head_dim;
  } else {
    row_off = (((int64_t)seq * p.n_kv_heads + hh) * p.capacity + pos) * p.head_dim;
  }
  const int N = 2 * p.n_kv_heads * p.head_dim;
  const int ck = hh * p.head_dim + j;
  const int cv = p.n_kv_heads * p.head_dim + ck;
  const float* base = p.part + (int64_t)m * N;
  f32x4 k0 = *reinterpret_cast<const f32x4*>(base + ck);
  f32x4 k1 = *reinterpret_cast<const f32x4*>(base + ck + half);
  f32x4 v0 = *reinterpret_cast<const f32x4*>(base + cv);
  f32x4 v1 = *reinterpret_cast<const f32x4*>(base + cv + half);
  for (int z = 1; z < p.splits; ++z) {
    const float* bz = base + (int64_t)z * p.M * N;
    k0 += *reinterpret_cast<const f32x4*>(bz + ck);
    k1 += *reinterpret_cast<const f32x4*>(bz + ck + half);
    v0 += *reinterpret_cast<const f32x4*>(bz + cv);
    v1 += *reinterpret_cast<const f32x4*>(bz + cv + half);
  }
  const f32x4 c = *reinterpret_cast<const f32x4*>(p.rope_cos + (int64_t)pos * half + j);
  const f32x4 s = *reinterpret_cast<const f32x4*>(p.rope_sin + (int64_t)pos * half + j);
  f32x4 y0, y1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float a, b;
    rope_pair(k0[e], k1[e], c[e], s[e], a, b);
    y0[e] = a;
    y1[e] = b;
  }
  uint16_t* kd = p.k_cache + row_off;
  uint16_t* vd = p.v_cache + row_off;
  *reinterpret_cast<u32x2*>(kd + j) = (u32x2){pack_bf16x2(y0[0], y0[1]), pack_bf16x2(y0[2], y0[3])};
  *reinterpret_cast<u32x2*>(kd + j + half) = (u32x2){pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
  *reinterpret_cast<u32x2*>(vd + j) = (u32x2){pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3])};
  *reinterpret_cast<u32x2*>(vd + j + half) = (u32x2){pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
}

// Split K so that ~2 workgroups land on every CU, while the fp32 partial sums
// (splits x M x N x 4 bytes, written and read back once) stay under a quarter of
// the weight bytes (N x K x 2) and every split keeps >= 4 stages.
int split_count(int tiles, int M, int K, int target) {
  if (tiles < 1) tiles = 1;
  int splits = (target + tiles - 1) / tiles;
  const int by_traffic = (int)((int64_t)K / (8 * (int64_t)(M > 0 ? M : 1)));
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

ProjPlan plan_ctx_proj(int n_rows, int k_fc, int hidden, int kv_width, bool has_fc, int num_cu) {
  ProjPlan pl{};
  const int target = 2 * (num_cu > 0 ? num_cu : 256);
  const int mtiles = (n_rows + GBM - 1) / GBM;
  pl.fc_small = pl.kv_small = n_rows <= GBM;
  if (has_fc) {
    pl.fc_kps = k_per_split(k_fc, split_count(mtiles * ((hidden + GBN - 1) / GBN), n_rows, k_fc, target));
    pl.fc_splits = (k_fc + pl.fc_kps - 1) / pl.fc_kps;  // every split has a non-empty K range
  }
  pl.kv_kps = k_per_split(hidden, split_count(mtiles * ((kv_width + GBN - 1) / GBN), n_rows, hidden, target));
  pl.kv_splits = (hidden + pl.kv_kps - 1) / pl.kv_kps;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 256;  // word 0: device error mask
  pl.off_fc = off;
  if (has_fc) off = align(off + sizeof(float) * (size_t)pl.fc_splits * n_rows * hidden);
  pl.off_c = off;
  if (has_fc) off = align(off + 2 * (size_t)n_rows * hidden);
  pl.off_kv = off;
  off = align(off + sizeof(float) * (size_t)pl.kv_splits * n_rows * kv_width);
  pl.ws_bytes = off;
  return pl;
}

hipError_t launch_gemm_nt(const GemmParams& p, int splits, bool /*small_m*/, hipStream_t stream) {
  dim3 grid((p.N + GBN - 1) / GBN, (p.M + GBM - 1) / GBM, splits);
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fc_reduce(const FcReduceParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.M * p.N / 4;
  hipLaunchKernelGGL(fc_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_epilogue(const KvEpilogueParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.M * p.n_kv_heads * (p.head_dim / 8);
  hipLaunchKernelGGL(kv_epilogue_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dflash
