// Internal kernel parameter blocks and launchers (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

// Split plans are made for the MI355X CU count so the workspace-size queries
// (which run without a device) and the launches always agree.
constexpr int kPlanCUs = 256;
// Arrival counters live in a region of fixed size at the start of a workspace
// (after the 256-byte error area): one 128-byte line per sequence (verify) or
// per sequence x kv head (attention), for up to kMaxCountSlots of them.  Every
// call's counters are a prefix of that region and no call writes anything else
// there, so a workspace keeps its counters at zero whatever sequence of call
// sizes it serves.
constexpr int kMaxCountSlots = 8192;
constexpr size_t kCountRegionBytes = 128 * (size_t)kMaxCountSlots;

// ---------------------------------------------------------------- verify
constexpr int kVerifyChunk = 8192;  // logits per workgroup (256 threads x 4 x 8)
constexpr int kVerifyCntStride = 32;  // uint32 words per arrival counter (one 128-byte line)

struct VerifyParams {
  const uint16_t* logits;
  int64_t ld;
  int vocab;
  int n_chunks;
  const int32_t* block_tokens;
  const int32_t* kv_len_in;
  int32_t* posterior;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t* kv_len_out;
  int32_t* commit_pos;  // may be null
  int32_t* n_pages;     // may be null
  int32_t page_size;
  uint64_t* part;       // [batch*16*n_chunks] per-chunk keys
  uint32_t* count;      // [batch][kVerifyCntStride] arrival counters (one-kernel form; zero between calls)
  uint32_t* err;        // sticky device error word (workspace word 0)
  uint32_t xcc_mask;    // XCDs of the partition - 1: workgroup i must run on XCD i & xcc_mask
  // draft tokens (launch_draft_argmax only; the verify fields above stay unused there)
  int32_t* draft_block;   // [batch][16]: slots 1..15 written, slot 0 from staged
  const int32_t* staged;  // [batch] or null (slot 0 left as it is)
};
hipError_t launch_verify_accept(const VerifyParams& p, int batch, hipStream_t stream);
hipError_t launch_draft_argmax(const VerifyParams& p, int batch, hipStream_t stream);

// ---------------------------------------------------------------- RoPE tables
hipError_t launch_rope_tables(double base, int head_dim, int max_pos, float* cos_out, float* sin_out,
                              hipStream_t stream);

// ---------------------------------------------------------------- block attention
struct AttnParams {
  const uint16_t* q_blk;
  const uint16_t* q_lo;     // null: q_blk is the pre-RoPE q; else q_blk / q_lo are the rotated Q's
                            // bf16 hi / lo parts and k_blk the rotated block K (fused q/k/v path)
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* ctx_len;
  const float* rope_cos;
  const float* rope_sin;
  float* out;
  float* ws_o;      // [units][n_splits][G][D/16][64 lanes][4] partial outputs
  float* ws_ml;     // [units][n_splits][G][16][2] running max (log2 domain) and sum
  uint32_t* err;    // sticky device error word
  uint32_t* count;  // [units] arrival counters of the fused merge (zero between calls)
  int fused;        // 1: the last split of a unit merges; 0: attn_merge_kernel does
  uint32_t xcc_mask; // XCDs of the partition - 1: workgroup i must run on XCD i & xcc_mask
  int batch, n_q_heads, n_kv_heads;
  int capacity;     // dense rows per (seq, head) | page-table columns
  int num_pages;
  int max_ctx;
  int window;       // > 0: sliding window of this many positions, cache a ring of that many rows
  int kps;          // context keys per split (multiple of 64)
  int n_splits;     // splits per unit at max_ctx
  int n_units;      // batch * n_kv_heads
  float scale_log2; // softmax scale * log2(e)
};
struct AttnPlan {
  int kps;
  int n_splits;
  bool fused;
  size_t ws_bytes;
  size_t off_cnt, off_ml, off_o;
};
AttnPlan plan_block_attn(int batch, int n_q_heads, int n_kv_heads, int head_dim, int max_ctx, int num_cu);
hipError_t launch_block_attn(const AttnParams& p, int head_dim, int group, bool paged, hipStream_t stream);

// ---------------------------------------------------------------- context projection
constexpr int kMaxLayers = 8;

struct GemmParams {
  const uint16_t* a_seg[kMaxLayers];  // A = [seg_0 | seg_1 | ...] along K, each [M][lda]
  int64_t lda;
  int seg_k;                           // K width of one segment (multiple of 64)
  const uint16_t* b0;                  // rows [0, n_b0) of B, each [K]
  const uint16_t* b1;                  // rows [n_b0, N) of B (row index - n_b0)
  int n_b0;
  int M, N, K;
  int k_per_split;                     // multiple of 64
  float* out;                          // [splits][M][N] fp32 partial sums
  const uint16_t* xp;                  // skinny path: A packed as [K/64][mp][64] (64-K steps)
  int mp;                              // rows of a packed step (M rounded up to 32)
  int m_off, m_rows;                   // skinny path: this launch's rows [m_off, m_off + m_rows) of M
  uint16_t* act;                       // SwiGLU epilogue: bf16(silu(B0 row) * B1 row) as [M][n_b0]
};
struct PackParams {
  const uint16_t* a_seg[kMaxLayers];  // as GemmParams
  int64_t lda;
  int seg_k, M, K, mp;
  uint16_t* xp;                        // [K/64][mp][64]; rows >= M are zero
};
hipError_t launch_pack_rows(const PackParams& p, hipStream_t stream);
struct ProjPlan {
  int fc_splits, kv_splits;
  int fc_kps, kv_kps;       // K elements per split (multiples of 64)
  bool fc_small, kv_small;  // small-M tile shape (M <= 128)
  size_t ws_bytes;
  size_t off_fc, off_c, off_kv;
  int mp;                   // skinny path: packed activation rows (M rounded up to 32)
  size_t off_cp;            // skinny path: packed C (the K/V product's activations)
};
ProjPlan plan_ctx_proj(int n_rows, int k_fc, int hidden, int kv_width, bool has_fc, int num_cu);
hipError_t launch_gemm_nt(const GemmParams& p, int splits, bool small_m, hipStream_t stream);
// One-split skinny product of B0 = gate and B1 = up rows (n_b0 each) with the SwiGLU of
// the two results as its epilogue: act = bf16(silu(x w_gate^T) * (x w_up^T)).  M <= 256.
hipError_t launch_gemm_swiglu(const GemmParams& p, hipStream_t stream);

struct FcReduceParams {
  const float* part;   // [splits][M][N]
  int splits, M, N;
  uint16_t* c_buf;     // [M][N] bf16 (row-major; may be null when c_pack is set)
  uint16_t* c_out;     // optional copy
  uint16_t* c_pack;    // optional: C packed as [N/64][mp][64] for the skinny K/V product
  int mp;
};
hipError_t launch_fc_reduce(const FcReduceParams& p, hipStream_t stream);

// Block q/k/v projection: the projection's split-K GEMM over [W_q; W_k; W_v], then a
// reduce that rounds to bf16 and splits the columns into the three outputs.
struct QkvPlan {
  int splits, kps;   // K split count and K elements per split (multiple of 64)
  bool small;        // skinny weight-streaming GEMM (rows <= kSkinnyMaxRows)
  int mp;            // skinny path: packed activation rows
  size_t off_part, ws_bytes;
};
QkvPlan plan_block_qkv(int n_rows, int hidden, int n_out, int num_cu);
struct QkvReduceParams {
  const float* part;   // [splits][M][N], N = nq + 2 nk
  int splits, M, N, nq, nk;
  uint16_t *q, *k, *v; // [M][nq], [M][nk], [M][nk] bf16
};
hipError_t launch_qkv_reduce(const QkvReduceParams& p, hipStream_t stream);

// The block's q/k/v for the attention directly: sum of the splits, then per RoPE pair
// (j, j + d/2) q rotated at the row's block position and kept as a bf16 hi/lo pair, k
// rotated exactly and rounded once to bf16, v rounded to bf16.
struct QkvRopeParams {
  const float* part;         // [splits][M][N], N = nq + 2 nk
  int splits, M, N, nq, nk, head_dim;
  const int32_t* ctx_len;    // [M / 16]: block row i of sequence b at position ctx_len[b] + i
  int max_ctx;
  const float* rope_cos;     // [max_pos][d/2]
  const float* rope_sin;
  uint16_t* q_hi;            // [M][nq] bf16: the rotated q, rounded
  uint16_t* q_lo;            // [M][nq] bf16: what that rounding left, rounded
  uint16_t* k_out;           // [M][nk] bf16: the rotated k
  uint16_t* v_out;           // [M][nk] bf16
  uint32_t* err;
};
hipError_t launch_qkv_rope(const QkvRopeParams& p, hipStream_t stream);

struct KvEpilogueParams {
  const float* part;   // [splits][M][2*Hkv*d]
  int splits, M;
  int n_kv_heads, head_dim;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const float* rope_cos;
  const float* rope_sin;
  int max_pos;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* page_table;
  int batch, page_size, capacity, num_pages;
  int window;          // > 0: position p goes to ring row p mod window
  uint32_t* err;
};
hipError_t launch_kv_epilogue(const KvEpilogueParams& p, hipStream_t stream);

// ---------------------------------------------------------------- draft layer around the attention
struct RmsNormParams {
  const uint16_t* x;
  int64_t ld_x;
  const uint16_t* w;
  float eps;
  uint16_t* out;
  int64_t ld_out;
  int rows, cols;
};
hipError_t launch_rmsnorm(const RmsNormParams& p, hipStream_t stream);

struct LayerPostParams {
  int M, hidden, attn_cols, inter;  // rows (16 B), D, Hq*d, I
  float eps;
  const uint16_t* x;        // [M][D] layer input (residual)
  const float* attn;        // [M][attn_cols] attention output
  const uint16_t* w_o;      // [D][attn_cols]
  const uint16_t* w_post;   // [D]
  const uint16_t* w_gate;   // [I][D]
  const uint16_t* w_up;     // [I][D]
  const uint16_t* w_down;   // [D][I]
  uint16_t* x_out;          // [M][D]
  // workspace pieces
  uint16_t* a_bf16;         // [M][attn_cols]
  float* part_o;            // [splits_o][M][D]
  uint16_t* x1;             // [M][D]
  uint16_t* n2;             // [M][D]
  float* part_gu;           // [splits_gu][M][2I]
  uint16_t* act;            // [M][I]
  float* part_d;            // [splits_d][M][D]
  int splits_o, splits_gu, splits_d;
};
struct LayerPlan {
  QkvPlan o, gu, dn;        // split plans of the three products
  size_t off_a, off_po, off_x1, off_n2, off_pgu, off_act, off_pd, ws_bytes;
};
LayerPlan plan_draft_layer_post(int rows, int hidden, int attn_cols, int inter, int num_cu);
hipError_t launch_draft_layer_post(const LayerPostParams& p, const LayerPlan& pl, hipStream_t stream);

// ---------------------------------------------------------------- recurrent-state tape replay
struct GdnReplayParams {
  int batch, n_heads, dk, dv;
  const float* state_in;     // [B][H][dv][dk] fp32
  float* state_out;          // same layout; may alias state_in
  const uint16_t* k_tape;    // [B][16][H][dk] bf16
  const float* g_tape;       // [B][16][H]
  const float* delta_tape;   // [B][16][H][dv]
  const int32_t* accept_len; // [B]
  uint32_t* err;             // optional sticky error word
};
hipError_t launch_gdn_replay(const GdnReplayParams& p, hipStream_t stream);

}  // namespace dflash
