/*
 * dflash.h -- C ABI of the DFlash draft block-attention / greedy-verify hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * Operations (pages cited by title and section):
 *   - context projection: target-layer hidden states, selected by layer id and
 *     concatenated, are projected into the draft's context K/V ("DFlash dual
 *     implementations: PyTorch vs MLX", §4 target hidden states and §2
 *     attention; "dflash-mlx: lossless speculative decoding", section
 *     "block-diffusion draft": the draft reads the target's hidden states);
 *   - dual-source block attention: Q from the 16 block tokens only, K/V =
 *     [context ; block], no causal mask inside the block ("DFlash dual
 *     implementations", §2 attention), RoPE as in Qwen3 (same page, §1);
 *   - greedy verify: target argmax at the 16 block positions, accepted prefix
 *     length sum(cumprod(draft == posterior)), next staged token, commit of
 *     1 + accept tokens and crop of the KV length ("dflash-mlx", "single-forward
 *     verify" steps 6-9 and guarantees 2-3; "DFlash dual implementations", §3);
 *   - around them, the rest of a cycle on the device: the block's own q / k / v
 *     (the attention's inputs, same §2), alone or in one call with the attention
 *     (Q carried unrounded as a bf16 hi/lo pair); the draft-side greedy tokens
 *     at the 15 mask slots ("dflash-mlx", "single-forward verify" steps 3-4); the
 *     rest of a draft layer (RMSNorm, o_proj, SwiGLU MLP: "DFlash dual
 *     implementations", §1); the sliding-window cache (dflash_dims.window, §3);
 *     and the rollback of recurrent state by replaying the accepted steps of an
 *     innovation tape ("dflash-mlx", guarantee 3);
 *   - the block attention once more, for callers that cannot allocate: a form
 *     that takes no workspace (a fixed scratch array inside the library).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller unless a
 *     comment says "host".  The library allocates no memory, never copies
 *     between host and device and never synchronizes: work is enqueued on the
 *     caller's stream and the call returns at once.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16).  Pointers must
 *     be 16-byte aligned; innermost strides are 1 element; row strides given
 *     explicitly must be multiples of 8 elements.
 *   - Every argument is validated on the host BEFORE anything is launched.  On
 *     any error nothing is enqueued and no output is touched.
 *   - Workspaces are caller-owned device buffers of at least the size the
 *     matching *_workspace_size() query returns.  Zero a workspace once before
 *     its first use; every call leaves it fit for the next one.  The block
 *     attention keeps per-(sequence, kv head) arrival counters in it, and the
 *     verify and the draft argmax with 8 or more sequences keep per-sequence
 *     ones.  They sit in a region of fixed size (1 MiB after the 256-byte error
 *     area; at most 8192 counters, hence batch <= 8192 and, for the attention,
 *     batch * n_kv_heads <= 8192) that nothing else is written to, and each
 *     call returns its counters to zero.  So one buffer serves any number of
 *     calls on the same stream, in any order of sizes, as long as each call's
 *     own *_workspace_size() fits in it.  Calls that run concurrently
 *     (different streams) need distinct workspaces.
 *   - Word 0 of every workspace is a sticky device-side error mask
 *     (DFLASH_DEVERR_*): data-dependent faults found by the kernels (a context
 *     length, page id or row position out of range) are clamped or skipped so
 *     no access leaves its buffer, and the fault is OR-ed into this word.  The
 *     library never clears it: zero it once, and read / reset it at will.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define DFLASH_OK               0
#define DFLASH_ERR_NULL        -1  /* a required pointer is NULL */
#define DFLASH_ERR_SHAPE       -2  /* a size is out of range or inconsistent */
#define DFLASH_ERR_ALIGN       -3  /* a pointer or stride is misaligned */
#define DFLASH_ERR_WORKSPACE   -4  /* workspace missing or too small */
#define DFLASH_ERR_CAPACITY    -5  /* cache or RoPE table too small for the request */
#define DFLASH_ERR_UNSUPPORTED -6  /* current device is not gfx950, or a size has no kernel */
#define DFLASH_ERR_LAUNCH      -7  /* the HIP runtime reported an error at launch */

/* ---- device-side error bits (workspace word 0) ------------------------- */
#define DFLASH_DEVERR_CTX_LEN   1u  /* ctx_len[b] < 0 or > max_ctx_len (clamped) */
#define DFLASH_DEVERR_PAGE_ID   2u  /* page-table entry < 0 or >= num_pages (page 0 read instead) */
#define DFLASH_DEVERR_ROW       4u  /* row_seq / row_pos out of range (row's cache write skipped) */
#define DFLASH_DEVERR_MERGE     8u  /* block attention: a split's partial never arrived (bounded
                                      wait gave up; that unit's output is wrong).  Not expected:
                                      reports a broken workspace counter, e.g. a workspace shared
                                      by two calls in flight */
#define DFLASH_DEVERR_XCD      16u  /* a workgroup of a one-launch hand-off (block attention's split
                                      merge, the verify's or draft argmax's accept step at batch >= 8)
                                      ran on another accelerator die (XCD) than the dispatch order
                                      the hand-off relies on.  That call's outputs may be wrong or
                                      stale and its arrival counters may be left non-zero: zero the
                                      whole workspace before reusing it.  Not expected on MI355X */
#define DFLASH_DEVERR_ACCEPT   32u  /* recurrent-state replay: accept_len[b] outside [0, 15] (clamped) */

/* Block of draft tokens: the staged token plus 15 mask slots
 * ("dflash-mlx", "block-diffusion draft"). */
#define DFLASH_BLOCK 16

/* Shapes of the draft attention.  A context cache is either
 *   dense: k_cache / v_cache [batch][n_kv_heads][kv_capacity][head_dim] bf16, or
 *   paged: k_cache / v_cache [num_pages][n_kv_heads][page_size][head_dim] bf16
 *          with page_table [batch][kv_capacity] int32 (page ids; token t of
 *          sequence b lives in page page_table[b][t / page_size], row t % page_size). */
typedef struct dflash_dims {
    int32_t batch;         /* B >= 1 sequences                                   */
    int32_t block;         /* tokens per draft block; must be DFLASH_BLOCK (16)  */
    int32_t n_q_heads;     /* Hq; a multiple of n_kv_heads, Hq / Hkv in [1, 8]    */
    int32_t n_kv_heads;    /* Hkv >= 1                                           */
    int32_t head_dim;      /* d: 64 or 128                                       */
    int32_t hidden;        /* D: draft hidden size, width of the context feature */
    int32_t page_size;     /* 0 = dense cache, 16 = paged cache                  */
    int32_t kv_capacity;   /* dense: token rows per (seq, kv head);
                              paged: page-table columns per sequence             */
    int32_t num_pages;     /* paged: pages in the pool; dense: ignored           */
    float   softmax_scale; /* <= 0 selects 1/sqrt(head_dim)                      */
    int32_t window;        /* 0: the context is every committed position.  W > 0:
                              sliding window -- the context is the last min(L, W)
                              positions and the cache is a ring of W rows per
                              (sequence, kv head): position p lives in row p mod W
                              (dense: W <= kv_capacity; paged: W % 16 == 0 and
                              W / 16 <= kv_capacity, the page table then holding
                              the ring's W / 16 pages).  Violations return
                              DFLASH_ERR_CAPACITY.  "DFlash dual
                              implementations" §3: RotatingKVCache               */
} dflash_dims;

/* Human-readable name of a status code (static string, never NULL). */
const char* dflash_status_str(int status);

/* ABI version: (major << 16) | minor. */
int dflash_version(void);

/* ---- RoPE tables --------------------------------------------------------
 * cos_out / sin_out [max_pos][head_dim/2] fp32, device.  Entry (p, j) holds
 * cos / sin of p * base^(-2j/head_dim), computed in double precision and
 * rounded to fp32 (rotary embedding reused from Qwen3, "DFlash dual
 * implementations" §1).  head_dim even in [2, 256], max_pos >= 1, base > 1. */
int dflash_rope_tables(float base, int32_t head_dim, int32_t max_pos,
                       float* cos_out, float* sin_out, hipStream_t stream);

/* ---- context projection (a1-a3) -----------------------------------------
 * For every row r < n_rows of target hidden states:
 *   X_cat[r] = [x_layers[0][r] | ... | x_layers[n_layers-1][r]]   (n_layers*d_target)
 *   C[r]     = bf16(X_cat[r] W_fc^T)                               (hidden)
 *   K[r]     = bf16(RoPE(C[r] W_k^T, row_pos[r])),  V[r] = bf16(C[r] W_v^T)
 * and K[r], V[r] (n_kv_heads x head_dim each) are written to the context cache
 * of sequence row_seq[r] at token position row_pos[r] (with a sliding window W:
 * ring row row_pos[r] mod W; a call must then not commit two positions of one
 * sequence W or more apart, whose rows would collide).  Rows with row_pos < 0
 * are computed but not written (uncommitted block slots).  fp32 accumulation;
 * K is the bf16 value nearest to the exact rotation of the fp32 product.
 *
 *   x_layers   HOST array of n_layers (1..8) device pointers, each [n_rows][ld_x] bf16
 *   d_target   width of each target layer (multiple of 64); ld_x >= d_target, % 8 == 0
 *   row_seq    [n_rows] int32 in [0, batch);  row_pos [n_rows] int32
 *   w_fc       [hidden][n_layers*d_target] bf16 (nn.Linear layout); NULL means the
 *              rows already are C: then n_layers must be 1, d_target == hidden and
 *              c_out NULL
 *   w_k, w_v   [n_kv_heads*head_dim][hidden] bf16
 *   rope_*     tables from dflash_rope_tables (max_pos rows)
 *   c_out      optional [n_rows][hidden] bf16 copy of C (NULL = not stored)
 *   k_cache, v_cache, page_table: the context cache described by dims
 * A row whose row_seq or row_pos exceeds the cache, or whose row_pos >= max_pos,
 * is skipped and DFLASH_DEVERR_ROW is set.  hidden % 64 == 0. */
size_t dflash_ctx_proj_workspace_size(const dflash_dims* dims, int32_t n_rows,
                                      int32_t n_layers, int32_t d_target);
int dflash_ctx_proj(const dflash_dims* dims, int32_t n_rows,
                    const void* const* x_layers, int32_t n_layers, int32_t d_target,
                    int64_t ld_x, const int32_t* row_seq, const int32_t* row_pos,
                    const void* w_fc, const void* w_k, const void* w_v,
                    const float* rope_cos, const float* rope_sin, int32_t max_pos,
                    void* c_out, void* k_cache, void* v_cache, const int32_t* page_table,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- dual-source block attention (a4-a6) ---------------------------------
 * For sequence b with L = ctx_len[b] committed context tokens and q head h
 * (kv head g = h / (Hq/Hkv)), block rows i = 0..15 sit at positions L + i:
 *   Q   = bf16(RoPE(q_blk[b,i,h]))                                 [16, d]
 *   Keys= [ K_cache[b,g,0:L] ; bf16(RoPE(k_blk[b,:,g])) ]          [L+16, d]
 *   Vals= [ V_cache[b,g,0:L] ; v_blk[b,:,g] ]
 *   out[b,i,h,:] = softmax(Q Keys^T * scale) Vals   over all L+16 keys, no mask.
 * bf16 operands, fp32 accumulation, fp32 output.  The rotated Q and block K are
 * the bf16 values nearest to the exact rotation with the fp32 tables.  With a
 * sliding window W (dims->window) the context rows are the last Lw = min(L, W)
 * positions L-Lw .. L-1, read from ring rows (position mod W); the block still
 * sits at L .. L+15.
 *
 *   q_blk   [B][16][Hq][d] bf16, before RoPE
 *   k_blk   [B][16][Hkv][d] bf16, before RoPE;  v_blk [B][16][Hkv][d] bf16
 *   k_cache, v_cache, page_table: context cache (K already rotated), see dims
 *   ctx_len [B] int32 device; max_ctx_len: host bound >= every ctx_len[b]
 *           (without a window: dense <= kv_capacity, paged <= kv_capacity*page_size)
 *   rope_*  tables with max_pos >= max_ctx_len + 16
 *   out     [B][16][Hq][d] fp32 */
size_t dflash_block_attn_workspace_size(const dflash_dims* dims, int32_t max_ctx_len);
int dflash_block_attn(const dflash_dims* dims, const void* q_blk, const void* k_blk,
                      const void* v_blk, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* ctx_len, int32_t max_ctx_len,
                      const float* rope_cos, const float* rope_sin, int32_t max_pos,
                      float* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- block attention without a workspace ----------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): dflash_block_attn with
 * the workspace replaced by a library-owned scratch array of
 * DFLASH_NOALLOC_SCRATCH_BYTES per device (a static device array, zero at load,
 * held until the process ends).  Same arguments, results and errors as
 * dflash_block_attn, except:
 *   - no workspace arguments; a call whose dflash_block_attn_workspace_size()
 *     exceeds DFLASH_NOALLOC_SCRATCH_BYTES returns DFLASH_ERR_WORKSPACE and
 *     launches nothing (the batched 8 x 8192 and long 32768-token shapes fit;
 *     a ragged batch of 32 x 16384 does not);
 *   - dev_err: optional device pointer to a uint32 (4-byte aligned) into which the
 *     DFLASH_DEVERR_* bits are OR-ed; NULL leaves them in the scratch, unreported;
 *   - the call allocates nothing (no hipMalloc / hipFree, no allocating library
 *     routine).  The first call on a device looks the scratch's address up once.
 * Every call on a device shares that device's scratch: calls that overlap in time
 * on one device (different streams, or threads) race and give wrong results.
 * Serialise them, e.g. on one stream. */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int dflash_block_attn_noalloc(const dflash_dims* dims, const void* q_blk, const void* k_blk,
                              const void* v_blk, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* ctx_len,
                              int32_t max_ctx_len, const float* rope_cos, const float* rope_sin,
                              int32_t max_pos, float* out, uint32_t* dev_err, hipStream_t stream);

/* ---- greedy verify, accept, commit and crop (a7-a9) ----------------------
 * For each sequence b (block == 16):
 *   posterior[b,i] = lowest index of the maximum of logits[b,i,0:vocab]
 *                    (NaN ranks above every number; -0 == +0)
 *   accept_len[b]  = sum_i cumprod_i(block_tokens[b,i+1] == posterior[b,i]),  i < 15
 *   next_token[b]  = posterior[b, accept_len[b]]        (the next staged token)
 *   kv_len_out[b]  = kv_len_in[b] + 1 + accept_len[b]   (staged + accepted drafts)
 *   commit_pos[b,i]= kv_len_in[b] + i if i <= accept_len[b] else -1   (optional)
 *   n_pages[b]     = ceil(kv_len_out[b] / page_size)     (optional, page_size > 0)
 *
 *   logits       [B][16][ld_logits] bf16, ld_logits >= vocab, ld_logits % 8 == 0
 *   block_tokens [B][16] int32: staged token then drafts d_1..d_15
 *   kv_len_in    [B] int32 committed length before the block; kv_len_out may alias it
 *   posterior [B][16], accept_len [B], next_token [B], kv_len_out [B]: int32 outputs
 *   commit_pos   [B][16] int32 or NULL;  n_pages [B] int32 or NULL (needs page_size > 0)
 * vocab in [1, 2^31 - 1).  Results are bit-exact and independent of launch shape. */
size_t dflash_verify_workspace_size(int32_t batch, int32_t block, int32_t vocab);
int dflash_verify_accept(int32_t batch, int32_t block, int32_t vocab,
                         const void* logits, int64_t ld_logits, const int32_t* block_tokens,
                         const int32_t* kv_len_in, int32_t* posterior, int32_t* accept_len,
                         int32_t* next_token, int32_t* kv_len_out, int32_t* commit_pos,
                         int32_t page_size, int32_t* n_pages,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- the block's own q / k / v (inputs of dflash_block_attn) ---------------
 * Q comes from the block tokens only, and the block's K/V join the context's
 * as the second source ("DFlash dual implementations", §2).  One bias-free
 * linear map over the draft's block hidden states, M = 16 * batch rows:
 *   Y = h . w_qkv^T  (fp32 accumulation of bf16 products), rounded to bf16
 *   q_blk = Y[:, 0 : Hq*d], k_blk = Y[:, Hq*d : (Hq+Hkv)*d], v_blk = the rest
 * No RoPE here: dflash_block_attn rotates Q and the block K.
 *
 *   dims       as for dflash_block_attn; uses batch, n_q_heads, n_kv_heads,
 *              head_dim and hidden (a multiple of 64, at most 65536)
 *   h          [16*batch][ld_h] bf16, sequence-major; ld_h >= hidden, ld_h % 8 == 0
 *   w_qkv      [(Hq + 2*Hkv)*d][hidden] bf16, nn.Linear layout: the Hq query
 *              heads' rows, then the Hkv key heads', then the Hkv value heads'
 *   q_blk      [batch][16][Hq][d] bf16 output; k_blk, v_blk [batch][16][Hkv][d]
 * The workspace holds split-K partial sums (h is read in place); it keeps no
 * state between calls.  Results agree with the exact
 * product rounded to bf16 to within one bf16 ulp (fp32 summation order). */
size_t dflash_block_qkv_workspace_size(const dflash_dims* dims);
int dflash_block_qkv(const dflash_dims* dims, const void* h, int64_t ld_h, const void* w_qkv,
                     void* q_blk, void* k_blk, void* v_blk,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- the block's q/k/v and the attention in one call ------------------------
 * dflash_block_qkv followed by dflash_block_attn, with the hand-off between them
 * fused ("DFlash dual implementations", §2: Q from the block tokens only, the
 * block's K/V as the second source).  Per sequence b, block row i at position
 * L + i (L = ctx_len[b]):
 *   q, k, v = h[b,i] . w_qkv^T                     (fp32 accumulation, not rounded)
 *   Q      = RoPE(q)                               (carried as a bf16 pair hi + lo,
 *                                                    ~16 significant bits: no bf16
 *                                                    rounding of q or Q on the way)
 *   K_blk  = bf16(RoPE(k)),  V_blk = bf16(v)       (rounded once)
 *   out    = the attention of dflash_block_attn over [context ; block] (dims->window
 *            honoured), fp32.
 * Three launches on `stream`: the split-K q/k/v product (fp32 partial sums), one
 * kernel that sums the splits and writes Q (hi, lo), K_blk and V_blk, and the
 * attention, which reads Q as hi + lo and K_blk already rotated.  Arguments as for
 * dflash_block_qkv (h, ld_h, w_qkv) and dflash_block_attn (cache, ctx_len,
 * max_ctx_len, rope tables, out).  The workspace
 * (dflash_block_qkv_attn_workspace_size) holds the attention's region, then the
 * partial sums and the q/k/v outputs; zero it once before first use, as for the
 * attention.  A ctx_len outside [0, max_ctx_len] is clamped and reported in the
 * attention's error word (DFLASH_DEVERR_CTX_LEN), as there. */
size_t dflash_block_qkv_attn_workspace_size(const dflash_dims* dims, int32_t max_ctx_len);
int dflash_block_qkv_attn(const dflash_dims* dims, const void* h, int64_t ld_h, const void* w_qkv,
                          const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* ctx_len, int32_t max_ctx_len, const float* rope_cos,
                          const float* rope_sin, int32_t max_pos, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ---- draft-side greedy tokens (the step before the verify) ----------------
 * One draft forward over the block [staged, mask x 15] yields the 15
 * candidate tail tokens ("dflash-mlx: lossless speculative decoding",
 * "single-forward verify" steps 3-4; "block-diffusion draft").  Greedy
 * drafting: the candidate at mask slot i is the argmax of the draft's logits
 * in row i, by the same rule as the verify's posterior.  For each b:
 *   block_tokens[b,i] = lowest index of the maximum of logits[b,i,0:vocab],
 *                       i = 1..15  (NaN ranks above every number; -0 == +0)
 *   block_tokens[b,0] = staged[b]  if staged != NULL, else left unchanged
 *
 *   logits       [B][16][ld_logits] bf16, ld_logits >= vocab, ld_logits % 8 == 0:
 *                the draft's logits over the block; row 0 (the staged slot) is
 *                not read
 *   staged       [B] int32 or NULL, e.g. the verify's next_token of the
 *                previous cycle; must not overlap block_tokens
 *   block_tokens [B][16] int32 output, in the layout dflash_verify_accept reads
 * The workspace is the verify's: at least dflash_verify_workspace_size(batch,
 * block, vocab) bytes, zeroed once; one buffer may serve both calls on one
 * stream.  Errors as for dflash_verify_accept.  Results are bit-exact and
 * independent of launch shape. */
int dflash_draft_argmax(int32_t batch, int32_t block, int32_t vocab,
                        const void* logits, int64_t ld_logits, const int32_t* staged,
                        int32_t* block_tokens, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ---- the rest of a draft layer around the attention ------------------------
 * The draft model reuses Qwen3's RMSNorm and MLP around its attention ("DFlash
 * dual implementations", §1 model definition).  A pre-norm residual layer over
 * the M = 16 * batch block rows (sequence-major), x the layer's input:
 *   n1 = RMSNorm(x; w_in)                 -> dflash_rmsnorm, then dflash_block_qkv
 *   attn = dflash_block_attn(q, k, v, ...)
 *   x1 = x + bf16(attn) W_o^T,  n2 = RMSNorm(x1; w_post)
 *   x_out = x1 + bf16(silu(n2 W_gate^T) * (n2 W_up^T)) W_down^T
 * RMSNorm(x; w) = x / sqrt(mean(x^2) + eps) * w;  silu(g) = g / (1 + exp(-g)).
 * No biases.  Every stored tensor is bf16 (rounded to nearest even), products
 * accumulate in fp32, the RMSNorm factor is computed in fp64. */

/* out[r] = bf16(RMSNorm(x[r]; weight)) for r < rows.
 *   x [rows][ld_x] bf16, weight [hidden] bf16, out [rows][ld_out] bf16;
 *   hidden % 8 == 0, ld_x, ld_out >= hidden and % 8 == 0; eps >= 0.
 * No workspace.  out may equal x only if ld_out == ld_x (rows are independent). */
int dflash_rmsnorm(int32_t rows, int32_t hidden, const void* x, int64_t ld_x, const void* weight,
                   float eps, void* out, int64_t ld_out, hipStream_t stream);

/* o_proj + residual, RMSNorm, SwiGLU MLP + residual (the layer after the attention).
 *   dims          uses batch, n_q_heads, head_dim, hidden (a multiple of 64, <= 16384)
 *   intermediate  I, the MLP width (a multiple of 64, <= 131072)
 *   x             [16*batch][hidden] bf16, the layer's input (the residual)
 *   attn_out      [batch][16][n_q_heads][head_dim] fp32, dflash_block_attn's output
 *   w_o           [hidden][n_q_heads*head_dim] bf16;  w_post_norm [hidden] bf16
 *   w_gate, w_up  [I][hidden] bf16;  w_down [hidden][I] bf16 (nn.Linear layouts)
 *   x_out         [16*batch][hidden] bf16 (must not overlap x)
 * The workspace holds the intermediate tensors and split-K partial sums; it keeps
 * no state between calls. */
size_t dflash_draft_layer_post_workspace_size(const dflash_dims* dims, int32_t intermediate);
int dflash_draft_layer_post(const dflash_dims* dims, int32_t intermediate, const void* x,
                            const float* attn_out, const void* w_o, const void* w_post_norm,
                            const void* w_gate, const void* w_up, const void* w_down, float eps,
                            void* x_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- rollback of recurrent state by tape replay ----------------------------
 * Verifying the block advances a recurrent (GatedDeltaNet) layer's state by all
 * 16 candidate steps; it cannot be cropped like an attention cache.  During the
 * verify a tape of per-step keys, gates and increments is recorded, and after
 * acceptance only the accepted steps are replayed onto the state saved before
 * the block ("dflash-mlx: lossless speculative decoding", guarantee 3;
 * "DFlash dual implementations", §7).  With the gated delta rule (per head,
 * state S [d_v][d_k], S_t = exp(g_t) S_{t-1} + delta_t k_t^T, where the tape's
 * innovation is delta_t = beta_t (v_t - exp(g_t) S_{t-1} k_t)), for each b, h:
 *   S = state_in[b,h];  for t = 0 .. accept_len[b]:
 *       S = exp(g_tape[b,t,h]) * S + delta_tape[b,t,h,:] (x) k_tape[b,t,h,:]
 *   state_out[b,h] = S
 * i.e. the state after the staged token and the accepted drafts (1 + accept_len
 * steps).  fp32 arithmetic.
 *   state_in, state_out [batch][n_heads][d_v][d_k] fp32; state_out == state_in
 *               replays in place (any other overlap is refused)
 *   k_tape      [batch][16][n_heads][d_k] bf16;  g_tape [batch][16][n_heads] fp32
 *   delta_tape  [batch][16][n_heads][d_v] fp32;  accept_len [batch] int32, e.g.
 *               dflash_verify_accept's output
 *   dev_err     optional uint32 (device): DFLASH_DEVERR_ACCEPT is OR-ed in when an
 *               accept_len lies outside [0, 15] (it is clamped)
 * d_k a multiple of 4 in [4, 256], d_v in [1, 4096], batch x n_heads x ceil(d_v / 32) at
 * most 2^24 (else DFLASH_ERR_SHAPE).  No workspace. */
int dflash_gdn_tape_replay(int32_t batch, int32_t n_heads, int32_t d_k, int32_t d_v,
                           const float* state_in, float* state_out, const void* k_tape,
                           const float* g_tape, const float* delta_tape, const int32_t* accept_len,
                           uint32_t* dev_err, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
