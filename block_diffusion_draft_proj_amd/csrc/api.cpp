// C ABI of the DFlash hot path: host-side validation, workspace planning and
// kernel dispatch.  Every check runs before the first HIP call, so invalid
// arguments are reported without touching the device (and are testable on a
// machine without a GPU).  The library keeps no state beyond a per-device
// cache of the architecture check.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <atomic>

#include "../../include/dflash.h"
#include "launch.h"

using namespace dflash;

namespace {

constexpr int kMaxDevices = 64;
// Per device: 0 unknown, 2 unsupported, else 1 + the partition's XCD count
// (1, 2, 4 or 8) in the bits above bit 0.
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Current device must be a gfx950 (MI355X class) part: the kernels use its MFMA
// and bf16 conversion instructions.  On success *xcc_mask is the partition's XCD
// count - 1 (count 1, 2, 4 or 8; 8 if the runtime reports anything else).  With
// round-robin dispatch workgroup i runs on XCD i & xcc_mask, so equal i mod 8 share
// a die; the one-launch hand-offs count arrivals in that die's L2, and their
// kernels check their die against this mask (DFLASH_DEVERR_XCD).
int check_device(uint32_t* xcc_mask = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DFLASH_ERR_UNSUPPORTED;
  if (dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DFLASH_ERR_UNSUPPORTED;
    int n_xcc = 0;
    if (hipDeviceGetAttribute(&n_xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) n_xcc = 0;
    if (n_xcc != 1 && n_xcc != 2 && n_xcc != 4 && n_xcc != 8) n_xcc = 8;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 + 2 * n_xcc : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  if (st == 2) return DFLASH_ERR_UNSUPPORTED;
  if (xcc_mask) *xcc_mask = (uint32_t)(st >> 1) - 1u;
  return DFLASH_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_LAUNCH; }

// Shape checks shared by attention and projection.
int check_cache_dims(const dflash_dims* d) {
  if (!d) return DFLASH_ERR_NULL;
  if (d->batch < 1 || d->batch > (1 << 20)) return DFLASH_ERR_SHAPE;
  if (d->block != DFLASH_BLOCK) return DFLASH_ERR_SHAPE;
  if (d->n_kv_heads < 1 || d->n_kv_heads > 1024) return DFLASH_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if (d->page_size != 0 && d->page_size != 16) return DFLASH_ERR_UNSUPPORTED;
  if (d->kv_capacity < 1) return DFLASH_ERR_SHAPE;
  if (d->page_size > 0 && d->num_pages < 1) return DFLASH_ERR_SHAPE;
  // Sliding window: a ring of `window` rows per (sequence, kv head) inside the
  // capacity; paged rings hold whole pages.
  if (d->window < 0) return DFLASH_ERR_SHAPE;
  if (d->window > 0) {
    if (d->page_size > 0 ? (d->window % 16 || d->window / 16 > d->kv_capacity) : d->window > d->kv_capacity)
      return DFLASH_ERR_CAPACITY;
  }
  return DFLASH_OK;
}

// The attention's sizes (shared by the calls and their workspace queries).
int check_attn_sizes(const dflash_dims* dims, int32_t max_ctx_len) {
  const int st = check_cache_dims(dims);
  if (st != DFLASH_OK) return st;
  if (dims->n_q_heads < dims->n_kv_heads || dims->n_q_heads % dims->n_kv_heads) return DFLASH_ERR_SHAPE;
  if ((int64_t)dims->batch * dims->n_kv_heads > kMaxCountSlots) return DFLASH_ERR_SHAPE;
  if (dims->n_q_heads / dims->n_kv_heads > 8) return DFLASH_ERR_UNSUPPORTED;
  if (max_ctx_len < 0 || max_ctx_len > (1 << 24)) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

// Context keys a call attends per sequence at most: the window bounds them.
int32_t attended_keys(const dflash_dims* d, int32_t max_ctx_len) {
  return d->window > 0 && d->window < max_ctx_len ? d->window : max_ctx_len;
}

}  // namespace

extern "C" {

const char* dflash_status_str(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_NULL: return "required pointer is NULL";
    case DFLASH_ERR_SHAPE: return "size out of range or inconsistent";
    case DFLASH_ERR_ALIGN: return "pointer or stride misaligned (16-byte pointers, strides multiple of 8)";
    case DFLASH_ERR_WORKSPACE: return "workspace missing or too small";
    case DFLASH_ERR_CAPACITY: return "cache or RoPE table too small for the request";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported device (needs gfx950) or size";
    case DFLASH_ERR_LAUNCH: return "HIP runtime reported an error at launch";
  }
  return "unknown status";
}

int dflash_version(void) { return (1 << 16) | 0; }

int dflash_rope_tables(float base, int32_t head_dim, int32_t max_pos, float* cos_out, float* sin_out,
                       hipStream_t stream) {
  if (!cos_out || !sin_out) return DFLASH_ERR_NULL;
  if (!(base > 1.0f) || !isfinite(base)) return DFLASH_ERR_SHAPE;
  if (head_dim < 2 || head_dim > 256 || (head_dim & 1)) return DFLASH_ERR_SHAPE;
  if (max_pos < 1 || (int64_t)max_pos * (head_dim / 2) > (int64_t)1 << 31) return DFLASH_ERR_SHAPE;
  if (!aligned16(cos_out) || !aligned16(sin_out)) return DFLASH_ERR_ALIGN;
  int st = check_device();
  if (st != DFLASH_OK) return st;
  return launch_status(launch_rope_tables((double)base, head_dim, max_pos, cos_out, sin_out, stream));
}

// ------------------------------------------------------------------ verify
// Workspace: word 0 error mask (256 bytes), the per-sequence arrival counters
// (the fixed-size counter region, 128 bytes per sequence), then the chunk keys.
constexpr size_t kVerifyKeysOffset = 256 + kCountRegionBytes;
static_assert(sizeof(uint32_t) * kVerifyCntStride * kMaxCountSlots == kCountRegionBytes, "counter region");

size_t dflash_verify_workspace_size(int32_t batch, int32_t block, int32_t vocab) {
  if (batch < 1 || batch > kMaxCountSlots || block != DFLASH_BLOCK || vocab < 1) return 0;
  const size_t n_chunks = ((size_t)vocab + kVerifyChunk - 1) / kVerifyChunk;
  return kVerifyKeysOffset + sizeof(uint64_t) * (size_t)batch * DFLASH_BLOCK * n_chunks;
}

int dflash_verify_accept(int32_t batch, int32_t block, int32_t vocab, const void* logits, int64_t ld_logits,
                         const int32_t* block_tokens, const int32_t* kv_len_in, int32_t* posterior,
                         int32_t* accept_len, int32_t* next_token, int32_t* kv_len_out, int32_t* commit_pos,
                         int32_t page_size, int32_t* n_pages, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!logits || !block_tokens || !kv_len_in || !posterior || !accept_len || !next_token || !kv_len_out)
    return DFLASH_ERR_NULL;
  if (batch < 1 || batch > kMaxCountSlots || block != DFLASH_BLOCK || vocab < 1 || vocab == 0x7fffffff)
    return DFLASH_ERR_SHAPE;
  if (ld_logits < vocab) return DFLASH_ERR_SHAPE;
  if (page_size < 0 || (n_pages && page_size == 0)) return DFLASH_ERR_SHAPE;
  if ((ld_logits & 7) || !aligned16(logits)) return DFLASH_ERR_ALIGN;
  const int64_t n_chunks = ((int64_t)vocab + kVerifyChunk - 1) / kVerifyChunk;
  if ((int64_t)batch * DFLASH_BLOCK * n_chunks > 0x7fffffffLL) return DFLASH_ERR_SHAPE;
  const size_t need = dflash_verify_workspace_size(batch, block, vocab);
  if (!workspace || workspace_bytes < need) return DFLASH_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DFLASH_ERR_ALIGN;
  uint32_t xcc_mask = 0;
  int st = check_device(&xcc_mask);
  if (st != DFLASH_OK) return st;
  char* ws = static_cast<char*>(workspace);
  VerifyParams p{};
  p.err = reinterpret_cast<uint32_t*>(ws);
  p.xcc_mask = xcc_mask;
  p.logits = static_cast<const uint16_t*>(logits);
  p.ld = ld_logits;
  p.vocab = vocab;
  p.n_chunks = (int)n_chunks;
  p.block_tokens = block_tokens;
  p.kv_len_in = kv_len_in;
  p.posterior = posterior;
  p.accept_len = accept_len;
  p.next_token = next_token;
  p.kv_len_out = kv_len_out;
  p.commit_pos = commit_pos;
  p.n_pages = n_pages;
  p.page_size = page_size;
  p.part = reinterpret_cast<uint64_t*>(ws + kVerifyKeysOffset);
  p.count = reinterpret_cast<uint32_t*>(ws + 256);
  return launch_status(launch_verify_accept(p, batch, stream));
}

int dflash_draft_argmax(int32_t batch, int32_t block, int32_t vocab, const void* logits, int64_t ld_logits,
                        const int32_t* staged, int32_t* block_tokens, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!logits || !block_tokens) return DFLASH_ERR_NULL;
  if (batch < 1 || batch > kMaxCountSlots || block != DFLASH_BLOCK || vocab < 1 || vocab == 0x7fffffff)
    return DFLASH_ERR_SHAPE;
  if (ld_logits < vocab) return DFLASH_ERR_SHAPE;
  if ((ld_logits & 7) || !aligned16(logits)) return DFLASH_ERR_ALIGN;
  const int64_t n_chunks = ((int64_t)vocab + kVerifyChunk - 1) / kVerifyChunk;
  if ((int64_t)batch * DFLASH_BLOCK * n_chunks > 0x7fffffffLL) return DFLASH_ERR_SHAPE;
  const size_t need = dflash_verify_workspace_size(batch, block, vocab);
  if (!workspace || workspace_bytes < need) return DFLASH_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DFLASH_ERR_ALIGN;
  uint32_t xcc_mask = 0;
  int st = check_device(&xcc_mask);
  if (st != DFLASH_OK) return st;
  char* ws = static_cast<char*>(workspace);
  VerifyParams p{};
  p.err = reinterpret_cast<uint32_t*>(ws);
  p.xcc_mask = xcc_mask;
  p.logits = static_cast<const uint16_t*>(logits);
  p.ld = ld_logits;
  p.vocab = vocab;
  p.n_chunks = (int)n_chunks;
  p.part = reinterpret_cast<uint64_t*>(ws + kVerifyKeysOffset);
  p.count = reinterpret_cast<uint32_t*>(ws + 256);
  p.draft_block = block_tokens;
  p.staged = staged;
  return launch_status(launch_draft_argmax(p, batch, stream));
}

// ------------------------------------------------------------------ block q/k/v
static int check_qkv_dims(const dflash_dims* dims) {
  const int st = check_cache_dims(dims);
  if (st != DFLASH_OK) return st;
  if (dims->n_q_heads < dims->n_kv_heads || dims->n_q_heads % dims->n_kv_heads) return DFLASH_ERR_SHAPE;
  if (dims->n_q_heads > 1024) return DFLASH_ERR_SHAPE;
  if (dims->hidden < 64 || dims->hidden % 64 || dims->hidden > (1 << 16)) return DFLASH_ERR_SHAPE;
  if ((int64_t)dims->batch * DFLASH_BLOCK > (1 << 22)) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

size_t dflash_block_qkv_workspace_size(const dflash_dims* dims) {
  if (check_qkv_dims(dims) != DFLASH_OK) return 0;
  const int n_out = (dims->n_q_heads + 2 * dims->n_kv_heads) * dims->head_dim;
  return plan_block_qkv(dims->batch * DFLASH_BLOCK, dims->hidden, n_out, kPlanCUs).ws_bytes;
}

int dflash_block_qkv(const dflash_dims* dims, const void* h, int64_t ld_h, const void* w_qkv, void* q_blk,
                     void* k_blk, void* v_blk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_qkv_dims(dims);
  if (st != DFLASH_OK) return st;
  if (!h || !w_qkv || !q_blk || !k_blk || !v_blk) return DFLASH_ERR_NULL;
  if (ld_h < dims->hidden) return DFLASH_ERR_SHAPE;
  if (ld_h & 7) return DFLASH_ERR_ALIGN;
  const void* ptrs[] = {h, w_qkv, q_blk, k_blk, v_blk};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DFLASH_ERR_ALIGN;
  const int M = dims->batch * DFLASH_BLOCK;
  const int nq = dims->n_q_heads * dims->head_dim, nk = dims->n_kv_heads * dims->head_dim;
  const int n_out = nq + 2 * nk;
  const QkvPlan pl = plan_block_qkv(M, dims->hidden, n_out, kPlanCUs);
  if (!workspace || workspace_bytes < pl.ws_bytes) return DFLASH_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DFLASH_ERR_ALIGN;
  st = check_device();
  if (st != DFLASH_OK) return st;
  char* ws = static_cast<char*>(workspace);
  GemmParams g{};
  g.a_seg[0] = static_cast<const uint16_t*>(h);
  g.lda = ld_h;
  g.seg_k = dims->hidden;
  // g.xp stays null: the skinny product reads h in place (one segment, rows ld_h apart)
  g.b0 = static_cast<const uint16_t*>(w_qkv);
  g.b1 = g.b0;
  g.n_b0 = n_out;
  g.M = M;
  g.N = n_out;
  g.K = dims->hidden;
  g.k_per_split = pl.kps;
  g.out = reinterpret_cast<float*>(ws + pl.off_part);
  if (launch_gemm_nt(g, pl.splits, pl.small, stream) != hipSuccess) return DFLASH_ERR_LAUNCH;
  QkvReduceParams r{};
  r.part = g.out;
  r.splits = pl.splits;
  r.M = M;
  r.N = n_out;
  r.nq = nq;
  r.nk = nk;
  r.q = static_cast<uint16_t*>(q_blk);
  r.k = static_cast<uint16_t*>(k_blk);
  r.v = static_cast<uint16_t*>(v_blk);
  return launch_status(launch_qkv_reduce(r, stream));
}

// ------------------------------------------------------------------ block attention
size_t dflash_block_attn_workspace_size(const dflash_dims* dims, int32_t max_ctx_len) {
  if (check_attn_sizes(dims, max_ctx_len) != DFLASH_OK) return 0;
  return plan_block_attn(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                         attended_keys(dims, max_ctx_len), kPlanCUs)
      .ws_bytes;
}

}  // extern "C"

namespace {

// Validation, planning and launch of the block attention on workspace `ws` of
// `ws_bytes` bytes; `err` is the device error word (word 0 of ws when null).
int block_attn_run(const dflash_dims* dims, const void* q_blk, const void* k_blk, const void* v_blk,
                   const void* k_cache, const void* v_cache, const int32_t* page_table, const int32_t* ctx_len,
                   int32_t max_ctx_len, const float* rope_cos, const float* rope_sin, int32_t max_pos, float* out,
                   char* ws, size_t ws_bytes, uint32_t* err, char* (*scratch_of_device)(), hipStream_t stream,
                   const void* q_lo = nullptr, bool launch = true) {
  int st = check_cache_dims(dims);
  if (st != DFLASH_OK) return st;
  if (!q_blk || !k_blk || !v_blk || !k_cache || !v_cache || !ctx_len || !rope_cos || !rope_sin || !out)
    return DFLASH_ERR_NULL;
  if (dims->page_size > 0 && !page_table) return DFLASH_ERR_NULL;
  st = check_attn_sizes(dims, max_ctx_len);
  if (st != DFLASH_OK) return st;
  const int group = dims->n_q_heads / dims->n_kv_heads;
  const int64_t cap_tokens =
      dims->page_size > 0 ? (int64_t)dims->kv_capacity * dims->page_size : (int64_t)dims->kv_capacity;
  if (dims->window == 0 && max_ctx_len > cap_tokens) return DFLASH_ERR_CAPACITY;
  if ((int64_t)max_pos < (int64_t)max_ctx_len + DFLASH_BLOCK) return DFLASH_ERR_CAPACITY;
  const void* ptrs[] = {q_blk, k_blk, v_blk, k_cache, v_cache, rope_cos, rope_sin, out};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DFLASH_ERR_ALIGN;
  if (err && (reinterpret_cast<uintptr_t>(err) & 3u)) return DFLASH_ERR_ALIGN;
  const AttnPlan pl = plan_block_attn(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                                      attended_keys(dims, max_ctx_len), kPlanCUs);
  if ((!ws && !scratch_of_device) || ws_bytes < pl.ws_bytes) return DFLASH_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return DFLASH_ERR_ALIGN;
  const int64_t grid = (int64_t)8 * pl.n_splits * (((int64_t)dims->batch * dims->n_kv_heads + 7) / 8);
  if (grid > 0x7fffffffLL) return DFLASH_ERR_SHAPE;
  uint32_t xcc_mask = 0;
  st = check_device(&xcc_mask);
  if (st != DFLASH_OK || !launch) return st;
  if (!ws) {
    ws = scratch_of_device();
    if (!ws) return DFLASH_ERR_LAUNCH;
  }
  AttnParams p{};
  p.xcc_mask = xcc_mask;
  p.q_blk = static_cast<const uint16_t*>(q_blk);
  p.q_lo = static_cast<const uint16_t*>(q_lo);
  p.k_blk = static_cast<const uint16_t*>(k_blk);
  p.v_blk = static_cast<const uint16_t*>(v_blk);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.page_table = page_table;
  p.ctx_len = ctx_len;
  p.rope_cos = rope_cos;
  p.rope_sin = rope_sin;
  p.out = out;
  p.ws_o = reinterpret_cast<float*>(ws + pl.off_o);
  p.ws_ml = reinterpret_cast<float*>(ws + pl.off_ml);
  p.err = err ? err : reinterpret_cast<uint32_t*>(ws);
  p.count = reinterpret_cast<uint32_t*>(ws + pl.off_cnt);
  p.fused = pl.fused ? 1 : 0;
  p.batch = dims->batch;
  p.n_q_heads = dims->n_q_heads;
  p.n_kv_heads = dims->n_kv_heads;
  p.capacity = dims->kv_capacity;
  p.num_pages = dims->page_size > 0 ? dims->num_pages : 0;
  p.max_ctx = max_ctx_len;
  p.window = dims->window;
  p.kps = pl.kps;
  p.n_splits = pl.n_splits;
  p.n_units = dims->batch * dims->n_kv_heads;
  const double scale = dims->softmax_scale > 0.f ? (double)dims->softmax_scale : 1.0 / sqrt((double)dims->head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634);
  return launch_status(launch_block_attn(p, dims->head_dim, group, dims->page_size > 0, stream));
}

// Scratch of the allocation-free attention entry point: one array per device,
// zero at load (the arrival counters must start at zero; every call leaves them
// at zero), held until the process ends.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = DFLASH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
std::atomic<char*> g_scratch_ptr[kMaxDevices];

char* scratch_of_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  char* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    ptr = static_cast<char*>(addr);
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // same value from any racing thread
  }
  return ptr;
}

}  // namespace

extern "C" {

int dflash_block_attn(const dflash_dims* dims, const void* q_blk, const void* k_blk, const void* v_blk,
                      const void* k_cache, const void* v_cache, const int32_t* page_table, const int32_t* ctx_len,
                      int32_t max_ctx_len, const float* rope_cos, const float* rope_sin, int32_t max_pos,
                      float* out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return block_attn_run(dims, q_blk, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, max_ctx_len, rope_cos,
                        rope_sin, max_pos, out, static_cast<char*>(workspace), workspace_bytes, nullptr, nullptr,
                        stream);
}

int dflash_block_attn_noalloc(const dflash_dims* dims, const void* q_blk, const void* k_blk, const void* v_blk,
                              const void* k_cache, const void* v_cache, const int32_t* page_table,
                              const int32_t* ctx_len, int32_t max_ctx_len, const float* rope_cos,
                              const float* rope_sin, int32_t max_pos, float* out, uint32_t* dev_err,
                              hipStream_t stream) {
  return block_attn_run(dims, q_blk, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, max_ctx_len, rope_cos,
                        rope_sin, max_pos, out, nullptr, kNoAllocScratchBytes, dev_err, scratch_of_current_device,
                        stream);
}

// ------------------------------------------------------------------ context projection
// The projection's sizes (shared by the call and its workspace query): rows, layers,
// and the two widths, so that every product below stays far inside int32.
static int check_proj_sizes(const dflash_dims* dims, int32_t n_rows, int32_t n_layers, int32_t d_target) {
  const int st = check_cache_dims(dims);
  if (st != DFLASH_OK) return st;
  if (n_rows < 0 || n_rows > (1 << 22)) return DFLASH_ERR_SHAPE;
  if (n_layers < 1 || n_layers > kMaxLayers) return DFLASH_ERR_SHAPE;
  if (dims->hidden < 64 || dims->hidden % 64 || dims->hidden > (1 << 16)) return DFLASH_ERR_SHAPE;
  if (d_target < 64 || d_target % 64 || d_target > (1 << 16)) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

size_t dflash_ctx_proj_workspace_size(const dflash_dims* dims, int32_t n_rows, int32_t n_layers, int32_t d_target) {
  if (check_proj_sizes(dims, n_rows, n_layers, d_target) != DFLASH_OK) return 0;
  // Planned for the fc path; the same size also serves a call without fc.
  return plan_ctx_proj(n_rows, n_layers * d_target, dims->hidden, 2 * dims->n_kv_heads * dims->head_dim, true,
                       kPlanCUs)
      .ws_bytes;
}

int dflash_ctx_proj(const dflash_dims* dims, int32_t n_rows, const void* const* x_layers, int32_t n_layers,
                    int32_t d_target, int64_t ld_x, const int32_t* row_seq, const int32_t* row_pos,
                    const void* w_fc, const void* w_k, const void* w_v, const float* rope_cos,
                    const float* rope_sin, int32_t max_pos, void* c_out, void* k_cache, void* v_cache,
                    const int32_t* page_table, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_cache_dims(dims);
  if (st != DFLASH_OK) return st;
  if (!x_layers || !row_seq || !row_pos || !w_k || !w_v || !rope_cos || !rope_sin || !k_cache || !v_cache)
    return DFLASH_ERR_NULL;
  if (dims->page_size > 0 && !page_table) return DFLASH_ERR_NULL;
  st = check_proj_sizes(dims, n_rows, n_layers, d_target);
  if (st != DFLASH_OK) return st;
  if (ld_x < d_target) return DFLASH_ERR_SHAPE;
  if (!w_fc && (n_layers != 1 || d_target != dims->hidden || c_out)) return DFLASH_ERR_SHAPE;
  if (max_pos < 1) return DFLASH_ERR_CAPACITY;
  if (ld_x & 7) return DFLASH_ERR_ALIGN;
  for (int l = 0; l < n_layers; ++l) {
    if (!x_layers[l]) return DFLASH_ERR_NULL;
    if (!aligned16(x_layers[l])) return DFLASH_ERR_ALIGN;
  }
  const void* ptrs[] = {w_k, w_v, rope_cos, rope_sin, k_cache, v_cache};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DFLASH_ERR_ALIGN;
  if ((w_fc && !aligned16(w_fc)) || (c_out && !aligned16(c_out))) return DFLASH_ERR_ALIGN;
  const bool has_fc = w_fc != nullptr;
  const int kv_width = 2 * dims->n_kv_heads * dims->head_dim;
  const int k_fc = n_layers * d_target;
  const ProjPlan pl = plan_ctx_proj(n_rows, k_fc, dims->hidden, kv_width, true, kPlanCUs);
  if (!workspace || workspace_bytes < pl.ws_bytes) return DFLASH_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DFLASH_ERR_ALIGN;
  if (n_rows == 0) return DFLASH_OK;
  st = check_device();
  if (st != DFLASH_OK) return st;

  char* ws = static_cast<char*>(workspace);
  const uint16_t* c_src;
  int64_t ld_c;
  uint16_t* c_pack = pl.kv_small ? reinterpret_cast<uint16_t*>(ws + pl.off_cp) : nullptr;
  if (has_fc) {
    GemmParams g{};
    for (int l = 0; l < n_layers; ++l) g.a_seg[l] = static_cast<const uint16_t*>(x_layers[l]);
    g.lda = ld_x;
    g.seg_k = d_target;
    // g.xp stays null: the skinny product reads the layers' rows in place
    g.b0 = static_cast<const uint16_t*>(w_fc);
    g.b1 = g.b0;
    g.n_b0 = dims->hidden;
    g.M = n_rows;
    g.N = dims->hidden;
    g.K = k_fc;
    g.k_per_split = pl.fc_kps;
    g.out = reinterpret_cast<float*>(ws + pl.off_fc);
    hipError_t e = launch_gemm_nt(g, pl.fc_splits, pl.fc_small, stream);
    if (e != hipSuccess) return DFLASH_ERR_LAUNCH;
    FcReduceParams r{};
    r.part = g.out;
    r.splits = pl.fc_splits;
    r.M = n_rows;
    r.N = dims->hidden;
    r.c_buf = pl.kv_small ? nullptr : reinterpret_cast<uint16_t*>(ws + pl.off_c);
    r.c_out = static_cast<uint16_t*>(c_out);
    r.c_pack = c_pack;
    r.mp = pl.mp;
    e = launch_fc_reduce(r, stream);
    if (e != hipSuccess) return DFLASH_ERR_LAUNCH;
    c_src = r.c_buf;
    ld_c = dims->hidden;
  } else {
    c_src = static_cast<const uint16_t*>(x_layers[0]);
    ld_c = ld_x;
    if (c_pack) {
      PackParams pk{};
      pk.a_seg[0] = c_src;
      pk.lda = ld_x;
      pk.seg_k = dims->hidden;
      pk.M = n_rows;
      pk.K = dims->hidden;
      pk.mp = pl.mp;
      pk.xp = c_pack;
      if (launch_pack_rows(pk, stream) != hipSuccess) return DFLASH_ERR_LAUNCH;
    }
  }
  GemmParams g{};
  g.xp = c_pack;
  g.mp = pl.mp;
  g.a_seg[0] = c_src;
  g.lda = ld_c;
  g.seg_k = dims->hidden;
  g.b0 = static_cast<const uint16_t*>(w_k);
  g.b1 = static_cast<const uint16_t*>(w_v);
  g.n_b0 = dims->n_kv_heads * dims->head_dim;
  g.M = n_rows;
  g.N = kv_width;
  g.K = dims->hidden;
  g.k_per_split = pl.kv_kps;
  g.out = reinterpret_cast<float*>(ws + pl.off_kv);
  hipError_t e = launch_gemm_nt(g, pl.kv_splits, pl.kv_small, stream);
  if (e != hipSuccess) return DFLASH_ERR_LAUNCH;
  KvEpilogueParams k{};
  k.part = g.out;
  k.splits = pl.kv_splits;
  k.M = n_rows;
  k.n_kv_heads = dims->n_kv_heads;
  k.head_dim = dims->head_dim;
  k.row_seq = row_seq;
  k.row_pos = row_pos;
  k.rope_cos = rope_cos;
  k.rope_sin = rope_sin;
  k.max_pos = max_pos;
  k.k_cache = static_cast<uint16_t*>(k_cache);
  k.v_cache = static_cast<uint16_t*>(v_cache);
  k.page_table = page_table;
  k.batch = dims->batch;
  k.page_size = dims->page_size;
  k.capacity = dims->kv_capacity;
  k.num_pages = dims->page_size > 0 ? dims->num_pages : 0;
  k.window = dims->window;
  k.err = reinterpret_cast<uint32_t*>(ws);
  return launch_status(launch_kv_epilogue(k, stream));
}

// ------------------------------------------------------------------ draft layer around the attention
int dflash_rmsnorm(int32_t rows, int32_t hidden, const void* x, int64_t ld_x, const void* weight, float eps,
                   void* out, int64_t ld_out, hipStream_t stream) {
  if (!x || !weight || !out) return DFLASH_ERR_NULL;
  if (rows < 0 || rows > (1 << 24) || hidden < 8 || hidden % 8 || hidden > (1 << 20)) return DFLASH_ERR_SHAPE;
  if (ld_x < hidden || ld_out < hidden || !(eps >= 0.f) || !isfinite(eps)) return DFLASH_ERR_SHAPE;
  if ((ld_x & 7) || (ld_out & 7) || !aligned16(x) || !aligned16(weight) || !aligned16(out)) return DFLASH_ERR_ALIGN;
  if (rows == 0) return DFLASH_OK;
  const int st = check_device();
  if (st != DFLASH_OK) return st;
  RmsNormParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.ld_x = ld_x;
  p.w = static_cast<const uint16_t*>(weight);
  p.eps = eps;
  p.out = static_cast<uint16_t*>(out);
  p.ld_out = ld_out;
  p.rows = rows;
  p.cols = hidden;
  return launch_status(launch_rmsnorm(p, stream));
}

static int check_layer_dims(const dflash_dims* dims, int32_t intermediate) {
  if (!dims) return DFLASH_ERR_NULL;
  if (dims->batch < 1 || (int64_t)dims->batch * DFLASH_BLOCK > (1 << 22) || dims->block != DFLASH_BLOCK)
    return DFLASH_ERR_SHAPE;
  if (dims->n_q_heads < 1 || dims->n_q_heads > 1024) return DFLASH_ERR_SHAPE;
  if (dims->head_dim != 64 && dims->head_dim != 128) return DFLASH_ERR_UNSUPPORTED;
  if (dims->hidden < 64 || dims->hidden % 64 || dims->hidden > 16384) return DFLASH_ERR_SHAPE;
  if (intermediate < 64 || intermediate % 64 || intermediate > (1 << 17)) return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}

size_t dflash_draft_layer_post_workspace_size(const dflash_dims* dims, int32_t intermediate) {
  if (check_layer_dims(dims, intermediate) != DFLASH_OK) return 0;
  return plan_draft_layer_post(dims->batch * DFLASH_BLOCK, dims->hidden, dims->n_q_heads * dims->head_dim,
                               intermediate, kPlanCUs)
      .ws_bytes;
}

int dflash_draft_layer_post(const dflash_dims* dims, int32_t intermediate, const void* x, const float* attn_out,
                            const void* w_o, const void* w_post_norm, const void* w_gate, const void* w_up,
                            const void* w_down, float eps, void* x_out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  int st = check_layer_dims(dims, intermediate);
  if (st != DFLASH_OK) return st;
  if (!x || !attn_out || !w_o || !w_post_norm || !w_gate || !w_up || !w_down || !x_out) return DFLASH_ERR_NULL;
  if (!(eps >= 0.f) || !isfinite(eps)) return DFLASH_ERR_SHAPE;
  const void* ptrs[] = {x, attn_out, w_o, w_post_norm, w_gate, w_up, w_down, x_out};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DFLASH_ERR_ALIGN;
  const int M = dims->batch * DFLASH_BLOCK, D = dims->hidden, A = dims->n_q_heads * dims->head_dim;
  const LayerPlan pl = plan_draft_layer_post(M, D, A, intermediate, kPlanCUs);
  if (!workspace || workspace_bytes < pl.ws_bytes) return DFLASH_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DFLASH_ERR_ALIGN;
  st = check_device();
  if (st != DFLASH_OK) return st;
  char* ws = static_cast<char*>(workspace);
  LayerPostParams p{};
  p.M = M;
  p.hidden = D;
  p.attn_cols = A;
  p.inter = intermediate;
  p.eps = eps;
  p.x = static_cast<const uint16_t*>(x);
  p.attn = attn_out;
  p.w_o = static_cast<const uint16_t*>(w_o);
  p.w_post = static_cast<const uint16_t*>(w_post_norm);
  p.w_gate = static_cast<const uint16_t*>(w_gate);
  p.w_up = static_cast<const uint16_t*>(w_up);
  p.w_down = static_cast<const uint16_t*>(w_down);
  p.x_out = static_cast<uint16_t*>(x_out);
  p.a_bf16 = reinterpret_cast<uint16_t*>(ws + pl.off_a);
  p.part_o = reinterpret_cast<float*>(ws + pl.off_po);
  p.x1 = reinterpret_cast<uint16_t*>(ws + pl.off_x1);
  p.n2 = reinterpret_cast<uint16_t*>(ws + pl.off_n2);
  p.part_gu = reinterpret_cast<float*>(ws + pl.off_pgu);
  p.act = reinterpret_cast<uint16_t*>(ws + pl.off_act);
  p.part_d = reinterpret_cast<float*>(ws + pl.off_pd);
  p.splits_o = pl.o.splits;
  p.splits_gu = pl.gu.splits;
  p.splits_d = pl.dn.splits;
  return launch_status(launch_draft_layer_post(p, pl, stream));
}

// ------------------------------------------------------------------ recurrent-state tape replay
int dflash_gdn_tape_replay(int32_t batch, int32_t n_heads, int32_t d_k, int32_t d_v, const float* state_in,
                           float* state_out, const void* k_tape, const float* g_tape, const float* delta_tape,
                           const int32_t* accept_len, uint32_t* dev_err, hipStream_t stream) {
  if (!state_in || !state_out || !k_tape || !g_tape || !delta_tape || !accept_len) return DFLASH_ERR_NULL;
  if (batch < 1 || n_heads < 1 || (int64_t)batch * n_heads > (1 << 24)) return DFLASH_ERR_SHAPE;
  if (d_k < 4 || d_k > 256 || d_k % 4 || d_v < 1 || d_v > 4096) return DFLASH_ERR_SHAPE;
  // one workgroup of 256 threads per 32 state rows: the grid's thread count fits 32 bits
  if ((int64_t)batch * n_heads * ((d_v + 31) / 32) > (1 << 24)) return DFLASH_ERR_SHAPE;
  const void* ptrs[] = {state_in, state_out, k_tape, g_tape, delta_tape};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return DFLASH_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(accept_len) & 3u) || (reinterpret_cast<uintptr_t>(dev_err) & 3u))
    return DFLASH_ERR_ALIGN;
  // The state is replayed in place when state_out == state_in; partial overlap is not allowed.
  const size_t state_bytes = sizeof(float) * (size_t)batch * n_heads * d_v * d_k;
  const char* si = reinterpret_cast<const char*>(state_in);
  const char* so = reinterpret_cast<const char*>(state_out);
  if (si != so && si < so + state_bytes && so < si + state_bytes) return DFLASH_ERR_SHAPE;
  const int st = check_device();
  if (st != DFLASH_OK) return st;
  GdnReplayParams p{};
  p.batch = batch;
  p.n_heads = n_heads;
  p.dk = d_k;
  p.dv = d_v;
  p.state_in = state_in;
  p.state_out = state_out;
  p.k_tape = static_cast<const uint16_t*>(k_tape);
  p.g_tape = g_tape;
  p.delta_tape = delta_tape;
  p.accept_len = accept_len;
  p.err = dev_err;
  return launch_status(launch_gdn_replay(p, stream));
}

// ------------------------------------------------------------------ fused block q/k/v -> attention
// Workspace: the attention's (error word, counter region, split partials), then the
// q/k/v product's partial tiles and its outputs (Q hi, Q lo, rotated K, V).  The two
// kernels run one after the other and both leave their counters at zero, so they share
// the counter region.
struct FusedPlan {
  QkvPlan qkv;
  AttnPlan attn;
  size_t off_part, off_qhi, off_qlo, off_k, off_v, ws_bytes;
};

// Workspace: the attention's own region first (its error word and counters at the
// start), then the q/k/v product's fp32 split partials and the attention's inputs.
static FusedPlan plan_fused(const dflash_dims* dims, int32_t max_ctx_len) {
  FusedPlan f{};
  const int M = dims->batch * DFLASH_BLOCK;
  const int nq = dims->n_q_heads * dims->head_dim, nk = dims->n_kv_heads * dims->head_dim;
  const int n_out = nq + 2 * nk;
  f.qkv = plan_block_qkv(M, dims->hidden, n_out, kPlanCUs);
  f.attn = plan_block_attn(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                           attended_keys(dims, max_ctx_len), kPlanCUs);
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = align(f.attn.ws_bytes);
  f.off_part = off;
  off = align(off + sizeof(float) * (size_t)f.qkv.splits * M * n_out);
  f.off_qhi = off;
  off = align(off + 2 * (size_t)M * nq);
  f.off_qlo = off;
  off = align(off + 2 * (size_t)M * nq);
  f.off_k = off;
  off = align(off + 2 * (size_t)M * nk);
  f.off_v = off;
  off = align(off + 2 * (size_t)M * nk);
  f.ws_bytes = off;
  return f;
}

size_t dflash_block_qkv_attn_workspace_size(const dflash_dims* dims, int32_t max_ctx_len) {
  if (check_qkv_dims(dims) != DFLASH_OK || check_attn_sizes(dims, max_ctx_len) != DFLASH_OK) return 0;
  return plan_fused(dims, max_ctx_len).ws_bytes;
}

int dflash_block_qkv_attn(const dflash_dims* dims, const void* h, int64_t ld_h, const void* w_qkv,
                          const void* k_cache, const void* v_cache, const int32_t* page_table,
                          const int32_t* ctx_len, int32_t max_ctx_len, const float* rope_cos,
                          const float* rope_sin, int32_t max_pos, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  int st = check_qkv_dims(dims);
  if (st != DFLASH_OK) return st;
  if (!h || !w_qkv || !k_cache || !v_cache || !ctx_len || !rope_cos || !rope_sin || !out) return DFLASH_ERR_NULL;
  if (ld_h < dims->hidden) return DFLASH_ERR_SHAPE;
  if ((ld_h & 7) || !aligned16(h) || !aligned16(w_qkv)) return DFLASH_ERR_ALIGN;
  if (max_ctx_len < 0 || max_ctx_len > (1 << 24)) return DFLASH_ERR_SHAPE;
  if ((int64_t)max_pos < (int64_t)max_ctx_len + DFLASH_BLOCK) return DFLASH_ERR_CAPACITY;
  const FusedPlan f = plan_fused(dims, max_ctx_len);
  if (!workspace || workspace_bytes < f.ws_bytes) return DFLASH_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DFLASH_ERR_ALIGN;
  char* ws = static_cast<char*>(workspace);
  const int M = dims->batch * DFLASH_BLOCK;
  const int nq = dims->n_q_heads * dims->head_dim, nk = dims->n_kv_heads * dims->head_dim;
  const int n_out = nq + 2 * nk;
  uint16_t* qhi = reinterpret_cast<uint16_t*>(ws + f.off_qhi);
  uint16_t* qlo = reinterpret_cast<uint16_t*>(ws + f.off_qlo);
  uint16_t* kr = reinterpret_cast<uint16_t*>(ws + f.off_k);
  uint16_t* vv = reinterpret_cast<uint16_t*>(ws + f.off_v);
  // The attention's checks first (nothing is launched before every part validates); the
  // q/k/v outputs are its inputs.
  st = block_attn_run(dims, qhi, kr, vv, k_cache, v_cache, page_table, ctx_len, max_ctx_len, rope_cos, rope_sin,
                      max_pos, out, ws, f.attn.ws_bytes, nullptr, nullptr, nullptr, qlo, /*launch=*/false);
  if (st != DFLASH_OK) return st;
  GemmParams g{};
  g.a_seg[0] = static_cast<const uint16_t*>(h);
  g.lda = ld_h;
  g.seg_k = dims->hidden;
  g.b0 = g.b1 = static_cast<const uint16_t*>(w_qkv);
  g.n_b0 = n_out;
  g.M = M;
  g.N = n_out;
  g.K = dims->hidden;
  g.k_per_split = f.qkv.kps;
  g.out = reinterpret_cast<float*>(ws + f.off_part);
  if (launch_gemm_nt(g, f.qkv.splits, f.qkv.small, stream) != hipSuccess) return DFLASH_ERR_LAUNCH;
  QkvRopeParams r{};
  r.part = g.out;
  r.splits = f.qkv.splits;
  r.M = M;
  r.N = n_out;
  r.nq = nq;
  r.nk = nk;
  r.head_dim = dims->head_dim;
  r.ctx_len = ctx_len;
  r.max_ctx = max_ctx_len;
  r.rope_cos = rope_cos;
  r.rope_sin = rope_sin;
  r.q_hi = qhi;
  r.q_lo = qlo;
  r.k_out = kr;
  r.v_out = vv;
  r.err = reinterpret_cast<uint32_t*>(ws);  // the attention's error word
  if (launch_qkv_rope(r, stream) != hipSuccess) return DFLASH_ERR_LAUNCH;
  return block_attn_run(dims, qhi, kr, vv, k_cache, v_cache, page_table, ctx_len, max_ctx_len, rope_cos, rope_sin,
                        max_pos, out, ws, f.attn.ws_bytes, nullptr, nullptr, stream, qlo);
}

}  // extern "C"
