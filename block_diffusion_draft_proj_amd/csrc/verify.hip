// Greedy verify: vocab-wide argmax at the 16 block positions, matched-prefix
// accept length, next staged token, commit positions and crop of the KV length.
//
// Pages: "dflash-mlx: lossless speculative decoding" -- "what is lossless"
// (every emitted token is the target's greedy argmax), "single-forward verify"
// steps 6-9, guarantee 2 (accept = sum(cumprod(draft == posterior)), no skipping
// past a mismatch; the target token at the first rejected slot is the next staged
// token) and guarantee 3 / "DFlash dual implementations" §3 (crop the attention KV
// to the committed length).
//
// Design (HBM-bound stream of B*16*V bf16 logits):
//  * one workgroup per (row, 8192-element chunk): 256 threads, 4 x 16-byte
//    coalesced loads per thread, all issued before any arithmetic;
//  * values are mapped to order-preserving 16-bit keys with packed 16-bit integer
//    ops (two elements per instruction), so the per-element cost is ~2.5 VALU ops;
//  * the first index of the chunk maximum is found in a second pass over the keys
//    held in registers, by only the threads whose own maximum matched;
//  * each chunk publishes one 64-bit key (value key << 32 | ~index), so the row
//    maximum with the lowest index is an order-independent max();
//  * cross-lane steps use DPP lane moves and the gfx950 row-swap permutes, not LDS
//    shuffles;
//  * with 8 or more sequences, the last workgroup of each sequence reduces its 16
//    rows and runs accept / commit / crop inside the same kernel: all workgroups
//    of a sequence sit on one XCD and hand over through its L2 (arrival counted by
//    an L2 atomic), with no device-wide fence.  Only wave 0 takes part in the
//    hand-off and the accept step, so the other waves leave once the chunk key is
//    known and their slots go to the remaining workgroups;
//  * with fewer sequences, a second kernel (one wave per sequence) does that
//    step: a kernel boundary is then the cheapest device-wide hand-off, since
//    handing off across XCDs inside one kernel would need an L2 writeback
//    (agent-scope release) from every workgroup.  No host round trip.
//
// The draft side of the cycle ("single-forward verify" steps 3-4: one draft
// forward over [staged, mask x 15] yields the 15 candidate tail tokens) runs on
// the same kernels: the greedy draft token at mask slot i is the argmax of the
// draft's logits in row i, so only the row map (rows 1..15 of each sequence)
// and the last step (write the tokens into the block) differ.
#include "common.h"
#include "launch.h"

namespace dflash {

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;

// Ordered keys of two packed bf16 values: negative -> ~bits, non-negative -> bits|0x8000.
// Monotone in value for non-NaN inputs, except -0 (0x7fff) sits just below +0 (0x8000).
// Positive NaNs land above +inf (0xff80), negative NaNs below -inf (0x007f).
__device__ __forceinline__ uint32_t order_keys(uint32_t w) {
  const i16x2 v = __builtin_bit_cast(i16x2, w);
  const uint32_t s = __builtin_bit_cast(uint32_t, (i16x2)(v >> (i16x2){15, 15}));
  return w ^ (s | 0x80008000u);
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

constexpr uint32_t kKeyNegInf = 0x007fu;  // key of -inf; masked tail elements use it too
constexpr uint32_t kKeyPosInf = 0xff80u;
constexpr uint32_t kNegInfBits2 = 0xff80ff80u;

__device__ __forceinline__ bool is_zero_key(uint32_t k) { return k == 0x7fffu || k == 0x8000u; }
__device__ __forceinline__ bool is_nan_key(uint32_t k) { return k < kKeyNegInf || k > kKeyPosInf; }

// DPP lane moves (gfx9 encodings): swaps inside quads, rotations inside 16-lane rows.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// Reduction of an associative, commutative op over the 16 lanes of each row: after the
// two quad swaps every lane holds its quad's result, after the rotations by 4 and 8 its
// row's.  All VALU: no LDS round trip per step, as a shuffle would take.
template <typename Op>
__device__ __forceinline__ uint32_t row_reduce(uint32_t v, Op op) {
  v = op(v, dpp<kDppQuadXor1>(v));
  v = op(v, dpp<kDppQuadXor2>(v));
  v = op(v, dpp<kDppRowRor4>(v));
  return op(v, dpp<kDppRowRor8>(v));
}
// ... then over the four rows with the gfx950 row-swap permutes (lanes l ^ 16, l ^ 32).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = row_reduce(v, op);
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(a[0], a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(c[0], c[1]);
}

template <typename Op>
__device__ __forceinline__ uint32_t wg_reduce(uint32_t v, Op op, uint32_t* s_buf) {
  v = wave_reduce(v, op);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_buf[wave] = v;
  __syncthreads();
  uint32_t r = s_buf[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) r = op(r, s_buf[w]);
  return r;
}

// The chunk's 64-bit key: (order key of its maximum << 32) | ~(first index of it),
// so the row maximum with the lowest index is an order-independent max().
// Returned by thread 0.
__device__ __forceinline__ uint64_t chunk_key(const VerifyParams& p, int row, int chunk, uint32_t* s_red) {
  const int tid = threadIdx.x;
  const uint16_t* rp = p.logits + (int64_t)row * p.ld;
  const int c0 = chunk * kVerifyChunk;
  const int c1 = min(p.vocab, c0 + kVerifyChunk);

  // Pass 1: all loads first, then order keys with running packed max / min.
  u32x4 w[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int e = c0 + (i * kThreads + tid) * 8;
    // ld is a multiple of 8 and >= vocab, so a vector that starts inside the row
    // ends inside the row's allocation.
    w[i] = (e < c1) ? ld16(rp + e) : (u32x4){kNegInfBits2, kNegInfBits2, kNegInfBits2, kNegInfBits2};
  }
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int e = c0 + (i * kThreads + tid) * 8;
    if (e < c1 && e + 8 > c1) {  // partial vector at the end of the row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t x = w[i][j];
        if (e + 2 * j >= c1) x = (x & 0xffff0000u) | 0xff80u;
        if (e + 2 * j + 1 >= c1) x = (x & 0x0000ffffu) | 0xff800000u;
        w[i][j] = x;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t k = order_keys(w[i][j]);
      w[i][j] = k;
      kmax = pk_max(kmax, k);
      kmin = pk_min(kmin, k);
    }
  }
  const uint32_t tmax = max(kmax & 0xffffu, kmax >> 16);
  const uint32_t tmin = min(kmin & 0xffffu, kmin >> 16);
  // One reduction for both: the maximum in the high half, 0xffff - minimum in the low.
  const uint32_t both = wg_reduce((tmax << 16) | (0xffffu - tmin), [](uint32_t a, uint32_t c) { return pk_max(a, c); }, s_red);
  const uint32_t cmax = both >> 16, cmin = 0xffffu - (both & 0xffffu);

  // Pass 2: first element index holding the chunk maximum.
  const bool has_nan = (cmin < kKeyNegInf) || (cmax > kKeyPosInf);
  const bool zero = !has_nan && is_zero_key(cmax);
  bool mine;
  if (has_nan) mine = is_nan_key(tmin) || is_nan_key(tmax);
  else mine = zero ? is_zero_key(tmax) : (tmax == cmax);
  uint32_t idx = 0xffffffffu;
  if (mine) {
#pragma unroll
    for (int i = kVec - 1; i >= 0; --i) {  // descending so the last hit is the lowest index
      const int e = c0 + (i * kThreads + tid) * 8;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
#pragma unroll
        for (int h = 1; h >= 0; --h) {
          const uint32_t k = (w[i][j] >> (16 * h)) & 0xffffu;
          const bool hit = has_nan ? is_nan_key(k) : (zero ? is_zero_key(k) : (k == cmax));
          if (hit) idx = (uint32_t)(e + 2 * j + h);
        }
      }
    }
  }
  idx = wg_reduce(idx, [](uint32_t a, uint32_t c) { return min(a, c); }, s_red);

  const uint64_t canon = has_nan ? 0x10000u : (zero ? 0x8000u : cmax);
  return (canon << 32) | (uint64_t)(0xffffffffu - idx);
}

// Rows a sequence reads: all 16 for the verify, the 15 mask rows (1..15) for the
// draft tokens.  seq_row<DRAFT>(r) is the logit row of the sequence's r-th one.
template <bool DRAFT>
constexpr int kRowsPerSeq = DRAFT ? kBlock - 1 : kBlock;
template <bool DRAFT>
__device__ __forceinline__ int seq_row(int b, int r) {
  return b * kBlock + (DRAFT ? 1 : 0) + r;
}

template <bool DRAFT>
__global__ __launch_bounds__(kThreads) void verify_argmax_kernel(VerifyParams p) {
  __shared__ uint32_t s_red[kThreads / kWave];
  const int r = blockIdx.x / p.n_chunks;
  const int chunk = blockIdx.x - r * p.n_chunks;
  const int b = r / kRowsPerSeq<DRAFT>;
  const int row = seq_row<DRAFT>(b, r - b * kRowsPerSeq<DRAFT>);
  const uint64_t key = chunk_key(p, row, chunk, s_red);
  if (threadIdx.x == 0) p.part[(int64_t)row * p.n_chunks + chunk] = key;
}

// The accept step runs on one wave (64 lanes, 4 per block row: lane = 4 * row + sub), so
// the fused kernel's other three waves of every workgroup leave as soon as the chunk key
// is known.  No LDS and no barrier: the row maxima are combined by DPP quad swaps and the
// per-row values are exchanged across lanes.
constexpr int kAcceptThreads = kWave;
constexpr int kRowLoads = 8;  // chunk keys per lane in flight (up to 32 chunks per round trip)

// Largest chunk key of logit row `row` over its first n_chunks chunks, reduced over the 4
// lanes of the row (lane `sub` reads chunks sub, sub + 4, ...).  Every lane of the row
// returns it (0 when n_chunks is 0).  All loads of a round are issued before any is
// compared.
__device__ __forceinline__ uint64_t row_best(const VerifyParams& p, int row, int sub, int n_chunks) {
  const uint64_t* pr = p.part + (int64_t)row * p.n_chunks;
  uint64_t best = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += 4 * kRowLoads) {
    // Chunks past the end re-read the last one: a repeated key leaves the maximum
    // unchanged, and unconditional loads all go out before the first wait.
    uint64_t k[kRowLoads];
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i) k[i] = pr[min(c0 + sub + 4 * i, n_chunks - 1)];
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i) best = k[i] > best ? k[i] : best;
  }
  auto step = [](uint64_t v, uint32_t lo, uint32_t hi) {
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
  };
  best = step(best, dpp<kDppQuadXor1>((uint32_t)best), dpp<kDppQuadXor1>((uint32_t)(best >> 32)));
  return step(best, dpp<kDppQuadXor2>((uint32_t)best), dpp<kDppQuadXor2>((uint32_t)(best >> 32)));
}
__device__ __forceinline__ int32_t key_index(uint64_t key) { return (int32_t)(0xffffffffu - (uint32_t)key); }

// Sequence b: reduce the chunk keys of its 16 rows, then accept, next staged token,
// KV-length crop, commit positions and page count.  One wave; every global load (chunk
// keys, block tokens, input length) is issued before the first is used.
__device__ __forceinline__ void accept_seq(const VerifyParams& p, int b) {
  const int lane = threadIdx.x;
  const int row = lane >> 2, sub = lane & 3;
  const int32_t blk = lane < kBlock ? p.block_tokens[b * kBlock + lane] : 0;
  const int32_t kvin = p.kv_len_in[b];
  const int32_t post = key_index(row_best(p, b * kBlock + row, sub, p.n_chunks));
  if (sub == 0) p.posterior[b * kBlock + row] = post;
  // Lane t < 15 compares draft token t + 1 with the target's token at position t.
  const int t = lane < kBlock - 1 ? lane : kBlock - 2;
  const int32_t post_t = __shfl(post, 4 * t);
  const int32_t blk_next = __shfl(blk, t + 1);
  const uint64_t miss = __ballot(lane < kBlock - 1 && blk_next != post_t);
  const int a = miss ? (int)__builtin_ctzll(miss) : kBlock - 1;  // leading matches, uniform
  const int32_t next = __builtin_amdgcn_readlane(post, 4 * a);
  const int32_t kv_out = kvin + 1 + a;
  if (lane == 0) {
    p.accept_len[b] = a;
    p.next_token[b] = next;
    p.kv_len_out[b] = kv_out;
    if (p.n_pages) p.n_pages[b] = (int32_t)(((int64_t)kv_out + p.page_size - 1) / p.page_size);
  }
  if (p.commit_pos && lane < kBlock) p.commit_pos[b * kBlock + lane] = (lane <= a) ? kvin + lane : -1;
}

// Sequence b's draft tokens: the argmax of each mask row (1..15) from its chunk keys,
// written to block[b][1..15]; slot 0 gets staged[b] when staged is given.  Row 0's keys
// are never computed, so its lanes take no chunks (they still join the quad swaps of
// their own row, which read no other row).
__device__ __forceinline__ void draft_seq(const VerifyParams& p, int b) {
  const int lane = threadIdx.x;
  const int row = lane >> 2, sub = lane & 3;
  const uint64_t best = row_best(p, b * kBlock + row, sub, row ? p.n_chunks : 0);
  if (sub == 0 && row) p.draft_block[b * kBlock + row] = key_index(best);
  if (lane == 0 && p.staged) p.draft_block[b * kBlock] = p.staged[b];
}

// Second kernel of the two-kernel form: one workgroup per sequence.  Running after
// the argmax kernel on the same stream, it sees every chunk key without any
// device-wide fence.
template <bool DRAFT>
__global__ __launch_bounds__(kAcceptThreads) void verify_accept_kernel(VerifyParams p) {
  if (DRAFT) draft_seq(p, blockIdx.x);
  else accept_seq(p, blockIdx.x);
}

// One-kernel form for batch >= 8 (every XCD holds whole sequences): workgroup i runs
// on XCD i % 8 (round-robin dispatch) and the decode puts every workgroup of
// sequence b on XCD b % 8, so its chunk keys and its arrival counter stay in one
// L2.  A workgroup stores its chunk key, waits until the L2 acknowledges it, and
// counts its arrival with an atomic performed in that L2; the last of the
// sequence's 16 * n_chunks workgroups clears the counter and runs the accept step.
// This saves the second launch (~5 us on this part) for ~1-2 us of tail.  Below 8
// sequences some XCDs would sit idle, so the two-kernel form is used there.
template <bool DRAFT>
__global__ __launch_bounds__(kThreads) void verify_fused_kernel(VerifyParams p, int batch) {
  __shared__ uint32_t s_red[kThreads / kWave];
  const int per = kRowsPerSeq<DRAFT> * p.n_chunks;  // workgroups per sequence
  // A workgroup off the expected die would count its arrival in another L2, and the
  // sequence's accept step would never run: raise DEVERR_XCD instead of staying silent.
  if (threadIdx.x == 0 && ((xcc_id() ^ blockIdx.x) & p.xcc_mask) != 0) set_dev_error(p.err, kDevErrXcd);
  const int xcd = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
  const int b = xcd + kNumXcd * (j / per);
  if (b >= batch) return;
  const int rem = j - (j / per) * per;
  const int row_in = rem / p.n_chunks, chunk = rem - row_in * p.n_chunks;
  const int row = seq_row<DRAFT>(b, row_in);
  const uint64_t key = chunk_key(p, row, chunk, s_red);
  // Waves 1..3 are done: leaving now frees their slots for the next workgroups while
  // wave 0 hands the key over.
  if (threadIdx.x >= kWave) return;
  uint32_t last = 0;
  if (threadIdx.x == 0) {
    p.part[(int64_t)row * p.n_chunks + chunk] = key;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    wait_vmcnt<0>();  // the key is in the L2
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t* cnt = p.count + (int64_t)b * kVerifyCntStride;
    const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    last = prev == (uint32_t)(per - 1) ? 1u : 0u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (!__builtin_amdgcn_readlane(last, 0)) return;
  // The loads below are served by the L2: the sequence's chunk keys are read once,
  // here, and its key block (16 rows x n_chunks x 8 bytes = 128 * n_chunks bytes
  // from a 256-byte aligned base) shares no cache line with another sequence's, so
  // no CU can hold an older copy of them in its L1 (which every launch starts empty).
  if (DRAFT) draft_seq(p, b);
  else accept_seq(p, b);
}

template <bool DRAFT>
hipError_t launch_argmax_seq(const VerifyParams& p, int batch, hipStream_t stream) {
  if (batch >= kNumXcd) {
    const int grid = kNumXcd * ((batch + kNumXcd - 1) / kNumXcd) * kRowsPerSeq<DRAFT> * p.n_chunks;
    hipLaunchKernelGGL(verify_fused_kernel<DRAFT>, dim3(grid), dim3(kThreads), 0, stream, p, batch);
    return hipGetLastError();
  }
  const int grid = batch * kRowsPerSeq<DRAFT> * p.n_chunks;
  hipLaunchKernelGGL(verify_argmax_kernel<DRAFT>, dim3(grid), dim3(kThreads), 0, stream, p);
  hipLaunchKernelGGL(verify_accept_kernel<DRAFT>, dim3(batch), dim3(kAcceptThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_accept(const VerifyParams& p, int batch, hipStream_t stream) {
  return launch_argmax_seq<false>(p, batch, stream);
}

hipError_t launch_draft_argmax(const VerifyParams& p, int batch, hipStream_t stream) {
  return launch_argmax_seq<true>(p, batch, stream);
}

}  // namespace dflash
