"""CPU oracle for the DFlash draft block-attention and greedy-verify hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, helpers or tables); both sides consume the same seeded
inputs from ``block_diffusion_draft_proj_amd.synth``, which draws data and
computes nothing of the method.

Everything is plain NumPy in float64, slow and literal: each function states
the definition it writes out and the page passage it follows.  Pages:

* "DFlash dual implementations: PyTorch vs MLX code architecture"
  (hotelren.com/news/4396892) -- §1 model definition (RoPE reused from Qwen3),
  §2 attention (dual-source K/V = [ctx ; block], Q from the block only,
  non-causal inside the block), §3 KV cache (crop to the accepted prefix),
  §4 target hidden states (select layers by id and concatenate).
* "dflash-mlx: lossless speculative decoding" (dpshk.com/news/6100553) --
  "what is lossless" (every emitted token is the target's greedy argmax),
  "block-diffusion draft" (block = staged token + 15 mask slots; the draft
  reads target hidden states), "single-forward verify" (the 9-step cycle),
  guarantee 2 (acceptance = sum of cumprod of draft == posterior, no skipping;
  the target token at the first rejected slot becomes the next staged token),
  guarantee 3 (attention KV is cropped to the committed length).

Readings where the pages are silent (each is listed with its reason in the
design notes): two-stage projection fc -> shared W_k/W_v with the context
feature C held in bf16; rotate-half RoPE with base 1e6 applied to Q and K
only; softmax scale d^-1/2; q head h uses kv head floor(h/G); block Q and K are
rounded to bf16 after RoPE, ctx K/V are bf16 in the cache; argmax takes the
lowest index among equal maxima, NaN ranks above everything, -0 == +0.
The rotated block Q / K are rounded to bf16 once, from the exact rotation with
the float32 cos / sin tables; everything else is float64.

Parity note: the projection/norm/RoPE structure of the real draft model is not
fixed by the pages; the oracle pins the method *under the readings above*.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16


# --------------------------------------------------------------------------
# bf16 encode / decode (own implementation; bf16 = top 16 bits of float32)
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # NaN payloads convert quietly
        return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits.  Rounding is done once, from float64, by
    scaling the mantissa to an integer grid and using round-half-even.  Values
    below the smallest normal bf16 (2^-126) round on the subnormal grid 2^-133;
    values beyond the largest finite bf16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e = np.frexp(xf)                    # xf = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                # below 2^-126 keep the subnormal spacing
    q = np.ldexp(1.0, (e - 8).astype(np.int64))   # spacing of the 8-bit grid
    r = np.rint(xf / q) * q                # np.rint rounds half to even
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bf16
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (nearest even) and return the uint16 bit patterns."""
    r = round_bf16(x).astype(np.float32)   # exact: r is on the bf16 grid
    bits = (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x))
    bits[nan] = 0x7FC0
    return bits


# --------------------------------------------------------------------------
# RoPE  (page "DFlash dual implementations", §1: the draft reuses the Qwen3
# rotary embedding).  Reading: rotate-half pairs (j, j + d/2), angle
# theta_j(pos) = pos * base^(-2j/d), computed in float64.
# --------------------------------------------------------------------------
def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / head_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def apply_rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate x[..., n, H, d] at positions pos[n] (same position for every head).

    For each pair (x_j, x_{j+d/2}):  (x_j cos - x_{j+d/2} sin,  x_{j+d/2} cos + x_j sin).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    th = rope_angles(pos, d, base)          # [n, d/2]
    c = np.cos(th)[:, None, :]              # broadcast over heads
    s = np.sin(th)[:, None, :]
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_tables_f32(pos: np.ndarray, head_dim: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos / sin of the RoPE angles at ``pos`` [n]: computed in float64 and rounded
    to float32 (the tables every side of the path reads), returned as float64 [n, d/2]."""
    th = rope_angles(pos, head_dim, base)
    return (np.cos(th).astype(np.float32).astype(np.float64),
            np.sin(th).astype(np.float32).astype(np.float64))


def round_bf16_sum(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """bf16 nearest-even rounding of the EXACT sum a + b of float64 arrays.

    s = fl64(a + b) and its rounding error e (error-free two-sum) hold the exact
    value s + e.  Rounding s to bf16 gives the same answer as rounding s + e,
    except when s lies exactly halfway between two bf16 neighbours and e != 0:
    then the exact value is off the midpoint, on the side of e's sign.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    r = round_bf16(s)
    _, ex = np.frexp(s)
    half = np.ldexp(1.0, (np.maximum(ex, -125) - 9).astype(np.int64))   # half a bf16 step at |s|
    tie = (np.abs(s - r) == half) & (e != 0) & np.isfinite(s)
    r[tie] = s[tie] + np.sign(e[tie]) * half[tie]
    return r


def rope_bf16(x_bits: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """bf16(RoPE(x)) for bf16 inputs x[..., n, H, d], as float64 values.

    The plain definition: rotate each pair with the float32 cos / sin tables,
      y_j = x_j c - x_{j+d/2} s,   y_{j+d/2} = x_{j+d/2} c + x_j s,
    and round each exact y once to bf16 (nearest even).  A bf16 value times a
    float32 value is exact in float64 (8 + 24 significant bits), and the sum of
    the two products is rounded from its exact value (``round_bf16_sum``).
    """
    x = bf16_to_f64(x_bits)
    d = x.shape[-1]
    c, s = rope_tables_f32(pos, d, base)
    c, s = c[:, None, :], s[:, None, :]
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([round_bf16_sum(lo * c, -(hi * s)), round_bf16_sum(hi * c, lo * s)], axis=-1)


# --------------------------------------------------------------------------
# a1-a3: context feature, projection to K/V, RoPE, cache rows
# (page "DFlash dual implementations" §4: select target layers by id and
# concatenate; §2: ctx K/V come from the projected target hidden states;
# dflash-mlx page "block-diffusion draft": the draft reads target_hidden.)
# --------------------------------------------------------------------------
def ctx_proj_ref(x_layers: Sequence[np.ndarray], w_fc: np.ndarray, w_k: np.ndarray,
                 w_v: np.ndarray, row_pos: np.ndarray, n_kv_heads: int, head_dim: int,
                 base: float) -> dict:
    """Context projection of M rows of target hidden states.

    X_cat = [X_1 | ... | X_nt]  (feature concat, in the order given)
    C     = X_cat W_fc^T, held as bf16 (the draft's context feature)
    K     = RoPE(C W_k^T, pos),  V = C W_v^T  (per kv head), then bf16 in the cache.
    Rows with pos < 0 are not committed; their K is returned unrotated.
    Returns float64 arrays: C (exact), Cb (bf16-rounded), K, V (before the
    final bf16 rounding) and Kb, Vb (rounded).
    """
    X = np.concatenate([bf16_to_f64(x) for x in x_layers], axis=1)
    C = X @ bf16_to_f64(w_fc).T
    Cb = round_bf16(C)
    M = X.shape[0]
    Kraw = (Cb @ bf16_to_f64(w_k).T).reshape(M, n_kv_heads, head_dim)
    V = (Cb @ bf16_to_f64(w_v).T).reshape(M, n_kv_heads, head_dim)
    pos = np.asarray(row_pos, dtype=np.int64)
    K = Kraw.copy()
    live = pos >= 0
    if live.any():
        K[live] = apply_rope(Kraw[live], pos[live], base)
    return {"C": C, "Cb": Cb, "K": K, "V": V, "Kb": round_bf16(K), "Vb": round_bf16(V)}


# --------------------------------------------------------------------------
# The block's own q / k / v, the attention's first inputs (page "DFlash dual
# implementations" §2: Q comes from the block tokens only, and the block's K/V
# are the second source beside the context's).  Reading: one bias-free linear
# map over the draft's block hidden states, nn.Linear layout, the weight rows
# ordered q heads, then k heads, then v heads; exact products (float64), each
# output rounded once to bf16; no RoPE here (the attention rotates Q and the
# block K at their positions).
# --------------------------------------------------------------------------
def block_qkv_ref(h: np.ndarray, w_qkv: np.ndarray, n_q_heads: int, n_kv_heads: int,
                  head_dim: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """q, k, v bf16 bits for M = 16 B block rows (sequence-major).

    h [M, hidden] bf16 bits; w_qkv [(Hq + 2 Hkv) d, hidden] bf16 bits.
      Y = h . w_qkv^T  (float64), rounded to bf16
      q = Y[:, 0 : Hq d]              as [M, Hq, d]
      k = Y[:, Hq d : (Hq + Hkv) d]   as [M, Hkv, d]
      v = Y[:, (Hq + Hkv) d : ]       as [M, Hkv, d]
    """
    M = h.shape[0]
    nq, nk = n_q_heads * head_dim, n_kv_heads * head_dim
    assert w_qkv.shape[0] == nq + 2 * nk and w_qkv.shape[1] == h.shape[1]
    Y = f64_to_bf16_bits(bf16_to_f64(h) @ bf16_to_f64(w_qkv).T)
    q = Y[:, :nq].reshape(M, n_q_heads, head_dim)
    k = Y[:, nq:nq + nk].reshape(M, n_kv_heads, head_dim)
    v = Y[:, nq + nk:].reshape(M, n_kv_heads, head_dim)
    return q, k, v


# --------------------------------------------------------------------------
# a4-a6: dual-source non-causal block attention
# (page "DFlash dual implementations" §2: K/V = [ctx ; block tokens], Q from
# the block tokens only, non-causal inside the block.)
# --------------------------------------------------------------------------
def gather_pages(cache: np.ndarray, page_table: np.ndarray, b: int, length: int) -> np.ndarray:
    """Dense [Hkv, length, d] view of sequence b from a paged [P, Hkv, ps, d] cache."""
    return gather_rows(cache, page_table, b, np.arange(length))


def gather_rows(cache: np.ndarray, page_table: Optional[np.ndarray], b: int, rows: np.ndarray) -> np.ndarray:
    """Storage rows ``rows`` of sequence b as [Hkv, len(rows), d]: from a dense
    [B, Hkv, cap, d] cache, or through the page table of a paged [P, Hkv, ps, d] one."""
    rows = np.asarray(rows, dtype=np.int64)
    if page_table is None:
        return cache[b][:, rows, :]
    ps = cache.shape[2]
    pages = page_table[b, rows // ps]
    return np.transpose(cache[pages, :, rows % ps, :], (1, 0, 2))


def block_attn_unit_ref(q_b: np.ndarray, k_b: np.ndarray, v_b: np.ndarray,
                        k_ctx: np.ndarray, v_ctx: np.ndarray, ctx_len: int, g: int,
                        group: int, base: float, scale: Optional[float] = None,
                        return_probs: bool = False, block_pos: Optional[int] = None):
    """Attention of one (sequence, kv head g) unit.

    q_b [16, Hq, d], k_b / v_b [16, Hkv, d] bf16 bits (q, k pre-RoPE);
    k_ctx / v_ctx [>=ctx_len, d] bf16 bits of kv head g (K already rotated): the
    first ctx_len rows are the context keys, in position order.  Block positions
    are block_pos .. block_pos+15 (block_pos defaults to ctx_len; a sliding window
    passes fewer context rows than the block's position).  For each q head h:
      Q_h   = bf16(RoPE(q_h))                        [16, d]
      Keys  = [K_ctx[0:L] ; bf16(RoPE(k_blk[:, g]))] [L+16, d]
      Vals  = [V_ctx[0:L] ; v_blk[:, g]]
      S = Q_h Keys^T * scale,  P = softmax over all L+16 keys (no mask),  O = P Vals.
    The rotated block rows are rounded once from their exact values
    (``rope_bf16``); the rest is float64.  Returns O [16, group, d] (and P [group, 16, L+16] if asked).
    """
    d = q_b.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    L = int(ctx_len)
    pos = (L if block_pos is None else int(block_pos)) + np.arange(BLOCK)
    hs = slice(g * group, (g + 1) * group)
    Q = rope_bf16(q_b[:, hs, :], pos, base)                                      # [16, G, d]
    Kblk = rope_bf16(k_b[:, g:g + 1, :], pos, base)[:, 0, :]
    Keys = np.concatenate([bf16_to_f64(k_ctx[:L]), Kblk], axis=0)
    Vals = np.concatenate([bf16_to_f64(v_ctx[:L]), bf16_to_f64(v_b[:, g, :])], axis=0)
    out = np.empty((BLOCK, group, d))
    probs = np.empty((group, BLOCK, L + BLOCK))
    for hh in range(group):
        s = (Q[:, hh, :] @ Keys.T) * scale
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        probs[hh] = p
        out[:, hh, :] = p @ Vals
    return (out, probs) if return_probs else out


def block_attn_ref(q_blk: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray,
                   k_cache: np.ndarray, v_cache: np.ndarray, ctx_len: np.ndarray,
                   base: float, page_table: Optional[np.ndarray] = None,
                   scale: Optional[float] = None,
                   units: Optional[Sequence[Tuple[int, int]]] = None,
                   window: int = 0) -> np.ndarray:
    """O [B, 16, Hq, d] float64 for every (b, kv head) unit, or only ``units``.

    k_cache / v_cache: dense [B, Hkv, cap, d] or, with ``page_table``, paged
    [P, Hkv, page, d]; the oracle gathers pages itself.  Entries of units not
    computed are NaN.

    Sliding window (page "DFlash dual implementations" §3: the MLX side trims a
    rotating cache).  Reading: with window W > 0 the cache keeps the last W
    committed positions in a ring of W rows (position t in row t mod W), and the
    context of sequence b is positions max(0, L-W) .. L-1; the block stays at
    positions L .. L+15.
    """
    B, _, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    out = np.full((B, BLOCK, Hq, d), np.nan)
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        L = int(ctx_len[b])
        first = max(0, L - window) if window > 0 else 0
        t = np.arange(first, L)                               # context positions
        rows = t % window if window > 0 else t                # their storage rows
        kc = gather_rows(k_cache, page_table, b, rows)[g]
        vc = gather_rows(v_cache, page_table, b, rows)[g]
        out[b, :, g * G:(g + 1) * G, :] = block_attn_unit_ref(
            q_blk[b], k_blk[b], v_blk[b], kc, vc, L - first, g, G, base, scale, block_pos=L)
    return out


# --------------------------------------------------------------------------
# The block's q/k/v and the attention as one step (page "DFlash dual
# implementations", §2: Q comes from the block tokens only, the block's K/V are
# the second source).  Reading: the products are exact; the rotated Q enters the
# attention unrounded (no bf16 storage of q between the two steps); the rotated
# block K and the block V are rounded once to bf16 from their exact values, as
# they sit beside the bf16 context cache.  The rotation uses the float32 tables.
# --------------------------------------------------------------------------
def attend_ref(Q: np.ndarray, Keys: np.ndarray, Vals: np.ndarray, scale: float) -> np.ndarray:
    """softmax(Q Keys^T scale) Vals over all keys (no mask), float64; Q [n, d]."""
    s = (Q @ Keys.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ Vals


def block_qkv_attn_ref(h: np.ndarray, w_qkv: np.ndarray, n_q_heads: int, n_kv_heads: int,
                       k_cache: np.ndarray, v_cache: np.ndarray, ctx_len: np.ndarray, base: float,
                       page_table: Optional[np.ndarray] = None, scale: Optional[float] = None,
                       units: Optional[Sequence[Tuple[int, int]]] = None, window: int = 0) -> np.ndarray:
    """O [B, 16, Hq, d] float64 for the block hidden states h [16 B, hidden] (bf16 bits).

      Y = h w_qkv^T (exact), split into q [B,16,Hq,d], k, v [B,16,Hkv,d]
      Q      = RoPE(q) at positions L .. L+15               (not rounded)
      K_blk  = bf16(RoPE(k)),  V_blk = bf16(v)              (rounded once)
      O      = attention over [context ; block] as in block_attn_ref (window W > 0: the
               last min(L, W) context positions, from ring rows).
    """
    Hq, Hkv = n_q_heads, n_kv_heads
    M = h.shape[0]
    B = M // BLOCK
    d = w_qkv.shape[0] // (Hq + 2 * Hkv)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    Y = bf16_to_f64(h) @ bf16_to_f64(w_qkv).T
    q = Y[:, :Hq * d].reshape(B, BLOCK, Hq, d)
    k = Y[:, Hq * d:(Hq + Hkv) * d].reshape(B, BLOCK, Hkv, d)
    v = Y[:, (Hq + Hkv) * d:].reshape(B, BLOCK, Hkv, d)
    out = np.full((B, BLOCK, Hq, d), np.nan)
    todo = units if units is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in todo:
        L = int(ctx_len[b])
        pos = L + np.arange(BLOCK)
        c, s_ = rope_tables_f32(pos, d, base)
        rot = lambda x: np.concatenate([x[:, :d // 2] * c - x[:, d // 2:] * s_,
                                        x[:, d // 2:] * c + x[:, :d // 2] * s_], axis=1)
        first = max(0, L - window) if window > 0 else 0
        t = np.arange(first, L)
        rows = t % window if window > 0 else t
        Keys = np.concatenate([bf16_to_f64(gather_rows(k_cache, page_table, b, rows)[g]),
                               round_bf16(rot(k[b, :, g]))], axis=0)
        Vals = np.concatenate([bf16_to_f64(gather_rows(v_cache, page_table, b, rows)[g]),
                               round_bf16(v[b, :, g])], axis=0)
        for hh in range(G):
            hd = g * G + hh
            out[b, :, hd, :] = attend_ref(rot(q[b, :, hd]), Keys, Vals, scale)
    return out


# --------------------------------------------------------------------------
# a7-a9: greedy verify, prefix acceptance, commit and crop
# (dflash-mlx page: "what is lossless" -- emitted tokens are the target's
# greedy argmax; "single-forward verify" steps 6-9; guarantee 2 -- the
# printed acceptance expression sum(cumprod(equal(drafted, posterior))) and
# its no-skip reading, the first rejected slot's target token is the next
# staged token; guarantee 3 / page "DFlash dual implementations" §3 -- the
# attention KV cache is cropped to the committed length.)
# --------------------------------------------------------------------------
def argmax_first(values: np.ndarray) -> np.ndarray:
    """Greedy token per row: the lowest index of the maximum.

    NaN ranks above every number (the first NaN wins); -0 and +0 are equal.
    numpy.argmax has exactly these semantics on float arrays.
    """
    return np.argmax(values, axis=-1).astype(np.int32)


def verify_accept_ref(logits: np.ndarray, block_tokens: np.ndarray, kv_len: np.ndarray,
                      page_size: int = 0) -> dict:
    """One verify cycle for B sequences.

    logits [B, 16, V] bf16 bits; block_tokens [B, 16] = [staged, d_1 .. d_15];
    kv_len [B] = committed length before the block.
      post[b, i]   = argmax_v logits[b, i, v]          (target greedy token after slot i)
      accept[b]    = sum(cumprod(block_tokens[b, 1:] == post[b, :15]))   in [0, 15]
      next[b]      = post[b, accept[b]]                 (next staged token)
      kv_len'[b]   = kv_len[b] + 1 + accept[b]          (commit staged + accepted drafts)
      commit[b, i] = kv_len[b] + i if i <= accept[b] else -1
      n_pages[b]   = ceil(kv_len'[b] / page_size)       (paged caches only)
    """
    B = logits.shape[0]
    post = np.empty((B, BLOCK), dtype=np.int32)
    for b in range(B):                      # row-wise decode keeps memory bounded
        post[b] = argmax_first(bf16_to_f64(logits[b]))
    blk = np.asarray(block_tokens, dtype=np.int64)
    matches = (blk[:, 1:] == post[:, :BLOCK - 1]).astype(np.int32)
    accept = np.sum(np.cumprod(matches, axis=1), axis=1).astype(np.int32)
    nxt = post[np.arange(B), accept].astype(np.int32)
    kv_in = np.asarray(kv_len, dtype=np.int64)
    kv_out = (kv_in + 1 + accept).astype(np.int32)
    i = np.arange(BLOCK)[None, :]
    commit = np.where(i <= accept[:, None], kv_in[:, None] + i, -1).astype(np.int32)
    res = {"post": post, "accept": accept, "next": nxt, "kv_len": kv_out, "commit_pos": commit}
    if page_size > 0:
        res["n_pages"] = ((kv_out.astype(np.int64) + page_size - 1) // page_size).astype(np.int32)
    return res


# --------------------------------------------------------------------------
# Draft side of the cycle: the draft's greedy tokens at the 15 mask slots
# (dflash-mlx page: "single-forward verify" steps 3-4 -- the draft receives the
# block [staged, mask x 15] and one forward yields the 15 candidate tail
# tokens; "block-diffusion draft" -- the whole block is filled in one forward.)
# Reading: greedy drafting -- each candidate is the lowest-index maximum of the
# draft's logits at its own slot, by the same argmax rule as the target's.
# --------------------------------------------------------------------------
def draft_block_ref(draft_logits: np.ndarray, staged: np.ndarray) -> np.ndarray:
    """block_tokens [B, 16] for one cycle, as the verify step consumes them.

    draft_logits [B, 16, V] bf16 bits: the draft's logits over the block
    [staged, mask x 15]; row 0 (the staged slot) is not read.  staged [B].
      block[b, 0] = staged[b]
      block[b, i] = argmax_v draft_logits[b, i, v]        i = 1 .. 15
    """
    B = draft_logits.shape[0]
    blk = np.empty((B, BLOCK), dtype=np.int32)
    blk[:, 0] = np.asarray(staged, dtype=np.int32)
    for b in range(B):                      # row-wise decode keeps memory bounded
        blk[b, 1:] = argmax_first(bf16_to_f64(draft_logits[b, 1:]))
    return blk


# --------------------------------------------------------------------------
# The rest of a draft layer around the attention (page "DFlash dual
# implementations", §1 model definition: the draft model reuses Qwen3's RMSNorm,
# MLP and rotary embedding; §2: the attention).  Reading: a pre-norm residual
# decoder layer --
#   n1 = RMSNorm(x; w_in)                       -> the block q/k/v projection
#   x1 = x + bf16(attn) W_o^T                   (o_proj, residual add)
#   n2 = RMSNorm(x1; w_post)
#   x2 = x1 + (silu(n2 W_gate^T) * (n2 W_up^T)) W_down^T    (SwiGLU MLP)
# with RMSNorm(x; w) = x / sqrt(mean(x^2) + eps) * w, silu(g) = g / (1 + e^-g),
# no biases, and every tensor a bf16 model stores between the steps (attn
# output, x1, n1 / n2, the MLP activation, x2) rounded once to bf16; all
# arithmetic in between is float64 here.
# --------------------------------------------------------------------------
def rmsnorm_ref(x: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """bf16(x / sqrt(mean(x^2) + eps) * w) per row of float64 values x [M, D], as float64."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return round_bf16(x * r * bf16_to_f64(w_bits))


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def draft_layer_post_ref(x_bits: np.ndarray, attn: np.ndarray, w_o: np.ndarray, w_post: np.ndarray,
                         w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, eps: float) -> dict:
    """The layer after the attention, for M = 16 B block rows.

    x_bits [M, D] bf16 bits (the layer's input, the residual); attn [M, Hq*d] the
    attention output (float values, rounded to bf16 here); weights bf16 bits in
    nn.Linear layout: w_o [D, Hq*d], w_gate / w_up [I, D], w_down [D, I]; w_post [D].
    Returns float64 arrays: a, x1, n2, g, u, act, x2_exact, x2 (= bf16(x2_exact)).
    """
    a = round_bf16(np.asarray(attn, dtype=np.float64))
    x1 = round_bf16(bf16_to_f64(x_bits) + a @ bf16_to_f64(w_o).T)
    n2 = rmsnorm_ref(x1, w_post, eps)
    g = n2 @ bf16_to_f64(w_gate).T
    u = n2 @ bf16_to_f64(w_up).T
    act = round_bf16(silu(g) * u)
    x2 = x1 + act @ bf16_to_f64(w_down).T
    return {"a": a, "x1": x1, "n2": n2, "g": g, "u": u, "act": act, "x2_exact": x2, "x2": round_bf16(x2)}


def rmsnorm_brute(row: Sequence[float], w: Sequence[float], eps: float) -> List[float]:
    """Scalar twin of ``rmsnorm_ref`` for one row (exact rational sum of squares)."""
    ss = sum(Fraction(float(v)) ** 2 for v in row)
    ms = float(ss / len(row)) + eps
    r = 1.0 / math.sqrt(ms)
    return [float(round_bf16(np.array([float(v) * r * float(wj)]))[0]) for v, wj in zip(row, w)]


# --------------------------------------------------------------------------
# Rollback of recurrent (GatedDeltaNet) state by tape replay (page "dflash-mlx:
# lossless speculative decoding", guarantee 3: verifying the block advances the
# recurrent state by all 16 candidate steps; the state cannot be cropped, so
# during the verify an "innovation tape" of per-step k, g and increments is
# recorded, and after acceptance only the accepted steps are replayed onto the
# state saved before the block; page "DFlash dual implementations" §7: the state
# is rolled back along the accepted prefix).
# Reading: the gated delta rule of Gated DeltaNet (Yang, Kautz, Hatamizadeh,
# "Gated Delta Networks", ICLR 2025), per head, state S [d_v, d_k]:
#   alpha_t = exp(g_t),  delta_t = beta_t (v_t - alpha_t S_{t-1} k_t)   (innovation)
#   S_t = alpha_t S_{t-1} + delta_t k_t^T
# The tape holds (k_t, g_t, delta_t); replay of the committed steps t = 0..a
# (the staged token and a accepted drafts) needs no S k product.
# --------------------------------------------------------------------------
def gdn_block_ref(S0: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
                  beta: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The verify's pass over the 16 block steps of one head, float64.

    S0 [d_v, d_k]; k [16, d_k]; v [16, d_v]; g, beta [16].  Returns the states
    after each step [16, d_v, d_k] and the innovations delta [16, d_v]."""
    S = np.asarray(S0, dtype=np.float64).copy()
    states, delta = [], []
    for t in range(k.shape[0]):
        alpha = math.exp(float(g[t]))
        d = float(beta[t]) * (v[t] - alpha * (S @ k[t]))
        S = alpha * S + np.outer(d, k[t])
        states.append(S.copy())
        delta.append(d)
    return np.stack(states), np.stack(delta)


def gdn_replay_ref(S0: np.ndarray, k_tape: np.ndarray, g_tape: np.ndarray, delta_tape: np.ndarray,
                   accept: np.ndarray) -> np.ndarray:
    """Rolled-back states [B, H, d_v, d_k]: S = S0[b, h], then for t = 0..accept[b]:
    S = exp(g[b, t, h]) S + delta[b, t, h] k[b, t, h]^T.

    S0 [B, H, d_v, d_k] float; k_tape [B, 16, H, d_k] bf16 bits; g_tape [B, 16, H] and
    delta_tape [B, 16, H, d_v] float; accept [B] in [0, 15]."""
    out = np.array(S0, dtype=np.float64)
    k = bf16_to_f64(k_tape)
    B = out.shape[0]
    for b in range(B):
        for t in range(int(accept[b]) + 1):
            alpha = np.exp(np.asarray(g_tape[b, t], dtype=np.float64))          # [H]
            d = np.asarray(delta_tape[b, t], dtype=np.float64)                  # [H, d_v]
            out[b] = alpha[:, None, None] * out[b] + d[:, :, None] * k[b, t][:, None, :]
    return out


def gdn_block_brute(S0, k, v, g, beta) -> List[np.ndarray]:
    """Scalar twin of ``gdn_block_ref`` in the delta rule's matrix form,
    S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, with loops."""
    dv, dk = len(S0), len(S0[0])
    S = [[float(S0[i][j]) for j in range(dk)] for i in range(dv)]
    out = []
    for t in range(len(k)):
        a, bt = math.exp(float(g[t])), float(beta[t])
        P = [[a * ((1.0 if r == c else 0.0) - bt * float(k[t][r]) * float(k[t][c])) for c in range(dk)]
             for r in range(dk)]
        S = [[sum(S[i][r] * P[r][j] for r in range(dk)) + bt * float(v[t][i]) * float(k[t][j])
              for j in range(dk)] for i in range(dv)]
        out.append(np.array(S))
    return out


# --------------------------------------------------------------------------
# Brute-force twins for tiny shapes: scalar Python loops, float64 math.
# --------------------------------------------------------------------------
def argmax_brute(row: Sequence[float]) -> int:
    best_i, best = 0, float(row[0])
    for i in range(1, len(row)):
        if math.isnan(best):
            break
        x = float(row[i])
        if math.isnan(x) or x > best:
            best_i, best = i, x
    return best_i


def accept_brute(drafts: Sequence[int], post: Sequence[int]) -> int:
    """Length of the matched prefix: index of the first draft that differs from post."""
    a = 0
    while a < BLOCK - 1 and int(drafts[a + 1]) == int(post[a]):
        a += 1
    return a


def rope_brute(vec: Sequence[float], pos: int, base: float) -> List[float]:
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for j in range(h):
        th = pos * base ** (-2.0 * j / d)
        c, s = math.cos(th), math.sin(th)
        out[j] = vec[j] * c - vec[j + h] * s
        out[j + h] = vec[j + h] * c + vec[j] * s
    return out


def bf16_round_fraction(v: Fraction) -> float:
    """Nearest-even bf16 value of an exact rational (finite range), by integer arithmetic."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                                               # subnormal grid below 2^-126
    step = Fraction(2) ** (e - 7)
    q, rem = divmod(a, step)                                       # a = q * step + rem
    if rem * 2 > step or (rem * 2 == step and q % 2 == 1):
        q += 1
    return sign * float(q * step)


def rope_brute_bf16(vec: Sequence[float], pos: int, base: float) -> List[float]:
    """Scalar twin of ``rope_bf16`` for one bf16-valued vector, in exact rational
    arithmetic: float32 cos / sin of the float64 angle, exact rotation, one
    nearest-even rounding to bf16."""
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for j in range(h):
        th = pos * base ** (-2.0 * j / d)
        c = Fraction(float(np.float32(math.cos(th))))
        s = Fraction(float(np.float32(math.sin(th))))
        a, b = Fraction(float(vec[j])), Fraction(float(vec[j + h]))
        out[j] = bf16_round_fraction(a * c - b * s)
        out[j + h] = bf16_round_fraction(b * c + a * s)
    return out


def block_attn_brute(q_b, k_b, v_b, k_ctx, v_ctx, ctx_len: int, g: int, group: int,
                     base: float, scale: Optional[float] = None, first: int = 0) -> np.ndarray:
    """Scalar-loop twin of ``block_attn_unit_ref`` for tiny shapes: k_ctx / v_ctx
    hold the rows of positions 0 .. ctx_len-1 in order, and the context keys are
    positions first .. ctx_len-1 (first > 0: a sliding window)."""
    d = q_b.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    L = int(ctx_len)
    f = lambda a: [float(t) for t in bf16_to_f64(a)]
    keys, vals = [], []
    for t in range(first, L):
        keys.append(f(k_ctx[t]))
        vals.append(f(v_ctx[t]))
    for i in range(BLOCK):
        keys.append(rope_brute_bf16(f(k_b[i, g]), L + i, base))
        vals.append(f(v_b[i, g]))
    out = np.zeros((BLOCK, group, d))
    for hh in range(group):
        h = g * group + hh
        for i in range(BLOCK):
            q = rope_brute_bf16(f(q_b[i, h]), L + i, base)
            sc = [sum(q[c] * key[c] for c in range(d)) * scale for key in keys]
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            z = sum(w)
            for c in range(d):
                out[i, hh, c] = sum(w[t] * vals[t][c] for t in range(len(keys))) / z
    return out
