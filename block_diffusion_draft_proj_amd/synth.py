"""Seeded synthetic inputs for the DFlash draft-attention / verify hot path.

This module only *draws* inputs: shapes, value distributions and structure
(planted accepted-prefix lengths, ragged context lengths, a shuffled page
table).  It performs none of the method's arithmetic -- no projection, no RoPE,
no attention, no argmax, no acceptance -- so that the CPU oracle and the HIP
path can both consume its output without sharing any computation.

Workload shapes follow the five configurations the hot path is specified on
(tiny, Qwen3-8B-shaped, batched serving, long context, ragged paged).  Value
distributions: target hidden states N(0,1), weights N(0, 0.02^2), verify
logits N(0,1), all rounded to bf16 (round to nearest even).  Block q/k/v and
the context K/V cache are drawn directly with the standard deviation that the
corresponding projection of N(0,1) hiddens through N(0,0.02^2) weights would
have (sqrt(fan_in) * 0.02 per projection), instead of being computed.

Verify logits carry a planted argmax: every row gets one entry set to 8.0
while all other entries are N(0,1) clipped to [-7, 7].  The target's greedy
token of each row is therefore known by construction, and draft tokens are
built to agree with it on a Geometric(p) prefix (the "block of 16 = staged
token + 15 drafts" layout of the dflash-mlx page, section on block-diffusion
drafting).  Rows without a spike (``spike=False``) keep plain N(0,1) logits,
where tied maxima are frequent.

bf16 values travel as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

BLOCK = 16  # 1 staged token + 15 mask slots per draft block

# Order of the independent random streams spawned from one config seed.
_STREAMS = (
    "x_ctx", "w_fc", "w_k", "w_v", "w_q", "x_blk", "logits", "staged",
    "accept", "mismatch", "tail", "ragged_L", "page_perm", "kv_ctx",
)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    ctx_len: Optional[int]        # fixed context length, None for ragged
    ragged: Optional[tuple]       # (lo, hi) inclusive for uniform ragged lengths
    hidden: int                   # draft hidden size D
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_target_layers: int          # number of concatenated target layers
    target_hidden: int            # hidden size of each target layer
    vocab: int
    accept_p: float               # Geometric parameter of planted prefixes
    page_size: int                # 0 = dense cache, 16 = paged
    seed: int
    rope_base: float = 1.0e6
    intermediate: int = 0         # draft MLP width I (0: 3 x hidden)

    @property
    def inter(self) -> int:
        return self.intermediate or 3 * self.hidden

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def ctx_width(self) -> int:
        return self.n_target_layers * self.target_hidden

    @property
    def q_std(self) -> float:
        # block q/k/v = hidden N(0,1) through a N(0,0.02^2) [*, D] weight
        return math.sqrt(self.hidden) * 0.02

    @property
    def kv_ctx_std(self) -> float:
        # ctx K/V = (X_cat W_fc^T) W_k^T: two N(0,0.02^2) projections of N(0,1)
        return math.sqrt(self.ctx_width) * 0.02 * math.sqrt(self.hidden) * 0.02


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 1, 64, None, 256, 4, 2, 64, 2, 256, 1024, 0.15, 0, 1001),
    "qwen3_8b": Config("qwen3_8b", 1, 2048, None, 4096, 32, 8, 128, 5, 4096, 151936, 0.10, 0, 1002,
                       intermediate=12288),
    "batched": Config("batched", 8, 8192, None, 4096, 32, 8, 128, 5, 4096, 151936, 0.10, 0, 1003,
                      intermediate=12288),
    "long_ctx": Config("long_ctx", 1, 32768, None, 5120, 40, 8, 128, 5, 5120, 151936, 0.10, 0, 1004,
                       intermediate=17408),
    "ragged": Config("ragged", 32, None, (512, 16384), 4096, 32, 8, 128, 5, 4096, 151936, 0.10, 16, 1005,
                     intermediate=12288),
}


def streams(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(ss)) for name, ss in zip(_STREAMS, children)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Only used to encode freshly drawn random numbers (no NaN handling needed)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0, clip: Optional[float] = None,
                chunk: int = 1 << 24) -> np.ndarray:
    """N(0, std^2) draws in float32, rounded to bf16 bits; drawn in chunks to bound memory."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if clip is not None:
            np.clip(v, -clip, clip, out=v)
        out[s:e] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def context_lengths(cfg: Config, rngs=None) -> np.ndarray:
    if cfg.ragged is None:
        return np.full(cfg.batch, cfg.ctx_len, dtype=np.int32)
    rngs = rngs or streams(cfg.seed)
    lo, hi = cfg.ragged
    return rngs["ragged_L"].integers(lo, hi, size=cfg.batch, endpoint=True).astype(np.int32)


def max_positions(ctx_len: np.ndarray) -> int:
    """RoPE table length that covers every context and block position (+ one commit)."""
    return int(ctx_len.max()) + 2 * BLOCK


@dataclasses.dataclass
class AttnInputs:
    cfg: Config
    q_blk: np.ndarray        # [B,16,Hq,d] bf16 bits, pre-RoPE
    k_blk: np.ndarray        # [B,16,Hkv,d] bf16 bits, pre-RoPE
    v_blk: np.ndarray        # [B,16,Hkv,d] bf16 bits
    ctx_len: np.ndarray      # [B] int32
    k_cache: np.ndarray      # dense [B,Hkv,cap,d] or paged [P,Hkv,16,d] bf16 bits (post-RoPE K)
    v_cache: np.ndarray
    page_table: Optional[np.ndarray]  # [B, pages_per_seq] int32 or None
    capacity: int            # dense: tokens per (seq, head); paged: page-table width
    num_pages: int           # paged: pool size (0 for dense)


def attn_inputs(cfg: Config, ctx_len: Optional[np.ndarray] = None, seed: Optional[int] = None,
                page_size: Optional[int] = None) -> AttnInputs:
    """Block q/k/v plus a context K/V cache holding ``ctx_len[b]`` valid rows.

    Cache rows beyond a sequence's length hold unrelated values on purpose: a
    kernel that reads past ``ctx_len`` gives a wrong answer instead of a lucky one.
    """
    rngs = streams(cfg.seed if seed is None else seed)
    if ctx_len is None:
        ctx_len = context_lengths(cfg, rngs)
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    B, Hq, Hkv, d = len(ctx_len), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    ps = cfg.page_size if page_size is None else page_size
    q = normal_bf16(rngs["x_blk"], (B, BLOCK, Hq, d), cfg.q_std)
    k = normal_bf16(rngs["x_blk"], (B, BLOCK, Hkv, d), cfg.q_std)
    v = normal_bf16(rngs["x_blk"], (B, BLOCK, Hkv, d), cfg.q_std)
    need = int(ctx_len.max()) + BLOCK if B else BLOCK  # room for one commit of up to 16 rows
    if ps == 0:
        cap = need
        kc = normal_bf16(rngs["kv_ctx"], (B, Hkv, cap, d), cfg.kv_ctx_std)
        vc = normal_bf16(rngs["kv_ctx"], (B, Hkv, cap, d), cfg.kv_ctx_std)
        return AttnInputs(cfg, q, k, v, ctx_len, kc, vc, None, cap, 0)
    width = (need + ps - 1) // ps
    per_seq = (ctx_len.astype(np.int64) + BLOCK + ps - 1) // ps
    n_pages = int(per_seq.sum())
    perm = rngs["page_perm"].permutation(n_pages).astype(np.int32)
    table = np.full((B, width), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :per_seq[b]] = perm[off:off + per_seq[b]]
        off += per_seq[b]
    kc = normal_bf16(rngs["kv_ctx"], (n_pages, Hkv, ps, d), cfg.kv_ctx_std)
    vc = normal_bf16(rngs["kv_ctx"], (n_pages, Hkv, ps, d), cfg.kv_ctx_std)
    return AttnInputs(cfg, q, k, v, ctx_len, kc, vc, table, width, n_pages)


@dataclasses.dataclass
class VerifyInputs:
    cfg: Config
    logits: np.ndarray        # [B,16,V] bf16 bits
    block_tokens: np.ndarray  # [B,16] int32: staged token then 15 drafts
    kv_len: np.ndarray        # [B] int32, committed length before the block
    planted_post: Optional[np.ndarray]   # [B,16] greedy tokens by construction (spike rows)
    planted_accept: Optional[np.ndarray]  # [B] planted accept length


def verify_inputs(cfg: Config, batch: Optional[int] = None, spike: bool = True,
                  seed: Optional[int] = None, p: Optional[float] = None,
                  kv_len: Optional[np.ndarray] = None) -> VerifyInputs:
    rngs = streams(cfg.seed if seed is None else seed)
    B = cfg.batch if batch is None else batch
    V = cfg.vocab
    p = cfg.accept_p if p is None else p
    if kv_len is None:
        if cfg.ragged is None:
            kv_len = np.full(B, cfg.ctx_len, dtype=np.int32)
        else:
            lo, hi = cfg.ragged
            kv_len = rngs["ragged_L"].integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    kv_len = np.asarray(kv_len, dtype=np.int32)
    logits = normal_bf16(rngs["logits"], (B, BLOCK, V), 1.0, clip=7.0 if spike else None)
    staged = rngs["staged"].integers(0, V, size=B).astype(np.int32)
    blk = np.empty((B, BLOCK), dtype=np.int32)
    blk[:, 0] = staged
    if not spike:
        blk[:, 1:] = rngs["tail"].integers(0, V, size=(B, BLOCK - 1))
        return VerifyInputs(cfg, logits, blk, kv_len, None, None)
    post = rngs["logits"].integers(0, V, size=(B, BLOCK)).astype(np.int32)
    spike_bits = f32_to_bf16_bits(np.array([8.0], dtype=np.float32))[0]
    for b in range(B):
        logits[b, np.arange(BLOCK), post[b]] = spike_bits
    # Geometric(p) has support {1,2,...}; the planted accept length is G-1 capped at 15.
    a_true = np.minimum(BLOCK - 1, rngs["accept"].geometric(p, size=B) - 1).astype(np.int32)
    for b in range(B):
        a = int(a_true[b])
        blk[b, 1:a + 1] = post[b, :a]
        if a < BLOCK - 1:
            r = int(rngs["mismatch"].integers(0, V - 1)) if V > 1 else 0
            blk[b, a + 1] = (post[b, a] + 1 + r) % V
            for i in range(a + 2, BLOCK):
                if rngs["tail"].random() < 0.25:
                    blk[b, i] = post[b, i - 1]   # a later chance match must not count
                else:
                    blk[b, i] = rngs["tail"].integers(0, V)
    return VerifyInputs(cfg, logits, blk, kv_len, post, a_true)


@dataclasses.dataclass
class CtxProjInputs:
    cfg: Config
    x_layers: List[np.ndarray]  # n_t x [M, D_t] bf16 bits
    w_fc: np.ndarray            # [D, n_t*D_t] bf16 bits (nn.Linear layout)
    w_k: np.ndarray             # [Hkv*d, D]
    w_v: np.ndarray             # [Hkv*d, D]


def ctx_proj_inputs(cfg: Config, n_rows: int, seed: Optional[int] = None,
                    weights_only: bool = False) -> CtxProjInputs:
    rngs = streams(cfg.seed if seed is None else seed)
    D, Dt, nt, kvw = cfg.hidden, cfg.target_hidden, cfg.n_target_layers, cfg.n_kv_heads * cfg.head_dim
    w_fc = normal_bf16(rngs["w_fc"], (D, nt * Dt), 0.02)
    w_k = normal_bf16(rngs["w_k"], (kvw, D), 0.02)
    w_v = normal_bf16(rngs["w_v"], (kvw, D), 0.02)
    xs = [] if weights_only else [normal_bf16(rngs["x_ctx"], (n_rows, Dt), 1.0) for _ in range(nt)]
    return CtxProjInputs(cfg, xs, w_fc, w_k, w_v)



@dataclasses.dataclass
class BlockQkvInputs:
    cfg: Config
    h: np.ndarray               # [16 B, hidden] bf16 bits: the draft's block hidden states
    w_qkv: np.ndarray           # [(Hq + 2 Hkv) d, hidden] bf16 bits: q heads, k heads, v heads


def block_qkv_inputs(cfg: Config, batch: Optional[int] = None, seed: Optional[int] = None,
                     w_std: float = 0.02) -> BlockQkvInputs:
    """Block hidden states N(0, 1) and a fused q/k/v weight N(0, w_std^2), bf16."""
    rngs = streams(cfg.seed if seed is None else seed)
    B = cfg.batch if batch is None else batch
    n_out = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    h = normal_bf16(rngs["x_blk"], (B * BLOCK, cfg.hidden), 1.0)
    w = normal_bf16(rngs["w_q"], (n_out, cfg.hidden), w_std)
    return BlockQkvInputs(cfg, h, w)


@dataclasses.dataclass
class DraftLayerInputs:
    cfg: Config
    x: np.ndarray               # [16 B, D] bf16 bits: the layer's input (the residual stream)
    attn: np.ndarray            # [16 B, Hq d] float32: an attention output
    w_in: np.ndarray            # [D] bf16 bits: input RMSNorm weight
    w_o: np.ndarray             # [D, Hq d]
    w_post: np.ndarray          # [D]: post-attention RMSNorm weight
    w_gate: np.ndarray          # [I, D]
    w_up: np.ndarray            # [I, D]
    w_down: np.ndarray          # [D, I]
    eps: float = 1e-6


def draft_layer_inputs(cfg: Config, batch: Optional[int] = None, seed: Optional[int] = None,
                       attn_std: float = 0.5) -> DraftLayerInputs:
    """Random weights of a Qwen3-shaped draft layer: projections N(0, 0.02^2), norm
    weights N(1, 0.05^2); the layer input N(0, 1) and an attention output
    N(0, attn_std^2) in float32 (a weighted mean of value rows is narrower than
    the rows themselves)."""
    rngs = streams((cfg.seed if seed is None else seed) + 77)
    B = cfg.batch if batch is None else batch
    M, D, A, I = B * BLOCK, cfg.hidden, cfg.n_q_heads * cfg.head_dim, cfg.inter
    x = normal_bf16(rngs["x_blk"], (M, D), 1.0)
    attn = rngs["tail"].standard_normal((M, A), dtype=np.float32) * np.float32(attn_std)
    w_in = f32_to_bf16_bits(1 + 0.05 * rngs["w_k"].standard_normal(D, dtype=np.float32))
    w_post = f32_to_bf16_bits(1 + 0.05 * rngs["w_k"].standard_normal(D, dtype=np.float32))
    w_o = normal_bf16(rngs["w_q"], (D, A), 0.02)
    w_gate = normal_bf16(rngs["w_fc"], (I, D), 0.02)
    w_up = normal_bf16(rngs["w_fc"], (I, D), 0.02)
    w_down = normal_bf16(rngs["w_v"], (D, I), 0.02)
    return DraftLayerInputs(cfg, x, attn, w_in, w_o, w_post, w_gate, w_up, w_down)


@dataclasses.dataclass
class GdnTapeInputs:
    state: np.ndarray           # [B, H, d_v, d_k] float32: recurrent state saved before the block
    k_tape: np.ndarray          # [B, 16, H, d_k] bf16 bits: unit-norm keys
    g_tape: np.ndarray          # [B, 16, H] float32: log-gates (< 0)
    delta_tape: np.ndarray      # [B, 16, H, d_v] float32: innovations
    accept: np.ndarray          # [B] int32 accept lengths


def gdn_tape_inputs(batch: int, n_heads: int, d_k: int, d_v: int, accept_p: float = 0.1,
                    seed: int = 2024) -> GdnTapeInputs:
    """A saved recurrent state N(0, 0.05^2), keys uniform on the unit sphere, gates
    alpha = exp(g) uniform in [0.9, 1), innovations N(0, 0.1^2), and planted accept
    lengths min(15, Geometric(accept_p) - 1)."""
    rngs = streams(seed)
    state = rngs["kv_ctx"].standard_normal((batch, n_heads, d_v, d_k), dtype=np.float32) * np.float32(0.05)
    k = rngs["x_blk"].standard_normal((batch, BLOCK, n_heads, d_k))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = np.log(rngs["tail"].uniform(0.9, 1.0, (batch, BLOCK, n_heads))).astype(np.float32)
    delta = rngs["w_v"].standard_normal((batch, BLOCK, n_heads, d_v), dtype=np.float32) * np.float32(0.1)
    accept = np.minimum(BLOCK - 1, rngs["accept"].geometric(accept_p, batch) - 1).astype(np.int32)
    return GdnTapeInputs(state, f32_to_bf16_bits(k.astype(np.float32)), g, delta, accept)
