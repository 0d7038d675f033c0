"""GPU parity of dflash_block_qkv_attn (the block's q/k/v and the attention in one
call) against the oracle's one-step definition (block_qkv_attn_ref): exact
products, the rotated Q unrounded, the rotated block K and V rounded once.

The call carries Q as a bf16 hi/lo pair from an fp32-accumulated product
(relative error ~1e-6 before the split, ~2^-17 after it), so the attention sees
Q within ~1e-5 of the oracle's; block K / V differ from the oracle's exact
rounding by one bf16 step where fp32 accumulation straddles a midpoint (rare,
and one key among L + 16).  The bound is the attention's: max-abs 2e-2 on the
fp32 outputs, at the configurations' own weight and hidden-state distributions.
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from tests.gpu_util import DEV, attn_dims, i32, log, rope_tables, u16

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _paged_copy(at):
    B, Hkv, cap, d = at.k_cache.shape
    width = (cap + 15) // 16
    table = np.random.default_rng(7).permutation(B * width).astype(np.int32).reshape(B, width)
    kp = np.zeros((B * width, Hkv, 16, d), np.uint16)
    vp = np.zeros_like(kp)
    for b in range(B):
        for pg in range(width):
            t0, t1 = pg * 16, min(cap, pg * 16 + 16)
            kp[table[b, pg], :, :t1 - t0] = at.k_cache[b, :, t0:t1]
            vp[table[b, pg], :, :t1 - t0] = at.v_cache[b, :, t0:t1]
    return dataclasses.replace(at, k_cache=kp, v_cache=vp, page_table=table, capacity=width, num_pages=B * width)


def _run(cfg, at, qi, window=0, units=None, ws=None):
    B = len(at.ctx_len)
    max_ctx = int(at.ctx_len.max())
    dims = attn_dims(cfg, at, window)
    cos, sin = rope_tables(cfg.head_dim, max_ctx + 2 * synth.BLOCK, cfg.rope_base)
    if ws is None:
        ws = dfl.workspace(dfl.dflash_block_qkv_attn_workspace_size(dims, max_ctx), DEV)
    out = torch.full((B, synth.BLOCK, cfg.n_q_heads, cfg.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    log(f"block qkv+attn {cfg.name}: B={B} L<={max_ctx} window={window} paged={at.page_table is not None}")
    dfl.dflash_block_qkv_attn(dims, u16(qi.h), u16(qi.w_qkv), u16(at.k_cache), u16(at.v_cache),
                              None if at.page_table is None else i32(at.page_table), i32(at.ctx_len), max_ctx,
                              cos, sin, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = orc.block_qkv_attn_ref(qi.h, qi.w_qkv, cfg.n_q_heads, cfg.n_kv_heads, at.k_cache, at.v_cache,
                                 at.ctx_len, cfg.rope_base, page_table=at.page_table, units=units, window=window)
    mask = ~np.isnan(ref)
    err = float(np.max(np.abs(got[mask] - ref[mask])))
    log(f"  max-abs err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0
    assert not ws[256:256 + 128 * 4096].any()          # the attention's counters back at zero
    assert err <= TOL, err
    return got, ws


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b", "batched", "long_ctx"])
def test_block_qkv_attn_configs(name):
    cfg = synth.CONFIGS[name]
    _run(cfg, synth.attn_inputs(cfg), synth.block_qkv_inputs(cfg))


def test_block_qkv_attn_ragged_paged_sampled():
    cfg = synth.CONFIGS["ragged"]
    at = synth.attn_inputs(cfg)
    bs = [0, 7, 13, 31]
    _run(cfg, at, synth.block_qkv_inputs(cfg), units=[(b, g) for b in bs for g in (0, cfg.n_kv_heads - 1)])


@pytest.mark.parametrize("B,hq,hkv,d,paged,window", [
    (3, 8, 2, 128, False, 0),     # 48 rows: 4 activation tiles
    (20, 4, 2, 64, True, 0),      # 320 rows: two chunks of the product; d = 64; paged
    (5, 12, 2, 128, False, 0),    # 6 heads per group: one wave group
    (2, 8, 2, 128, True, 1024),   # sliding window over a paged ring
    (40, 8, 2, 64, False, 0),     # 640 rows: the tiled product (above the skinny kernel's 512)
])
def test_block_qkv_attn_shapes(B, hq, hkv, d, paged, window):
    cfg = dataclasses.replace(synth.CONFIGS["qwen3_8b"], batch=B, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                              hidden=1024, seed=B * 100 + hq)
    lens = np.random.default_rng(B).integers(1, 3000, B)
    at = synth.attn_inputs(cfg, ctx_len=lens, page_size=0)
    if paged:
        at = _paged_copy(at)
    _run(cfg, at, synth.block_qkv_inputs(cfg), window=window)


def test_block_qkv_attn_repeats_bitwise_on_one_workspace():
    cfg = synth.CONFIGS["batched"]
    at = synth.attn_inputs(cfg, ctx_len=np.array([8192, 3000, 17, 5000, 1, 900, 4000, 2048]))
    qi = synth.block_qkv_inputs(cfg)
    a, ws = _run(cfg, at, qi)
    b, _ = _run(cfg, at, qi, ws=ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
