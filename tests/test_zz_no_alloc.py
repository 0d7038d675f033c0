"""The allocation-free block attention (dflash_block_attn_noalloc) against the
workspace entry point (dflash_block_attn): same kernels and plan, so the outputs
must be bit-identical.  Two calls in a row on the library's static scratch, the
second smaller than the first (the scratch keeps the last call's contents; every
call must leave its arrival counters at zero for the next one).  Sizes beyond the
scratch are refused before anything is launched."""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from tests.gpu_util import DEV, attn_dims, i32, log, rope_tables, u16

pytestmark = pytest.mark.gpu


def _both(cfg, at):
    max_ctx = int(at.ctx_len.max())
    dims = attn_dims(cfg, at)
    cos, sin = rope_tables(cfg.head_dim, max_ctx + 2 * synth.BLOCK, cfg.rope_base)
    args = [u16(at.q_blk), u16(at.k_blk), u16(at.v_blk), u16(at.k_cache), u16(at.v_cache),
            None if at.page_table is None else i32(at.page_table), i32(at.ctx_len), max_ctx, cos, sin]
    shape = (len(at.ctx_len), synth.BLOCK, cfg.n_q_heads, cfg.head_dim)
    ws = dfl.workspace(dfl.dflash_block_attn_workspace_size(dims, max_ctx), DEV)
    ref = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    dfl.dflash_block_attn(dims, *args, ref, ws)
    got = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dfl.dflash_block_attn_noalloc(dims, *args, got, err)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy(), int(err.cpu()[0]), int(ws[:4].cpu().numpy().view(np.uint32)[0])


def test_noalloc_matches_workspace_entry_point_two_calls_second_smaller():
    big = synth.CONFIGS["batched"]
    small = dataclasses.replace(synth.CONFIGS["tiny"], batch=3)
    cases = [(big, synth.attn_inputs(big)),
             (small, synth.attn_inputs(small, ctx_len=np.array([64, 17, 3000]), seed=small.seed + 9))]
    for cfg, at in cases:
        log(f"noalloc attention: {cfg.name} B={len(at.ctx_len)} L<={int(at.ctx_len.max())}")
        ref, got, err, ws_err = _both(cfg, at)
        assert err == 0 and ws_err == 0
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), "differs from dflash_block_attn"
        units = [(0, 0), (len(at.ctx_len) - 1, cfg.n_kv_heads - 1)]
        oref = orc.block_attn_ref(at.q_blk, at.k_blk, at.v_blk, at.k_cache, at.v_cache, at.ctx_len,
                                  cfg.rope_base, units=units)
        mask = ~np.isnan(oref)
        assert float(np.max(np.abs(got[mask] - oref[mask]))) <= 2e-2


def test_noalloc_refuses_sizes_beyond_the_scratch():
    cfg = synth.CONFIGS["ragged"]
    dims = dfl.make_dims(32, 32, 8, 128, page_size=16, kv_capacity=1100, num_pages=32 * 1100)
    need = dfl.dflash_block_attn_workspace_size(dims, 16384)
    assert need > dfl.NOALLOC_SCRATCH_BYTES
    t = lambda *s, dt=torch.int16: torch.zeros(*s, dtype=dt, device=DEV)
    out = t(32, 16, 32, 128, dt=torch.float32)
    cos, sin = rope_tables(128, 16384 + 32, cfg.rope_base)
    with pytest.raises(dfl.DflashError) as e:
        dfl.dflash_block_attn_noalloc(dims, t(32, 16, 32, 128), t(32, 16, 8, 128), t(32, 16, 8, 128),
                                      t(32 * 1100, 8, 16, 128), t(32 * 1100, 8, 16, 128),
                                      t(32, 1100, dt=torch.int32), t(32, dt=torch.int32), 16384, cos, sin, out)
    assert e.value.code == -4
