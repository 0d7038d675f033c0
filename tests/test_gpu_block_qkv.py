"""GPU parity of dflash_block_qkv (the block's own q / k / v) against the oracle.

Tolerance, derived from the arithmetic: both sides round the same dot product to
bf16 once.  The oracle takes it exactly (float64); the kernel sums bf16 x bf16
products in fp32, split over K, then adds the split partials.  The fp32 result is
within ~sqrt(K) * 2^-24 * sum|h w| of the exact one (K <= 5120 here: ~1e-6 of
rms(Y)), so the two roundings agree except where that error straddles a bf16
rounding boundary, and then they are one ulp apart.  Hence per element
|gpu - ref| <= ulp_bf16(ref) + 1e-5 * rms(ref), and at least 99 % of the entries
must be bit-identical."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from tests.gpu_util import DEV, host_u16, log, u16

pytestmark = pytest.mark.gpu


def ulp_bf16(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _run(cfg, qi, B, ld_pad=0):
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    dims = dfl.make_dims(B, Hq, Hkv, d, hidden=cfg.hidden, kv_capacity=1)
    ws = dfl.workspace(dfl.dflash_block_qkv_workspace_size(dims), DEV)
    h = qi.h
    if ld_pad:
        h = np.concatenate([h, np.full((h.shape[0], ld_pad), 0x7FC0, np.uint16)], axis=1)  # NaN padding
    q = torch.full((B, 16, Hq, d), -1, dtype=torch.int16, device=DEV)
    k = torch.full((B, 16, Hkv, d), -1, dtype=torch.int16, device=DEV)
    v = torch.full((B, 16, Hkv, d), -1, dtype=torch.int16, device=DEV)
    dfl.dflash_block_qkv(dims, u16(h), u16(qi.w_qkv), q, k, v, ws)
    torch.cuda.synchronize()
    return host_u16(q), host_u16(k), host_u16(v), ws


def _check(cfg, qi, B, label, ld_pad=0):
    log(f"block qkv {label}: B={B} M={16 * B} hidden={cfg.hidden}")
    got = _run(cfg, qi, B, ld_pad)
    ref = orc.block_qkv_ref(qi.h, qi.w_qkv, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    for name, g, r in zip("qkv", got[:3], ref):
        r = r.reshape(B, 16, *r.shape[1:])
        gf, rf = orc.bf16_to_f64(g), orc.bf16_to_f64(r)
        rms = float(np.sqrt(np.mean(rf ** 2)))
        err = np.abs(gf - rf)
        same = float(np.mean(g == r))
        log(f"  {name}: max err {err.max():.3e} (rms {rms:.3f}), bit-identical {100 * same:.3f} %")
        assert np.all(np.isfinite(gf))
        assert np.all(err <= ulp_bf16(rf) + 1e-5 * rms), name
        assert same >= 0.99, name
    assert got[3][:4].cpu().numpy().view(np.uint32)[0] == 0


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_block_qkv_full_size(name):
    cfg = synth.CONFIGS[name]
    _check(cfg, synth.block_qkv_inputs(cfg), cfg.batch, name)


def test_block_qkv_padded_rows_and_tiled_path():
    # Rows past hidden hold NaN and must not be read; 40 sequences (640 rows) take the
    # tiled GEMM instead of the skinny one.
    cfg = synth.CONFIGS["tiny"]
    _check(cfg, synth.block_qkv_inputs(cfg, batch=3, seed=61), 3, "tiny ld+64", ld_pad=64)
    _check(cfg, synth.block_qkv_inputs(cfg, batch=40, seed=62), 40, "tiny 640 rows")
    cfg = synth.CONFIGS["qwen3_8b"]
    _check(cfg, synth.block_qkv_inputs(cfg, batch=40, seed=63), 40, "qwen3_8b 640 rows")


@pytest.mark.parametrize("B,Hq,Hkv,d,hidden", [
    (1, 1, 1, 64, 64),       # one head of each kind, the smallest hidden: 192 outputs < one weight tile
    (2, 2, 2, 128, 128),     # group size 1
    (33, 8, 1, 128, 192),    # 528 rows (just past the skinny path), one kv head, hidden 3 x 64
    (5, 12, 4, 64, 320),     # group 3
])
def test_block_qkv_degenerate_shapes(B, Hq, Hkv, d, hidden):
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, hidden=hidden)
    _check(cfg, synth.block_qkv_inputs(cfg, batch=B, seed=64 + B), B, f"{Hq}q/{Hkv}kv d={d} hidden={hidden}")


@pytest.mark.parametrize("B,Hq,Hkv,d,hidden", [
    (768, 4, 2, 64, 256),    # 12288 rows: 48 rows of tiles, six per XCD, in bands of 4 and 2
    (200, 8, 2, 64, 128),    # 3200 rows: 13 rows of tiles (one or two per XCD); 3 column tiles, the last partial
])
def test_block_qkv_tiled_tile_order(B, Hq, Hkv, d, hidden):
    # The tiled product's per-XCD tile order with several bands, a short last band and a
    # partial last column of tiles: every output element is written exactly once.
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, hidden=hidden)
    _check(cfg, synth.block_qkv_inputs(cfg, batch=B, seed=90 + B), B, f"{16 * B} rows, {Hq}q/{Hkv}kv d={d}")
