"""GPU parity of dflash_ctx_proj against the oracle.

Tolerance (derived from the arithmetic): the cache holds bf16(K) and bf16(V); the
oracle's K/V are exact (float64) functions of the bf16-rounded context feature C.
The GPU accumulates in fp32, so (a) its C differs from the oracle's C by one bf16
step wherever the exact C lies within fp32 accumulation error of a rounding
midpoint (a few entries in 10^4), and each such flip moves the K/V entries of
that row by ulp(C_i) * |W[o, i]| <= 2^-7 |C_i| |W[o, i]|, which at 4-sigma C and
W is up to 0.125/sqrt(hidden) of rms(K) -- 6e-3 rms at hidden 256; (b) its final
rounding of K/V can land one ulp off where the fp32 result straddles a bf16
midpoint.  Hence per element |gpu - ref| <= 1 ulp_bf16(ref) + 6e-3 * rms(ref);
the normwise relative error must stay <= 4e-3 (bf16 rounding alone gives
~1.6e-3), and at least 99% of entries must be within half an ulp plus 1e-4 rms
(so the flip allowance cannot hide a systematic error).  Rows with a negative
position must leave the cache untouched; the optional C copy must round the
exact C to bf16 up to the same flips (on < 0.1% of entries).
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from tests.gpu_util import DEV, host_u16, i32, log, rope_tables, u16

pytestmark = pytest.mark.gpu


def ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _close(got, ref, label):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    bound = ulp_bf16(ref) + 6e-3 * rms
    worst = float(np.max(err / bound))
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    tight = float(np.mean(err <= 0.5 * ulp_bf16(ref) + 1e-4 * rms))
    log(f"ctx_proj {label}: max err/bound {worst:.3f}, normwise rel {rel:.2e}, "
        f"within half-ulp {100 * tight:.3f}%, rms {rms:.3f}")
    assert worst <= 1.0, worst
    assert rel <= 4e-3, rel
    assert tight >= 0.99, tight


def _commit_positions(kv_len, rng):
    B = len(kv_len)
    pos = np.full((B, 16), -1, np.int32)
    for b in range(B):
        a = int(rng.integers(0, 16))
        pos[b, :a + 1] = kv_len[b] + np.arange(a + 1)
    return pos.reshape(-1)


def _run(cfg, n_rows, row_seq, row_pos, capacity, paged_table=None, num_pages=0, with_fc=True,
         c_out=True, seed=None, ld_pad=0, window=0):
    pj = synth.ctx_proj_inputs(cfg, n_rows, seed=seed)
    Hkv, d, D = cfg.n_kv_heads, cfg.head_dim, cfg.hidden
    B = cfg.batch
    if paged_table is None:
        kc = torch.zeros(B, Hkv, capacity, d, dtype=torch.int16, device=DEV)
        dims = dfl.make_dims(B, cfg.n_q_heads, Hkv, d, hidden=D, kv_capacity=capacity, window=window)
    else:
        kc = torch.zeros(num_pages, Hkv, 16, d, dtype=torch.int16, device=DEV)
        dims = dfl.make_dims(B, cfg.n_q_heads, Hkv, d, hidden=D, page_size=16,
                             kv_capacity=paged_table.shape[1], num_pages=num_pages, window=window)
    vc = torch.zeros_like(kc)
    max_pos = int(max(np.max(row_pos), 0)) + 32
    cos, sin = rope_tables(d, max_pos, cfg.rope_base)
    if with_fc:
        xs, wfc, n_layers, dt = pj.x_layers, pj.w_fc, cfg.n_target_layers, cfg.target_hidden
    else:  # the rows already are the context feature C
        xs = [synth.normal_bf16(synth.streams(7)["x_ctx"], (n_rows, D), 2.86)]
        wfc, n_layers, dt = None, 1, D
    ws = dfl.workspace(dfl.dflash_ctx_proj_workspace_size(dims, n_rows, n_layers, dt), DEV)
    cbuf = torch.zeros(n_rows, D, dtype=torch.int16, device=DEV) if (c_out and with_fc) else None
    log(f"ctx_proj {cfg.name}: M={n_rows} K={n_layers * dt} D={D} paged={paged_table is not None} "
        f"ld_x={dt + ld_pad}")
    if ld_pad:   # each layer's rows lie ld_x = d_target + ld_pad elements apart (a strided view)
        dev_x = [torch.cat([u16(x), torch.full((n_rows, ld_pad), 0x7FC0, dtype=torch.int16, device=DEV)],
                           dim=1)[:, :dt] for x in xs]
    else:
        dev_x = [u16(x) for x in xs]
    dfl.dflash_ctx_proj(dims, dev_x, i32(row_seq), i32(row_pos),
                        None if wfc is None else u16(wfc), u16(pj.w_k), u16(pj.w_v), cos, sin, cbuf, kc, vc,
                        None if paged_table is None else i32(paged_table), ws)
    torch.cuda.synchronize()
    if with_fc:
        ref = orc.ctx_proj_ref(xs, wfc, pj.w_k, pj.w_v, row_pos, Hkv, d, cfg.rope_base)
    else:
        eye = orc.f64_to_bf16_bits(np.eye(D))
        ref = orc.ctx_proj_ref(xs, eye, pj.w_k, pj.w_v, row_pos, Hkv, d, cfg.rope_base)
    err = int(ws[:4].cpu().numpy().view(np.uint32)[0])
    return ref, host_u16(kc), host_u16(vc), (None if cbuf is None else host_u16(cbuf)), err


def _gather_rows(cache, row_seq, row_pos, table=None, window=0):
    """[n_live, Hkv, d] cache rows at the committed (seq, pos) of each live row (ring row
    pos mod window under a sliding window)."""
    live = np.nonzero(row_pos >= 0)[0]
    rows = []
    for m in live:
        s, p = int(row_seq[m]), int(row_pos[m])
        if window:
            p %= window
        rows.append(cache[s, :, p] if table is None else cache[table[s, p // 16], :, p % 16])
    return live, orc.bf16_to_f64(np.stack(rows))


def _check(cfg, n_rows, row_seq, row_pos, capacity, table=None, num_pages=0, with_fc=True, label="", ld_pad=0,
           window=0):
    ref, kc, vc, cb, err = _run(cfg, n_rows, row_seq, row_pos, capacity, table, num_pages, with_fc,
                                ld_pad=ld_pad, window=window)
    assert err == 0
    live, k = _gather_rows(kc, row_seq, row_pos, table, window)
    _, v = _gather_rows(vc, row_seq, row_pos, table, window)
    _close(k, ref["K"][live], label + " K")
    _close(v, ref["V"][live], label + " V")
    # only committed rows were written
    written = np.count_nonzero(np.any(kc != 0, axis=-1))
    assert written == len(live) * cfg.n_kv_heads
    if cb is not None:
        c = orc.bf16_to_f64(cb)
        same = np.mean(c == ref["Cb"])
        assert same >= 0.999, same
        # half a bf16 step plus fp32 accumulation error; the latter scales with the
        # running partial sums (~ rms(C)), not with |C|, so it dominates tiny entries
        rms_c = float(np.sqrt(np.mean(ref["C"] ** 2)))
        assert np.all(np.abs(c - ref["C"]) <= 0.5 * ulp_bf16(ref["C"]) + 1e-4 * rms_c)


def test_ctx_proj_tiny_rows_on_64_row_weight_tiles():
    # 200 rows of the tiny shape: both products run on 16 activation tiles (MT = 16) with
    # 64-row weight tiles (their grids of 4 and 2 workgroups fill far less than half the
    # CUs), the fc product reading the layers in place, the K/V product the packed C.
    cfg = synth.CONFIGS["tiny"]
    n = 200
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32) + 100
    pos[::5] = -1
    _check(cfg, n, seq, pos, capacity=320, label="tiny 200 rows")


def test_ctx_proj_tiny_prefill_dense_and_paged():
    cfg = synth.CONFIGS["tiny"]
    n = 64
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32)
    _check(cfg, n, seq, pos, capacity=80, label="tiny prefill dense")
    table = np.array([[3, 0, 4, 1, 2]], np.int32)
    _check(cfg, n, seq, pos, capacity=0, table=table, num_pages=6, label="tiny prefill paged")


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b", "batched", "long_ctx"])
def test_ctx_proj_committed_block_rows(name):
    cfg = synth.CONFIGS[name]
    kv_len = synth.context_lengths(cfg)
    rng = np.random.default_rng(cfg.seed)
    pos = _commit_positions(kv_len, rng)
    seq = np.repeat(np.arange(cfg.batch, dtype=np.int32), 16)
    _check(cfg, 16 * cfg.batch, seq, pos, capacity=int(kv_len.max()) + 16, label=f"{name} block rows")


def test_ctx_proj_ragged_paged_block_rows():
    cfg = synth.CONFIGS["ragged"]
    at_len = synth.context_lengths(cfg)
    rng = np.random.default_rng(11)
    pos = _commit_positions(at_len, rng)
    seq = np.repeat(np.arange(cfg.batch, dtype=np.int32), 16)
    width = int((at_len.max() + 16 + 15) // 16)
    # Only the pages holding committed rows are backed (a shuffled pool); the
    # kernel reads the table only at those rows.
    need = sorted({(int(s), int(p) // 16) for s, p in zip(seq, pos) if p >= 0})
    perm = rng.permutation(len(need)).astype(np.int32)
    table = np.full((cfg.batch, width), -1, np.int32)
    for (s, pg), phys in zip(need, perm):
        table[s, pg] = phys
    _check(cfg, 16 * cfg.batch, seq, pos, capacity=0, table=table, num_pages=len(need), label="ragged paged")


# 300 rows: the tiled kernel, last row tile ragged; 200 rows: the skinny kernel's 16
# activation tiles (MT = 16) with the last 56 rows clamped; 80 rows: 6 tiles (MT = 6).
@pytest.mark.parametrize("n", [300, 200, 80])
def test_ctx_proj_prefill_chunk_with_ragged_row_tail(n):
    cfg = dataclasses.replace(synth.CONFIGS["qwen3_8b"], n_target_layers=2)
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32) + 1000
    pos[::7] = -1
    _check(cfg, n, seq, pos, capacity=1400, label=f"prefill {n} rows")


def test_ctx_proj_without_fc():
    cfg = synth.CONFIGS["tiny"]
    n = 40
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32)
    _check(cfg, n, seq, pos, capacity=80, with_fc=False, label="no fc")


def test_ctx_proj_bad_rows_flagged_and_skipped():
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], batch=2)
    n = 16
    seq = np.array([0] * 8 + [5] * 8, np.int32)          # sequence 5 does not exist
    pos = np.arange(n, dtype=np.int32)
    pos[3] = 500                                          # beyond capacity
    ref, kc, vc, cb, err = _run(cfg, n, seq, pos, capacity=80)
    assert err & dfl.DEVERR_ROW
    assert np.count_nonzero(np.any(kc != 0, axis=-1)) == 7 * cfg.n_kv_heads


# Above 256 rows (prefill chunks) the projection takes the tiled MFMA GEMM, whose A
# operand walks the layers' row pointers at run time and whose C is row-major.
def test_ctx_proj_qwen3_8b_full_prefill_2048_rows():
    cfg = synth.CONFIGS["qwen3_8b"]
    n = 2048
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32)
    _check(cfg, n, seq, pos, capacity=n + 16, label="qwen3_8b prefill 2048 rows x 5 layers")


def test_ctx_proj_ragged_prefill_1000_rows_strided_layers():
    # Two sequences' rows interleaved in runs, every ninth row uncommitted, and layer rows
    # 64 elements wider than the layer (ld_x > d_target; the padding holds NaN).
    cfg = dataclasses.replace(synth.CONFIGS["qwen3_8b"], batch=2, n_target_layers=3)
    n = 1000
    seq = (np.arange(n) // 37 % 2).astype(np.int32)
    pos = np.zeros(n, np.int32)
    for b in range(2):
        rows = np.nonzero(seq == b)[0]
        pos[rows] = 100 + 3 * b + np.arange(len(rows))
    pos[::9] = -1
    _check(cfg, n, seq, pos, capacity=700, label="ragged prefill 1000 rows, ld_x > d_target", ld_pad=64)


# Narrow layers on the tiled path: with 64-wide layers every K stage of the A operand
# starts a new layer, with 128-wide ones every second stage; 1024 columns of K take two
# K splits, the second starting inside the layer list.
@pytest.mark.parametrize("d_target", [64, 128])
def test_ctx_proj_tiled_narrow_layers(d_target):
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], n_target_layers=8, target_hidden=d_target)
    n = 600
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32) + 5
    pos[::11] = -1
    _check(cfg, n, seq, pos, capacity=n + 16, label=f"tiled, 8 layers of {d_target}")


def test_ctx_proj_paged_prefill_700_rows():
    cfg = dataclasses.replace(synth.CONFIGS["qwen3_8b"], n_target_layers=2)
    n = 700
    seq = np.zeros(n, np.int32)
    pos = np.arange(n, dtype=np.int32) + 5
    width = (n + 5 + 15) // 16
    table = np.random.default_rng(3).permutation(width).astype(np.int32)[None, :]
    _check(cfg, n, seq, pos, capacity=0, table=table, num_pages=width, label="paged prefill 700 rows")


def test_ctx_proj_skinny_rows_strided_layers():
    # Per-cycle rows (<= 256) read the layers in place too: layer rows ld_x > d_target apart.
    cfg = synth.CONFIGS["batched"]
    n = 128
    seq = np.repeat(np.arange(cfg.batch, dtype=np.int32), 16)
    pos = np.tile(np.arange(16, dtype=np.int32), cfg.batch) + 200
    pos[5::16] = -1
    _check(cfg, n, seq, pos, capacity=240, label="batched block rows, ld_x > d_target", ld_pad=128)


@pytest.mark.parametrize("paged", [False, True])
def test_ctx_proj_sliding_window_ring_rows(paged):
    # Committed rows of 8 sequences straddle the ring's wrap (window 96 rows): position
    # p goes to row p mod 96, and nothing else in the ring is written.
    cfg = synth.CONFIGS["batched"]
    W = 96
    kv_len = np.array([90, 85, 95, 96, 1000, 190, 5, 300], np.int32)
    pos = _commit_positions(kv_len, np.random.default_rng(4))
    seq = np.repeat(np.arange(cfg.batch, dtype=np.int32), 16)
    if paged:
        table = np.random.default_rng(5).permutation(cfg.batch * W // 16).astype(np.int32).reshape(cfg.batch, -1)
        _check(cfg, 16 * cfg.batch, seq, pos, capacity=0, table=table, num_pages=cfg.batch * W // 16,
               label="window 96, paged ring", window=W)
    else:
        _check(cfg, 16 * cfg.batch, seq, pos, capacity=W, label="window 96, dense ring", window=W)
