#!/usr/bin/env python3
"""Benchmark of the DFlash draft hot path on one MI355X.

One step = one pass of the whole hot path over one batch, in cycle order:
  1. dflash_block_attn   dual-source block attention (draft layer) over [ctx ; block]
  2. dflash_verify_accept greedy verify of the 16 block positions: argmax, accept,
                          next staged token, commit positions, KV-length crop
  3. dflash_ctx_proj     projection of the committed rows' target hidden states into
                          the context cache (fc + K/V + RoPE + scatter)
A pass after the timed steps also times the rest of a cycle that runs on the device
(dflash_draft_argmax and dflash_block_qkv), reported beside the step, not in it.
Everything runs on seeded synthetic inputs of the batched-serving workload (B=8, L=8192, 32q/8kv,
d=128, 5x4096 target features, V=151936).  Inputs are resident in HBM and rotated
over several copies so the bytes touched between two uses of one copy exceed 2 GiB
(4x the 256 MB Infinity Cache): the numbers are cold-cache numbers.

Prints one JSON line.  `value` = draft tokens per second through the whole step
(B*16 block tokens per step).  `roofline` describes the dominant kernel (block
attention): algorithmic HBM bytes per launch over its mean launch time, measured
with HIP events (created without the system-scope fence, which only adds a cache
writeback) on the launch stream inside the timed region.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per block-attention call (one kernel; splits merged inside it) on the batched
# workload, from two rocprofv3 counter passes over this script (FETCH_SIZE, then
# WRITE_SIZE), each scaled by what the same counter reads for a device-to-device
# copy of known size (--copy-mib).  Valid only for the kernel sources it was taken
# on: any change to them turns the reported traffic into null.
ATTN_TRAFFIC_SOURCES = ("block_diffusion_draft_proj_amd/csrc/block_attn.hip",
                        "block_diffusion_draft_proj_amd/csrc/common.h",
                        "block_diffusion_draft_proj_amd/csrc/launch.h",
                        "block_diffusion_draft_proj_amd/csrc/api.cpp")
ATTN_TRAFFIC = {"sha256": "23037427eeb941e41dd5c6434b069e214b9cb0d73d26cf1da1a0b3295ddc1d26",
                "workload": "batched", "read": 273973818, "write": 8505784}


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    t = ATTN_TRAFFIC
    if t is None or t["workload"] != workload or t["sha256"] != sources_sha256(ATTN_TRAFFIC_SOURCES):
        return None
    return int(t["read"] + t["write"])


class HipTimingEvents:
    """Timing events on one HIP stream, created with hipEventDisableSystemFence.

    A default HIP event performs a system-scope fence when it is recorded: an L2
    writeback and invalidate that costs several microseconds of GPU time per event and
    slows the kernel after it.  Events that only time kernels do not need that fence,
    and without it the per-kernel spans agree with the profiler's kernel durations.
    Uses the HIP runtime that torch has already loaded (same soname, one instance)."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, stream_handle):
        import ctypes
        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._stream = ctypes.c_void_p(stream_handle)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._ok(self._hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)),
                     "hipEventCreateWithFlags")
            self.ev.append(e)

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, i):
        self._ok(self._hip.hipEventRecord(self.ev[i], self._stream), "hipEventRecord")

    def elapsed_ms(self, i, j):
        f = self._ct.c_float()
        self._ok(self._hip.hipEventElapsedTime(self._ct.byref(f), self.ev[i], self.ev[j]), "hipEventElapsedTime")
        return f.value

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def copy_yardstick(mib):
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    # On a freshly started GPU the first ~60 steps (~10 ms) run up to 10% slower while
    # the clocks settle (per-step spans measured on MI355X).  Before the warm-up steps,
    # the step runs untimed for this long; reported as its own field ("settle").
    ap.add_argument("--settle-s", type=float, default=2.0)
    ap.add_argument("--config", default="batched")
    ap.add_argument("--rotate", type=int, default=0, help="input copies (0 = enough for >= 2 GiB between reuses)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-rows", type=int, default=0,
                    help="instead of the step, time dflash_ctx_proj over one prefill chunk of this many rows "
                         "(qwen3_8b-shaped: 5 x 4096 target features -> 4096 -> 8 x 128 K/V) and print its "
                         "TFLOP/s against the bf16 MFMA peak")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the step, copy a buffer of this many MiB device to device 5 times: the "
                         "yardstick that converts the HBM byte counters of a profiler into bytes")
    return ap.parse_args()


def attn_bytes(cfg, ctx_len):
    B, Hq, Hkv, d = len(ctx_len), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    b = 4 * Hkv * d * int(ctx_len.sum()) + 2 * 16 * B * Hq * d + 4 * 16 * B * Hkv * d + 4 * 16 * B * Hq * d + 4 * B
    if cfg.page_size:
        b += 4 * int(((ctx_len + 15) // 16).sum())
    return b


def window_size(cfg, max_ctx):
    """The window the bench times the sliding-window attention with: half the longest
    context, a multiple of 16 (a whole number of pages), at least 16."""
    return max(16, (max_ctx // 2) // 16 * 16)


def verify_bytes(cfg, B):
    return 2 * 16 * B * cfg.vocab + 4 * 16 * B * 3 + 4 * B * 4


def draft_bytes(cfg, B):
    # the draft's logits at the 15 mask slots, the staged tokens in, the block out
    return B * 15 * cfg.vocab * 2 + B * 4 + B * 16 * 4


def qkv_bytes(cfg, B):
    # the fused q/k/v weight, the block hidden states, and q, k, v out
    n_out = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    return 2 * (n_out * cfg.hidden + 16 * B * cfg.hidden + 16 * B * n_out)


def fused_bytes(cfg, ctx_len):
    # the fused q/k/v weight and the block hidden states in, the context K/V cache read,
    # the fp32 attention output out (the block's q/k/v never leave the call)
    B, Hq, Hkv, d = len(ctx_len), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    n_out = (Hq + 2 * Hkv) * d
    b = 2 * (n_out * cfg.hidden + 16 * B * cfg.hidden) + 4 * Hkv * d * int(ctx_len.sum()) + 4 * 16 * B * Hq * d + 4 * B
    if cfg.page_size:
        b += 4 * int(((ctx_len + 15) // 16).sum())
    return b


def layer_bytes(cfg, B):
    # the draft layer around the attention: input RMSNorm (x in, n1 out, weight) and the
    # post-attention part (o_proj, gate/up, down weights; x and the fp32 attention output
    # in, x_out out; the post-norm weight)
    M, D, A, I = 16 * B, cfg.hidden, cfg.n_q_heads * cfg.head_dim, cfg.inter
    norm = 2 * M * D * 2 + 2 * D
    post = 2 * (D * A + 2 * I * D + D * I) + 4 * M * A + 2 * M * D * 2 + 2 * D
    return norm, post


def replay_bytes(B, H, dk, dv, accept):
    # the fp32 state in and out, and the accepted steps of the tape (k bf16, delta fp32, g)
    steps = int((accept.astype(np.int64) + 1).sum())
    return 2 * 4 * B * H * dv * dk + steps * H * (2 * dk + 4 * dv + 4) + 4 * B


def proj_bytes(cfg, M, committed):
    kvw = cfg.n_kv_heads * cfg.head_dim
    return (2 * cfg.hidden * cfg.ctx_width + 2 * 2 * kvw * cfg.hidden + 2 * M * cfg.ctx_width
            + 2 * 2 * committed * kvw + 8 * M)


def cpu_baseline(cfg, at, vi, pj, row_pos, t_budget=20.0, repeats=3):
    """Oracle on a bounded sample of the same step, scaled to draft tokens/s; the
    median of ``repeats`` timings of the sample."""
    import numpy as np
    from oracle import dflash_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    B, Hkv = len(at.ctx_len), cfg.n_kv_heads
    units = [(b, g) for b in range(B) for g in range(Hkv)]
    nb = max(1, min(B, 2))
    m = 32
    budget = t_budget / repeats
    n_u = len(units)
    times = []
    for _ in range(repeats):
        done = 0
        t0 = time.perf_counter()
        for (b, g) in units[:n_u]:
            orc.block_attn_ref(at.q_blk, at.k_blk, at.v_blk, at.k_cache, at.v_cache, at.ctx_len, cfg.rope_base,
                               units=[(b, g)])
            done += 1
            if time.perf_counter() - t0 > budget * 0.4:
                break
        n_u = done  # later repeats time the same sample of units
        t_attn = (time.perf_counter() - t0) / n_u * len(units)
        t0 = time.perf_counter()
        orc.verify_accept_ref(vi.logits[:nb], vi.block_tokens[:nb], vi.kv_len[:nb])
        t_ver = (time.perf_counter() - t0) / nb * B
        t0 = time.perf_counter()
        orc.ctx_proj_ref([x[:m] for x in pj.x_layers], pj.w_fc, pj.w_k, pj.w_v, row_pos[:m], Hkv, cfg.head_dim,
                         cfg.rope_base)
        t_proj = (time.perf_counter() - t0) / m * len(row_pos)
        times.append((t_attn + t_ver + t_proj, t_attn, t_ver, t_proj))
    t_step, t_attn, t_ver, t_proj = sorted(times)[len(times) // 2]
    return {"value": 16 * B / t_step, "unit": "draft tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_u} of {len(units)} attention units, verify of {nb} of {B} sequences, "
                      f"projection of {m} of {len(row_pos)} rows; scaled to one full step; median of "
                      f"{repeats} ({t_step:.2f} s/step: attn {t_attn:.2f}, verify {t_ver:.2f}, proj {t_proj:.2f})"}


def prefill(rows, steps, warmup):
    """One prefill chunk of the context projection (fc + K/V + RoPE + scatter), timed with
    HIP events per call; flops = 2 M (n_t D_t D + 2 D Hkv d)."""
    import torch
    from block_diffusion_draft_proj_amd import dflash as dfl
    from block_diffusion_draft_proj_amd import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["qwen3_8b"]
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    pj = synth.ctx_proj_inputs(cfg, 0, weights_only=True)
    Dt, nt, D, Hkv, d = cfg.target_hidden, cfg.n_target_layers, cfg.hidden, cfg.n_kv_heads, cfg.head_dim
    xs = [(torch.randn(rows, Dt, device=dev) * 1.0).to(torch.bfloat16).view(torch.int16) for _ in range(nt)]
    dims = dfl.make_dims(1, cfg.n_q_heads, Hkv, d, hidden=D, kv_capacity=rows + 16)
    kc = torch.zeros(1, Hkv, rows + 16, d, dtype=torch.int16, device=dev)
    vc = torch.zeros_like(kc)
    cos = torch.empty(rows + 32, d // 2, dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    dfl.dflash_rope_tables(cfg.rope_base, d, rows + 32, cos, sin)
    seq = torch.zeros(rows, dtype=torch.int32, device=dev)
    pos = torch.arange(rows, dtype=torch.int32, device=dev)
    ws = dfl.workspace(dfl.dflash_ctx_proj_workspace_size(dims, rows, nt, Dt), dev)
    wfc, wk, wv = u16(pj.w_fc), u16(pj.w_k), u16(pj.w_v)
    call = lambda: dfl.dflash_ctx_proj(dims, xs, seq, pos, wfc, wk, wv, cos, sin, None, kc, vc, None, ws)
    for _ in range(warmup):
        call()
    ev = HipTimingEvents(2 * steps, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for s in range(steps):
        ev.record(2 * s)
        call()
        ev.record(2 * s + 1)
    torch.cuda.synchronize()
    t = float(np.mean([ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(steps)])) * 1e-3
    ev.close()
    flops = 2.0 * rows * (nt * Dt * D + 2 * D * Hkv * d)
    print(json.dumps({"prefill": {"rows": rows, "us": round(t * 1e6, 1), "flops": flops,
                                  "TFLOP_s": round(flops / t / 1e12, 1),
                                  "pct_bf16_mfma_peak": round(100 * flops / t / 2.5e15, 2),
                                  "workload": "qwen3_8b-shaped context projection, one chunk: "
                                              f"{rows} x {nt * Dt} -> {D} -> {2 * Hkv * d}"}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is a "
              f"design note, not a built path.", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_yardstick(args.copy_mib)
        return
    if args.prefill_rows:
        prefill(args.prefill_rows, max(1, min(args.steps, 20)), max(1, min(args.warmup, 5)))
        return
    import numpy as np
    import torch
    from block_diffusion_draft_proj_amd import dflash as dfl
    from block_diffusion_draft_proj_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(dev)

    at = synth.attn_inputs(cfg)
    vi = synth.verify_inputs(cfg, kv_len=at.ctx_len)
    B = len(at.ctx_len)
    M = 16 * B
    pj = synth.ctx_proj_inputs(cfg, M)
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    max_ctx = int(at.ctx_len.max())
    max_pos = max_ctx + 2 * synth.BLOCK

    dims = dfl.make_dims(B, Hq, Hkv, d, hidden=cfg.hidden, page_size=cfg.page_size, kv_capacity=at.capacity,
                         num_pages=at.num_pages)
    a_b = attn_bytes(cfg, at.ctx_len)
    v_b = verify_bytes(cfg, B)
    committed = int((vi.planted_accept + 1).sum())
    p_b = proj_bytes(cfg, M, committed)
    step_bytes = a_b + v_b + p_b
    R = args.rotate or max(2, int(np.ceil(2 * (1 << 30) / step_bytes)))  # >= 2 GiB between reuses

    # resident inputs: copy 0 from the seeded recipe, copies 1..R-1 are clones (cold addresses)
    q, k, v = u16(at.q_blk), u16(at.k_blk), u16(at.v_blk)
    kc0, vc0 = u16(at.k_cache), u16(at.v_cache)
    lg0 = u16(vi.logits)
    xs0 = [u16(x) for x in pj.x_layers]
    wfc0 = u16(pj.w_fc)
    kcs, vcs, lgs, xss, wfcs = [kc0], [vc0], [lg0], [xs0], [wfc0]
    for _ in range(R - 1):
        kcs.append(kc0.clone()); vcs.append(vc0.clone()); lgs.append(lg0.clone())
        xss.append([x.clone() for x in xs0]); wfcs.append(wfc0.clone())
    wk, wv = u16(pj.w_k), u16(pj.w_v)
    table = i32(at.page_table) if at.page_table is not None else None
    ctx = i32(at.ctx_len)
    blk = i32(vi.block_tokens)
    kv_in = i32(vi.kv_len)
    row_seq = i32(np.repeat(np.arange(B), 16))
    cos = torch.empty(max_pos, d // 2, dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    dfl.dflash_rope_tables(cfg.rope_base, d, max_pos, cos, sin)
    out = torch.empty(B, 16, Hq, d, dtype=torch.float32, device=dev)
    z = lambda *s: torch.zeros(*s, dtype=torch.int32, device=dev)
    post, acc, nxt, kv_out, commit = z(B, 16), z(B), z(B), z(B), z(B, 16)
    ws_a = dfl.workspace(dfl.dflash_block_attn_workspace_size(dims, max_ctx), dev)
    ws_v = dfl.workspace(dfl.dflash_verify_workspace_size(B, 16, cfg.vocab), dev)
    ws_p = dfl.workspace(dfl.dflash_ctx_proj_workspace_size(dims, M, cfg.n_target_layers, cfg.target_hidden), dev)
    torch.cuda.synchronize()

    # Timed steps carry two events, around the attention call (the roofline kernel).  Each
    # recorded event still costs the command processor a few microseconds between kernels,
    # so the verify / projection split comes from a short pass after the timed region,
    # with events after each of the three calls.
    # The same pass times the draft-side greedy tokens (dflash_draft_argmax), the step
    # before the verify in a decode loop; it is not part of the timed step.  It runs
    # at the end of each pass step, on the next copy of the logits, with the verify's
    # next_token as its staged tokens.
    N_SPLIT = 50
    PASS_HOLD_CYCLES = 2_000_000  # ~1 ms of the shader clock: longer than the host needs to enqueue a pass step
    NEV = 11
    tev = HipTimingEvents(2 * args.steps, torch.cuda.current_stream().cuda_stream)
    sev = HipTimingEvents(NEV * N_SPLIT, torch.cuda.current_stream().cuda_stream)
    dblk = z(B, 16)
    # ... and the block's own q / k / v (dflash_block_qkv), the attention's inputs,
    # into separate buffers so the attention's inputs stay as drawn.
    qi = synth.block_qkv_inputs(cfg)
    h_blk, w_qkv = u16(qi.h), u16(qi.w_qkv)
    q2, k2, v2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_q = dfl.workspace(dfl.dflash_block_qkv_workspace_size(dims), dev)
    # ... the draft layer around the attention (input RMSNorm; o_proj, post-norm, MLP),
    # on the attention output of the step, with random Qwen3-shaped weights ...
    li = synth.draft_layer_inputs(cfg, batch=B)
    lx, lw_in, lw_o, lw_post = u16(li.x), u16(li.w_in), u16(li.w_o), u16(li.w_post)
    lw_gate, lw_up, lw_down = u16(li.w_gate), u16(li.w_up), u16(li.w_down)
    n1 = torch.empty_like(lx)
    lx_out = torch.empty_like(lx)
    ws_l = dfl.workspace(dfl.dflash_draft_layer_post_workspace_size(dims, cfg.inter), dev)
    # ... and the rollback of a recurrent layer's state to the accepted prefix, with the
    # verify's accept lengths (32 heads of 128 x 128 state per sequence)
    GH, GD = 32, 128
    gi = synth.gdn_tape_inputs(B, GH, GD, GD, seed=cfg.seed)
    g_state, g_out = torch.from_numpy(gi.state).to(dev), torch.empty(B, GH, GD, GD, dtype=torch.float32, device=dev)
    g_k, g_g, g_d = u16(gi.k_tape), torch.from_numpy(gi.g_tape).to(dev), torch.from_numpy(gi.delta_tape).to(dev)
    # ... and the block's q/k/v with the attention in one call (dflash_block_qkv_attn), on
    # the same hidden states and weight as dflash_block_qkv, into its own output
    ws_f = dfl.workspace(dfl.dflash_block_qkv_attn_workspace_size(dims, max_ctx), dev)
    out_f = torch.empty_like(out)
    # ... and the attention over a sliding window (a ring cache of W rows per sequence and
    # kv head: the context is the last min(L, W) positions), on the same cache buffers
    W = window_size(cfg, max_ctx)
    dims_w = dfl.make_dims(B, Hq, Hkv, d, hidden=cfg.hidden, page_size=cfg.page_size, kv_capacity=at.capacity,
                           num_pages=at.num_pages, window=W)
    ws_w = dfl.workspace(dfl.dflash_block_attn_workspace_size(dims_w, max_ctx), dev)
    out_w = torch.empty_like(out)

    # The attention calls are prepared once per input copy (checks and argument conversion
    # done here), so the event before a call is followed at once by the launch: with an
    # idle GPU (the first timed step) the span would otherwise include the host's
    # marshalling time.
    attn_calls = [dfl.bind_block_attn(dims, q, k, v, kcs[i], vcs[i], table, ctx, max_ctx, cos, sin, out, ws_a)
                  for i in range(R)]
    attn_w_calls = [dfl.bind_block_attn(dims_w, q, k, v, kcs[i], vcs[i], table, ctx, max_ctx, cos, sin, out_w, ws_w)
                    for i in range(R)]

    def step(i, ev=None, base=0, split=False):
        if ev is not None:
            ev.record(base)
        attn_calls[i]()
        if ev is not None:
            ev.record(base + 1)
        dfl.dflash_verify_accept(lgs[i], blk, kv_in, post, acc, nxt, kv_out, commit, 0, None, ws_v)
        if split:
            ev.record(base + 2)
        dfl.dflash_ctx_proj(dims, xss[i], row_seq, commit.view(-1), wfcs[i], wk, wv, cos, sin, None, kcs[i],
                            vcs[i], table, ws_p)
        if split:
            ev.record(base + 3)
            dfl.dflash_draft_argmax(lgs[(i + 1) % R], nxt, dblk, ws_v)
            ev.record(base + 4)
            dfl.dflash_block_qkv(dims, h_blk, w_qkv, q2, k2, v2, ws_q)
            ev.record(base + 5)
            dfl.dflash_rmsnorm(lx, lw_in, li.eps, n1)
            ev.record(base + 6)
            dfl.dflash_draft_layer_post(dims, cfg.inter, lx, out, lw_o, lw_post, lw_gate, lw_up, lw_down, li.eps,
                                        lx_out, ws_l)
            ev.record(base + 7)
            dfl.dflash_gdn_tape_replay(g_state, g_out, g_k, g_g, g_d, acc)
            ev.record(base + 8)
            dfl.dflash_block_qkv_attn(dims, h_blk, w_qkv, kcs[i], vcs[i], table, ctx, max_ctx, cos, sin, out_f, ws_f)
            ev.record(base + 9)
            attn_w_calls[i]()
            ev.record(base + 10)

    n_settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(64):
            step(n_settle % R)
            n_settle += 1
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle
    for s in range(args.warmup):
        step(s % R)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s % R, tev, 2 * s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Each pass step starts behind a short spin kernel, so that the host has enqueued the
    # whole step before its first event fires: the calls then run back to back and the
    # spans hold GPU time only, not the host's argument checks between two calls.
    for s in range(N_SPLIT):
        torch.cuda._sleep(PASS_HOLD_CYCLES)
        step(s % R, sev, NEV * s, split=True)
    torch.cuda.synchronize()

    ms_step = (t1 - t0) / args.steps * 1e3
    t_attn = float(np.mean([tev.elapsed_ms(2 * s, 2 * s + 1) for s in range(args.steps)])) * 1e-3
    span = lambda i, j: float(np.mean([sev.elapsed_ms(NEV * s + i, NEV * s + j) for s in range(N_SPLIT)])) * 1e-3
    t_ver, t_proj, t_draft, t_qkv = span(1, 2), span(2, 3), span(3, 4), span(4, 5)
    t_norm, t_post, t_replay, t_fused = span(5, 6), span(6, 7), span(7, 8), span(8, 9)
    t_win = span(9, 10)
    f_b = fused_bytes(cfg, at.ctx_len)
    w_b = attn_bytes(cfg, np.minimum(at.ctx_len, W))
    nb, pb = layer_bytes(cfg, B)
    rb = replay_bytes(B, GH, GD, GD, acc.cpu().numpy())
    d_b = draft_bytes(cfg, B)
    q_b = qkv_bytes(cfg, B)
    tev.close()
    sev.close()
    ok = bool(np.array_equal(acc.cpu().numpy(), vi.planted_accept))
    attn_gbs = a_b / t_attn / 1e9
    res = {
        "metric": "block-attn draft tokens/s & HBM GB/s (% peak); verify cycles/s at 1 GPU",
        "value": round(16 * B / (ms_step * 1e-3), 1),
        "unit": "draft tokens/s (whole hot-path step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"seconds": round(t_settle, 3), "steps": n_settle,
                   "what": "untimed steps before the warm-up, while the GPU clocks settle"},
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded, resident in HBM, %d rotated copies, cold cache)" % R,
        "config": {"workload": f"{cfg.name}: B={B}, block=16, L={max_ctx if cfg.ragged is None else 'ragged'}, "
                               f"{Hq}q/{Hkv}kv, d={d}, ctx {cfg.n_target_layers}x{cfg.target_hidden}->"
                               f"{cfg.hidden}, V={cfg.vocab}", "batch": B, "block": 16},
        "block_attn": {"us": round(t_attn * 1e6, 2), "draft_tokens_per_s": round(16 * B / t_attn, 1),
                       "GB_s": round(attn_gbs, 1), "pct_hbm_peak": round(100 * attn_gbs / HBM_PEAK_GBS, 2),
                       "bytes": a_b},
        "verify": {"us": round(t_ver * 1e6, 2), "cycles_per_s": round(1 / t_ver, 1),
                   "committed_tokens_per_s": round(committed / t_ver, 1),
                   "GB_s": round(v_b / t_ver / 1e9, 1), "bytes": v_b, "accept_matches_planted": ok},
        "ctx_proj": {"us": round(t_proj * 1e6, 2), "GB_s": round(p_b / t_proj / 1e9, 1), "bytes": p_b,
                     "rows": M, "committed_rows": committed},
        "draft_argmax": {"us": round(t_draft * 1e6, 2), "GB_s": round(d_b / t_draft / 1e9, 1),
                         "pct_hbm_peak": round(100 * d_b / t_draft / 1e9 / HBM_PEAK_GBS, 2), "bytes": d_b,
                         "scope": "draft-side greedy tokens at the 15 mask slots; not in the timed step"},
        "block_qkv": {"us": round(t_qkv * 1e6, 2), "GB_s": round(q_b / t_qkv / 1e9, 1),
                      "pct_hbm_peak": round(100 * q_b / t_qkv / 1e9 / HBM_PEAK_GBS, 2), "bytes": q_b,
                      "scope": "the block's own q/k/v (two kernels: split-K GEMM, reduce); "
                               "not in the timed step"},
        "draft_layer": {"rmsnorm_us": round(t_norm * 1e6, 2), "post_us": round(t_post * 1e6, 2),
                        "post_GB_s": round(pb / t_post / 1e9, 1),
                        "post_pct_hbm_peak": round(100 * pb / t_post / 1e9 / HBM_PEAK_GBS, 2),
                        "bytes": {"rmsnorm": nb, "post": pb}, "intermediate": cfg.inter,
                        "forward_us": round((t_norm + t_qkv + t_attn + t_post) * 1e6, 2),
                        "scope": "one random-weight draft layer around the step's attention: input RMSNorm, "
                                 "then (after q/k/v and the attention) o_proj + residual, RMSNorm, SwiGLU MLP + "
                                 "residual; forward_us = rmsnorm + block_qkv + block_attn + post; not in the "
                                 "timed step"},
        "gdn_replay": {"us": round(t_replay * 1e6, 2), "GB_s": round(rb / t_replay / 1e9, 1),
                       "pct_hbm_peak": round(100 * rb / t_replay / 1e9 / HBM_PEAK_GBS, 2), "bytes": rb,
                       "shape": f"B={B}, 32 heads, 128x128 fp32 state, the verify's accept lengths",
                       "scope": "rollback of recurrent state to the accepted prefix; not in the timed step"},
        "block_qkv_attn": {"us": round(t_fused * 1e6, 2), "GB_s": round(f_b / t_fused / 1e9, 1),
                            "pct_hbm_peak": round(100 * f_b / t_fused / 1e9 / HBM_PEAK_GBS, 2), "bytes": f_b,
                            "unfused_us": round((t_qkv + t_attn) * 1e6, 2),
                            "scope": "the block's q/k/v and the attention in one call (split-K GEMM, a "
                                     "reduce that rotates Q into a bf16 hi/lo pair and K, then the attention); "
                                     "unfused_us = block_qkv + block_attn; not in the timed step"},
        "block_attn_window": {"window": W, "us": round(t_win * 1e6, 2), "GB_s": round(w_b / t_win / 1e9, 1),
                              "pct_hbm_peak": round(100 * w_b / t_win / 1e9 / HBM_PEAK_GBS, 2), "bytes": w_b,
                              "scope": "the attention over a sliding window: the context is the last min(L, W) "
                                       "positions of a ring cache of W rows; not in the timed step"},
        "timing": "block_attn: HIP events around every timed call; the other calls: events in a %d-step "
                  "pass after the timed region, each pass step enqueued behind a short spin kernel so that "
                  "its spans hold no host time" % N_SPLIT,
        "roofline": {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name),
                     "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": a_b},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, at, vi, pj, commit.view(-1).cpu().numpy())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
