"""GPU parity of the draft layer around the attention: dflash_rmsnorm and
dflash_draft_layer_post against the oracle (random Qwen3-shaped weights).

Tolerances, from the arithmetic:
* RMSNorm: the factor is computed in fp64 on both sides and each output rounded
  once from its fp64 value, so they agree bit for bit unless an exact output lies
  within fp64 summation-order error of a bf16 midpoint: >= 99.99% identical, the
  rest one bf16 step apart.
* Layer after the attention: the products accumulate in fp32 (the oracle's are
  exact), so a stored intermediate (x1, n2, the MLP activation) lands one bf16 step
  off wherever its exact value lies within fp32 accumulation error of a rounding
  midpoint (measured at the batched shape: 0.009% of x1 and n2, 0.4% of the
  activations).  A flipped x1 element moves the same output element by one step of
  x1 (x_out = x1 + MLP, and the MLP part can cancel x1 almost exactly, so this step
  can dwarf the output's own).  Each flipped activation moves an output by
  ulp(act) |W_down| ~ 2^-8 * 0.7 * 0.02 ~ 5.5e-5.  In most rows ~0.4% of the
  activations flip; in a row with a flipped n2 element every gate / up output moves by
  ~ulp(n2) * 0.02 ~ 1.6e-4, which flips ~10% of that row's activations (measured: up to
  ~1500 of 12288), and their effects add like a random walk to sigma ~ 2e-3 ~ 8e-4 of
  rms(out) (2.5 - 3.7).  Hence per element |gpu - ref| <= ulp_bf16(x1_ref) +
  ulp_bf16(ref) + 5e-3 rms(ref) (about 6 sigma), normwise <= 4e-3, and >= 99% of
  elements within one ulp_bf16(ref) + 1e-4 rms (a systematic error would move far more).
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from tests.gpu_util import DEV, host_u16, log, u16

pytestmark = pytest.mark.gpu


def ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("name,ld_pad", [("tiny", 0), ("batched", 0), ("long_ctx", 64), ("qwen3_8b", 8)])
def test_rmsnorm(name, ld_pad):
    cfg = synth.CONFIGS[name]
    li = synth.draft_layer_inputs(cfg)
    M, D = li.x.shape
    xs = torch.full((M, D + ld_pad), 0x7FC0, dtype=torch.int16, device=DEV)   # NaN padding is never read
    xs[:, :D] = u16(li.x)
    out = torch.full((M, D + 2 * ld_pad), -1, dtype=torch.int16, device=DEV)
    dfl.dflash_rmsnorm(xs[:, :D], u16(li.w_in), li.eps, out[:, :D])
    torch.cuda.synchronize()
    got = orc.bf16_to_f64(host_u16(out)[:, :D])
    ref = orc.rmsnorm_ref(orc.bf16_to_f64(li.x), li.w_in, li.eps)
    same = float(np.mean(got == ref))
    log(f"rmsnorm {name}: {100 * same:.4f}% bit-identical")
    assert same >= 0.9999
    assert np.all(np.abs(got - ref) <= ulp_bf16(ref))
    assert np.all(host_u16(out)[:, D:] == 0xFFFF)                              # row padding untouched


def _layer(cfg, li):
    B = li.x.shape[0] // 16
    dims = dfl.make_dims(B, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, hidden=cfg.hidden)
    ws = dfl.workspace(dfl.dflash_draft_layer_post_workspace_size(dims, cfg.inter), DEV)
    out = torch.zeros(li.x.shape, dtype=torch.int16, device=DEV)
    attn = torch.from_numpy(li.attn).to(DEV)
    log(f"draft layer {cfg.name}: M={li.x.shape[0]} D={cfg.hidden} I={cfg.inter} ws={ws.numel()} B")
    dfl.dflash_draft_layer_post(dims, cfg.inter, u16(li.x), attn, u16(li.w_o), u16(li.w_post), u16(li.w_gate),
                                u16(li.w_up), u16(li.w_down), li.eps, out, ws)
    torch.cuda.synchronize()
    return orc.bf16_to_f64(host_u16(out))


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b", "batched", "long_ctx"])
def test_draft_layer_post(name):
    cfg = synth.CONFIGS[name]
    li = synth.draft_layer_inputs(cfg)
    got = _layer(cfg, li)
    ref = orc.draft_layer_post_ref(li.x, li.attn, li.w_o, li.w_post, li.w_gate, li.w_up, li.w_down, li.eps)
    want = ref["x2"]
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = np.abs(got - want)
    worst = float(np.max(err / (ulp_bf16(ref["x1"]) + ulp_bf16(want) + 5e-3 * rms)))
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    tight = float(np.mean(err <= ulp_bf16(want) + 1e-4 * rms))
    same = float(np.mean(got == want))
    inc = ref["x2_exact"] - ref["x1"]
    log(f"draft layer {name}: max err/bound {worst:.3f}, normwise rel {rel:.2e}, within one ulp "
        f"{100 * tight:.3f}%, identical {100 * same:.2f}%, rms {rms:.3f} "
        f"(MLP increment rms {float(np.sqrt(np.mean(inc ** 2))):.3f})")
    assert np.all(np.isfinite(got))
    assert worst <= 1.0, worst
    assert rel <= 4e-3, rel
    assert tight >= 0.99, tight


def test_draft_layer_post_sizes_and_workspace_reuse():
    # Four batch sizes on one buffer sized for the largest (the workspace keeps no state).
    # 192, 80, 32 and 48 rows: 16, 6, 2 and 4 activation tiles, the gate/up product with
    # its SwiGLU epilogue (one K split) at 192, 80 and 48 rows and with separate partials
    # (two splits) at 32.
    cfg = synth.CONFIGS["tiny"]
    big = dataclasses.replace(cfg, batch=12)
    dims = dfl.make_dims(12, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, hidden=cfg.hidden)
    ws = dfl.workspace(dfl.dflash_draft_layer_post_workspace_size(dims, cfg.inter), DEV)
    for B in (12, 5, 2, 3):
        c = dataclasses.replace(big, batch=B)
        li = synth.draft_layer_inputs(c, seed=900 + B)
        d = dfl.make_dims(B, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, hidden=cfg.hidden)
        out = torch.zeros(li.x.shape, dtype=torch.int16, device=DEV)
        dfl.dflash_draft_layer_post(d, cfg.inter, u16(li.x), torch.from_numpy(li.attn).to(DEV), u16(li.w_o),
                                    u16(li.w_post), u16(li.w_gate), u16(li.w_up), u16(li.w_down), li.eps, out, ws)
        torch.cuda.synchronize()
        got = orc.bf16_to_f64(host_u16(out))
        r = orc.draft_layer_post_ref(li.x, li.attn, li.w_o, li.w_post, li.w_gate, li.w_up, li.w_down, li.eps)
        want = r["x2"]
        bound = ulp_bf16(r["x1"]) + ulp_bf16(want) + 5e-3 * float(np.sqrt(np.mean(want ** 2)))
        assert np.all(np.abs(got - want) <= bound)
