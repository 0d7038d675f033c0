"""GPU parity of dflash_gdn_tape_replay (rollback of recurrent state to the
accepted prefix) against the oracle.

Tolerance, from the arithmetic: per replayed step the kernel evaluates
S * alpha + delta * k in fp32 (three roundings, each <= 2^-24 relative) with
alpha = expf(g) (<= 2 ulp), while the oracle is float64; errors of earlier steps
are scaled by alpha <= 1.  So per element
|gpu - ref| <= 2^-21 * sum_{t <= a} (|alpha_t S_{t-1}| + |delta_t k_t| + |S_t|),
evaluated from the oracle's own intermediate states.
"""
import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from tests.gpu_util import DEV, i32, log, u16

pytestmark = pytest.mark.gpu


def _bound(inp, accept):
    B = inp.state.shape[0]
    k = orc.bf16_to_f64(inp.k_tape)
    tot = np.zeros(inp.state.shape)
    prev = inp.state.astype(np.float64)
    for t in range(16):
        cur = orc.gdn_replay_ref(inp.state, inp.k_tape, inp.g_tape, inp.delta_tape, np.full(B, t))
        alpha = np.exp(inp.g_tape[:, t].astype(np.float64))[:, :, None, None]
        term = np.abs(alpha * prev) + np.abs(inp.delta_tape[:, t].astype(np.float64)[:, :, :, None] *
                                             k[:, t][:, :, None, :]) + np.abs(cur)
        live = (t <= np.asarray(accept))[:, None, None, None]
        tot += np.where(live, term, 0.0)
        prev = cur
    return 2.0 ** -21 * tot


def _run(inp, accept, in_place):
    st = torch.from_numpy(inp.state).to(DEV)
    out = st if in_place else torch.full_like(st, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dfl.dflash_gdn_tape_replay(st, out, u16(inp.k_tape), torch.from_numpy(inp.g_tape).to(DEV),
                               torch.from_numpy(inp.delta_tape).to(DEV), i32(accept), err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.cpu()[0])


@pytest.mark.parametrize("in_place", [False, True])
# The kernel takes 16 state rows per workgroup where 32 rows would give fewer than 2048
# workgroups, else 32: the last two shapes take the 32-row form (the last with a ragged d_v).
@pytest.mark.parametrize("B,H,dk,dv", [(1, 2, 64, 64), (8, 32, 128, 128), (3, 3, 96, 40), (16, 1, 4, 1),
                                       (16, 32, 64, 128), (20, 32, 64, 100)])
def test_gdn_replay_matches_oracle(B, H, dk, dv, in_place):
    inp = synth.gdn_tape_inputs(B, H, dk, dv, seed=B * 1000 + dk)
    accept = inp.accept if B != 16 else np.arange(16, dtype=np.int32)   # every accept length once
    got, err = _run(inp, accept, in_place)
    ref = orc.gdn_replay_ref(inp.state, inp.k_tape, inp.g_tape, inp.delta_tape, accept)
    bound = _bound(inp, accept)
    worst = float(np.max(np.abs(got - ref) / bound))
    log(f"gdn replay B={B} H={H} dk={dk} dv={dv} in_place={in_place} accept={accept.tolist()[:8]}: "
        f"max err/bound {worst:.3f}, max-abs err {float(np.max(np.abs(got - ref))):.2e}")
    assert err == 0
    assert worst <= 1.0


def test_gdn_replay_flags_and_clamps_an_accept_length_out_of_range():
    inp = synth.gdn_tape_inputs(3, 2, 64, 64, seed=7)
    accept = np.array([3, 99, -4], np.int32)
    got, err = _run(inp, accept, False)
    assert err & dfl.DEVERR_ACCEPT
    ref = orc.gdn_replay_ref(inp.state, inp.k_tape, inp.g_tape, inp.delta_tape, np.array([3, 15, 0]))
    assert np.max(np.abs(got - ref)) <= 1e-5
