"""Helpers shared by the GPU parity tests: host <-> device marshalling of the
synthetic inputs and calls through the C-ABI binding.  No method arithmetic."""
import sys

import numpy as np
import torch

from block_diffusion_draft_proj_amd import dflash as dfl
from block_diffusion_draft_proj_amd import synth

DEV = torch.device("cuda:0")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def rope_tables(head_dim: int, max_pos: int, base: float = 1.0e6):
    cos = torch.empty(max_pos, head_dim // 2, dtype=torch.float32, device=DEV)
    sin = torch.empty_like(cos)
    dfl.dflash_rope_tables(base, head_dim, max_pos, cos, sin)
    return cos, sin


def attn_dims(cfg: synth.Config, at: "synth.AttnInputs", window: int = 0) -> "dfl.dflash_dims":
    return dfl.make_dims(len(at.ctx_len), cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, hidden=cfg.hidden,
                         page_size=16 if at.page_table is not None else 0, kv_capacity=at.capacity,
                         num_pages=at.num_pages, window=window)


def run_block_attn(cfg: synth.Config, at: "synth.AttnInputs", max_ctx=None, ws=None, cos_sin=None,
                   ctx_len_override=None, window=0):
    """Runs dflash_block_attn on device copies of ``at``; returns (out, workspace)."""
    B = len(at.ctx_len)
    max_ctx = int(at.ctx_len.max()) if max_ctx is None else max_ctx
    dims = attn_dims(cfg, at, window)
    cos, sin = cos_sin if cos_sin is not None else rope_tables(cfg.head_dim, max_ctx + 2 * synth.BLOCK,
                                                              cfg.rope_base)
    if ws is None:
        ws = dfl.workspace(dfl.dflash_block_attn_workspace_size(dims, max_ctx), DEV)
    out = torch.full((B, synth.BLOCK, cfg.n_q_heads, cfg.head_dim), float("nan"), dtype=torch.float32,
                     device=DEV)
    ctx = at.ctx_len if ctx_len_override is None else ctx_len_override
    dfl.dflash_block_attn(dims, u16(at.q_blk), u16(at.k_blk), u16(at.v_blk), u16(at.k_cache), u16(at.v_cache),
                          None if at.page_table is None else i32(at.page_table), i32(ctx), max_ctx, cos, sin,
                          out, ws)
    torch.cuda.synchronize()
    return out, ws


def run_verify(logits: np.ndarray, block_tokens, kv_len, page_size=0, vocab=None, ws=None, alias_kv=False):
    B = logits.shape[0]
    ld = logits.shape[2]
    V = ld if vocab is None else vocab
    if ws is None:
        ws = dfl.workspace(dfl.dflash_verify_workspace_size(B, synth.BLOCK, V), DEV)
    z = lambda *s: torch.full(s, -7, dtype=torch.int32, device=DEV)
    post, acc, nxt, cp = z(B, 16), z(B), z(B), z(B, 16)
    kvi = i32(kv_len)
    kvo = kvi if alias_kv else z(B)
    npg = z(B) if page_size > 0 else None
    dfl.dflash_verify_accept(u16(logits), i32(block_tokens), kvi, post, acc, nxt, kvo, cp, page_size, npg, ws,
                             vocab=V)
    torch.cuda.synchronize()
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0, "device error word set"
    res = {"post": post.cpu().numpy(), "accept": acc.cpu().numpy(), "next": nxt.cpu().numpy(),
           "kv_len": kvo.cpu().numpy(), "commit_pos": cp.cpu().numpy()}
    if npg is not None:
        res["n_pages"] = npg.cpu().numpy()
    return res, ws


def run_draft(logits: np.ndarray, staged, vocab=None, ws=None, init=-7):
    """Runs dflash_draft_argmax; returns (block_tokens [B, 16] as numpy, workspace)."""
    B, ld = logits.shape[0], logits.shape[2]
    V = ld if vocab is None else vocab
    if ws is None:
        ws = dfl.workspace(dfl.dflash_verify_workspace_size(B, synth.BLOCK, V), DEV)
    blk = torch.full((B, synth.BLOCK), init, dtype=torch.int32, device=DEV)
    dfl.dflash_draft_argmax(u16(logits), None if staged is None else i32(staged), blk, ws, vocab=V)
    torch.cuda.synchronize()
    assert int(ws[:4].cpu().numpy().view(np.uint32)[0]) == 0, "device error word set"
    return blk.cpu().numpy(), ws
