"""Python binding of the DFlash hot-path C ABI (``include/dflash.h``).

Argument marshalling only: each function checks tensor dtypes / devices /
contiguity, passes raw device pointers and the current HIP stream to the entry
point of the same name in ``lib/libdflash.so``, and raises ``DflashError`` on a
non-zero status.  All computation happens in the library's HIP kernels; there is
no fallback path.  Importing this module fails loudly if the library has not
been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

# DFLASH_LIB names another build of the same library (the host-sanitizer build of
# build_sanitized.py); by default the in-tree build.
_LIB_PATH = os.environ.get("DFLASH_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                         "libdflash.so")

BLOCK = 16
DEVERR_CTX_LEN, DEVERR_PAGE_ID, DEVERR_ROW, DEVERR_MERGE, DEVERR_XCD, DEVERR_ACCEPT = 1, 2, 4, 8, 16, 32

_c_int, _c_i64, _c_sz, _c_f, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p


class dflash_dims(ctypes.Structure):
    _fields_ = [
        ("batch", _c_int), ("block", _c_int), ("n_q_heads", _c_int), ("n_kv_heads", _c_int),
        ("head_dim", _c_int), ("hidden", _c_int), ("page_size", _c_int), ("kv_capacity", _c_int),
        ("num_pages", _c_int), ("softmax_scale", _c_f), ("window", _c_int),
    ]


class DflashError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: status {code} ({msg})")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build the HIP library first "
                          f"(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(dflash_dims)
    sig = {
        "dflash_status_str": (ctypes.c_char_p, [_c_int]),
        "dflash_version": (_c_int, []),
        "dflash_rope_tables": (_c_int, [_c_f, _c_int, _c_int, _vp, _vp, _vp]),
        "dflash_ctx_proj_workspace_size": (_c_sz, [P, _c_int, _c_int, _c_int]),
        "dflash_ctx_proj": (_c_int, [P, _c_int, ctypes.POINTER(_vp), _c_int, _c_int, _c_i64, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp]),
        "dflash_block_attn_workspace_size": (_c_sz, [P, _c_int]),
        "dflash_block_attn": (_c_int, [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int,
                                       _vp, _vp, _c_sz, _vp]),
        "dflash_block_attn_noalloc": (_c_int, [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int,
                                               _vp, _vp, _vp]),
        "dflash_rmsnorm": (_c_int, [_c_int, _c_int, _vp, _c_i64, _vp, _c_f, _vp, _c_i64, _vp]),
        "dflash_draft_layer_post_workspace_size": (_c_sz, [P, _c_int]),
        "dflash_draft_layer_post": (_c_int, [P, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_f, _vp, _vp, _c_sz,
                                             _vp]),
        "dflash_gdn_tape_replay": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "dflash_block_qkv_attn_workspace_size": (_c_sz, [P, _c_int]),
        "dflash_block_qkv_attn": (_c_int, [P, _vp, _c_i64, _vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp,
                                           _vp, _c_sz, _vp]),
        "dflash_verify_workspace_size": (_c_sz, [_c_int, _c_int, _c_int]),
        "dflash_draft_argmax": (_c_int, [_c_int, _c_int, _c_int, _vp, _c_i64, _vp, _vp, _vp, _c_sz, _vp]),
        "dflash_block_qkv_workspace_size": (_c_sz, [P]),
        "dflash_block_qkv": (_c_int, [P, _vp, _c_i64, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp]),
        "dflash_verify_accept": (_c_int, [_c_int, _c_int, _c_int, _vp, _c_i64, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _c_int, _vp, _vp, _c_sz, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()
LIB_PATH = _LIB_PATH

# Names the public header declares (kept in step with include/dflash.h).
EXPORTS = (
    "dflash_status_str", "dflash_version", "dflash_rope_tables", "dflash_ctx_proj_workspace_size",
    "dflash_ctx_proj", "dflash_block_attn_workspace_size", "dflash_block_attn",
    "dflash_verify_workspace_size", "dflash_verify_accept", "dflash_draft_argmax",
    "dflash_block_qkv_workspace_size", "dflash_block_qkv", "dflash_block_attn_noalloc",
    "dflash_rmsnorm", "dflash_draft_layer_post_workspace_size", "dflash_draft_layer_post",
    "dflash_gdn_tape_replay", "dflash_block_qkv_attn_workspace_size", "dflash_block_qkv_attn",
)
NOALLOC_SCRATCH_BYTES = 32 << 20


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise DflashError(fn, code, dflash_status_str(code))


def _stream(stream) -> _vp:
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _dev(t: Optional[torch.Tensor], name: str, dtypes, contiguous: bool = True) -> _vp:
    if t is None:
        return _vp(None)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _vp(t.data_ptr())


def _numel(t: Optional[torch.Tensor], want: int, name: str, at_least: bool = False) -> None:
    """Size check before a pointer is handed over: the kernels trust these sizes."""
    if t is None:
        return
    n = t.numel()
    if (n < want) if at_least else (n != want):
        raise ValueError(f"{name} holds {n} elements, {'at least ' if at_least else ''}{want} needed")


def _cache_numel(dims: "dflash_dims") -> int:
    if dims.page_size > 0:
        return dims.num_pages * dims.n_kv_heads * dims.page_size * dims.head_dim
    return dims.batch * dims.n_kv_heads * dims.kv_capacity * dims.head_dim


def _check_rope(rope_cos: torch.Tensor, rope_sin: torch.Tensor, head_dim: int) -> None:
    if rope_cos.dim() != 2 or rope_cos.shape[1] != head_dim // 2 or tuple(rope_sin.shape) != tuple(rope_cos.shape):
        raise ValueError(f"rope_cos / rope_sin must both be [max_pos, {head_dim // 2}]")


def make_dims(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, hidden: int = 0,
              page_size: int = 0, kv_capacity: int = 0, num_pages: int = 0,
              softmax_scale: float = 0.0, window: int = 0) -> dflash_dims:
    return dflash_dims(batch, BLOCK, n_q_heads, n_kv_heads, head_dim, hidden, page_size, kv_capacity,
                       num_pages, softmax_scale, window)


def dflash_status_str(code: int) -> str:
    return _lib.dflash_status_str(code).decode()


def dflash_version() -> int:
    return int(_lib.dflash_version())


def dflash_rope_tables(base: float, head_dim: int, max_pos: int, cos_out: torch.Tensor,
                       sin_out: torch.Tensor, stream=None) -> None:
    _numel(cos_out, max_pos * (head_dim // 2), "cos_out", at_least=True)
    _numel(sin_out, max_pos * (head_dim // 2), "sin_out", at_least=True)
    _check("dflash_rope_tables", _lib.dflash_rope_tables(
        base, head_dim, max_pos, _dev(cos_out, "cos_out", (torch.float32,)),
        _dev(sin_out, "sin_out", (torch.float32,)), _stream(stream)))


def dflash_ctx_proj_workspace_size(dims: dflash_dims, n_rows: int, n_layers: int, d_target: int) -> int:
    return int(_lib.dflash_ctx_proj_workspace_size(ctypes.byref(dims), n_rows, n_layers, d_target))


def dflash_ctx_proj(dims: dflash_dims, x_layers: Sequence[torch.Tensor], row_seq: torch.Tensor,
                    row_pos: torch.Tensor, w_fc: Optional[torch.Tensor], w_k: torch.Tensor,
                    w_v: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                    c_out: Optional[torch.Tensor], k_cache: torch.Tensor, v_cache: torch.Tensor,
                    page_table: Optional[torch.Tensor], workspace: torch.Tensor, stream=None) -> None:
    x0 = x_layers[0]
    n_rows, d_target = int(x0.shape[0]), int(x0.shape[1])
    ld = int(x0.stride(0))
    for i, x in enumerate(x_layers):
        if x.dim() != 2 or x.stride(1) != 1 or tuple(x.shape) != (n_rows, d_target) or x.stride(0) != ld:
            raise ValueError(f"x_layers[{i}] must be [n_rows, d_target] with unit inner stride and a common row stride")
    D, kvw = dims.hidden, dims.n_kv_heads * dims.head_dim
    _numel(row_seq, n_rows, "row_seq")
    _numel(row_pos, n_rows, "row_pos")
    _numel(w_fc, D * len(x_layers) * d_target, "w_fc")
    _numel(w_k, kvw * D, "w_k")
    _numel(w_v, kvw * D, "w_v")
    _numel(c_out, n_rows * D, "c_out", at_least=True)
    _numel(k_cache, _cache_numel(dims), "k_cache")
    _numel(v_cache, _cache_numel(dims), "v_cache")
    if dims.page_size > 0:
        _numel(page_table, dims.batch * dims.kv_capacity, "page_table")
    _check_rope(rope_cos, rope_sin, dims.head_dim)
    for i, x in enumerate(x_layers):
        _dev(x, f"x_layers[{i}]", _BF16, contiguous=False)
    arr = (_vp * len(x_layers))(*[x.data_ptr() for x in x_layers])
    _check("dflash_ctx_proj", _lib.dflash_ctx_proj(
        ctypes.byref(dims), n_rows, arr, len(x_layers), d_target, ld,
        _dev(row_seq, "row_seq", (torch.int32,)), _dev(row_pos, "row_pos", (torch.int32,)),
        _dev(w_fc, "w_fc", _BF16), _dev(w_k, "w_k", _BF16), _dev(w_v, "w_v", _BF16),
        _dev(rope_cos, "rope_cos", (torch.float32,)), _dev(rope_sin, "rope_sin", (torch.float32,)),
        int(rope_cos.shape[0]), _dev(c_out, "c_out", _BF16), _dev(k_cache, "k_cache", _BF16),
        _dev(v_cache, "v_cache", _BF16), _dev(page_table, "page_table", (torch.int32,)),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))


def dflash_block_attn_workspace_size(dims: dflash_dims, max_ctx_len: int) -> int:
    return int(_lib.dflash_block_attn_workspace_size(ctypes.byref(dims), max_ctx_len))


def dflash_block_attn(dims: dflash_dims, q_blk: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: Optional[torch.Tensor],
                      ctx_len: torch.Tensor, max_ctx_len: int, rope_cos: torch.Tensor,
                      rope_sin: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                      stream=None) -> None:
    B, Hq, Hkv, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    _numel(q_blk, B * BLOCK * Hq * d, "q_blk")
    _numel(k_blk, B * BLOCK * Hkv * d, "k_blk")
    _numel(v_blk, B * BLOCK * Hkv * d, "v_blk")
    _numel(k_cache, _cache_numel(dims), "k_cache")
    _numel(v_cache, _cache_numel(dims), "v_cache")
    if dims.page_size > 0:
        _numel(page_table, B * dims.kv_capacity, "page_table")
    _numel(ctx_len, B, "ctx_len")
    _numel(out, B * BLOCK * Hq * d, "out")
    _check_rope(rope_cos, rope_sin, d)
    _check("dflash_block_attn", _lib.dflash_block_attn(
        ctypes.byref(dims), _dev(q_blk, "q_blk", _BF16), _dev(k_blk, "k_blk", _BF16),
        _dev(v_blk, "v_blk", _BF16), _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(page_table, "page_table", (torch.int32,)), _dev(ctx_len, "ctx_len", (torch.int32,)),
        max_ctx_len, _dev(rope_cos, "rope_cos", (torch.float32,)),
        _dev(rope_sin, "rope_sin", (torch.float32,)), int(rope_cos.shape[0]),
        _dev(out, "out", (torch.float32,)), _dev(workspace, "workspace", (torch.uint8,)),
        workspace.numel(), _stream(stream)))


def bind_block_attn(dims: dflash_dims, q_blk: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: Optional[torch.Tensor],
                    ctx_len: torch.Tensor, max_ctx_len: int, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                    out: torch.Tensor, workspace: torch.Tensor, stream=None):
    """dflash_block_attn with every check and argument conversion done once, now: returns
    a function of no arguments that only calls the entry point (and raises on a non-zero
    status).  For loops that call the attention many times on the same buffers; the
    tensors must stay alive and in place while the function is used."""
    B, Hq, Hkv, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    _numel(q_blk, B * BLOCK * Hq * d, "q_blk")
    _numel(k_blk, B * BLOCK * Hkv * d, "k_blk")
    _numel(v_blk, B * BLOCK * Hkv * d, "v_blk")
    _numel(k_cache, _cache_numel(dims), "k_cache")
    _numel(v_cache, _cache_numel(dims), "v_cache")
    if dims.page_size > 0:
        _numel(page_table, B * dims.kv_capacity, "page_table")
    _numel(ctx_len, B, "ctx_len")
    _numel(out, B * BLOCK * Hq * d, "out")
    _check_rope(rope_cos, rope_sin, d)
    args = (ctypes.byref(dims), _dev(q_blk, "q_blk", _BF16), _dev(k_blk, "k_blk", _BF16),
            _dev(v_blk, "v_blk", _BF16), _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
            _dev(page_table, "page_table", (torch.int32,)), _dev(ctx_len, "ctx_len", (torch.int32,)),
            max_ctx_len, _dev(rope_cos, "rope_cos", (torch.float32,)),
            _dev(rope_sin, "rope_sin", (torch.float32,)), int(rope_cos.shape[0]),
            _dev(out, "out", (torch.float32,)), _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(),
            _stream(stream))
    fn = _lib.dflash_block_attn

    def call() -> None:
        code = fn(*args)
        if code != 0:
            _check("dflash_block_attn", code)
    return call


def dflash_block_attn_noalloc(dims: dflash_dims, q_blk: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor,
                              k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: Optional[torch.Tensor],
                              ctx_len: torch.Tensor, max_ctx_len: int, rope_cos: torch.Tensor,
                              rope_sin: torch.Tensor, out: torch.Tensor, dev_err: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    """dflash_block_attn on the library's static scratch (no workspace); the device
    error bits go to dev_err (one int32 on the device) when given."""
    B, Hq, Hkv, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    _numel(q_blk, B * BLOCK * Hq * d, "q_blk")
    _numel(k_blk, B * BLOCK * Hkv * d, "k_blk")
    _numel(v_blk, B * BLOCK * Hkv * d, "v_blk")
    _numel(k_cache, _cache_numel(dims), "k_cache")
    _numel(v_cache, _cache_numel(dims), "v_cache")
    if dims.page_size > 0:
        _numel(page_table, B * dims.kv_capacity, "page_table")
    _numel(ctx_len, B, "ctx_len")
    _numel(out, B * BLOCK * Hq * d, "out")
    _numel(dev_err, 1, "dev_err", at_least=True)
    _check_rope(rope_cos, rope_sin, d)
    _check("dflash_block_attn_noalloc", _lib.dflash_block_attn_noalloc(
        ctypes.byref(dims), _dev(q_blk, "q_blk", _BF16), _dev(k_blk, "k_blk", _BF16),
        _dev(v_blk, "v_blk", _BF16), _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(page_table, "page_table", (torch.int32,)), _dev(ctx_len, "ctx_len", (torch.int32,)),
        max_ctx_len, _dev(rope_cos, "rope_cos", (torch.float32,)),
        _dev(rope_sin, "rope_sin", (torch.float32,)), int(rope_cos.shape[0]),
        _dev(out, "out", (torch.float32,)), _dev(dev_err, "dev_err", (torch.int32,)), _stream(stream)))


def dflash_verify_workspace_size(batch: int, block: int, vocab: int) -> int:
    return int(_lib.dflash_verify_workspace_size(batch, block, vocab))


def dflash_verify_accept(logits: torch.Tensor, block_tokens: torch.Tensor, kv_len_in: torch.Tensor,
                         posterior: torch.Tensor, accept_len: torch.Tensor, next_token: torch.Tensor,
                         kv_len_out: torch.Tensor, commit_pos: Optional[torch.Tensor],
                         page_size: int, n_pages: Optional[torch.Tensor], workspace: torch.Tensor,
                         vocab: Optional[int] = None, stream=None) -> None:
    """logits [B, 16, ld] (ld >= vocab, multiple of 8); vocab defaults to ld."""
    if logits.dim() != 3 or logits.stride(2) != 1 or logits.stride(1) != logits.shape[2] \
            or logits.stride(0) != logits.shape[1] * logits.shape[2]:
        raise ValueError("logits must be a contiguous [B, 16, ld] tensor")
    B, blk, ld = (int(s) for s in logits.shape)
    for name, t, n in (("block_tokens", block_tokens, B * blk), ("kv_len_in", kv_len_in, B),
                       ("posterior", posterior, B * blk), ("accept_len", accept_len, B),
                       ("next_token", next_token, B), ("kv_len_out", kv_len_out, B),
                       ("commit_pos", commit_pos, B * blk), ("n_pages", n_pages, B)):
        _numel(t, n, name)
    _check("dflash_verify_accept", _lib.dflash_verify_accept(
        B, blk, ld if vocab is None else vocab, _dev(logits, "logits", _BF16), ld,
        _dev(block_tokens, "block_tokens", (torch.int32,)), _dev(kv_len_in, "kv_len_in", (torch.int32,)),
        _dev(posterior, "posterior", (torch.int32,)), _dev(accept_len, "accept_len", (torch.int32,)),
        _dev(next_token, "next_token", (torch.int32,)), _dev(kv_len_out, "kv_len_out", (torch.int32,)),
        _dev(commit_pos, "commit_pos", (torch.int32,)), page_size, _dev(n_pages, "n_pages", (torch.int32,)),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))


def dflash_block_qkv_workspace_size(dims: dflash_dims) -> int:
    return int(_lib.dflash_block_qkv_workspace_size(ctypes.byref(dims)))


def dflash_block_qkv(dims: dflash_dims, h: torch.Tensor, w_qkv: torch.Tensor, q_blk: torch.Tensor,
                     k_blk: torch.Tensor, v_blk: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """q/k/v of the block: h [16B, ld_h] bf16 (row stride ld_h), w_qkv [(Hq+2Hkv)d, hidden]."""
    if h.dim() != 2 or h.stride(1) != 1:
        raise ValueError("h must be a [rows, ld_h] tensor with unit inner stride")
    B, Hq, Hkv, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    if h.shape[0] != BLOCK * B or h.shape[1] < dims.hidden:
        raise ValueError(f"h must hold {BLOCK * B} rows of at least {dims.hidden} features")
    if tuple(w_qkv.shape) != ((Hq + 2 * Hkv) * d, dims.hidden):
        raise ValueError(f"w_qkv must be [{(Hq + 2 * Hkv) * d}, {dims.hidden}]")
    for name, t, heads in (("q_blk", q_blk, Hq), ("k_blk", k_blk, Hkv), ("v_blk", v_blk, Hkv)):
        if t.numel() != B * BLOCK * heads * d:
            raise ValueError(f"{name} must hold [{B}, {BLOCK}, {heads}, {d}] elements")
    _check("dflash_block_qkv", _lib.dflash_block_qkv(
        ctypes.byref(dims), _dev(h, "h", _BF16, contiguous=False), int(h.stride(0)),
        _dev(w_qkv, "w_qkv", _BF16), _dev(q_blk, "q_blk", _BF16), _dev(k_blk, "k_blk", _BF16),
        _dev(v_blk, "v_blk", _BF16), _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(),
        _stream(stream)))


def dflash_block_qkv_attn_workspace_size(dims: dflash_dims, max_ctx_len: int) -> int:
    return int(_lib.dflash_block_qkv_attn_workspace_size(ctypes.byref(dims), max_ctx_len))


def dflash_block_qkv_attn(dims: dflash_dims, h: torch.Tensor, w_qkv: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, page_table: Optional[torch.Tensor], ctx_len: torch.Tensor,
                          max_ctx_len: int, rope_cos: torch.Tensor, rope_sin: torch.Tensor, out: torch.Tensor,
                          workspace: torch.Tensor, stream=None) -> None:
    """The block's q/k/v and the attention in one call: h [16B, ld_h] bf16, w_qkv [(Hq+2Hkv)d, hidden]."""
    if h.dim() != 2 or h.stride(1) != 1:
        raise ValueError("h must be a [rows, ld_h] tensor with unit inner stride")
    B, Hq, Hkv, d = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    if h.shape[0] != BLOCK * B or h.shape[1] < dims.hidden:
        raise ValueError(f"h must hold {BLOCK * B} rows of at least {dims.hidden} features")
    _numel(w_qkv, (Hq + 2 * Hkv) * d * dims.hidden, "w_qkv")
    _numel(k_cache, _cache_numel(dims), "k_cache")
    _numel(v_cache, _cache_numel(dims), "v_cache")
    if dims.page_size > 0:
        _numel(page_table, B * dims.kv_capacity, "page_table")
    _numel(ctx_len, B, "ctx_len")
    _numel(out, B * BLOCK * Hq * d, "out")
    _check_rope(rope_cos, rope_sin, d)
    _check("dflash_block_qkv_attn", _lib.dflash_block_qkv_attn(
        ctypes.byref(dims), _dev(h, "h", _BF16, contiguous=False), int(h.stride(0)), _dev(w_qkv, "w_qkv", _BF16),
        _dev(k_cache, "k_cache", _BF16), _dev(v_cache, "v_cache", _BF16),
        _dev(page_table, "page_table", (torch.int32,)), _dev(ctx_len, "ctx_len", (torch.int32,)), max_ctx_len,
        _dev(rope_cos, "rope_cos", (torch.float32,)), _dev(rope_sin, "rope_sin", (torch.float32,)),
        int(rope_cos.shape[0]), _dev(out, "out", (torch.float32,)), _dev(workspace, "workspace", (torch.uint8,)),
        workspace.numel(), _stream(stream)))


def dflash_draft_argmax(logits: torch.Tensor, staged: Optional[torch.Tensor], block_tokens: torch.Tensor,
                        workspace: torch.Tensor, vocab: Optional[int] = None, stream=None) -> None:
    """Draft tokens: block_tokens[b, 1:16] = argmax of the draft's logits rows 1..15;
    block_tokens[b, 0] = staged[b] when staged is given.  logits [B, 16, ld]."""
    if logits.dim() != 3 or logits.stride(2) != 1 or logits.stride(1) != logits.shape[2] \
            or logits.stride(0) != logits.shape[1] * logits.shape[2]:
        raise ValueError("logits must be a contiguous [B, 16, ld] tensor")
    B, blk, ld = (int(s) for s in logits.shape)
    if block_tokens.numel() != B * blk or (staged is not None and staged.numel() < B):
        raise ValueError(f"block_tokens must be [{B}, {blk}] and staged hold {B} tokens")
    _check("dflash_draft_argmax", _lib.dflash_draft_argmax(
        B, blk, ld if vocab is None else vocab, _dev(logits, "logits", _BF16), ld,
        _dev(staged, "staged", (torch.int32,)), _dev(block_tokens, "block_tokens", (torch.int32,)),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))


def dflash_rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, out: torch.Tensor, stream=None) -> None:
    """out[r] = bf16(RMSNorm(x[r]; weight)): x, out [rows, >= hidden] with unit inner stride."""
    if x.dim() != 2 or out.dim() != 2 or x.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("x and out must be [rows, ld] tensors with unit inner stride")
    rows, hidden = int(x.shape[0]), int(weight.numel())
    if x.shape[1] < hidden or tuple(out.shape) != (rows, int(out.shape[1])) or out.shape[1] < hidden \
            or out.shape[0] != rows:
        raise ValueError(f"x and out must hold {rows} rows of at least {hidden} features")
    _check("dflash_rmsnorm", _lib.dflash_rmsnorm(
        rows, hidden, _dev(x, "x", _BF16, contiguous=False), int(x.stride(0)), _dev(weight, "weight", _BF16),
        float(eps), _dev(out, "out", _BF16, contiguous=False), int(out.stride(0)), _stream(stream)))


def dflash_draft_layer_post_workspace_size(dims: dflash_dims, intermediate: int) -> int:
    return int(_lib.dflash_draft_layer_post_workspace_size(ctypes.byref(dims), intermediate))


def dflash_draft_layer_post(dims: dflash_dims, intermediate: int, x: torch.Tensor, attn_out: torch.Tensor,
                            w_o: torch.Tensor, w_post_norm: torch.Tensor, w_gate: torch.Tensor,
                            w_up: torch.Tensor, w_down: torch.Tensor, eps: float, x_out: torch.Tensor,
                            workspace: torch.Tensor, stream=None) -> None:
    """o_proj + residual, RMSNorm, SwiGLU MLP + residual over the 16*batch block rows."""
    M, D, A, I = BLOCK * dims.batch, dims.hidden, dims.n_q_heads * dims.head_dim, intermediate
    for name, t, n in (("x", x, M * D), ("attn_out", attn_out, M * A), ("w_o", w_o, D * A),
                       ("w_post_norm", w_post_norm, D), ("w_gate", w_gate, I * D), ("w_up", w_up, I * D),
                       ("w_down", w_down, D * I), ("x_out", x_out, M * D)):
        _numel(t, n, name)
    _check("dflash_draft_layer_post", _lib.dflash_draft_layer_post(
        ctypes.byref(dims), I, _dev(x, "x", _BF16), _dev(attn_out, "attn_out", (torch.float32,)),
        _dev(w_o, "w_o", _BF16), _dev(w_post_norm, "w_post_norm", _BF16), _dev(w_gate, "w_gate", _BF16),
        _dev(w_up, "w_up", _BF16), _dev(w_down, "w_down", _BF16), float(eps), _dev(x_out, "x_out", _BF16),
        _dev(workspace, "workspace", (torch.uint8,)), workspace.numel(), _stream(stream)))


def dflash_gdn_tape_replay(state_in: torch.Tensor, state_out: torch.Tensor, k_tape: torch.Tensor,
                           g_tape: torch.Tensor, delta_tape: torch.Tensor, accept_len: torch.Tensor,
                           dev_err: Optional[torch.Tensor] = None, stream=None) -> None:
    """Recurrent state after the accepted steps: state [B, H, d_v, d_k] fp32 (out may be in),
    k_tape [B, 16, H, d_k] bf16, g_tape [B, 16, H] fp32, delta_tape [B, 16, H, d_v] fp32."""
    if state_in.dim() != 4:
        raise ValueError("state_in must be [batch, n_heads, d_v, d_k]")
    B, H, dv, dk = (int(x) for x in state_in.shape)
    for name, t, n in (("state_out", state_out, B * H * dv * dk), ("k_tape", k_tape, B * BLOCK * H * dk),
                       ("g_tape", g_tape, B * BLOCK * H), ("delta_tape", delta_tape, B * BLOCK * H * dv),
                       ("accept_len", accept_len, B)):
        _numel(t, n, name)
    _numel(dev_err, 1, "dev_err", at_least=True)
    _check("dflash_gdn_tape_replay", _lib.dflash_gdn_tape_replay(
        B, H, dk, dv, _dev(state_in, "state_in", (torch.float32,)), _dev(state_out, "state_out", (torch.float32,)),
        _dev(k_tape, "k_tape", _BF16), _dev(g_tape, "g_tape", (torch.float32,)),
        _dev(delta_tape, "delta_tape", (torch.float32,)), _dev(accept_len, "accept_len", (torch.int32,)),
        _dev(dev_err, "dev_err", (torch.int32,)), _stream(stream)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace buffer (the zero fill is needed once, before first use)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
