"""C-ABI checks that need no GPU: the library loads, exports every function the
public header declares, sizes workspaces, and rejects bad arguments on the host
before any HIP call (so nothing is launched and no output is touched)."""
import ctypes
import os
import re

import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")

# Validation-failure calls below pass fake (but aligned) addresses; they must never
# reach a device.  On a machine with a GPU a test bug could launch on them, so
# these run only where no device is visible.
no_device = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only validation tests")

FAKE = ctypes.c_void_p(0x100000)
MIS = ctypes.c_void_p(0x100008)  # 8-byte aligned, not 16


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 19, names
    lib = ctypes.CDLL(dfl.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(dfl.EXPORTS) == names


def test_status_strings_and_version():
    assert dfl.dflash_status_str(0) == "ok"
    for code in range(-7, 0):
        s = dfl.dflash_status_str(code)
        assert s and s != "unknown status"
    assert dfl.dflash_status_str(-99) == "unknown status"
    assert dfl.dflash_version() >> 16 == 1


def test_workspace_sizes():
    v = dfl.dflash_verify_workspace_size(8, 16, 151936)
    n_chunks = -(-151936 // 8192)
    counters = 8192 * 128                                       # fixed counter region, 1 MiB
    assert v == 256 + counters + 8 * 16 * 8 * n_chunks           # error word, counters, chunk keys
    assert dfl.dflash_verify_workspace_size(8192, 16, 10) > 0
    assert dfl.dflash_verify_workspace_size(8193, 16, 10) == 0
    assert dfl.dflash_verify_workspace_size(0, 16, 10) == 0
    assert dfl.dflash_verify_workspace_size(1, 15, 10) == 0
    dims = dfl.make_dims(8, 32, 8, 128, hidden=4096, kv_capacity=8208)
    a = dfl.dflash_block_attn_workspace_size(dims, 8192)
    assert a > 256 + counters + 8 * 8 * 4 and a % 256 == 0
    assert dfl.dflash_block_attn_workspace_size(dfl.make_dims(1024, 32, 8, 128, kv_capacity=64), 64) > 0
    assert dfl.dflash_block_attn_workspace_size(dfl.make_dims(1025, 32, 8, 128, kv_capacity=64), 64) == 0
    assert dfl.dflash_block_attn_workspace_size(dims, 16384) >= a
    bad = dfl.make_dims(8, 30, 8, 128, kv_capacity=8208)
    assert dfl.dflash_block_attn_workspace_size(bad, 8192) == 0
    p = dfl.dflash_ctx_proj_workspace_size(dims, 128, 5, 4096)
    assert p > 128 * 4096 * 2
    assert dfl.dflash_ctx_proj_workspace_size(dims, 0, 5, 4096) > 0


def _attn(dims, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, pt=None, ctx=FAKE, maxc=64, cos=FAKE, sin=FAKE,
             maxpos=128, out=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return dfl._lib.dflash_block_attn(ctypes.byref(dims), a["q"], a["k"], a["v"], a["kc"], a["vc"], a["pt"],
                                      a["ctx"], a["maxc"], a["cos"], a["sin"], a["maxpos"], a["out"], a["ws"],
                                      a["wsb"], None)


@no_device
def test_block_attn_rejects_bad_arguments():
    good = dfl.make_dims(2, 8, 2, 64, kv_capacity=80)
    assert _attn(dfl.make_dims(0, 8, 2, 64, kv_capacity=80)) == -2
    assert _attn(dfl.make_dims(2, 8, 3, 64, kv_capacity=80)) == -2           # Hq % Hkv
    assert _attn(dfl.make_dims(1025, 32, 8, 64, kv_capacity=80)) == -2       # units past the counter slots
    assert _attn(dfl.make_dims(2, 18, 2, 64, kv_capacity=80)) == -6          # group 9
    assert _attn(dfl.make_dims(2, 8, 2, 96, kv_capacity=80)) == -6           # head_dim
    assert _attn(dfl.make_dims(2, 8, 2, 64, page_size=8, kv_capacity=80)) == -6
    d = dfl.make_dims(2, 8, 2, 64, kv_capacity=80)
    d.block = 15
    assert _attn(d) == -2
    assert _attn(good, q=ctypes.c_void_p(None)) == -1
    assert _attn(good, ctx=ctypes.c_void_p(None)) == -1
    assert _attn(good, q=MIS) == -3
    assert _attn(good, maxc=81) == -5                                          # beyond capacity
    assert _attn(good, maxc=64, maxpos=79) == -5                               # RoPE table short
    assert _attn(good, maxc=-1) == -2
    assert _attn(good, ws=ctypes.c_void_p(None)) == -4
    assert _attn(good, wsb=16) == -4
    paged = dfl.make_dims(2, 8, 2, 64, page_size=16, kv_capacity=5, num_pages=10)
    assert _attn(paged) == -1                                                  # no page table
    assert _attn(paged, pt=FAKE, maxc=81) == -5                                # 5 pages * 16 = 80


def _verify(**kw):
    a = dict(B=2, blk=16, V=1000, logits=FAKE, ld=1000, bt=FAKE, kvi=FAKE, post=FAKE, acc=FAKE, nxt=FAKE,
             kvo=FAKE, cp=None, ps=0, npg=None, ws=FAKE, wsb=1 << 22)
    a.update(kw)
    return dfl._lib.dflash_verify_accept(a["B"], a["blk"], a["V"], a["logits"], a["ld"], a["bt"], a["kvi"],
                                         a["post"], a["acc"], a["nxt"], a["kvo"], a["cp"], a["ps"], a["npg"],
                                         a["ws"], a["wsb"], None)


@no_device
def test_verify_rejects_bad_arguments():
    assert _verify(B=0) == -2
    assert _verify(B=8193) == -2
    assert _verify(blk=8) == -2
    assert _verify(V=0) == -2
    assert _verify(ld=999) == -2
    assert _verify(ld=1004) == -3             # row stride not a multiple of 8
    assert _verify(logits=MIS) == -3
    assert _verify(post=ctypes.c_void_p(None)) == -1
    assert _verify(npg=FAKE, ps=0) == -2      # page count needs a page size
    assert _verify(ws=ctypes.c_void_p(None)) == -4
    assert _verify(wsb=100) == -4
    assert _verify(ws=MIS) == -3


def _draft(**kw):
    a = dict(B=2, blk=16, V=1000, logits=FAKE, ld=1000, staged=None, bt=FAKE, ws=FAKE, wsb=1 << 22)
    a.update(kw)
    return dfl._lib.dflash_draft_argmax(a["B"], a["blk"], a["V"], a["logits"], a["ld"], a["staged"], a["bt"],
                                        a["ws"], a["wsb"], None)


@no_device
def test_draft_argmax_rejects_bad_arguments():
    assert _draft(B=0) == -2
    assert _draft(B=8193) == -2               # more sequences than counter slots
    assert _draft(blk=15) == -2
    assert _draft(V=0) == -2
    assert _draft(V=0x7fffffff, ld=0x7fffffff + 1) == -2
    assert _draft(ld=999) == -2
    assert _draft(ld=1004) == -3              # row stride not a multiple of 8
    assert _draft(logits=MIS) == -3
    assert _draft(logits=ctypes.c_void_p(None)) == -1
    assert _draft(bt=ctypes.c_void_p(None)) == -1
    assert _draft(ws=ctypes.c_void_p(None)) == -4
    assert _draft(wsb=100) == -4               # the verify's workspace size is required
    assert _draft(ws=MIS) == -3


def _proj(dims, n_layers=2, **kw):
    xs = (ctypes.c_void_p * 8)(*([0x100000] * 8))
    a = dict(n=32, xs=xs, nl=n_layers, dt=256, ld=256, seq=FAKE, pos=FAKE, wfc=FAKE, wk=FAKE, wv=FAKE,
             cos=FAKE, sin=FAKE, maxpos=128, cout=None, kc=FAKE, vc=FAKE, pt=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return dfl._lib.dflash_ctx_proj(ctypes.byref(dims), a["n"], a["xs"], a["nl"], a["dt"], a["ld"], a["seq"],
                                    a["pos"], a["wfc"], a["wk"], a["wv"], a["cos"], a["sin"], a["maxpos"],
                                    a["cout"], a["kc"], a["vc"], a["pt"], a["ws"], a["wsb"], None)


@no_device
def test_ctx_proj_rejects_bad_arguments():
    dims = dfl.make_dims(1, 4, 2, 64, hidden=256, kv_capacity=80)
    assert _proj(dims, dt=100) == -2                    # d_target not a multiple of 64
    assert _proj(dims, nl=9) == -2
    assert _proj(dims, nl=0) == -2
    assert _proj(dims, ld=128) == -2                    # ld < d_target
    assert _proj(dims, ld=260) == -3                    # ld % 8
    assert _proj(dims, n=-1) == -2
    assert _proj(dims, wk=ctypes.c_void_p(None)) == -1
    assert _proj(dims, wfc=ctypes.c_void_p(None)) == -2  # no fc needs 1 layer of width hidden
    assert _proj(dims, wk=MIS) == -3
    assert _proj(dims, ws=ctypes.c_void_p(None)) == -4
    assert _proj(dims, wsb=64) == -4
    assert _proj(dims, maxpos=0) == -5
    xs = (ctypes.c_void_p * 8)(*([0x100000] + [0] * 7))
    assert _proj(dims, xs=xs) == -1                     # second layer pointer NULL
    h = dfl.make_dims(1, 4, 2, 64, hidden=200, kv_capacity=80)
    assert _proj(h) == -2                               # hidden % 64
    paged = dfl.make_dims(1, 4, 2, 64, hidden=256, page_size=16, kv_capacity=5, num_pages=4)
    assert _proj(paged) == -1                           # page table missing


def _qkv(dims, **kw):
    a = dict(h=FAKE, ld=256, w=FAKE, q=FAKE, k=FAKE, v=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return dfl._lib.dflash_block_qkv(ctypes.byref(dims), a["h"], a["ld"], a["w"], a["q"], a["k"], a["v"],
                                     a["ws"], a["wsb"], None)


@no_device
def test_block_qkv_rejects_bad_arguments():
    good = dfl.make_dims(2, 8, 2, 64, hidden=256, kv_capacity=80)
    assert dfl.dflash_block_qkv_workspace_size(good) > 256
    assert dfl.dflash_block_qkv_workspace_size(dfl.make_dims(2, 8, 2, 64, hidden=200, kv_capacity=80)) == 0
    assert _qkv(dfl.make_dims(2, 8, 2, 64, hidden=200, kv_capacity=80), ld=200) == -2    # hidden % 64
    assert _qkv(dfl.make_dims(2, 8, 3, 64, hidden=256, kv_capacity=80)) == -2            # Hq % Hkv
    assert _qkv(dfl.make_dims(2, 8, 2, 96, hidden=256, kv_capacity=80)) == -6            # head_dim
    assert _qkv(good, ld=128) == -2
    assert _qkv(good, ld=260) == -3
    assert _qkv(good, h=ctypes.c_void_p(None)) == -1
    assert _qkv(good, v=ctypes.c_void_p(None)) == -1
    assert _qkv(good, w=MIS) == -3
    assert _qkv(good, ws=ctypes.c_void_p(None)) == -4
    assert _qkv(good, wsb=300) == -4


# ---------------------------------------------------------------- binding size checks
# The Python wrappers check every tensor's size against the dims before any pointer
# is handed over (the kernels trust those sizes).  Host tensors of the right sizes get
# past the size checks and stop at the device check; wrong sizes stop earlier.
def _t(*shape, dtype=torch.int16):
    return torch.zeros(shape, dtype=dtype)


def _attn_args(B=2, Hq=8, Hkv=2, d=64, cap=80, **kw):
    dims = dfl.make_dims(B, Hq, Hkv, d, kv_capacity=cap)
    a = dict(q=_t(B, 16, Hq, d), k=_t(B, 16, Hkv, d), v=_t(B, 16, Hkv, d), kc=_t(B, Hkv, cap, d),
             vc=_t(B, Hkv, cap, d), pt=None, ctx=_t(B, dtype=torch.int32), cos=_t(100, d // 2, dtype=torch.float32),
             sin=_t(100, d // 2, dtype=torch.float32), out=_t(B, 16, Hq, d, dtype=torch.float32),
             ws=_t(1024, dtype=torch.uint8))
    a.update(kw)
    return dims, a


def _call_attn(dims, a):
    dfl.dflash_block_attn(dims, a["q"], a["k"], a["v"], a["kc"], a["vc"], a["pt"], a["ctx"], 64, a["cos"],
                          a["sin"], a["out"], a["ws"])


@pytest.mark.parametrize("name,bad", [
    ("q", _t(2, 16, 8, 32)), ("k", _t(2, 16, 1, 64)), ("v", _t(1, 16, 2, 64)), ("kc", _t(2, 2, 79, 64)),
    ("vc", _t(2, 2, 81, 64)), ("ctx", _t(1, dtype=torch.int32)), ("out", _t(2, 16, 8, 63, dtype=torch.float32)),
    ("cos", _t(100, 64, dtype=torch.float32)), ("sin", _t(99, 32, dtype=torch.float32)),
])
def test_binding_block_attn_checks_sizes(name, bad):
    dims, a = _attn_args(**{name: bad})
    with pytest.raises(ValueError, match="elements|rope_cos"):
        _call_attn(dims, a)
    dims, a = _attn_args()
    with pytest.raises(ValueError, match="device tensor"):
        _call_attn(dims, a)


def test_binding_block_attn_checks_page_table_size():
    dims = dfl.make_dims(2, 8, 2, 64, page_size=16, kv_capacity=5, num_pages=10)
    _, a = _attn_args(kc=_t(10, 2, 16, 64), vc=_t(10, 2, 16, 64), pt=_t(2, 4, dtype=torch.int32))
    with pytest.raises(ValueError, match="page_table"):
        _call_attn(dims, a)


def _proj_args(n=32, nl=2, dt=256, D=256, Hkv=2, d=64, cap=80, **kw):
    dims = dfl.make_dims(1, 4, Hkv, d, hidden=D, kv_capacity=cap)
    a = dict(xs=[_t(n, dt) for _ in range(nl)], seq=_t(n, dtype=torch.int32), pos=_t(n, dtype=torch.int32),
             wfc=_t(D, nl * dt), wk=_t(Hkv * d, D), wv=_t(Hkv * d, D), cos=_t(100, d // 2, dtype=torch.float32),
             sin=_t(100, d // 2, dtype=torch.float32), cout=None, kc=_t(1, Hkv, cap, d), vc=_t(1, Hkv, cap, d),
             pt=None, ws=_t(1024, dtype=torch.uint8))
    a.update(kw)
    return dims, a


def _call_proj(dims, a):
    dfl.dflash_ctx_proj(dims, a["xs"], a["seq"], a["pos"], a["wfc"], a["wk"], a["wv"], a["cos"], a["sin"],
                        a["cout"], a["kc"], a["vc"], a["pt"], a["ws"])


@pytest.mark.parametrize("name,bad", [
    ("seq", _t(31, dtype=torch.int32)), ("pos", _t(33, dtype=torch.int32)), ("wfc", _t(256, 256)),
    ("wk", _t(64, 256)), ("wv", _t(128, 255)), ("cout", _t(31, 256)), ("kc", _t(1, 2, 79, 64)),
    ("vc", _t(2, 2, 80, 64)), ("cos", _t(100, 16, dtype=torch.float32)),
])
def test_binding_ctx_proj_checks_sizes(name, bad):
    dims, a = _proj_args(**{name: bad})
    with pytest.raises(ValueError, match="elements|rope_cos"):
        _call_proj(dims, a)
    dims, a = _proj_args()
    with pytest.raises(ValueError, match="device tensor"):
        _call_proj(dims, a)


def _verify_args(B=3, **kw):
    i = lambda *s: _t(*s, dtype=torch.int32)
    a = dict(logits=_t(B, 16, 1000), bt=i(B, 16), kvi=i(B), post=i(B, 16), acc=i(B), nxt=i(B), kvo=i(B),
             cp=i(B, 16), npg=i(B))
    a.update(kw)
    return a


def _call_verify(a):
    dfl.dflash_verify_accept(a["logits"], a["bt"], a["kvi"], a["post"], a["acc"], a["nxt"], a["kvo"], a["cp"], 16,
                             a["npg"], _t(1024, dtype=torch.uint8))


@pytest.mark.parametrize("name", ["bt", "kvi", "post", "acc", "nxt", "kvo", "cp", "npg"])
def test_binding_verify_checks_sizes(name):
    a = _verify_args()
    a[name] = torch.zeros(a[name].numel() - 1, dtype=torch.int32)
    with pytest.raises(ValueError, match=name.replace("bt", "block_tokens").replace("kvi", "kv_len_in")
                       .replace("post", "posterior").replace("acc", "accept_len").replace("nxt", "next_token")
                       .replace("kvo", "kv_len_out").replace("cp", "commit_pos").replace("npg", "n_pages")):
        _call_verify(a)
    with pytest.raises(ValueError, match="device tensor"):
        _call_verify(_verify_args())


def test_deverr_bits_match_the_header():
    text = open(HEADER).read()
    bits = dict(re.findall(r"#define DFLASH_DEVERR_(\w+)\s+(\d+)u", text))
    assert {k: int(v) for k, v in bits.items()} == {
        "CTX_LEN": dfl.DEVERR_CTX_LEN, "PAGE_ID": dfl.DEVERR_PAGE_ID, "ROW": dfl.DEVERR_ROW,
        "MERGE": dfl.DEVERR_MERGE, "XCD": dfl.DEVERR_XCD, "ACCEPT": dfl.DEVERR_ACCEPT}


@no_device
def test_block_attn_noalloc_refuses_sizes_beyond_its_scratch():
    # A ragged batch of 32 x 16384 tokens needs more split partials than the scratch holds.
    dims = dfl.make_dims(32, 32, 8, 128, page_size=16, kv_capacity=1100, num_pages=40000)
    assert dfl.dflash_block_attn_workspace_size(dims, 16384) > dfl.NOALLOC_SCRATCH_BYTES
    rc = dfl._lib.dflash_block_attn_noalloc(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16384,
                                            FAKE, FAKE, 16400, FAKE, None, None)
    assert rc == -4
    assert dfl._lib.dflash_block_attn_noalloc(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                              16384, FAKE, FAKE, 16400, FAKE, ctypes.c_void_p(0x100002), None) == -3
    text = open(HEADER).read()
    assert "#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in text
    assert dfl.NOALLOC_SCRATCH_BYTES == 32 << 20


@no_device
def test_window_validation():
    d = dfl.make_dims(2, 8, 2, 64, kv_capacity=80, window=81)
    assert _attn(d) == -5                                   # dense ring wider than the capacity
    assert _attn(dfl.make_dims(2, 8, 2, 64, kv_capacity=80, window=-1)) == -2
    p = dfl.make_dims(2, 8, 2, 64, page_size=16, kv_capacity=5, num_pages=10, window=72)
    assert _attn(p, pt=FAKE) == -5                          # paged ring not whole pages
    p = dfl.make_dims(2, 8, 2, 64, page_size=16, kv_capacity=5, num_pages=10, window=96)
    assert _attn(p, pt=FAKE) == -5                          # 6 pages > 5 table columns
    # with a window the context may exceed the capacity (the ring keeps the last W rows)
    w = dfl.make_dims(2, 8, 2, 64, kv_capacity=80, window=64)
    assert dfl.dflash_block_attn_workspace_size(w, 100000) == dfl.dflash_block_attn_workspace_size(w, 64)
    assert _attn(w, maxc=100000, maxpos=100016, wsb=16) == -4   # past the capacity check, stops at the workspace
    assert _proj(dfl.make_dims(1, 4, 2, 64, hidden=256, kv_capacity=80, window=100)) == -5


@no_device
def test_gdn_tape_replay_rejects_bad_arguments():
    def call(B=2, H=4, dk=128, dv=128, si=FAKE, so=ctypes.c_void_p(0x200000), k=FAKE, g=FAKE, d=FAKE, a=FAKE,
             err=None):
        return dfl._lib.dflash_gdn_tape_replay(B, H, dk, dv, si, so, k, g, d, a, err, None)
    assert call(si=ctypes.c_void_p(None)) == -1
    assert call(a=ctypes.c_void_p(None)) == -1
    assert call(B=0) == -2
    assert call(dk=130) == -2                     # d_k % 4
    assert call(dk=260) == -2
    assert call(dv=0) == -2
    assert call(k=MIS) == -3
    assert call(err=ctypes.c_void_p(0x100002)) == -3
    assert call(so=ctypes.c_void_p(0x100000 + 4096)) == -2   # partial overlap with state_in
    assert call(B=1 << 16, H=256, dv=33) == -2    # 2^24 units x 2 workgroups: grid too large


def test_binding_prepared_attention_call_checks_sizes_once():
    dims, a = _attn_args(q=_t(2, 16, 8, 32))
    with pytest.raises(ValueError, match="q_blk"):
        dfl.bind_block_attn(dims, a["q"], a["k"], a["v"], a["kc"], a["vc"], a["pt"], a["ctx"], 64, a["cos"],
                            a["sin"], a["out"], a["ws"])
    dims, a = _attn_args()
    with pytest.raises(ValueError, match="device tensor"):
        dfl.bind_block_attn(dims, a["q"], a["k"], a["v"], a["kc"], a["vc"], a["pt"], a["ctx"], 64, a["cos"],
                            a["sin"], a["out"], a["ws"])
