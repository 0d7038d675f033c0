"""GPU parity of dflash_verify_accept against the oracle: bit-exact posterior,
accept length, next staged token, committed KV length, commit positions and
page counts, on every workload configuration at full size and on crafted rows
(ties across workgroup chunks, NaN of both signs, signed zeros, infinities,
vocabularies that are not a multiple of the vector width)."""
import numpy as np
import pytest

from block_diffusion_draft_proj_amd import synth
from oracle import dflash_oracle as orc
from block_diffusion_draft_proj_amd import dflash as dfl
from tests.gpu_util import DEV, log, run_draft, run_verify

pytestmark = pytest.mark.gpu

KEYS = ["post", "accept", "next", "kv_len", "commit_pos"]


def _compare(got, ref, page_size=0):
    for k in KEYS + (["n_pages"] if page_size > 0 else []):
        assert np.array_equal(got[k], ref[k]), (k, got[k], ref[k])


def _bits(x):
    a = np.asarray(x, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_verify_planted_full_size(name):
    cfg = synth.CONFIGS[name]
    vi = synth.verify_inputs(cfg)
    log(f"verify planted {name}: B={cfg.batch} V={cfg.vocab}")
    ps = 16
    got, _ = run_verify(vi.logits, vi.block_tokens, vi.kv_len, page_size=ps)
    ref = orc.verify_accept_ref(vi.logits, vi.block_tokens, vi.kv_len, page_size=ps)
    _compare(got, ref, ps)
    assert np.array_equal(got["accept"], vi.planted_accept)


@pytest.mark.parametrize("name", ["tiny", "batched"])
def test_verify_unplanted_normal_rows_with_ties(name):
    cfg = synth.CONFIGS[name]
    vi = synth.verify_inputs(cfg, spike=False, seed=cfg.seed + 5)
    ref = orc.verify_accept_ref(vi.logits, vi.block_tokens, vi.kv_len)
    # make drafts agree with the oracle posterior on a prefix so accept lengths vary
    blk = vi.block_tokens.copy()
    for b in range(len(blk)):
        a = b % 16
        blk[b, 1:a + 1] = ref["post"][b, :a]
    ref = orc.verify_accept_ref(vi.logits, blk, vi.kv_len)
    vals = orc.bf16_to_f64(vi.logits)
    ties = int(np.sum([(row == row.max()).sum() > 1 for row in vals.reshape(-1, vals.shape[-1])]))
    log(f"verify N(0,1) {name}: {ties} of {vals.shape[0] * 16} rows have a tied maximum")
    got, _ = run_verify(vi.logits, blk, vi.kv_len)
    _compare(got, ref)


# Batches of 8 or more run the one-kernel form (the accept step inside the argmax
# kernel, sequences grouped per XCD); smaller ones the two-kernel form.
@pytest.mark.parametrize("n_seq", [2, 10])
def test_verify_crafted_rows(n_seq):
    V = 20000  # 3 chunks of 8192 (last partial)
    rows = np.zeros((2, 16, V), np.float32)
    rng = np.random.default_rng(3)
    base = rng.standard_normal((2, 16, V)).astype(np.float32) * 0.5
    rows[:] = base
    nan, inf = np.float32("nan"), np.float32("inf")
    r = rows[0]
    r[0, [8191, 8192, 16384]] = 9.0                # tie straddling the first chunk boundary
    r[1, [19999]] = 9.0                             # max at the last element
    r[1, [5]] = 9.0                                 # ... and an earlier tie -> 5
    r[2, :] = -3.0                                  # all equal
    r[3, :] = -inf
    r[3, 12345] = -1e30                             # single finite value among -inf
    r[4, 100] = nan                                 # NaN anywhere wins
    r[4, 50] = 50.0
    r[5, :] = -1.0
    r[5, 7] = -0.0
    r[5, 9000] = 0.0                                # -0 first, +0 later -> 7
    r[6, :] = -1.0
    r[6, 17000] = 0.0
    r[6, 17001] = -0.0                              # +0 first -> 17000
    r[7, 3] = inf
    r[7, 4] = inf                                   # -> 3
    r[8, 8200] = inf
    r[8, 10] = nan                                  # NaN beats +inf -> 10
    r[9, :] = -2.0
    r[9, 12000] = -0.0                              # zero is the max, only -0 present
    logits = _bits(rows)
    # negative NaN (sign bit set) in row 10, positive NaN later in row 11
    logits[0, 10, 4000] = 0xFFC1
    logits[0, 11, 9000] = 0x7FC0
    logits[0, 11, 8999] = 0xFF81
    logits[0, 12, 16383] = 0x7F80                   # +inf at the very end of chunk 0..1 boundary
    logits[0, 12, 16384] = 0x7F80
    logits = np.tile(logits, (n_seq // 2, 1, 1))
    blk = rng.integers(0, V, (n_seq, 16)).astype(np.int32)
    kv = (5 + 4 * np.arange(n_seq)).astype(np.int32)
    ref = orc.verify_accept_ref(logits, blk, kv)
    blk[1, 1:6] = ref["post"][1, :5]                # a non-trivial accept length
    ref = orc.verify_accept_ref(logits, blk, kv)
    assert ref["post"][0, 0] == 8191 and ref["post"][0, 1] == 5 and ref["post"][0, 2] == 0
    assert ref["post"][0, 4] == 100 and ref["post"][0, 5] == 7 and ref["post"][0, 6] == 17000
    assert ref["post"][0, 10] == 4000 and ref["post"][0, 11] == 8999 and ref["post"][0, 12] == 16383
    got, _ = run_verify(logits, blk, kv)
    _compare(got, ref)


@pytest.mark.parametrize("B", [3, 9])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 8, 9, 1001, 8191, 8192, 8193, 16385])
def test_verify_small_and_ragged_vocab(V, B):
    ld = (V + 7) // 8 * 8
    rng = np.random.default_rng(V)
    vals = rng.standard_normal((B, 16, ld)).astype(np.float32)
    logits = _bits(vals)
    logits[:, :, V:] = 0x7F80                       # +inf padding past vocab must be ignored
    blk = rng.integers(0, V, (B, 16)).astype(np.int32)
    kv = (np.arange(B) * 37 % 101).astype(np.int32)
    post = orc.verify_accept_ref(logits[:, :, :V].copy(), blk, kv)["post"]
    blk[1, 1:8] = post[1, :7]
    blk[2, 1:16] = post[2, :15]
    ref = orc.verify_accept_ref(logits[:, :, :V].copy(), blk, kv, page_size=16)
    got, _ = run_verify(logits, blk, kv, page_size=16, vocab=V)
    _compare(got, ref, 16)


@pytest.mark.parametrize("B", [4, 12])
def test_verify_workspace_reuse_and_aliasing(B):
    # B = 12 also checks that the one-kernel form leaves its arrival counters at zero.
    cfg = synth.CONFIGS["qwen3_8b"]
    vi1 = synth.verify_inputs(cfg, batch=B, seed=7)
    vi2 = synth.verify_inputs(cfg, batch=B, seed=8)
    r1, ws = run_verify(vi1.logits, vi1.block_tokens, vi1.kv_len)
    r2, ws = run_verify(vi2.logits, vi2.block_tokens, vi2.kv_len, ws=ws)
    r3, ws = run_verify(vi1.logits, vi1.block_tokens, vi1.kv_len, ws=ws, alias_kv=True)
    _compare(r1, orc.verify_accept_ref(vi1.logits, vi1.block_tokens, vi1.kv_len))
    _compare(r2, orc.verify_accept_ref(vi2.logits, vi2.block_tokens, vi2.kv_len))
    for k in KEYS:
        assert np.array_equal(r1[k], r3[k]), k
    assert ws[:4].cpu().numpy().view(np.uint32)[0] == 0


def test_verify_workspace_serves_shrinking_and_growing_batches():
    # One buffer sized for 12 sequences serves 12, 9, 3, 12 and 8 of them (both launch
    # forms) with the draft argmax interleaved on it: the per-sequence arrival counters
    # sit in a fixed region ahead of the chunk keys, so no call's keys land on another
    # call's counters.
    cfg = synth.CONFIGS["qwen3_8b"]
    ws = dfl.workspace(dfl.dflash_verify_workspace_size(12, 16, cfg.vocab), DEV)
    for i, B in enumerate([12, 9, 3, 12, 8]):
        vi = synth.verify_inputs(cfg, batch=B, seed=50 + i)
        log(f"verify workspace reuse, call {i}: B={B}")
        got, ws = run_verify(vi.logits, vi.block_tokens, vi.kv_len, ws=ws)
        _compare(got, orc.verify_accept_ref(vi.logits, vi.block_tokens, vi.kv_len))
        d, ws = run_draft(vi.logits, vi.block_tokens[:, 0], ws=ws)
        assert np.array_equal(d, orc.draft_block_ref(vi.logits, vi.block_tokens[:, 0]))
    assert ws[:4].cpu().numpy().view(np.uint32)[0] == 0
    assert not ws[256:256 + 128 * 12].any()          # every counter back at zero
