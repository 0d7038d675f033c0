"""The oracle's pins must reject plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle source -- a dropped term,
a wrong sign, an off-by-one position or alignment, a transposed head, a missing
rounding -- and runs the pin suite against that copy in a fresh interpreter.
The pins pass on the real oracle (tests/test_oracle_pins.py); here every mutant
must make at least one of them fail.  The real oracle file is never modified.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "dflash_oracle.py")

MUTANTS = {
    "rope_sign": ("return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)",
                  "return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)"),
    "rope_freq": ("inv_freq = base ** (-2.0 * j / head_dim)", "inv_freq = base ** (-1.0 * j / head_dim)"),
    "q_not_rounded": ("Q = rope_bf16(q_b[:, hs, :], pos, base)",
                      "Q = apply_rope(bf16_to_f64(q_b[:, hs, :]), pos, base)"),
    "rope_f64_tables": ("return (np.cos(th).astype(np.float32).astype(np.float64),\n"
                        "            np.sin(th).astype(np.float32).astype(np.float64))",
                        "return (np.cos(th), np.sin(th))"),
    "rope_no_two_sum": ("r[tie] = s[tie] + np.sign(e[tie]) * half[tie]", "r[tie] = r[tie]"),
    "rope_sum_sign": ("round_bf16_sum(lo * c, -(hi * s))", "round_bf16_sum(lo * c, hi * s)"),
    "window_first": ("first = max(0, L - window) if window > 0 else 0\n        t = np.arange(first, L)  ",
                     "first = max(0, L - window + 1) if window > 0 else 0\n        t = np.arange(first, L)  "),
    "window_ring_rows": ("rows = t % window if window > 0 else t                # their storage rows",
                         "rows = t                # their storage rows"),
    "window_block_pos": ("L - first, g, G, base, scale, block_pos=L)", "L - first, g, G, base, scale)"),
    "rms_no_square": ("r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                      "r = 1.0 / np.sqrt(np.mean(np.abs(x), axis=-1, keepdims=True) + eps)"),
    "rms_no_eps": ("r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                   "r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))"),
    "silu_sign": ("return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))"),
    "layer_no_residual": ("x1 = round_bf16(bf16_to_f64(x_bits) + a @ bf16_to_f64(w_o).T)",
                          "x1 = round_bf16(a @ bf16_to_f64(w_o).T)"),
    "layer_gate_up_swapped": ("act = round_bf16(silu(g) * u)", "act = round_bf16(silu(u) * g)"),
    "layer_act_not_rounded": ("act = round_bf16(silu(g) * u)", "act = silu(g) * u"),
    "layer_w_o_transposed": ("x1 = round_bf16(bf16_to_f64(x_bits) + a @ bf16_to_f64(w_o).T)",
                             "x1 = round_bf16(bf16_to_f64(x_bits) + a @ bf16_to_f64(w_o))"),
    "replay_off_by_one": ("for t in range(int(accept[b]) + 1):", "for t in range(int(accept[b])):"),
    "replay_no_decay": ("out[b] = alpha[:, None, None] * out[b] + d[:, :, None] * k[b, t][:, None, :]",
                        "out[b] = out[b] + d[:, :, None] * k[b, t][:, None, :]"),
    "replay_outer_transposed": ("out[b] = alpha[:, None, None] * out[b] + d[:, :, None] * k[b, t][:, None, :]",
                                "out[b] = alpha[:, None, None] * out[b] + (d[:, :, None] * k[b, t][:, None, :])"
                                "[:, ::-1, ::-1]"),
    "gdn_innovation_no_alpha": ("d = float(beta[t]) * (v[t] - alpha * (S @ k[t]))",
                                "d = float(beta[t]) * (v[t] - (S @ k[t]))"),
    "fused_q_rounded": ("out[b, :, hd, :] = attend_ref(rot(q[b, :, hd]), Keys, Vals, scale)",
                        "out[b, :, hd, :] = attend_ref(round_bf16(rot(q[b, :, hd])), Keys, Vals, scale)"),
    "fused_k_not_rotated": ("round_bf16(rot(k[b, :, g]))], axis=0)", "round_bf16(k[b, :, g])], axis=0)"),
    "fused_v_slice": ("v = Y[:, (Hq + Hkv) * d:].reshape(B, BLOCK, Hkv, d)",
                      "v = Y[:, Hq * d:(Hq + Hkv) * d].reshape(B, BLOCK, Hkv, d)"),
    "drop_block_keys": ("Keys = np.concatenate([bf16_to_f64(k_ctx[:L]), Kblk], axis=0)\n"
                        "    Vals = np.concatenate([bf16_to_f64(v_ctx[:L]), bf16_to_f64(v_b[:, g, :])], axis=0)",
                        "Keys = bf16_to_f64(k_ctx[:L+16])\n    Vals = bf16_to_f64(v_ctx[:L+16])"),
    "softmax_scale": ("scale = 1.0 / math.sqrt(d)\n    L = int(ctx_len)\n    pos",
                      "scale = 1.0 / d\n    L = int(ctx_len)\n    pos"),
    "accept_alignment": ("matches = (blk[:, 1:] == post[:, :BLOCK - 1])",
                         "matches = (blk[:, :BLOCK - 1] == post[:, :BLOCK - 1])"),
    "commit_count": ("kv_out = (kv_in + 1 + accept)", "kv_out = (kv_in + accept)"),
    "block_positions": ("pos = (L if block_pos is None else int(block_pos)) + np.arange(BLOCK)",
                        "pos = (L if block_pos is None else int(block_pos)) + 1 + np.arange(BLOCK)"),
    "wrong_kv_head": ("kc = gather_rows(k_cache, page_table, b, rows)[g]\n        vc = gather_rows(v_cache, page_table, b, rows)[g]",
                      "kc = gather_rows(k_cache, page_table, b, rows)[(g + 1) % Hkv]\n        vc = gather_rows(v_cache, page_table, b, rows)[(g + 1) % Hkv]"),
    "c_not_rounded": ("Cb = round_bf16(C)", "Cb = C"),
    "commit_positions": ("np.where(i <= accept[:, None]", "np.where(i < accept[:, None]"),
    "draft_alignment": ("blk[b, 1:] = argmax_first(bf16_to_f64(draft_logits[b, 1:]))",
                        "blk[b, 1:] = argmax_first(bf16_to_f64(draft_logits[b, :BLOCK - 1]))"),
    "draft_staged_slot": ("blk[:, 0] = np.asarray(staged, dtype=np.int32)",
                          "blk[:, 0] = argmax_first(bf16_to_f64(draft_logits[:, 0]))"),
    "qkv_k_v_swapped": ("k = Y[:, nq:nq + nk].reshape(M, n_kv_heads, head_dim)\n    v = Y[:, nq + nk:]",
                        "k = Y[:, nq + nk:].reshape(M, n_kv_heads, head_dim)\n    v = Y[:, nq:nq + nk]"),
    "qkv_not_rounded": ("Y = f64_to_bf16_bits(bf16_to_f64(h) @ bf16_to_f64(w_qkv).T)",
                        "Y = (bf16_to_f64(h) @ bf16_to_f64(w_qkv).T).astype(np.float32).view(np.uint32) >> 16"),
    "rope_on_v": ("V = (Cb @ bf16_to_f64(w_v).T).reshape(M, n_kv_heads, head_dim)",
                  "V = apply_rope((Cb @ bf16_to_f64(w_v).T).reshape(M, n_kv_heads, head_dim), "
                  "np.maximum(np.asarray(row_pos), 0), base)"),
}


def _run_pins(mutant_path):
    env = dict(os.environ, DFLASH_ORACLE_MUTANT=mutant_path)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, (r.stdout.strip().splitlines() or [""])[-1]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(ORACLE).read()
    paths = {}
    for name, (good, bad) in MUTANTS.items():
        assert src.count(good) == 1, f"mutation site of {name} not found once in the oracle"
        p = tmp_path / f"mutant_{name}.py"
        p.write_text(src.replace(good, bad))
        paths[name] = str(p)
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = dict(zip(paths, ex.map(_run_pins, paths.values())))
    survivors = {n: last for n, (rc, last) in results.items() if rc == 0}
    assert not survivors, f"mutants that pass every pin: {survivors}"
    # a collection or import error is not a pin failure
    for n, (rc, last) in results.items():
        assert rc == 1, f"{n}: pytest exit {rc} ({last})"
