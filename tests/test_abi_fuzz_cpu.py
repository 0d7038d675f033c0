"""Randomised argument checks of every C entry point, host only.

Each call gets dims fields, sizes and strides drawn from edge values (0, 1, -1,
powers of two around the limits, INT32_MIN / INT32_MAX), null, misaligned or fake
aligned pointers and extreme float scales.  Every call must return one of the
header's status codes and every size query 0 or a size below 2^48 bytes, without
touching memory it was not given.  Run under the host-sanitizer build
(tests/test_host_sanitized.py), an out-of-bounds host access or a signed overflow
in the size arithmetic ends the run.

The pointers are fake device addresses, so these calls must never reach a launch:
they run only where no GPU is visible, where the device check fails first.
"""
import ctypes

import numpy as np
import pytest
import torch

from block_diffusion_draft_proj_amd import dflash as dfl

no_device = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only validation tests")

STATUS = set(range(-7, 1))
INT_EDGES = [0, 1, 2, 3, -1, 15, 16, 17, 63, 64, 128, 255, 256, 512, 4096, 8192, 8193, 65536, 1 << 20, 1 << 24,
             (1 << 24) + 1, (1 << 30), 2**31 - 1, -2**31]
I64_EDGES = [0, 1, 8, 9, 64, 4096, 1 << 31, 2**62, -8, -(2**62)]
SZ_EDGES = [0, 1, 255, 1 << 20, 1 << 30, 1 << 40, 2**63, 2**64 - 1]
F_EDGES = [0.0, -1.0, 1e-3, 0.088, 1.0, 1e6, float("inf"), float("nan")]
PTRS = [None, ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100002), ctypes.c_void_p(0x7FFF00000000)]
DIM_FIELDS = [f for f, _ in dfl.dflash_dims._fields_]


def _dims(rng):
    d = dfl.dflash_dims()
    for f in DIM_FIELDS:
        if f == "softmax_scale":
            setattr(d, f, float(rng.choice(F_EDGES)))
        elif rng.random() < 0.5:  # a plausible value, so later checks are reached too
            setattr(d, f, {"batch": 8, "block": 16, "n_q_heads": 32, "n_kv_heads": 8, "head_dim": 128,
                           "hidden": 4096, "page_size": 16, "kv_capacity": 8208, "num_pages": 4096,
                           "window": 0}[f])
        else:
            setattr(d, f, int(rng.choice(INT_EDGES)))
    return d


def _arg(rng, t, keep):
    if t is dfl._c_int:
        return int(rng.choice(INT_EDGES))
    if t is dfl._c_i64:
        return int(rng.choice(I64_EDGES))
    if t is dfl._c_sz:
        return int(rng.choice(SZ_EDGES))
    if t is dfl._c_f:
        return float(rng.choice(F_EDGES))
    if t is dfl._vp:
        return PTRS[rng.integers(len(PTRS))]
    if t is ctypes.POINTER(dfl.dflash_dims):
        d = _dims(rng)
        keep.append(d)
        return ctypes.byref(d)
    if t is ctypes.POINTER(dfl._vp):
        # a host array of 8 layer pointers: the library reads at most 8 (its layer limit)
        arr = (dfl._vp * 8)(*[0x100000 + 4096 * i for i in range(8)])
        keep.append(arr)
        return arr
    raise TypeError(t)


def _entry_points():
    out = []
    for name in dfl.EXPORTS:
        if name in ("dflash_status_str", "dflash_version"):
            continue
        f = getattr(dfl._lib, name)
        out.append((name, f))
    return out


@no_device
@pytest.mark.parametrize("name,f", _entry_points(), ids=[n for n, _ in _entry_points()])
def test_random_arguments_return_a_status(name, f):
    rng = np.random.default_rng(abs(hash(name)) % (2**32))
    for _ in range(1500):
        keep = []
        args = [_arg(rng, t, keep) for t in f.argtypes]
        r = f(*args)
        if name.endswith("_workspace_size"):
            assert r == 0 or (r % 8 == 0 and r < 2**48), (name, r)
        else:
            assert r in STATUS, (name, r)
