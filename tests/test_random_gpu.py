"""Seeded random-shape GPU parity sweep, through the C ABI, against the float64
CPU oracle.

Each case draws a head size, dtype, batch and head counts, query and key
lengths (equal or not, ragged or whole tiles), a causal mask (none, the default
diagonal, or an explicit offset), BHSD or BSHD storage, a tile variant, a
scale and a grid size (the library's, or a few workgroups that each run many
items in turn), and compares every output element.  Same bar as the other parity tests:
max |dO| <= 2e-2, mean |dO| <= 2e-3 against the unrounded oracle, max |dLSE|
<= 1e-3 (rows that see no key must give O = 0 and LSE = -inf on both sides).
"""

import math
import os
import sys

import numpy as np
import pytest
import torch

import dense_attention_amd as da
import workloads as W
from oracle import attention_forward

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
# More cases or another draw on request: ATTN_RANDOM_CASES, ATTN_RANDOM_SEED.
N_CASES = int(os.environ.get("ATTN_RANDOM_CASES", "60"))
SEED = int(os.environ.get("ATTN_RANDOM_SEED", "20261202"))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.load_library()
    yield
    torch.cuda.synchronize()


def _variants(D, dtype):
    code = da.ATTN_F16 if dtype == "fp16" else da.ATTN_BF16
    return [v["id"] for v in da.attn_variants() if v["head_dim"] == D and v["dtype"] == code]


def _draw(rng):
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Sq = int(rng.choice([rng.integers(1, 700), 64 * rng.integers(1, 11), 128 * rng.integers(1, 6)]))
    Skv = Sq if rng.random() < 0.5 else int(rng.integers(1, 700))
    mode = int(rng.integers(0, 3))
    causal = False if mode == 0 else (True if mode == 1 else int(rng.integers(-50, 51)))
    layout = str(rng.choice(["bhsd", "bshd"]))
    variant = int(rng.choice([0] + _variants(D, dtype)))
    # Up to twice the usual scale either way: sharper rows make O a single V row,
    # where bf16 rounding alone of |O| >= 4 approaches the bar.
    scale = 1.0 / math.sqrt(D) if rng.random() < 0.7 else float(rng.uniform(-2.0, 2.0)) / math.sqrt(D)
    return D, dtype, B, H, Sq, Skv, causal, layout, variant, scale


def _device_view(t, layout):
    if layout == "bshd":
        return t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    return t.cuda()


def test_random_shapes_sweep():
    rng = np.random.default_rng(SEED)
    grid_rng = np.random.default_rng(77)  # its own stream: the shapes stay as they were
    for n in range(N_CASES):
        D, dtype, B, H, Sq, Skv, causal, layout, variant, scale = _draw(rng)
        grid = int(grid_rng.choice([0, 0, 1, 2, 5]))
        tag = (f"case {n}: B={B} H={H} Sq={Sq} Skv={Skv} D={D} {dtype} causal={causal} "
               f"{layout} variant={variant} scale={scale:.4f} grid={grid}")
        say(tag)
        q, _, _ = W.gaussian_qkv(B, H, Sq, D, dtype, seed=3000 + n)
        _, k, v = W.gaussian_qkv(B, H, Skv, D, dtype, seed=4000 + n)
        qd, kd, vd = (_device_view(t, layout) for t in (q, k, v))
        if layout == "bshd":
            od = torch.empty((B, Sq, H, D), dtype=q.dtype, device="cuda").transpose(1, 2)
        else:
            od = torch.empty((B, H, Sq, D), dtype=q.dtype, device="cuda")
        o, lse = da.attn_fwd_strided(qd, kd, vd, od, scale=scale, variant=variant, causal=causal,
                                     grid=grid)
        torch.cuda.synchronize()
        offset = None if causal is False else (Skv - Sq if causal is True else causal)
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale,
                                   causal_offset=offset)
        go = o.cpu().to(torch.float64).numpy()
        gl = lse.cpu().to(torch.float64).numpy()
        err = np.abs(go - ro)
        none = np.isneginf(rl)
        assert np.array_equal(np.isneginf(gl), none), tag
        lerr = np.abs(gl[~none] - rl[~none]).max() if (~none).any() else 0.0
        say(f"  O max {err.max():.3e} mean {err.mean():.3e} LSE max {lerr:.3e}")
        assert np.all(np.isfinite(go)), tag
        assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr <= LSE_MAX, tag
