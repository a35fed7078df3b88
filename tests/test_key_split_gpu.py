"""GPU parity tests of the key-split tiling (the two wave groups of a workgroup
hold the same 128 query rows, each streams half of the keys, and the halves are
merged through LDS), called through the C ABI, against the float64 CPU oracle.

Bar as everywhere: max |dO| <= 2e-2, mean |dO| <= 2e-3 against the unrounded
oracle, max |dLSE| <= 1e-3; rows without a visible key give O = 0, LSE = -inf.
"""

import math
import sys

import numpy as np
import pytest
import torch

import dense_attention_amd as da
import workloads as W
from oracle import attention_forward

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.load_library()
    yield
    torch.cuda.synchronize()


def split_variants(D, dtype):
    """Every key-split tiling for (D, dtype) with hardware exp2 (64- and 128-key tiles)."""
    code = da.ATTN_F16 if dtype == "fp16" else da.ATTN_BF16
    ids = [v["id"] for v in da.attn_variants()
           if v["head_dim"] == D and v["dtype"] == code and v["key_split"] == 1
           and v["soft_exp"] == 0]
    assert ids, (D, dtype)
    return ids


def compare(o, lse, ro, rl, tag):
    go = o.detach().cpu().to(torch.float64).numpy()
    err = np.abs(go - ro)
    gl = lse.detach().cpu().double().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), f"{tag}: rows without keys differ"
    le = np.abs(gl[~empty] - rl[~empty]) if (~empty).any() else np.zeros(1)
    say(f"  {tag}: O max {err.max():.3e} mean {err.mean():.3e} LSE max {le.max():.3e}")
    assert np.all(np.isfinite(go)), tag
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, tag
    assert le.max() <= LSE_MAX, tag


def test_default_choice_follows_grid_fill():
    """Few 256-row items: the key split; enough to fill the device: the shared stream."""
    small = da.attn_get_config(1, 8, 4096, 64, torch.float16)      # 128 items of 256 rows
    assert small["block_m"] == 128 and small["waves"] == 8
    assert [v for v in da.attn_variants() if v["id"] == small["variant"]][0]["key_split"] == 1
    big = da.attn_get_config(2, 16, 8192, 128, torch.bfloat16)     # 1024 items of 256 rows
    assert big["block_m"] == 256
    assert [v for v in da.attn_variants() if v["id"] == big["variant"]][0]["key_split"] == 0


# Key tiles of 64: 1 tile (group 1 idle), 2, 3 and 5 (group 1 one tile short), ragged tails.
LENGTHS = [1, 64, 65, 129, 192, 300, 320, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
def test_tile_counts_and_tails(D, dtype):
    for S in LENGTHS:
        q, k, v = W.gaussian_qkv(2, 3, S, D, dtype, seed=4000 + S)
        scale = 1.0 / math.sqrt(D)
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale)
        for var in split_variants(D, dtype):
            say(f"key split S={S} D={D} {dtype} variant {var}")
            o, lse = da.attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), scale=scale, variant=var)
            torch.cuda.synchronize()
            compare(o, lse, ro, rl, f"S={S} D={D} {dtype} v{var}")


@pytest.mark.parametrize("thr", [0.0, 8.0, 64.0])
def test_halves_with_far_apart_maxima(thr):
    """Keys 512-1023 scaled x4: the second half's running maximum lies far above
    the first half's, so the merge weights 2^(m_g - m) span many octaves."""
    q, k, v = W.forced_rebase_qkv()
    kf, vf = k.flip(2).contiguous(), v.flip(2).contiguous()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / 8)
    rof, rlf = attention_forward(W.to_f64(q), W.to_f64(kf), W.to_f64(vf), 1 / 8)
    for var in split_variants(64, "bf16"):
        o, lse = da.attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), scale=1 / 8, variant=var,
                                rescale_threshold=thr)
        torch.cuda.synchronize()
        compare(o, lse, ro, rl, f"forced rebase thr={thr} v{var}")
        # The same with the large keys in the first half instead.
        o, lse = da.attn_fwd_ex(q.cuda(), kf.cuda(), vf.cuda(), scale=1 / 8, variant=var,
                                rescale_threshold=thr)
        torch.cuda.synchronize()
        compare(o, lse, rof, rlf, f"forced rebase flipped thr={thr} v{var}")


@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16")])
def test_negative_scale_and_causal(D, dtype):
    q, k, v = W.gaussian_qkv(1, 2, 333, D, dtype, seed=4100)
    for var in split_variants(D, dtype):
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), -0.1)
        o, lse = da.attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), scale=-0.1, variant=var)
        torch.cuda.synchronize()
        compare(o, lse, ro, rl, f"scale=-0.1 v{var}")
        for off in [0, -70, 200]:
            ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(D),
                                       causal_offset=off)
            o, lse = da.attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), variant=var,
                                    causal=True if off == 0 else off)
            torch.cuda.synchronize()
            compare(o, lse, ro, rl, f"causal offset {off} v{var}")


@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16")])
def test_with_kv_ranges_and_strided_layouts(D, dtype):
    """Key split inside each KV range of attn_fwd_split, and over BSHD views
    with Sq != Skv."""
    q, k, v = W.gaussian_qkv(1, 4, 1500, D, dtype, seed=4200)
    scale = 1.0 / math.sqrt(D)
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale)
    qs = W.gaussian_qkv(1, 4, 211, D, dtype, seed=4201)[0]
    to_bshd = lambda t: t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    ros, rls = attention_forward(W.to_f64(qs), W.to_f64(k), W.to_f64(v), scale)
    for var in split_variants(D, dtype):
        for n in [2, 3]:
            o, lse = da.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), scale=scale, kv_splits=n,
                                       variant=var)
            torch.cuda.synchronize()
            compare(o, lse, ro, rl, f"kv_splits={n} v{var}")
        o, lse = da.attn_fwd_strided(to_bshd(qs), to_bshd(k), to_bshd(v), scale=scale, variant=var)
        torch.cuda.synchronize()
        compare(o, lse, ros, rls, f"bshd Sq=211 Skv=1500 v{var}")


def test_grid_sizes_agree_bit_for_bit():
    q, k, v = W.gaussian_qkv(1, 3, 777, 64, "fp16", seed=4300)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(64))
    for var in split_variants(64, "fp16"):
        ref, ref_l = da.attn_fwd_ex(qd, kd, vd, variant=var)
        torch.cuda.synchronize()
        compare(ref, ref_l, ro, rl, f"grid reference launch v{var}")
        for g in [1, 5, 8, 17]:
            o, lse = da.attn_fwd_ex(qd, kd, vd, variant=var, grid=g)
            torch.cuda.synchronize()
            assert torch.equal(o, ref) and torch.equal(lse, ref_l), (var, g)
