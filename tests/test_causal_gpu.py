"""GPU parity tests of the causal mask (query row i sees keys j <= i + offset),
called through the C ABI, against the float64 CPU oracle with the same mask.

Bar as for the unmasked forward: max |dO| <= 2e-2, mean |dO| <= 2e-3 against
the unrounded oracle, max |dLSE| <= 1e-3; rows that see no key must come out
as O = 0 and LSE = -inf exactly.
"""

import math
import sys

import numpy as np
import pytest
import torch

import dense_attention_amd as da
import workloads as W
from oracle import attention_forward
from tests.oracle_by_head import forward_by_head

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


def compare(o, lse, ro, rl, tag):
    go = o.detach().cpu().to(torch.float64).numpy()
    err = np.abs(go - ro)
    gl = lse.detach().cpu().double().numpy()
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), f"{tag}: rows without keys differ"
    le = np.abs(gl[~empty] - rl[~empty]) if (~empty).any() else np.zeros(1)
    say(f"  {tag}: O max {err.max():.3e} mean {err.mean():.3e} LSE max {le.max():.3e}"
        f" ({int(empty.sum())} rows without keys)")
    assert np.all(np.isfinite(go)), tag
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, tag
    assert le.max() <= LSE_MAX, tag


def variants_for(D, dtype):
    code = da.ATTN_F16 if dtype == "fp16" else da.ATTN_BF16
    return [v["id"] for v in da.attn_variants() if v["head_dim"] == D and v["dtype"] == code]


RAGGED = [1, 2, 31, 64, 65, 100, 255, 256, 257, 600, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
def test_causal_ragged_all_variants(D, dtype):
    for S in RAGGED:
        q, k, v = W.gaussian_qkv(2, 3, S, D, dtype, seed=2000 + S)
        scale = 1.0 / math.sqrt(D)
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal_offset=0)
        for var in variants_for(D, dtype):
            say(f"causal S={S} D={D} {dtype} variant {var}")
            o, lse = da.attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), scale=scale, variant=var,
                                    causal=True)
            torch.cuda.synchronize()
            compare(o, lse, ro, rl, f"causal S={S} D={D} {dtype} v{var}")


def test_causal_s4096_d64_fp16_full():
    w = W.BY_NAME["b1_h8_s4096_d64_fp16"]
    q, k, v = W.workload_qkv(w)
    o, lse = da.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), w.scale, causal_offset=0)
    compare(o, lse, ro, rl, f"{w.name} causal")
    # row 0 sees key 0 only
    assert (o[:, :, 0].float().cpu() - v[:, :, 0].float()).abs().max().item() <= 1e-2


@pytest.mark.parametrize("name", ["b4_h16_s4096_d128_bf16", "b2_h16_s8192_d128_bf16"])
def test_causal_hd128_full(name):
    """The hd128 workloads with the causal mask, every element against the oracle."""
    w = W.BY_NAME[name]
    q, k, v = W.workload_qkv(w)
    say(f"{w.name} causal")
    o, lse = da.attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    ro, rl = forward_by_head(q, k, v, w.scale, causal_offset=0)
    compare(o, lse, ro, rl, f"{w.name} causal, whole output")


@pytest.mark.parametrize("Sq,Skv,offset", [(100, 300, None), (300, 100, None), (257, 257, 64),
                                           (257, 257, -64), (129, 1000, -100), (64, 64, -64)])
def test_causal_offsets_and_lengths(Sq, Skv, offset):
    """offset None: the last query row sees every key (offset = Skv - Sq)."""
    for D, dtype in [(64, "fp16"), (128, "bf16")]:
        q = W.gaussian_qkv(1, 2, Sq, D, dtype, seed=3100 + Sq)[0]
        _, k, v = W.gaussian_qkv(1, 2, Skv, D, dtype, seed=3200 + Skv)
        off = Skv - Sq if offset is None else offset
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(D),
                                   causal_offset=off)
        o, lse = da.attn_fwd_strided(q.cuda(), k.cuda(), v.cuda(),
                                     causal=True if offset is None else offset)
        torch.cuda.synchronize()
        compare(o, lse, ro, rl, f"Sq={Sq} Skv={Skv} offset={off} D={D}")


def test_causal_negative_scale_and_forced_rebase():
    q, k, v = W.gaussian_qkv(1, 2, 333, 64, "bf16", seed=3300)
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), -0.125, causal_offset=0)
    o, lse = da.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=-0.125, causal=True)
    torch.cuda.synchronize()
    compare(o, lse, ro, rl, "causal scale=-0.125")
    q, k, v = W.forced_rebase_qkv()
    for thr in [0.0, 8.0]:
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / 8, causal_offset=0)
        o, lse = da.attn_fwd_ex(q.cuda(), k.cuda(), v.cuda(), causal=True, rescale_threshold=thr)
        torch.cuda.synchronize()
        compare(o, lse, ro, rl, f"causal forced rebase thr={thr}")


def test_causal_key_shards_merge():
    """Sequence-sharded causal attention: each key shard [a, b) is a partial
    with offset (Skv - Sq) - a; shards entirely after a query's diagonal give
    O = 0, LSE = -inf for it, and the merge ignores them."""
    B, H, S, D = 1, 2, 1100, 128
    q, k, v = W.gaussian_qkv(B, H, S, D, "bf16", seed=3400)
    qn, kn, vn = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    scale = 1 / math.sqrt(D)
    ro, rl = attention_forward(qn, kn, vn, scale, causal_offset=0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    edges = [0, 1, 300, 301, 640, 1100]
    parts = list(zip(edges[:-1], edges[1:]))
    op = torch.empty(len(parts), B, H, S, D, dtype=torch.float32, device="cuda")
    lp = torch.empty(len(parts), B, H, S, dtype=torch.float32, device="cuda")
    for g, (a, b) in enumerate(parts):
        da.attn_fwd_partial(qd, kd[:, :, a:b], vd[:, :, a:b], op[g], lp[g], causal=-a)
    torch.cuda.synchronize()
    for g, (a, b) in enumerate(parts):
        po, pl = attention_forward(qn, kn[:, :, a:b], vn[:, :, a:b], scale, causal_offset=-a)
        compare(op[g], lp[g], po, pl, f"causal partial [{a},{b})")
    o, lse = da.attn_merge(op, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    compare(o, lse, ro, rl, "causal merge of key shards")


@pytest.mark.parametrize("splits", [2, 5])
def test_causal_split_kv(splits):
    w = W.BY_NAME["b1_h8_s4096_d64_fp16"]
    q, k, v = W.workload_qkv(w)
    o, lse = da.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), kv_splits=splits, causal=True)
    torch.cuda.synchronize()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), w.scale, causal_offset=0)
    compare(o, lse, ro, rl, f"causal split {splits}")


def test_causal_grid_sizes_agree():
    """One workgroup per item (default) and persistent grids give identical bits."""
    q, k, v = W.gaussian_qkv(2, 4, 1111, 128, "bf16", seed=3500)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref, ref_l = da.attn_fwd_ex(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(128),
                               causal_offset=0)
    compare(ref, ref_l, ro, rl, "causal grid reference launch")
    for g in [1, 7, 64]:
        o, lse = da.attn_fwd_ex(qd, kd, vd, causal=True, grid=g)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lse, ref_l), g
