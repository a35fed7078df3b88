"""GPU parity tests of the strided-layout, key-range (partial), merge and split-KV
entry points, called through the C ABI, against the float64 CPU oracle.

Same bar as the plain forward: max |dO| <= 2e-2, mean |dO| <= 2e-3 against the
unrounded oracle, max |dLSE| <= 1e-3.  A partial over keys [a, b) is checked
against the oracle run on exactly those keys; a merge of partials against the
oracle on their union.
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


def compare(o, lse, ro, rl, tag):
    go = o.detach().cpu().to(torch.float64).numpy()
    err = np.abs(go - ro)
    msg = f"  {tag}: O max {err.max():.3e} mean {err.mean():.3e}"
    if lse is not None:
        le = np.abs(lse.cpu().double().numpy() - rl)
        msg += f" LSE max {le.max():.3e}"
    say(msg)
    assert np.all(np.isfinite(go)), tag
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, tag
    if lse is not None:
        assert le.max() <= LSE_MAX, tag


def variants_for(D, dtype):
    code = da.ATTN_F16 if dtype == "fp16" else da.ATTN_BF16
    return [v["id"] for v in da.attn_variants() if v["head_dim"] == D and v["dtype"] == code]


# --- strided layouts -----------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
def test_bshd_layout_matches_oracle(D, dtype):
    """Contiguous BSHD storage, seen as [B, H, S, D] through transpose(1, 2)."""
    for S in [129, 1000]:
        q, k, v = W.gaussian_qkv(2, 3, S, D, dtype, seed=300 + S)
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(D))
        # BSHD copies of the same values
        qs, ks, vs = (t.transpose(1, 2).contiguous().cuda() for t in (q, k, v))
        o_s = torch.empty_like(qs)
        for var in variants_for(D, dtype):
            say(f"BSHD S={S} D={D} {dtype} variant {var}")
            o, lse = da.attn_fwd_strided(qs.transpose(1, 2), ks.transpose(1, 2), vs.transpose(1, 2),
                                         o_s.transpose(1, 2), variant=var)
            torch.cuda.synchronize()
            assert o.data_ptr() == o_s.data_ptr()
            compare(o_s.transpose(1, 2), lse, ro, rl, f"BSHD S={S} D={D} {dtype} v{var}")


def test_mixed_layouts_and_padded_rows():
    """q in BSHD, k in BHSD, v with padded rows, o with padded rows: all at once."""
    B, H, S, D = 1, 4, 777, 128
    q, k, v = W.gaussian_qkv(B, H, S, D, "bf16", seed=310)
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 0.09)
    qd = q.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    kd = k.cuda()
    vpad = torch.zeros(B, H, S, D + 64, dtype=v.dtype, device="cuda")
    vpad[..., :D] = v.cuda()
    opad = torch.full((B, H, S, D + 32), 7.0, dtype=v.dtype, device="cuda")
    o, lse = da.attn_fwd_strided(qd, kd, vpad[..., :D], opad[..., :D], scale=0.09)
    torch.cuda.synchronize()
    compare(opad[..., :D], lse, ro, rl, "mixed layouts")
    assert bool((opad[..., D:] == 7.0).all()), "row padding of o was written"


@pytest.mark.parametrize("Sq,Skv", [(1, 300), (100, 1), (257, 64), (1000, 129), (64, 4096)])
def test_cross_lengths(Sq, Skv):
    """Sq queries over Skv keys (a key set of another length)."""
    for D, dtype in [(64, "fp16"), (128, "bf16")]:
        q = W.gaussian_qkv(2, 2, Sq, D, dtype, seed=320 + Sq)[0]
        _, k, v = W.gaussian_qkv(2, 2, Skv, D, dtype, seed=330 + Skv)
        ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(D))
        o, lse = da.attn_fwd_strided(q.cuda(), k.cuda(), v.cuda())
        torch.cuda.synchronize()
        compare(o, lse, ro, rl, f"Sq={Sq} Skv={Skv} D={D}")


# --- key ranges (partials) and their merge -------------------------------------------

def _ranges(S, cuts):
    edges = [0] + list(cuts) + [S]
    return [(a, b) for a, b in zip(edges[:-1], edges[1:])]


@pytest.mark.parametrize("D,dtype", [(64, "fp16"), (128, "bf16")])
def test_partials_over_key_slices_and_merge(D, dtype):
    """Each device of a sequence-sharded run holds a key slice; here the slices
    are views of one tensor.  Uneven cuts, a one-key slice, a ragged tail."""
    B, H, S = 1, 4, 1500
    q, k, v = W.gaussian_qkv(B, H, S, D, dtype, seed=340)
    qn, kn, vn = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    scale = 1 / math.sqrt(D)
    ro, rl = attention_forward(qn, kn, vn, scale)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for cuts in [(700,), (1, 64, 65, 1000), (128, 256, 384, 512, 640, 768, 896)]:
        parts = _ranges(S, cuts)
        o_parts = torch.empty(len(parts), B, H, S, D, dtype=torch.float32, device="cuda")
        lse_parts = torch.empty(len(parts), B, H, S, dtype=torch.float32, device="cuda")
        for g, (a, b) in enumerate(parts):
            da.attn_fwd_partial(qd, kd[:, :, a:b], vd[:, :, a:b], o_parts[g], lse_parts[g])
        torch.cuda.synchronize()
        # each partial is the oracle over its own keys
        for g, (a, b) in enumerate(parts):
            po, pl = attention_forward(qn, kn[:, :, a:b], vn[:, :, a:b], scale)
            compare(o_parts[g], lse_parts[g], po, pl, f"partial [{a},{b}) D={D}")
        out_dtype = q.dtype
        o, lse = da.attn_merge(o_parts, lse_parts, out_dtype=out_dtype)
        torch.cuda.synchronize()
        compare(o, lse, ro, rl, f"merge of {len(parts)} D={D}")
        o32, lse32 = da.attn_merge(o_parts, lse_parts, out_dtype=torch.float32)
        torch.cuda.synchronize()
        compare(o32, lse32, ro, rl, f"fp32 merge of {len(parts)} D={D}")


def test_merge_is_associative_and_skips_empty_parts():
    """Merging (A, B) then C equals merging A, B, C; a part with lse = -inf has no weight."""
    B, H, S, D = 1, 2, 600, 64
    q, k, v = W.gaussian_qkv(B, H, S, D, "bf16", seed=350)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    parts = _ranges(S, (200, 400))
    op = torch.empty(3, B, H, S, D, dtype=torch.float32, device="cuda")
    lp = torch.empty(3, B, H, S, dtype=torch.float32, device="cuda")
    for g, (a, b) in enumerate(parts):
        da.attn_fwd_partial(qd, kd[:, :, a:b], vd[:, :, a:b], op[g], lp[g])
    ab_o, ab_l = da.attn_merge(op[:2].contiguous(), lp[:2].contiguous(), out_dtype=torch.float32)
    two_o = torch.stack([ab_o, op[2]]).contiguous()
    two_l = torch.stack([ab_l, lp[2]]).contiguous()
    o2, l2 = da.attn_merge(two_o, two_l, out_dtype=torch.float32)
    o3, l3 = da.attn_merge(op, lp, out_dtype=torch.float32)
    # an extra empty part (lse = -inf, garbage O) must not change anything
    junk_o = torch.full((1, B, H, S, D), 1e30, dtype=torch.float32, device="cuda")
    junk_l = torch.full((1, B, H, S), -float("inf"), dtype=torch.float32, device="cuda")
    o4, l4 = da.attn_merge(torch.cat([op, junk_o]).contiguous(), torch.cat([lp, junk_l]).contiguous(),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o2 - o3).abs().max().item() <= 1e-6 and (l2 - l3).abs().max().item() <= 1e-6
    assert (o4 - o3).abs().max().item() <= 1e-6 and (l4 - l3).abs().max().item() <= 1e-6
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(D))
    compare(o3, l3, ro, rl, "three-way merge")
    # all parts empty: O = 0, LSE = -inf
    o5, l5 = da.attn_merge(junk_o.contiguous(), junk_l.contiguous(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool((o5 == 0).all()) and bool(torch.isneginf(l5).all())


# --- split-KV in one call ----------------------------------------------------------------

@pytest.mark.parametrize("splits", [0, 2, 3, 8])
def test_split_kv_config_s4096_d64_fp16(splits):
    w = W.BY_NAME["b1_h8_s4096_d64_fp16"]
    q, k, v = W.workload_qkv(w)
    say(f"{w.name} kv_splits={splits}")
    o, lse = da.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), kv_splits=splits)
    torch.cuda.synchronize()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), w.scale)
    compare(o, lse, ro, rl, f"{w.name} split {splits}")


def test_split_kv_small_config_and_ragged():
    for (B, H, S, D, dtype, splits) in [(1, 4, 128, 64, "fp16", 2), (2, 3, 1000, 128, "bf16", 3),
                                        (1, 2, 65, 64, "bf16", 8), (1, 1, 3000, 128, "fp16", 0)]:
        q, k, v = W.gaussian_qkv(B, H, S, D, dtype, seed=360 + S)
        for var in variants_for(D, dtype):
            say(f"split S={S} D={D} {dtype} splits={splits} variant {var}")
            o, lse = da.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), kv_splits=splits, variant=var)
            torch.cuda.synchronize()
            ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(D))
            compare(o, lse, ro, rl, f"split S={S} D={D} v{var} n={splits}")


def test_split_kv_forced_rebase():
    q, k, v = W.forced_rebase_qkv()
    o, lse = da.attn_fwd_split(q.cuda(), k.cuda(), v.cuda(), kv_splits=4)
    torch.cuda.synchronize()
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(64))
    compare(o, lse, ro, rl, "split forced rebase")


def test_split_rejects_small_workspace():
    q, k, v = W.gaussian_qkv(1, 2, 1024, 64, "fp16", seed=370)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(da.AttnError) as e:
        da.attn_fwd_split(qd, kd, vd, kv_splits=4, workspace=ws)
    assert e.value.status == -8
