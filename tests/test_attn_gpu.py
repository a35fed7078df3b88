"""GPU parity tests: the HIP attention forward, called through the C ABI, against
the float64 CPU oracle on the same seeded inputs.

Bar (O against the unrounded float64 oracle, LSE absolute):
    max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-3.
Every element is compared, the five workloads at their full sizes included
(in the launch configuration the benchmark times; the oracle runs head by
head in parallel threads).  Only the inputs past 2^31 elements and the
S = 32785 case, whose oracle would not fit the time, are checked on sampled
rows, each computed by the oracle against all keys.
"""

import math
import sys

import numpy as np
import pytest
import torch

import dense_attention_amd as da
import workloads as W
from oracle import attention_forward, attention_rows
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


def gpu_run(q, k, v, scale, **kw):
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = da.attn_fwd_ex(qd, kd, vd, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def check_full(o, lse, q, k, v, scale, tag=""):
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale)
    go = o.cpu().to(torch.float64).numpy()
    err = np.abs(go - ro)
    say(f"  {tag} O max {err.max():.3e} mean {err.mean():.3e}" +
        (f" LSE max {np.abs(lse.cpu().double().numpy() - rl).max():.3e}" if lse is not None else ""))
    assert np.all(np.isfinite(go))
    assert err.max() <= O_MAX and err.mean() <= O_MEAN, tag
    if lse is not None:
        gl = lse.cpu().to(torch.float64).numpy()
        assert np.all(np.isfinite(gl))
        assert np.abs(gl - rl).max() <= LSE_MAX, tag
    return ro, rl


def variants_for(D, dtype):
    code = da.ATTN_F16 if dtype == "fp16" else da.ATTN_BF16
    return [v["id"] for v in da.attn_variants() if v["head_dim"] == D and v["dtype"] == code]


# --- the five workloads ------------------------------------------------------

def test_config_small_fp16_all_variants():
    w = W.BY_NAME["b1_h4_s128_d64_fp16"]
    q, k, v = W.workload_qkv(w)
    for var in [0] + variants_for(w.D, w.dtype):
        say(f"{w.name} variant {var}")
        o, lse = gpu_run(q, k, v, w.scale, variant=var)
        check_full(o, lse, q, k, v, w.scale, tag=f"{w.name}/v{var}")


def test_config_s4096_d64_fp16_full():
    w = W.BY_NAME["b1_h8_s4096_d64_fp16"]
    q, k, v = W.workload_qkv(w)
    say(f"{w.name} default launch")
    o, lse = gpu_run(q, k, v, w.scale)
    check_full(o, lse, q, k, v, w.scale, tag=w.name)


def _sample_rows(S, n, rng, tile=128):
    rows = set(rng.choice(S, size=n, replace=False).tolist())
    rows |= {0, 1, tile - 1, tile, S // 2, S - tile, S - 1}
    return np.array(sorted(r for r in rows if 0 <= r < S))


@pytest.mark.parametrize("name", ["b4_h16_s4096_d128_bf16", "b2_h16_s8192_d128_bf16",
                                  "b1_h16_s16384_d128_bf16"])
def test_config_hd128_bf16_full(name):
    """The three hd128 workloads in the benchmark's launch configuration, every
    element of O and LSE against the oracle (heads computed in parallel)."""
    w = W.BY_NAME[name]
    q, k, v = W.workload_qkv(w)
    say(f"{w.name} default launch (the benchmark's)")
    o, lse = gpu_run(q, k, v, w.scale)
    go = o.cpu().double().numpy()
    gl = lse.cpu().double().numpy()
    del o, lse
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    ro, rl = forward_by_head(q, k, v, w.scale)
    err = np.abs(go - ro)
    lerr = np.abs(gl - rl).max()
    say(f"  {w.name} whole output: O max {err.max():.3e} mean {err.mean():.3e} "
        f"LSE max {lerr:.3e} ({err.size} elements)")
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr <= LSE_MAX


def test_bench_bshd_and_split_launches_full():
    """The benchmark's other launch paths at the S = 8192, D = 128 size: BSHD
    storage through attn_fwd_strided (``--layout bshd``) and split-KV with the
    library's own range count (``--kv-splits 0``); every element against the oracle."""
    w = W.BY_NAME["b2_h16_s8192_d128_bf16"]
    q, k, v = W.workload_qkv(w)
    ro, rl = forward_by_head(q, k, v, w.scale)

    def whole(o, lse, tag):
        err = np.abs(o.cpu().double().numpy() - ro)
        lerr = np.abs(lse.cpu().double().numpy() - rl).max()
        say(f"  {tag} whole output: O max {err.max():.3e} mean {err.mean():.3e} LSE max {lerr:.3e}")
        assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr <= LSE_MAX, tag

    say(f"{w.name} BSHD storage through attn_fwd_strided")
    qd, kd, vd = (t.transpose(1, 2).contiguous().cuda().transpose(1, 2) for t in (q, k, v))
    od = torch.empty((w.B, w.S, w.H, w.D), dtype=q.dtype, device="cuda").transpose(1, 2)
    o, lse = da.attn_fwd_strided(qd, kd, vd, od, scale=w.scale)
    torch.cuda.synchronize()
    assert o.data_ptr() == od.data_ptr()
    whole(o, lse, "bshd")
    del qd, kd, vd, od, o, lse
    say(f"{w.name} split-KV, library range count")
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    nbytes = da.attn_fwd_split_workspace_size(w.B, w.H, w.S, w.D, 0)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    o, lse = da.attn_fwd_split(qd, kd, vd, scale=w.scale, kv_splits=0, workspace=ws)
    torch.cuda.synchronize()
    whole(o, lse, "split")


# --- edge cases -----------------------------------------------------------------

RAGGED = [1, 2, 31, 64, 65, 100, 127, 129, 200, 257, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
def test_ragged_lengths_all_variants(D, dtype):
    for S in RAGGED:
        q, k, v = W.gaussian_qkv(2, 3, S, D, dtype, seed=1000 + S)
        scale = 1.0 / math.sqrt(D)
        for var in variants_for(D, dtype):
            say(f"ragged S={S} D={D} {dtype} variant {var}")
            o, lse = gpu_run(q, k, v, scale, variant=var)
            check_full(o, lse, q, k, v, scale, tag=f"S{S}/D{D}/{dtype}/v{var}")


# Lengths whose steady loops (tiles minus four, per wave group) run zero to
# sixteen steps, so the loop unrolled by the ring depth ends with every
# remainder, with and without a ragged last tile.
STEADY_LENGTHS = [320, 383, 448, 511, 576, 640, 700, 768, 900, 1024, 1280]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
def test_steady_loop_lengths_all_variants(D, dtype):
    for S in STEADY_LENGTHS:
        q, k, v = W.gaussian_qkv(1, 2, S, D, dtype, seed=2000 + S)
        scale = 1.0 / math.sqrt(D)
        for var in variants_for(D, dtype):
            say(f"steady S={S} D={D} {dtype} variant {var}")
            o, lse = gpu_run(q, k, v, scale, variant=var)
            check_full(o, lse, q, k, v, scale, tag=f"S{S}/D{D}/{dtype}/v{var}")


def test_empty_problem_launches_nothing():
    q = torch.zeros(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = da.attn_fwd(q, q, q)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    q = torch.zeros(1, 1, 0, 128, dtype=torch.float16, device="cuda")
    o, lse = da.attn_fwd(q, q, q)
    torch.cuda.synchronize()
    assert o.numel() == 0


def test_lse_pointer_may_be_null():
    q, k, v = W.gaussian_qkv(1, 2, 300, 128, "bf16", seed=7)
    o, lse = gpu_run(q, k, v, 1 / math.sqrt(128), return_lse=False)
    assert lse is None
    check_full(o, None, q, k, v, 1 / math.sqrt(128), tag="lse=NULL")


def test_zero_query_gives_mean_of_v_and_ln_s():
    for D, dtype, S in [(64, "fp16", 384), (128, "bf16", 1000)]:
        _, k, v = W.gaussian_qkv(1, 2, S, D, dtype, seed=21)
        q = torch.zeros_like(k)
        o, lse = gpu_run(q, k, v, 1 / math.sqrt(D))
        mean_v = W.to_f64(v).mean(axis=2, keepdims=True)
        err = np.abs(o.cpu().double().numpy() - mean_v)
        say(f"  Q=0 D={D} S={S} O max {err.max():.3e}")
        assert err.max() <= O_MAX and err.mean() <= O_MEAN
        assert np.abs(lse.cpu().double().numpy() - math.log(S)).max() <= LSE_MAX


def test_constant_v():
    q, k, _ = W.gaussian_qkv(1, 2, 777, 128, "bf16", seed=22)
    c = torch.linspace(-2, 2, 128).to(torch.bfloat16)
    v = c.expand(1, 2, 777, 128).contiguous()
    o, _ = gpu_run(q, k, v, 1 / math.sqrt(128))
    err = (o.cpu().double() - c.double()).abs()
    assert err.max() <= O_MAX and err.mean() <= O_MEAN


def test_scale_zero_negative_and_sharp():
    q, k, v = W.gaussian_qkv(1, 2, 333, 64, "bf16", seed=23)
    for scale in [0.0, -0.125, 1.0]:
        say(f"scale {scale}")
        o, lse = gpu_run(q, k, v, scale)
        check_full(o, lse, q, k, v, scale, tag=f"scale={scale}")


@pytest.mark.parametrize("thr", [0.0, 8.0, 64.0])
def test_forced_rebase_thresholds(thr):
    q, k, v = W.forced_rebase_qkv()
    o, lse = gpu_run(q, k, v, 1 / math.sqrt(64), rescale_threshold=thr)
    check_full(o, lse, q, k, v, 1 / math.sqrt(64), tag=f"threshold {thr}")


@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "fp16")])
def test_forced_rebase_all_variants(D, dtype):
    """The rebase path past the first tile in every tiling: the second half of
    the keys scaled x4 moves the row maxima mid-stream, and keys growing along
    the sequence move them on every tile."""
    q, k, v = W.forced_rebase_qkv(B=1, H=2, S=1000, D=D, dtype=dtype, seed=31)
    ramp = W.gaussian_qkv(1, 2, 1000, D, dtype, seed=32)
    qr = ramp[0]
    kr = (ramp[1].float() * torch.linspace(0.25, 3.0, 1000).view(1, 1, -1, 1)).to(ramp[1].dtype)
    vr = v  # uniform on (-1, 1): peaked rows keep |O| small
    scale = 1 / math.sqrt(D)
    for var in variants_for(D, dtype):
        for thr in [0.0, 8.0]:
            say(f"forced rebase D={D} {dtype} variant {var} thr {thr}")
            o, lse = gpu_run(q, k, v, scale, variant=var, rescale_threshold=thr)
            check_full(o, lse, q, k, v, scale, tag=f"forced v{var} thr {thr}")
        say(f"growing keys D={D} {dtype} variant {var}")
        o, lse = gpu_run(qr, kr, vr, scale, variant=var)
        check_full(o, lse, qr, kr, vr, scale, tag=f"growing keys v{var}")


@pytest.mark.parametrize("D", [64, 128])
def test_fp16_threshold_15_keeps_p_finite(D):
    """fp16 P at the largest threshold fp16 allows.  With a kept maximum p reaches
    2^threshold; 2^15 is finite in fp16 (65504 is its largest value), 2^16 is not,
    so 15 is the bound.  On these inputs (keys of the second half scaled x4) about
    two thirds of the rows see their maximum rise by 8 to 15 log2 units after the
    first tile (kept, so p runs up to 2^15) and the rest by more than 15 (moved).
    Every fp16 tiling, with and without the causal mask; 16 is refused."""
    q, k, v = W.forced_rebase_qkv(B=1, H=2, S=1000, D=D, dtype="fp16", seed=31)
    scale = 1 / math.sqrt(D)
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale)
    rco, rcl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale, causal_offset=0)
    for var in variants_for(D, "fp16"):
        for causal in (False, True):
            say(f"fp16 threshold 15 D={D} variant {var} causal={causal}")
            o, lse = gpu_run(q, k, v, scale, variant=var, rescale_threshold=15.0, causal=causal)
            go = o.cpu().double().numpy()
            assert np.all(np.isfinite(go)), f"v{var} causal={causal}: non-finite O"
            err = np.abs(go - (rco if causal else ro))
            le = np.abs(lse.cpu().double().numpy() - (rcl if causal else rl)).max()
            say(f"  O max {err.max():.3e} mean {err.mean():.3e} LSE max {le:.3e}")
            assert err.max() <= O_MAX and err.mean() <= O_MEAN and le <= LSE_MAX
    with pytest.raises(da.AttnError):
        gpu_run(q, k, v, scale, rescale_threshold=16.0)


def test_tile_signature_exact():
    """Q = 0 and a one-hot V per 64-key tile: every stale, skipped or doubled tile shows."""
    for D, dtype in [(128, "bf16"), (64, "fp16")]:
        S = 4096
        for var in variants_for(D, dtype):
            v = W.tile_signature_v(1, 2, S, D, dtype, tile=64)
            q = torch.zeros_like(v)
            k = W.gaussian_qkv(1, 2, S, D, dtype, seed=24)[1]
            o, lse = gpu_run(q, k, v, 1 / math.sqrt(D), variant=var)
            expect = np.zeros(D)
            cols = (np.arange(S) // 64) % D
            np.add.at(expect, cols, 1.0 / S)
            err = np.abs(o.cpu().double().numpy() - expect)
            say(f"  tile signature D={D} variant {var}: max err {err.max():.3e}")
            assert err.max() <= 1e-6


def test_grid_sizes_give_identical_results():
    """Every grid size gives the default launch's bits, and those match the oracle."""
    q, k, v = W.gaussian_qkv(2, 4, 1111, 128, "bf16", seed=25)
    ref, ref_l = gpu_run(q, k, v, 0.088)
    check_full(ref, ref_l, q, k, v, 0.088, tag="grid reference launch")
    for g in [1, 3, 8, 13, 64]:
        say(f"grid {g}")
        o, lse = gpu_run(q, k, v, 0.088, grid=g)
        assert torch.equal(o, ref) and torch.equal(lse, ref_l), g


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16"), (128, "fp16"), (64, "bf16")])
def test_persistent_rounds_all_variants(D, dtype):
    """Grids far below the item count, every tiling: each workgroup runs many
    items in turn, ragged last query tiles among them.  On non-causal grids an
    item issues the next item's first copies and Q rows ahead of its own
    output stores, which go through LDS where the tiling has room for it."""
    scale = 1 / math.sqrt(D)
    q, k, v = W.gaussian_qkv(1, 3, 1111, D, dtype, seed=37)
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale)
    for var in variants_for(D, dtype):
        for g in (1, 5):
            say(f"rounds D={D} {dtype} variant {var} grid {g}")
            o, lse = gpu_run(q, k, v, scale, variant=var, grid=g)
            err = np.abs(o.cpu().to(torch.float64).numpy() - ro)
            el = np.abs(lse.cpu().to(torch.float64).numpy() - rl)
            say(f"  O max {err.max():.3e} mean {err.mean():.3e} LSE max {el.max():.3e}")
            assert np.all(np.isfinite(err)) and np.all(np.isfinite(el))
            assert err.max() <= O_MAX and err.mean() <= O_MEAN and el.max() <= LSE_MAX, (var, g)


def test_non_default_stream():
    q, k, v = W.gaussian_qkv(1, 4, 512, 64, "fp16", seed=26)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = da.attn_fwd(qd, kd, vd, stream=s)
    s.synchronize()
    check_full(o, lse, q, k, v, 1 / math.sqrt(64), tag="side stream")


def test_long_sequence_sampled():
    S = 32768 + 17
    q, k, v = W.gaussian_qkv(1, 1, S, 128, "bf16", seed=27)
    o, lse = gpu_run(q, k, v, 1 / math.sqrt(128))
    rng = np.random.default_rng(27)
    rows = _sample_rows(S, 64, rng)
    ro, rl = attention_rows(W.to_f64(q), W.to_f64(k), W.to_f64(v), 1 / math.sqrt(128), 0, 0, rows)
    e = np.abs(o[0, 0].cpu()[rows].double().numpy() - ro)
    say(f"  S={S} sampled O max {e.max():.3e}")
    assert e.max() <= O_MAX and e.mean() <= O_MEAN
    assert np.abs(lse[0, 0].cpu()[rows].double().numpy() - rl).max() <= LSE_MAX


@pytest.mark.parametrize("layout", ["bhsd", "bshd"])
def test_tensors_past_4gib_sampled(layout):
    """Largest-size case: Q, K, V and O of 4.3 GB each, i.e. more than 2^31 elements,
    so head offsets, row offsets (BSHD), K/V tile addresses and O/LSE stores of the
    last heads need more than 32 bits.  Inputs are drawn on the device from a seeded
    generator (host memory would not hold the float32 draws); sampled rows of the
    first head, the heads on either side of element 2^31 and the last head are
    checked against the oracle, which receives exactly the same rounded values."""
    B, H, S, D = 2, 2056, 4096, 128
    assert B * H * S * D > 2**31
    scale = 1 / math.sqrt(D)
    g = torch.Generator(device="cuda")
    g.manual_seed(41)
    shape = (B, H, S, D) if layout == "bhsd" else (B, S, H, D)
    q, k, v = (torch.randn(shape, device="cuda", dtype=torch.bfloat16, generator=g)
               for _ in range(3))
    say(f"  {layout} B={B} H={H} S={S} D={D}: {q.numel() * 2 / 2**30:.2f} GiB per tensor")
    if layout == "bhsd":
        o, lse = da.attn_fwd_ex(q, k, v, scale=scale)
    else:
        q, k, v = (t.transpose(1, 2) for t in (q, k, v))
        o = torch.empty(shape, device="cuda", dtype=torch.bfloat16).transpose(1, 2)
        o, lse = da.attn_fwd_strided(q, k, v, o, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(41)
    heads_per_2g = 2**31 // (S * D)  # head index whose first element is element 2^31
    for bh in (0, heads_per_2g - 1, heads_per_2g, B * H - 1):
        b, h = divmod(bh, H)
        rows = _sample_rows(S, 24, rng)
        qs, ks, vs = (W.to_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
        ro, rl = attention_rows(qs, ks, vs, scale, 0, 0, rows)
        e = np.abs(o[b, h].cpu()[rows].double().numpy() - ro)
        le = np.abs(lse[b, h].cpu()[rows].double().numpy() - rl).max()
        say(f"  b={b} h={h}: O max {e.max():.3e} LSE max {le:.3e}")
        assert e.max() <= O_MAX and e.mean() <= O_MEAN and le <= LSE_MAX, bh
    del q, k, v, o, lse
    torch.cuda.empty_cache()
