"""GPU test of attn_fwd_split_noalloc, the entry point whose key-range partials
live in the library's static device scratch: called through the C ABI, its
output must equal attn_fwd_split's (same kernels, same ranges, a caller
workspace) bit for bit and meet the oracle's bar, on consecutive calls that
reuse the scratch, the second smaller than the first."""

import gc
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


def _one(B, H, S, D, dtype, seed, kv_splits, causal=False):
    q, k, v = W.gaussian_qkv(B, H, S, D, dtype, seed=seed)
    scale = 1 / math.sqrt(D)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    need = da.attn_fwd_split_workspace_size(B, H, S, D, kv_splits)
    assert need <= da.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ref_o, ref_l = da.attn_fwd_split(qd, kd, vd, scale=scale, kv_splits=kv_splits, workspace=ws,
                                     causal=causal)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    # Tensors of earlier tests that the garbage collector frees during the
    # call would lower the allocated bytes: collect first, and compare the
    # allocator's cumulative count of allocations, which frees do not move.
    gc.collect()
    before = torch.cuda.memory_allocated()
    allocs = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    say(f"noalloc B={B} H={H} S={S} D={D} {dtype} kv_splits={kv_splits} causal={causal} "
        f"(partials {need} bytes)")
    da.attn_fwd_split_noalloc(qd, kd, vd, o, lse, scale=scale, kv_splits=kv_splits, causal=causal)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == allocs
    assert torch.cuda.memory_allocated() <= before
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), "differs from attn_fwd_split"
    ro, rl = attention_forward(W.to_f64(q), W.to_f64(k), W.to_f64(v), scale,
                               causal_offset=0 if causal else None)
    err = np.abs(o.cpu().double().numpy() - ro)
    lerr = np.abs(lse.cpu().double().numpy() - rl).max()
    say(f"  O max {err.max():.3e} mean {err.mean():.3e} LSE max {lerr:.3e}")
    assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr <= LSE_MAX


def test_noalloc_matches_split_on_consecutive_calls():
    # first call: 4 ranges over the fp16 hd64 benchmark shape (32.5 MiB of partials)
    _one(1, 8, 4096, 64, "fp16", seed=2, kv_splits=4)
    # second call reuses the scratch with a smaller problem, ragged length, other dtype and D
    _one(1, 2, 1000, 128, "bf16", seed=5100, kv_splits=3)
    # the library's own range count, then a causal split
    _one(1, 1, 2048, 64, "bf16", seed=5101, kv_splits=0)
    _one(2, 2, 777, 64, "fp16", seed=5102, kv_splits=2, causal=True)


def test_noalloc_refuses_a_problem_beyond_the_scratch():
    q = torch.zeros(1, 16, 4096, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(da.AttnError) as ei:
        da.attn_fwd_split_noalloc(q, q, q, o, kv_splits=8)
    assert ei.value.status == -9
