"""The forward captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI):
every replay, with eager work and synchronisation between replays and new
input values written into the captured buffers, must give the bits of the
eager call on the same inputs.  Covers the single-launch forward, the causal
forward and the two-launch split-KV paths (caller workspace and the library's
static scratch, whose entry point allocates nothing)."""

import math
import sys

import pytest
import torch

import dense_attention_amd as da
import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    da.load_library()
    yield
    torch.cuda.synchronize()


def _capture(fn):
    """Runs fn once on a side stream (warm-up, as capture requires), then
    captures it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _inputs(B, H, S, D, dtype, seed):
    return [t.cuda() for t in W.gaussian_qkv(B, H, S, D, dtype, seed=seed)]


@pytest.mark.parametrize("mode", ["fwd", "causal", "split", "split_noalloc"])
def test_graph_replays_match_eager(mode):
    B, H, S, D, dtype = 1, 4, 1000, 128, "bf16"
    scale = 1 / math.sqrt(D)
    q, k, v = _inputs(B, H, S, D, dtype, seed=61)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    kv_splits = 3
    ws = torch.empty(max(da.attn_fwd_split_workspace_size(B, H, S, D, kv_splits), 256),
                     dtype=torch.uint8, device="cuda")

    def call(qq, kk, vv, oo, ll):
        if mode == "fwd":
            da.attn_fwd(qq, kk, vv, oo, ll, scale=scale)
        elif mode == "causal":
            da.attn_fwd_ex(qq, kk, vv, oo, ll, scale=scale, causal=True)
        elif mode == "split":
            da.attn_fwd_split(qq, kk, vv, oo, ll, scale=scale, kv_splits=kv_splits, workspace=ws)
        else:
            da.attn_fwd_split_noalloc(qq, kk, vv, oo, ll, scale=scale, kv_splits=kv_splits)

    g = _capture(lambda: call(q, k, v, o, lse))
    for r in range(REPLAYS):
        # new inputs in the captured buffers, and eager work of our own
        nq, nk, nv = _inputs(B, H, S, D, dtype, seed=62 + r)
        q.copy_(nq); k.copy_(nk); v.copy_(nv)
        o.fill_(float("nan")); lse.fill_(float("nan"))
        ref_o = torch.empty_like(q)
        ref_l = torch.empty_like(lse)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(nq, nk, nv, ref_o, ref_l)  # eager, on separate buffers
        torch.cuda.synchronize()
        say(f"{mode} replay {r}: equal {torch.equal(o, ref_o) and torch.equal(lse, ref_l)}")
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), (mode, r)
