"""Runs the float64 oracle over every (batch, head) of a large problem, heads in
parallel threads.  Test infrastructure: each call is the unchanged oracle on
one head's [1, 1, S, D] slice, so the result is exactly what one
``attention_forward`` over the whole tensor would return; the threads only
spread the independent heads over the host's cores (NumPy's products and
exponentials release the GIL).  BLAS runs single-threaded inside the pool so
the threads do not oversubscribe the cores."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import threadpoolctl

import workloads as W
from oracle import attention_forward


def workers() -> int:
    # The GPU host gives a job 16 CPUs whatever os.cpu_count() reports.
    return max(1, min(16, os.cpu_count() or 1))


def forward_by_head(q, k, v, scale: float, causal_offset=None, row_block: int = 512):
    """(o [B,H,Sq,D], lse [B,H,Sq]) in float64 for torch fp16/bf16 inputs."""
    B, H, Sq, D = q.shape
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)

    def one(bh):
        b, h = divmod(bh, H)
        qs, ks, vs = (W.to_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
        ob, lb = attention_forward(qs, ks, vs, scale, row_block=row_block,
                                   causal_offset=causal_offset)
        o[b, h], lse[b, h] = ob[0, 0], lb[0, 0]

    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers()) as ex:
            list(ex.map(one, range(B * H)))
    return o, lse
