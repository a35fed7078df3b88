"""CPU float64 oracle for the dense (non-causal) attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, the package's smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels.

What it computes is the plain definition of softmax attention, written out
directly, materialising every full row of the score matrix:

    s_ij   = scale * sum_d q_id k_jd                      (scores)
    m_i    = max_j s_ij                                   (row maximum)
    e_ij   = exp(s_ij - m_i)
    l_i    = sum_j e_ij                                   (row sum)
    o_id   = (sum_j e_ij v_jd) / l_i                      (normalised output)
    lse_i  = m_i + ln l_i                                 (natural-log log-sum-exp)

With a causal mask the maximum, the sums and the log-sum-exp run over the
keys j <= i + offset only; a row that sees no key has o = 0 and lse = -inf.

Sources.  The per-(batch, head, query-tile) work split, the S = Q·Kᵀ / softmax
/ P·V sections and the final division by the row sum follow "B200 Attention
Kernel from Scratch to Near-SOTA in 60 Diagrams", Chapter 1, "ii. Work
Parallelization" and "B) Online Softmax (explaining S->P)".  The
materialise-then-reduce shape (scores for a whole row, then max, then
exp-and-sum, then normalise) is the unfused baseline of "Learning
FlashAttention the Hard Way - Part 2", "Move 0 - Scalar Streaming Kernel".
The log-sum-exp residual is kept in natural-log units as "Attention for sm90,
Line by Line" describes in "Why does the kernel use exp2 rather than exp?".

The online (tile-by-tile) softmax of the GPU path is exact in real arithmetic,
so the oracle does not emulate it: it evaluates the definition once per row in
float64.  Rows are processed in blocks only to bound memory; every row always
sees all S keys.
"""

from __future__ import annotations

import numpy as np

__all__ = ["attention_forward", "attention_rows"]


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError("expected a [B, H, S, D] array")
    return a


def _rows(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, mask=None):
    """Attention of the query rows ``qh`` [R, D] against one head's keys/values [Skv, D].

    ``mask`` (optional, bool [R, Skv]) marks the keys each row may attend to;
    a row with no such key gets o = 0 and lse = -inf.
    """
    s = scale * (qh @ kh.T)                 # [R, Skv] scores
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)        # [R, 1] row maxima
    seen = np.isfinite(m[:, 0])             # rows with at least one key
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)                  # [R, Skv]; masked scores give 0
    l = e.sum(axis=1, keepdims=True)        # [R, 1] row sums
    o = (e @ vh) / np.where(seen[:, None], l, 1.0)      # [R, D]
    lse = np.where(seen, m_safe[:, 0] + np.log(np.where(seen, l[:, 0], 1.0)), -np.inf)
    return o, lse


def causal_mask(rows, Skv: int, offset: int):
    """Keys visible to query rows ``rows`` under a causal mask: key j is
    visible to query row i iff j <= i + offset (offset = Skv - Sq aligns the
    last query row with the last key)."""
    rows = np.asarray(rows, dtype=np.int64)
    return np.arange(Skv)[None, :] <= rows[:, None] + offset


def attention_forward(q, k, v, scale: float, row_block: int = 1024, causal_offset=None):
    """Full forward.  q is [B, H, Sq, D]; k and v are [B, H, Skv, D] (Skv >= 1; the
    usual self-attention case has Skv = Sq).  Without a mask every query row
    attends to all Skv keys of its head; with ``causal_offset`` (an int) query
    row i attends to keys j <= i + causal_offset.  Returns (o [B,H,Sq,D],
    lse [B,H,Sq]) in float64."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, S, D = q.shape
    Skv = k.shape[2]
    if k.shape != (B, H, Skv, D) or v.shape != (B, H, Skv, D) or Skv < 1:
        raise ValueError("k and v must be [B, H, Skv, D] with Skv >= 1 and q's B, H, D")
    o = np.empty((B, H, S, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, S, row_block):
                r1 = min(S, r0 + row_block)
                mask = None if causal_offset is None else causal_mask(range(r0, r1), Skv, causal_offset)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _rows(q[b, h, r0:r1], k[b, h], v[b, h], scale, mask)
    return o, lse


def attention_rows(q, k, v, scale: float, b: int, h: int, rows, causal_offset=None):
    """The same definition for selected query rows of one (b, h) only, each against all keys
    (or the keys the causal mask lets it see).

    Used to check large problems on a sample of output rows.  Returns
    (o [len(rows), D], lse [len(rows)]) in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    qh = np.asarray(q[b, h], dtype=np.float64)[rows]
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    mask = None if causal_offset is None else causal_mask(rows, kh.shape[0], causal_offset)
    return _rows(qh, kh, vh, scale, mask)
