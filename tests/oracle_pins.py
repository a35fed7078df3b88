"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin takes a forward function ``fwd(q, k, v, scale) -> (o, lse)`` over
float64 [B, H, S, D] arrays and raises AssertionError when it disagrees with
mathematics fixed independently of the oracle's own code:

* hand-derived exact fractions (``tests/golden/powers_of_two.json``);
* brute force on tiny inputs through a differently arranged formula,
  w_ik = 1 / sum_j exp(s_ij - s_ik), summed with ``math.fsum``;
* the library routine ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 on the CPU, and ``scipy.special.logsumexp`` for the LSE;
* closed forms (zero query, zero scale, constant V, a single key, two keys,
  one dominant key at huge logits) and invariants (per-row logit shift, joint
  permutation of keys and values, permutation of queries, convex hull);
* for the causal mask: the brute force over the visible keys only, torch's
  is_causal (equal lengths) or an explicit lower-triangular boolean mask
  (other lengths), the first row (one key) and the last row (all keys), and
  rows that see no key.

The same pins are run against planted mistakes in ``test_oracle.py`` to show
that each plausible slip fails at least one of them.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "powers_of_two.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _parse_frac(s: str) -> float:
    return float(Fraction(s))


def _parse_ln(s: str) -> float:
    assert s.startswith("ln(") and s.endswith(")")
    return math.log(float(Fraction(s[3:-1])))


def pin_golden_fractions(fwd):
    with open(GOLDEN) as f:
        g = json.load(f)
    assert g["scale"] == "ln2"
    scale = math.log(2.0)
    for case in g["cases"]:
        q = np.array(case["q"], dtype=np.float64)[None, None]
        k = np.array(case["k"], dtype=np.float64)[None, None]
        v = np.array(case["v"], dtype=np.float64)[None, None]
        o, lse = fwd(q, k, v, scale)
        exp_o = np.array([[_parse_frac(x) for x in row] for row in case["expected_o"]])
        exp_l = np.array([_parse_ln(x) for x in case["expected_lse"]])
        np.testing.assert_allclose(np.asarray(o)[0, 0], exp_o, rtol=0, atol=1e-12,
                                   err_msg=case["name"])
        np.testing.assert_allclose(np.asarray(lse)[0, 0], exp_l, rtol=0, atol=1e-12,
                                   err_msg=case["name"])


def _brute(q, k, v, scale):
    """Independent arrangement: weight of key t for query i is 1 / sum_j exp(s_ij - s_it)."""
    B, H, S, D = q.shape
    Skv = k.shape[2]
    o = np.zeros((B, H, S, D))
    lse = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            for i in range(S):
                s = [scale * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D))
                     for j in range(Skv)]
                for t in range(Skv):
                    w = 1.0 / math.fsum(math.exp(s[j] - s[t]) for j in range(Skv))
                    for d in range(D):
                        o[b, h, i, d] += w * v[b, h, t, d]
                lse[b, h, i] = math.log(math.fsum(math.exp(x) for x in s))
    return o, lse


def pin_brute_force_tiny(fwd):
    rng = _rng(1234)
    for (B, H, S, D, scale) in [(1, 1, 1, 1, 0.7), (1, 1, 3, 2, 1.0), (2, 3, 5, 3, 0.5),
                                (1, 2, 7, 4, 1.3), (2, 1, 8, 3, 2.0 ** -0.5), (1, 1, 6, 6, 1.0)]:
        q = rng.integers(-3, 4, size=(B, H, S, D)).astype(np.float64)
        k = rng.integers(-3, 4, size=(B, H, S, D)).astype(np.float64)
        v = rng.normal(size=(B, H, S, D))
        o, lse = fwd(q, k, v, scale)
        bo, bl = _brute(q, k, v, scale)
        np.testing.assert_allclose(np.asarray(o), bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.asarray(lse), bl, rtol=0, atol=1e-12)
    # queries and keys of different lengths (a key subset, or cross attention)
    for (B, H, Sq, Skv, D, scale) in [(1, 1, 2, 5, 3, 0.8), (2, 1, 6, 1, 2, 1.0), (1, 2, 3, 8, 4, 0.5)]:
        q = rng.integers(-3, 4, size=(B, H, Sq, D)).astype(np.float64)
        k = rng.integers(-3, 4, size=(B, H, Skv, D)).astype(np.float64)
        v = rng.normal(size=(B, H, Skv, D))
        o, lse = fwd(q, k, v, scale)
        bo, bl = _brute(q, k, v, scale)
        np.testing.assert_allclose(np.asarray(o), bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.asarray(lse), bl, rtol=0, atol=1e-12)


def pin_torch_sdpa(fwd):
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    rng = _rng(99)
    for (B, H, S, Skv, D) in [(1, 4, 128, 128, 64), (1, 2, 512, 512, 64), (2, 2, 100, 100, 128),
                              (1, 1, 33, 33, 16), (1, 2, 37, 211, 64), (2, 1, 300, 7, 128)]:
        q = rng.standard_normal((B, H, S, D))
        k = rng.standard_normal((B, H, Skv, D))
        v = rng.standard_normal((B, H, Skv, D))
        scale = 1.0 / math.sqrt(D)
        o, lse = fwd(q, k, v, scale)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), scale=scale).numpy()
        np.testing.assert_allclose(np.asarray(o), ref, rtol=0, atol=1e-12)
        scores = scale * np.einsum("bhid,bhjd->bhij", q, k)
        np.testing.assert_allclose(np.asarray(lse), logsumexp(scores, axis=-1), rtol=0, atol=1e-12)


def pin_zero_query(fwd):
    rng = _rng(5)
    for (S, D) in [(1, 4), (9, 3), (128, 64), (300, 16)]:
        q = np.zeros((2, 1, S, D))
        k = rng.standard_normal((2, 1, S, D))
        v = rng.standard_normal((2, 1, S, D))
        o, lse = fwd(q, k, v, 0.3)
        mean_v = v.mean(axis=2, keepdims=True)
        np.testing.assert_allclose(np.asarray(o), np.broadcast_to(mean_v, o.shape), rtol=0,
                                   atol=1e-12)
        np.testing.assert_allclose(np.asarray(lse), np.full((2, 1, S), math.log(S)), rtol=0,
                                   atol=1e-12)


def pin_zero_scale(fwd):
    rng = _rng(6)
    q, k, v = (rng.standard_normal((1, 2, 37, 8)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.0)
    np.testing.assert_allclose(np.asarray(o), np.broadcast_to(v.mean(axis=2, keepdims=True),
                                                              o.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.asarray(lse), math.log(37), rtol=0, atol=1e-12)


def pin_constant_v(fwd):
    rng = _rng(7)
    q, k = (rng.standard_normal((1, 3, 50, 8)) * 3 for _ in range(2))
    c = rng.standard_normal(8)
    v = np.broadcast_to(c, (1, 3, 50, 8)).copy()
    o, _ = fwd(q, k, v, 0.9)
    np.testing.assert_allclose(np.asarray(o), v, rtol=0, atol=1e-12)


def pin_single_key(fwd):
    rng = _rng(8)
    q, k, v = (rng.standard_normal((3, 2, 1, 5)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.8)
    np.testing.assert_allclose(np.asarray(o), v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.asarray(lse), 0.8 * (q * k).sum(-1), rtol=0, atol=1e-12)


def pin_two_keys_logistic(fwd):
    """With two keys the weight of key 1 is the logistic sigmoid of the score gap."""
    rng = _rng(9)
    q = rng.standard_normal((1, 1, 2, 6))
    k = rng.standard_normal((1, 1, 2, 6))
    v = rng.standard_normal((1, 1, 2, 6))
    scale = 0.75
    o, lse = fwd(q, k, v, scale)
    for i in range(2):
        s0 = scale * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = scale * float(q[0, 0, i] @ k[0, 0, 1])
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        exp_o = (1.0 - w1) * v[0, 0, 0] + w1 * v[0, 0, 1]
        np.testing.assert_allclose(np.asarray(o)[0, 0, i], exp_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(np.asarray(lse)[0, 0, i], np.logaddexp(s0, s1), rtol=0,
                                   atol=1e-12)


def pin_dominant_key_huge_logits(fwd):
    """Scores near 1e4 with one key ahead by >= 64: O is that key's V; no overflow allowed."""
    S, D = 16, 4
    q = np.zeros((1, 1, S, D))
    k = np.zeros((1, 1, S, D))
    q[0, 0, :, 0] = 100.0
    k[0, 0, :, 0] = 100.0 - np.arange(S) * 0.64   # key 0 has the largest score
    rng = _rng(10)
    for i in range(S):
        q[0, 0, i, 1] = 1.0
    k[0, 0, :, 1] = 0.0
    v = rng.standard_normal((1, 1, S, D))
    o, lse = fwd(q, k, v, 1.0)
    o, lse = np.asarray(o), np.asarray(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # Gaps are 64, 128, ... so exp(-64) ~ 1.6e-28 is the largest neglected weight.
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 0], (S, D)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.full(S, 100.0 * 100.0), rtol=0, atol=1e-9)


def pin_row_shift(fwd):
    """Adding delta*c to every score of one row leaves O unchanged and moves LSE by delta*c*scale."""
    rng = _rng(11)
    B, H, S, D = 1, 2, 40, 8
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    k[..., 0] = 1.5                      # every key shares component 0
    scale = 0.6
    o0, l0 = fwd(q, k, v, scale)
    delta = rng.standard_normal((B, H, S)) * 4.0
    q2 = q.copy()
    q2[..., 0] += delta
    o1, l1 = fwd(q2, k, v, scale)
    np.testing.assert_allclose(np.asarray(o1), np.asarray(o0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.asarray(l1), np.asarray(l0) + scale * 1.5 * delta, rtol=0,
                               atol=1e-11)


def pin_permutations(fwd):
    rng = _rng(12)
    B, H, S, D = 2, 2, 24, 6
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.7)
    pk = rng.permutation(S)
    o2, l2 = fwd(q, k[:, :, pk], v[:, :, pk], 0.7)
    np.testing.assert_allclose(np.asarray(o2), np.asarray(o), rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.asarray(l2), np.asarray(lse), rtol=0, atol=1e-12)
    pq = rng.permutation(S)
    o3, l3 = fwd(q[:, :, pq], k, v, 0.7)
    np.testing.assert_allclose(np.asarray(o3), np.asarray(o)[:, :, pq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.asarray(l3), np.asarray(lse)[:, :, pq], rtol=0, atol=1e-12)


def pin_convex_hull(fwd):
    rng = _rng(13)
    q, k, v = (rng.standard_normal((1, 2, 64, 8)) * 2 for _ in range(3))
    o, _ = fwd(q, k, v, 1.0)
    o = np.asarray(o)
    lo = v.min(axis=2, keepdims=True)
    hi = v.max(axis=2, keepdims=True)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


# --- causal mask: key j is visible to query row i iff j <= i + offset -----------------

def _brute_causal(q, k, v, scale, offset):
    """Independent arrangement over the visible keys only; a row without any
    visible key is defined as o = 0, lse = -inf."""
    B, H, S, D = q.shape
    Skv = k.shape[2]
    o = np.zeros((B, H, S, D))
    lse = np.full((B, H, S), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(S):
                vis = [j for j in range(Skv) if j - i <= offset]
                if not vis:
                    continue
                s = {j: scale * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) for j in vis}
                for t in vis:
                    w = 1.0 / math.fsum(math.exp(s[j] - s[t]) for j in vis)
                    for d in range(D):
                        o[b, h, i, d] += w * v[b, h, t, d]
                lse[b, h, i] = math.log(math.fsum(math.exp(x) for x in s.values()))
    return o, lse


def pin_causal_brute_force(fwd):
    rng = _rng(4321)
    for (B, H, Sq, Skv, D, scale, off) in [(1, 1, 5, 5, 3, 1.0, 0), (2, 1, 7, 7, 2, 0.5, 0),
                                           (1, 2, 3, 8, 4, 0.7, 5), (1, 1, 8, 3, 2, 1.0, -5),
                                           (1, 1, 6, 6, 3, 0.9, 2), (1, 1, 6, 6, 3, 0.9, -2)]:
        q = rng.integers(-3, 4, size=(B, H, Sq, D)).astype(np.float64)
        k = rng.integers(-3, 4, size=(B, H, Skv, D)).astype(np.float64)
        v = rng.normal(size=(B, H, Skv, D))
        o, lse = fwd(q, k, v, scale, causal_offset=off)
        bo, bl = _brute_causal(q, k, v, scale, off)
        np.testing.assert_allclose(np.asarray(o), bo, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(np.asarray(lse)), np.isneginf(bl))
        fin = np.isfinite(bl)
        np.testing.assert_allclose(np.asarray(lse)[fin], bl[fin], rtol=0, atol=1e-12)


def pin_causal_torch_sdpa(fwd):
    """Equal lengths: torch's is_causal.  Other lengths: the boolean mask
    tril(diagonal = Skv - Sq), i.e. the last query row sees every key."""
    import torch
    import torch.nn.functional as F

    rng = _rng(77)
    for (B, H, Sq, Skv, D) in [(1, 2, 128, 128, 64), (2, 1, 100, 100, 32), (1, 2, 37, 211, 64),
                               (1, 1, 200, 200, 16)]:
        q = rng.standard_normal((B, H, Sq, D))
        k = rng.standard_normal((B, H, Skv, D))
        v = rng.standard_normal((B, H, Skv, D))
        scale = 1.0 / math.sqrt(D)
        o, lse = fwd(q, k, v, scale, causal_offset=Skv - Sq)
        tq, tk, tv = torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)
        if Sq == Skv:
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale).numpy()
        else:
            m = torch.ones(Sq, Skv, dtype=torch.bool).tril(diagonal=Skv - Sq)
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale).numpy()
        np.testing.assert_allclose(np.asarray(o), ref, rtol=0, atol=1e-12)
        scores = scale * np.einsum("bhid,bhjd->bhij", q, k)
        vis = np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + (Skv - Sq)
        mx = np.where(vis, scores, -np.inf).max(axis=-1)
        ref_l = mx + np.log(np.where(vis, np.exp(scores - mx[..., None]), 0.0).sum(axis=-1))
        np.testing.assert_allclose(np.asarray(lse), ref_l, rtol=0, atol=1e-12)


def pin_causal_first_and_last_rows(fwd):
    """Equal lengths: row 0 sees key 0 only (o = v_0, lse = scale q_0·k_0);
    the last row sees every key, as in torch's unmasked attention."""
    import torch
    import torch.nn.functional as F

    rng = _rng(78)
    q = rng.standard_normal((2, 2, 50, 8))
    k = rng.standard_normal((2, 2, 50, 8))
    v = rng.standard_normal((2, 2, 50, 8))
    o, lse = fwd(q, k, v, 0.4, causal_offset=0)
    np.testing.assert_allclose(np.asarray(o)[:, :, 0], v[:, :, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(np.asarray(lse)[:, :, 0], 0.4 * (q[:, :, 0] * k[:, :, 0]).sum(-1),
                               rtol=0, atol=1e-13)
    full = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                          torch.from_numpy(v), scale=0.4).numpy()
    np.testing.assert_allclose(np.asarray(o)[:, :, -1], full[:, :, -1], rtol=0, atol=1e-12)


def pin_causal_rows_without_keys(fwd):
    """More queries than keys, last rows aligned: the first Sq - Skv rows see
    nothing (o = 0, lse = -inf); row Sq - Skv sees key 0 only."""
    rng = _rng(79)
    q = rng.standard_normal((1, 1, 9, 4))
    k = rng.standard_normal((1, 1, 4, 4))
    v = rng.standard_normal((1, 1, 4, 4))
    o, lse = fwd(q, k, v, 0.5, causal_offset=4 - 9)
    o, lse = np.asarray(o), np.asarray(lse)
    assert np.all(o[0, 0, :5] == 0.0) and np.all(np.isneginf(lse[0, 0, :5]))
    np.testing.assert_allclose(o[0, 0, 5], v[0, 0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0, 5], 0.5 * q[0, 0, 5] @ k[0, 0, 0], rtol=0, atol=1e-13)


ALL_PINS = [
    pin_causal_brute_force,
    pin_causal_torch_sdpa,
    pin_causal_first_and_last_rows,
    pin_causal_rows_without_keys,
    pin_golden_fractions,
    pin_brute_force_tiny,
    pin_torch_sdpa,
    pin_zero_query,
    pin_zero_scale,
    pin_constant_v,
    pin_single_key,
    pin_two_keys_logistic,
    pin_dominant_key_huge_logits,
    pin_row_shift,
    pin_permutations,
    pin_convex_hull,
]
