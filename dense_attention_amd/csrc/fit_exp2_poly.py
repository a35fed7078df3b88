"""Fits the cubic used by the kernel's optional software exp2.

2^x = 2^n · 2^f with n = floor(x) and f = x - n in [0, 1); 2^f is replaced by
c0 + c1·f + c2·f² + c3·f³.  The coefficients minimise the maximum relative
error on [0, 1) (a Remez exchange on the relative error, starting from
Chebyshev nodes), with c0 pinned to 1 so that integer x give exact powers of
two.  Run it to reprint the constants in attn_fwd_kernel.h:

    python dense_attention_amd/csrc/fit_exp2_poly.py
"""

import numpy as np


def fit(iters: int = 30):
    # Unknowns c1, c2, c3 and the levelled error E at 4 reference points:
    # (1 + c1 f + c2 f² + c3 f³) / 2^f - 1 = (-1)^k E.
    k = np.arange(4)
    f = 0.5 - 0.5 * np.cos(np.pi * (k + 0.5) / 4)
    grid = np.linspace(0.0, 1.0, 200001)
    for _ in range(iters):
        t = 2.0 ** f
        A = np.stack([f / t, f ** 2 / t, f ** 3 / t, -((-1.0) ** k)], axis=1)
        rhs = 1.0 - 1.0 / t
        c1, c2, c3, E = np.linalg.solve(A, rhs)
        err = (1 + c1 * grid + c2 * grid ** 2 + c3 * grid ** 3) / 2.0 ** grid - 1
        # new reference: the extremum of each sign-alternating segment
        sign = np.sign(err)
        cuts = np.flatnonzero(np.diff(sign) != 0) + 1
        segs = np.split(np.arange(grid.size), cuts)
        ext = [s[np.argmax(np.abs(err[s]))] for s in segs]
        if len(ext) >= 4:
            ext = sorted(ext, key=lambda i: -abs(err[i]))[:4]
            f = np.sort(grid[ext])
    err = (1 + c1 * grid + c2 * grid ** 2 + c3 * grid ** 3) / 2.0 ** grid - 1
    return (1.0, c1, c2, c3), float(np.abs(err).max())


if __name__ == "__main__":
    c, e = fit()
    print("c0..c3 =", ", ".join(f"{x:.9g}" for x in c))
    print(f"max relative error on [0, 1): {e:.3e}")
