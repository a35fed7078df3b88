"""CPU check of the software exp2 constants compiled into the kernel (the
optional selective software exp2).  The polynomial is evaluated in float32 the
way the kernel evaluates it: x clamped at -127, f = x - floor(x), three FMAs
in Horner form, then scaling by 2^floor(x).  Its relative error against the
exact 2^x must stay below 1e-4 everywhere the softmax can feed it (x <= 64),
well inside the rounding of P to bf16 (2^-9) or fp16 (2^-11)."""

import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(__file__), "..", "dense_attention_amd", "csrc", "attn_fwd_kernel.h")


def kernel_coefficients():
    src = open(HDR).read()
    body = src[src.index("float exp2_poly(float x)"):]
    body = body[:body.index("}")]
    c = [float(x) for x in re.findall(r"([0-9]+\.[0-9]*)f", body)]
    # clamp, then c3, c2, c1, c0 in order of appearance
    assert c[0] == 127.0
    return c[1], c[2], c[3], c[4]


def poly_exp2_f32(x, c3, c2, c1, c0):
    x = np.maximum(np.float32(x), np.float32(-127.0)).astype(np.float32)
    n = np.floor(x).astype(np.float32)
    f = (x - n).astype(np.float32)
    p = np.float32(c3) * f + np.float32(c2)
    p = (p * f + np.float32(c1)).astype(np.float32)
    p = (p * f + np.float32(c0)).astype(np.float32)
    return np.ldexp(p.astype(np.float64), n.astype(np.int64))


def test_constants_are_the_fitted_ones():
    c3, c2, c1, c0 = kernel_coefficients()
    assert c0 == 1.0
    assert abs(c1 - 0.695116786) < 1e-9 and abs(c2 - 0.227644991) < 1e-9 and abs(c3 - 0.077067042) < 1e-9


def test_relative_error_bound():
    c3, c2, c1, c0 = kernel_coefficients()
    x = np.concatenate([np.linspace(-126.0, 64.0, 400001), -np.arange(0, 127, dtype=np.float64),
                        np.arange(0, 65, dtype=np.float64) - 1e-6]).astype(np.float32)
    approx = poly_exp2_f32(x, c3, c2, c1, c0)
    exact = np.exp2(x.astype(np.float64))
    rel = np.abs(approx / exact - 1.0)
    assert rel.max() < 1e-4, rel.max()
    # just below integers (where x - fract(x) would not be an integer)
    near = (np.arange(-20, 9, dtype=np.float64)[:, None] - np.array([1e-8, 3e-8, 1e-7, 6e-8])[None, :]).ravel()
    near = near.astype(np.float32)
    rel = np.abs(poly_exp2_f32(near, c3, c2, c1, c0) / np.exp2(near.astype(np.float64)) - 1.0)
    assert rel.max() < 1e-4, rel.max()
    # integer arguments are exact powers of two
    ints = np.arange(-126, 65, dtype=np.float32)
    assert np.array_equal(poly_exp2_f32(ints, c3, c2, c1, c0), np.exp2(ints.astype(np.float64)))


def test_far_negative_arguments_give_negligible_values():
    c3, c2, c1, c0 = kernel_coefficients()
    v = poly_exp2_f32(np.array([-127.0, -200.0, -1e30], dtype=np.float32), c3, c2, c1, c0)
    assert np.all(v <= 2.0 ** -126)


def test_fit_script_reproduces_the_constants():
    import importlib.util
    path = os.path.join(os.path.dirname(HDR), "fit_exp2_poly.py")
    spec = importlib.util.spec_from_file_location("fit_exp2_poly", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    (c0, c1, c2, c3), err = mod.fit()
    k3, k2, k1, k0 = kernel_coefficients()
    assert abs(c1 - k1) < 5e-9 and abs(c2 - k2) < 5e-9 and abs(c3 - k3) < 5e-9
    assert err < 1e-4
